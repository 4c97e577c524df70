// Dense bf16 products of the grouped-GEMM path (prefill-sized batches): the
// router logits and the shared expert, whose weights are plain bf16 (model
// card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model": the routers
// and the shared experts sit in the dense part of each layer).
//
// One kernel, C = A B^T with A [M][K] and B [N][K] both bf16 (rows along K),
// fp32 accumulation on the 32x32x16 bf16 matrix cores, two parts per launch:
//   part 0  plain columns: C0[m][n] = (A B0^T)[m][n] (+ bias[n]), fp32 --
//           the router logits (B0 = W_r, bias = the per-expert bias) or the
//           shared down projection (A = a_sh, B0 = W_down, no bias);
//   part 1  SwiGLU columns (optional): u = A W_up^T, g = A W_gate^T over the
//           shared expert's up|gate rows, a_sh[m][o] = bf16_rne(silu(g) u).
// The router and the shared up|gate read the same A (the tokens), so they run
// as the two parts of one launch.
//
// Tiles: 128 rows of A x 256 rows of B, K steps of 32; four waves in a 2 x 2
// arrangement, wave (wm, wn) owns rows 64 wm .. +63 of the A tile and rows
// 128 wn .. +127 of the B tile (2 x 4 accumulators of 32 x 32); both operands
// staged through two LDS stages (16-byte chunks, XOR swizzle), one barrier
// per K step, the next step's chunks loaded into registers a step ahead.  In
// SwiGLU tiles wave wn's 128 B rows are 64 up rows and the 64 gate rows of
// the same outputs, so u and g of an output meet in one lane.
#include "moe_kernels.hpp"

namespace moe {

namespace {

constexpr int DBM = 128, DBN = 256, DBK = 32;
constexpr int kDChunks = DBK / 8;                    // 16-byte chunks per row per K step

struct DenseArgs {
    const uint16_t* A;   // [M][K]
    const uint16_t* B0;  // part 0 rows [N0][K]
    const uint16_t* B1;  // part 1 rows [2 Is][K] (up rows, then gate rows), or null
    const float* bias;   // part 0 bias [N0] or null
    float* C0;           // part 0 output [M][N0]
    uint16_t* A1;        // part 1 output bf16 [M][Is]
    int M, K, N0, Is;
    int nt0, nt1;        // N tiles of each part
    int mpx;             // M tiles per XCD
};

// LDS slot of chunk c of row r: rows of kDChunks chunks; the chunk index is
// XORed with bits of the row so that the fragment reads (32 consecutive rows
// at one chunk) and the stores (two rows of four chunks per 8 lanes) hit
// distinct bank groups, for LDS of 32 or 64 four-byte banks.
__device__ __forceinline__ int dslot(int r, int c) {
    return r * kDChunks + (c ^ (((r >> 1) ^ (r >> 3)) & 3));
}

__device__ __forceinline__ float silu_mul_exact(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace

template <bool VEC>   // VEC: N0 a multiple of 4, C0 and bias 16-byte aligned
__global__ void __launch_bounds__(256, 2) k_dense(DenseArgs g) {
    __shared__ u32x4 As[2][DBM * kDChunks];           // 2 x 8 KB
    __shared__ u32x4 Bs[2][DBN * kDChunks];           // 2 x 16 KB
    const int tid = threadIdx.x, lane = __lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- tile: blocks reach the 8 XCDs in turn; XCD x takes the M tiles
    // [x mpx, (x + 1) mpx), all N tiles of one M tile back to back (they share
    // its A rows in that XCD's L2)
    const int ntl = g.nt0 + g.nt1;
    const int bid = blockIdx.x, xcd = bid & 7, li = bid >> 3;
    const int mt = xcd * g.mpx + li / ntl, nt = li % ntl;
    if (li / ntl >= g.mpx || mt * DBM >= g.M) return;
    const bool swi = nt >= g.nt0;                      // part 1 tile
    const int m0 = mt * DBM;

    // ---- global source of each of this thread's chunks.  A: 512 chunks,
    // thread t loads rows t / 4 and 64 + t / 4, chunk t % 4.  B: 1024 chunks,
    // rows t / 4 + 64 i (i = 0..3).  Rows past the matrices read the last row.
    const int cc = tid & 3;
    const uint16_t* asrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = (tid >> 2) + 64 * i;
        asrc[i] = g.A + (int64_t)min(m0 + r, g.M - 1) * g.K + cc * 8;
    }
    const uint16_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = (tid >> 2) + 64 * i;             // B tile row
        int64_t src;
        if (!swi) {
            src = min(nt * DBN + b, g.N0 - 1);
            bsrc[i] = g.B0 + src * g.K + cc * 8;
        } else {
            // wave wn's rows 128 wn .. +127: 64 up rows then the 64 gate rows
            // of outputs o0 + 64 wn .. +63
            const int o0 = (nt - g.nt0) * (DBN / 2), q = b & 127, wv = b >> 7;
            const int o = min(o0 + 64 * wv + (q & 63), g.Is - 1);
            src = q < 64 ? o : g.Is + o;
            bsrc[i] = g.B1 + src * g.K + cc * 8;
        }
    }
    struct Raw {
        u32x4 a[2], b[4];
    };
    auto load = [&](int kt, Raw& R) {
        const int ko = kt * DBK;
#pragma unroll
        for (int i = 0; i < 2; ++i) R.a[i] = *reinterpret_cast<const u32x4*>(asrc[i] + ko);
#pragma unroll
        for (int i = 0; i < 4; ++i) R.b[i] = *reinterpret_cast<const u32x4*>(bsrc[i] + ko);
    };
    auto put = [&](int st, const Raw& R) {
#pragma unroll
        for (int i = 0; i < 2; ++i) As[st][dslot((tid >> 2) + 64 * i, cc)] = R.a[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) Bs[st][dslot((tid >> 2) + 64 * i, cc)] = R.b[i];
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int nk = g.K / DBK;
    Raw R;
    load(0, R);
    put(0, R);
    if (nk > 1) load(1, R);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {               // two K16 halves of the step
            u32x4 fa[2], fb[4];
#pragma unroll
            for (int sm = 0; sm < 2; ++sm) fa[sm] = As[st][dslot(64 * wm + 32 * sm + l32, 2 * kk + hh)];
#pragma unroll
            for (int sn = 0; sn < 4; ++sn) fb[sn] = Bs[st][dslot(128 * wn + 32 * sn + l32, 2 * kk + hh)];
#pragma unroll
            for (int sm = 0; sm < 2; ++sm)
#pragma unroll
                for (int sn = 0; sn < 4; ++sn) acc[sm][sn] = mfma32_bf16(fb[sn], fa[sm], acc[sm][sn]);
        }
        if (kt + 1 < nk) {
            put(st ^ 1, R);                            // stage st ^ 1 was last read in step kt - 1
            if (kt + 2 < nk) load(kt + 2, R);
        }
        __syncthreads();
    }

    // ---- epilogue.  The tiles are computed transposed (B fragment first):
    // lane l, register r of accumulator (sm, sn) holds row 32 sm + l % 32 of
    // the wave's A rows and column 8 (r / 4) + 4 (l / 32) + r % 4 of its sn-th
    // group of 32, so each register group r / 4 is four consecutive columns,
    // stored at once (one by one when the row length N0 is not a multiple of
    // 4; Is is a multiple of 64).
#pragma unroll
    for (int sm = 0; sm < 2; ++sm) {
        const int m = m0 + 64 * wm + 32 * sm + l32;
        if (m >= g.M) continue;
        if (!swi) {
#pragma unroll
            for (int sn = 0; sn < 4; ++sn) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = nt * DBN + 128 * wn + 32 * sn + 8 * j + 4 * hh;
                    float* out = g.C0 + (int64_t)m * g.N0 + n;
                    if constexpr (VEC) {
                        if (n >= g.N0) continue;
                        float4 v = make_float4(acc[sm][sn][4 * j], acc[sm][sn][4 * j + 1],
                                               acc[sm][sn][4 * j + 2], acc[sm][sn][4 * j + 3]);
                        if (g.bias) {
                            const float4 b = *reinterpret_cast<const float4*>(g.bias + n);
                            v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
                        }
                        *reinterpret_cast<float4*>(out) = v;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (n + i < g.N0) out[i] = acc[sm][sn][4 * j + i] + (g.bias ? g.bias[n + i] : 0.f);
                    }
                }
            }
        } else {
#pragma unroll
            for (int sn = 0; sn < 2; ++sn) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int o = (nt - g.nt0) * (DBN / 2) + 64 * wn + 32 * sn + 8 * j + 4 * hh;
                    if (o >= g.Is) continue;
                    uint32_t h[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        h[i] = f32_to_bf16(silu_mul_exact(acc[sm][sn + 2][4 * j + i], acc[sm][sn][4 * j + i]));
                    *reinterpret_cast<uint2*>(g.A1 + (int64_t)m * g.Is + o) =
                        make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launchers

namespace {

void launch_dense(const DenseArgs& in, hipStream_t st) {
    DenseArgs a = in;
    const int mtiles = (a.M + DBM - 1) / DBM;
    a.mpx = (mtiles + 7) / 8;
    const unsigned grid = (unsigned)(8 * a.mpx * (a.nt0 + a.nt1));
    const bool vec = (a.N0 & 3) == 0 && ((uintptr_t)a.C0 & 15) == 0 && ((uintptr_t)a.bias & 15) == 0;
    if (vec) k_dense<true><<<grid, 256, 0, st>>>(a);
    else k_dense<false><<<grid, 256, 0, st>>>(a);
}

}  // namespace

bool dense_supported(int K) { return K % DBK == 0; }

void launch_dense_router_shared(const uint16_t* x, int T, int H, int E, const uint16_t* w_r,
                                const float* bias, float* logits, const uint16_t* sh_ug, int Is,
                                uint16_t* a_sh, hipStream_t st) {
    DenseArgs a{};
    a.A = x; a.M = T; a.K = H;
    a.B0 = w_r; a.bias = bias; a.C0 = logits; a.N0 = E;
    a.nt0 = w_r ? (E + DBN - 1) / DBN : 0;
    a.B1 = sh_ug; a.A1 = a_sh; a.Is = Is;
    a.nt1 = (sh_ug && Is > 0) ? (Is + DBN / 2 - 1) / (DBN / 2) : 0;
    if (a.nt0 + a.nt1 == 0) return;
    launch_dense(a, st);
}

void launch_dense_shared_down(const uint16_t* a_sh, int T, int Is, const uint16_t* sh_down, int H,
                              float* y_sh, hipStream_t st) {
    DenseArgs a{};
    a.A = a_sh; a.M = T; a.K = Is;
    a.B0 = sh_down; a.C0 = y_sh; a.N0 = H;
    a.nt0 = (H + DBN - 1) / DBN;
    launch_dense(a, st);
}

}  // namespace moe
