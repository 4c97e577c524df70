// Grouped-GEMM path of the layer (prefill-sized batches).  One kernel
// template, five uses:
//   UG_Q3   routed up|gate: A = token rows gathered through the permutation
//           (fp16), B = Q3S-256 weights dequantised into LDS, epilogue SwiGLU
//   DN_NL4  routed down: A = the expert's rows of a (fp16), B = NL4-32
//           weights dequantised into LDS, epilogue fp32 store (permuted rows)
//   UG_BF16 shared up|gate (bf16 x bf16), epilogue SwiGLU
//   DN_BF16 shared down (bf16 x bf16), epilogue fp32 store
//   ROUTER  router logits (bf16 x bf16), epilogue fp32 store + bias
// Tile 128 x 128 x 64, 256 threads = 2 x 2 waves of 64 x 64, 32x32x16 MFMA,
// double-buffered LDS with a 16-byte XOR swizzle, one barrier per K step.
//
// Numerics: Q3S weights enter the matrix cores as s*c (an fp16 integer,
// |s*c| <= 1016, exact) and d/128 is applied in fp32 to the partial sum of
// each 256-weight block, so up|gate use the exact weights.  NL4 weights enter
// as fp16_rne(d * T4[q] / 128) (one rounding, relative error <= 2^-11).
//
// Layer: "Avalon" README, opening paragraphs; model card "Qwen3.8-Flash-Next
// - Avalon GGUF", "Files / Main model" (codecs, up | gate | down packing).
#include "moe_kernels.hpp"

namespace moe {

typedef _Float16 h2g __attribute__((ext_vector_type(2)));

enum GemmMode { UG_Q3 = 0, DN_NL4 = 1, UG_BF16 = 2, DN_BF16 = 3, ROUTER = 4 };

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int kRowChunks = BK / 8;       // 16-byte chunks per LDS row

struct GemmArgs {
    const uint8_t* experts;
    int64_t estride;
    const int32_t* tiles;
    const int32_t* ntiles;
    int max_tiles;           // M tiles covered by the grid
    const int32_t* perm;
    int k;                   // top-k (token of a permuted row = perm / k)
    const uint16_t* A;       // x16 / a16_perm / x / a_sh
    int lda;                 // row length of A (elements) = K
    int T;                   // tokens (shared / router row count)
    const uint16_t* Bw;      // bf16 weights (shared / router)
    int N;                   // output columns (GEMM N)
    int K;                   // reduction length
    int half_n;              // up|gate: rows of the up half (I or I_s)
    int H, I;                // layer shape (routed record layout)
    const float* bias;       // router bias or null
    uint16_t* out16;         // a16_perm / a_sh
    float* out32;            // y_perm / y_sh / logits
    int ldo;                 // output row length
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowChunks + (chunk ^ (row & 7)); }

template <int MODE>
__global__ void __launch_bounds__(256, 2) k_gemm(GemmArgs g) {
    __shared__ u32x4 As[2][BM * kRowChunks];
    __shared__ u32x4 Bs[2][BN * kRowChunks];
    __shared__ uint32_t lut[256];
    __shared__ float ds_d[2][BN];

    constexpr bool kQ3 = MODE == UG_Q3;
    constexpr bool kNL = MODE == DN_NL4;
    constexpr bool kSwi = MODE == UG_Q3 || MODE == UG_BF16;
    constexpr bool kRouted = MODE == UG_Q3 || MODE == DN_NL4;
    constexpr bool kF16 = MODE == UG_Q3 || MODE == DN_NL4;

    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // ---- tile coordinates (XCD-aware: the N tiles of one M tile share an XCD)
    const int NT = (g.N + BN - 1) / BN;
    const int bid = blockIdx.x, xcd = bid & 7, li = bid >> 3;
    const int mt = (li / NT) * 8 + xcd, nt = li % NT;
    int row0, rows, e = 0;
    if (kRouted) {
        if (mt >= *g.ntiles) return;
        e = g.tiles[3 * mt];
        row0 = g.tiles[3 * mt + 1];
        rows = g.tiles[3 * mt + 2];
    } else {
        row0 = mt * BM;
        if (row0 >= g.T) return;
        rows = min(BM, g.T - row0);
    }

    // ---- per-thread A rows (4 chunks: rows (tid>>3) + 32 i, chunk tid & 7)
    const int ach = tid & 7;
    const uint16_t* arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        if (r < rows) {
            int64_t src;
            if (MODE == UG_Q3) src = (int64_t)(g.perm[row0 + r] / g.k);
            else src = row0 + r;
            arow[i] = g.A + src * g.lda + ach * 8;
        } else {
            arow[i] = nullptr;
        }
    }

    // ---- B rows
    // SwiGLU modes: tile row rr -> output o = nt*64 + (rr>>6)*32 + (rr&31);
    // weight row o (up, (rr>>5)&1 == 0) or half_n + o (gate).
    auto wrow_of = [&](int rr) -> int {
        if (kSwi) {
            const int o = nt * 64 + (rr >> 6) * 32 + (rr & 31);
            return ((rr >> 5) & 1) ? g.half_n + o : o;
        }
        return nt * BN + rr;
    };
    // bf16 modes: 4 chunks per thread like A
    const uint16_t* brow[4];
    // quantized modes: one sub-block (Q3) / block (NL4) per thread: row tid>>1, part tid&1
    const uint8_t* qrow = nullptr;
    const int qrr = tid >> 1, qsub = tid & 1;
    if (kF16) {
        const uint8_t* W = g.experts + (int64_t)e * g.estride;
        if (kQ3) {
            const int64_t rb = (int64_t)(g.H / kQ3Weights) * kQ3Bytes;
            qrow = W + (int64_t)wrow_of(qrr) * rb;
        } else {
            const int64_t rb = (int64_t)(g.I / 32) * kNL4Bytes;
            const int64_t ug = (int64_t)2 * g.I * (g.H / kQ3Weights) * kQ3Bytes;
            qrow = W + ug + (int64_t)wrow_of(qrr) * rb;
        }
        // LUT: Q3 pair -> (C3[lo], C3[hi]); NL4 byte -> (T4[lo]/128, T4[hi]/128)
        if (kQ3) {
            if (tid < 64)
                lut[tid] = pack2(f32_to_f16_bits((float)kC3[tid & 7]), f32_to_f16_bits((float)kC3[tid >> 3]));
        } else {
            lut[tid] = pack2(f32_to_f16_bits((float)kT4[tid & 15] * 0.0078125f),
                             f32_to_f16_bits((float)kT4[tid >> 4] * 0.0078125f));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = (tid >> 3) + 32 * i;
            const int wr = wrow_of(rr);
            brow[i] = (kSwi || wr < g.N) ? g.Bw + (int64_t)wr * g.K + ach * 8 : nullptr;
        }
    }

    // ---- staging registers
    u32x4 ra[4], rb4[4];
    uint32_t qi[5];
    uint64_t qt = 0;

    auto load_a = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = arow[i] ? ld16(arow[i] + kt * BK) : zero;
    };
    auto load_b = [&](int kt) {
        if (kQ3) {
            const int j = 2 * kt + qsub;                 // sub-block index along the row
            const int b = j >> 3, js = j & 7;
            const uint8_t* p = qrow + b * kQ3Bytes;
            qi[0] = ld4(p + 12 * js);
            qi[1] = ld4(p + 12 * js + 4);
            qi[2] = ld4(p + 12 * js + 8);
            qt = *reinterpret_cast<const uint64_t*>(p + 96);
        } else if (kNL) {
            const int j = 2 * kt + qsub;                 // NL4 block index along the row
            const uint8_t* p = qrow + 18 * j - ((j & 1) ? 2 : 0);
#pragma unroll
            for (int u = 0; u < 5; ++u) qi[u] = ld4(p + 4 * u);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) rb4[i] = brow[i] ? ld16_stream(brow[i] + kt * BK) : zero;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) As[buf][swz((tid >> 3) + 32 * i, ach)] = ra[i];
    };
    auto store_b = [&](int buf, int kt) {
        if (kQ3) {
            const int js = (2 * kt + qsub) & 7;
            const _Float16 s = (_Float16)(float)q3_tail_s(qt, js);
            const h2g s2 = {s, s};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 v;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int P = 24 * c + 6 * p;
                    uint32_t pr;
                    if ((P & 31) <= 26) pr = (qi[P >> 5] >> (P & 31)) & 63u;
                    else pr = __builtin_amdgcn_alignbit(qi[(P >> 5) + 1], qi[P >> 5], P & 31) & 63u;
                    v[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2g, lut[pr]) * s2);
                }
                Bs[buf][swz(qrr, qsub * 4 + c)] = v;
            }
            if (qsub == 0) ds_d[buf][qrr] = q3_tail_d(qt) * 0.0078125f;
        } else if (kNL) {
            const int j = 2 * kt + qsub;
            uint32_t dbits, nb[4];
            if (j & 1) {
                dbits = qi[0] >> 16;
#pragma unroll
                for (int u = 0; u < 4; ++u) nb[u] = qi[u + 1];
            } else {
                dbits = qi[0] & 0xffffu;
#pragma unroll
                for (int u = 0; u < 4; ++u) nb[u] = __builtin_amdgcn_alignbit(qi[u + 1], qi[u], 16);
            }
            const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)dbits);
            const h2g d2 = {d, d};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 v;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    v[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2g, lut[(nb[c] >> (8 * p)) & 255u]) * d2);
                Bs[buf][swz(qrr, qsub * 4 + c)] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) Bs[buf][swz((tid >> 3) + 32 * i, ach)] = rb4[i];
        }
    };

    f32x16 acc[2][2], tmp[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[a][b][r] = 0.f;
                tmp[a][b][r] = 0.f;
            }

    const int nk = g.K / BK;
    if (kF16) __syncthreads();                 // LUT ready
    load_a(0);
    load_b(0);
    store_a(0);
    store_b(0, 0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_a(kt + 1);
            load_b(kt + 1);
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            u32x4 fa[2], fb[2];
            const int ch = 2 * kk + (lane >> 5);
#pragma unroll
            for (int sm = 0; sm < 2; ++sm) fa[sm] = As[cur][swz(wm * 64 + sm * 32 + (lane & 31), ch)];
#pragma unroll
            for (int sn = 0; sn < 2; ++sn) fb[sn] = Bs[cur][swz(wn * 64 + sn * 32 + (lane & 31), ch)];
#pragma unroll
            for (int sm = 0; sm < 2; ++sm)
#pragma unroll
                for (int sn = 0; sn < 2; ++sn) {
                    if (kQ3) tmp[sm][sn] = mfma32_f16(fa[sm], fb[sn], tmp[sm][sn]);
                    else if (kF16) acc[sm][sn] = mfma32_f16(fa[sm], fb[sn], acc[sm][sn]);
                    else acc[sm][sn] = mfma32_bf16(fa[sm], fb[sn], acc[sm][sn]);
                }
        }
        if (kQ3 && (kt & 3) == 3) {             // end of a 256-weight block: apply d/128
#pragma unroll
            for (int sn = 0; sn < 2; ++sn) {
                const float dcol = ds_d[cur][wn * 64 + sn * 32 + (lane & 31)];
#pragma unroll
                for (int sm = 0; sm < 2; ++sm)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc[sm][sn][r] += tmp[sm][sn][r] * dcol;
                        tmp[sm][sn][r] = 0.f;
                    }
            }
        }
        if (kt + 1 < nk) {
            store_a(cur ^ 1);
            store_b(cur ^ 1, kt + 1);
        }
        __syncthreads();
    }

    // ---- epilogue.  Lane l, register r of sub-tile (sm, sn): row
    // wm*64 + sm*32 + 8(r/4) + 4(l/32) + r%4, column (l & 31) of the sub-tile.
    const int lc = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int sm = 0; sm < 2; ++sm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = wm * 64 + sm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (m >= rows) continue;
            if (kSwi) {
                const int o = nt * 64 + wn * 32 + lc;
                const float u = acc[sm][0][r], gv = acc[sm][1][r];
                const uint32_t bf = f32_to_bf16(gv / (1.0f + expf(-gv)) * u);
                const uint16_t v = kF16 ? (uint16_t)f32_to_f16_bits(bf16_to_f32(bf)) : (uint16_t)bf;
                g.out16[(int64_t)(row0 + m) * g.ldo + o] = v;
            } else {
#pragma unroll
                for (int sn = 0; sn < 2; ++sn) {
                    const int n = nt * BN + wn * 64 + sn * 32 + lc;
                    if (n < g.N) {
                        float v = acc[sm][sn][r];
                        if (MODE == ROUTER && g.bias) v += g.bias[n];
                        g.out32[(int64_t)(row0 + m) * g.ldo + n] = v;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launchers

static unsigned gemm_grid(int n_cols, int m_tiles) {
    const int NT = (n_cols + BN - 1) / BN;
    const int MTp = ((m_tiles + 7) / 8) * 8;
    return (unsigned)(NT * MTp);
}

void launch_gemm_router(const uint16_t* x, int T, int H, int E, const uint16_t* w_r,
                        const float* bias, float* logits, hipStream_t st) {
    GemmArgs a{};
    a.A = x; a.lda = H; a.T = T; a.Bw = w_r; a.N = E; a.K = H; a.bias = bias;
    a.out32 = logits; a.ldo = E;
    const int mtiles = (T + BM - 1) / BM;
    k_gemm<ROUTER><<<gemm_grid(E, mtiles), 256, 0, st>>>(a);
}

void launch_gemm_upgate(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                        const int32_t* ntiles, int max_tiles, const int32_t* perm, int k,
                        const uint16_t* x16, int H, int I, uint16_t* a16_perm, hipStream_t st) {
    GemmArgs a{};
    a.experts = experts; a.estride = estride; a.tiles = tiles; a.ntiles = ntiles;
    a.max_tiles = max_tiles; a.perm = perm; a.k = k; a.A = x16; a.lda = H;
    a.N = 2 * I; a.K = H; a.half_n = I; a.H = H; a.I = I; a.out16 = a16_perm; a.ldo = I;
    k_gemm<UG_Q3><<<gemm_grid(2 * I, max_tiles), 256, 0, st>>>(a);
}

void launch_gemm_down(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                      const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int H,
                      int I, float* y_perm, hipStream_t st) {
    GemmArgs a{};
    a.experts = experts; a.estride = estride; a.tiles = tiles; a.ntiles = ntiles;
    a.max_tiles = max_tiles; a.A = a16_perm; a.lda = I; a.N = H; a.K = I; a.H = H; a.I = I;
    a.out32 = y_perm; a.ldo = H;
    k_gemm<DN_NL4><<<gemm_grid(H, max_tiles), 256, 0, st>>>(a);
}

void launch_gemm_shared(const uint16_t* x, int T, int H, const uint16_t* sh_ug,
                        const uint16_t* sh_down, int Is, uint16_t* a_sh, float* y_sh,
                        hipStream_t st) {
    const int mtiles = (T + BM - 1) / BM;
    GemmArgs a{};
    a.A = x; a.lda = H; a.T = T; a.Bw = sh_ug; a.N = 2 * Is; a.K = H; a.half_n = Is;
    a.out16 = a_sh; a.ldo = Is;
    k_gemm<UG_BF16><<<gemm_grid(2 * Is, mtiles), 256, 0, st>>>(a);
    GemmArgs b{};
    b.A = a_sh; b.lda = Is; b.T = T; b.Bw = sh_down; b.N = H; b.K = Is; b.out32 = y_sh; b.ldo = H;
    k_gemm<DN_BF16><<<gemm_grid(H, mtiles), 256, 0, st>>>(b);
}

}  // namespace moe
