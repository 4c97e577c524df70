// Bandwidth path of the layer (T <= 16 tokens): every weight byte of the
// router, of each routed expert hit by the batch and of the shared expert is
// streamed from HBM once, in four launches:
//   1. router partial logits + shared-expert up|gate (both need only x),
//   2. routing + counting sort (moe_kernels_small.hip),
//   3. routed up|gate + SwiGLU (weight rows staged through LDS),
//   4. down projections (routed + shared) fused with the weighted combine.
// The matrix cores do the arithmetic (16x16x32 steps); decoding costs one
// table lookup per pair of weights, from tables replicated once per LDS bank
// so that random indices never conflict.
//
// Layer: "Avalon" README, opening paragraphs (10 of 512 experts per token);
// model card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model"
// (routers and shared experts in the dense part; routed up/gate 3.25 bpw,
// down IQ4_NL; expert records packed up | gate | down).
#include <mutex>

#include "moe_kernels.hpp"

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---------------------------------------------------------------- stage 1
// Items [0, n_r): router partial logits over one 256-wide K chunk,
// part[kc][t][e]; 8 waves, one 16-expert tile each; A = tokens (bf16, rows
// >= T zero), B = W_r rows.  Items [n_r, ...): shared expert, 16 up rows and
// the 16 matching gate rows, waves splitting K; a_sh = bf16(silu(g) * u).
__global__ void __launch_bounds__(512) k_dec_stage1(const uint16_t* __restrict__ x, int T, int H,
                                                    int E, const uint16_t* __restrict__ w_r,
                                                    float* __restrict__ part, int n_r,
                                                    const uint16_t* __restrict__ sh_ug, int Is,
                                                    uint16_t* __restrict__ a_sh) {
    __shared__ f32x4 red[8][2][64];
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool vt = r < T;
    const int item = blockIdx.x;

    if (item < n_r) {
        const int n_et = (E + 127) / 128;
        const int et = item % n_et, kc = item / n_et;
        const int e0 = (et * 8 + w) * 16;
        if (e0 >= E) return;
        const int e = e0 + r;
        const bool ve = e < E;
        const uint16_t* brow = w_r + (int64_t)(ve ? e : 0) * H + kc * kRouterKChunk + 8 * g;
        const uint16_t* arow = x + (int64_t)(vt ? r : 0) * H + kc * kRouterKChunk + 8 * g;
        u32x4 a[8], b[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            a[s] = vt ? ld16(arow + 32 * s) : zero;
            b[s] = ve ? ld16_stream(brow + 32 * s) : zero;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma16_bf16(a[s], b[s], acc);
        float* pp = part + (int64_t)kc * T * E;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < T && ve) pp[(int64_t)m * E + e] = acc[i];
        }
        return;
    }

    const int n0 = (item - n_r) * 16;
    const uint16_t* urow = sh_ug + (int64_t)(n0 + r) * H + 8 * g;
    const uint16_t* grow = sh_ug + (int64_t)(Is + n0 + r) * H + 8 * g;
    const uint16_t* xrow = x + (int64_t)(vt ? r : 0) * H + 8 * g;
    f32x4 au = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
    const int nsteps = H / 32;
#pragma unroll 4
    for (int s = w; s < nsteps; s += 8) {
        const u32x4 a = vt ? ld16(xrow + 32 * s) : zero;
        const u32x4 bu = ld16_stream(urow + 32 * s);
        const u32x4 bg = ld16_stream(grow + 32 * s);
        au = mfma16_bf16(a, bu, au);
        ag = mfma16_bf16(a, bg, ag);
    }
    red[w][0][lane] = au;
    red[w][1][lane] = ag;
    __syncthreads();
    if (w == 0) {
        f32x4 u = red[0][0][lane], gg = red[0][1][lane];
#pragma unroll
        for (int v = 1; v < 8; ++v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[i] += red[v][0][lane][i];
                gg[i] += red[v][1][lane][i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < T) a_sh[(int64_t)m * Is + n0 + r] = (uint16_t)f32_to_bf16(silu_mul(gg[i], u[i]));
        }
    }
}

// ---------------------------------------------------------------- up|gate
// One block = (active expert a, 16-column slice): the 16 up rows and the 16
// matching gate rows are staged into LDS with coalesced 8-byte loads, then
// 8 waves split K in groups of 128 (4 sub-blocks).  Lane group g of a
// 16x16x32 step takes one whole 32-weight sub-block (12 index bytes), so the
// B operand of a step spans 4 sub-blocks of one 256-weight block: the
// sub-scale is folded into B exactly (|s*c| <= 1016 is an fp16 integer) and
// the block scale d/128 multiplies the fp32 partial of the group.
// Epilogue: a = bf16_rne(silu(g) * u), stored as fp16 (exact) for the down
// projection.  Dynamic LDS: 32 rows of rb + 8 bytes, then the pair table.
template <int GPW>
__global__ void __launch_bounds__(512) k_upgate_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ x16, int H, int I, uint16_t* __restrict__ a16_perm) {
    extern __shared__ uint8_t dsm[];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int nsl = I / 16;
    const int at = blockIdx.x / nsl;
    const int n0 = (blockIdx.x % nsl) * 16;
    if (at >= *ntiles) return;
    const int e = tiles[3 * at], row0 = tiles[3 * at + 1], rows = tiles[3 * at + 2];

    const int rb = (H / kQ3Weights) * kQ3Bytes;    // bytes per row (multiple of 8)
    const int rbp = rb + 8;                         // padded LDS row
    uint8_t* stage = dsm;
    uint32_t* lut = reinterpret_cast<uint32_t*>(dsm + (32 * rbp > 16384 ? 32 * rbp : 16384));
    f32x4* red = reinterpret_cast<f32x4*>(dsm);     // reuses the staging rows afterwards

    // ---- stage 32 rows (up n0.., then gate I+n0..), both contiguous in memory
    const uint8_t* W = experts + (int64_t)e * estride;
    const uint64_t* src_u = reinterpret_cast<const uint64_t*>(W + (int64_t)n0 * rb);
    const uint64_t* src_g = reinterpret_cast<const uint64_t*>(W + (int64_t)(I + n0) * rb);
    const int qpr = rb / 8, nq = 16 * qpr;
#pragma unroll 8
    for (int q = tid; q < 2 * nq; q += 512) {
        const int half = q >= nq;
        const int qq = half ? q - nq : q;
        const uint64_t v = __builtin_nontemporal_load(half ? src_g + qq : src_u + qq);
        const int row = qq / qpr + 16 * half, col = qq % qpr;
        *reinterpret_cast<uint64_t*>(stage + row * rbp + col * 8) = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 512 * i;
        const int pr = idx >> 5;
        lut[idx] = pack2(f32_to_f16_bits((float)kC3[pr & 7]), f32_to_f16_bits((float)kC3[pr >> 3]));
    }
    // tokens of this expert (rows >= rows stay zero)
    const bool vm = r < rows;
    const int t = vm ? perm[row0 + r] / k : 0;
    const uint16_t* xr = x16 + (int64_t)t * H + 32 * g;
    const int NG = H / 128;
    u32x4 av[GPW][4];
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int q = w + 8 * gi;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[gi][i] = (q < NG && vm) ? ld16(xr + q * 128 + 8 * i) : zero;
    }
    __syncthreads();

    const uint32_t* L = lut + (lane & 31);
    const uint8_t* up = stage + r * rbp;
    const uint8_t* gt = stage + (16 + r) * rbp;
    f32x4 acc_u = {0.f, 0.f, 0.f, 0.f}, acc_g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int q = w + 8 * gi;
        if (q < NG) {
            const int b = q >> 1, js = 4 * (q & 1) + g;
            const int off = b * kQ3Bytes + 12 * js;
            const uint32_t iu[3] = {ld4(up + off), ld4(up + off + 4), ld4(up + off + 8)};
            const uint32_t ig[3] = {ld4(gt + off), ld4(gt + off + 4), ld4(gt + off + 8)};
            const uint64_t tu = *reinterpret_cast<const uint64_t*>(up + b * kQ3Bytes + 96);
            const uint64_t tg = *reinterpret_cast<const uint64_t*>(gt + b * kQ3Bytes + 96);
            const _Float16 su = (_Float16)(float)q3_tail_s(tu, js);
            const _Float16 sg = (_Float16)(float)q3_tail_s(tg, js);
            const h2 su2 = {su, su}, sg2 = {sg, sg};
            f32x4 pu = {0.f, 0.f, 0.f, 0.f}, pg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 bu, bg;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int P = 24 * i + 6 * p;          // bit of the pair in the 96-bit string
                    uint32_t vu, vg;
                    if ((P & 31) <= 26) {
                        vu = (iu[P >> 5] >> (P & 31)) & 63u;
                        vg = (ig[P >> 5] >> (P & 31)) & 63u;
                    } else {
                        vu = __builtin_amdgcn_alignbit(iu[(P >> 5) + 1], iu[P >> 5], P & 31) & 63u;
                        vg = __builtin_amdgcn_alignbit(ig[(P >> 5) + 1], ig[P >> 5], P & 31) & 63u;
                    }
                    bu[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, L[vu * 32]) * su2);
                    bg[p] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, L[vg * 32]) * sg2);
                }
                pu = mfma16_f16(av[gi][i], bu, pu);
                pg = mfma16_f16(av[gi][i], bg, pg);
            }
            const float du = q3_tail_d(tu) * 0.0078125f;
            const float dg = q3_tail_d(tg) * 0.0078125f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc_u[i] += pu[i] * du;
                acc_g[i] += pg[i] * dg;
            }
        }
    }
    __syncthreads();                                   // staging rows are free again
    red[(w * 2 + 0) * 64 + lane] = acc_u;
    red[(w * 2 + 1) * 64 + lane] = acc_g;
    __syncthreads();
    if (w == 0) {
        f32x4 u = red[lane], gg = red[64 + lane];
#pragma unroll
        for (int v = 1; v < 8; ++v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[i] += red[(v * 2) * 64 + lane][i];
                gg[i] += red[(v * 2 + 1) * 64 + lane][i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < rows) {
                const uint32_t bf = f32_to_bf16(silu_mul(gg[i], u[i]));
                a16_perm[(int64_t)(row0 + m) * I + n0 + r] = (uint16_t)f32_to_f16_bits(bf16_to_f32(bf));
            }
        }
    }
}

// ---------------------------------------------------------------- down + combine
// One block = 16 output rows n0.. of y, all tokens.  The M = 16 rows of each
// 16x16x32 step are the tokens themselves: for routed expert e, token t's A
// row is its activation a (permuted row tok_slot[t], zero if t did not pick
// e), so the step yields D[t][n] = (W_down[e] a_t)[n] and the combine is an
// in-register y[t] += w[t][e] * D[t].  Waves take the active experts
// round-robin (and the shared expert's K steps); their partial y are summed
// in wave order, so the result is deterministic.  Each NL4 block is one
// step: B = table integers T4[q] (exact fp16), the block scale d/128
// multiplies the fp32 partial.  Weight rows of the next expert are loaded
// (coalesced dwords) while the current one is decoded from LDS.
constexpr int kDnRowDw = 73;                      // 72 dwords per 16-block row chunk + 1 pad

struct DownPrefetch {
    uint32_t bw[18];
    u32x4 av[16];
    f32x4 wt;
};

__global__ void __launch_bounds__(512) k_down_comb_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const int32_t* __restrict__ tok_slot,
    const float* __restrict__ tok_w, const uint16_t* __restrict__ a16_perm, int T, int H, int I,
    const uint16_t* __restrict__ sh_down, const uint16_t* __restrict__ a_sh, int Is,
    float* __restrict__ y) {
    __shared__ uint32_t lut[256 * 32];             // byte -> (T4[lo], T4[hi]) fp16
    __shared__ uint32_t wbuf[8][16 * kDnRowDw];
    __shared__ f32x4 red[8][64];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int n0 = blockIdx.x * 16;

    for (int idx = tid; idx < 256 * 32; idx += 512) {
        const int byte = idx >> 5;
        lut[idx] = pack2(f32_to_f16_bits((float)kT4[byte & 15]), f32_to_f16_bits((float)kT4[byte >> 4]));
    }
    f32x4 yacc = {0.f, 0.f, 0.f, 0.f};

    // shared expert (weight 1): K steps w, w+8, ...
    if (sh_down) {
        const bool vt = r < T;
        const uint16_t* brow = sh_down + (int64_t)(n0 + r) * Is + 8 * g;
        const uint16_t* arow = a_sh + (int64_t)(vt ? r : 0) * Is + 8 * g;
#pragma unroll 2
        for (int s = w; s < Is / 32; s += 8) {
            const u32x4 a = vt ? ld16(arow + 32 * s) : zero;
            yacc = mfma16_bf16(a, ld16_stream(brow + 32 * s), yacc);
        }
    }
    __syncthreads();                                // table ready

    const int nt = *ntiles;
    const int nb = I / 32;
    const int ncb = (nb + 15) / 16;                 // K chunks of <= 16 blocks (I % 64 == 0: even)
    const int64_t rb = (int64_t)nb * kNL4Bytes;
    const int64_t ug_bytes = (int64_t)2 * I * (H / kQ3Weights) * kQ3Bytes;
    const int nitems = ((nt - w + 7) / 8) * ncb;    // this wave's (expert, chunk) items

    auto load = [&](int it, DownPrefetch& pf) {
        const int a = w + 8 * (it / ncb), c = it % ncb;
        const int cb = min(16, nb - 16 * c);
        const int dpr = cb * kNL4Bytes / 4;        // dwords per row in this chunk
        const uint32_t rcp = ((1u << 20) + dpr - 1) / dpr;   // j / dpr exact for j < 1152
        const int e = tiles[3 * a];
        const uint8_t* base = experts + (int64_t)e * estride + ug_bytes + (int64_t)n0 * rb + 288 * c;
#pragma unroll
        for (int i = 0; i < 18; ++i) {
            const int j = lane + 64 * i;
            const int row = (int)(((uint32_t)j * rcp) >> 20), col = j - row * dpr;
            pf.bw[i] = (j < 16 * dpr) ? __builtin_nontemporal_load(
                                            reinterpret_cast<const uint32_t*>(base + row * rb) + col)
                                      : 0u;
        }
        const int p = (r < T) ? tok_slot[16 * a + r] : -1;
        const uint16_t* arow = a16_perm + (int64_t)(p < 0 ? 0 : p) * I + 512 * c + 8 * g;
#pragma unroll
        for (int b = 0; b < 16; ++b) pf.av[b] = (p >= 0 && b < cb) ? ld16(arow + 32 * b) : zero;
#pragma unroll
        for (int i = 0; i < 4; ++i) pf.wt[i] = tok_w[16 * a + 4 * g + i];
    };

    DownPrefetch cur, nxt;
    if (nitems > 0) load(0, cur);
    f32x4 eacc = {0.f, 0.f, 0.f, 0.f};
    uint32_t* wb = wbuf[w];
    const uint32_t* L = lut + (lane & 31);
    for (int it = 0; it < nitems; ++it) {
        const int c = it % ncb;
        const int cb = min(16, nb - 16 * c);
        const int dpr = cb * kNL4Bytes / 4;
        const uint32_t rcp = ((1u << 20) + dpr - 1) / dpr;
#pragma unroll
        for (int i = 0; i < 18; ++i) {
            const int j = lane + 64 * i;
            const int row = (int)(((uint32_t)j * rcp) >> 20), col = j - row * dpr;
            if (j < 16 * dpr) wb[row * kDnRowDw + col] = cur.bw[i];
        }
        if (it + 1 < nitems) load(it + 1, nxt);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const uint32_t* wr = wb + r * kDnRowDw;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            if (b < cb) {
                const int o = 18 * b + 2 + 4 * g;          // index bytes of lane group g
                const uint32_t nib = (b & 1) ? wr[o >> 2]
                                             : __builtin_amdgcn_alignbit(wr[(o >> 2) + 1], wr[o >> 2], 16);
                const uint32_t dw = wr[(18 * b) >> 2];
                const float d = f16_bits_to_f32((b & 1) ? (dw >> 16) : (dw & 0xffffu)) * 0.0078125f;
                u32x4 bv;
#pragma unroll
                for (int p = 0; p < 4; ++p) bv[p] = L[((nib >> (8 * p)) & 255u) * 32];
                const f32x4 part = mfma16_f16(cur.av[b], bv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) eacc[i] += part[i] * d;
            }
        }
        if (c == ncb - 1) {                          // expert done: weighted combine
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yacc[i] += cur.wt[i] * eacc[i];
                eacc[i] = 0.f;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (it + 1 < nitems) cur = nxt;
    }

    red[w][lane] = yacc;
    __syncthreads();
    if (w == 0) {
        f32x4 s = red[0][lane];
#pragma unroll
        for (int v = 1; v < 8; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] += red[v][lane][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < T) y[(int64_t)m * H + n0 + r] = s[i];
        }
    }
}

// ---------------------------------------------------------------- launchers

void launch_dec_stage1(const uint16_t* x, int T, int H, int E, const uint16_t* w_r, float* part,
                       const uint16_t* sh_ug, int Is, uint16_t* a_sh, hipStream_t st) {
    const int n_r = w_r ? ((E + 127) / 128) * (H / kRouterKChunk) : 0;
    const int n_s = (sh_ug && Is > 0) ? Is / 16 : 0;
    if (n_r + n_s == 0) return;
    k_dec_stage1<<<n_r + n_s, 512, 0, st>>>(x, T, H, E, w_r, part, n_r, sh_ug, Is, a_sh);
}

template <int GPW>
static void upgate_dec_t(unsigned grid, size_t lds, hipStream_t st, const uint8_t* experts,
                         int64_t estride, const int32_t* tiles, const int32_t* ntiles,
                         const int32_t* perm, int k, const uint16_t* x16, int H, int I,
                         uint16_t* a16_perm) {
    static std::once_flag once;
    std::call_once(once, [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_upgate_dec<GPW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    });
    k_upgate_dec<GPW><<<grid, 512, lds, st>>>(experts, estride, tiles, ntiles, perm, k, x16, H, I,
                                              a16_perm);
}

void launch_upgate_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                       const int32_t* ntiles, int max_tiles, const int32_t* perm, int k,
                       const uint16_t* x16, int T, int H, int I, uint16_t* a16_perm,
                       hipStream_t st) {
    (void)T;
    const unsigned grid = (unsigned)(max_tiles * (I / 16));
    const int rb = (H / kQ3Weights) * kQ3Bytes;
    const size_t stage = (size_t)32 * (rb + 8);
    const size_t lds = (stage > 16384 ? stage : 16384) + 64 * 32 * 4;
    const int gpw = (H / 128 + 7) / 8;
#define MOE_UG(G)                                                                               \
    case G:                                                                                     \
        upgate_dec_t<G>(grid, lds, st, experts, estride, tiles, ntiles, perm, k, x16, H, I,     \
                        a16_perm);                                                              \
        break;
    switch (gpw) {
        MOE_UG(1) MOE_UG(2) MOE_UG(3) MOE_UG(4) MOE_UG(5) MOE_UG(6) MOE_UG(7) MOE_UG(8)
        default: break;
    }
#undef MOE_UG
}

void launch_down_comb_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                          const int32_t* ntiles, const int32_t* tok_slot, const float* tok_w,
                          const uint16_t* a16_perm, int T, int H, int I, const uint16_t* sh_down,
                          const uint16_t* a_sh, int Is, float* y, hipStream_t st) {
    k_down_comb_dec<<<H / 16, 512, 0, st>>>(experts, estride, tiles, ntiles, tok_slot, tok_w,
                                            a16_perm, T, H, I, sh_down, a_sh, Is, y);
}

}  // namespace moe
