// Bandwidth path of the layer (T <= 16 tokens): every weight byte of the
// router, of each routed expert hit by the batch and of the shared expert is
// streamed from HBM once.  The tokens of one expert (at most T) form the
// M = 16 rows of 16x16x32 matrix-core steps, so the decode cost per weight is
// one table lookup per pair of weights; the arithmetic itself rides on MFMA.
//
// Layer: "Avalon" README, opening paragraphs (10 of 512 experts per token);
// model card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model"
// (routers and shared experts in the dense part; routed up/gate 3.25 bpw,
// down IQ4_NL; expert records packed up | gate | down).
#include "moe_kernels.hpp"

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- router
// Partial logits over one 256-wide K chunk: part[kc][t][e] (bias and the sum
// over chunks are applied by the routing kernel).  Block = 4 waves, one
// 16-expert tile each.  A = tokens (bf16, rows >= T are zero), B = W_r rows.
__global__ void __launch_bounds__(256) k_router_partial(const uint16_t* __restrict__ x, int T,
                                                        int H, int E,
                                                        const uint16_t* __restrict__ w_r,
                                                        float* __restrict__ part) {
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int e0 = (blockIdx.x * 4 + w) * 16;
    if (e0 >= E) return;
    const int kc = blockIdx.y;
    const int e = e0 + r;
    const bool ve = e < E, vt = r < T;
    const uint16_t* brow = w_r + (int64_t)(ve ? e : 0) * H + kc * kRouterKChunk + 8 * g;
    const uint16_t* arow = x + (int64_t)(vt ? r : 0) * H + kc * kRouterKChunk + 8 * g;
    const u32x4 zero = {0u, 0u, 0u, 0u};
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
}

// ---------------------------------------------------------------- up|gate
// One block = one work item of 8 waves.
//  * items [0, n_sh): shared expert, 16 up rows + the 16 matching gate rows,
//    bf16 weights and tokens, all T tokens.
//  * items [n_sh, ...): routed (active expert a, 16-column slice).  Waves
//    split the K dimension in groups of 128 (4 sub-blocks); lane group g of a
//    16x16x32 step takes one whole 32-weight sub-block (12 index bytes), so
//    the B operand of a step spans 4 sub-blocks of one 256-weight block: the
//    sub-scale is folded into B exactly (|s*c| <= 1016 is an fp16 integer) and
//    the block scale d/128 is applied to the fp32 partial of the group.
// Epilogue: a = bf16_rne(silu(g) * u), stored as fp16 (exact) for the
// routed down projection, as bf16 for the shared one.
template <int GPW>
__global__ void __launch_bounds__(512) k_upgate_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ x16, const uint16_t* __restrict__ x, int T, int H, int I,
    const uint16_t* __restrict__ sh_ug, int Is, int n_sh, uint16_t* __restrict__ a16_perm,
    uint16_t* __restrict__ a_sh) {
    __shared__ uint32_t lut[64 * 32];        // pair -> (C3[lo], C3[hi]) fp16, one copy per bank
    __shared__ f32x4 red[8][2][64];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    f32x4 acc_u = {0.f, 0.f, 0.f, 0.f}, acc_g = {0.f, 0.f, 0.f, 0.f};
    const int item = blockIdx.x;
    const bool is_sh = item < n_sh;
    int rows, row0 = 0, n0;

    if (is_sh) {
        n0 = item * 16;
        rows = T;
        const uint16_t* urow = sh_ug + (int64_t)(n0 + r) * H + 8 * g;
        const uint16_t* grow = sh_ug + (int64_t)(Is + n0 + r) * H + 8 * g;
        const bool vt = r < T;
        const uint16_t* xrow = x + (int64_t)(vt ? r : 0) * H + 8 * g;
        const int nsteps = H / 32;
        for (int s = w; s < nsteps; s += 8) {
            const u32x4 a = vt ? ld16(xrow + 32 * s) : zero;
            const u32x4 bu = ld16_stream(urow + 32 * s);
            const u32x4 bg = ld16_stream(grow + 32 * s);
            acc_u = mfma16_bf16(a, bu, acc_u);
            acc_g = mfma16_bf16(a, bg, acc_g);
        }
    } else {
        const int ritem = item - n_sh, nsl = I / 16;
        const int at = ritem / nsl;
        n0 = (ritem % nsl) * 16;
        if (at >= *ntiles) return;
        const int e = tiles[3 * at];
        row0 = tiles[3 * at + 1];
        rows = tiles[3 * at + 2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 512 * i;
            const int pr = idx >> 5;
            lut[idx] = pack2(f32_to_f16_bits((float)kC3[pr & 7]), f32_to_f16_bits((float)kC3[pr >> 3]));
        }
        __syncthreads();

        const int NG = H / 128;
        const int64_t row_bytes = (int64_t)(H / kQ3Weights) * kQ3Bytes;
        const uint8_t* W = experts + (int64_t)e * estride;
        const uint8_t* up = W + (int64_t)(n0 + r) * row_bytes;
        const uint8_t* gt = W + (int64_t)(I + n0 + r) * row_bytes;
        const bool vm = r < rows;
        const int t = vm ? perm[row0 + r] / k : 0;
        const uint16_t* xr = x16 + (int64_t)t * H + 32 * g;
        const uint32_t* L = lut + (lane & 31);

        uint32_t iu[GPW][3], ig[GPW][3];
        uint64_t tu[GPW], tg[GPW];
        u32x4 av[GPW][4];
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int q = w + 8 * gi;
            if (q < NG) {
                const int b = q >> 1, js = 4 * (q & 1) + g;
                const int off = b * kQ3Bytes + 12 * js;
                iu[gi][0] = ld4(up + off);
                iu[gi][1] = ld4(up + off + 4);
                iu[gi][2] = ld4(up + off + 8);
                ig[gi][0] = ld4(gt + off);
                ig[gi][1] = ld4(gt + off + 4);
                ig[gi][2] = ld4(gt + off + 8);
                tu[gi] = *reinterpret_cast<const uint64_t*>(up + b * kQ3Bytes + 96);
                tg[gi] = *reinterpret_cast<const uint64_t*>(gt + b * kQ3Bytes + 96);
#pragma unroll
                for (int i = 0; i < 4; ++i) av[gi][i] = vm ? ld16(xr + q * 128 + 8 * i) : zero;
            }
        }
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int q = w + 8 * gi;
            if (q < NG) {
                const int js = 4 * (q & 1) + g;
                const _Float16 su = (_Float16)(float)q3_tail_s(tu[gi], js);
                const _Float16 sg = (_Float16)(float)q3_tail_s(tg[gi], js);
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
                            vu = (iu[gi][P >> 5] >> (P & 31)) & 63u;
                            vg = (ig[gi][P >> 5] >> (P & 31)) & 63u;
                        } else {
                            vu = __builtin_amdgcn_alignbit(iu[gi][(P >> 5) + 1], iu[gi][P >> 5], P & 31) & 63u;
                            vg = __builtin_amdgcn_alignbit(ig[gi][(P >> 5) + 1], ig[gi][P >> 5], P & 31) & 63u;
                        }
                        const h2 cu = __builtin_bit_cast(h2, L[vu * 32]) * su2;
                        const h2 cg = __builtin_bit_cast(h2, L[vg * 32]) * sg2;
                        bu[p] = __builtin_bit_cast(uint32_t, cu);
                        bg[p] = __builtin_bit_cast(uint32_t, cg);
                    }
                    pu = mfma16_f16(av[gi][i], bu, pu);
                    pg = mfma16_f16(av[gi][i], bg, pg);
                }
                const float du = q3_tail_d(tu[gi]) * 0.0078125f;
                const float dg = q3_tail_d(tg[gi]) * 0.0078125f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc_u[i] += pu[i] * du;
                    acc_g[i] += pg[i] * dg;
                }
            }
        }
    }

    red[w][0][lane] = acc_u;
    red[w][1][lane] = acc_g;
    __syncthreads();
    if (w == 0) {
        f32x4 u = red[0][0][lane], gg = red[0][1][lane];
#pragma unroll
        for (int v = 1; v < 8; ++v) {
            const f32x4 a = red[v][0][lane], b = red[v][1][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[i] += a[i];
                gg[i] += b[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < rows) {
                const float gv = gg[i];
                const float act = gv / (1.0f + expf(-gv)) * u[i];
                const uint32_t bf = f32_to_bf16(act);
                if (is_sh)
                    a_sh[(int64_t)m * Is + n0 + r] = (uint16_t)bf;
                else
                    a16_perm[(int64_t)(row0 + m) * I + n0 + r] = (uint16_t)f32_to_f16_bits(bf16_to_f32(bf));
            }
        }
    }
}

// ---------------------------------------------------------------- down
// One block = 4 waves; wave = 16 output rows.  Items [0, n_sh): shared
// expert (bf16 weights, bf16 activations); then (active expert, 64 rows).
// Routed: one 16x16x32 step per NL4-32 block (lane group g takes 8 weights =
// 4 index bytes), B = table integers T4[q] (exact fp16), and the block scale
// d/128 multiplies the fp32 partial of the step: the result is exact up to
// fp32 accumulation.
__global__ void __launch_bounds__(256) k_down_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const uint16_t* __restrict__ a16_perm, int T, int H,
    int I, const uint16_t* __restrict__ sh_down, const uint16_t* __restrict__ a_sh, int Is,
    int n_sh, float* __restrict__ y_perm, float* __restrict__ y_sh) {
    __shared__ uint32_t lut[256 * 32];       // byte -> (T4[lo], T4[hi]) fp16, one copy per bank
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int item = blockIdx.x;

    if (item < n_sh) {
        const int n0 = item * 64 + w * 16;
        const uint16_t* brow = sh_down + (int64_t)(n0 + r) * Is + 8 * g;
        const bool vt = r < T;
        const uint16_t* arow = a_sh + (int64_t)(vt ? r : 0) * Is + 8 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < Is / 32; ++s) {
            const u32x4 a = vt ? ld16(arow + 32 * s) : zero;
            const u32x4 b = ld16_stream(brow + 32 * s);
            acc = mfma16_bf16(a, b, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < T) y_sh[(int64_t)m * H + n0 + r] = acc[i];
        }
        return;
    }

    const int ritem = item - n_sh, nsl = H / 64;
    const int at = ritem / nsl;
    if (at >= *ntiles) return;
    const int n0 = (ritem % nsl) * 64 + w * 16;
    const int e = tiles[3 * at], row0 = tiles[3 * at + 1], rows = tiles[3 * at + 2];
    for (int idx = tid; idx < 256 * 32; idx += 256) {
        const int byte = idx >> 5;
        lut[idx] = pack2(f32_to_f16_bits((float)kT4[byte & 15]), f32_to_f16_bits((float)kT4[byte >> 4]));
    }
    __syncthreads();

    const int nb = I / 32;
    const int64_t rb = (int64_t)nb * kNL4Bytes;
    const int64_t ug_bytes = (int64_t)2 * I * (H / kQ3Weights) * kQ3Bytes;
    const uint8_t* row = experts + (int64_t)e * estride + ug_bytes + (int64_t)(n0 + r) * rb;
    const bool vm = r < rows;
    const uint16_t* arow = a16_perm + (int64_t)(row0 + (vm ? r : 0)) * I + 8 * g;
    const uint32_t* L = lut + (lane & 31);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < nb; ++b) {
        // index bytes [18b + 2 + 4g, +4): 4-aligned for odd b, 2 mod 4 for even b
        const uint8_t* ip = row + 18 * b + 2 + 4 * g;
        uint32_t nib;
        if (b & 1) {
            nib = ld4(ip);
        } else {
            const uint32_t lo = ld4(ip - 2), hi = ld4(ip + 2);
            nib = __builtin_amdgcn_alignbit(hi, lo, 16);
        }
        const uint32_t dw = ld4(row + 18 * b - ((b & 1) ? 2 : 0));
        const float d = f16_bits_to_f32((b & 1) ? (dw >> 16) : (dw & 0xffffu)) * 0.0078125f;
        u32x4 bv;
#pragma unroll
        for (int p = 0; p < 4; ++p) bv[p] = L[((nib >> (8 * p)) & 255u) * 32];
        const u32x4 a = vm ? ld16(arow + 32 * b) : zero;
        const f32x4 part = mfma16_f16(a, bv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += part[i] * d;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < rows) y_perm[(int64_t)(row0 + m) * H + n0 + r] = acc[i];
    }
}

// ---------------------------------------------------------------- launchers

void launch_router_partial(const uint16_t* x, int T, int H, int E, const uint16_t* w_r,
                           float* part, hipStream_t st) {
    dim3 grid((E + 63) / 64, H / kRouterKChunk);
    k_router_partial<<<grid, 256, 0, st>>>(x, T, H, E, w_r, part);
}

template <int GPW>
static void upgate_dec_t(dim3 grid, hipStream_t st, const uint8_t* experts, int64_t estride,
                         const int32_t* tiles, const int32_t* ntiles, const int32_t* perm, int k,
                         const uint16_t* x16, const uint16_t* x, int T, int H, int I,
                         const uint16_t* sh_ug, int Is, int n_sh, uint16_t* a16_perm,
                         uint16_t* a_sh) {
    k_upgate_dec<GPW><<<grid, 512, 0, st>>>(experts, estride, tiles, ntiles, perm, k, x16, x, T,
                                            H, I, sh_ug, Is, n_sh, a16_perm, a_sh);
}

void launch_upgate_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                       const int32_t* ntiles, int max_tiles, const int32_t* perm, int k,
                       const uint16_t* x16, const uint16_t* x, int T, int H, int I,
                       const uint16_t* sh_ug, int Is, uint16_t* a16_perm, uint16_t* a_sh,
                       hipStream_t st) {
    const int n_sh = (sh_ug && Is > 0) ? Is / 16 : 0;
    dim3 grid(n_sh + max_tiles * (I / 16));
    const int gpw = (H / 128 + 7) / 8;
#define MOE_UG(G)                                                                               \
    case G:                                                                                     \
        upgate_dec_t<G>(grid, st, experts, estride, tiles, ntiles, perm, k, x16, x, T, H, I,    \
                        sh_ug, Is, n_sh, a16_perm, a_sh);                                       \
        break;
    switch (gpw) {
        MOE_UG(1) MOE_UG(2) MOE_UG(3) MOE_UG(4) MOE_UG(5) MOE_UG(6) MOE_UG(7) MOE_UG(8)
        default: break;
    }
#undef MOE_UG
}

void launch_down_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                     const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int T,
                     int H, int I, const uint16_t* sh_down, const uint16_t* a_sh, int Is,
                     float* y_perm, float* y_sh, hipStream_t st) {
    const int n_sh = (sh_down && Is > 0) ? H / 64 : 0;
    dim3 grid(n_sh + max_tiles * (H / 64));
    k_down_dec<<<grid, 256, 0, st>>>(experts, estride, tiles, ntiles, a16_perm, T, H, I, sh_down,
                                     a_sh, Is, n_sh, y_perm, y_sh);
}

}  // namespace moe
