// Bandwidth path of the layer (T <= 16 tokens): every weight byte of the
// router, of each routed expert hit by the batch and of the shared expert is
// streamed from HBM once, in four launches:
//   1. router partial logits + shared-expert up|gate (both need only x),
//   2. routing + counting sort (moe_kernels_small.hip),
//   3. routed up|gate + SwiGLU (weight rows staged through LDS),
//   4. down projections (routed + shared), then the weighted combine.
// The matrix cores do the arithmetic (16x16x32 steps); decoding costs one
// table lookup per pair of weights, from tables replicated once per LDS bank
// so that random indices never conflict.
//
// Layer: "Avalon" README, opening paragraphs (10 of 512 experts per token);
// model card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model"
// (routers and shared experts in the dense part; routed up/gate 3.25 bpw,
// down IQ4_NL; expert records packed up | gate | down).
#include "moe_kernels.hpp"

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---------------------------------------------------------------- stage 1
// Wave-sized items, no block-level synchronisation.  Items [0, n_r): router
// partial logits of 16 experts over one 256-wide K chunk, part[kc][t][e].
// Items [n_r, n_r + n_s): shared expert up|gate partials of 16 rows (rows
// 0..Is-1 up, Is..2Is-1 gate) over one K chunk, shp[kc][t][2 Is]; summed and
// passed through SwiGLU by the up|gate kernel.  A = tokens (bf16, rows >= T
// zero), B = bf16 weight rows, 16x16x32 bf16 steps.  The last H/256 waves
// write the fp16 copy of the tokens, one 256-wide K chunk each.
__global__ void __launch_bounds__(512) k_dec_stage1(const uint16_t* __restrict__ x, int T, int H,
                                                    int E, const uint16_t* __restrict__ w_r,
                                                    float* __restrict__ part, int n_r,
                                                    const uint16_t* __restrict__ sh_ug, int Is,
                                                    float* __restrict__ shp, int n_s,
                                                    uint16_t* __restrict__ x16) {
    const int lane = __lane_id();
    const int wi = blockIdx.x * 8 + (int)(threadIdx.x >> 6);
    const int n_x = H / kRouterKChunk;               // waves [n_r + n_s, +n_x): fp16 copy of x
    if (wi >= n_r + n_s && wi < n_r + n_s + n_x) {
        const int k0 = (wi - n_r - n_s) * kRouterKChunk;
        for (int i = lane; i < T * (kRouterKChunk / 4); i += 64) {
            const int t = i / (kRouterKChunk / 4), c = (i % (kRouterKChunk / 4)) * 4;
            const uint2 v = *reinterpret_cast<const uint2*>(x + (int64_t)t * H + k0 + c);
            *reinterpret_cast<uint2*>(x16 + (int64_t)t * H + k0 + c) = make_uint2(
                pack2(f32_to_f16_bits(bf16_to_f32(v.x & 0xffffu)), f32_to_f16_bits(bf16_to_f32(v.x >> 16))),
                pack2(f32_to_f16_bits(bf16_to_f32(v.y & 0xffffu)), f32_to_f16_bits(bf16_to_f32(v.y >> 16))));
        }
        return;
    }
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool vt = r < T;
    const uint16_t* W;
    int rows_total, row0, kc, ld_out;
    float* out;
    if (wi < n_r) {
        const int n_et = (E + 15) / 16;
        row0 = (wi % n_et) * 16;
        kc = wi / n_et;
        W = w_r;
        rows_total = E;
        out = part + (int64_t)kc * T * E;
        ld_out = E;
    } else if (wi < n_r + n_s) {
        const int si = wi - n_r, n_st = 2 * Is / 16;
        row0 = (si % n_st) * 16;
        kc = si / n_st;
        W = sh_ug;
        rows_total = 2 * Is;
        out = shp + (int64_t)kc * T * 2 * Is;
        ld_out = 2 * Is;
    } else {
        return;
    }
    const int row = row0 + r;
    const bool vr = row < rows_total;
    const uint16_t* brow = W + (int64_t)(vr ? row : 0) * H + kc * kRouterKChunk + 8 * g;
    const uint16_t* arow = x + (int64_t)(vt ? r : 0) * H + kc * kRouterKChunk + 8 * g;
    u32x4 a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        a[s] = vt ? ld16(arow + 32 * s) : zero;
        b[s] = vr ? ld16_stream(brow + 32 * s) : zero;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma16_bf16(a[s], b[s], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < T && vr) out[(int64_t)m * ld_out + row] = acc[i];
    }
}

// ---------------------------------------------------------------- up|gate
// Decode table: entry (s, v, c) = (fp16(s*C3[v & 7]), fp16(s*C3[v >> 3])) for
// sub-scale s in [-8, 7], index pair v, and copy c = lane & 7 (8 copies spread
// the random lookups over the LDS banks).  Byte address s'*2048 + v*32 + c*4
// with s' = s + 8, so a pair's six index bits land on the address with one
// shift and one and-or.
constexpr int kQ3Lut = 16 * 64 * 8;               // dwords

__device__ __forceinline__ void build_q3_lut(uint32_t* lut, int tid, int nthr) {
    // one (s, v) entry per step, its 8 copies written as two 16-byte stores
    for (int sv = tid; sv < 16 * 64; sv += nthr) {
        const int sp = sv >> 6, v = sv & 63;
        const float s = (float)(sp - 8);
        const uint32_t val = pack2(f32_to_f16_bits(s * (float)kC3[v & 7]),
                                   f32_to_f16_bits(s * (float)kC3[v >> 3]));
        const u32x4 q = {val, val, val, val};
        reinterpret_cast<u32x4*>(lut)[2 * sv] = q;
        reinterpret_cast<u32x4*>(lut)[2 * sv + 1] = q;
    }
}

// Byte address (bits 5..10) of the index pair starting at bit P of the
// 96-bit index string w[0..2], or-ed onto `base`.
template <int P>
__device__ __forceinline__ uint32_t q3_pair_addr(const uint32_t* w, uint32_t base) {
    constexpr int wd = P >> 5, lo = P & 31;
    uint32_t v;
    if constexpr (lo + 6 > 32) v = __builtin_amdgcn_alignbit(w[wd + 1], w[wd], lo - 5);
    else if constexpr (lo >= 5) v = w[wd] >> (lo - 5);
    else if constexpr (wd > 0) v = __builtin_amdgcn_alignbit(w[wd], w[wd - 1], 27 + lo);
    else v = w[wd] << (5 - lo);
    return (v & 0x7e0u) | base;
}

// One block = an item of 8 waves.  Items [0, n_fin): shared expert finish,
// a_sh[t][o] = bf16(silu(sum_c g) * sum_c u) over the stage-1 chunks (chunk
// order).  Items [n_fin, ...): (active expert a, 16-column slice): the 16 up
// rows and the 16 matching gate rows, waves splitting K in groups of 128
// (4 sub-blocks).  Lane group g of a 16x16x32 step takes one whole 32-weight
// sub-block (12 index bytes), so the B operand of a step spans 4 sub-blocks
// of one 256-weight block: B = s*c from the table (exact fp16 integers,
// |s*c| <= 1016) and the block scale d/128 multiplies the fp32 partial of the
// group.  Epilogue: a = bf16_rne(silu(g) * u), stored as fp16 (exact).
template <int GPW, bool FULL>
__global__ void __launch_bounds__(512) k_upgate_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const int32_t* __restrict__ perm, int k,
    const uint16_t* __restrict__ x16, int T, int H, int I, uint16_t* __restrict__ a16_perm,
    const float* __restrict__ shp, int nkc, int Is, int n_fin, uint16_t* __restrict__ a_sh) {
    __shared__ uint32_t lut[kQ3Lut];
    __shared__ f32x4 red[8][2][64];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    if ((int)blockIdx.x < n_fin) {                 // shared expert: sum partials, SwiGLU
        const int i = blockIdx.x * 512 + tid;
        if (i < T * Is) {
            const int t = i / Is, o = i - t * Is;
            float u = 0.f, gg = 0.f;
            for (int c0 = 0; c0 < nkc; c0 += 8) {      // 16 loads in flight, summed in chunk order
                float pu[8], pg[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float* p = shp + ((int64_t)(c0 + c) * T + t) * 2 * Is;
                    pu[c] = c0 + c < nkc ? p[o] : 0.f;
                    pg[c] = c0 + c < nkc ? p[Is + o] : 0.f;
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    u += pu[c];
                    gg += pg[c];
                }
            }
            a_sh[i] = (uint16_t)f32_to_bf16(silu_mul(gg, u));
        }
        return;
    }
    const int nsl = I / 16;
    const int item = blockIdx.x - n_fin;
    const int at = item / nsl;
    const int n0 = (item - at * nsl) * 16;
    if (at >= *ntiles) return;
    const int e = tiles[3 * at], row0 = tiles[3 * at + 1], rows = tiles[3 * at + 2];

    const int64_t row_bytes = (int64_t)(H / kQ3Weights) * kQ3Bytes;
    const uint8_t* W = experts + (int64_t)e * estride;
    const uint8_t* up = W + (int64_t)(n0 + r) * row_bytes;
    const uint8_t* gt = W + (int64_t)(I + n0 + r) * row_bytes;
    // rows >= rows reuse the first row's token: their results are never stored
    const int t = perm[row0 + (r < rows ? r : 0)] / k;
    const uint16_t* xr = x16 + (int64_t)t * H + 32 * g;
    const int NG = FULL ? 8 * GPW : H / 128;

    // all loads of the item first
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
            for (int i = 0; i < 4; ++i) av[gi][i] = ld16(xr + q * 128 + 8 * i);
        }
    }
    build_q3_lut(lut, tid, 512);
    __syncthreads();

    const uint8_t* Lb = reinterpret_cast<const uint8_t*>(lut);
    const uint32_t cbase = (uint32_t)(lane & 7) * 4u;
    f32x4 acc_u = {0.f, 0.f, 0.f, 0.f}, acc_g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
        const int q = w + 8 * gi;
        if (q < NG) {
            const int js = 4 * (q & 1) + g;
            const uint32_t bu_s = (uint32_t)(q3_tail_s(tu[gi], js) + 8) * 2048u + cbase;
            const uint32_t bg_s = (uint32_t)(q3_tail_s(tg[gi], js) + 8) * 2048u + cbase;
            f32x4 pu = {0.f, 0.f, 0.f, 0.f}, pg = {0.f, 0.f, 0.f, 0.f};
            u32x4 bu[4], bg[4];
#define MOE_PAIR(I_, P_)                                                                  \
    bu[I_][P_] = *reinterpret_cast<const uint32_t*>(Lb + q3_pair_addr<24 * I_ + 6 * P_>(iu[gi], bu_s)); \
    bg[I_][P_] = *reinterpret_cast<const uint32_t*>(Lb + q3_pair_addr<24 * I_ + 6 * P_>(ig[gi], bg_s));
#define MOE_STEP(I_) MOE_PAIR(I_, 0) MOE_PAIR(I_, 1) MOE_PAIR(I_, 2) MOE_PAIR(I_, 3)
            MOE_STEP(0) MOE_STEP(1) MOE_STEP(2) MOE_STEP(3)
#undef MOE_STEP
#undef MOE_PAIR
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pu = mfma16_f16(av[gi][i], bu[i], pu);
                pg = mfma16_f16(av[gi][i], bg[i], pg);
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
    red[w][0][lane] = acc_u;
    red[w][1][lane] = acc_g;
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
            if (m < rows) {
                const uint32_t bf = f32_to_bf16(silu_mul(gg[i], u[i]));
                a16_perm[(int64_t)(row0 + m) * I + n0 + r] = (uint16_t)f32_to_f16_bits(bf16_to_f32(bf));
            }
        }
    }
}

// ---------------------------------------------------------------- down + combine
// One block = 4 waves; wave = 16 output rows.  Items per 64-row slice sl:
// routed (active expert a, sl) and, if present, the shared expert (sl).
// Routed: the wave's 16 down rows (16 x 288 bytes per 16-block K chunk) are
// staged into LDS with coalesced dword loads, then one 16x16x32 step per
// NL4-32 block (lane group g takes 8 weights = 4 index bytes, B = table
// integers T4[q], exact fp16) and the block scale d/128 multiplies the fp32
// partial of the step.  M rows = the expert's permuted rows (<= 16).  Output:
// y_perm (unweighted, permuted rows) or y_sh; the combine kernel sums them.
constexpr int kDnRowDw = 73;                      // 72 dwords per 16-block row chunk + 1 pad

template <bool FULL16>                            // every K chunk has 16 blocks (I % 512 == 0)
__global__ void __launch_bounds__(256) k_down_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, int max_tiles, const uint16_t* __restrict__ a16_perm,
    int T, int H, int I, int k, const uint16_t* __restrict__ sh_down,
    const uint16_t* __restrict__ a_sh, int Is, float* __restrict__ y_perm,
    float* __restrict__ y_sh) {
    __shared__ uint32_t lut[256 * 32];             // byte -> (T4[lo], T4[hi]) fp16, 32 copies
    __shared__ uint32_t wbuf[4][16 * kDnRowDw];
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int nsl = H / 64;
    const int sl = blockIdx.x % nsl;
    const int a = blockIdx.x / nsl;               // 0..max_tiles-1 routed, max_tiles = shared
    const bool is_sh = a == max_tiles;
    if (is_sh ? sh_down == nullptr : a >= *ntiles) return;
    const int n0 = sl * 64 + w * 16;

    if (is_sh) {
        const uint16_t* brow = sh_down + (int64_t)(n0 + r) * Is + 8 * g;
        const uint16_t* arow = a_sh + (int64_t)(r < T ? r : 0) * Is + 8 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int s2 = 0; s2 < Is / 32; ++s2)
            acc = mfma16_bf16(ld16(arow + 32 * s2), ld16_stream(brow + 32 * s2), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < T) y_sh[(int64_t)m * H + n0 + r] = acc[i];
        }
    } else {
        const int e = tiles[3 * a], row0 = tiles[3 * a + 1], rows = tiles[3 * a + 2];
        if (tid < 256) {                           // entry tid, its 32 copies as 8 16-byte stores
            const uint32_t val = pack2(f32_to_f16_bits((float)kT4[tid & 15]),
                                       f32_to_f16_bits((float)kT4[tid >> 4]));
            const u32x4 q = {val, val, val, val};
#pragma unroll
            for (int c = 0; c < 8; ++c) reinterpret_cast<u32x4*>(lut)[8 * tid + c] = q;
        }
        const int nb = I / 32;
        const int64_t rb = (int64_t)nb * kNL4Bytes;
        const int64_t ug_bytes = (int64_t)2 * I * (H / kQ3Weights) * kQ3Bytes;
        const uint8_t* base = experts + (int64_t)e * estride + ug_bytes + (int64_t)n0 * rb;
        // rows >= rows reuse the first row: their results are never stored
        const uint16_t* arow = a16_perm + (int64_t)(row0 + (r < rows ? r : 0)) * I + 8 * g;
        uint32_t* wb = wbuf[w];
        const uint8_t* Lb = reinterpret_cast<const uint8_t*>(lut);
        const uint32_t cb = (uint32_t)(lane & 31) * 4u;   // byte b: address b*128 + copy*4
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        __syncthreads();                           // table ready
        for (int c = 0; c < (nb + 15) / 16; ++c) {  // K chunks of 16 blocks (nb is even)
            const int cbk = FULL16 ? 16 : min(16, nb - 16 * c);
            const int dpr = FULL16 ? 72 : cbk * kNL4Bytes / 4;   // dwords per row in this chunk
            uint32_t bw[18];
#pragma unroll
            for (int i = 0; i < 18; ++i) {
                const int j = lane + 64 * i, row = j / dpr, col = j - dpr * row;
                const bool ok = FULL16 || j < 16 * dpr;
                bw[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const uint32_t*>(base + (ok ? row : 0) * rb + 288 * c) + (ok ? col : 0));
            }
            u32x4 av[16];
#pragma unroll
            for (int b = 0; b < 16; ++b) av[b] = ld16(arow + 512 * c + 32 * (b < cbk ? b : 0));
#pragma unroll
            for (int i = 0; i < 18; ++i) {
                const int j = lane + 64 * i, row = j / dpr, col = j - dpr * row;
                if (FULL16 || j < 16 * dpr) wb[row * kDnRowDw + col] = bw[i];
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const uint32_t* wr = wb + r * kDnRowDw;
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                if (b < cbk) {
                    const int o = 18 * b + 2 + 4 * g;      // index bytes of lane group g
                    const uint32_t nib = (b & 1) ? wr[o >> 2]
                                                 : __builtin_amdgcn_alignbit(wr[(o >> 2) + 1], wr[o >> 2], 16);
                    const uint32_t dw = wr[(18 * b) >> 2];
                    const float d = f16_bits_to_f32((b & 1) ? (dw >> 16) : (dw & 0xffffu)) * 0.0078125f;
                    u32x4 bv;
                    bv[0] = *reinterpret_cast<const uint32_t*>(Lb + (((nib << 7) & 0x7f80u) | cb));
                    bv[1] = *reinterpret_cast<const uint32_t*>(Lb + (((nib >> 1) & 0x7f80u) | cb));
                    bv[2] = *reinterpret_cast<const uint32_t*>(Lb + (((nib >> 9) & 0x7f80u) | cb));
                    bv[3] = *reinterpret_cast<const uint32_t*>(Lb + (((nib >> 17) & 0x7f80u) | cb));
                    const f32x4 part = mfma16_f16(av[b], bv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] += part[i] * d;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < rows) y_perm[(int64_t)(row0 + m) * H + n0 + r] = acc[i];
        }
    }

}

// ---------------------------------------------------------------- launchers

void launch_dec_stage1(const uint16_t* x, int T, int H, int E, const uint16_t* w_r, float* part,
                       const uint16_t* sh_ug, int Is, float* shp, uint16_t* x16, hipStream_t st) {
    const int nkc = H / kRouterKChunk;
    const int n_r = w_r ? ((E + 15) / 16) * nkc : 0;
    const int n_s = (sh_ug && Is > 0) ? (2 * Is / 16) * nkc : 0;
    const int n_x = x16 ? nkc : 0;
    if (n_r + n_s + n_x == 0) return;
    k_dec_stage1<<<(n_r + n_s + n_x + 7) / 8, 512, 0, st>>>(x, T, H, E, w_r, part, n_r, sh_ug, Is,
                                                            shp, n_s, x16);
}

template <int GPW, bool FULL>
static void upgate_dec_t(unsigned grid, hipStream_t st, const uint8_t* experts, int64_t estride,
                         const int32_t* tiles, const int32_t* ntiles, const int32_t* perm, int k,
                         const uint16_t* x16, int T, int H, int I, uint16_t* a16_perm,
                         const float* shp, int nkc, int Is, int n_fin, uint16_t* a_sh) {
    k_upgate_dec<GPW, FULL><<<grid, 512, 0, st>>>(experts, estride, tiles, ntiles, perm, k, x16, T,
                                                  H, I, a16_perm, shp, nkc, Is, n_fin, a_sh);
}

void launch_upgate_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                       const int32_t* ntiles, int max_tiles, const int32_t* perm, int k,
                       const uint16_t* x16, int T, int H, int I, uint16_t* a16_perm,
                       const float* shp, int Is, uint16_t* a_sh, hipStream_t st) {
    const int n_fin = (shp && Is > 0) ? (T * Is + 511) / 512 : 0;
    const unsigned grid = (unsigned)(n_fin + max_tiles * (I / 16));
    const int nkc = H / kRouterKChunk;
    const int gpw = (H / 128 + 7) / 8;
    const bool full = (H / 128) == 8 * gpw;
#define MOE_UG(G)                                                                               \
    case G:                                                                                     \
        if (full)                                                                               \
            upgate_dec_t<G, true>(grid, st, experts, estride, tiles, ntiles, perm, k, x16, T, H, \
                                  I, a16_perm, shp, nkc, Is, n_fin, a_sh);                      \
        else                                                                                    \
            upgate_dec_t<G, false>(grid, st, experts, estride, tiles, ntiles, perm, k, x16, T,  \
                                   H, I, a16_perm, shp, nkc, Is, n_fin, a_sh);                  \
        break;
    switch (gpw) {
        MOE_UG(1) MOE_UG(2) MOE_UG(3) MOE_UG(4) MOE_UG(5) MOE_UG(6) MOE_UG(7) MOE_UG(8)
        default: break;
    }
#undef MOE_UG
}

void launch_down_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                     const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int T, int H,
                     int I, int k, const uint16_t* sh_down, const uint16_t* a_sh, int Is,
                     float* y_perm, float* y_sh, hipStream_t st) {
    const unsigned grid = (unsigned)((max_tiles + 1) * (H / 64));
    if (I % 512 == 0)
        k_down_dec<true><<<grid, 256, 0, st>>>(experts, estride, tiles, ntiles, max_tiles, a16_perm,
                                               T, H, I, k, sh_down, a_sh, Is, y_perm, y_sh);
    else
        k_down_dec<false><<<grid, 256, 0, st>>>(experts, estride, tiles, ntiles, max_tiles, a16_perm,
                                                T, H, I, k, sh_down, a_sh, Is, y_perm, y_sh);
}

}  // namespace moe
