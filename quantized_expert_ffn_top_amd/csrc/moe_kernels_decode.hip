// Bandwidth path of the layer (T <= 16 tokens): every weight byte of the
// router, of each routed expert hit by the batch and of the shared expert is
// streamed from HBM once, in three launches before the combine:
//   1. router logits + shared-expert up|gate partials (both need only x),
//   2. routing (top-k, softmax, counting sort, redundantly in every block)
//      followed by the routed up|gate + SwiGLU (weight rows staged through
//      LDS) and the shared SwiGLU,
//   3. down projections (routed + shared); the weighted combine follows
//      (moe_kernels_small.hip).
// The matrix cores do the arithmetic (16x16x32 steps); decoding costs one
// table lookup per pair of weights, from tables replicated once per LDS bank
// so that random indices never conflict.
//
// Layer: "Avalon" README, opening paragraphs (10 of 512 experts per token);
// model card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model"
// (routers and shared experts in the dense part; routed up/gate 3.25 bpw,
// down IQ4_NL; expert records packed up | gate | down).
#include <algorithm>

#include "moe_decoders.hpp"
#include "moe_kernels.hpp"

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }
// silu(g) * u from the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g)) * u;
}

// ---------------------------------------------------------------- stage 1
// Blocks of 4 waves, spread over the whole chip.  Blocks [0, n_rb): router
// logits of 16 experts over one of kp equal K parts (block = tile * kp +
// part): the waves split the part in 4 (16x16x32 bf16 steps, A = tokens,
// rows >= T zero; a wave's loads, up to 24 steps, are all in flight at once)
// and their partial sums are added in wave order through LDS.  kp = 1: the
// bias is added last, logits[t][e]; kp > 1: partial planes logits[part][t][e]
// without the bias, summed in part order (then the bias) by the routing.  Blocks [n_rb, ...): wave
// items, no block synchronisation.  Items [0, n_s): shared expert up|gate
// partials of 16 rows (rows 0..Is-1 up, Is..2Is-1 gate) over one 256-wide K
// chunk, shp[kc][t][2 Is]; summed and passed through SwiGLU by the up|gate
// kernel.  The last H/256 wave items write the fp16 copy of the tokens, one
// 256-wide K chunk each.
constexpr int kS1Waves = 4;
constexpr int kS1Batch = 24;                    // K steps in flight per wave
__global__ void __launch_bounds__(64 * kS1Waves) k_dec_stage1(const uint16_t* __restrict__ x, int T, int H,
                                                    int E, const uint16_t* __restrict__ w_r,
                                                    const float* __restrict__ bias,
                                                    float* __restrict__ logits, int n_rb, int kp,
                                                    const uint16_t* __restrict__ sh_ug, int Is,
                                                    float* __restrict__ shp, int n_s,
                                                    uint16_t* __restrict__ x16) {
    __shared__ f32x4 red[kS1Waves][64];
    const int lane = __lane_id(), w = (int)(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool vt = r < T;
    if ((int)blockIdx.x < n_rb) {
        const int tile = blockIdx.x / kp, part = blockIdx.x - tile * kp;
        const int row = tile * 16 + r;
        const bool vr = row < E;
        const int S = H / 32, pa = part * S / kp, pb = (part + 1) * S / kp;
        const int sa = pa + w * (pb - pa) / kS1Waves, sb = pa + (w + 1) * (pb - pa) / kS1Waves;   // this wave's K steps
        const uint16_t* brow = w_r + (int64_t)(vr ? row : 0) * H + 8 * g;
        const uint16_t* arow = x + (int64_t)(vt ? r : 0) * H + 8 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = sa; s0 < sb; s0 += kS1Batch) {
            u32x4 a[kS1Batch], b[kS1Batch];
#pragma unroll
            for (int s = 0; s < kS1Batch; ++s) {
                const bool ok = s0 + s < sb;
                a[s] = (vt && ok) ? ld16(arow + 32 * (s0 + s)) : zero;
                b[s] = (vr && ok) ? ld16_stream(brow + 32 * (s0 + s)) : zero;
            }
#pragma unroll
            for (int s = 0; s < kS1Batch; ++s) acc = mfma16_bf16(a[s], b[s], acc);
        }
        red[w][lane] = acc;
        __syncthreads();
        if (w == 0) {
            f32x4 sum = red[0][lane];
#pragma unroll
            for (int v = 1; v < kS1Waves; ++v)
#pragma unroll
                for (int i = 0; i < 4; ++i) sum[i] += red[v][lane][i];
            const float bb = (vr && bias && kp == 1) ? bias[row] : 0.f;
            float* out = logits + (int64_t)part * T * E;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * g + i;
                if (m < T && vr) out[(int64_t)m * E + row] = sum[i] + bb;
            }
        }
        return;
    }
    const int wi = (blockIdx.x - n_rb) * kS1Waves + w;
    const int n_x = H / kShKChunk;               // waves [n_s, n_s + n_x): fp16 copy of x
    if (wi >= n_s) {
        if (wi >= n_s + n_x) return;
        const int k0 = (wi - n_s) * kShKChunk;
        for (int i = lane; i < T * (kShKChunk / 4); i += 64) {
            const int t = i / (kShKChunk / 4), c = (i % (kShKChunk / 4)) * 4;
            const uint2 v = *reinterpret_cast<const uint2*>(x + (int64_t)t * H + k0 + c);
            *reinterpret_cast<uint2*>(x16 + (int64_t)t * H + k0 + c) = make_uint2(
                pack2(f32_to_f16_bits(bf16_to_f32(v.x & 0xffffu)), f32_to_f16_bits(bf16_to_f32(v.x >> 16))),
                pack2(f32_to_f16_bits(bf16_to_f32(v.y & 0xffffu)), f32_to_f16_bits(bf16_to_f32(v.y >> 16))));
        }
        return;
    }
    const int n_st = 2 * Is / 16;
    const int row0 = (wi % n_st) * 16, kc = wi / n_st;
    const int row = row0 + r;
    const uint16_t* brow = sh_ug + (int64_t)row * H + kc * kShKChunk + 8 * g;
    const uint16_t* arow = x + (int64_t)(vt ? r : 0) * H + kc * kShKChunk + 8 * g;
    u32x4 a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        a[s] = vt ? ld16(arow + 32 * s) : zero;
        b[s] = ld16_stream(brow + 32 * s);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma16_bf16(a[s], b[s], acc);
    float* out = shp + (int64_t)kc * T * 2 * Is;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < T) out[(int64_t)m * 2 * Is + row] = acc[i];
    }
}

// ---------------------------------------------------------------- routing
// Block-wide exclusive scan of one int per thread (NT threads, <= 16 waves);
// `total` receives the sum.  lds: >= 33 ints.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* lds, int& total) {
    constexpr int NW = NT / 64;
    const int lane = __lane_id(), wid = threadIdx.x >> 6;
    const int incl = wave_incl_scan_dpp(v);
    if (lane == 63) lds[wid] = incl;
    __syncthreads();
    if (threadIdx.x < 64) {
        const int sv = lane < NW ? lds[lane] : 0;
        const int si = wave_incl_scan_dpp(sv);
        if (lane < NW) lds[16 + lane] = si - sv;
        if (lane == NW - 1) lds[32] = si;
    }
    __syncthreads();
    total = lds[32];
    const int r = lds[16 + wid] + incl - v;
    __syncthreads();
    return r;
}

// Routing of T <= 16 tokens by one block of NT threads (README of the
// model: 10 of 512 experts per token; softmax over the selected logits):
// top-k per token (one wave per token: larger logit first, lower expert
// index on ties), the softmax of the selected logits, then the stable
// counting sort of the T*k slots by expert.  A token selects an expert at
// most once, so the rank of slot (t, j) in expert e is the number of earlier
// tokens that selected e: a popcount of the token mask of e.  Results in LDS:
// s_tiles (active experts in ascending order: expert, first slot, slots),
// s_perm (slot -> flat index t*k + j) and *s_nt; with `publish` also to global
// memory (ids, w, the optional copies, offsets [E+1], perm, inv, tiles,
// ntiles).  The logits are np planes [np][T][E] summed in plane order, plus
// `bias` when given (np = 1, no bias: the logits as they are).  scr: >=
// route_scratch_bytes(T, E, NT / 64) of LDS (the sums are staged there before
// the top-k reads them; then each wave's top-k scratch).
__host__ __device__ constexpr int route_log_end(int T, int E) { return (10752 + T * E * 4 + 7) & ~7; }
__host__ __device__ constexpr int route_scratch_bytes(int T, int E, int waves) {
    return route_log_end(T, E) + waves * kTopkScratch * 8;
}

template <int NT>
__device__ __forceinline__ void route_block(const float* __restrict__ logits, int np,
                                            const float* __restrict__ bias, int T, int E, int k,
                                            uint8_t* scr, int* s_tiles, int* s_perm, int* s_nt,
                                            bool publish, int32_t* ids, float* wts,
                                            int32_t* ids_out, float* w_out, int32_t* offsets,
                                            int32_t* perm, int32_t* inv, int32_t* tiles,
                                            int32_t* ntiles) {
    uint32_t* s_mask = reinterpret_cast<uint32_t*>(scr);          // [1024]
    int* s_first = reinterpret_cast<int*>(scr + 4096);             // [1024]
    int* s_ids = reinterpret_cast<int*>(scr + 8192);               // [512]
    int* s_scan = reinterpret_cast<int*>(scr + 10240);             // [40]
    float* s_log = reinterpret_cast<float*>(scr + 10752);          // [T][E]
    uint64_t* s_tk = reinterpret_cast<uint64_t*>(scr + route_log_end(T, E)) + (threadIdx.x >> 6) * kTopkScratch;
    const int tid = threadIdx.x, lane = __lane_id(), wid = threadIdx.x >> 6;
    for (int e = tid; e < 1024; e += NT) s_mask[e] = 0u;
    const int nl = T * E;
    for (int i0 = tid; i0 < nl; i0 += 8 * NT) {                    // 8 x (np + 1) loads in flight
        float v[8][kMaxLogitParts + 1];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = min(i0 + u * NT, nl - 1);
#pragma unroll
            for (int p = 0; p < kMaxLogitParts; ++p) v[u][p] = p < np ? logits[(int64_t)p * nl + i] : 0.f;
            v[u][kMaxLogitParts] = bias ? bias[i % E] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (i0 + u * NT < nl) {
                float sum = v[u][0];
#pragma unroll
                for (int p = 1; p < kMaxLogitParts; ++p)
                    if (p < np) sum += v[u][p];
                s_log[i0 + u * NT] = bias ? sum + v[u][kMaxLogitParts] : sum;
            }
        }
    }
    __syncthreads();
    for (int t = wid; t < T; t += NT / 64) {
        const float* row = s_log + t * E;
        int id;
        float v;
        wave_topk([&](int e) { return row[e]; }, E, k, s_tk, id, v);
        const float wt = wave_softmax_selected(v, k);
        if (lane < k) {
            s_ids[t * k + lane] = id;
            atomicOr(&s_mask[id], 1u << t);
            if (publish) {
                ids[t * k + lane] = id;
                wts[t * k + lane] = wt;
                if (ids_out) ids_out[t * k + lane] = id;
                if (w_out) w_out[t * k + lane] = wt;
            }
        }
    }
    __syncthreads();
    // thread tid owns experts QE*tid .. QE*tid + QE - 1 (in order)
    constexpr int QE = (1024 + NT - 1) / NT;
    int c[QE], cs = 0, as = 0;
#pragma unroll
    for (int q = 0; q < QE; ++q) {
        const int e = QE * tid + q;
        c[q] = e < E ? __popc(s_mask[e]) : 0;
        cs += c[q];
        as += c[q] > 0 ? 1 : 0;
    }
    // one scan of both counts: slots (< 2^9) in the low half, experts (< 2^11) above
    int tot;
    const int pre = block_excl_scan<NT>(cs | (as << 16), s_scan, tot);
    int off = pre & 0xffff, ai = pre >> 16;
    const int tot_c = tot & 0xffff, tot_a = tot >> 16;
#pragma unroll
    for (int q = 0; q < QE; ++q) {
        const int e = QE * tid + q;
        if (e < E) {
            s_first[e] = off;
            if (publish) offsets[e] = off;
            if (c[q] > 0) {
                s_tiles[3 * ai] = e;
                s_tiles[3 * ai + 1] = off;
                s_tiles[3 * ai + 2] = c[q];
                if (publish) {
                    tiles[3 * ai] = e;
                    tiles[3 * ai + 1] = off;
                    tiles[3 * ai + 2] = c[q];
                }
                ++ai;
            }
            off += c[q];
        }
    }
    if (tid == 0) {
        *s_nt = tot_a;
        if (publish) {
            offsets[E] = tot_c;
            *ntiles = tot_a;
        }
    }
    __syncthreads();
    for (int f = tid; f < T * k; f += NT) {
        const int t = f / k, e = s_ids[f];
        const int p = s_first[e] + __popc(s_mask[e] & ((1u << t) - 1u));
        s_perm[p] = f;
        if (publish) {
            perm[p] = f;
            inv[f] = p;
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- up|gate
// Decode table: the Q3S-256 pair table (moe_decoders.hpp).  The sub-scale s
// multiplies each looked-up pair afterwards (s*c is an exact fp16 integer,
// |s*c| <= 1016).

// LDS budget of the up|gate kernel besides the table: the partial sums of
// two items (WAVES x (up, gate) x 64 lanes x 4 floats each) and two staged
// items of 32 rows at a stride of (row bytes + 8).
__host__ __device__ constexpr int ug_red_bytes(int waves) { return 2 * waves * 2 * 64 * 16; }

__host__ __device__ constexpr int ug_stage_stride(int H) { return (H / 256) * 104 + 8; }
// static LDS of the up|gate kernel: the table, the tiles and slot map of the routing
constexpr int kUgStaticLds = kQ3LutDw * 4 + 4 * (4 * kMaxSlots + 1) + 16;
// one stage: 32 rows and a 16-byte scratch slot for the loads past the rows
__host__ __device__ constexpr int ug_stage_bytes(int H) { return 32 * ug_stage_stride(H) + 16; }
// waves that load, stage and finish the items, besides the decoding waves
constexpr int kUgLoadWaves = 4;
// decoding waves (two per SIMD, with one loader wave)
__host__ __device__ constexpr int ug_waves(int H) {
    (void)H;
    return 8;
}

// Persistent: one block per CU of WAVES decoding waves and kUgLoadWaves
// loading waves; each block owns a contiguous range of items (active expert
// a, 16-column slice): the 16 up rows and the 16 matching gate rows (32 x
// H/256 packed blocks).  The loading waves fetch an item's rows with
// coalesced CH-byte loads into registers while the item before it is in the
// other LDS stage, write them to their stage when their turn comes (row stride = row bytes + 8, so that the
// per-lane reads of 16 rows hit distinct banks) and run the item's epilogue;
// the decoding waves only decode.  They split K in groups of 128 (4
// sub-blocks; wave w takes groups w + WAVES*i); lane group g of a
// 16x16x32 step takes one whole 32-weight sub-block (12 index bytes), so the
// B operand of a step spans 4 sub-blocks of one 256-weight block:
// B = s*c (exact fp16 integers) and the block scale d/128 multiplies the
// fp32 partial of the group.  The A operand holds every token of the batch
// (row m = token m, rows >= T zero): each item multiplies all tokens and
// keeps the routed ones.  Epilogue (loading waves): partials of the
// decoding waves summed in wave order through LDS, a = bf16_rne(silu(g) * u),
// stored as fp16 (exact).
// After the routed items every block finishes its share of the shared
// expert: a_sh[t][o] = bf16(silu(sum_c g) * sum_c u) over the stage-1 chunks.
template <int GPW, bool FULL, int WAVES>
__global__ void __launch_bounds__(64 * (WAVES + kUgLoadWaves), 1) k_upgate_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const float* __restrict__ logits, int np,
    const float* __restrict__ lbias, int E, int k, const uint16_t* __restrict__ x16, int T, int H,
    int I, uint16_t* __restrict__ a16_perm,
    const float* __restrict__ shp, int nkc, int Is, uint16_t* __restrict__ a_sh, RouteOut ro) {
    constexpr int NT = 64 * (WAVES + kUgLoadWaves);         // threads
    constexpr int NL = 64 * kUgLoadWaves;                   // loader threads
    constexpr int CH = FULL ? 16 : 8;                       // bytes per staging load
    // chunks per loader thread: 32 rows of <= 52 * WAVES * GPW bytes
    constexpr int NCH = (32 * 52 * WAVES * GPW / CH + NL - 1) / NL;
    __shared__ __attribute__((aligned(8192))) uint32_t lut[kQ3LutDw];  // pair bits OR onto the address
    __shared__ int s_tiles[3 * kMaxSlots], s_perm[kMaxSlots], s_nt;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    f32x4 (*red)[WAVES][2][64] = reinterpret_cast<f32x4 (*)[WAVES][2][64]>(dyn);
    uint8_t* stage = dyn + ug_red_bytes(WAVES);

    const int tid = threadIdx.x, lane = __lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // the decode table first, while the routing's logit loads are in flight
    // (the routing's barriers make it visible)
    q3_pair_table_fill(lut, tid, NT);
    if (logits) {
        // routing (every block; block 0 publishes it), in the partial-sum space
        route_block<NT>(logits, np, lbias, T, E, k, dyn, s_tiles, s_perm, &s_nt, blockIdx.x == 0, ro.ids,
                        ro.w, ro.ids_out, ro.w_out, ro.offsets, ro.perm, ro.inv, ro.tiles, ro.ntiles);
    } else {
        // routing given (the expert FFN export): its tile list (one tile per
        // active expert, in expert order) and permutation
        const int ntl = *ro.ntiles;
        for (int i = tid; i < 3 * ntl; i += NT) s_tiles[i] = ro.tiles[i];
        for (int i = tid; i < T * k; i += NT) s_perm[i] = ro.perm[i];
        if (tid == 0) s_nt = ntl;
        __syncthreads();
    }
    const int nsl = I / 16;
    const int n_items = __builtin_amdgcn_readfirstlane(s_nt) * nsl;
    const int G = gridDim.x;
    const int i0 = (int)((int64_t)blockIdx.x * n_items / G);
    const int i1 = (int)((int64_t)(blockIdx.x + 1) * n_items / G);
    const int rb = (H / kQ3Weights) * kQ3Bytes;
    const int RS = rb + 8;
    const int NG = FULL ? WAVES * GPW : H / 128;

    // The two roles run separate loops with the same number of barriers, so
    // their register state never overlaps: a decoder keeps the A operand
    // (every token of the batch, its K groups), a loader two items in
    // flight.
    constexpr int RA = GPW * 16, RB = NCH * CH / 4;
    uint32_t R[RA];                                         // decoders: A
    uint32_t L0[RB], L1[RB];                                // loaders: item ring
    const bool loader = w >= WAVES;
    const int lt = tid - 64 * WAVES;                        // loader thread (loaders only)
    auto av = [&](int gi, int i) {
        return u32x4{R[16 * gi + 4 * i], R[16 * gi + 4 * i + 1], R[16 * gi + 4 * i + 2], R[16 * gi + 4 * i + 3]};
    };

    // staging map of a loader thread (the same for every item): chunk j covers
    // CH bytes of row `row` (0..15 up, 16..31 gate) at column `col`, packed
    // as row << 16 | col (row 32: past the rows, a scratch slot)
    const int cpr = rb / CH;                                // chunks per row
    int rc[NCH];
    // the larger variants decode rc where it is used (kept decoded out of
    // the loop, the offsets would not fit the registers)
    constexpr bool kPinRc = GPW >= 4 || (GPW == 3 && !FULL);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int c = lt + NL * j;
        const int row = c / cpr, col = (c - row * cpr) * CH;
        rc[j] = (c >= 0 && row < 32) ? (row << 16 | col) : 32 << 16;
    }

    // item i -> S.  Every step issues the same loads (a fixed count, so the
    // compiler's waits on one slot never cover the other slot's loads): an
    // item past the block's last one loads one shared 16-byte line.
    auto issue = [&](int i, uint32_t (&S)[RB]) {
        const bool live = i < i1;
        const int ic = min(i, max(0, min(i1, n_items) - 1)), at = ic / nsl, sl = ic - at * nsl;
        const int e = __builtin_amdgcn_readfirstlane(s_tiles[3 * at]);
        const uint8_t* base = experts + (int64_t)e * estride + (int64_t)(16 * sl) * rb;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            int v = rc[c];
            if constexpr (kPinRc) __asm__ volatile("" : "+v"(v));
            const int row = v >> 16, col = v & 0xffff;
            const int go = (live && row < 32) ? (row < 16 ? row : I - 16 + row) * rb + col : 0;
            if constexpr (CH == 16) {
                const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + go));
                S[4 * c] = t[0]; S[4 * c + 1] = t[1]; S[4 * c + 2] = t[2]; S[4 * c + 3] = t[3];
            } else {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + go));
                S[2 * c] = t[0]; S[2 * c + 1] = t[1];
            }
        }
    };
    auto put = [&](int sb, const uint32_t (&S)[RB]) {       // S -> stage sb (8-byte stores)
        uint8_t* st = stage + sb * ug_stage_bytes(H);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            int v = rc[c];
            if constexpr (kPinRc) __asm__ volatile("" : "+v"(v));
            const int lo = (v >> 16) * RS + (v & 0xffff);
#pragma unroll
            for (int h = 0; h < CH / 8; ++h)
                *reinterpret_cast<uint2*>(st + lo + 8 * h) =
                    make_uint2(S[(CH / 4) * c + 2 * h], S[(CH / 4) * c + 2 * h + 1]);
        }
    };

    const uint32_t cbase = lut_copy_base(lds_addr(lut), lane);
    const uint32_t kmag = (65536u + (uint32_t)k - 1u) / (uint32_t)k;   // t = (f * kmag) >> 16 for f < 512
    const __amdgpu_buffer_rsrc_t a_out =
        __builtin_amdgcn_make_buffer_rsrc(a16_perm, 0, (int)(T * k * I * 2), 0x00020000);
    // this lane's bytes in a staged row: group gi at + (WAVES / 2) * 104 * gi
    const int r_idx = r * RS + (w >> 1) * kQ3Bytes + 12 * (4 * (w & 1) + g);
    const int r_tail = r * RS + (w >> 1) * kQ3Bytes + 96;

    auto decode = [&](int it, int sb) {                     // decoders; sb: stage of item it
        const uint32_t st = lds_addr(stage + sb * ug_stage_bytes(H));
        f32x4 acc_u = {0.f, 0.f, 0.f, 0.f}, acc_g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int q = w + WAVES * gi;
            if (FULL || q < NG) {
                const uint32_t ou = st + r_idx + (WAVES / 2) * kQ3Bytes * gi, og = ou + 16 * RS;
                const uint32_t iu[3] = {lds_ld(ou), lds_ld(ou + 4), lds_ld(ou + 8)};
                const uint32_t ig[3] = {lds_ld(og), lds_ld(og + 4), lds_ld(og + 8)};
                const uint32_t tu = st + r_tail + (WAVES / 2) * kQ3Bytes * gi, tg = tu + 16 * RS;
                const uint64_t tlu = ((uint64_t)lds_ld(tu + 4) << 32) | lds_ld(tu);
                const uint64_t tlg = ((uint64_t)lds_ld(tg + 4) << 32) | lds_ld(tg);
                const int js = 4 * (q & 1) + g;
                const _Float16 su = (_Float16)(float)q3_tail_s(tlu, js);
                const _Float16 sg = (_Float16)(float)q3_tail_s(tlg, js);
                const h2 su2 = {su, su}, sg2 = {sg, sg};
                f32x4 pu = {0.f, 0.f, 0.f, 0.f}, pg = {0.f, 0.f, 0.f, 0.f};
                // the group's 32 table reads in two halves of 16, each half in
                // flight before any of it is used
#define MOE_PAIR(I_, P_)                                                        \
    lu[4 * ((I_) & 1) + P_] = lds_ld(q3_pair_addr<24 * (I_) + 6 * P_>(iu, cbase)); \
    lg[4 * ((I_) & 1) + P_] = lds_ld(q3_pair_addr<24 * (I_) + 6 * P_>(ig, cbase));
#define MOE_STEP(I_) MOE_PAIR(I_, 0) MOE_PAIR(I_, 1) MOE_PAIR(I_, 2) MOE_PAIR(I_, 3)
#define MOE_HALF(H_)                                                            \
    {                                                                           \
        uint32_t lu[8], lg[8];                                                  \
        MOE_STEP(2 * H_) MOE_STEP(2 * H_ + 1)                                   \
        __builtin_amdgcn_sched_barrier(0);                                      \
        u32x4 bu[2], bg[2];                                                     \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                         \
            bu[i >> 2][i & 3] = mul_pair(lu[i], su2);                           \
            bg[i >> 2][i & 3] = mul_pair(lg[i], sg2);                           \
        }                                                                       \
        _Pragma("unroll") for (int i = 0; i < 2; ++i) {                         \
            pu = mfma16_f16(av(gi, 2 * H_ + i), bu[i], pu);                     \
            pg = mfma16_f16(av(gi, 2 * H_ + i), bg[i], pg);                     \
        }                                                                       \
    }
                MOE_HALF(0) MOE_HALF(1)
#undef MOE_HALF
#undef MOE_STEP
#undef MOE_PAIR
                const float du = q3_tail_d(tlu) * 0.0078125f;
                const float dg = q3_tail_d(tlg) * 0.0078125f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc_u[i] += pu[i] * du;
                    acc_g[i] += pg[i] * dg;
                }
            }
        }
        const int buf = it & 1;
        red[buf][w][0][lane] = acc_u;
        red[buf][w][1][lane] = acc_g;
    };

    // loaders: thread (slot j, column n) of item it; D row m = token tj sits
    // at lane (m/4)*16 + n, element m%4 of each decoder's partials, summed in
    // decoder order.  Every loader thread issues the store (equal memory-op
    // counts on all paths); those without an output store out of range, which
    // the buffer unit drops.
    auto finish = [&](int it0, bool valid) {                // !valid: the store is dropped
        const int it = valid ? it0 : i0;
        const int at = it / nsl, sl = it - at * nsl;
        const int row0 = __builtin_amdgcn_readfirstlane(s_tiles[3 * at + 1]);
        const int rows = __builtin_amdgcn_readfirstlane(s_tiles[3 * at + 2]);
        const int buf = it & 1;
        const int j = lt >> 4, n = lt & 15;
        const int slot = s_perm[row0 + (j < rows ? j : 0)];
        const int tj = (int)(((uint32_t)slot * kmag) >> 16);
        const float* ru = reinterpret_cast<const float*>(&red[buf][0][0][(tj >> 2) * 16 + n]) + (tj & 3);
        float u = 0.f, gg = 0.f;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
            u += ru[v * 2 * 64 * 4];
            gg += ru[v * 2 * 64 * 4 + 64 * 4];
        }
        const uint16_t av16 = (uint16_t)f32_to_f16_bits(bf16_to_f32(f32_to_bf16(silu_mul_fast(gg, u))));
        const uint32_t off = (valid && j < rows) ? (uint32_t)(((row0 + j) * I + 16 * sl + n) * 2) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b16(av16, a_out, off, 0, 0);
    };

    // Pipeline, one barrier per item in both roles.  Step it: the decoders
    // decode item it from stage (it - i0) % 2 into red[it % 2]; the loaders
    // write item it + 1 from its ring slot to stage (it + 1 - i0) % 2, load
    // item it + 3 into that slot and finish item it - 1 from red[(it - 1) % 2].
    // Items it + 2 and it + 3 are in flight during the decode of item it (a
    // load has two steps to arrive); loads stop at the block's last item (a
    // block without items loads item min(i0, n_items - 1) in the prologue).
    // The loader loop takes two steps per trip so that the ring slots are
    // fixed registers.
    if (loader) {
        issue(i0, L0);
        issue(i0 + 1, L1);
        put(0, L0);
        issue(i0 + 2, L0);
        __syncthreads();                                    // stage 0 written
        int it = i0;
        for (; it + 1 < i1; it += 2) {
            put(1, L1);                                     // item it + 1 (it - i0 even)
            __builtin_amdgcn_sched_barrier(0);
            issue(it + 3, L1);
            __builtin_amdgcn_sched_barrier(0);
            finish(it - 1, it > i0);
            __syncthreads();
            put(0, L0);                                     // step it + 1: item it + 2 (unread if none)
            __builtin_amdgcn_sched_barrier(0);
            issue(it + 4, L0);
            __builtin_amdgcn_sched_barrier(0);
            finish(it, true);
            __syncthreads();
        }
        if (it < i1) {                                      // the last step when i1 - i0 is odd
            finish(it - 1, it > i0);
            __syncthreads();
        }
        if (i1 > i0) finish(i1 - 1, true);
    } else {
        const bool vt = r < T;
        const uint16_t* xr = x16 + (int64_t)(vt ? r : 0) * H + 32 * g;
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
            const int q = w + WAVES * gi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = ((FULL || q < NG) && vt) ? ld16(xr + q * 128 + 8 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int c = 0; c < 4; ++c) R[16 * gi + 4 * i + c] = v[c];
            }
        }
        __syncthreads();                                    // stage 0 written
        for (int it = i0; it < i1; ++it) {
            decode(it, (it - i0) & 1);
            __syncthreads();
        }
    }

    if (shp) {                                              // shared expert: sum partials, SwiGLU
        for (int i = blockIdx.x * NT + tid; i < T * Is; i += G * NT) {
            const int t = i / Is, o = i - t * Is;
            float u = 0.f, gg = 0.f;
            for (int c0 = 0; c0 < nkc; c0 += 8) {           // 16 loads in flight, summed in chunk order
                float pu[8], pg[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {                // clamped: no branch around the loads
                    const float* p = shp + ((int64_t)min(c0 + c, nkc - 1) * T + t) * 2 * Is;
                    pu[c] = p[o];
                    pg[c] = p[Is + o];
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    if (c0 + c < nkc) {
                        u += pu[c];
                        gg += pg[c];
                    }
                }
            }
            a_sh[i] = (uint16_t)f32_to_bf16(silu_mul(gg, u));
        }
    }
}

// ---------------------------------------------------------------- down
// Decode table: the NL4-32 pair table (moe_decoders.hpp), (T4[lo], T4[hi])
// per index byte, built once per block.

constexpr int kDnWaves = 8;
constexpr int kDnChunkDw = 72;                    // 16 NL4 blocks of a row (288 bytes)
constexpr int kDnStageDw = kDnChunkDw + 2;        // stage row stride (= 10 mod 32: the 16 rows x 2 lane groups of a half-wave hit distinct banks)
constexpr int kDnLoads = 16 * kDnChunkDw / 64;    // dword loads per lane per staged chunk (18)
constexpr int kDnChunk16 = 16 * kDnChunkDw / 4;   // 16-byte pieces of a whole chunk (288)
constexpr int kDnLoads16 = (kDnChunk16 + 63) / 64;   // 16-byte loads per lane (5; the last by lanes 0-31)
constexpr int kDnShSteps = 16;                    // shared down: 16x16x32 steps per load batch (Is <= 512 at once)

// Persistent: blocks of kDnWaves waves; after the table is built every wave works
// alone.  The waves are dealt to the active experts (2 shares each) and to
// the shared expert (7 shares, its rows being bf16) in proportion; the waves
// of one expert split its H/16 slices of 16 output rows.  A wave keeps the
// A operand of its expert (the routed rows' fp16 activations, <= 16 slots)
// in registers.  Routed slice: the 16 rows x 16 blocks of a K chunk (4608
// contiguous bytes) are loaded with coalesced 16-byte loads two units ahead,
// written to the wave's LDS stage and decoded from there: one 16x16x32 step
// per NL4 block (lane group g takes 8 weights = 4 index bytes; B = table
// integers T4[q], exact fp16) and the block scale d/128 multiplies the fp32
// partial of the step.  Output y_perm[slot][h] (unweighted, permuted rows);
// the combine kernel sums them.  Shared slice: bf16 rows x a_sh (bf16), 16x16x32
// bf16 steps, output y_sh[t][h].
template <bool FULL16, bool ONEK>   // I % 512 == 0; I <= 512 (A kept for all slices)
__global__ void __launch_bounds__(64 * kDnWaves, 1) k_down_dec(
    const uint8_t* __restrict__ experts, int64_t estride, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const uint16_t* __restrict__ a16_perm, int T, int H, int I,
    const uint16_t* __restrict__ sh_down, const uint16_t* __restrict__ a_sh, int Is,
    float* __restrict__ y_perm, float* __restrict__ y_sh) {
    __shared__ __attribute__((aligned(32768))) uint32_t lut[kNl4LutDw];   // byte bits OR onto the address
    __shared__ __attribute__((aligned(16))) uint32_t stg[kDnWaves][16 * kDnStageDw];
    __shared__ int s_claim[kDnWaves];                       // slices taken, per group of waves
    __shared__ int s_spare[kDnWaves][64];                   // the other lanes' claims land here
    const int tid = threadIdx.x, lane = __lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int nt = __builtin_amdgcn_readfirstlane(*ntiles);  // in flight during the table build
    nl4_pair_table_fill(lut, tid, 64 * kDnWaves);
    if (lane == 0) s_claim[w] = 0;
    __syncthreads();

    // this wave's expert (its team: the waves dealt to it)
    const bool has_sh = sh_down != nullptr;
    const int total = 2 * nt + (has_sh ? 7 : 0);
    const int GW = gridDim.x * kDnWaves, gw = blockIdx.x * kDnWaves + w;
    const int u = (int)((int64_t)gw * total / GW);
    const int t = u < 2 * nt ? (u >> 1) : nt;               // t == nt: shared expert
    const int us = 2 * t, ue = t < nt ? 2 * t + 2 : total;
    const int ws = (int)(((int64_t)us * GW + total - 1) / total);
    const int we = (int)(((int64_t)ue * GW + total - 1) / total);
    const int nsl = H / 16;
    const int s0 = (int)((int64_t)(gw - ws) * nsl / (we - ws));
    const int s1 = (int)((int64_t)(gw - ws + 1) * nsl / (we - ws));
    // When the wave keeps all of K in registers, the waves of the team in
    // this block share their slices [g0, g1) through an LDS counter (owned by
    // the group's first wave, wf) and take them one at a time, so that the
    // group finishes together whichever of its waves runs faster; otherwise
    // each wave keeps its share [s0, s1).
    const int bw = blockIdx.x * kDnWaves;
    const int wf = max(ws, bw) - bw, wl = min(we, bw + kDnWaves) - 1 - bw;
    const int g0 = (int)((int64_t)(bw + wf - ws) * nsl / (we - ws));
    const int g1 = (int)((int64_t)(bw + wl + 1 - ws) * nsl / (we - ws));
    // lane 0 receives the count of slices taken so far.  Every lane adds, to
    // its own word but lane 0: an address that differs across the wave keeps
    // the add a plain LDS atomic (the same address everywhere would become one
    // add broadcast at once, with the wait for it right there).
    auto claim = [&]() -> int {
        int* p = lane == 0 ? &s_claim[wf] : &s_spare[w][lane];
        return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // the claimed slice as a scalar (nsl: none left), read here and not earlier
    auto take = [&](int v) {
        __asm__ volatile("" : "+v"(v));
        const int c = __builtin_amdgcn_readfirstlane(v);
        return c < g1 - g0 ? g0 + c : nsl;
    };

    if (t == nt) {                                          // shared expert, bf16
        const bool vt = r < T;
        const uint16_t* arow = a_sh + (int64_t)(vt ? r : 0) * Is + 8 * g;
        const __amdgpu_buffer_rsrc_t yo = __builtin_amdgcn_make_buffer_rsrc(y_sh, 0, T * H * 4, 0x00020000);
        auto store = [&](int sl, const f32x4& acc) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * g + i;
                const uint32_t off = m < T ? (uint32_t)((m * H + 16 * sl + r) * 4) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i]), yo, off, 0, 0);
            }
        };
        const int nks = Is / 32;
        if (nks <= kDnShSteps) {
            // A in registers; a slice's whole K (<= 1 KB per lane group row)
            // loaded at once, the next slice in flight during the steps.  Steps
            // past Is and slices past the last load nothing (out-of-range
            // buffer offsets read zero).
            const __amdgpu_buffer_rsrc_t bsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(sh_down), 0, H * Is * 2, 0x00020000);
            u32x4 a[kDnShSteps], B0[kDnShSteps], B1[kDnShSteps];
#pragma unroll
            for (int i = 0; i < kDnShSteps; ++i)
                a[i] = (vt && i < nks) ? ld16(arow + 32 * i) : u32x4{0u, 0u, 0u, 0u};
            auto load_b = [&](int sl, u32x4* B) {
                const uint32_t rowo = sl < nsl ? (uint32_t)(((16 * sl + r) * Is + 8 * g) * 2) : 0x80000000u;
#pragma unroll
                for (int i = 0; i < kDnShSteps; ++i)
                    B[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        bsrc, i < nks ? rowo + 64u * i : 0x80000000u, 0, 0));
            };
            auto steps = [&](int sl, const u32x4* B) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < kDnShSteps; ++i) acc = mfma16_bf16(a[i], B[i], acc);
                store(sl, acc);
            };
            // each claim is made before the loads of the step ahead of its use
            const int p0 = claim();
            int pend = claim();
            int sa = take(p0);
            load_b(sa, B0);
            while (sa < nsl) {
                const int sb = take(pend);
                pend = claim();
                load_b(sb, B1);
                steps(sa, B0);
                if (sb >= nsl) return;
                const int sc = take(pend);
                pend = claim();
                load_b(sc, B0);
                steps(sb, B1);
                sa = sc;
            }
            return;
        }
        for (int sl = s0; sl < s1; ++sl) {
            const uint16_t* brow = sh_down + (int64_t)(16 * sl + r) * Is + 8 * g;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < nks; k0 += kDnShSteps) {  // kDnShSteps loads in flight
                u32x4 av[kDnShSteps], bv[kDnShSteps];
#pragma unroll
                for (int i = 0; i < kDnShSteps; ++i) {
                    const bool ok = k0 + i < nks;
                    av[i] = (vt && ok) ? ld16(arow + 32 * (k0 + i)) : u32x4{0u, 0u, 0u, 0u};
                    bv[i] = ok ? ld16_stream(brow + 32 * (k0 + i)) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < kDnShSteps; ++i) acc = mfma16_bf16(av[i], bv[i], acc);
            }
            store(sl, acc);
        }
        return;
    }

    const int e = tiles[3 * t], row0 = tiles[3 * t + 1], rows = tiles[3 * t + 2];
    const int nb = I / 32, nkc = (nb + 15) / 16;
    const int rb = nb * kNL4Bytes;
    const uint8_t* W = experts + (int64_t)e * estride + (int64_t)2 * I * (H / kQ3Weights) * kQ3Bytes;
    const uint16_t* arow = a16_perm + (int64_t)(row0 + (r < rows ? r : 0)) * I + 8 * g;
    const __amdgpu_buffer_rsrc_t yo =
        __builtin_amdgcn_make_buffer_rsrc(y_perm, 0, (row0 + rows) * H * 4, 0x00020000);
    const uint32_t cbase = lut_copy_base(lds_addr(lut), lane);
    uint32_t* st = stg[w];

    // whole chunks (16 NL4 blocks per row): the lane's 16-byte pieces,
    // (global byte offset | stage dword << 16); piece j is bytes 16 (j % 18)
    // of row j / 18
    uint32_t off[kDnLoads16];
#pragma unroll
    for (int i = 0; i < kDnLoads16; ++i) {
        const int j = min(lane + 64 * i, kDnChunk16 - 1), row = j / 18, col = j - row * 18;
        off[i] = (uint32_t)(row * rb + 16 * col) | ((uint32_t)(row * kDnStageDw + 4 * col) << 16);
    }
    // A operand of the expert: chunk c, block b -> av[b]
    u32x4 av[16];
    auto load_a = [&](int c) {
#pragma unroll
        for (int b = 0; b < 16; ++b)
            av[b] = (16 * c + b < nb) ? ld16(arow + 32 * (16 * c + b)) : u32x4{0u, 0u, 0u, 0u};
    };
    if (ONEK) load_a(0);

    struct Buf {
        uint32_t v[FULL16 ? 4 * kDnLoads16 : kDnLoads];
    };
    Buf P0, P1;
    // the expert's down rows as a buffer: 32-bit lane offsets, the unit's start
    // in a scalar (out of range past the last slice: nothing loaded)
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W), 0, H * rb, 0x00020000);
    auto issue = [&](int sl, int c, Buf& B) {               // chunk c of slice sl
        const int soff = sl < nsl ? 16 * sl * rb + 288 * c : 0x7ff00000;
        if constexpr (FULL16) {
            // 16-byte loads (lanes 32-63 load their fifth piece again: the
            // chunk has 4.5 pieces per lane; the copy is not stored)
#pragma unroll
            for (int i = 0; i < kDnLoads16; ++i) {
                const u32x4 t = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, off[i] & 0xffffu, soff, 0));
#pragma unroll
                for (int q = 0; q < 4; ++q) B.v[4 * i + q] = t[q];
            }
        } else {
            const int cbk = min(16, nb - 16 * c);
            const int dpr = cbk * kNL4Bytes / 4;
#pragma unroll
            for (int i = 0; i < kDnLoads; ++i) {
                const int j = lane + 64 * i, row = j / dpr, col = j - row * dpr;
                const uint32_t go = j < 16 * dpr ? (uint32_t)(row * rb + 4 * col) : 0u;
                B.v[i] = __builtin_amdgcn_raw_buffer_load_b32(wsrc, go, soff, 0);
            }
        }
    };
    auto put = [&](int c, const Buf& B) {
        if constexpr (FULL16) {
            // the stage's row stride (74 dwords) keeps pieces 8-byte aligned
#pragma unroll
            for (int i = 0; i < kDnLoads16; ++i) {
                if (i + 1 < kDnLoads16 || lane + 64 * i < kDnChunk16) {
                    uint2* d2 = reinterpret_cast<uint2*>(st + (off[i] >> 16));
                    d2[0] = make_uint2(B.v[4 * i], B.v[4 * i + 1]);
                    d2[1] = make_uint2(B.v[4 * i + 2], B.v[4 * i + 3]);
                }
            }
        } else {
            const int cbk = min(16, nb - 16 * c);
            const int dpr = cbk * kNL4Bytes / 4;
#pragma unroll
            for (int i = 0; i < kDnLoads; ++i) {
                const int j = lane + 64 * i, row = j / dpr, col = j - row * dpr;
                if (j < 16 * dpr) st[row * kDnStageDw + col] = B.v[i];
            }
        }
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto decode = [&](int sl, int c) {
        if (!ONEK) load_a(c);
        const int cbk = FULL16 ? 16 : min(16, nb - 16 * c);
        const uint32_t* wr = st + r * kDnStageDw;
        // four blocks at a time: their index words and scales, then all 16
        // table reads, then four independent steps
#pragma unroll
        for (int b0 = 0; b0 < 16; b0 += 4) {
            if (b0 < cbk) {
                uint32_t nib[4];
                float d[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const int b = b0 + k4;
                    const int o = 18 * b + 2 + 4 * g;          // index bytes of lane group g
                    nib[k4] = (b & 1) ? wr[o >> 2] : __builtin_amdgcn_alignbit(wr[(o >> 2) + 1], wr[o >> 2], 16);
                    const uint32_t dw = wr[(18 * b) >> 2];
                    d[k4] = f16_bits_to_f32((b & 1) ? (dw >> 16) : (dw & 0xffffu)) * 0.0078125f;
                }
                u32x4 bv[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    bv[k4][0] = lds_ld(nl4_byte_addr<0>(nib[k4], cbase));
                    bv[k4][1] = lds_ld(nl4_byte_addr<1>(nib[k4], cbase));
                    bv[k4][2] = lds_ld(nl4_byte_addr<2>(nib[k4], cbase));
                    bv[k4][3] = lds_ld(nl4_byte_addr<3>(nib[k4], cbase));
                }
                f32x4 part[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
                    part[k4] = mfma16_f16(av[b0 + k4], bv[k4], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    if (FULL16 || b0 + k4 < cbk) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] += part[k4][i] * d[k4];
                    }
                }
            }
        }
        if (ONEK || c == nkc - 1) {                         // slice done: rows m = 4g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * g + i;
                const uint32_t o = m < rows ? (uint32_t)(((row0 + m) * H + 16 * sl + r) * 4) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i]), yo, o, 0, 0);
                acc[i] = 0.f;
            }
        }
    };
    // one unit: stage the unit in B, load the unit two ahead into B, decode
    auto step = [&](int sl, int c, Buf& B, int sl2, int c2) {
        put(c, B);
        __builtin_amdgcn_sched_barrier(0);
        issue(sl2, c2, B);
        __builtin_amdgcn_sched_barrier(0);
        decode(sl, c);
    };

    if constexpr (ONEK) {
        // claimed slices, two units in flight while one is decoded; each claim
        // is made before the loads of the step ahead of its use
        const int p0 = claim(), p1 = claim();
        int pend = claim();
        int sa = take(p0);
        int sb = take(p1);
        // the two units' loads in order (interleaved, the loop's waits for
        // the first would also wait for the second)
        issue(sa, 0, P0);
        __builtin_amdgcn_sched_barrier(0);
        issue(sb, 0, P1);
        __builtin_amdgcn_sched_barrier(0);
        // (the exits return: a break that joins the loop's back edge would
        // make the waits for a buffer's loads cover the other buffer's too)
        while (sa < nsl) {
            const int sc = take(pend);
            pend = claim();
            step(sa, 0, P0, sc, 0);
            if (sb >= nsl) return;
            const int sd = take(pend);
            pend = claim();
            step(sb, 0, P1, sd, 0);
            sa = sc;
            sb = sd;
        }
    } else {
        if (s0 >= s1) return;
        // unit q = (slice s0 + q / nkc, chunk q % nkc); nothing loaded past the last
        const int nu = (s1 - s0) * nkc;
        auto unit_sl = [&](int q) { return q < nu ? s0 + q / nkc : nsl; };
        auto unit_c = [&](int q) { return q < nu ? q % nkc : 0; };
        issue(unit_sl(0), unit_c(0), P0);
        __builtin_amdgcn_sched_barrier(0);
        issue(unit_sl(1), unit_c(1), P1);
        __builtin_amdgcn_sched_barrier(0);
        for (int q = 0; q < nu; q += 2) {
            step(unit_sl(q), unit_c(q), P0, unit_sl(q + 2), unit_c(q + 2));
            if (q + 1 >= nu) break;
            step(unit_sl(q + 1), unit_c(q + 1), P1, unit_sl(q + 3), unit_c(q + 3));
        }
    }
}

// ---------------------------------------------------------------- launchers

void launch_dec_stage1(const uint16_t* x, int T, int H, int E, const uint16_t* w_r,
                       const float* bias, float* logits, const uint16_t* sh_ug, int Is,
                       float* shp, uint16_t* x16, int kp, hipStream_t st) {
    const int nkc = H / kShKChunk;
    const int n_rb = w_r ? (E + 15) / 16 * kp : 0;
    const int n_s = (sh_ug && Is > 0) ? (2 * Is / 16) * nkc : 0;
    const int n_x = x16 ? nkc : 0;
    const int n_wb = (n_s + n_x + kS1Waves - 1) / kS1Waves;
    if (n_rb + n_wb == 0) return;
    k_dec_stage1<<<n_rb + n_wb, 64 * kS1Waves, 0, st>>>(x, T, H, E, w_r, bias, logits, n_rb, kp, sh_ug, Is,
                                                        shp, n_s, x16);
}

template <int GPW, bool FULL, int WAVES>
static void upgate_dec_t(unsigned grid, hipStream_t st, const uint8_t* experts, int64_t estride,
                         const float* logits, int np, const float* lbias, int E, int k,
                         const uint16_t* x16, int T, int H,
                         int I, uint16_t* a16_perm, const float* shp, int nkc, int Is,
                         uint16_t* a_sh, const RouteOut& ro) {
    const size_t dyn = std::max((size_t)ug_red_bytes(WAVES) + 2 * (size_t)ug_stage_bytes(H),
                                (size_t)route_scratch_bytes(T, E, WAVES + kUgLoadWaves));
    static bool attr = false;                      // opt in to more than 64 KB of LDS once
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)&k_upgate_dec<GPW, FULL, WAVES>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024 - kUgStaticLds);
        attr = true;
    }
    k_upgate_dec<GPW, FULL, WAVES><<<grid, 64 * (WAVES + kUgLoadWaves), dyn, st>>>(
        experts, estride, logits, np, lbias, E, k, x16, T, H, I, a16_perm, shp, nkc, Is, a_sh, ro);
}

void launch_upgate_dec(const uint8_t* experts, int64_t estride, const float* logits, int np,
                       const float* lbias, int E, int k, int max_tiles, const uint16_t* x16, int T, int H, int I,
                       uint16_t* a16_perm, const float* shp, int Is, uint16_t* a_sh,
                       const RouteOut& ro, int n_cu, hipStream_t st) {
    const int max_items = max_tiles * (I / 16);
    const unsigned grid = (unsigned)std::max(1, std::min(n_cu, max_items));
    const int nkc = H / kShKChunk;
    // 8 decoding waves; K groups per wave: GPW (the last waves' share short
    // when H / 128 is not a multiple of 8)
    const int NG = H / 128;
    const int waves = ug_waves(H);
    const int gpw = (NG + waves - 1) / waves;
    const bool full = NG == waves * gpw;
    shp = (Is > 0) ? shp : nullptr;
#define MOE_UGT(G, F, W) upgate_dec_t<G, F, W>(grid, st, experts, estride, logits, np, lbias, E, k, \
                                               x16, T, H, I, a16_perm, shp, nkc, Is, a_sh, ro)
    switch (gpw) {
#define MOE_UG(G)                          \
    case G:                                \
        if (full) MOE_UGT(G, true, 8);     \
        else MOE_UGT(G, false, 8);         \
        break;
        MOE_UG(1) MOE_UG(2) MOE_UG(3) MOE_UG(4)
#undef MOE_UG
        default: break;
    }
#undef MOE_UGT
}

bool upgate_dec_supported(int H, int T, int E) {
    const int dyn = std::max(ug_red_bytes(ug_waves(H)) + 2 * ug_stage_bytes(H),
                             route_scratch_bytes(T, E, ug_waves(H) + kUgLoadWaves));
    return H / 128 <= 8 * 4 && kUgStaticLds + dyn <= 160 * 1024;
}

void launch_down_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                     const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int T, int H,
                     int I, int k, const uint16_t* sh_down, const uint16_t* a_sh, int Is,
                     float* y_perm, float* y_sh, int n_cu, hipStream_t st) {
    (void)k;
    // every expert needs at least one wave: 2 shares each, 7 for the shared one
    const int shares = 2 * max_tiles + 7;
    const unsigned grid = (unsigned)std::max(n_cu, (shares + kDnWaves - 1) / kDnWaves);
    if (Is <= 0) sh_down = nullptr;
#define MOE_DN(F, O)                                                                             \
    k_down_dec<F, O><<<grid, 64 * kDnWaves, 0, st>>>(experts, estride, tiles, ntiles, a16_perm, T, \
                                                     H, I, sh_down, a_sh, Is, y_perm, y_sh)
    if (I % 512 == 0) {
        if (I == 512) MOE_DN(true, true);
        else MOE_DN(true, false);
    } else {
        if (I < 512) MOE_DN(false, true);
        else MOE_DN(false, false);
    }
#undef MOE_DN
}

}  // namespace moe
