// Latency-bound kernels of the layer: dequantization (debug export), fp16
// staging of the tokens, exact top-k routing, the counting-sort permutation,
// the expert tile list, the weighted combine and the inter-layer RMSNorm.
//
// Routing: every token goes to the k largest router logits ("Avalon" README,
// opening paragraphs: 10 of 512 experts), ordered by (value desc, index asc),
// with softmax weights over the selected logits; nothing is pruned or
// dropped ("Betelgeuse" post: every routed expert is computed).
#include <type_traits>

#include "moe_decoders.hpp"
#include "moe_kernels.hpp"

namespace moe {

// ---------------------------------------------------------------- dequant

// One thread per 32-weight sub-block of a Q3S-256 block.
__global__ void k_dequant_q3s(const uint8_t* __restrict__ blocks, int64_t n_sub,
                              float* __restrict__ out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_sub) return;
    const uint8_t* b = blocks + (i >> 3) * kQ3Bytes;
    const int j = (int)(i & 7);
    const uint32_t* idx = reinterpret_cast<const uint32_t*>(b + 12 * j);
    uint32_t w0 = idx[0], w1 = idx[1], w2 = idx[2];
    uint64_t tail = *reinterpret_cast<const uint64_t*>(b + 96);
    float d = q3_tail_d(tail);
    int s = q3_tail_s(tail, j);
    float* o = out + i * 32;
#pragma unroll
    for (int w = 0; w < 32; ++w) o[w] = q3_value(d, s, q3_index(w0, w1, w2, w));
}

// One thread per NL4-32 block (18 bytes, 2-byte aligned: read bytewise).
__global__ void k_dequant_nl4(const uint8_t* __restrict__ blocks, int64_t n_blk,
                              float* __restrict__ out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_blk) return;
    const uint8_t* b = blocks + i * kNL4Bytes;
    float d = f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8));
    float* o = out + i * 32;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        uint32_t byte = b[2 + w];
        o[2 * w] = nl4_value(d, (int)(byte & 15u));
        o[2 * w + 1] = nl4_value(d, (int)(byte >> 4));
    }
}

// One thread per 32-weight sub-block of a Q2S-256 block (80 bytes: sub-block
// j's 8 index bytes at 8j, d and the sub-scales at 64, the Q3S tail layout).
__global__ void k_dequant_q2s(const uint8_t* __restrict__ blocks, int64_t n_sub,
                              float* __restrict__ out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_sub) return;
    const uint8_t* b = blocks + (i >> 3) * kQ2SBytes;
    const int j = (int)(i & 7);
    const uint64_t idx = *reinterpret_cast<const uint64_t*>(b + 8 * j);
    const uint64_t tail = *reinterpret_cast<const uint64_t*>(b + 64);
    const float d = q3_tail_d(tail);
    const int s = q3_tail_s(tail, j);
    float* o = out + i * 32;
#pragma unroll
    for (int w = 0; w < 32; ++w) o[w] = q2s_value(d, s, (int)((idx >> (2 * w)) & 3u));
}

// One thread per Q2-32 block (10 bytes, 2-byte aligned: read bytewise).
__global__ void k_dequant_q2(const uint8_t* __restrict__ blocks, int64_t n_blk,
                             float* __restrict__ out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_blk) return;
    const uint8_t* b = blocks + i * kQ2Bytes;
    const float d = f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8));
    float* o = out + i * 32;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t byte = b[2 + w];
#pragma unroll
        for (int t = 0; t < 4; ++t) o[4 * w + t] = q2_value(d, (int)((byte >> (2 * t)) & 3u));
    }
}

// One thread per 16-weight sub-block of a Q3K-256 block (110 bytes, 2-byte
// aligned: read bytewise): index bytes 6j .. 6j + 5, d at 96, the 6-bit
// sub-scale j at bits 6j of the 96-bit field at 98.
__global__ void k_dequant_q3k(const uint8_t* __restrict__ blocks, int64_t n_sub,
                              float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_sub) return;
    const uint8_t* b = blocks + (i >> 4) * kQ3KBytes;
    const int j = (int)(i & 15);
    uint64_t idx = 0;
#pragma unroll
    for (int t = 0; t < 6; ++t) idx |= (uint64_t)b[6 * j + t] << (8 * t);
    const float d = f16_bits_to_f32((uint32_t)b[96] | ((uint32_t)b[97] << 8));
    const int bit = 6 * j, by = 98 + (bit >> 3);
    // (the second byte only when the field crosses into it: the last field
    // ends with the block)
    const uint32_t w = (uint32_t)b[by] | ((bit & 7) > 2 ? (uint32_t)b[by + 1] << 8 : 0u);
    const int s = sext6(w >> (bit & 7));
    float* o = out + i * 16;
#pragma unroll
    for (int t = 0; t < 16; ++t) o[t] = q3_value(d, s, (int)((idx >> (3 * t)) & 7u));
}

// One thread per 32-weight sub-block of an NL4S-256 block (136 bytes, 8-byte
// aligned): index bytes 16j .. 16j + 15, d at 128, the 6-bit sub-scale j at
// bits 6j of the 48-bit field at 130.
__global__ void k_dequant_nl4s(const uint8_t* __restrict__ blocks, int64_t n_sub,
                               float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_sub) return;
    const uint8_t* b = blocks + (i >> 3) * kNL4SBytes;
    const int j = (int)(i & 7);
    const float d = f16_bits_to_f32((uint32_t)b[128] | ((uint32_t)b[129] << 8));
    const int bit = 6 * j, by = 130 + (bit >> 3);
    const uint32_t w = (uint32_t)b[by] | ((bit & 7) > 2 ? (uint32_t)b[by + 1] << 8 : 0u);
    const float ds = d * (float)sext6(w >> (bit & 7));
    float* o = out + i * 32;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t byte = b[16 * j + t];
        o[2 * t] = ds * (float)kT4[byte & 15u] * 0.0078125f;
        o[2 * t + 1] = ds * (float)kT4[byte >> 4] * 0.0078125f;
    }
}

// ---------------------------------------------------------------- staging

// x bf16 -> fp16 (the matrix-core operand type of the quantized experts).
__global__ void k_to_f16(const uint16_t* __restrict__ x, uint16_t* __restrict__ x16, int64_t n) {
    int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i + 3 < n) {
        uint2 v = *reinterpret_cast<const uint2*>(x + i);
        uint32_t a = f32_to_f16_bits(bf16_to_f32(v.x & 0xffffu));
        uint32_t b = f32_to_f16_bits(bf16_to_f32(v.x >> 16));
        uint32_t c = f32_to_f16_bits(bf16_to_f32(v.y & 0xffffu));
        uint32_t d = f32_to_f16_bits(bf16_to_f32(v.y >> 16));
        *reinterpret_cast<uint2*>(x16 + i) = make_uint2(pack2(a, b), pack2(c, d));
    } else {
        for (; i < n; ++i) x16[i] = (uint16_t)f32_to_f16_bits(bf16_to_f32(x[i]));
    }
}

// ---------------------------------------------------------------- routing

// Generic top-k: one wave per token.  Logits from `logits` (fp32 [T][E]).
// With x16 (H a multiple of 256): the wave also writes the fp16 copy of its
// token's row x[t] (the matrix-core operand of the routed GEMMs), its loads
// issued before the top-k so that they are in flight meanwhile.
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w,
                                              int32_t* __restrict__ ids2, float* __restrict__ w2,
                                              const uint16_t* __restrict__ x, uint16_t* __restrict__ x16,
                                              int H) {
    __shared__ uint64_t scr[4][kTopkScratch];
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = __lane_id();
    // the lane's 4-element pieces of the row: the first kPre loaded before
    // the top-k, any others (H > 3072) after it
    constexpr int kPre = 12;
    uint2 xr[kPre];
    const int nx = x16 ? H / 256 : 0;
    const uint2* xs = reinterpret_cast<const uint2*>(x + (int64_t)t * H);
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (i < nx) xr[i] = xs[lane + 64 * i];
    const float* row = logits + (int64_t)t * E;
    int id;
    float v;
    wave_topk([&](int e) { return row[e]; }, E, k, scr[threadIdx.x >> 6], id, v);
    float wt = wave_softmax_selected(v, k);
    if (lane < k) {
        ids[t * k + lane] = id;
        w[t * k + lane] = wt;
        if (ids2) ids2[t * k + lane] = id;
        if (w2) w2[t * k + lane] = wt;
    }
    uint2* xd = reinterpret_cast<uint2*>(x16 + (int64_t)t * H);
    auto cvt = [](uint2 q) {
        return make_uint2(
            pack2(f32_to_f16_bits(bf16_to_f32(q.x & 0xffffu)), f32_to_f16_bits(bf16_to_f32(q.x >> 16))),
            pack2(f32_to_f16_bits(bf16_to_f32(q.y & 0xffffu)), f32_to_f16_bits(bf16_to_f32(q.y >> 16))));
    };
#pragma unroll
    for (int i = 0; i < kPre; ++i)
        if (i < nx) xd[lane + 64 * i] = cvt(xr[i]);
    for (int i = kPre; i < nx; ++i) xd[lane + 64 * i] = cvt(xs[lane + 64 * i]);
}


// Block-wide exclusive scan of one int per thread (blockDim must be 1024).
// `total` receives the sum over the block.  lds: >= 33 ints.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* lds, int& total) {
    const int lane = __lane_id(), wid = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) lds[wid] = incl;
    __syncthreads();
    if (threadIdx.x < 64) {
        int s = (lane < 16) ? lds[lane] : 0;
        int si = s;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int o = __shfl_up(si, off, 64);
            if (lane >= off) si += o;
        }
        if (lane < 16) lds[16 + lane] = si - s;
        if (lane == 15) lds[32] = si;
    }
    __syncthreads();
    total = lds[32];
    int r = lds[16 + wid] + incl - v;
    __syncthreads();
    return r;
}

// Stable counting sort of the n = T*k slots of at most 16 tokens, by one
// workgroup of 1024 threads.  s_ids holds the expert of each slot and
// s_mask[e] the set of tokens (bit t) that selected expert e; a token
// selects an expert at most once, so the rank of slot (t, j) inside expert e
// is the number of set bits of s_mask[e] below bit t.  Writes offsets [E+1],
// perm, inv and (if `tiles`) the active experts as tiles (expert, first row,
// rows) in ascending expert order.
__device__ __forceinline__ void small_counting_sort(const int* s_ids, const uint32_t* s_mask,
                                                    int* s_first, int* s_scan, int T, int E, int k,
                                                    int32_t* offsets, int32_t* perm, int32_t* inv,
                                                    int32_t* tiles, int32_t* ntiles) {
    const int tid = threadIdx.x;
    const int c = (tid < E) ? __popc(s_mask[tid]) : 0;
    int tot_c, tot_a;
    const int off = block_excl_scan_1024(c, s_scan, tot_c);
    const int aidx = block_excl_scan_1024(c > 0 ? 1 : 0, s_scan, tot_a);
    if (tid < E) {
        offsets[tid] = off;
        s_first[tid] = off;
        if (c > 0 && tiles) {
            tiles[3 * aidx + 0] = tid;
            tiles[3 * aidx + 1] = off;
            tiles[3 * aidx + 2] = c;
        }
    }
    if (tid == 0) {
        offsets[E] = tot_c;
        if (ntiles) *ntiles = tot_a;
    }
    __syncthreads();
    if (tid < T * k) {
        const int t = tid / k, e = s_ids[tid];
        const int p = s_first[e] + __popc(s_mask[e] & ((1u << t) - 1u));
        perm[p] = tid;
        inv[tid] = p;
    }
}

// Stand-alone counting sort for T <= 16.
__global__ void __launch_bounds__(1024) k_permute_small(
    const int32_t* __restrict__ ids, int T, int E, int k, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int s_ids[16 * 32];
    __shared__ uint32_t s_mask[1024];
    __shared__ int s_first[1024];
    __shared__ int s_scan[40];
    const int tid = threadIdx.x;
    s_mask[tid] = 0u;
    __syncthreads();
    if (tid < T * k) {
        s_ids[tid] = ids[tid];
        atomicOr(&s_mask[ids[tid]], 1u << (tid / k));
    }
    __syncthreads();
    small_counting_sort(s_ids, s_mask, s_first, s_scan, T, E, k, offsets, perm, inv, nullptr,
                        nullptr);
}

// ---------------------------------------------------------------- permute
// Stable counting sort for any T, in chunks of 64 tokens (one per lane of a
// wave).  A token selects each expert at most once, so the rank of slot (t, j)
// inside its expert e is the number of earlier tokens that selected e: inside
// a chunk that is a popcount of a 64-bit token mask per expert; across chunks
// it is the running sum of the per-chunk counts.

// Per-chunk token masks -> per-chunk counts cnt[chunk][e].
__global__ void k_perm_count(const int32_t* __restrict__ ids, int T, int k, int E,
                             int32_t* __restrict__ hist) {
    __shared__ unsigned long long mask[1024];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) mask[e] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * 64 + lane;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicOr(&mask[ids[t * k + j]], 1ull << lane);
    __syncthreads();
    int32_t* h = hist + (int64_t)blockIdx.x * E;
    for (int e = lane; e < E; e += 64) h[e] = __popcll(mask[e]);
}

// One workgroup of 1024 threads: chunk bases per expert (exclusive running
// sums within the expert; the scatter adds the expert's offset), expert
// offsets, and the BM-row tile list.
__global__ void __launch_bounds__(1024) k_perm_scan(int32_t* __restrict__ hist, int nch, int E,
                                                    int BM, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ ntiles) {
    __shared__ int s_scan[40];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        int c = 0;
        for (; c + 32 <= nch; c += 32) {                  // 32 loads in flight
            int v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = hist[(int64_t)(c + u) * E + e];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                hist[(int64_t)(c + u) * E + e] = run;
                run += v[u];
            }
        }
        for (; c < nch; ++c) {
            int v = hist[(int64_t)c * E + e];
            hist[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    int tot, ntot;
    int off = block_excl_scan_1024(e < E ? run : 0, s_scan, tot);
    int nt = (e < E) ? (run + BM - 1) / BM : 0;
    int t0 = block_excl_scan_1024(nt, s_scan, ntot);
    if (e < E) {
        offsets[e] = off;
        for (int i = 0; i < nt; ++i) {
            tiles[3 * (t0 + i) + 0] = e;
            tiles[3 * (t0 + i) + 1] = off + i * BM;
            tiles[3 * (t0 + i) + 2] = min(BM, run - i * BM);
        }
    }
    if (e == 0) {
        offsets[E] = tot;
        ntiles[0] = ntot;
        ntiles[1] = 0;       // the down GEMM's fp16 range flag (the layer's workspace)
    }
}

__global__ void k_perm_scatter(const int32_t* __restrict__ ids, int T, int k, int E,
                               const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
                               int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ unsigned long long mask[1024];
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += 64) mask[e] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * 64 + lane;
    if (t < T)
        for (int j = 0; j < k; ++j) atomicOr(&mask[ids[t * k + j]], 1ull << lane);
    __syncthreads();
    if (t >= T) return;
    const int32_t* b = base + (int64_t)blockIdx.x * E;
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
        const int f = t * k + j;
        const int e = ids[f];
        const int p = offsets[e] + b[e] + __popcll(mask[e] & lt);
        perm[p] = f;
        inv[f] = p;
    }
}

// Tile list from given offsets (stage entry point): one thread per expert.
__global__ void __launch_bounds__(1024) k_build_tiles(const int32_t* __restrict__ offsets, int E,
                                                      int BM, int32_t* __restrict__ tiles,
                                                      int32_t* __restrict__ ntiles) {
    __shared__ int s_scan[40];
    const int e = threadIdx.x;
    int c = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    int nt = (c + BM - 1) / BM, tot;
    int t0 = block_excl_scan_1024(nt, s_scan, tot);
    if (e < E) {
        for (int i = 0; i < nt; ++i) {
            tiles[3 * (t0 + i) + 0] = e;
            tiles[3 * (t0 + i) + 1] = offsets[e] + i * BM;
            tiles[3 * (t0 + i) + 2] = min(BM, c - i * BM);
        }
    }
    if (e == 0) *ntiles = tot;
}

// ---------------------------------------------------------------- combine

// Four consecutive values of row `row` (float4 column c) of the unweighted
// routed rows: fp32, or fp16 (the grouped-GEMM path's range-checked form).
template <bool H16>
__device__ __forceinline__ float4 yrow4(const float* __restrict__ y_perm, int64_t row, int H, int c) {
    if constexpr (H16) {
        const uint2 v = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(y_perm) + row * H)[c];
        return make_float4(f16_bits_to_f32(v.x & 0xffffu), f16_bits_to_f32(v.x >> 16),
                           f16_bits_to_f32(v.y & 0xffffu), f16_bits_to_f32(v.y >> 16));
    } else {
        return reinterpret_cast<const float4*>(y_perm + row * H)[c];
    }
}

// Float4 column c of token t's combined output: sum_j w[t][j] *
// y_perm[inv[t k + j]][4c..4c+3] (j in order) + shared[t][4c..4c+3] (when
// given).  The rows are fp16 when h16, else fp32.  Four rows in flight.
__device__ __forceinline__ float4 combine4(const float* __restrict__ y_perm, bool h16,
                                           const int32_t* __restrict__ inv, const float* __restrict__ w,
                                           int t, int k, int H, const float* __restrict__ shared, int c) {
    auto sum = [&](auto h16c) {
        constexpr bool F16 = decltype(h16c)::value;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int j = 0;
        for (; j + 4 <= k; j += 4) {
            float4 v[4];
            float wt[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                wt[u] = w[t * k + j + u];
                v[u] = yrow4<F16>(y_perm, inv[t * k + j + u], H, c);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc.x += wt[u] * v[u].x;
                acc.y += wt[u] * v[u].y;
                acc.z += wt[u] * v[u].z;
                acc.w += wt[u] * v[u].w;
            }
        }
        for (; j < k; ++j) {
            const float wt = w[t * k + j];
            const float4 v = yrow4<F16>(y_perm, inv[t * k + j], H, c);
            acc.x += wt * v.x;
            acc.y += wt * v.y;
            acc.z += wt * v.z;
            acc.w += wt * v.w;
        }
        return acc;
    };
    float4 acc = h16 ? sum(std::true_type{}) : sum(std::false_type{});
    if (shared) {
        const float4 sv = *reinterpret_cast<const float4*>(shared + (int64_t)t * H + 4 * c);
        acc.x += sv.x;
        acc.y += sv.y;
        acc.z += sv.z;
        acc.w += sv.w;
    }
    return acc;
}

// y[t][h..h+3] = combine4(t, h / 4).  The rows are fp16 when fp16_unless is
// given and *fp16_unless == 0 (the down GEMM's range check passed), else
// fp32.  One float4 column per thread.
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y_perm,
                                                       const int* __restrict__ fp16_unless,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w, int k, int H,
                                                       const float* __restrict__ shared,
                                                       float* __restrict__ y) {
    // block b: token b / ncb, float4 columns 256 (b % ncb) .. +255 (a
    // one-dimensional grid: any T up to the library's limit)
    const int ncb = (H / 4 + 255) / 256;
    const int t = blockIdx.x / ncb;
    const int c = (blockIdx.x - t * ncb) * blockDim.x + threadIdx.x, h = 4 * c;
    if (h >= H) return;
    const bool h16 = fp16_unless && *fp16_unless == 0;
    *reinterpret_cast<float4*>(y + (int64_t)t * H + h) = combine4(y_perm, h16, inv, w, t, k, H, shared, c);
}

// ---------------------------------------------------------------- RMSNorm

// One workgroup (256 threads) per token row; the general form (any H).
__global__ void k_rmsnorm_residual(float* __restrict__ h, const float* __restrict__ delta,
                                   const float* __restrict__ gamma, float eps, int H,
                                   uint16_t* __restrict__ normed) {
    __shared__ float s_red[4];
    float* row = h + (int64_t)blockIdx.x * H;
    const float* drow = delta ? delta + (int64_t)blockIdx.x * H : nullptr;
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += blockDim.x) {
        float v = row[i];
        if (drow) {
            v += drow[i];
            row[i] = v;
        }
        ss += v * v;
    }
    if (!normed) return;
    ss = wave_sum_f32(ss);
    if (__lane_id() == 0) s_red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += s_red[i];
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    uint16_t* nrow = normed + (int64_t)blockIdx.x * H;
    for (int i = threadIdx.x; i < H; i += blockDim.x)
        nrow[i] = (uint16_t)f32_to_bf16(gamma[i] * (row[i] * r));
}

// Register form for rows of H = 4m floats (m <= 2048) with 16-byte aligned
// operands: one block of TPB = min(m rounded up to 64, 1024) threads per row,
// thread i holding float4 columns i + TPB j (j < NV) in registers between the
// residual add, the sum of squares and the scaling, so the row is read once
// and written once (the bf16 output as 8-byte stores).  The sum of squares is
// reduced in a fixed order: per thread, per wave, then the waves' sums in
// wave order.
template <int NV>
__device__ __forceinline__ void norm_row(const float4 (&v)[NV], int n4, int H, const float* __restrict__ gamma,
                                         float eps, uint16_t* __restrict__ normed_row, float* s_red) {
    const int tpb = blockDim.x;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum_f32(ss);
    if (__lane_id() == 0) s_red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int q = 0; q < (tpb >> 6); ++q) tot += s_red[q];
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    const float4* g4 = reinterpret_cast<const float4*>(gamma);
    uint2* nrow = reinterpret_cast<uint2*>(normed_row);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = threadIdx.x + tpb * j;
        if (i < n4) {
            const float4 g = g4[i];
            uint2 o;
            o.x = f32_to_bf16(g.x * (v[j].x * r)) | (f32_to_bf16(g.y * (v[j].y * r)) << 16);
            o.y = f32_to_bf16(g.z * (v[j].z * r)) | (f32_to_bf16(g.w * (v[j].w * r)) << 16);
            nrow[i] = o;
        }
    }
}

template <int NV, bool DELTA>
__global__ void __launch_bounds__(1024) k_rmsnorm_residual_v(float* __restrict__ h, const float* __restrict__ delta,
                                                             const float* __restrict__ gamma, float eps, int H,
                                                             uint16_t* __restrict__ normed) {
    __shared__ float s_red[16];
    const int n4 = H >> 2, tpb = blockDim.x;
    float4* row = reinterpret_cast<float4*>(h + (int64_t)blockIdx.x * H);
    float4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = threadIdx.x + tpb * j;
        v[j] = i < n4 ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (DELTA) {
        const float4* drow = reinterpret_cast<const float4*>(delta + (int64_t)blockIdx.x * H);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = threadIdx.x + tpb * j;
            if (i < n4) {
                const float4 d = drow[i];
                v[j].x += d.x;
                v[j].y += d.y;
                v[j].z += d.z;
                v[j].w += d.w;
                row[i] = v[j];
            }
        }
    }
    if (!normed) return;
    norm_row<NV>(v, n4, H, gamma, eps, normed + (int64_t)blockIdx.x * H, s_red);
}

// The layer's combine fused with the residual add and the next layer's
// RMSNorm, in the register form above: h[t] += combine4(t, .) and, with
// gamma, normed[t] = bf16(gamma * h[t] / sqrt(mean(h[t]^2) + eps)).  The same
// column mapping, sums and reduction as k_combine followed by
// k_rmsnorm_residual_v, so the results are the same bits.
template <int NV>
__global__ void __launch_bounds__(1024) k_combine_norm(const float* __restrict__ y_perm,
                                                       const int* __restrict__ fp16_unless,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w, int k, int H,
                                                       const float* __restrict__ shared, float* __restrict__ h,
                                                       const float* __restrict__ gamma, float eps,
                                                       uint16_t* __restrict__ normed) {
    __shared__ float s_red[16];
    const int t = blockIdx.x, n4 = H >> 2, tpb = blockDim.x;
    const bool h16 = fp16_unless && *fp16_unless == 0;
    float4* row = reinterpret_cast<float4*>(h + (int64_t)t * H);
    float4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = threadIdx.x + tpb * j;
        v[j] = i < n4 ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = threadIdx.x + tpb * j;
        if (i < n4) {
            const float4 d = combine4(y_perm, h16, inv, w, t, k, H, shared, i);
            v[j].x += d.x;
            v[j].y += d.y;
            v[j].z += d.z;
            v[j].w += d.w;
            row[i] = v[j];
        }
    }
    if (!normed) return;
    norm_row<NV>(v, n4, H, gamma, eps, normed + (int64_t)t * H, s_red);
}

// ---------------------------------------------------------------- kernel-path dequant
// Dequantization through the table decoders that the layer's kernels inline
// (moe_decoders.hpp): the same table fill, the same lookup addresses, the
// same fp16 multiply by the sub-scale or by d, then the factor each kernel
// applies in fp32 afterwards (d / 128, or d s / 128, on the partial sums of a
// block or sub-block; the NL4 fold's 1 / 16).  One thread per 32 weights:
// a 32-weight sub-block (Q3S-256, Q2S-256, NL4S-256), a 32-weight block
// (NL4-32, Q2-32) or two 16-weight sub-blocks (Q3K-256), read from the block
// bytes as the format lays them out.
enum { kDqpQ3Pair, kDqpQ3Quad, kDqpNl4Pair, kDqpNl4Fold, kDqpQ2S, kDqpQ2, kDqpQ3K, kDqpNl4S };

// Weights 8 C .. 8 C + 7 of a Q3S sub-block from the pair table, times s.
template <int C>
__device__ __forceinline__ void q3_pair_decode8(const uint32_t* w, uint32_t base, f16x2_t s2, uint32_t (&f)[4]) {
    f[0] = mul_pair(lds_ld(q3_pair_addr<24 * C + 0>(w, base)), s2);
    f[1] = mul_pair(lds_ld(q3_pair_addr<24 * C + 6>(w, base)), s2);
    f[2] = mul_pair(lds_ld(q3_pair_addr<24 * C + 12>(w, base)), s2);
    f[3] = mul_pair(lds_ld(q3_pair_addr<24 * C + 18>(w, base)), s2);
}
// Weights 8 C .. 8 C + 7 of a 2-bit index word pair from the nibble table, times m.
template <int C>
__device__ __forceinline__ void nib_decode8(const uint32_t (&ix)[2], uint32_t base, f16x2_t m2, uint32_t (&f)[4]) {
    f[0] = mul_pair(lds_ld(nib_lut_addr<16 * C + 0>(ix, base)), m2);
    f[1] = mul_pair(lds_ld(nib_lut_addr<16 * C + 4>(ix, base)), m2);
    f[2] = mul_pair(lds_ld(nib_lut_addr<16 * C + 8>(ix, base)), m2);
    f[3] = mul_pair(lds_ld(nib_lut_addr<16 * C + 12>(ix, base)), m2);
}
// The four pairs of one index word nb (8 NL4 weights), table entries SH apart.
template <int SH>
__device__ __forceinline__ void nl4_read8(uint32_t nb, uint32_t base, uint32_t (&f)[4]) {
    f[0] = lds_ld(nl4_byte_addr<0, SH>(nb, base));
    f[1] = lds_ld(nl4_byte_addr<1, SH>(nb, base));
    f[2] = lds_ld(nl4_byte_addr<2, SH>(nb, base));
    f[3] = lds_ld(nl4_byte_addr<3, SH>(nb, base));
}
// Sign-extended 6-bit field at bit b of a 96-bit little-endian string.
__device__ __forceinline__ int field6(const uint32_t (&w)[3], int b) {
    const int wd = b >> 5, o = b & 31;
    uint32_t v = w[wd] >> o;
    if (o > 26) v |= w[wd + 1] << (32 - o);
    return sext6(v & 63u);
}

template <int V>
__global__ void __launch_bounds__(256) k_dequant_path(const uint8_t* __restrict__ blocks, int64_t n_units,
                                                      float* __restrict__ out) {
    constexpr int kDw = (V == kDqpQ3Pair || V == kDqpQ3K) ? kQ3LutDw : V == kDqpQ3Quad ? kQ3QuadDw
                        : (V == kDqpNl4Pair || V == kDqpNl4Fold) ? kNl4LutDw : V == kDqpNl4S ? 256 * 16 : kNibLutDw;
    __shared__ __attribute__((aligned(32768))) uint32_t lut[kDw];
    const int tid = threadIdx.x, lane = __lane_id();
    if constexpr (V == kDqpQ3Pair || V == kDqpQ3K) q3_pair_table_fill(lut, tid, 256);
    else if constexpr (V == kDqpQ3Quad) q3_quad_table_fill(lut, tid, 256);
    else if constexpr (V == kDqpNl4Pair) nl4_pair_table_fill<32>(lut, tid, 256);
    else if constexpr (V == kDqpNl4Fold) nl4_fold_table_fill(lut, tid, 256);
    else if constexpr (V == kDqpNl4S) nl4_pair_table_fill<16>(lut, tid, 256);
    else nib_table_fill<V == kDqpQ2S>(lut, tid, 256);
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * 256 + tid;
    if (i >= n_units) return;
    float* o = out + i * 32;
    const uint32_t base32 = lut_copy_base(lds_addr(lut), lane);
    uint32_t f[4][4];                                  // 4 groups of 8 weights as fp16 pairs
    float scale;
    if constexpr (V == kDqpQ3Pair || V == kDqpQ3Quad) {
        const uint8_t* b = blocks + (i >> 3) * kQ3Bytes;
        const int j = (int)(i & 7);
        const uint32_t* ip = reinterpret_cast<const uint32_t*>(b + 12 * j);
        const uint32_t q[3] = {ip[0], ip[1], ip[2]};
        const uint64_t tail = *reinterpret_cast<const uint64_t*>(b + 96);
        const _Float16 s = (_Float16)(float)q3_tail_s(tail, j);
        const f16x2_t s2 = {s, s};
        scale = q3_tail_d(tail) * 0.0078125f;
        if constexpr (V == kDqpQ3Pair) {
            q3_pair_decode8<0>(q, base32, s2, f[0]);
            q3_pair_decode8<1>(q, base32, s2, f[1]);
            q3_pair_decode8<2>(q, base32, s2, f[2]);
            q3_pair_decode8<3>(q, base32, s2, f[3]);
        } else {
            const uint32_t base = lds_addr(lut);
            q3_quad_decode8<0>(q, base, s2, f[0]);
            q3_quad_decode8<1>(q, base, s2, f[1]);
            q3_quad_decode8<2>(q, base, s2, f[2]);
            q3_quad_decode8<3>(q, base, s2, f[3]);
        }
    } else if constexpr (V == kDqpNl4Pair || V == kDqpNl4Fold) {
        // 18-byte blocks are 2-byte aligned: d and the index bytes as halves
        const uint16_t* h = reinterpret_cast<const uint16_t*>(blocks + i * kNL4Bytes);
        const uint32_t dbits = h[0];
        const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)dbits);
        const f16x2_t d2 = {d, d};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            nl4_read8<7>((uint32_t)h[1 + 2 * c] | ((uint32_t)h[2 + 2 * c] << 16), base32, f[c]);
            if constexpr (V == kDqpNl4Fold) {
#pragma unroll
                for (int p = 0; p < 4; ++p) f[c][p] = mul_pair(f[c][p], d2);
            }
        }
        scale = V == kDqpNl4Fold ? 0.0625f : f16_bits_to_f32(dbits) * 0.0078125f;
    } else if constexpr (V == kDqpQ2S) {
        const uint8_t* b = blocks + (i >> 3) * kQ2SBytes;
        const int j = (int)(i & 7);
        const uint32_t* ip = reinterpret_cast<const uint32_t*>(b + 8 * j);
        const uint32_t ix[2] = {ip[0], ip[1]};
        const uint64_t tail = *reinterpret_cast<const uint64_t*>(b + 64);
        const _Float16 s = (_Float16)(float)q3_tail_s(tail, j);
        const f16x2_t s2 = {s, s};
        scale = q3_tail_d(tail) * 0.0078125f;
        nib_decode8<0>(ix, base32, s2, f[0]);
        nib_decode8<1>(ix, base32, s2, f[1]);
        nib_decode8<2>(ix, base32, s2, f[2]);
        nib_decode8<3>(ix, base32, s2, f[3]);
    } else if constexpr (V == kDqpQ2) {
        // 10-byte blocks are 2-byte aligned
        const uint16_t* h = reinterpret_cast<const uint16_t*>(blocks + i * kQ2Bytes);
        const _Float16 d = __builtin_bit_cast(_Float16, h[0]);
        const f16x2_t d2 = {d, d};
        const uint32_t ix[2] = {(uint32_t)h[1] | ((uint32_t)h[2] << 16), (uint32_t)h[3] | ((uint32_t)h[4] << 16)};
        scale = 1.0f;
        nib_decode8<0>(ix, base32, d2, f[0]);
        nib_decode8<1>(ix, base32, d2, f[1]);
        nib_decode8<2>(ix, base32, d2, f[2]);
        nib_decode8<3>(ix, base32, d2, f[3]);
    } else if constexpr (V == kDqpQ3K) {
        // 110-byte blocks are 2-byte aligned: read as halves.  This thread's
        // sub-blocks j0, j0 + 1 (16 weights, 6 index bytes at 6 j each), d at
        // byte 96, the 6-bit sub-scales at bits 6 j of the 96-bit field at 98
        const uint16_t* h = reinterpret_cast<const uint16_t*>(blocks + (i >> 3) * kQ3KBytes);
        const int j0 = 2 * (int)(i & 7);
        const float dl = f16_bits_to_f32(h[48]) * 0.0078125f;
        const uint32_t sw[3] = {(uint32_t)h[49] | ((uint32_t)h[50] << 16), (uint32_t)h[51] | ((uint32_t)h[52] << 16),
                                (uint32_t)h[53] | ((uint32_t)h[54] << 16)};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = j0 + u;
            const uint64_t w48 = (uint64_t)h[3 * j] | ((uint64_t)h[3 * j + 1] << 16) | ((uint64_t)h[3 * j + 2] << 32);
            f16x2_t lo2, hi2;
            q3k_split(field6(sw, 6 * j), lo2, hi2);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const uint32_t fw[1] = {(uint32_t)(w48 >> (24 * g)) & 0xFFFFFFu};
                const uint32_t fb[4] = {lds_ld(q3_pair_addr<0>(fw, base32)), lds_ld(q3_pair_addr<6>(fw, base32)),
                                        lds_ld(q3_pair_addr<12>(fw, base32)), lds_ld(q3_pair_addr<18>(fw, base32))};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    // the two exact parts, as the two MFMAs sum them, then d / 128
                    const f16x2_t b1 = __builtin_bit_cast(f16x2_t, mul_pair(fb[p], lo2));
                    const f16x2_t b2 = __builtin_bit_cast(f16x2_t, mul_pair(fb[p], hi2));
                    o[16 * u + 8 * g + 2 * p] = ((float)b1[0] + (float)b2[0]) * dl;
                    o[16 * u + 8 * g + 2 * p + 1] = ((float)b1[1] + (float)b2[1]) * dl;
                }
            }
        }
        return;
    } else {
        // NL4S-256: 136-byte blocks, 8-byte aligned; sub-block j's 16 index
        // bytes at 16 j, d at 128, the 6-bit sub-scales at bits 6 j of the
        // 48-bit field at 130; table in 16 copies
        const uint8_t* b = blocks + (i >> 3) * kNL4SBytes;
        const int j = (int)(i & 7);
        const uint32_t* ip = reinterpret_cast<const uint32_t*>(b + 16 * j);
        const uint16_t* h = reinterpret_cast<const uint16_t*>(b);
        const uint32_t sw[3] = {(uint32_t)h[65] | ((uint32_t)h[66] << 16), (uint32_t)h[67], 0u};
        scale = f16_bits_to_f32(h[64]) * 0.0078125f * (float)field6(sw, 6 * j);
        const uint32_t base16 = lds_addr(lut) + (uint32_t)(lane & 15) * 4u;
#pragma unroll
        for (int c = 0; c < 4; ++c) nl4_read8<6>(ip[c], base16, f[c]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f16x2_t v = __builtin_bit_cast(f16x2_t, f[c][p]);
            o[8 * c + 2 * p] = (float)v[0] * scale;
            o[8 * c + 2 * p + 1] = (float)v[1] * scale;
        }
}

// ---------------------------------------------------------------- launchers

static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

void launch_dequant(int fmt, const void* blocks, int64_t n_weights, float* out, hipStream_t st) {
    const int64_t n32 = n_weights / 32;              // sub-blocks / blocks of 32 weights
    const uint8_t* b = (const uint8_t*)blocks;
    if (fmt == kFmtQ3S256) k_dequant_q3s<<<cdiv(n32, 256), 256, 0, st>>>(b, n32, out);
    else if (fmt == kFmtNL4) k_dequant_nl4<<<cdiv(n32, 256), 256, 0, st>>>(b, n32, out);
    else if (fmt == kFmtQ2S256) k_dequant_q2s<<<cdiv(n32, 256), 256, 0, st>>>(b, n32, out);
    else if (fmt == kFmtQ3K256) k_dequant_q3k<<<cdiv(2 * n32, 256), 256, 0, st>>>(b, 2 * n32, out);
    else if (fmt == kFmtNL4S256) k_dequant_nl4s<<<cdiv(n32, 256), 256, 0, st>>>(b, n32, out);
    else k_dequant_q2<<<cdiv(n32, 256), 256, 0, st>>>(b, n32, out);
}

void launch_dequant_path(int fmt, int path, const void* blocks, int64_t n_weights, float* out, hipStream_t st) {
    const int64_t n32 = n_weights / 32;
    const uint8_t* b = (const uint8_t*)blocks;
    const unsigned grid = cdiv(n32, 256);
#define MOE_DQP(V) k_dequant_path<V><<<grid, 256, 0, st>>>(b, n32, out)
    if (fmt == kFmtQ3S256) {
        if (path == 0) MOE_DQP(kDqpQ3Pair);
        else MOE_DQP(kDqpQ3Quad);
    } else if (fmt == kFmtNL4) {
        if (path == 0) MOE_DQP(kDqpNl4Pair);
        else MOE_DQP(kDqpNl4Fold);
    } else if (fmt == kFmtQ2S256) {
        MOE_DQP(kDqpQ2S);
    } else if (fmt == kFmtQ2) {
        MOE_DQP(kDqpQ2);
    } else if (fmt == kFmtQ3K256) {
        MOE_DQP(kDqpQ3K);
    } else {
        MOE_DQP(kDqpNl4S);
    }
#undef MOE_DQP
}

void launch_to_f16(const uint16_t* x, uint16_t* x16, int64_t n, hipStream_t st) {
    k_to_f16<<<cdiv(cdiv(n, 4), 256), 256, 0, st>>>(x, x16, n);
}

void launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 int32_t* ids2, float* w2, const uint16_t* x, uint16_t* x16, int H, hipStream_t st) {
    k_topk<<<cdiv(T, 4), 256, 0, st>>>(logits, T, E, k, ids, w, ids2, w2, x, x16, H);
}

void launch_permute_small(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t st) {
    k_permute_small<<<1, 1024, 0, st>>>(ids, T, E, k, offsets, perm, inv);
}

void launch_permute_large(const int32_t* ids, int T, int k, int E, int BM, int32_t* hist,
                          int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles,
                          int32_t* ntiles, hipStream_t st) {
    const int nch = (int)cdiv(T, 64);
    k_perm_count<<<nch, 64, 0, st>>>(ids, T, k, E, hist);
    k_perm_scan<<<1, 1024, 0, st>>>(hist, nch, E, BM, offsets, tiles, ntiles);
    k_perm_scatter<<<nch, 64, 0, st>>>(ids, T, k, E, hist, offsets, perm, inv);
}

void launch_build_tiles(const int32_t* offsets, int E, int BM, int32_t* tiles, int32_t* ntiles,
                        hipStream_t st) {
    k_build_tiles<<<1, 1024, 0, st>>>(offsets, E, BM, tiles, ntiles);
}

void launch_combine(const float* y_perm, const int* fp16_unless, const int32_t* inv, const float* w,
                    int T, int k, int H, const float* shared, float* y, hipStream_t st) {
    k_combine<<<(unsigned)(cdiv(H / 4, 256) * T), 256, 0, st>>>(y_perm, fp16_unless, inv, w, k, H, shared, y);
}

// Block width of the register-form row kernels: m = H / 4 float4 columns,
// one per thread up to 1024 (rounded up to whole waves), two beyond.
static inline int row_tpb(int H) {
    const int n4 = H >> 2;
    return n4 <= 1024 ? ((n4 + 63) & ~63) : 1024;
}

void launch_combine_norm(const float* y_perm, const int* fp16_unless, const int32_t* inv, const float* w,
                         int T, int k, int H, const float* shared, float* h, const float* gamma,
                         float eps, uint16_t* normed, hipStream_t st) {
    const int tpb = row_tpb(H);
    if ((H >> 2) <= 1024)
        k_combine_norm<1><<<T, tpb, 0, st>>>(y_perm, fp16_unless, inv, w, k, H, shared, h, gamma, eps, normed);
    else
        k_combine_norm<2><<<T, tpb, 0, st>>>(y_perm, fp16_unless, inv, w, k, H, shared, h, gamma, eps, normed);
}

void launch_rmsnorm(float* h, const float* delta, const float* gamma, float eps, int T, int H,
                    uint16_t* normed, hipStream_t st) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    const bool vec = (H & 3) == 0 && H <= 8192 && a16(h) && (!delta || a16(delta)) &&
                     (!normed || (a16(gamma) && ((uintptr_t)normed & 7) == 0));
    const int tpb = row_tpb(H);
    if (!vec) {
        k_rmsnorm_residual<<<T, 256, 0, st>>>(h, delta, gamma, eps, H, normed);
    } else if ((H >> 2) <= 1024) {
        if (delta) k_rmsnorm_residual_v<1, true><<<T, tpb, 0, st>>>(h, delta, gamma, eps, H, normed);
        else k_rmsnorm_residual_v<1, false><<<T, tpb, 0, st>>>(h, delta, gamma, eps, H, normed);
    } else {
        if (delta) k_rmsnorm_residual_v<2, true><<<T, tpb, 0, st>>>(h, delta, gamma, eps, H, normed);
        else k_rmsnorm_residual_v<2, false><<<T, tpb, 0, st>>>(h, delta, gamma, eps, H, normed);
    }
}

}  // namespace moe
