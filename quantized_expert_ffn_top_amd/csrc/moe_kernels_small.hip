// Latency-bound kernels of the layer: dequantization (debug export), fp16
// staging of the tokens, exact top-k routing, the counting-sort permutation,
// the expert tile list, the weighted combine and the inter-layer RMSNorm.
//
// Routing: every token goes to the k largest router logits ("Avalon" README,
// opening paragraphs: 10 of 512 experts), ordered by (value desc, index asc),
// with softmax weights over the selected logits; nothing is pruned or
// dropped ("Betelgeuse" post: every routed expert is computed).
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
__global__ void k_topk(const float* __restrict__ logits, int T, int E, int k,
                       int32_t* __restrict__ ids, float* __restrict__ w,
                       int32_t* __restrict__ ids2, float* __restrict__ w2) {
    __shared__ uint64_t scr[4][kTopkScratch];
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (int64_t)t * E;
    int id;
    float v;
    wave_topk([&](int e) { return row[e]; }, E, k, scr[threadIdx.x >> 6], id, v);
    float wt = wave_softmax_selected(v, k);
    const int lane = __lane_id();
    if (lane < k) {
        ids[t * k + lane] = id;
        w[t * k + lane] = wt;
        if (ids2) ids2[t * k + lane] = id;
        if (w2) w2[t * k + lane] = wt;
    }
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
        *ntiles = ntot;
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

// y[t][h] = sum_j w[t][j] * y_perm[inv[t*k+j]][h] (+ shared[t][h]); 4 h per thread.
// y[t][h..h+3] = sum_j w[t][j] * y_perm[inv[t k + j]][h..h+3] (j in order)
// + shared[t][h..h+3]; y_perm fp32 or fp16.
template <typename YT>
__device__ __forceinline__ float4 load4(const YT* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_float4(f16_bits_to_f32(v.x & 0xffffu), f16_bits_to_f32(v.x >> 16),
                       f16_bits_to_f32(v.y & 0xffffu), f16_bits_to_f32(v.y >> 16));
}
template <typename YT>
__global__ void k_combine(const YT* __restrict__ y_perm, const int32_t* __restrict__ inv,
                          const float* __restrict__ w, int T, int k, int H,
                          const float* __restrict__ shared, float* __restrict__ y) {
    const int t = blockIdx.y;
    const int h = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (h >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = 0;
    for (; j + 4 <= k; j += 4) {                      // four rows in flight
        float4 v[4];
        float wt[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            wt[u] = w[t * k + j + u];
            v[u] = load4(y_perm + (int64_t)inv[t * k + j + u] * H + h);
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
        const float4 v = load4(y_perm + (int64_t)inv[t * k + j] * H + h);
        acc.x += wt * v.x;
        acc.y += wt * v.y;
        acc.z += wt * v.z;
        acc.w += wt * v.w;
    }
    if (shared) {
        const float4 s = *reinterpret_cast<const float4*>(shared + (int64_t)t * H + h);
        acc.x += s.x;
        acc.y += s.y;
        acc.z += s.z;
        acc.w += s.w;
    }
    *reinterpret_cast<float4*>(y + (int64_t)t * H + h) = acc;
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

// The same for rows of H = 4m <= 1024 NV floats with 16-byte aligned operands:
// each thread keeps its NV float4 of the row in registers between the sum of
// squares and the scaling, so the row is read once and written once (with the
// bf16 output as 8-byte stores).
template <int NV, bool DELTA>
__global__ void __launch_bounds__(256) k_rmsnorm_residual_v(float* __restrict__ h, const float* __restrict__ delta,
                                                            const float* __restrict__ gamma, float eps, int H,
                                                            uint16_t* __restrict__ normed) {
    __shared__ float s_red[4];
    const int n4 = H >> 2;
    float4* row = reinterpret_cast<float4*>(h + (int64_t)blockIdx.x * H);
    float4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = threadIdx.x + 256 * j;
        v[j] = i < n4 ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (DELTA) {
        const float4* drow = reinterpret_cast<const float4*>(delta + (int64_t)blockIdx.x * H);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = threadIdx.x + 256 * j;
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
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum_f32(ss);
    if (__lane_id() == 0) s_red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    const float4* g4 = reinterpret_cast<const float4*>(gamma);
    uint2* nrow = reinterpret_cast<uint2*>(normed + (int64_t)blockIdx.x * H);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = threadIdx.x + 256 * j;
        if (i < n4) {
            const float4 g = g4[i];
            uint2 o;
            o.x = f32_to_bf16(g.x * (v[j].x * r)) | (f32_to_bf16(g.y * (v[j].y * r)) << 16);
            o.y = f32_to_bf16(g.z * (v[j].z * r)) | (f32_to_bf16(g.w * (v[j].w * r)) << 16);
            nrow[i] = o;
        }
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
    else k_dequant_q2<<<cdiv(n32, 256), 256, 0, st>>>(b, n32, out);
}

void launch_to_f16(const uint16_t* x, uint16_t* x16, int64_t n, hipStream_t st) {
    k_to_f16<<<cdiv(cdiv(n, 4), 256), 256, 0, st>>>(x, x16, n);
}

void launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 int32_t* ids2, float* w2, hipStream_t st) {
    k_topk<<<cdiv(T, 4), 256, 0, st>>>(logits, T, E, k, ids, w, ids2, w2);
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

void launch_combine(const float* y_perm, const int32_t* inv, const float* w, int T, int k, int H,
                    const float* shared, float* y, hipStream_t st) {
    dim3 grid(cdiv(H / 4, 256), T);
    k_combine<float><<<grid, 256, 0, st>>>(y_perm, inv, w, T, k, H, shared, y);
}

void launch_combine16(const uint16_t* y_perm16, const int32_t* inv, const float* w, int T, int k,
                      int H, const float* shared, float* y, hipStream_t st) {
    dim3 grid(cdiv(H / 4, 256), T);
    k_combine<uint16_t><<<grid, 256, 0, st>>>(y_perm16, inv, w, T, k, H, shared, y);
}

void launch_rmsnorm(float* h, const float* delta, const float* gamma, float eps, int T, int H,
                    uint16_t* normed, hipStream_t st) {
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    const bool vec = (H & 3) == 0 && H <= 8192 && a16(h) && (!delta || a16(delta)) &&
                     (!normed || (a16(gamma) && ((uintptr_t)normed & 7) == 0));
    if (!vec) {
        k_rmsnorm_residual<<<T, 256, 0, st>>>(h, delta, gamma, eps, H, normed);
    } else if (H <= 4096) {
        if (delta) k_rmsnorm_residual_v<4, true><<<T, 256, 0, st>>>(h, delta, gamma, eps, H, normed);
        else k_rmsnorm_residual_v<4, false><<<T, 256, 0, st>>>(h, delta, gamma, eps, H, normed);
    } else {
        if (delta) k_rmsnorm_residual_v<8, true><<<T, 256, 0, st>>>(h, delta, gamma, eps, H, normed);
        else k_rmsnorm_residual_v<8, false><<<T, 256, 0, st>>>(h, delta, gamma, eps, H, normed);
    }
}

}  // namespace moe
