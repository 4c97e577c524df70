// Device-side helpers shared by the libmoe kernels (gfx950 only).
//
// Block codecs decoded here (model card "Qwen3.8-Flash-Next - Avalon GGUF",
// "Files / Main model": routed up/gate at 3.25 bpw with a scale per
// 256-weight block and sub-scales per 32 weights; routed down in a 4-bit
// non-linear 32-weight type).  Byte layouts (a reading; the page gives none):
//   Q3S-256, 104 B: [0,96) 3-bit indices, LSB-first stream; [96,98) fp16 d;
//                   [98,102) eight signed nibbles s_j; [102,104) reserved.
//                   w = d * s_j * C3[q] / 128.
//   NL4-32,   18 B: [0,2) fp16 d; [2,18) 4-bit indices, even weight in the
//                   low nibble.  w = d * T4[q] / 128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Codebooks (value = entry / 128): int8 levels at normal quantiles, sorted,
// asymmetric with an exact zero.
__constant__ const int8_t kC3[8] = {-127, -67, -31, 0, 23, 48, 78, 127};
__constant__ const int8_t kT4[16] = {-127, -88, -66, -50, -36, -23, -11, 0,
                                     10, 20, 31, 43, 56, 71, 91, 127};

// 2-bit codebook of the 2.5-bpw up/gate codec, by the same rule.
__constant__ const int8_t kC2[4] = {-127, 0, 54, 127};

constexpr int kQ3Bytes = 104;
constexpr int kQ3Weights = 256;
constexpr int kNL4Bytes = 18;
constexpr int kNL4Weights = 32;
constexpr int kQ2SBytes = 80;
constexpr int kQ2Bytes = 10;
constexpr int kQ3KBytes = 110;      // Q3K-256: 96 index bytes, fp16 d, 16 six-bit sub-scales
constexpr int kNL4SBytes = 136;     // NL4S-256: 128 index bytes, fp16 d, 8 six-bit sub-scales

// Format numbers (the C ABI's moe_format) and their block sizes.
constexpr int kFmtQ3S256 = 2, kFmtNL4 = 3, kFmtQ2S256 = 4, kFmtQ2 = 5, kFmtQ3K256 = 6, kFmtNL4S256 = 7;
__host__ __device__ constexpr int fmt_block_weights(int f) {
    return (f == kFmtQ3S256 || f == kFmtQ2S256 || f == kFmtQ3K256 || f == kFmtNL4S256) ? 256 : 32;
}
__host__ __device__ constexpr int fmt_block_bytes(int f) {
    return f == kFmtQ3S256 ? kQ3Bytes : f == kFmtNL4 ? kNL4Bytes : f == kFmtQ2S256 ? kQ2SBytes
           : f == kFmtQ3K256 ? kQ3KBytes : f == kFmtNL4S256 ? kNL4SBytes : kQ2Bytes;
}
// bytes of a [rows][cols] matrix, blocks along cols
__host__ __device__ constexpr int64_t fmt_matrix_bytes(int f, int rows, int cols) {
    return (int64_t)rows * (cols / fmt_block_weights(f)) * fmt_block_bytes(f);
}

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two fp16 halves packed into one dword.
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) {
    return (lo & 0xffffu) | (hi << 16);
}

// ---------------------------------------------------------------- MFMA
// 16x16x32: lane l holds A[l%16][8(l/16) .. 8(l/16)+7], B[same k][l%16];
// D lane l holds D[4(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 32x32x16: lane l holds A[l%32][8(l/32) .. +7], B[same k][l%32];
// D lane l, register r holds D[8(r/4) + 4(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS by address
// 32-bit LDS addresses, so that table lookups compose their address with
// integer and/or operations (one v_and_or_b32 per lookup).
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_u32*)p;
}
__device__ __forceinline__ uint32_t lds_ld(uint32_t a) {
    return *(const lds_u32*)(uintptr_t)a;
}

// ---------------------------------------------------------------- loads

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ uint32_t ld4(const void* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}
// Streaming (read-once) 16-byte load: bypass-friendly cache policy.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- top-k
// Total order used by the routing: larger logit first, then lower expert
// index.  Logits are compared through an order-preserving u32 key (-0.0 is
// folded onto +0.0 so equal values compare equal).
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave-wide max / min of a u32 through DPP row permutations (max over each
// 16-lane row) and four lane reads; the result is wave-uniform.
// (Every lane of a full row is a valid source for these patterns, so the
// moves carry no old value and fold into the max / min as DPP operands.)
#define MOE_DPP(v, ctrl) ((uint32_t)__builtin_amdgcn_mov_dpp((int)(v), (ctrl), 0xF, 0xF, true))
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, MOE_DPP(v, 0xB1));                  // xor 1
    v = max(v, MOE_DPP(v, 0x4E));                  // xor 2
    v = max(v, MOE_DPP(v, 0x141));                 // half mirror
    v = max(v, MOE_DPP(v, 0x140));                 // mirror
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, MOE_DPP(v, 0xB1));
    v = min(v, MOE_DPP(v, 0x4E));
    v = min(v, MOE_DPP(v, 0x141));
    v = min(v, MOE_DPP(v, 0x140));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return min(min(a, b), min(c, d));
}
#undef MOE_DPP

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Wave-wide sum of a float through DPP (sums of 16-lane rows, then the four
// row sums added as (r0 + r1) + (r2 + r3)); the result is wave-uniform and
// the same for equal inputs.
__device__ __forceinline__ float wave_sum_f32_dpp(float v) {
#define MOE_DPPF(x, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), (ctrl), 0xF, 0xF, true))
    v += MOE_DPPF(v, 0xB1);                        // xor 1
    v += MOE_DPPF(v, 0x4E);                        // xor 2
    v += MOE_DPPF(v, 0x141);                       // half mirror
    v += MOE_DPPF(v, 0x140);                       // mirror
#undef MOE_DPPF
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

// Inclusive scan of an int over the wave through DPP: shifts by 1, 2, 4, 8
// within each 16-lane row, then row 0's last lane into row 1 and rows 0-1's
// last lane into rows 2-3 (rows that do not take a step add zero).
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Round-based exact top-k of one row of E logits by one wave64 (E <= 1024,
// k <= 32; the fallback of wave_topk for rows with many equal logits).
// Lane j < k returns (id_j, L_j) in selection order; other lanes return
// (-1, 0).  `get(e)` yields the fp32 logit of expert e (lane l holds experts
// l, l+64, ...).  Each lane first sorts its Q candidates by (logit desc,
// expert asc) with a sorting network (all pairs distinct, so any network
// gives the one order); then each round takes the largest head over the wave
// (then the lowest expert among equal heads: looked for only when a ballot
// finds the largest head on more than one lane) and the winning lane drops
// its head.
template <int Q>
__device__ __forceinline__ void lane_sort_desc(uint32_t* key, int* idx) {
    auto ce = [&](int a, int b) {                  // a < b: put the larger (key, -idx) first
        const bool sw = key[b] > key[a] || (key[b] == key[a] && idx[b] < idx[a]);
        const uint32_t ka = key[a], kb = key[b];
        const int ia = idx[a], ib = idx[b];
        key[a] = sw ? kb : ka;
        key[b] = sw ? ka : kb;
        idx[a] = sw ? ib : ia;
        idx[b] = sw ? ia : ib;
    };
    if constexpr (Q == 8) {                        // Batcher's odd-even merge sort, 19 pairs
        ce(0, 1); ce(2, 3); ce(4, 5); ce(6, 7);
        ce(0, 2); ce(1, 3); ce(4, 6); ce(5, 7);
        ce(1, 2); ce(5, 6);
        ce(0, 4); ce(1, 5); ce(2, 6); ce(3, 7);
        ce(2, 4); ce(3, 5);
        ce(1, 2); ce(3, 4); ce(5, 6);
    } else {                                       // odd-even transposition sort
#pragma unroll
        for (int rd = 0; rd < Q; ++rd)
#pragma unroll
            for (int a = rd & 1; a + 1 < Q; a += 2) ce(a, a + 1);
    }
}

template <int Q, typename Get>
__device__ __forceinline__ void wave_topk_q(Get get, int E, int k, int& out_id, float& out_val) {
    const int lane = __lane_id();
    uint32_t key[Q];
    int idx[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? order_key(get(e)) : 0u;     // 0 sorts last (below every real key)
        idx[i] = (e < E) ? i : 1024;
    }
    lane_sort_desc<Q>(key, idx);
    out_id = -1;
    out_val = 0.f;
    for (int j = 0; j < k; ++j) {
        const bool has = idx[0] < 1024;
        const uint32_t m = wave_max_u32(has ? key[0] : 0u);
        const bool at = has && key[0] == m;
        const uint64_t tied = __ballot(at);
        uint32_t win;
        if (__popcll(tied) == 1) {                       // one lane holds the largest head
            const int wl = __ffsll((unsigned long long)tied) - 1;
            win = (uint32_t)(wl + 64 * __builtin_amdgcn_readlane(idx[0], wl));
        } else {
            win = wave_min_u32(at ? (uint32_t)(lane + 64 * idx[0]) : 0xffffffffu);
        }
        if ((int)(win & 63u) == lane) {                  // drop the head
#pragma unroll
            for (int i = 0; i + 1 < Q; ++i) {
                key[i] = key[i + 1];
                idx[i] = idx[i + 1];
            }
            key[Q - 1] = 0u;
            idx[Q - 1] = 1024;
        }
        if (lane == j) {
            out_id = (int)win;
            out_val = order_key_value(m);
        }
    }
}

// Value of `v` held by lane ^ D, D = 1, 2, ..., 32.  Every move runs with all
// lanes active (a move placed under a lane condition would read inactive
// lanes as zero), then the lane picks its partner's copy.
#define MOE_DPPU(v, ctrl) ((uint32_t)__builtin_amdgcn_mov_dpp((int)(v), (ctrl), 0xF, 0xF, true))
template <int D>
__device__ __forceinline__ uint32_t xor_partner(uint32_t v) {
    const int lane = __lane_id();
    if constexpr (D == 1) {
        return MOE_DPPU(v, 0xB1);                  // quad_perm [1,0,3,2]
    } else if constexpr (D == 2) {
        return MOE_DPPU(v, 0x4E);                  // quad_perm [2,3,0,1]
    } else if constexpr (D == 4) {
        const uint32_t from_m4 = MOE_DPPU(v, 0x124), from_p4 = MOE_DPPU(v, 0x12C);   // row_ror 4 / 12
        return (lane & 4) ? from_m4 : from_p4;
    } else if constexpr (D == 8) {
        return MOE_DPPU(v, 0x128);                 // row_ror 8
    } else if constexpr (D == 16) {                // odd rows swap with even rows
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? p[0] : p[1];
    } else {                                       // upper half swaps with lower half
        static_assert(D == 32, "xor partner distance");
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? p[0] : p[1];
    }
}
#undef MOE_DPPU

// One compare-exchange step of a bitonic sorting network over the wave:
// merge blocks of S lanes, partner lane ^ D; blocks with lane & S == 0 come
// out in descending order (the whole wave for S = 64).
template <int S, int D>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t v) {
    const int lane = __lane_id();
    const uint32_t o = xor_partner<D>(v);
    const bool keep_max = ((lane & D) == 0) == ((lane & S) == 0);
    return keep_max ? max(v, o) : min(v, o);
}

// The 64 lane values in descending order (lane 0 holds the largest).
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t v) {
    v = bitonic_step<2, 1>(v);
    v = bitonic_step<4, 2>(v);
    v = bitonic_step<4, 1>(v);
    v = bitonic_step<8, 4>(v);
    v = bitonic_step<8, 2>(v);
    v = bitonic_step<8, 1>(v);
    v = bitonic_step<16, 8>(v);
    v = bitonic_step<16, 4>(v);
    v = bitonic_step<16, 2>(v);
    v = bitonic_step<16, 1>(v);
    v = bitonic_step<32, 16>(v);
    v = bitonic_step<32, 8>(v);
    v = bitonic_step<32, 4>(v);
    v = bitonic_step<32, 2>(v);
    v = bitonic_step<32, 1>(v);
    v = bitonic_step<64, 32>(v);
    v = bitonic_step<64, 16>(v);
    v = bitonic_step<64, 8>(v);
    v = bitonic_step<64, 4>(v);
    v = bitonic_step<64, 2>(v);
    v = bitonic_step<64, 1>(v);
    return v;
}

// LDS scratch of the wave top-k: 64 candidates and 32 results, 8 bytes each.
constexpr int kTopkScratch = 96;

// The same top-k as wave_topk_q, by a threshold and exact ranks.  tau = the
// k-th largest of the 64 lanes' largest keys: k distinct keys are >= tau, so
// every one of the k best is among the candidates (keys >= tau).  Those are
// written to LDS as (key, 0xFFFF - expert) pairs, whose u64 order is the
// routing order, and each candidate's rank is the number of candidates above
// it; the candidate of rank j goes to lane j.  More than 64 candidates (many
// equal logits): the round-based selection instead.  scr: kTopkScratch u64 of
// this wave's LDS.
template <int Q, typename Get>
__device__ __forceinline__ void wave_topk_rank(Get get, int E, int k, uint64_t* scr, int& out_id,
                                               float& out_val) {
    const int lane = __lane_id();
    uint32_t key[Q];
    bool real[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int e = lane + 64 * i;
        real[i] = e < E;
        key[i] = real[i] ? order_key(get(e)) : 0u;
    }
    uint32_t h = key[0];
#pragma unroll
    for (int i = 1; i < Q; ++i) h = max(h, key[i]);
    const uint32_t tau = __builtin_amdgcn_readlane(wave_sort_desc_u32(h), k - 1);
    int c = 0;
#pragma unroll
    for (int i = 0; i < Q; ++i) c += (real[i] && key[i] >= tau) ? 1 : 0;
    const int incl = wave_incl_scan_dpp(c);
    const int C = __builtin_amdgcn_readlane(incl, 63);
    if (C > 64) {
        wave_topk_q<Q>(get, E, k, out_id, out_val);
        return;
    }
    int pos = incl - c;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        if (real[i] && key[i] >= tau) {
            scr[pos] = ((uint64_t)key[i] << 32) | (uint32_t)(0xFFFFu - (uint32_t)(lane + 64 * i));
            ++pos;
        }
    }
    const uint64_t mine = lane < C ? scr[lane] : 0ull;
    int rank = 0;
    for (int j = 0; j < C; j += 8) {                // 8 broadcast reads in flight
        uint64_t c8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c8[u] = scr[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += (j + u < C && c8[u] > mine) ? 1 : 0;
    }
    uint64_t* res = scr + 64;
    if (lane < C && rank < k) res[rank] = mine;
    out_id = -1;
    out_val = 0.f;
    if (lane < k) {
        const uint64_t r = res[lane];
        out_id = (int)(0xFFFFu - (uint32_t)r);
        out_val = order_key_value((uint32_t)(r >> 32));
    }
}

// Exact top-k of one row of E logits by one wave64 (E <= 1024, k <= 32);
// lane j < k returns (id_j, L_j) in routing order.  scr: kTopkScratch u64 of
// LDS owned by this wave.
template <typename Get>
__device__ __forceinline__ void wave_topk(Get get, int E, int k, uint64_t* scr, int& out_id, float& out_val) {
    if (E <= 64) wave_topk_rank<1>(get, E, k, scr, out_id, out_val);
    else if (E <= 128) wave_topk_rank<2>(get, E, k, scr, out_id, out_val);
    else if (E <= 256) wave_topk_rank<4>(get, E, k, scr, out_id, out_val);
    else if (E <= 512) wave_topk_rank<8>(get, E, k, scr, out_id, out_val);
    else wave_topk_rank<16>(get, E, k, scr, out_id, out_val);
}

// Softmax over the k selected logits held by lanes 0..k-1 (lane 0 = max).
__device__ __forceinline__ float wave_softmax_selected(float v, int k) {
    const int lane = __lane_id();
    const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float ex = (lane < k) ? expf(v - m) : 0.f;
    return ex / wave_sum_f32_dpp(ex);
}

// ---------------------------------------------------------------- decoders
// Q3S-256 tail (bytes 96..103 of a block, loaded as one 8-byte word):
// d = bits 0..15, s_j = bits 16+4j .. 19+4j (signed).
__device__ __forceinline__ float q3_tail_d(uint64_t tail) {
    return f16_bits_to_f32((uint32_t)(tail & 0xffffu));
}
__device__ __forceinline__ int q3_tail_s(uint64_t tail, int j) {
    int nib = (int)((tail >> (16 + 4 * j)) & 0xfu);
    return (nib ^ 8) - 8;
}
// 3-bit index i (0..31) of a sub-block whose 12 index bytes are w0,w1,w2.
__device__ __forceinline__ int q3_index(uint32_t w0, uint32_t w1, uint32_t w2, int i) {
    uint64_t lo = ((uint64_t)w1 << 32) | w0;
    int bit = 3 * i;
    if (bit <= 61) return (int)((lo >> bit) & 7u);
    if (bit == 63) return (int)(((w1 >> 31) & 1u) | ((w2 & 3u) << 1));
    return (int)((w2 >> (bit - 64)) & 7u);
}
// Exact fp32 value d * s * c / 128 (d*s exact in 15 bits, *c in 22 bits, /128
// a power of two).
__device__ __forceinline__ float q3_value(float d, int s, int q) {
    return (d * (float)s) * (float)kC3[q] * 0.0078125f;
}
__device__ __forceinline__ float nl4_value(float d, int q) {
    return d * (float)kT4[q] * 0.0078125f;
}
// Exact fp32 value d * s * C2[q] / 128 (Q2S-256) and d * (q - 2) (Q2-32).
__device__ __forceinline__ float q2s_value(float d, int s, int q) {
    return (d * (float)s) * (float)kC2[q] * 0.0078125f;
}
__device__ __forceinline__ float q2_value(float d, int q) {
    return d * (float)(q - 2);
}
// Two's-complement 6-bit field at the low bits of f.
__device__ __forceinline__ int sext6(uint32_t f) { return (int)((f & 63u) ^ 32u) - 32; }

}  // namespace moe
