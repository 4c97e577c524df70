// Table decoders that the layer's kernels inline, in one place: the tables'
// contents, how they are filled, and how a lookup address is formed from the
// packed index bits.  The kernel-path dequantization export
// (moe_dequantize_path) decodes with these same functions, so its bit-exact
// test covers the decoders the bandwidth-path and grouped-GEMM kernels run.
//
// Codecs: model card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model"
// (routed up/gate at 3.25 bpw, a scale per 256-weight block and sub-scales
// per 32 weights; routed down in the 4-bit non-linear 32-weight type; the
// other layers' 3.44-bpw, 2-bit and 4.25-bpw up/gate and 2-bit down types).
#pragma once

#include "moe_common.hpp"

namespace moe {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The codebooks as int8 bytes (entry q in byte q), so that a table fill needs
// no memory load: C3 (8 entries), T4 (16 entries, low and high half).
constexpr uint64_t kC3Bytes = 0x7F4E301700E1BD81ull;
constexpr uint64_t kT4Lo = 0x00F5E9DCCEBEA881ull, kT4Hi = 0x7F5B47382B1F140Aull;

__device__ __forceinline__ float c3_entry(int q) {
    return (float)(int8_t)(uint8_t)(kC3Bytes >> (8 * q));
}
__device__ __forceinline__ float t4_entry(int q) {
    return (float)(int8_t)(uint8_t)((q < 8 ? kT4Lo : kT4Hi) >> (8 * (q & 7)));
}

// 8-byte LDS read (a must be a multiple of 8): one ds_read_b64.
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ u32x2 lds_ld2(uint32_t a) {
    return *(const lds_u32x2*)(uintptr_t)a;
}

// Two fp16 table values times an fp16 factor (v_pk_mul_f16): the sub-scale
// (s * c, an exact fp16 integer, |s * c| <= 1016) or the NL4 fold's d.
__device__ __forceinline__ uint32_t mul_pair(uint32_t pair, f16x2_t m2) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, pair) * m2);
}

// The lane's copy of a table in 32 copies (entry-major, 4-byte copies): the
// table's LDS address plus the lane's bank offset.
__device__ __forceinline__ uint32_t lut_copy_base(uint32_t lut_lds, int lane) {
    return lut_lds + (uint32_t)(lane & 31) * 4u;
}

// ---------------------------------------------------------------- Q3S-256 pair table
// Bandwidth-path up|gate.  Entry v = (fp16(C3[v & 7]), fp16(C3[v >> 3])) for
// an index pair v (two 3-bit codes, the first in the low bits), in 32 copies
// (copy = lane & 31) so that the random lookups of a half-wave fall in
// distinct LDS banks.  Byte address v*128 + c*4: a pair's six index bits
// reach it with one shift and one and-or.  8 KB, 8 KB-aligned.
constexpr int kQ3LutCopies = 32;
constexpr int kQ3LutDw = 64 * kQ3LutCopies;

// Fill by threads tid = 0 .. nt - 1 of a block (16-byte chunk i: a quarter
// of one entry's copies).
__device__ __forceinline__ void q3_pair_table_fill(uint32_t* lut, int tid, int nt) {
    for (int i = tid; i < kQ3LutDw / 4; i += nt) {
        const int v = i >> 3;
        const uint32_t val = pack2(f32_to_f16_bits(c3_entry(v & 7)), f32_to_f16_bits(c3_entry(v >> 3)));
        reinterpret_cast<u32x4*>(lut)[i] = u32x4{val, val, val, val};
    }
}
// Byte address (bits 7..12) of the index pair starting at bit P of the
// 96-bit index string w[0..2], or-ed onto `base`.
template <int P>
__device__ __forceinline__ uint32_t q3_pair_addr(const uint32_t* w, uint32_t base) {
    constexpr int wd = P >> 5, lo = P & 31;
    uint32_t v;
    if constexpr (lo + 6 > 32) v = __builtin_amdgcn_alignbit(w[wd + 1], w[wd], lo - 7);
    else if constexpr (lo >= 7) v = w[wd] >> (lo - 7);
    else if constexpr (wd > 0) v = __builtin_amdgcn_alignbit(w[wd], w[wd - 1], 25 + lo);
    else v = w[wd] << (7 - lo);
    return (v & 0x1f80u) | base;
}

// ---------------------------------------------------------------- Q3S-256 quad table
// Grouped-GEMM up|gate.  Entry v (12 bits: four 3-bit codes, the first in
// the low bits) holds the four codebook values (C3[v & 7], C3[v >> 3 & 7],
// C3[v >> 6 & 7], C3[v >> 9]) as fp16, 8 bytes, in one copy (4096 entries,
// 32 KB, 32 KB-aligned).  One 8-byte read decodes four weights, so the index
// bits are moved into place once per four weights, not once per two as with
// the pair table.
constexpr int kQ3QuadDw = 4096 * 2;

// Fill by threads tid = 0 .. nt - 1 (16-byte chunk i: entries 2i, 2i + 1).
__device__ __forceinline__ void q3_quad_table_fill(uint32_t* lut, int tid, int nt) {
    for (int i = tid; i < kQ3QuadDw / 4; i += nt) {
        u32x4 qv;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int en = 2 * i + h;
            qv[2 * h] = pack2(f32_to_f16_bits(c3_entry(en & 7)), f32_to_f16_bits(c3_entry((en >> 3) & 7)));
            qv[2 * h + 1] = pack2(f32_to_f16_bits(c3_entry((en >> 6) & 7)), f32_to_f16_bits(c3_entry(en >> 9)));
        }
        reinterpret_cast<u32x4*>(lut)[i] = qv;
    }
}
// Byte address of the entry for the four codes at bits P .. P + 11 of the
// 96-bit index string q[0..2]: the field lands at address bits 3..14, or-ed
// onto `base` (the table's LDS address).
template <int P> __device__ __forceinline__ uint32_t q3_quad_addr(const uint32_t (&q)[3], uint32_t base) {
    constexpr int wd = P >> 5, lo = P & 31;
    uint32_t v;
    if constexpr (lo + 12 > 32) v = __builtin_amdgcn_alignbit(q[wd + 1], q[wd], lo - 3);
    else if constexpr (lo >= 3) v = q[wd] >> (lo - 3);
    else v = q[wd] << (3 - lo);
    return (v & 0x7ff8u) | base;
}
// Weights 8 KK .. 8 KK + 7 of a 32-weight sub-block (index string q) as four
// fp16 pairs s * c (exact integers).
template <int KK>
__device__ __forceinline__ void q3_quad_decode8(const uint32_t (&q)[3], uint32_t base, f16x2_t s2,
                                                uint32_t (&f)[4]) {
    const u32x2 c0 = lds_ld2(q3_quad_addr<24 * KK>(q, base));
    const u32x2 c1 = lds_ld2(q3_quad_addr<24 * KK + 12>(q, base));
    f[0] = mul_pair(c0[0], s2);
    f[1] = mul_pair(c0[1], s2);
    f[2] = mul_pair(c1[0], s2);
    f[3] = mul_pair(c1[1], s2);
}

// ---------------------------------------------------------------- Q3K-256 (3.44 bpw)
// Grouped GEMM.  The Q3S pair table above, read with q3_pair_addr; s * c
// (|s| <= 32) reaches 4064, past fp16's exact integers (2048), so a pair
// enters as two exact fp16 parts, c (s mod 16) and c 16 floor(s / 16), summed
// by two MFMAs; d / 128 goes on the block's fp32 partial sums.
__device__ __forceinline__ void q3k_split(int s, f16x2_t& lo2, f16x2_t& hi2) {
    const _Float16 lo = (_Float16)(float)(s & 15), hi = (_Float16)(float)(16 * (s >> 4));
    lo2 = f16x2_t{lo, lo};
    hi2 = f16x2_t{hi, hi};
}

// ---------------------------------------------------------------- 2-bit nibble tables
// Grouped GEMM, the 2-bit codecs.  Entry v (4 bits: two 2-bit codes, the
// first in the low bits) = two fp16 values, in 32 copies (byte address
// v*128 + c*4), filled over 8 KB (entries 16..63 repeat the first 16 and are
// never read).  Q2S-256: (C2[lo], C2[hi]), times the sub-scale s, then d /
// 128 on the block's partial sums.  Q2-32: (lo - 2, hi - 2), times d (exact
// in fp16).
constexpr uint32_t kC2Bytes = 0x7F360081u;       // C2 = (-127, 0, 54, 127), entry q in byte q
constexpr int kNibLutDw = 2048;

__device__ __forceinline__ float c2_entry(int q) {
    return (float)(int8_t)(uint8_t)(kC2Bytes >> (8 * q));
}
template <bool Q2S>
__device__ __forceinline__ void nib_table_fill(uint32_t* lut, int tid, int nt) {
    for (int i = tid; i < kNibLutDw / 4; i += nt) {
        const int en = (i >> 3) & 15;
        const int lo = en & 3, hi = en >> 2;
        const uint32_t v = Q2S ? pack2(f32_to_f16_bits(c2_entry(lo)), f32_to_f16_bits(c2_entry(hi)))
                               : pack2(f32_to_f16_bits((float)(lo - 2)), f32_to_f16_bits((float)(hi - 2)));
        reinterpret_cast<u32x4*>(lut)[i] = u32x4{v, v, v, v};
    }
}
// LDS address of the entry for the 4-bit field at bit P of a 64-bit index
// word (two 2-bit codes): the field lands at address bits 7..10, or-ed onto
// cb.
template <int P> __device__ __forceinline__ uint32_t nib_lut_addr(const uint32_t (&q)[2], uint32_t cb) {
    constexpr int w = P >> 5, b = P & 31;
    uint32_t x;
    if constexpr (b >= 7) x = q[w] >> (b - 7);
    else x = q[w] << (7 - b);
    return (x & 0x780u) | cb;
}

// ---------------------------------------------------------------- NL4-32 byte tables
// Entry v = the two weights of one index byte (even weight in the low
// nibble) as fp16, in 32 copies (copy = lane & 31): byte address v*128 + c*4.
// 32 KB, 32 KB-aligned.  Bandwidth-path down and grouped-GEMM NL4-32 up|gate:
// (T4[v & 15], T4[v >> 4]), d / 128 applied in fp32 to the partial sums (the
// NL4S-256 up|gate the same table in 16 copies, d s / 128 per sub-block).  Grouped-GEMM down (the fold):
// (T4[lo] / 8, T4[hi] / 8) (exact), multiplied by d in fp16, so that a
// fragment holds fp16_rne(16 d T4 / 128) (one rounding; the factor 16 keeps
// the small entries of small-d blocks out of fp16's subnormals) and the
// epilogue divides by 16.
constexpr int kNl4LutDw = 256 * 32;

// (COPIES = 16: the NL4S-256 up|gate table, 16 KB, byte address v*64 + c*4.)
template <int COPIES = 32>   // 32 or 16
__device__ __forceinline__ void nl4_pair_table_fill(uint32_t* lut, int tid, int nt) {
    for (int i = tid; i < 256 * COPIES / 4; i += nt) {        // 16-byte chunk i: COPIES / 4 per entry
        const int v = i >> (COPIES == 32 ? 3 : 2);
        const uint32_t val = pack2(f32_to_f16_bits(t4_entry(v & 15)), f32_to_f16_bits(t4_entry(v >> 4)));
        reinterpret_cast<u32x4*>(lut)[i] = u32x4{val, val, val, val};
    }
}
__device__ __forceinline__ void nl4_fold_table_fill(uint32_t* lut, int tid, int nt) {
    for (int i = tid; i < kNl4LutDw / 4; i += nt) {
        const int v = i >> 3;
        const uint32_t val = pack2(f32_to_f16_bits(t4_entry(v & 15) * 0.125f),
                                   f32_to_f16_bits(t4_entry(v >> 4) * 0.125f));
        reinterpret_cast<u32x4*>(lut)[i] = u32x4{val, val, val, val};
    }
}
// Byte address of the entry for index byte B of the word nb, with entries
// 1 << SH bytes apart (SH = 7: 32 copies; 6: 16 copies), or-ed onto `base`.
template <int B, int SH = 7>
__device__ __forceinline__ uint32_t nl4_byte_addr(uint32_t nb, uint32_t base) {
    constexpr uint32_t mask = 0xFFu << SH;
    const uint32_t v = B == 0 ? (nb << SH) : (nb >> (8 * B - SH));
    return (v & mask) | base;
}

}  // namespace moe
