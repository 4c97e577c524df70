// Grouped-GEMM path of the layer (prefill-sized batches).  One kernel
// template, seven uses (the routed experts; the router and the shared expert
// are dense bf16 products, in moe_kernels_dense.hip):
//   UG_Q3   routed up|gate: A = token rows gathered through the permutation
//           (fp16), B = Q3S-256 weights, epilogue SwiGLU
//   UG_Q2S  the same with Q2S-256 weights, UG_NL4 with NL4-32 weights, UG_Q3K
//           with Q3K-256 and UG_NL4S with NL4S-256 weights (the mixed-format
//           layers and the draft head)
//   DN_NL4  routed down: A = the expert's rows of a (fp16), B = NL4-32
//           weights, epilogue fp32 (or range-checked fp16) store (permuted rows)
//   DN_Q2   the same with Q2-32 weights
//
// Tile 64 token rows x 256 weight rows, K steps of 64; four waves, wave w
// owns 64 weight rows (SwiGLU modes: 32 up rows and the 32 gate rows of the
// same outputs) against all 64 token rows, 32x32x16 MFMA; two blocks per CU.
//
// Loads go through registers (the compiler tracks them exactly):
//   A: the tile's 64 rows x 64 k, loaded two K steps ahead and written into
//      one of two LDS stages one step ahead (XOR-swizzled 16-byte chunks);
//      one barrier per K step.
//   B, quantized: the packed bytes of the wave's 64 weight rows for one
//      period (a 256-weight block = 4 K steps, or four 32-weight blocks = 2
//      K steps) are
//      loaded coalesced, a period ahead, into a per-wave LDS area; each lane
//      reads back the bytes of its own MFMA fragment (one 32-weight
//      sub-block or block of one row per 32-column half) and decodes them
//      with an LDS table chunk by chunk between the MFMAs.
// The MFMA's reduction order within a K step is permuted (lane half h takes
// k = 32h .. 32h + 31) so that a lane's fragment is one contiguous sub-block;
// A is read from LDS in the same order.
//
// Numerics: Q3S and Q2S weights enter the matrix cores as s*c (an fp16
// integer, |s*c| <= 1016, exact) and d/128 is applied in fp32 to the partial
// sum of each 256-weight block, so those weights are exact.  NL4 down weights
// enter as fp16_rne(16 d * T4[q] / 128) (one rounding, relative error <= 2^-11
// for every normal d up to 4126; the factor 16 keeps the smallest entries of
// small-d blocks out of fp16's subnormals and is divided out in the epilogue);
// Q2 weights as d * (q - 2), exact in fp16.  NL4 up|gate weights stay exact
// too (a rounding there would move the bf16 rounding of the SwiGLU output):
// that mode keeps the natural K order, so the two MFMAs of a chunk pair cover
// one 32-weight block, B = T4[q] (exact), and d/128 goes on the block's fp32
// partial sums.
//
// Layer: "Avalon" README, opening paragraphs; model card "Qwen3.8-Flash-Next
// - Avalon GGUF", "Files / Main model" (codecs, up | gate | down packing).
#include "moe_decoders.hpp"
#include "moe_kernels.hpp"

namespace moe {

typedef _Float16 h2g __attribute__((ext_vector_type(2)));

template <int N> struct Cnt { static constexpr int value = N; };

// (the numbers are the kernels' names in traces: k_gemm<0>, <1>, <5> .. <9>)
enum GemmMode { UG_Q3 = 0, DN_NL4 = 1, UG_Q2S = 5, UG_NL4 = 6, DN_Q2 = 7, UG_Q3K = 8, UG_NL4S = 9 };
// quantized B formats of the routed modes
enum BFmt { BF_NONE, BF_Q3, BF_Q2S, BF_NL4, BF_Q2, BF_Q3K, BF_NL4S };
template <int MODE> constexpr int bfmt() {
    return MODE == UG_Q3 ? BF_Q3 : MODE == UG_Q2S ? BF_Q2S : (MODE == DN_NL4 || MODE == UG_NL4) ? BF_NL4
           : MODE == DN_Q2 ? BF_Q2 : MODE == UG_Q3K ? BF_Q3K : MODE == UG_NL4S ? BF_NL4S : BF_NONE;
}

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int kStages = 2;               // A stages in LDS
// Token rows per tile: 64 (two blocks per CU, ragged expert tails).
constexpr int kLutDw = 2048;             // decode table dwords (8 KB)

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
    int N;                   // output columns (GEMM N)
    int K;                   // reduction length
    int half_n;              // up|gate: rows of the up half (I or I_s)
    int H, I;                // layer shape (routed record layout)
    int64_t dn_off;          // routed down: byte offset of the down matrix in a record
    uint16_t* out16;         // a16_perm / a_sh
    float* out32;            // y_perm
    // routed down, fp16 form: y_perm as fp16 to y16 (range-checked: a wave
    // whose stored values exceed 65504, or are all below 2^-10 without being
    // all zero, adds 1 to *range_flag), else fp32 to out32
    uint16_t* y16;
    int* range_flag;
    const int* only_if;      // non-null: the launch does nothing unless *only_if != 0
    int ldo;                 // output row length
    int npb;                 // routed: N tiles per block (consecutive, same M tile)
};

// A tile in LDS: row r, 16-byte chunk c at slot r*8 + (c ^ ((r/2) % 8)), so
// that 16 consecutive rows read at one chunk hit 16 distinct bank groups.
__device__ __forceinline__ int aslot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int MODE>
__global__ void __launch_bounds__(256, 2) k_gemm(GemmArgs g) {
    constexpr int kBF = bfmt<MODE>();
    constexpr bool kQ3 = kBF == BF_Q3;
    constexpr bool kNL = kBF == BF_NL4;
    constexpr bool kB256 = kBF == BF_Q3 || kBF == BF_Q2S;     // 256-weight blocks: d on the partial sums
    // 6-bit sub-scaled 256-weight blocks (Q3K-256: sub-blocks of 16, NL4S-256:
    // of 32), natural K order.  Q3K-256: B = s * c as two exact fp16 parts,
    // d / 128 on the block's partial sums; NL4S-256: B = the table integers,
    // d * s / 128 applied in fp32 to each 32-weight sub-block's partial sums
    constexpr bool kQ3K = kBF == BF_Q3K, kNLS = kBF == BF_NL4S, kSub = kQ3K || kNLS;
    constexpr bool kNat = MODE == UG_NL4 || kSub;              // natural K order
    constexpr bool kNLTab = kNL || kNLS;                       // the NL4 table (8 copies)
    constexpr bool kSwi = MODE == UG_Q3 || MODE == UG_Q2S || MODE == UG_NL4 || kSub;
    // the down modes compute the transposed tile (weights as the MFMA's first
    // operand): a lane then holds 4 consecutive output columns per register
    // group, stored with one vector store
    constexpr bool kTr = !kSwi;
    static_assert(kBF != BF_NONE, "a routed mode");
    if (g.only_if && *g.only_if == 0) return;
    constexpr int TBM = BM;
    constexpr int kAL = TBM * 8 / 256;              // A 16-byte loads per lane per K step
    constexpr int kSMX = TBM / 32;                  // 32-row groups per tile

    __shared__ u32x4 As[kStages][TBM * 8];
    // Decode tables.  Q3S-256: the quad table, 12-bit index -> four fp16
    // codebook values, one copy (a lookup decodes four weights; random
    // 8-byte reads meet some bank conflicts, which cost less than the second
    // address the pair table took).  The others replicated so that random
    // indices spread over the banks:
    // Q3K-256 pair (6-bit) -> (C3[lo], C3[hi]), 32 copies (entry * 32 + lane % 32);
    // NL4 byte -> (T4[lo], T4[hi]) (/ 8 for the down fold), 32 or 16 copies
    // (entry * copies + lane % copies);
    // Q2S nibble -> (C2[lo], C2[hi]) and Q2 nibble -> (lo - 2, hi - 2), 32
    // copies (entry * 32 + lane % 32).
    // NL4 tables: 32 copies (16 with the larger NL4S-256 period area, so
    // that two blocks still fit a CU's LDS)
    constexpr int kNLCopies = kNLS ? 16 : 32;
    constexpr int kNLSh = kNLS ? 6 : 7;                        // log2(copies * 4)
    // Q3S-256: the quad table (12-bit index -> four fp16 codebook values, one
    // copy, 32 KB)
    constexpr int kTabDw = kQ3 ? kQ3QuadDw : kNLTab ? 256 * kNLCopies : kLutDw;
    __shared__ __attribute__((aligned(kTabDw * 4))) uint32_t lut[kTabDw];
    constexpr int kPer = (kB256 || kSub) ? 4 : 2;   // quantized B: K steps per period
    // bytes of a weight row per period in LDS (Q3K-256: the 110-byte block
    // inside the 112-byte dword-aligned window that holds it)
    constexpr int kRowB = kBF == BF_Q3 ? 104 : kBF == BF_Q2S ? 80 : kBF == BF_NL4 ? 72 : kBF == BF_Q3K ? 112
                          : kBF == BF_NL4S ? 136 : 40;
    constexpr int kUB = kQ3K ? 4 : 8;               // bytes per load unit (Q3K-256 windows are 4-aligned)
    constexpr int kUPR = kRowB / kUB;               // load units per row = per lane
    __shared__ __attribute__((aligned(16))) uint8_t Bq[4][64 * kRowB];

    const int tid = threadIdx.x, lane = __lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- tile coordinates (XCD-aware).  Blocks are dealt to the 8 XCDs in
    // turn (XCD = block id mod 8); XCD x takes the contiguous M tiles
    // [x mpx, (x + 1) mpx), mpx = ceil(ntiles / 8), in order, so the M tiles of
    // one expert (and the N tiles of one M tile) run together under one L2 and
    // share its copy of the expert's weights.  A block takes npb consecutive N
    // tiles [nt0, nt1) of its M tile, one after the other, with the loads
    // running on across them.  The grid holds 8 ceil(max_tiles / 8) NGr
    // blocks, so every (M tile, N group) pair is covered once.
    const int NT = kSwi ? (g.half_n + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
    const int npb = g.npb;
    const int NGr = (NT + npb - 1) / npb;
    const int bid = blockIdx.x, xcd = bid & 7, li = bid >> 3;
    const int ntl = *g.ntiles, mpx = (ntl + 7) >> 3;
    const int mt = xcd * mpx + li / NGr, nt0 = (li % NGr) * npb, nt1 = min(nt0 + npb, NT);
    int row0, rows, e = 0;
    {
        if (li / NGr >= mpx || mt >= ntl) return;
        e = g.tiles[3 * mt];
        row0 = g.tiles[3 * mt + 1];
        rows = g.tiles[3 * mt + 2];
    }

    // ---- A: lane's load i (0..kAL-1) is row (kAL w + i) * 8 + lane / 8,
    // physical chunk lane % 8 of the stage.  Rows past the tile's end read its
    // last row again (their outputs are never stored).
    const uint16_t* asrc[kAL];
#pragma unroll
    for (int i = 0; i < kAL; ++i) {
        const int r = (kAL * w + i) * 8 + (lane >> 3);
        const int rc = min(r, rows - 1);
        int64_t src;
        if (kSwi) src = (int64_t)(g.perm[row0 + rc] / g.k);
        else src = row0 + rc;
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        asrc[i] = g.A + src * g.lda + c * 8;
    }

    // ---- B: weight row of this lane for column half sn (0, 1) of N tile nt
    auto brow_of = [&](int nt, int sn) {
        if (kSwi) {
            const int oc = min(nt * (BN / 2) + 32 * w + l32, g.half_n - 1);
            return sn ? g.half_n + oc : oc;
        }
        return min(nt * BN + 64 * w + 32 * sn + l32, g.N - 1);
    };
    auto ocol_of = [&](int nt, int sn) {                  // the column holds an output
        if (kSwi) return nt * (BN / 2) + 32 * w + l32 < g.half_n;
        return nt * BN + 64 * w + 32 * sn + l32 < g.N;
    };
    // ---- A loads into registers (the compiler tracks them exactly)
    struct RawA {
        u32x4 v[kAL];
    };
    auto load_a = [&](int kt, RawA& R) {
#pragma unroll
        for (int i = 0; i < kAL; ++i) R.v[i] = *reinterpret_cast<const u32x4*>(asrc[i] + kt * BK);
    };
    // A(kt) from registers into stage st: load i of wave w fills slots
    // (kAL w + i) * 64 + lane.
    auto put_a = [&](int st, const RawA& R) {
#pragma unroll
        for (int i = 0; i < kAL; ++i) As[st][(kAL * w + i) * 64 + lane] = R.v[i];
    };

    // ---- quantized B: the packed bytes of one period (Q3: one 256-weight
    // block = 4 K steps, 104 B per row; NL4: four 32-weight blocks = 2 K
    // steps, 72 B per row) of the wave's 64 weight rows (row r = 32 sn + l,
    // l = lane % 32 of the fragments) are loaded with 8-byte loads in
    // row-major unit order (unit u = lane + 64 i = r * UPR + part), one period
    // ahead, into registers, then written to the wave's LDS area in the same
    // order; each lane reads its fragment's bytes back per K step.  Reads past
    // a row's last block (NL4, odd step count) stay inside the expert record
    // or return zeros (buffer loads) and are never used.
    __amdgpu_buffer_rsrc_t wsrc;
    int rb_w = 0, mbase = 0;                         // row bytes, matrix offset in the record
    {
        const uint8_t* W = g.experts + (int64_t)e * g.estride;
        wsrc = __builtin_amdgcn_make_buffer_rsrc((void*)W, 0, (int)g.estride, 0x00020000);
        constexpr int nwb = (kB256 || kSub) ? 256 : 32;
        constexpr int nbb = kQ3K ? kQ3KBytes : kRowB / ((kB256 || kSub) ? 1 : 4);
        rb_w = (g.K / nwb) * nbb;
        mbase = kSwi ? 0 : (int)g.dn_off;
    }
    // byte offset in the record of unit i of this lane, N tile nt, period 0
    auto unit_off = [&](int nt, int i) {
        const int u = lane + 64 * i, r = u / kUPR, part = u - r * kUPR;
        int wr;
        if (kSwi) {
            const int oc = min(nt * (BN / 2) + 32 * w + (r & 31), g.half_n - 1);
            wr = (r >> 5) ? g.half_n + oc : oc;
        } else {
            wr = min(nt * BN + 64 * w + r, g.N - 1);
        }
        if constexpr (kQ3K) return mbase + wr * rb_w;   // the row's start (unit part = u % kUPR)
        return mbase + wr * rb_w + 8 * part;
    };
    struct RawP {
        uint32_t u[kUPR * (kUB / 4)];
    };
    auto load_period = [&](int nt, int p, RawP& R) {
        // Q3K-256: the units' offsets are formed here each time (28 of them
        // kept live across the loop would not fit the registers)
        int ln = lane;
        if constexpr (kQ3K) __asm__ volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < kUPR; ++i) {
            if constexpr (kQ3K) {
                // the dword-aligned 112-byte window holding block p of the row
                const int u = ln + 64 * i, r = u / kUPR, part = u - r * kUPR;
                const int oc = min(nt * (BN / 2) + 32 * w + (r & 31), g.half_n - 1);
                const int rs = ((r >> 5) ? g.half_n + oc : oc) * rb_w;
                const int wo = ((rs + kQ3KBytes * p) & ~3) + 4 * part;
                R.u[i] = __builtin_amdgcn_raw_buffer_load_b32(wsrc, wo, 0, 0);
            } else {
                const u32x2 v = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(wsrc, unit_off(nt, i) + p * kRowB, 0, 0));
                R.u[2 * i] = v[0];
                R.u[2 * i + 1] = v[1];
            }
        }
    };
    auto put_period = [&](const RawP& R) {
#pragma unroll
        for (int i = 0; i < kUPR; ++i) {
            if constexpr (kQ3K) {
                *reinterpret_cast<uint32_t*>(&Bq[w][4 * (lane + 64 * i)]) = R.u[i];   // Q3K: kSwi only
            } else {
                *reinterpret_cast<u32x2*>(&Bq[w][8 * (lane + 64 * i)]) = u32x2{R.u[2 * i], R.u[2 * i + 1]};
            }
        }
    };
    // The lane's raw bytes of step kt from the period area: Q3 q[sn][0..2] =
    // the 12 index bytes of sub-block 2 (kt % 4) + h, q[sn][3..4] = the tail;
    // Q2S q[sn][0..1] = the 8 index bytes of sub-block 2 (kt % 4) + h,
    // q[sn][3..4] = d and the sub-scales; NL4 q[sn][0..4] = the 20
    // dword-aligned bytes holding block b = 2 (kt % 2) + h; Q2 q[sn][0..2] =
    // the 12 dword-aligned bytes holding block b (d at byte 2h).
    constexpr int kRawDw = 5;
    // natural order: only block j = 2 (kt % 2) + jb of the step (20
    // dword-aligned bytes, d at byte 2 jb), read before its two chunks
    auto read_blk = [&](int kt, int jb, uint32_t (&q)[2][kRawDw]) {
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
            const uint8_t* rb = &Bq[w][(32 * sn + l32) * kRowB];
            const uint32_t* ip = reinterpret_cast<const uint32_t*>(rb + kNL4Bytes * (2 * (kt & 1) + jb) - 2 * jb);
#pragma unroll
            for (int u = 0; u < 5; ++u) q[sn][u] = ip[u];
        }
    };
    auto read_raw = [&](int kt, uint32_t (&q)[2][kRawDw]) {
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
            const uint8_t* rb = &Bq[w][(32 * sn + l32) * kRowB];
            if constexpr (kQ3) {
                const uint32_t* ip = reinterpret_cast<const uint32_t*>(rb + 12 * (2 * (kt & 3) + hh));
                q[sn][0] = ip[0];
                q[sn][1] = ip[1];
                q[sn][2] = ip[2];
                const u32x2 t = *reinterpret_cast<const u32x2*>(rb + 96);
                q[sn][3] = t[0];
                q[sn][4] = t[1];
            } else if constexpr (kBF == BF_Q2S) {
                const u32x2 ix = *reinterpret_cast<const u32x2*>(rb + 8 * (2 * (kt & 3) + hh));
                q[sn][0] = ix[0];
                q[sn][1] = ix[1];
                const u32x2 t = *reinterpret_cast<const u32x2*>(rb + 64);
                q[sn][3] = t[0];
                q[sn][4] = t[1];
            } else if constexpr (kNL) {
                const uint32_t* ip = reinterpret_cast<const uint32_t*>(rb + kNL4Bytes * (2 * (kt & 1) + hh) - 2 * hh);
#pragma unroll
                for (int u = 0; u < 5; ++u) q[sn][u] = ip[u];
            } else {
                const uint32_t* ip = reinterpret_cast<const uint32_t*>(rb + kQ2Bytes * (2 * (kt & 1) + hh) - 2 * hh);
#pragma unroll
                for (int u = 0; u < 3; ++u) q[sn][u] = ip[u];
            }
        }
    };


    // LDS byte address of a table entry = cb | entry << 7 (32 copies) or
    // << kNLSh (NL4).
    const uint32_t cb = kQ3 ? lds_addr(lut)
                      : lds_addr(lut) | (kNLTab ? (uint32_t)(lane & (kNLCopies - 1)) * 4u : (uint32_t)l32 * 4u);
    // NL4: table address of index byte B of the word nb
    auto nl_addr = [&](uint32_t nb, auto bc) { return nl4_byte_addr<decltype(bc)::value, kNLSh>(nb, cb); };

    // Fragments of one K step: f[sn][kk] = weights k = 32h + 8kk .. +7 of
    // column half sn; 256-weight blocks: dl[sn] = d / 128 of the lane's
    // column in this block.
    struct Frag {
        u32x4 f[2][4];
        float dl[2];
        float db[2][2];      // natural order: d / 128 of [half][block of the step]
    };
    // Chunk kk of both halves from the step's raw bytes.
    auto decode_kk = [&](int kt, const uint32_t (&R)[2][kRawDw], Frag& F, auto kkc) {
        constexpr int kk = decltype(kkc)::value;
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
            if constexpr (kNat) {
                // chunk kk = weights 16 (kk % 2) + 8h .. +7 of block j = kk / 2:
                // index bytes 2 + 2j + 8 (kk % 2) + 4h of its 20 raw bytes
                constexpr int j = kk >> 1, c = kk & 1;
                const uint32_t* Rb = &R[sn][0];                // block j's bytes (read_blk)
                if (c == 0) {
                    const uint32_t dbits = j ? (Rb[0] >> 16) : (Rb[0] & 0xffffu);
                    F.db[sn][j] = f16_bits_to_f32(dbits) * 0.0078125f;
                }
                uint32_t nb;
                if constexpr (j == 0) {
                    const uint32_t lo = hh ? Rb[2 * c + 1] : Rb[2 * c], hi = hh ? Rb[2 * c + 2] : Rb[2 * c + 1];
                    nb = __builtin_amdgcn_perm(hi, lo, 0x05040302u);
                } else {
                    nb = hh ? Rb[2 * c + 2] : Rb[2 * c + 1];
                }
                const uint32_t aa[4] = {nl_addr(nb, Cnt<0>{}), nl_addr(nb, Cnt<1>{}), nl_addr(nb, Cnt<2>{}),
                                        nl_addr(nb, Cnt<3>{})};
#pragma unroll
                for (int p = 0; p < 4; ++p) F.f[sn][kk][p] = lds_ld(aa[p]);   // (T4[lo], T4[hi]), exact
            } else if constexpr (kQ3) {
                const uint64_t tail = ((uint64_t)R[sn][4] << 32) | R[sn][3];
                const _Float16 s = (_Float16)(float)q3_tail_s(tail, 2 * (kt & 3) + hh);
                const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(R[sn][3] & 0xffffu));
                const h2g s2 = {s, s};
                if (kk == 0) F.dl[sn] = (float)d * 0.0078125f;
                const uint32_t q[3] = {R[sn][0], R[sn][1], R[sn][2]};
                uint32_t fq[4];
                q3_quad_decode8<kk>(q, cb, s2, fq);        // c * s, exact fp16 integers
#pragma unroll
                for (int p = 0; p < 4; ++p) F.f[sn][kk][p] = fq[p];
            } else if constexpr (kNL) {
                // h = 0: d in bytes 0-1, indices in bytes 2..17;
                // h = 1: d in bytes 2-3, indices in bytes 4..19.
                const uint32_t dbits = __builtin_amdgcn_perm(0u, R[sn][0], hh ? 0x0c0c0302u : 0x0c0c0100u);
                const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)dbits);
                const h2g d2 = {d, d};
                const uint32_t nb = __builtin_amdgcn_perm(R[sn][kk + 1], R[sn][kk], hh ? 0x07060504u : 0x05040302u);
                const uint32_t aa[4] = {nl_addr(nb, Cnt<0>{}), nl_addr(nb, Cnt<1>{}), nl_addr(nb, Cnt<2>{}),
                                        nl_addr(nb, Cnt<3>{})};
#pragma unroll
                for (int p = 0; p < 4; ++p) F.f[sn][kk][p] = mul_pair(lds_ld(aa[p]), d2);
            } else {
                // two 2-bit indices per table entry: chunk kk is bits 16 kk ..
                // 16 kk + 15 of the 64-bit index word
                uint32_t ix[2];
                _Float16 m;                                // multiplier of the table pairs
                if constexpr (kBF == BF_Q2S) {
                    const uint64_t tail = ((uint64_t)R[sn][4] << 32) | R[sn][3];
                    m = (_Float16)(float)q3_tail_s(tail, 2 * (kt & 3) + hh);
                    if (kk == 0) F.dl[sn] = f16_bits_to_f32(R[sn][3] & 0xffffu) * 0.0078125f;
                    ix[0] = R[sn][0];
                    ix[1] = R[sn][1];
                } else {
                    // h = 0: d in bytes 0-1, indices in bytes 2..9;
                    // h = 1: d in bytes 2-3, indices in bytes 4..11.
                    const uint32_t dbits = __builtin_amdgcn_perm(0u, R[sn][0], hh ? 0x0c0c0302u : 0x0c0c0100u);
                    m = __builtin_bit_cast(_Float16, (uint16_t)dbits);
                    ix[0] = __builtin_amdgcn_perm(R[sn][1], R[sn][0], hh ? 0x07060504u : 0x05040302u);
                    ix[1] = __builtin_amdgcn_perm(R[sn][2], R[sn][1], hh ? 0x07060504u : 0x05040302u);
                }
                const h2g m2 = {m, m};
                const uint32_t aa[4] = {nib_lut_addr<16 * kk + 0>(ix, cb), nib_lut_addr<16 * kk + 4>(ix, cb),
                                        nib_lut_addr<16 * kk + 8>(ix, cb), nib_lut_addr<16 * kk + 12>(ix, cb)};
#pragma unroll
                for (int p = 0; p < 4; ++p) F.f[sn][kk][p] = mul_pair(lds_ld(aa[p]), m2);   // exact: small integers times m
            }
        }
    };

    // acc: the output sums; Q3: tmp holds the current 256-weight block's sums
    // of x * s * c, added to acc times d / 128 at the block's end.
    f32x16 acc[kSMX][2], tmp[(kB256 || kQ3K) ? kSMX : 1][2];
#pragma unroll
    for (int a = 0; a < kSMX; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    if constexpr (kB256 || kQ3K) {
#pragma unroll
        for (int a = 0; a < kSMX; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) tmp[a][b][r] = 0.f;
    }

    // MFMAs of chunk kk of a K step (A from stage st) over the first SM
    // 32-row groups of the tile.
    auto mma_kk = [&](int st, int kk, const u32x4 (&fb)[2][4], auto smc) {
        constexpr int SM = decltype(smc)::value;
        u32x4 fa[SM];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) fa[sm] = As[st][aslot(32 * sm + l32, kNat ? 2 * kk + hh : 4 * hh + kk)];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm)
#pragma unroll
            for (int sn = 0; sn < 2; ++sn) {
                if constexpr (kB256) tmp[sm][sn] = mfma32_f16(fa[sm], fb[sn][kk], tmp[sm][sn]);
                else if constexpr (kTr) acc[sm][sn] = mfma32_f16(fb[sn][kk], fa[sm], acc[sm][sn]);
                else acc[sm][sn] = mfma32_f16(fa[sm], fb[sn][kk], acc[sm][sn]);
            }
    };
    // 256-weight blocks, at a block's end: acc += tmp * d / 128, tmp = 0.
    auto apply_d = [&](const Frag& F, auto smc) {
        constexpr int SM = decltype(smc)::value;
        if constexpr (kB256) {
#pragma unroll
            for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                for (int sn = 0; sn < 2; ++sn)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc[sm][sn][r] += tmp[sm][sn][r] * F.dl[sn];
                        tmp[sm][sn][r] = 0.f;
                    }
        }
    };

    // Natural order, block j of a step (chunks 2j and 2j + 1, decoded into
    // F): per 32-row group and half, the two MFMAs chain into a fresh
    // partial, then acc += partial * d / 128 of the block.
    auto nat_block = [&](int st, const Frag& F, auto jc, auto smc) {
        constexpr int j = decltype(jc)::value, SM = decltype(smc)::value;
        u32x4 fa[SM][2];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm)
#pragma unroll
            for (int c = 0; c < 2; ++c) fa[sm][c] = As[st][aslot(32 * sm + l32, 2 * (2 * j + c) + hh)];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm)
#pragma unroll
            for (int sn = 0; sn < 2; ++sn) {
                f32x16 t = {};
                t = mfma32_f16(fa[sm][0], F.f[sn][2 * j], t);
                t = mfma32_f16(fa[sm][1], F.f[sn][2 * j + 1], t);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[sm][sn][r] += t[r] * F.db[sn][j];
            }
    };

    // ---- epilogue of N tile nt.  Lane l, register r of group (sm, sn): row
    // 32 sm + 8 (r / 4) + 4 (l / 32) + r % 4, the lane's column of half sn.
    auto epilogue = [&](int nt, auto smc) {
        constexpr int SM = decltype(smc)::value;
        const int br0 = brow_of(nt, 0), br1 = brow_of(nt, 1);
        const bool oc0 = ocol_of(nt, 0), oc1 = ocol_of(nt, 1);
        // the tile's first row, opaque to loop-invariant code motion: the
        // output addresses are formed at their stores, not kept in registers
        // across the N-tile loop
        int r0 = row0;
        __asm__ volatile("" : "+s"(r0));
        float amax = 0.f;                            // fp16 form: largest |value| stored by the lane
        if constexpr (kTr) {
            // transposed: lane l, register r of group (sm, sn) holds token row
            // 32 sm + l % 32 and output column 64 w + 32 sn + 8 (r / 4) +
            // 4 (l / 32) + r % 4 of the tile (N is a multiple of 32, so a
            // half is in range or not as a whole)
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const int m = 32 * sm + l32;
                if (m >= rows) continue;
#pragma unroll
                for (int sn = 0; sn < 2; ++sn) {
                    const int c0 = nt * BN + 64 * w + 32 * sn;
                    if (c0 >= g.N) continue;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float v[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v[i] = acc[sm][sn][4 * j + i];
                            if constexpr (kNL) v[i] *= 0.0625f;    // the fold's factor 16
                        }
                        const int64_t o = (int64_t)(r0 + m) * g.ldo + c0 + 8 * j + 4 * hh;
                        if (g.y16) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[i]));
                            *reinterpret_cast<uint2*>(g.y16 + o) =
                                make_uint2(pack2(f32_to_f16_bits(v[0]), f32_to_f16_bits(v[1])),
                                           pack2(f32_to_f16_bits(v[2]), f32_to_f16_bits(v[3])));
                        } else {
                            *reinterpret_cast<float4*>(g.out32 + o) = make_float4(v[0], v[1], v[2], v[3]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int sm = 0; sm < (kTr ? 0 : SM); ++sm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * sm + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (m >= rows) continue;
                if constexpr (kSwi) {
                    if (!oc0) continue;
                    const float u = acc[sm][0][r], gv = acc[sm][1][r];
                    const uint32_t bf = f32_to_bf16(gv / (1.0f + expf(-gv)) * u);
                    const uint16_t v = (uint16_t)f32_to_f16_bits(bf16_to_f32(bf));
                    g.out16[(int64_t)(r0 + m) * g.ldo + br0] = v;
                } else {
#pragma unroll
                    for (int sn = 0; sn < 2; ++sn) {
                        if (!(sn ? oc1 : oc0)) continue;
                        const int br = sn ? br1 : br0;
                        float v = acc[sm][sn][r];
                        if constexpr (kNL) v *= 0.0625f;           // the fold's factor 16
                        const int64_t o = (int64_t)(r0 + m) * g.ldo + br;
                        if (g.y16) {
                            amax = fmaxf(amax, fabsf(v));
                            g.y16[o] = (uint16_t)f32_to_f16_bits(v);
                        } else {
                            g.out32[o] = v;
                        }
                    }
                }
            }
        }
        if constexpr (!kSwi) {
            if (g.y16) {
                // the wave's largest value: beyond fp16's range, or a tile of
                // tiny nonzero values (where fp16 keeps few bits), sends the
                // layer's routed rows to the fp32 form
                float wm = amax;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o));
                if (lane == 0 && (wm > 65504.f || (wm > 0.f && wm < 0x1p-10f))) atomicAdd(g.range_flag, 1);
            }
        }
    };

    // ---- pipeline (two LDS stages for A, A registers alternating by step
    // parity).  Step kt: A(kt + 1) registers -> stage (kt + 1) % 2 (read last
    // in step kt - 1, before the barrier that ended it); load A(kt + 3) into
    // the freed registers; then, quantized: if step kt opens a period, its
    // bytes (loaded a period ago) go to the wave's area and the next period is
    // loaded; the lane's raw bytes of step kt are read, and per chunk kk the
    // fragments are decoded and the MFMAs issued.  Barrier.  Past the last step, loads repeat the last step or read unused
    // bytes.
    const int nk = g.K / BK;
    {
        // the decode tables (moe_decoders.hpp)
        if constexpr (kQ3) q3_quad_table_fill(lut, tid, 256);
        else if constexpr (kQ3K) q3_pair_table_fill(lut, tid, 256);
        else if constexpr (kNLS) nl4_pair_table_fill<16>(lut, tid, 256);
        else if constexpr (kNat) nl4_pair_table_fill<32>(lut, tid, 256);
        else if constexpr (kNL) nl4_fold_table_fill(lut, tid, 256);
        else nib_table_fill<kBF == BF_Q2S>(lut, tid, 256);
    }
    RawA A0, A1;
    load_a(0, A0);
    load_a(1 % nk, A1);
    put_a(0, A0);
    load_a(2 % nk, A0);

    auto run = [&](auto smc) {
        {
            // N tiles nt0 .. nt1 - 1 back to back: nk is even (or npb = 1), so the
            // A stages, A register slots and B periods carry on across tiles; A
            // rows are the same for every N tile, so A is loaded at k mod K.
            RawP P;
            load_period(nt0, 0, P);
            __syncthreads();                         // stage 0 and the table written
            const int npt = (nk + kPer - 1) / kPer;  // periods per N tile (the last may be half)
            // Ra: A(kt + 1) (refilled with kt + 3); opens: step kt starts a period
            auto step = [&](int nt, int kt, RawA& Ra, bool opens, Frag& F) {
                const int st = kt & 1;
                put_a(st ^ 1, Ra);
                if (opens) put_period(P);
                if constexpr (kB256) {               // a single N tile
                    load_a(min(kt + 3, nk - 1), Ra);
                    if (opens) load_period(nt, kt / kPer + 1, P);
                } else {
                    load_a((kt + 3) % nk, Ra);
                    if (opens) {
                        const int pn = kt / kPer + 1;    // next period: this tile's or the next tile's first
                        if (pn < npt) load_period(nt, pn, P);
                        else load_period(min(nt + 1, NT - 1), 0, P);
                    }
                }
                uint32_t q[2][kRawDw];
                if constexpr (kNat) {
                    read_blk(kt, 0, q);
                    decode_kk(kt, q, F, Cnt<0>{});
                    decode_kk(kt, q, F, Cnt<1>{});
                    nat_block(st, F, Cnt<0>{}, smc);
                    read_blk(kt, 1, q);
                    decode_kk(kt, q, F, Cnt<2>{});
                    decode_kk(kt, q, F, Cnt<3>{});
                    nat_block(st, F, Cnt<1>{}, smc);
                } else {
                    read_raw(kt, q);
                    decode_kk(kt, q, F, Cnt<0>{});
                    mma_kk(st, 0, F.f, smc);
                    decode_kk(kt, q, F, Cnt<1>{});
                    mma_kk(st, 1, F.f, smc);
                    decode_kk(kt, q, F, Cnt<2>{});
                    mma_kk(st, 2, F.f, smc);
                    decode_kk(kt, q, F, Cnt<3>{});
                    mma_kk(st, 3, F.f, smc);
                }
                __syncthreads();
            };
            Frag F;
            if constexpr (kB256) {
                // one N tile per block (48 steps at H = 3072); K = H is a multiple
                // of 256: a period per four steps, d applied after the fourth
                for (int kt = 0; kt < nk; kt += 4) {
                    step(nt0, kt, A1, true, F);
                    step(nt0, kt + 1, A0, false, F);
                    step(nt0, kt + 2, A1, false, F);
                    step(nt0, kt + 3, A0, false, F);
                    apply_d(F, smc);
                }
                epilogue(nt0, smc);
            } else {
                for (int nt = nt0; nt < nt1; ++nt) {
                    if (nt > nt0) {
#pragma unroll
                        for (int a = 0; a < kSMX; ++a)
#pragma unroll
                            for (int b = 0; b < 2; ++b)
#pragma unroll
                                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
                    }
                    int kt = 0;
                    for (; kt + 2 <= nk; kt += 2) {
                        step(nt, kt, A1, true, F);
                        step(nt, kt + 1, A0, false, F);
                    }
                    if (kt < nk) step(nt, kt, A1, true, F);
                    epilogue(nt, smc);
                }
            }
        }
    };
    // ---- the 6-bit sub-scaled codecs (one N tile per block, a period per
    // 256-weight block = 4 K steps).  Per step x of a block and column half
    // sn, the lane's raw bytes come from its row's window in the wave's
    // period area; Q3K-256 windows start 0 or 2 bytes before the block (the
    // block's dword alignment), so its words are realigned with a funnel
    // shift.
    auto run_sub = [&](auto smc) {
        constexpr int SM = decltype(smc)::value;
        RawP P;
        load_period(nt0, 0, P);
        __syncthreads();                             // stage 0 and the table written
        int rs[2];                                   // record offset of the lane's row, per half
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) rs[sn] = brow_of(nt0, sn) * rb_w;
        auto step_sub = [&](int kt, RawA& Ra) {
            const int x = kt & 3;                    // step within the block (wave-uniform)
            const int st = kt & 1;
            put_a(st ^ 1, Ra);
            if (x == 0) put_period(P);
            load_a(min(kt + 3, nk - 1), Ra);
            if (x == 0) load_period(nt0, kt / kPer + 1, P);
            if constexpr (kQ3K) {
                // per half: the step's 24 index bytes (6 words), d / 128 and the
                // step's four 6-bit sub-scales (bits 24 x .. 24 x + 23 of the 96)
                uint32_t fq[2][4], f24[2];
                float dl[2];
#pragma unroll
                for (int sn = 0; sn < 2; ++sn) {
                    const uint32_t* rw = reinterpret_cast<const uint32_t*>(&Bq[w][(32 * sn + l32) * kRowB]);
                    const bool sh = ((rs[sn] + kQ3KBytes * (kt >> 2)) & 2) != 0;
                    auto al = [&](uint32_t lo, uint32_t hi) { return sh ? __builtin_amdgcn_alignbit(hi, lo, 16) : lo; };
                    uint32_t dw[7], q[6];
#pragma unroll
                    for (int i = 0; i < 7; ++i) dw[i] = rw[6 * x + i];
#pragma unroll
                    for (int i = 0; i < 6; ++i) q[i] = al(dw[i], dw[i + 1]);
                    // the lane's 8 codes of chunk kk: bits 48 kk + 24 h of the 192
                    fq[sn][0] = hh ? __builtin_amdgcn_alignbit(q[1], q[0], 24) : q[0];
                    fq[sn][1] = hh ? (q[2] >> 8) : __builtin_amdgcn_alignbit(q[2], q[1], 16);
                    fq[sn][2] = hh ? __builtin_amdgcn_alignbit(q[4], q[3], 24) : q[3];
                    fq[sn][3] = hh ? (q[5] >> 8) : __builtin_amdgcn_alignbit(q[5], q[4], 16);
                    const uint32_t t24 = rw[24], t25 = rw[25], t26 = rw[26], t27 = rw[27];
                    const uint32_t W0 = al(t24, t25), W1 = al(t25, t26), W2 = al(t26, t27);
                    const uint32_t W3 = sh ? (t27 >> 16) : t27;
                    const uint32_t S0 = __builtin_amdgcn_alignbit(W1, W0, 16);
                    const uint32_t S1 = __builtin_amdgcn_alignbit(W2, W1, 16);
                    const uint32_t S2 = __builtin_amdgcn_alignbit(W3, W2, 16);
                    f24[sn] = x == 0 ? S0 : x == 1 ? __builtin_amdgcn_alignbit(S1, S0, 24)
                              : x == 2 ? __builtin_amdgcn_alignbit(S2, S1, 16) : (S2 >> 8);   // bits 24 x ..
                    dl[sn] = f16_bits_to_f32(W0 & 0xffffu) * 0.0078125f;
                }
                // chunk kk = the 16-weight sub-block 4 x + kk.  B = s * c with
                // |s c| up to 4064, beyond fp16's exact integers: it enters as
                // the two exact parts (s mod 16) c and 16 floor(s / 16) c, each
                // an fp16 integer, summed by two MFMAs into the block's
                // partial sums; d / 128 is applied to those at the block's end.
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    u32x4 fa[SM];
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm) fa[sm] = As[st][aslot(32 * sm + l32, 2 * kk + hh)];
#pragma unroll
                    for (int sn = 0; sn < 2; ++sn) {
                        const uint32_t f = fq[sn][kk];
                        // a plain array: clang lowers __builtin_bit_cast of an
                        // ext_vector element as a read of element 0
                        const uint32_t fw[1] = {f};
                        uint32_t fb[4];
                        fb[0] = lds_ld(q3_pair_addr<0>(fw, cb));
                        fb[1] = lds_ld(q3_pair_addr<6>(fw, cb));
                        fb[2] = lds_ld(q3_pair_addr<12>(fw, cb));
                        fb[3] = lds_ld(q3_pair_addr<18>(fw, cb));
                        f16x2_t slo2, shi2;
                        q3k_split(sext6(f24[sn] >> (6 * kk)), slo2, shi2);
                        u32x4 b1, b2;
#pragma unroll
                        for (int pq = 0; pq < 4; ++pq) {
                            b1[pq] = mul_pair(fb[pq], slo2);
                            b2[pq] = mul_pair(fb[pq], shi2);
                        }
#pragma unroll
                        for (int sm = 0; sm < SM; ++sm) {
                            tmp[sm][sn] = mfma32_f16(fa[sm], b1, tmp[sm][sn]);
                            tmp[sm][sn] = mfma32_f16(fa[sm], b2, tmp[sm][sn]);
                        }
                    }
                }
                if (x == 3) {                                // block done: acc += partial * d / 128
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                        for (int sn = 0; sn < 2; ++sn)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                acc[sm][sn][r] += tmp[sm][sn][r] * dl[sn];
                                tmp[sm][sn][r] = 0.f;
                            }
                }
            } else {
                // NL4S-256: sub-block 2 x + c is chunks 2c, 2c + 1 (one index
                // word each); d and the 48 sub-scale bits in words 32-33
                uint64_t sv[2];
                float dl[2];
#pragma unroll
                for (int sn = 0; sn < 2; ++sn) {
                    const uint32_t* rw = reinterpret_cast<const uint32_t*>(&Bq[w][(32 * sn + l32) * kRowB]);
                    const uint32_t t32 = rw[32], t33 = rw[33];
                    sv[sn] = ((uint64_t)t33 << 16) | (t32 >> 16);
                    dl[sn] = f16_bits_to_f32(t32 & 0xffffu) * 0.0078125f;
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 fa[SM][2];
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2) fa[sm][k2] = As[st][aslot(32 * sm + l32, 2 * (2 * c + k2) + hh)];
#pragma unroll
                    for (int sn = 0; sn < 2; ++sn) {
                        const uint32_t* rw = reinterpret_cast<const uint32_t*>(&Bq[w][(32 * sn + l32) * kRowB]);
                        u32x4 fb[2];
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2) {
                            const uint32_t nb = rw[8 * x + 2 * (2 * c + k2) + hh];
                            fb[k2][0] = lds_ld(nl_addr(nb, Cnt<0>{}));
                            fb[k2][1] = lds_ld(nl_addr(nb, Cnt<1>{}));
                            fb[k2][2] = lds_ld(nl_addr(nb, Cnt<2>{}));
                            fb[k2][3] = lds_ld(nl_addr(nb, Cnt<3>{}));
                        }
                        const float sc = dl[sn] * (float)sext6((uint32_t)(sv[sn] >> (12 * x + 6 * c)));
#pragma unroll
                        for (int sm = 0; sm < SM; ++sm) {
                            f32x16 t = mfma32_f16(fa[sm][0], fb[0], f32x16{});
                            t = mfma32_f16(fa[sm][1], fb[1], t);
#pragma unroll
                            for (int r = 0; r < 16; ++r) acc[sm][sn][r] += t[r] * sc;
                        }
                    }
                }
            }
            __syncthreads();
        };
        for (int kt = 0; kt < nk; kt += 2) {
            step_sub(kt, A1);
            step_sub(kt + 1, A0);
        }
        epilogue(nt0, smc);
    };

    // The loop is instantiated per count of live 32-row groups (ragged
    // expert tails skip the MFMAs of groups past their rows).
    const int nsm = __builtin_amdgcn_readfirstlane((rows + 31) >> 5);
    static_assert(kSMX == 2, "64-row tiles");
    if constexpr (kSub) {
        if (nsm == 2) run_sub(Cnt<2>{});
        else run_sub(Cnt<1>{});
    } else {
        if (nsm == 2) run(Cnt<2>{});
        else run(Cnt<1>{});
    }

}

// ---------------------------------------------------------------- launchers

static unsigned gemm_grid(int n_tiles, int m_tiles) {
    const int MTp = ((m_tiles + 7) / 8) * 8;
    return (unsigned)(n_tiles * MTp);
}
static int swi_tiles(int half_n) { return (half_n + BN / 2 - 1) / (BN / 2); }
static int col_tiles(int n) { return (n + BN - 1) / BN; }

void launch_gemm_upgate(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                        const int32_t* ntiles, int max_tiles, const int32_t* perm, int k,
                        const uint16_t* x16, int H, int I, uint16_t* a16_perm, int fmt,
                        hipStream_t st) {
    GemmArgs a{};
    a.experts = experts; a.estride = estride; a.tiles = tiles; a.ntiles = ntiles;
    a.max_tiles = max_tiles; a.perm = perm; a.k = k; a.A = x16; a.lda = H;
    a.N = 2 * I; a.K = H; a.half_n = I; a.H = H; a.I = I; a.out16 = a16_perm; a.ldo = I;
    a.npb = 1;
    const unsigned grid = gemm_grid((swi_tiles(I) + a.npb - 1) / a.npb, max_tiles);
    if (fmt == kFmtQ3S256) k_gemm<UG_Q3><<<grid, 256, 0, st>>>(a);
    else if (fmt == kFmtQ2S256) k_gemm<UG_Q2S><<<grid, 256, 0, st>>>(a);
    else if (fmt == kFmtQ3K256) k_gemm<UG_Q3K><<<grid, 256, 0, st>>>(a);
    else if (fmt == kFmtNL4S256) k_gemm<UG_NL4S><<<grid, 256, 0, st>>>(a);
    else k_gemm<UG_NL4><<<grid, 256, 0, st>>>(a);
}

void launch_gemm_down(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                      const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int H,
                      int I, int64_t dn_off, int fmt, float* y_perm, uint16_t* y_perm16,
                      int* range_flag, const int* only_if, hipStream_t st) {
    GemmArgs a{};
    a.experts = experts; a.estride = estride; a.tiles = tiles; a.ntiles = ntiles;
    a.max_tiles = max_tiles; a.A = a16_perm; a.lda = I; a.N = H; a.K = I; a.H = H; a.I = I;
    a.dn_off = dn_off; a.out32 = y_perm; a.y16 = y_perm16; a.range_flag = range_flag;
    a.only_if = only_if; a.ldo = H;
    a.npb = (I / BK) % 2 == 0 ? 4 : 1;               // tiles chain only with an even step count
    const unsigned grid = gemm_grid((col_tiles(H) + a.npb - 1) / a.npb, max_tiles);
    if (fmt == kFmtNL4) k_gemm<DN_NL4><<<grid, 256, 0, st>>>(a);
    else k_gemm<DN_Q2><<<grid, 256, 0, st>>>(a);
}

}  // namespace moe
