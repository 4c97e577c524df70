// Host-side launchers of the libmoe kernels (one per kernel family), called
// by the C ABI in moe_api.hip.  Every launcher only enqueues on `st`.
#pragma once

#include "moe_common.hpp"

namespace moe {

// Work sizes shared by host and device code.
constexpr int kDecMaxT = 16;          // tokens handled by the bandwidth path
constexpr int kShKChunk = 256;        // K per shared up|gate partial (bandwidth path)
constexpr int kDecLogitParts = 4;     // K parts of the layer's router on the bandwidth path
constexpr int kMaxLogitParts = 4;
constexpr int kMaxSlots = kDecMaxT * 32;  // T * k slots of the bandwidth path
constexpr int kGemmBM = 64;           // rows per grouped-GEMM tile
constexpr int kGemmBN = 256;          // weight rows per grouped-GEMM tile
constexpr int kGemmBK = 64;

// ---- small kernels (moe_kernels_small.hip)
void launch_dequant(int fmt, const void* blocks, int64_t n_weights, float* out, hipStream_t st);
// through the table decoders of the layer's kernels: fmt Q3S256 or NL4_32,
// path 0 (bandwidth-path kernels) or 1 (grouped GEMM)
void launch_dequant_path(int fmt, int path, const void* blocks, int64_t n_weights, float* out, hipStream_t st);
void launch_to_f16(const uint16_t* x, uint16_t* x16, int64_t n, hipStream_t st);
// with x16 (H a multiple of 256, at most 8192): also x16 = fp16(x), one row per token
void launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                 int32_t* ids2, float* w2, const uint16_t* x, uint16_t* x16, int H, hipStream_t st);
void launch_permute_small(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t st);
void launch_permute_large(const int32_t* ids, int T, int k, int E, int BM, int32_t* hist,
                          int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles,
                          int32_t* ntiles, hipStream_t st);
void launch_build_tiles(const int32_t* offsets, int E, int BM, int32_t* tiles, int32_t* ntiles,
                        hipStream_t st);
void launch_combine(const float* y_perm, const int* fp16_unless, const int32_t* inv, const float* w,
                    int T, int k, int H, const float* shared, float* y, hipStream_t st);
void launch_rmsnorm(float* h, const float* delta, const float* gamma, float eps, int T, int H,
                    uint16_t* normed, hipStream_t st);
// The combine with the residual add and the next RMSNorm: h [T][H] += the
// combined rows; normed = bf16(gamma * h / rms) when gamma is not null.
// H a multiple of 4 up to 8192; h, gamma 16-byte and normed 8-byte aligned.
void launch_combine_norm(const float* y_perm, const int* fp16_unless, const int32_t* inv, const float* w,
                         int T, int k, int H, const float* shared, float* h, const float* gamma,
                         float eps, uint16_t* normed, hipStream_t st);

// ---- bandwidth path (moe_kernels_decode.hip), T <= kDecMaxT and
// upgate_dec_supported(H, T, E) (the staged up|gate rows of two items and the
// routing scratch fit in LDS)
bool upgate_dec_supported(int H, int T, int E);
// kp: K parts of the router (1: logits[T][E] with the bias; > 1: partial
// planes logits[kp][T][E] without it, for the up|gate kernel's routing)
void launch_dec_stage1(const uint16_t* x, int T, int H, int E, const uint16_t* w_r,
                       const float* bias, float* logits, const uint16_t* sh_ug, int Is,
                       float* shp, uint16_t* x16, int kp, hipStream_t st);
// Routing results of the bandwidth path, written by the up|gate kernel.
struct RouteOut {
    int32_t* ids;
    float* w;
    int32_t* ids_out;        // optional copies for the caller
    float* w_out;
    int32_t* offsets;        // [E + 1]
    int32_t* perm;           // [T * k]
    int32_t* inv;            // [T * k]
    int32_t* tiles;          // [3 * active experts]
    int32_t* ntiles;
};
// logits: np planes [np][T][E] summed in plane order, then lbias if non-null
void launch_upgate_dec(const uint8_t* experts, int64_t estride, const float* logits, int np,
                       const float* lbias, int E, int k, int max_tiles, const uint16_t* x16, int T, int H, int I,
                       uint16_t* a16_perm, const float* shp, int Is, uint16_t* a_sh,
                       const RouteOut& ro, int n_cu, hipStream_t st);
void launch_down_dec(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                     const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int T, int H,
                     int I, int k, const uint16_t* sh_down, const uint16_t* a_sh, int Is,
                     float* y_perm, float* y_sh, int n_cu, hipStream_t st);

// ---- grouped-GEMM path (moe_kernels_gemm.hip)
// fmt: the up|gate format (Q3S-256, Q2S-256, NL4-32, Q3K-256 or NL4S-256)
void launch_gemm_upgate(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                        const int32_t* ntiles, int max_tiles, const int32_t* perm, int k,
                        const uint16_t* x16, int H, int I, uint16_t* a16_perm, int fmt,
                        hipStream_t st);
// dn_off: byte offset of the down matrix in an expert record; fmt: its format
// (NL4-32 or Q2-32).  The unweighted rows are stored fp32 to y_perm, or, with
// y_perm16, as fp16 there with the range check that adds to *range_flag
// (beyond 65504, or a wave's tile of tiny nonzero values).  only_if non-null:
// the launch does nothing unless *only_if != 0.
void launch_gemm_down(const uint8_t* experts, int64_t estride, const int32_t* tiles,
                      const int32_t* ntiles, int max_tiles, const uint16_t* a16_perm, int H,
                      int I, int64_t dn_off, int fmt, float* y_perm, uint16_t* y_perm16,
                      int* range_flag, const int* only_if, hipStream_t st);

// ---- dense bf16 products of the grouped-GEMM path (moe_kernels_dense.hip)
// One launch: router logits [T][E] (+ bias) if w_r is not null, and the
// shared expert's SwiGLU activations a_sh bf16 [T][Is] if sh_ug is not null.
void launch_dense_router_shared(const uint16_t* x, int T, int H, int E, const uint16_t* w_r,
                                const float* bias, float* logits, const uint16_t* sh_ug, int Is,
                                uint16_t* a_sh, hipStream_t st);
// The shared expert's down projection: y_sh fp32 [T][H] = a_sh W_down^T.
void launch_dense_shared_down(const uint16_t* a_sh, int T, int Is, const uint16_t* sh_down, int H,
                              float* y_sh, hipStream_t st);

}  // namespace moe
