/*
 * moe.h -- C ABI of libmoe.so: the routed, block-quantized Mixture-of-Experts
 * FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: "Avalon" README, opening paragraphs -- each token goes to
 * 10 of 512 experts, 48 layers; "Qwen3.8-Flash-Next - Avalon GGUF" model card,
 * "Files / Main model" -- routers and shared experts in the dense part, routed
 * up/gate in a 3.25-bpw type with a scale per 256-weight block and per-32
 * sub-scales, down in a 4-bit non-linear 32-weight type, experts packed
 * up | gate | down; "Betelgeuse" post (2026-11-01) -- every routed expert is
 * computed exactly, no gate pruning):
 *
 *   L[t][e]  = sum_h x[t][h] * W_r[e][h] + b[e]                 (router)
 *   ids[t]   = the k largest L[t][.], by (value desc, index asc)
 *   w[t][j]  = softmax over the k selected logits
 *   a        = bf16_rne( silu(W_gate x) * (W_up x) )              (per slot)
 *   o        = W_down a                                           (per slot)
 *   y[t]     = sum_j w[t][j] * o[t,j]  +  shared_expert(x[t])
 *
 * Conventions for every function below
 *   - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *     allocates and frees every buffer, the workspace included; the library
 *     never allocates or frees device memory and keeps no state except a cache
 *     of device properties and, for moe_layer_forward_noalloc only, one array
 *     per GPU that the library's own code holds.  Calls are re-entrant;
 *     concurrent calls need distinct workspaces and outputs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on it; no call synchronises the host.
 *   - All argument checks (null pointers, shapes, formats, alignment,
 *     workspace size, device architecture) run on the host BEFORE any launch.
 *     On failure the call returns a non-zero moe_status, launches nothing and
 *     leaves every output untouched; moe_last_error() then holds a message.
 *     A failed launch returns MOE_ERR_HIP.  Faults inside a kernel are
 *     asynchronous and surface at the caller's next synchronisation.
 *   - Element types: bf16 and fp16 are passed as uint16_t bit patterns.
 *   - Preconditions not checked on the device: expert ids given to
 *     moe_permute lie in [0, E) and are distinct within each token's row;
 *     logits are not NaN; weight scales d are finite, and |d| <= 32752 in
 *     MOE_FMT_Q2_32 blocks (the grouped GEMM forms d (q - 2) in fp16); the
 *     activations x and the SwiGLU outputs a (below) satisfy |v| <= 65504.
 *   - Numerics.  Accumulation is fp32 everywhere.  The matrix cores take x
 *     and a as fp16: a bf16 value v converts exactly when 2^-17 <= |v| <=
 *     65504 and with an absolute error <= 2^-25 below that (|v| > 65504
 *     would become inf).  Routed weights enter exactly (the quantized
 *     integers, with the scales applied in fp32 to partial sums, or the
 *     products d (q - 2) of Q2_32, exact in fp16 for |d| <= 32752), except the
 *     NL4_32 down weights of the grouped-GEMM path (T > 16 or the mixed
 *     formats), which enter as fp16_rne(16 d T4[q] / 128) / 16: relative
 *     error <= 2^-11 for every normal d up to 4126, absolute <= 2^-29 for a
 *     subnormal d.  The unweighted routed rows y_perm are fp32 on the bandwidth
 *     path; the grouped-GEMM path of moe_layer_forward holds them in fp16
 *     (relative error <= 2^-11) unless a range check in the down GEMM finds a
 *     value beyond 65504 or a tile of values all below 2^-10 (not all zero),
 *     and then recomputes them in fp32; moe_expert_ffn returns them in fp32.
 *     The shared expert and the router are bf16 x bf16 products.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,       /* a required pointer is NULL                     */
    MOE_ERR_SHAPE = 2,      /* a size is out of the supported range           */
    MOE_ERR_FORMAT = 3,     /* unknown or unsupported weight format           */
    MOE_ERR_ALIGN = 4,      /* a pointer or stride is not 16-byte aligned     */
    MOE_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than required        */
    MOE_ERR_DEVICE = 6,     /* current device is not gfx950                   */
    MOE_ERR_HIP = 7         /* a HIP runtime call or kernel launch failed     */
} moe_status;

/* Weight formats.
 *  MOE_FMT_BF16    plain bf16, row-major [out][in].
 *  MOE_FMT_Q3S256  3.25-bpw super-blocks of 256 weights, 104 bytes each:
 *                  bytes [0,96) 256 3-bit codebook indices as one little-endian
 *                  bit stream (weight i at bits 3i..3i+2); [96,98) fp16 scale d
 *                  (little-endian, any finite value, subnormals included);
 *                  [98,102) eight signed 4-bit sub-scales s_j (bits 4j..4j+3
 *                  of that little-endian u32, two's complement); [102,104)
 *                  reserved (ignored).  w_i = d * s_{i/32} * C3[q_i] / 128 with
 *                  C3 = {-127,-67,-31,0,23,48,78,127}.  (Model card, "Files /
 *                  Main model": 3.25 bpw, a scale per 256-weight block,
 *                  sub-scales per 32 weights.)
 *  MOE_FMT_NL4_32  4-bit non-linear 32-weight blocks, 18 bytes each: [0,2)
 *                  fp16 d; [2,18) 32 4-bit indices, even weight in the low
 *                  nibble.  w_i = d * T4[q_i] / 128 with T4 = {-127,-88,-66,
 *                  -50,-36,-23,-11,0,10,20,31,43,56,71,91,127}.  (Model card,
 *                  "Files / Main model": IQ4_NL down tensors.)
 *  MOE_FMT_Q2S256  2.5-bpw super-blocks of 256 weights, 80 bytes each: [0,64)
 *                  256 2-bit indices (weight i at bits 2i..2i+1 of the
 *                  little-endian stream); [64,66) fp16 d; [66,70) eight signed
 *                  4-bit sub-scales as in Q3S256; [70,80) reserved (ignored).
 *                  w_i = d * s_{i/32} * C2[q_i] / 128, C2 = {-127,0,54,127}.
 *                  (A reading of the model card's IQ2_S up/gate layers, which
 *                  the page names only.)
 *  MOE_FMT_Q2_32   2-bit 32-weight blocks, 10 bytes each: [0,2) fp16 d;
 *                  [2,10) 32 2-bit q (weight i at bits 2i..2i+1).  w_i =
 *                  d * (q_i - 2).  (A reading of the model card's Q2_0 down
 *                  layers, which the page names only.)
 *  MOE_FMT_Q3K256  3.4375-bpw super-blocks of 256 weights, 110 bytes each:
 *                  [0,96) 256 3-bit indices as in Q3S256; [96,98) fp16 d;
 *                  [98,110) sixteen signed 6-bit sub-scales, one per 16
 *                  weights (s_j = bits 6j..6j+5 of that little-endian 96-bit
 *                  field, two's complement).  w_i = d * s_{i/16} * C3[q_i] / 128.
 *                  (A reading of the model card's IQ3_K up/gate type, "3.44
 *                  bpw", and of the draft head's experts, "MTP sidecar".)
 *  MOE_FMT_NL4S256 4.25-bpw super-blocks of 256 weights, 136 bytes each:
 *                  [0,128) 256 4-bit indices as in NL4_32; [128,130) fp16 d;
 *                  [130,136) eight signed 6-bit sub-scales, one per 32 weights.
 *                  w_i = d * s_{i/32} * T4[q_i] / 128.  (A reading of the model
 *                  card's IQ4_XS up/gate type, 4.25 bpw.)
 * Matrices are stored [out rows][in] with blocks along the input dimension. */
typedef enum {
    MOE_FMT_BF16 = 1,
    MOE_FMT_Q3S256 = 2,
    MOE_FMT_NL4_32 = 3,
    MOE_FMT_Q2S256 = 4,
    MOE_FMT_Q2_32 = 5,
    MOE_FMT_Q3K256 = 6,
    MOE_FMT_NL4S256 = 7
} moe_format;

/* Layer shape.  Supported: hidden % 256 == 0 (and <= 8192); inter % 64 == 0
 * (and <= 4096); 1 <= top_k <= min(n_experts, 32); 1 <= n_experts <= 1024;
 * shared_inter == 0 (no shared expert) or shared_inter % 64 == 0 (<= 4096);
 * routed up|gate in MOE_FMT_Q3S256, MOE_FMT_Q2S256, MOE_FMT_NL4_32,
 * MOE_FMT_Q3K256 or MOE_FMT_NL4S256 and routed down in MOE_FMT_NL4_32 or
 * MOE_FMT_Q2_32 (the model card's mixed-format layers and draft head use
 * these); the shared expert and the router are always bf16.  Batches of T <= 16 tokens with Q3S256 / NL4_32
 * experts take the bandwidth kernels; every other case the grouped GEMMs. */
typedef struct {
    int32_t hidden;        /* H                                              */
    int32_t inter;         /* I, routed expert intermediate size             */
    int32_t n_experts;     /* E                                              */
    int32_t top_k;         /* k                                              */
    int32_t shared_inter;  /* I_s, 0 = no shared expert                      */
    int32_t upgate_fmt;    /* moe_format of the routed up|gate matrices      */
    int32_t down_fmt;      /* moe_format of the routed down matrices         */
} moe_layer_desc;

/* Layer weights (device pointers).  Each routed expert e is one record at
 * experts + e*expert_stride: its up|gate matrix [2I][H] (rows 0..I-1 = up,
 * I..2I-1 = gate; model card: "up | gate | down contiguous"), immediately
 * followed by its down matrix [H][I].  `experts` and `expert_stride` must be
 * 16-byte aligned and expert_stride >= the record size. */
typedef struct {
    const void*  experts;        /* E packed records                           */
    int64_t      expert_stride;  /* bytes between records                      */
    const void*  router_w;       /* bf16 [E][H], or NULL if logits are given   */
    const float* router_b;       /* fp32 [E], or NULL (no bias)                */
    const void*  shared_upgate;  /* bf16 [2*I_s][H] (up rows, then gate rows)  */
    const void*  shared_down;    /* bf16 [H][I_s]                              */
} moe_layer_weights;

/* Bytes of workspace moe_layer_forward / moe_expert_ffn / moe_permute need for
 * any T <= T_max.  Host-only, pure; returns 0 for an invalid desc/T_max. */
size_t moe_workspace_size(const moe_layer_desc* desc, int32_t T_max);

/* Router logits: logits[t][e] = sum_h x[t][h] * W_r[e][h] + b[e], fp32
 * accumulation.  x bf16 [T][H], w_r bf16 [E][H], b fp32 [E] or NULL, logits
 * fp32 [T][E].  Same kernels moe_layer_forward runs.  ws / ws_bytes are
 * not used (may be NULL / 0).
 * Reading: the pages place "routers" in the dense part (model card, "Files /
 * Main model") and give no formula; a linear router with a per-expert bias. */
moe_status moe_router_logits(const uint16_t* x, int32_t T, int32_t H, int32_t E,
                             const uint16_t* w_r, const float* b, float* logits,
                             void* ws, size_t ws_bytes, void* stream);

/* Top-k routing.  logits fp32 [T][E] -> topk_ids int32 [T][k] (by
 * descending logit, ties to the lower index) and topk_w fp32 [T][k] = softmax
 * of the selected logits.  No capacity limit, nothing dropped ("Betelgeuse":
 * every one of the routed experts is computed).  1 <= k <= min(E, 32),
 * E <= 1024, T >= 1. */
moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_w, void* stream);

/* Counting-sort permutation.  Each token's slots go to k experts ("Avalon"
 * README, opening paragraphs: 10 of 512 per token) and every selected expert
 * is computed ("Betelgeuse" post: none is dropped); grouping a batch's slots
 * by expert lets each expert's weights be read once per batch.
 * topk_ids int32 [T][k] (values in [0,E), distinct within a row) ->
 * offsets int32 [E+1] (expert e owns permuted rows offsets[e]..offsets[e+1]-1,
 * offsets[E] = T*k), perm int32 [T*k] (permuted row p holds flat slot
 * f = t*k + j; stable: ascending f within an expert) and inv_perm int32 [T*k]
 * (inv_perm[perm[p]] = p).  Bit-exact and deterministic. */
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs.  Model card, "Files / Main model": each routed expert
 * is an up, a gate and a down matrix (packed up | gate | down) in the
 * quantized types above; the shared expert sits in the dense bf16 part.  The
 * up/gate pair is read as a SwiGLU unit, and a is rounded to bf16, the
 * activation type of the dense part.  For every permuted row p of expert e
 * (token t = perm[p] / k): y_perm[p] = W_down[e] bf16_rne(silu(W_gate[e] x[t]) *
 * W_up[e] x[t]), unweighted, fp32 [T*k][H].  If shared_y is not NULL and
 * desc->shared_inter > 0 the shared expert's output for every token is
 * written to shared_y fp32 [T][H].  x bf16 [T][H]; offsets/perm as produced by
 * moe_permute (the library also rebuilds its internal tile list from them).
 * T <= 16 with Q3S_256 up|gate and NL4_32 down runs the bandwidth kernels
 * (routing taken from offsets/perm), anything else the grouped GEMMs. */
moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_layer_weights* wts,
                          const uint16_t* x, int32_t T, const int32_t* offsets,
                          const int32_t* perm, float* y_perm, float* shared_y,
                          void* ws, size_t ws_bytes, void* stream);

/* Weighted combine: the layer output is the router-weighted sum of the
 * token's k routed experts plus the shared expert ("Avalon" README, opening
 * paragraphs; model card, "Files / Main model").
 * y[t] = sum_{j<k} topk_w[t][j] * y_perm[inv_perm[t*k+j]] (+ shared_y[t] if
 * not NULL), summed in j order, fp32 [T][H]. */
moe_status moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                       int32_t T, int32_t k, int32_t H, const float* shared_y,
                       float* y, void* stream);

/* The whole layer, as the formula at the top of this file (its
 * sources there): y fp32 [T][H] from x bf16 [T][H].  If
 * logits_or_null is given (fp32 [T][E]) the router is skipped.  Optional
 * outputs: topk_ids_out int32 [T][k], topk_w_out fp32 [T][k].  Tokens T <= 16
 * take the bandwidth path (every weight byte streamed once), larger T the
 * grouped-GEMM path; both compute the same function, and each output row is
 * summed in a fixed order (runs repeat bit for bit). */
moe_status moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* wts,
                             const uint16_t* x, int32_t T, const float* logits_or_null,
                             float* y, int32_t* topk_ids_out, float* topk_w_out,
                             void* ws, size_t ws_bytes, void* stream);

/* The layer with the residual add and the next layer's RMSNorm of a pre-norm
 * stack fused into its combine: h[t] += y[t] for the layer output y of
 * moe_layer_forward (which is not written), then, if gamma and
 * normed_bf16_out are not NULL, normed[t] = bf16_rne(gamma * h[t] /
 * sqrt(mean(h[t]^2) + eps)).  The stack is the model card's 48 layers
 * ("Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model"); the pages do
 * not spell out where the norm sits, and each layer reading the normalised
 * residual stream and adding its output back is the plain reading.  h fp32 [T][H]
 * (updated in place, 16-byte aligned), gamma fp32 [H] (16-byte aligned),
 * normed bf16 [T][H] (8-byte aligned); the other arguments as in
 * moe_layer_forward.  The results are the same bits as moe_layer_forward
 * followed by moe_rmsnorm_residual(h, y, gamma, eps, ...). */
moe_status moe_layer_forward_residual(const moe_layer_desc* desc, const moe_layer_weights* wts,
                                      const uint16_t* x, int32_t T, const float* logits_or_null,
                                      float* h, const float* gamma, float eps,
                                      uint16_t* normed_bf16_out, int32_t* topk_ids_out,
                                      float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* Instrumented moe_layer_forward, for measurement: identical work, and in
 * addition events[0] (hipEvent_t, created by the caller) is recorded on
 * `stream` before the first kernel and events[i] after the i-th kernel, while
 * i < n_events.  *n_marks receives the number of marks the call wanted
 * (kernels + 1).  Kernel order -- T <= 16: stage 1 (router logits, shared
 * up|gate partials, fp16 copy of x), routed up|gate (routing, top-k and
 * permutation, at its start), down projections (routed + shared), combine;
 * T > 16: [router and shared up|gate GEMM (if no logits or a shared
 * expert)], top-k (with the fp16 copy of x), permutation (3 kernels, one mark), [shared
 * down GEMM], routed up|gate GEMM, routed down GEMM (fp16 rows), its fp32
 * repeat (does nothing unless the range check asked for it), combine. */
moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const moe_layer_weights* wts,
                                   const uint16_t* x, int32_t T, const float* logits_or_null,
                                   float* y, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                                   size_t ws_bytes, void* stream, void* const* events,
                                   int32_t n_events, int32_t* n_marks);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * exactly as moe_layer_forward (same kernels, same results bit for bit), with
 * no workspace argument: the workspace is an array of
 * MOE_NOALLOC_SCRATCH_BYTES owned by the library, one per GPU, allocated with
 * the library's code on that GPU and held until the process ends.  The call
 * itself allocates nothing.  Returns MOE_ERR_WORKSPACE (launching nothing)
 * when moe_workspace_size(desc, T) exceeds that size -- at the model's shape
 * (H = 3072, I = 512, 512 experts, top-10, I_s = 512) every batch up to 428
 * tokens fits.  All calls on one GPU share its array: calls that overlap in
 * time on one GPU (other streams, other host threads) race and must be
 * serialised by the caller; calls on one stream are. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const moe_layer_weights* wts,
                                     const uint16_t* x, int32_t T, const float* logits_or_null,
                                     float* y, int32_t* topk_ids_out, float* topk_w_out,
                                     void* stream);

/* Helper, not the method: dequantize n_weights weights of one quantized format
 * (Q3S256, NL4_32, Q2S256, Q2_32, Q3K256 or NL4S256; a whole number of
 * blocks, contiguous) to fp32 `out` with per-block device decoders.  Exact:
 * equal bit for bit to d*s*c/128 (Q3S256, Q2S256, Q3K256), d*t/128 (NL4_32),
 * d*s*t/128 (NL4S256) or d*(q-2) (Q2_32).  blocks must be 16-byte aligned. */
moe_status moe_dequantize(int32_t fmt, const void* blocks, int64_t n_weights, float* out,
                          void* stream);

/* Helper, not the method: dequantize through the table decoders that the
 * layer's kernels inline -- the same tables, lookup addresses and fp16
 * multiplies, then the fp32 factor the kernel applies to its partial sums --
 * so that a bit-exact comparison covers the decoders of the hot path (model
 * card "Qwen3.8-Flash-Next - Avalon GGUF", "Files / Main model": the routed
 * up/gate types with a scale per 256-weight block and sub-scales, the 4-bit
 * non-linear and 2-bit down types).  path:
 *   MOE_PATH_BANDWIDTH  the bandwidth-path kernels (T <= 16): Q3S256 from the
 *                       pair table (6-bit index -> two codebook values) times
 *                       s, then d/128; NL4_32 from its pair table (index byte
 *                       -> two values), then d/128 -- the decoder the grouped
 *                       GEMM's NL4_32 up|gate mode runs too.  Exact.
 *   MOE_PATH_GEMM       the grouped GEMM's down and up|gate modes: Q3S256 from
 *                       the quad table (12-bit index -> four values) times s,
 *                       then d/128; NL4_32 as down weights, fp16_rne(16 d t /
 *                       128) / 16 (the one rounding that path applies to
 *                       them); Q2S256 (nibble table times s, then d/128),
 *                       Q2_32 (nibble table of q - 2 times d in fp16: exact
 *                       for |d| <= 32752, +-inf for code 0 beyond), Q3K256 (pair
 *                       table times the two exact parts of s, summed, then
 *                       d/128), NL4S256 (the NL4 table in 16 copies, then
 *                       d s/128).  Exact except the NL4_32 fold and Q2_32
 *                       beyond its bound; a zero weight may carry either sign.
 * Other formats (or Q2S256, Q2_32, Q3K256, NL4S256 on the bandwidth path):
 * MOE_ERR_FORMAT.  Blocks contiguous and 16-byte aligned, n_weights a
 * positive multiple of the block size; out fp32. */
#define MOE_PATH_BANDWIDTH 0
#define MOE_PATH_GEMM 1
moe_status moe_dequantize_path(int32_t fmt, int32_t path, const void* blocks, int64_t n_weights,
                               float* out, void* stream);

/* Helper for stacked layers (pre-norm residual): if delta is not NULL,
 * h += delta; then, if gamma and normed_bf16_out are not NULL,
 * normed[t] = bf16_rne(gamma * h[t] / sqrt(mean(h[t]^2) + eps)).  h fp32 [T][H]
 * (updated in place), delta fp32 [T][H], gamma fp32 [H], normed bf16 [T][H]. */
moe_status moe_rmsnorm_residual(float* h, const float* delta, const float* gamma, float eps,
                                int32_t T, int32_t H, uint16_t* normed_bf16_out, void* stream);

/* Static description of a status code (host). */
const char* moe_status_string(moe_status s);
/* Detail of the last failure on the calling thread (host; "" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
