// C ABI of libmoe.so (declared in include/moe.h): argument checks, workspace
// carving and the enqueue order of the kernels.  No call allocates device
// memory, frees it, or synchronises the host.
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "moe_kernels.hpp"

using namespace moe;

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

// ---- device check (cached per device id)
std::mutex g_dev_mu;
int g_dev_ok[64];   // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[64];  // compute units of each checked device

// Checks that the current device is gfx950; `n_cu` (optional) receives its
// compute-unit count, the grid of the persistent kernels.
moe_status check_device(int* n_cu = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device id out of range");
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess)
            return fail(MOE_ERR_HIP, "hipGetDeviceProperties failed");
        g_dev_ok[dev] = (std::string(p.gcnArchName).rfind("gfx950", 0) == 0) ? 1 : 2;
        g_dev_cus[dev] = p.multiProcessorCount > 0 ? p.multiProcessorCount : 1;
    }
    if (g_dev_ok[dev] != 1) return fail(MOE_ERR_DEVICE, "current device is not gfx950");
    if (n_cu) *n_cu = g_dev_cus[dev];
    return MOE_OK;
}

moe_status launched(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return MOE_OK;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int kMaxT = 1 << 18;

size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }

// ---- workspace layout for one (shape, T)
struct Ws {
    size_t x16, shp, logits, ids, w, offsets, perm, inv, tiles, ntiles, a16, a_sh, y_perm,
        y_sh, hist, total;
    int max_tiles;
};

// The layer runs the bandwidth path for T <= kDecMaxT tokens when its experts
// are Q3S-256 up|gate and NL4-32 down and its up|gate kernel can stage two
// items of the hidden size; otherwise the grouped GEMMs.
bool std_formats(const moe_layer_desc* d) {
    return d->upgate_fmt == MOE_FMT_Q3S256 && d->down_fmt == MOE_FMT_NL4_32;
}
bool dec_path(int T, int H, int E, bool std_fmt) {
    return std_fmt && T <= kDecMaxT && upgate_dec_supported(H, T, E);
}

// tiles of the expert kernels: one per active expert (bandwidth path) or per
// kGemmBM rows of an expert (grouped GEMM)
int max_tiles_for(int T, int E, int k, bool dec) {
    const int n = T * k;
    if (dec) return n < E ? n : E;
    return (n + kGemmBM - 1) / kGemmBM + (n < E ? n : E);
}

Ws layout(int H, int I, int E, int k, int Is, int T, bool std_fmt) {
    Ws s{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += a256(bytes);
        return o;
    };
    const size_t n = (size_t)T * k;
    const int tdec = T < kDecMaxT ? T : kDecMaxT;
    const bool dec = dec_path(T, H, E, std_fmt);
    s.max_tiles = max_tiles_for(T, E, k, dec);
    s.x16 = take((size_t)T * H * 2);
    s.shp = take((size_t)(H / kShKChunk) * tdec * 2 * (Is > 0 ? Is : 1) * 4);
    s.logits = take((size_t)(dec ? kDecLogitParts : 1) * T * E * 4);
    s.ids = take(n * 4);
    s.w = take(n * 4);
    s.offsets = take((size_t)(E + 1) * 4);
    s.perm = take(n * 4);
    s.inv = take(n * 4);
    const int gemm_tiles = (int)((n + kGemmBM - 1) / kGemmBM) + (n < (size_t)E ? (int)n : E);
    s.tiles = take((size_t)(s.max_tiles > gemm_tiles ? s.max_tiles : gemm_tiles) * 12);
    s.ntiles = take(8);                     // tile count, then the down GEMM's fp16 range flag
    s.a16 = take(n * I * 2);
    s.a_sh = take((size_t)T * (Is > 0 ? Is : 1) * 2);
    s.y_perm = take(n * H * 4);
    s.y_sh = take((size_t)T * H * 4);
    s.hist = take((size_t)((T + 63) / 64) * E * 4);
    s.total = off;
    return s;
}

moe_status check_desc(const moe_layer_desc* d) {
    if (!d) return fail(MOE_ERR_NULL, "desc is NULL");
    if (d->hidden < 256 || d->hidden > 8192 || d->hidden % 256)
        return fail(MOE_ERR_SHAPE, "hidden must be a multiple of 256 in [256, 8192]");
    if (d->inter < 64 || d->inter > 4096 || d->inter % 64)
        return fail(MOE_ERR_SHAPE, "inter must be a multiple of 64 in [64, 4096]");
    if (d->n_experts < 1 || d->n_experts > 1024)
        return fail(MOE_ERR_SHAPE, "n_experts must be in [1, 1024]");
    if (d->top_k < 1 || d->top_k > 32 || d->top_k > d->n_experts)
        return fail(MOE_ERR_SHAPE, "top_k must be in [1, min(n_experts, 32)]");
    if (d->shared_inter < 0 || d->shared_inter > 4096 || d->shared_inter % 64)
        return fail(MOE_ERR_SHAPE, "shared_inter must be 0 or a multiple of 64 <= 4096");
    if (d->upgate_fmt != MOE_FMT_Q3S256 && d->upgate_fmt != MOE_FMT_Q2S256 &&
        d->upgate_fmt != MOE_FMT_NL4_32 && d->upgate_fmt != MOE_FMT_Q3K256 &&
        d->upgate_fmt != MOE_FMT_NL4S256)
        return fail(MOE_ERR_FORMAT, "routed up|gate must be Q3S256, Q2S256, NL4_32, Q3K256 or NL4S256");
    if (d->down_fmt != MOE_FMT_NL4_32 && d->down_fmt != MOE_FMT_Q2_32)
        return fail(MOE_ERR_FORMAT, "routed down must be NL4_32 or Q2_32");
    return MOE_OK;
}

// bytes of the up|gate matrix of a record (the down matrix follows it)
int64_t upgate_bytes(const moe_layer_desc* d) {
    return fmt_matrix_bytes(d->upgate_fmt, 2 * d->inter, d->hidden);
}
int64_t record_bytes(const moe_layer_desc* d) {
    return upgate_bytes(d) + fmt_matrix_bytes(d->down_fmt, d->hidden, d->inter);
}

moe_status check_weights(const moe_layer_desc* d, const moe_layer_weights* w, bool need_router,
                         bool need_shared) {
    if (!w) return fail(MOE_ERR_NULL, "weights is NULL");
    if (!w->experts) return fail(MOE_ERR_NULL, "weights->experts is NULL");
    if (!al16(w->experts) || (w->expert_stride & 15))
        return fail(MOE_ERR_ALIGN, "experts and expert_stride must be 16-byte aligned");
    if (w->expert_stride < record_bytes(d))
        return fail(MOE_ERR_SHAPE, "expert_stride is smaller than one expert record");
    if (need_router) {
        if (!w->router_w) return fail(MOE_ERR_NULL, "router_w is NULL and no logits given");
        if (!al16(w->router_w)) return fail(MOE_ERR_ALIGN, "router_w must be 16-byte aligned");
        if (w->router_b && !al4(w->router_b)) return fail(MOE_ERR_ALIGN, "router_b misaligned");
    }
    if (need_shared) {
        if (!w->shared_upgate || !w->shared_down)
            return fail(MOE_ERR_NULL, "shared_inter > 0 but shared weights are NULL");
        if (!al16(w->shared_upgate) || !al16(w->shared_down))
            return fail(MOE_ERR_ALIGN, "shared weights must be 16-byte aligned");
    }
    return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

size_t permute_ws_bytes(int T, int k, int E) {
    if (T <= kDecMaxT) return 0;
    const int mt = max_tiles_for(T, E, k, false);
    return a256((size_t)((T + 63) / 64) * E * 4) + a256((size_t)mt * 12) + 256;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "null pointer";
        case MOE_ERR_SHAPE: return "unsupported shape";
        case MOE_ERR_FORMAT: return "unsupported weight format";
        case MOE_ERR_ALIGN: return "misaligned pointer or stride";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_DEVICE: return "device is not gfx950";
        case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_size(const moe_layer_desc* desc, int32_t T_max) {
    if (check_desc(desc) != MOE_OK || T_max < 1 || T_max > kMaxT) return 0;
    // The bandwidth path (T <= kDecMaxT) lays the workspace out differently
    // from the grouped GEMMs (router partial planes, one tile per expert), so
    // the layout size is not monotone in T: take the largest over every
    // batch a call may bring.
    size_t m = 0;
    auto at_T = [&](int T) {
        const size_t s = layout(desc->hidden, desc->inter, desc->n_experts, desc->top_k,
                                desc->shared_inter, T, std_formats(desc)).total;
        if (s > m) m = s;
    };
    for (int T = 1; T <= T_max && T <= kDecMaxT; ++T) at_T(T);
    at_T(T_max);
    return m;
}

moe_status moe_router_logits(const uint16_t* x, int32_t T, int32_t H, int32_t E,
                             const uint16_t* w_r, const float* b, float* logits, void* ws,
                             size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (!x || !w_r || !logits) return fail(MOE_ERR_NULL, "x, w_r and logits must be non-NULL");
    if (T < 1 || T > kMaxT || H < 256 || H > 8192 || H % 256 || E < 1 || E > 1024)
        return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18, H % 256 == 0 in [256, 8192], 1 <= E <= 1024");
    if (!al16(x) || !al16(w_r) || !al4(logits) || (b && !al4(b)))
        return fail(MOE_ERR_ALIGN, "x and w_r must be 16-byte aligned");
    (void)ws;
    (void)ws_bytes;
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (T <= kDecMaxT) {
        launch_dec_stage1(x, T, H, E, w_r, b, logits, nullptr, 0, nullptr, nullptr, 1, st);
    } else {
        launch_dense_router_shared(x, T, H, E, w_r, b, logits, nullptr, 0, nullptr, st);
    }
    return launched("moe_router_logits");
}

moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_w, void* stream) {
    g_last_error.clear();
    if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_NULL, "null argument");
    if (T < 1 || T > kMaxT || E < 1 || E > 1024 || k < 1 || k > 32 || k > E)
        return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18, 1 <= E <= 1024, 1 <= k <= min(E, 32)");
    if (!al4(logits) || !al4(topk_ids) || !al4(topk_w)) return fail(MOE_ERR_ALIGN, "misaligned");
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    launch_topk(logits, T, E, k, topk_ids, topk_w, nullptr, nullptr, nullptr, nullptr, 0, (hipStream_t)stream);
    return launched("moe_route");
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                       int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (!topk_ids || !offsets || !perm || !inv_perm) return fail(MOE_ERR_NULL, "null argument");
    if (T < 1 || T > kMaxT || E < 1 || E > 1024 || k < 1 || k > 32 || k > E)
        return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18, 1 <= E <= 1024, 1 <= k <= min(E, 32)");
    if (!al4(topk_ids) || !al4(offsets) || !al4(perm) || !al4(inv_perm))
        return fail(MOE_ERR_ALIGN, "misaligned");
    const size_t need = permute_ws_bytes(T, k, E);
    if (need && (!ws || ws_bytes < need)) return fail(MOE_ERR_WORKSPACE, "workspace too small");
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    if (T <= kDecMaxT) {
        launch_permute_small(topk_ids, T, E, k, offsets, perm, inv_perm, st);
    } else {
        const size_t hist_b = a256((size_t)((T + 63) / 64) * E * 4);
        const int mt = max_tiles_for(T, E, k, false);
        int32_t* hist = at<int32_t>(ws, 0);
        int32_t* tiles = at<int32_t>(ws, hist_b);
        int32_t* nt = at<int32_t>(ws, hist_b + a256((size_t)mt * 12));
        launch_permute_large(topk_ids, T, k, E, kGemmBM, hist, offsets, perm, inv_perm, tiles, nt, st);
    }
    return launched("moe_permute");
}

moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_layer_weights* wts,
                          const uint16_t* x, int32_t T, const int32_t* offsets,
                          const int32_t* perm, float* y_perm, float* shared_y, void* ws,
                          size_t ws_bytes, void* stream) {
    g_last_error.clear();
    moe_status s = check_desc(desc);
    if (s != MOE_OK) return s;
    const bool do_sh = shared_y && desc->shared_inter > 0;
    s = check_weights(desc, wts, false, do_sh);
    if (s != MOE_OK) return s;
    if (!x || !offsets || !perm || !y_perm) return fail(MOE_ERR_NULL, "null argument");
    if (T < 1 || T > kMaxT) return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18");
    if (!al16(x) || !al4(offsets) || !al4(perm) || !al4(y_perm) || (shared_y && !al4(shared_y)))
        return fail(MOE_ERR_ALIGN, "x must be 16-byte aligned");
    const int H = desc->hidden, I = desc->inter, E = desc->n_experts, k = desc->top_k,
              Is = desc->shared_inter;
    const Ws L = layout(H, I, E, k, Is, T, std_formats(desc));
    if (!ws || ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace too small");
    const int n = T * k;
    const int gemm_tiles = (n + kGemmBM - 1) / kGemmBM + (n < E ? n : E);
    if ((size_t)gemm_tiles * 12 > L.ntiles - L.tiles)
        return fail(MOE_ERR_WORKSPACE, "workspace too small for the tile list");
    int n_cu = 0;
    s = check_device(&n_cu);
    if (s != MOE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* ex = (const uint8_t*)wts->experts;
    const uint16_t* sug = do_sh ? (const uint16_t*)wts->shared_upgate : nullptr;
    const uint16_t* sdn = do_sh ? (const uint16_t*)wts->shared_down : nullptr;
    int32_t* tiles = at<int32_t>(ws, L.tiles);
    int32_t* nt = at<int32_t>(ws, L.ntiles);
    uint16_t* x16 = at<uint16_t>(ws, L.x16);
    uint16_t* a16 = at<uint16_t>(ws, L.a16);
    uint16_t* ash = at<uint16_t>(ws, L.a_sh);
    if (dec_path(T, H, E, std_formats(desc))) {
        // the bandwidth kernels, with the routing given: one tile per active
        // expert, the shared up|gate partials and the fp16 copy of x in
        // stage 1, the routed and shared down rows in the down kernel
        float* shp = at<float>(ws, L.shp);
        launch_build_tiles(offsets, E, n, tiles, nt, st);
        launch_dec_stage1(x, T, H, E, nullptr, nullptr, nullptr, sug, Is, shp, x16, kDecLogitParts, st);
        const RouteOut ro{nullptr, nullptr, nullptr, nullptr, nullptr, const_cast<int32_t*>(perm),
                          nullptr, tiles, nt};
        launch_upgate_dec(ex, wts->expert_stride, nullptr, 1, nullptr, E, k, L.max_tiles, x16, T, H, I, a16,
                          do_sh ? shp : nullptr, Is, ash, ro, n_cu, st);
        launch_down_dec(ex, wts->expert_stride, tiles, nt, L.max_tiles, a16, T, H, I, k, sdn, ash, Is,
                        y_perm, do_sh ? shared_y : nullptr, n_cu, st);
        return launched("moe_expert_ffn");
    }
    launch_to_f16(x, x16, (int64_t)T * H, st);
    launch_build_tiles(offsets, E, kGemmBM, tiles, nt, st);
    if (do_sh) {
        launch_dense_router_shared(x, T, H, E, nullptr, nullptr, nullptr, sug, Is, ash, st);
        launch_dense_shared_down(ash, T, Is, sdn, H, shared_y, st);
    }
    launch_gemm_upgate(ex, wts->expert_stride, tiles, nt, gemm_tiles, perm, k, x16, H, I, a16,
                       desc->upgate_fmt, st);
    launch_gemm_down(ex, wts->expert_stride, tiles, nt, gemm_tiles, a16, H, I, upgate_bytes(desc),
                     desc->down_fmt, y_perm, nullptr, nullptr, nullptr, st);
    return launched("moe_expert_ffn");
}

moe_status moe_combine(const float* y_perm, const int32_t* inv_perm, const float* topk_w,
                       int32_t T, int32_t k, int32_t H, const float* shared_y, float* y,
                       void* stream) {
    g_last_error.clear();
    if (!y_perm || !inv_perm || !topk_w || !y) return fail(MOE_ERR_NULL, "null argument");
    if (T < 1 || T > kMaxT || k < 1 || k > 32 || H < 4 || H % 4)
        return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18, 1 <= k <= 32, H % 4 == 0");
    if (!al16(y_perm) || !al16(y) || (shared_y && !al16(shared_y)) || !al4(inv_perm) || !al4(topk_w))
        return fail(MOE_ERR_ALIGN, "y_perm, shared_y and y must be 16-byte aligned");
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    launch_combine(y_perm, nullptr, inv_perm, topk_w, T, k, H, shared_y, y, (hipStream_t)stream);
    return launched("moe_combine");
}

}  // extern "C"

namespace {

// Records events[i] after the i-th kernel of a layer call (events[0] before
// the first), as long as there are events left.
struct Marks {
    void* const* ev;
    int n;
    int used;
    hipStream_t st;
    void mark() {
        if (ev && used < n) (void)hipEventRecord((hipEvent_t)ev[used], st);
        ++used;
    }
};

// The residual add and the next RMSNorm fused into the layer's combine.
struct Fuse {
    float* h;
    const float* gamma;
    float eps;
    uint16_t* normed;
};

moe_status layer_forward_impl(const moe_layer_desc* desc, const moe_layer_weights* wts,
                              const uint16_t* x, int32_t T, const float* logits_or_null, float* y,
                              int32_t* topk_ids_out, float* topk_w_out, void* ws,
                              size_t ws_bytes, void* stream, Marks* mk, const Fuse* fz = nullptr) {
    g_last_error.clear();
    moe_status s = check_desc(desc);
    if (s != MOE_OK) return s;
    const bool has_sh = desc->shared_inter > 0;
    s = check_weights(desc, wts, logits_or_null == nullptr, has_sh);
    if (s != MOE_OK) return s;
    if (!x || (!y && !fz)) return fail(MOE_ERR_NULL, "x and y must be non-NULL");
    if (T < 1 || T > kMaxT) return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18");
    if (!al16(x) || (y && !al16(y)) || (logits_or_null && !al4(logits_or_null)) ||
        (topk_ids_out && !al4(topk_ids_out)) || (topk_w_out && !al4(topk_w_out)))
        return fail(MOE_ERR_ALIGN, "x and y must be 16-byte aligned");
    const int H = desc->hidden, I = desc->inter, E = desc->n_experts, k = desc->top_k,
              Is = desc->shared_inter;
    const bool std_fmt = std_formats(desc);
    const Ws L = layout(H, I, E, k, Is, T, std_fmt);
    if (!ws || ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace too small");
    int n_cu = 0;
    s = check_device(&n_cu);
    if (s != MOE_OK) return s;

    hipStream_t st = (hipStream_t)stream;
    mk->st = st;
    const uint8_t* ex = (const uint8_t*)wts->experts;
    const uint16_t* sug = has_sh ? (const uint16_t*)wts->shared_upgate : nullptr;
    const uint16_t* sdn = has_sh ? (const uint16_t*)wts->shared_down : nullptr;
    uint16_t* x16 = at<uint16_t>(ws, L.x16);
    float* shp = at<float>(ws, L.shp);
    float* lg = at<float>(ws, L.logits);
    int32_t* ids = at<int32_t>(ws, L.ids);
    float* wv = at<float>(ws, L.w);
    int32_t* offs = at<int32_t>(ws, L.offsets);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    int32_t* tiles = at<int32_t>(ws, L.tiles);
    int32_t* nt = at<int32_t>(ws, L.ntiles);
    uint16_t* a16 = at<uint16_t>(ws, L.a16);
    uint16_t* ash = at<uint16_t>(ws, L.a_sh);
    float* yp = at<float>(ws, L.y_perm);
    float* ysh = at<float>(ws, L.y_sh);
    int32_t* hist = at<int32_t>(ws, L.hist);

    mk->mark();
    if (dec_path(T, H, E, std_fmt)) {
        // stage 1 always runs: router logits (none given), shared up|gate
        // partials (shared expert present) and the fp16 copy of x
        launch_dec_stage1(x, T, H, E, logits_or_null ? nullptr : (const uint16_t*)wts->router_w,
                          wts->router_b, lg, sug, Is, shp, x16, kDecLogitParts, st);
        mk->mark();
        // routing runs inside the up|gate kernel (its block 0 writes it out)
        const RouteOut ro{ids, wv, topk_ids_out, topk_w_out, offs, perm, inv, tiles, nt};
        // given logits are used as they are; the router's are kDecLogitParts
        // partial planes, summed with the bias by the routing
        launch_upgate_dec(ex, wts->expert_stride, logits_or_null ? logits_or_null : lg,
                          logits_or_null ? 1 : kDecLogitParts,
                          (logits_or_null || kDecLogitParts == 1) ? nullptr : wts->router_b, E, k,
                          L.max_tiles, x16, T, H, I, a16, has_sh ? shp : nullptr, Is, ash, ro,
                          n_cu, st);
        mk->mark();
        launch_down_dec(ex, wts->expert_stride, tiles, nt, L.max_tiles, a16, T, H, I, k, sdn, ash,
                        Is, yp, ysh, n_cu, st);
        mk->mark();
    } else {
        // router logits (none given) and the shared expert's SwiGLU
        // activations: one launch, both read only x
        const float* L_use = logits_or_null ? logits_or_null : lg;
        if (!logits_or_null || has_sh) {
            launch_dense_router_shared(x, T, H, E,
                                       logits_or_null ? nullptr : (const uint16_t*)wts->router_w,
                                       wts->router_b, lg, sug, Is, ash, st);
            mk->mark();
        }
        launch_topk(L_use, T, E, k, ids, wv, topk_ids_out, topk_w_out, x, x16, H, st);
        mk->mark();
        launch_permute_large(ids, T, k, E, kGemmBM, hist, offs, perm, inv, tiles, nt, st);
        mk->mark();
        if (has_sh) {
            launch_dense_shared_down(ash, T, Is, sdn, H, ysh, st);
            mk->mark();
        }
        launch_gemm_upgate(ex, wts->expert_stride, tiles, nt, L.max_tiles, perm, k, x16, H, I, a16,
                           desc->upgate_fmt, st);
        mk->mark();
        // the unweighted rows go through memory as fp16 (half the bytes) unless
        // the down GEMM's range check finds values fp16 would not hold well;
        // then the second launch writes them in fp32 and the combine reads
        // those (it does nothing otherwise)
        int* range_flag = nt + 1;
        launch_gemm_down(ex, wts->expert_stride, tiles, nt, L.max_tiles, a16, H, I,
                         upgate_bytes(desc), desc->down_fmt, yp, reinterpret_cast<uint16_t*>(yp),
                         range_flag, nullptr, st);
        mk->mark();
        launch_gemm_down(ex, wts->expert_stride, tiles, nt, L.max_tiles, a16, H, I,
                         upgate_bytes(desc), desc->down_fmt, yp, nullptr, nullptr, range_flag, st);
        mk->mark();
        if (fz)
            launch_combine_norm(yp, range_flag, inv, wv, T, k, H, has_sh ? ysh : nullptr, fz->h,
                                fz->gamma, fz->eps, fz->normed, st);
        else
            launch_combine(yp, range_flag, inv, wv, T, k, H, has_sh ? ysh : nullptr, y, st);
        mk->mark();
        return launched("moe_layer_forward");
    }
    if (fz)
        launch_combine_norm(yp, nullptr, inv, wv, T, k, H, has_sh ? ysh : nullptr, fz->h, fz->gamma,
                            fz->eps, fz->normed, st);
    else
        launch_combine(yp, nullptr, inv, wv, T, k, H, has_sh ? ysh : nullptr, y, st);
    mk->mark();
    return launched("moe_layer_forward");
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* wts,
                             const uint16_t* x, int32_t T, const float* logits_or_null, float* y,
                             int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                             void* stream) {
    Marks mk{nullptr, 0, 0, nullptr};
    return layer_forward_impl(desc, wts, x, T, logits_or_null, y, topk_ids_out, topk_w_out, ws,
                              ws_bytes, stream, &mk);
}

moe_status moe_layer_forward_residual(const moe_layer_desc* desc, const moe_layer_weights* wts,
                                      const uint16_t* x, int32_t T, const float* logits_or_null,
                                      float* h, const float* gamma, float eps,
                                      uint16_t* normed_bf16_out, int32_t* topk_ids_out,
                                      float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    if (!h) return fail(MOE_ERR_NULL, "h is NULL");
    if ((gamma == nullptr) != (normed_bf16_out == nullptr))
        return fail(MOE_ERR_NULL, "gamma and normed_bf16_out must both be given or both NULL");
    if (!(eps >= 0.f)) return fail(MOE_ERR_SHAPE, "eps must be >= 0");
    if (!al16(h) || (gamma && !al16(gamma)) || ((uintptr_t)normed_bf16_out & 7))
        return fail(MOE_ERR_ALIGN, "h and gamma must be 16-byte, normed_bf16_out 8-byte aligned");
    const Fuse fz{h, gamma, eps, normed_bf16_out};
    Marks mk{nullptr, 0, 0, nullptr};
    return layer_forward_impl(desc, wts, x, T, logits_or_null, nullptr, topk_ids_out, topk_w_out, ws,
                              ws_bytes, stream, &mk, &fz);
}

moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const moe_layer_weights* wts,
                                   const uint16_t* x, int32_t T, const float* logits_or_null,
                                   float* y, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                                   size_t ws_bytes, void* stream, void* const* events,
                                   int32_t n_events, int32_t* n_marks) {
    if (!events || n_events < 1 || !n_marks) {
        g_last_error = "events, n_events >= 1 and n_marks are required";
        return MOE_ERR_NULL;
    }
    Marks mk{events, n_events, 0, nullptr};
    moe_status s = layer_forward_impl(desc, wts, x, T, logits_or_null, y, topk_ids_out, topk_w_out,
                                      ws, ws_bytes, stream, &mk);
    *n_marks = mk.used;
    return s;
}

}  // extern "C"

namespace {

// The workspace of moe_layer_forward_noalloc: a device array of the library
// (one per GPU the library runs on, held until the process ends).  Host code
// never uses its name as an address: the address is looked up once per
// device with that device current and kept per device.
constexpr size_t kNoAllocBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocBytes];

std::mutex g_scr_mu;
void* g_scr_ptr[64];

moe_status scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device id out of range");
    std::lock_guard<std::mutex> lk(g_scr_mu);
    if (!g_scr_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scr_ptr[dev] = p;
    }
    *out = g_scr_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const moe_layer_weights* wts,
                                     const uint16_t* x, int32_t T, const float* logits_or_null,
                                     float* y, int32_t* topk_ids_out, float* topk_w_out,
                                     void* stream) {
    g_last_error.clear();
    moe_status s = check_desc(desc);
    if (s != MOE_OK) return s;
    if (T < 1 || T > kMaxT) return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18");
    const size_t need = moe_workspace_size(desc, T);
    if (need > kNoAllocBytes)
        return fail(MOE_ERR_WORKSPACE, "this layer needs " + std::to_string(need) +
                                            " bytes of workspace at T = " + std::to_string(T) +
                                            "; the library's array holds " +
                                            std::to_string(kNoAllocBytes));
    s = check_device();
    if (s != MOE_OK) return s;
    void* ws = nullptr;
    s = scratch_address(&ws);
    if (s != MOE_OK) return s;
    Marks mk{nullptr, 0, 0, nullptr};
    return layer_forward_impl(desc, wts, x, T, logits_or_null, y, topk_ids_out, topk_w_out, ws,
                              kNoAllocBytes, stream, &mk);
}

moe_status moe_dequantize(int32_t fmt, const void* blocks, int64_t n_weights, float* out,
                          void* stream) {
    g_last_error.clear();
    if (!blocks || !out) return fail(MOE_ERR_NULL, "null argument");
    if (fmt != MOE_FMT_Q3S256 && fmt != MOE_FMT_NL4_32 && fmt != MOE_FMT_Q2S256 &&
        fmt != MOE_FMT_Q2_32 && fmt != MOE_FMT_Q3K256 && fmt != MOE_FMT_NL4S256)
        return fail(MOE_ERR_FORMAT, "moe_dequantize supports Q3S256, NL4_32, Q2S256, Q2_32, Q3K256, NL4S256");
    const int64_t unit = fmt_block_weights(fmt);
    if (n_weights < unit || n_weights % unit)
        return fail(MOE_ERR_SHAPE, "n_weights must be a positive multiple of the block size");
    if (!al16(blocks) || !al4(out)) return fail(MOE_ERR_ALIGN, "blocks must be 16-byte aligned");
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    launch_dequant(fmt, blocks, n_weights, out, (hipStream_t)stream);
    return launched("moe_dequantize");
}

moe_status moe_dequantize_path(int32_t fmt, int32_t path, const void* blocks, int64_t n_weights,
                               float* out, void* stream) {
    g_last_error.clear();
    if (!blocks || !out) return fail(MOE_ERR_NULL, "null argument");
    if (path != MOE_PATH_BANDWIDTH && path != MOE_PATH_GEMM)
        return fail(MOE_ERR_FORMAT, "path must be MOE_PATH_BANDWIDTH or MOE_PATH_GEMM");
    if (path == MOE_PATH_BANDWIDTH && fmt != MOE_FMT_Q3S256 && fmt != MOE_FMT_NL4_32)
        return fail(MOE_ERR_FORMAT, "the bandwidth path decodes Q3S256 and NL4_32");
    if (fmt != MOE_FMT_Q3S256 && fmt != MOE_FMT_NL4_32 && fmt != MOE_FMT_Q2S256 && fmt != MOE_FMT_Q2_32 &&
        fmt != MOE_FMT_Q3K256 && fmt != MOE_FMT_NL4S256)
        return fail(MOE_ERR_FORMAT, "moe_dequantize_path supports the six quantized formats");
    const int64_t unit = fmt_block_weights(fmt);
    if (n_weights < unit || n_weights % unit)
        return fail(MOE_ERR_SHAPE, "n_weights must be a positive multiple of the block size");
    if (!al16(blocks) || !al4(out)) return fail(MOE_ERR_ALIGN, "blocks must be 16-byte aligned");
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    launch_dequant_path(fmt, path, blocks, n_weights, out, (hipStream_t)stream);
    return launched("moe_dequantize_path");
}

moe_status moe_rmsnorm_residual(float* h, const float* delta, const float* gamma, float eps,
                                int32_t T, int32_t H, uint16_t* normed_bf16_out, void* stream) {
    g_last_error.clear();
    if (!h) return fail(MOE_ERR_NULL, "h is NULL");
    if ((gamma == nullptr) != (normed_bf16_out == nullptr))
        return fail(MOE_ERR_NULL, "gamma and normed_bf16_out must both be given or both NULL");
    if (T < 1 || T > kMaxT || H < 1 || H > 65536)
        return fail(MOE_ERR_SHAPE, "need 1 <= T <= 2^18, 1 <= H <= 65536");
    if (!(eps >= 0.f)) return fail(MOE_ERR_SHAPE, "eps must be >= 0");
    if (!al4(h) || (delta && !al4(delta)) || (gamma && !al4(gamma)))
        return fail(MOE_ERR_ALIGN, "misaligned");
    moe_status s = check_device();
    if (s != MOE_OK) return s;
    launch_rmsnorm(h, delta, gamma, eps, T, H, normed_bf16_out, (hipStream_t)stream);
    return launched("moe_rmsnorm_residual");
}

}  // extern "C"
