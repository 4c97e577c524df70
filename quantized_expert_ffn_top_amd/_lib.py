"""ctypes binding of libmoe.so (C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors used as device memory; the stream is
torch's current stream on the tensors' device.  A missing library raises at
load time -- there is no fallback path.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_FMT_BF16 = 1
MOE_FMT_Q3S256 = 2
MOE_FMT_NL4_32 = 3
MOE_FMT_Q2S256 = 4
MOE_FMT_Q2_32 = 5
MOE_FMT_Q3K256 = 6
MOE_FMT_NL4S256 = 7
MOE_PATH_BANDWIDTH = 0
MOE_PATH_GEMM = 1

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_FORMAT",
          4: "MOE_ERR_ALIGN", 5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_DEVICE", 7: "MOE_ERR_HIP"}

EXPORTS = ("moe_workspace_size", "moe_router_logits", "moe_route", "moe_permute",
           "moe_expert_ffn", "moe_combine", "moe_layer_forward", "moe_layer_forward_residual",
           "moe_layer_forward_timed",
           "moe_layer_forward_noalloc", "moe_dequantize", "moe_dequantize_path", "moe_rmsnorm_residual",
           "moe_status_string", "moe_last_error")


class MoeError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), detail))


class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("upgate_fmt", ctypes.c_int32),
                ("down_fmt", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("experts", ctypes.c_void_p), ("expert_stride", ctypes.c_int64),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("shared_upgate", ctypes.c_void_p), ("shared_down", ctypes.c_void_p)]


_lib = None


def load():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe.so is not built (run __graft_entry__.build() or "
                           "python -m quantized_expert_ffn_top_amd._build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                          ctypes.c_float)
    sig = {
        "moe_workspace_size": (SZ, [ctypes.POINTER(LayerDesc), I32]),
        "moe_router_logits": (I32, [P, I32, I32, I32, P, P, P, P, SZ, P]),
        "moe_route": (I32, [P, I32, I32, I32, P, P, P]),
        "moe_permute": (I32, [P, I32, I32, I32, P, P, P, P, SZ, P]),
        "moe_expert_ffn": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), P, I32,
                                 P, P, P, P, P, SZ, P]),
        "moe_combine": (I32, [P, P, P, I32, I32, I32, P, P, P]),
        "moe_layer_forward": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), P,
                                    I32, P, P, P, P, P, SZ, P]),
        "moe_layer_forward_residual": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                             P, I32, P, P, P, F, P, P, P, P, SZ, P]),
        "moe_layer_forward_timed": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                          P, I32, P, P, P, P, P, SZ, P, P, I32,
                                          ctypes.POINTER(I32)]),
        "moe_layer_forward_noalloc": (I32, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                            P, I32, P, P, P, P, P]),
        "moe_dequantize": (I32, [I32, P, I64, P, P]),
        "moe_dequantize_path": (I32, [I32, I32, P, I64, P, P]),
        "moe_rmsnorm_residual": (I32, [P, P, P, F, I32, I32, P, P]),
        "moe_status_string": (ctypes.c_char_p, [I32]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(*tensors):
    for t in tensors:
        if t is not None and t.is_cuda:
            return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def _check(status, where):
    if status != 0:
        raise MoeError(status, where, load().moe_last_error().decode())


def _u16(t):
    """bf16 / fp16 tensors are passed as their 16-bit patterns."""
    return t


def desc(hidden, inter, n_experts, top_k, shared_inter=0, upgate_fmt=MOE_FMT_Q3S256,
         down_fmt=MOE_FMT_NL4_32):
    return LayerDesc(hidden, inter, n_experts, top_k, shared_inter, upgate_fmt, down_fmt)


def weights(experts, expert_stride, router_w=None, router_b=None, shared_upgate=None,
            shared_down=None):
    """The device pointers of a layer's weights.  The record keeps the tensors
    alive: a tensor made inside the call (a zero bias, say) would otherwise be
    freed at once and its memory handed to the next allocation while the
    record still points at it."""
    w = LayerWeights(experts.data_ptr(), expert_stride,
                     None if router_w is None else router_w.data_ptr(),
                     None if router_b is None else router_b.data_ptr(),
                     None if shared_upgate is None else shared_upgate.data_ptr(),
                     None if shared_down is None else shared_down.data_ptr())
    w._keep = (experts, router_w, router_b, shared_upgate, shared_down)
    return w


# ---------------------------------------------------------------- entry points

def moe_workspace_size(d, T_max):
    return int(load().moe_workspace_size(ctypes.byref(d), T_max))


def workspace(d, T_max, device):
    """A workspace for every batch of up to T_max tokens of layers shaped like
    d (zero-filled, so that nothing of an earlier allocation leaks in)."""
    return torch.zeros(moe_workspace_size(d, T_max), dtype=torch.uint8, device=device)


def moe_router_logits(x, w_r, b, logits, ws=None):
    T, H = x.shape
    E = w_r.shape[0]
    _check(load().moe_router_logits(_ptr(x), T, H, E, _ptr(w_r), _ptr(b), _ptr(logits), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(x)), "moe_router_logits")


def moe_route(logits, k, topk_ids, topk_w):
    T, E = logits.shape
    _check(load().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w),
                            _stream(logits)), "moe_route")


def moe_permute(topk_ids, E, offsets, perm, inv_perm, ws=None):
    T, k = topk_ids.shape
    _check(load().moe_permute(_ptr(topk_ids), T, k, E, _ptr(offsets), _ptr(perm), _ptr(inv_perm),
                              _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(topk_ids)), "moe_permute")


def moe_expert_ffn(d, w, x, offsets, perm, y_perm, shared_y, ws):
    T = x.shape[0]
    _check(load().moe_expert_ffn(ctypes.byref(d), ctypes.byref(w), _ptr(x), T, _ptr(offsets),
                                 _ptr(perm), _ptr(y_perm), _ptr(shared_y), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(x)), "moe_expert_ffn")


def moe_combine(y_perm, inv_perm, topk_w, shared_y, y):
    T, k = topk_w.shape
    H = y.shape[1]
    _check(load().moe_combine(_ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), T, k, H, _ptr(shared_y),
                              _ptr(y), _stream(y)), "moe_combine")


def moe_layer_forward(d, w, x, y, ws, logits=None, topk_ids_out=None, topk_w_out=None):
    T = x.shape[0]
    _check(load().moe_layer_forward(ctypes.byref(d), ctypes.byref(w), _ptr(x), T, _ptr(logits),
                                    _ptr(y), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(x)),
           "moe_layer_forward")


def moe_layer_forward_residual(d, w, x, h, ws, gamma=None, eps=1e-6, normed=None, logits=None,
                               topk_ids_out=None, topk_w_out=None):
    """h += layer(x) in place; normed = bf16(gamma * h / rms(h)) when gamma is given."""
    T = x.shape[0]
    _check(load().moe_layer_forward_residual(ctypes.byref(d), ctypes.byref(w), _ptr(x), T,
                                             _ptr(logits), _ptr(h), _ptr(gamma), eps, _ptr(normed),
                                             _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(x)),
           "moe_layer_forward_residual")


def moe_layer_forward_timed(d, w, x, y, ws, events, logits=None, topk_ids_out=None,
                            topk_w_out=None):
    """events: raw hipEvent_t handles (ints).  Returns the number of marks the
    call recorded (kernels + 1)."""
    T = x.shape[0]
    arr = (ctypes.c_void_p * len(events))(*events)
    n = ctypes.c_int32(0)
    _check(load().moe_layer_forward_timed(ctypes.byref(d), ctypes.byref(w), _ptr(x), T,
                                          _ptr(logits), _ptr(y), _ptr(topk_ids_out),
                                          _ptr(topk_w_out), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(x), arr,
                                          len(events), ctypes.byref(n)),
           "moe_layer_forward_timed")
    return n.value


def moe_layer_forward_noalloc(d, w, x, y, logits=None, topk_ids_out=None, topk_w_out=None):
    """The layer with the library's own device array as its workspace."""
    T = x.shape[0]
    _check(load().moe_layer_forward_noalloc(ctypes.byref(d), ctypes.byref(w), _ptr(x), T,
                                            _ptr(logits), _ptr(y), _ptr(topk_ids_out),
                                            _ptr(topk_w_out), _stream(x)),
           "moe_layer_forward_noalloc")


def moe_dequantize(fmt, blocks, n_weights, out):
    _check(load().moe_dequantize(fmt, _ptr(blocks), n_weights, _ptr(out), _stream(blocks)),
           "moe_dequantize")


def moe_dequantize_path(fmt, path, blocks, n_weights, out):
    _check(load().moe_dequantize_path(fmt, path, _ptr(blocks), n_weights, _ptr(out), _stream(blocks)),
           "moe_dequantize_path")


def moe_rmsnorm_residual(h, delta, gamma, eps, normed):
    T, H = h.shape
    _check(load().moe_rmsnorm_residual(_ptr(h), _ptr(delta), _ptr(gamma), eps, T, H, _ptr(normed),
                                       _stream(h)), "moe_rmsnorm_residual")
