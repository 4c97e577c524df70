"""The C ABI library on the CPU: it loads, exports every function include/moe.h
declares, and rejects bad arguments on the host before touching a GPU (every
check runs before any launch, so these need no device)."""

import ctypes
import os
import re

import pytest

import quantized_expert_ffn_top_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

# fake, 256-aligned device addresses: never dereferenced by a failing check
P = 0x10000000
P2 = 0x20000000


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = Q.load()
    decl = _declared()
    assert set(decl) == set(Q.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = Q.load()
    for s in range(8):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(5) == b"workspace missing or too small"


def test_workspace_size_monotone_and_rejects_bad_desc():
    d = Q.desc(3072, 512, 512, 10, 512)
    sizes = [Q.moe_workspace_size(d, T) for T in (1, 3, 8, 16, 17, 64, 8192)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    bad = Q.desc(3000, 512, 512, 10, 512)
    assert Q.moe_workspace_size(bad, 4) == 0
    assert Q.moe_workspace_size(d, 0) == 0


@pytest.mark.parametrize("shape", [
    (3072, 512, 512, 1, 0), (3072, 512, 512, 4, 0), (3072, 512, 512, 10, 512),
    (256, 64, 1024, 1, 0), (256, 64, 1024, 32, 0), (8192, 64, 16, 2, 64), (512, 192, 24, 3, 64)])
@pytest.mark.parametrize("T_max", [1, 5, 16, 17, 20, 64])
def test_workspace_size_bounds_every_smaller_batch(shape, T_max):
    """moe_workspace_size(desc, T_max) is enough for every T <= T_max: the
    layer call's own workspace check (a host check that runs before any
    device call) accepts that size for each T, so the call gets past it and
    stops only at the device check (no GPU here)."""
    H, I, E, k, Is = shape
    d = Q.desc(H, I, E, k, Is)
    size = Q.moe_workspace_size(d, T_max)
    assert size > 0
    rec = 2 * I * (H // 256) * 104 + H * (I // 32) * 18
    w = _w(stride=(rec + 15) // 16 * 16, shared=(P, P) if Is else (None, None))
    for T in range(1, T_max + 1):
        st = _fwd(d, w, T=T, ws_bytes=size)
        assert st not in (0, 5), (T, st)
        assert _fwd(d, w, T=T, ws_bytes=256) == 5


def _fwd(d, w, T=4, ws_bytes=1 << 30, x=P, y=P2, logits=None):
    lib = Q.load()
    return lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), x, T, logits, y, None, None,
                                 P, ws_bytes, None)


def _w(experts=P, stride=45056, router=P, shared=(None, None)):
    return Q.LayerWeights(experts, stride, router, None, shared[0], shared[1])


@pytest.mark.parametrize("case,status", [
    (dict(hidden=100), 2), (dict(hidden=256 * 33 + 0, inter=96), 2), (dict(inter=32), 2),
    (dict(n_experts=0), 2), (dict(top_k=17, n_experts=16), 2), (dict(shared_inter=100), 2),
    (dict(upgate_fmt=1), 3), (dict(down_fmt=2), 3), (dict(upgate_fmt=5), 3),
    (dict(down_fmt=4), 3), (dict(upgate_fmt=8), 3), (dict(down_fmt=0), 3),
    (dict(down_fmt=6), 3), (dict(down_fmt=7), 3),
])
def test_layer_forward_rejects_bad_shapes(case, status):
    base = dict(hidden=256, inter=128, n_experts=16, top_k=2, shared_inter=0, upgate_fmt=2,
                down_fmt=3)
    base.update(case)
    d = Q.LayerDesc(**base)
    assert _fwd(d, _w()) == status
    assert Q.load().moe_last_error()


def test_layer_forward_error_paths():
    d = Q.desc(256, 128, 16, 2, 0)
    lib = Q.load()
    assert lib.moe_layer_forward(ctypes.byref(d), None, P, 4, None, P2, None, None, P, 1 << 30,
                                 None) == 1
    assert _fwd(d, _w(experts=None)) == 1                  # null experts
    assert _fwd(d, _w(experts=P + 8)) == 4                 # misaligned experts
    assert _fwd(d, _w(stride=45056 + 8)) == 4              # misaligned stride
    assert _fwd(d, _w(stride=45056 - 16)) == 2             # stride smaller than a record
    assert _fwd(d, _w(router=None)) == 1                   # no router and no logits
    assert _fwd(d, _w(), x=P + 2) == 4                     # misaligned x
    assert _fwd(d, _w(), T=0) == 2
    assert _fwd(d, _w(), ws_bytes=16) == 5                 # workspace too small
    d2 = Q.desc(256, 128, 16, 2, 64)
    assert _fwd(d2, _w()) == 1                             # shared_inter > 0, no shared weights


def test_layer_forward_residual_error_paths():
    """The fused residual entry point checks its own arguments first, then the
    layer's (bad descriptor, weights, workspace) as moe_layer_forward does."""
    d = Q.desc(256, 128, 16, 2, 0)
    lib = Q.load()
    w = _w()

    def call(h=P2, gamma=P, eps=1e-6, normed=P2, d_=d, ws_bytes=1 << 30):
        return lib.moe_layer_forward_residual(ctypes.byref(d_), ctypes.byref(w), P, 4, None, h, gamma,
                                              eps, normed, None, None, P, ws_bytes, None)
    assert call(h=None) == 1                               # no residual stream
    assert call(normed=None) == 1                          # gamma without an output
    assert call(gamma=None) == 1                           # an output without gamma
    assert call(eps=-1.0) == 2
    assert call(h=P2 + 8) == 4                             # h not 16-byte aligned
    assert call(gamma=P + 4) == 4
    assert call(normed=P2 + 2) == 4                        # normed not 8-byte aligned
    assert call(ws_bytes=16) == 5                          # then the layer's own checks
    bad = Q.desc(250, 128, 16, 2, 0)
    assert call(d_=bad) == 2
    assert Q.load().moe_last_error()


def test_stage_error_paths():
    lib = Q.load()
    assert lib.moe_route(None, 4, 16, 2, P, P2, None) == 1
    assert lib.moe_route(P, 4, 16, 17, P, P2, None) == 2
    assert lib.moe_route(P, 4, 2000, 2, P, P2, None) == 2
    assert lib.moe_permute(P, 100, 2, 16, P, P, P, None, 0, None) == 5   # needs workspace
    assert lib.moe_combine(P, P, P, 4, 2, 254, None, P2, None) == 2      # H % 4
    assert lib.moe_combine(P + 4, P, P, 4, 2, 256, None, P2, None) == 4
    assert lib.moe_dequantize(1, P, 256, P2, None) == 3
    assert lib.moe_dequantize(2, P, 100, P2, None) == 2
    assert lib.moe_dequantize(3, P + 8, 32, P2, None) == 4
    assert lib.moe_dequantize_path(4, 0, P, 256, P2, None) == 3          # Q2S256: no kernel path
    assert lib.moe_dequantize_path(2, 2, P, 256, P2, None) == 3          # no such path
    assert lib.moe_dequantize_path(2, 1, P, 100, P2, None) == 2
    assert lib.moe_dequantize_path(3, 0, P + 8, 32, P2, None) == 4
    assert lib.moe_dequantize_path(3, 1, None, 32, P2, None) == 1
    assert lib.moe_rmsnorm_residual(P, None, P, 1e-6, 4, 256, None, None) == 1
    assert lib.moe_router_logits(P, 4, 250, 16, P, None, P2, P, 1 << 20, None) == 2
    assert lib.moe_router_logits(None, 4, 256, 16, P, None, P2, None, 0, None) == 1


def test_noalloc_rejects_batches_beyond_its_array():
    """The no-allocation entry point refuses, before any device call, a batch
    whose workspace exceeds the library's array (MOE_ERR_WORKSPACE), and takes
    the largest one that fits past that check (stopping at the device check
    here); bad descriptors are refused as by moe_layer_forward."""
    lib = Q.load()
    d = Q.desc(3072, 512, 512, 10, 512)
    limit = 64 << 20
    T_fit = max(T for T in range(1, 1024) if Q.moe_workspace_size(d, T) <= limit)
    assert T_fit >= 256
    w = _w(stride=2162688, shared=(P, P))
    call = lambda T: lib.moe_layer_forward_noalloc(ctypes.byref(d), ctypes.byref(w), P, T, None, P2,
                                                   None, None, None)
    assert call(T_fit + 1) == 5
    assert b"workspace" in lib.moe_last_error()
    assert call(T_fit) not in (0, 5)
    bad = Q.desc(3000, 512, 512, 10, 512)
    assert lib.moe_layer_forward_noalloc(ctypes.byref(bad), ctypes.byref(w), P, 4, None, P2, None,
                                         None, None) == 2


def test_binding_fails_loudly_without_library(monkeypatch):
    import quantized_expert_ffn_top_amd._lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", "/nonexistent/libmoe.so")
    with pytest.raises(RuntimeError):
        L.load()


@pytest.mark.parametrize("ug,dn", [(2, 3), (4, 5), (3, 3), (2, 5), (4, 3), (3, 5)])
def test_workspace_size_for_every_supported_format_pair(ug, dn):
    """All up|gate x down pairs of the mixed-format layers are accepted (pure
    host call); pairs that would use the bandwidth kernels need the larger
    router-partials layout at small T."""
    d = Q.desc(3072, 512, 512, 10, 512, ug, dn)
    for T in (1, 8, 17, 9536):
        assert Q.moe_workspace_size(d, T) > 0
    d_bad = Q.desc(3072, 512, 512, 10, 512, dn if dn == 5 else 1, ug if ug == 2 else 4)
    assert Q.moe_workspace_size(d_bad, 8) == 0


def test_weights_record_keeps_its_tensors_alive():
    # a tensor made inside the call (a zero router bias, as the uniform-routing
    # prefill uses) must outlive the record that points at it
    import gc
    import weakref

    import torch

    experts = torch.zeros(64, dtype=torch.uint8)
    bias = torch.zeros(16, dtype=torch.float32)
    ref = weakref.ref(bias)
    w = Q.weights(experts, 64, None, bias)
    ptr = bias.data_ptr()
    del bias
    gc.collect()
    assert ref() is not None
    assert w.router_b == ptr
    del w
    gc.collect()
    assert ref() is None
