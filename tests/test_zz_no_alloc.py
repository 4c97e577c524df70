"""moe_layer_forward_noalloc (the layer with the library's own device array as
its workspace) against moe_layer_forward: the same results bit for bit, on two
calls in a row whose second batch is smaller (the array keeps the first call's
contents), on both paths (bandwidth kernels at T <= 16, grouped GEMMs above),
and through the C ABI."""

import numpy as np
import pytest
import torch

import quantized_expert_ffn_top_amd as Q
import synth
from tests._helpers import dev

pytestmark = pytest.mark.gpu


def _pair(sh, seed, Ts):
    lay = synth.real_layer(sh, seed, 0, zipf_s=1.0, device=dev())
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter, sh.upgate_fmt,
               sh.down_fmt)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    ws = Q.workspace(d, max(Ts), dev())
    for T in Ts:                                        # two calls in a row, the second smaller
        x = synth.tokens_bf16(T, sh.hidden, seed + T).to(dev())
        outs = []
        for fn in ("ref", "noalloc"):
            y = torch.full((T, sh.hidden), float("nan"), dtype=torch.float32, device=dev())
            ids = torch.full((T, sh.top_k), -1, dtype=torch.int32, device=dev())
            w = torch.full((T, sh.top_k), float("nan"), dtype=torch.float32, device=dev())
            if fn == "ref":
                Q.moe_layer_forward(d, wts, x, y, ws, topk_ids_out=ids, topk_w_out=w)
            else:
                Q.moe_layer_forward_noalloc(d, wts, x, y, topk_ids_out=ids, topk_w_out=w)
            torch.cuda.synchronize()
            outs.append((y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()))
        (y0, i0, w0), (y1, i1, w1) = outs
        assert np.all(np.isfinite(y1)), "T=%d" % T
        assert np.array_equal(i0, i1), "T=%d" % T
        assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32)), "T=%d" % T
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), "T=%d" % T
        print("[no-alloc] T=%d: bit-identical to moe_layer_forward" % T, flush=True)


def test_noalloc_decode_batches():
    _pair(synth.REAL, 31, (8, 3))


def test_noalloc_gemm_batches():
    _pair(synth.REAL, 32, (64, 17))


def test_noalloc_mixed_formats_then_small_shape():
    _pair(synth.Shape(512, 128, 24, 3, 64, synth.FMT_Q2S256, synth.FMT_Q2_32), 33, (40, 5))
    _pair(synth.Shape(256, 128, 16, 2, 0), 34, (16, 1))
