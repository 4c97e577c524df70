"""moe_layer_forward_residual (the layer with the residual add and the next
RMSNorm fused into its combine) against moe_layer_forward followed by
moe_rmsnorm_residual: the same bits, on both paths, with and without the
norm, through the fp32 form of the routed rows, at H up to 8192."""

import numpy as np
import pytest
import torch

import quantized_expert_ffn_top_amd as Q
import synth
from oracle import formats as F
from tests._helpers import dev

pytestmark = pytest.mark.gpu


def _layer(sh, seed, edit=None):
    lay = synth.real_layer(sh, seed, 0, zipf_s=1.0, device=dev())
    if edit:
        for e in range(sh.n_experts):
            edit(lay.experts[e])
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter, sh.upgate_fmt,
               sh.down_fmt)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    return d, wts, lay                   # lay keeps the tensors behind wts' pointers alive


def _compare(sh, T, seed, with_norm, edit=None, xscale=1.0):
    d, wts, lay = _layer(sh, seed, edit)
    x = (synth.tokens_bf16(T, sh.hidden, seed).float() * xscale).to(torch.bfloat16).to(dev())
    h0 = torch.randn((T, sh.hidden), generator=torch.Generator().manual_seed(seed)).to(dev())
    gamma = synth.norm_gain(sh.hidden, seed, 0).to(dev()) if with_norm else None
    ws = Q.workspace(d, T, dev())
    # unfused: y, then h += y and the norm
    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    ids_a = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev())
    h_a = h0.clone()
    n_a = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=dev()) if with_norm else None
    Q.moe_layer_forward(d, wts, x, y, ws, topk_ids_out=ids_a)
    Q.moe_rmsnorm_residual(h_a, y, gamma, 1e-6, n_a)
    # fused
    ids_b = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev())
    w_b = torch.empty((T, sh.top_k), dtype=torch.float32, device=dev())
    h_b = h0.clone()
    n_b = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=dev()) if with_norm else None
    Q.moe_layer_forward_residual(d, wts, x, h_b, ws, gamma=gamma, eps=1e-6, normed=n_b,
                                 topk_ids_out=ids_b, topk_w_out=w_b)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(h_a.view(torch.int32), h_b.view(torch.int32))
    if with_norm:
        assert torch.equal(n_a.view(torch.int16), n_b.view(torch.int16))
    assert torch.isfinite(h_b).all()
    del lay
    return y


@pytest.mark.parametrize("with_norm", [True, False], ids=["norm", "residual_only"])
@pytest.mark.parametrize("T", [1, 3, 16, 17, 300])
def test_fused_residual_matches_unfused_real(T, with_norm):
    _compare(synth.REAL, T, 61, with_norm)


@pytest.mark.parametrize("T", [5, 40])
def test_fused_residual_matches_unfused_wide_and_mixed(T):
    # H = 8192 (eight float4 columns per thread) and a mixed-format layer
    _compare(synth.Shape(8192, 64, 16, 2, 64), T, 62, True)
    _compare(synth.Shape(512, 128, 24, 3, 64, F.FMT_Q2S256, F.FMT_Q2_32), T, 63, True)


def test_fused_residual_through_the_fp32_rows():
    """Routed rows beyond fp16's range: the fused combine reads the fp32 form."""
    sh = synth.Shape(512, 128, 24, 3, 64, F.FMT_Q3S256, F.FMT_NL4_32)

    def big_down(rec):
        dn = rec[sh.upgate_bytes:].view(-1, 18)
        dn[:, 0] = 0x00
        dn[:, 1] = 0x68                              # d = 2048.0
        return rec

    y = _compare(sh, 40, 64, True, edit=big_down, xscale=4.0)
    assert np.abs(y.cpu().numpy()).max() > 65504.0 * 2
