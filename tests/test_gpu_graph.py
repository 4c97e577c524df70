"""The layer inside a captured HIP graph: a three-layer step (RMSNorm +
residual between layers, as two calls per layer or fused into the layer's
call) captured once with torch.cuda.graph and replayed
several times, with eager work and synchronisations between the replays;
every replay must equal the eager step bit for bit (the kernels are
deterministic).  Both regimes: a decode batch (bandwidth kernels) and a
GEMM-path batch."""

import pytest
import torch

import quantized_expert_ffn_top_amd as Q
import synth
from tests._helpers import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused_residual"])
@pytest.mark.parametrize("T", [3, 40])
def test_stack_step_graph_replay_matches_eager(T, fused):
    sh, nl, seed = synth.REAL, 3, 17
    layers = [synth.real_layer(sh, seed, l, zipf_s=1.0, device=dev()) for l in range(nl)]
    wts = [Q.weights(L.experts, sh.expert_bytes, L.router_w, L.router_b, L.shared_ug,
                     L.shared_down) for L in layers]
    gammas = [synth.norm_gain(sh.hidden, seed, l).to(dev()) for l in range(nl)]
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    ws = Q.workspace(d, T, dev())
    x0 = synth.tokens_bf16(T, sh.hidden, seed).float().to(dev())
    h = torch.empty_like(x0)
    normed = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=dev())
    normed2 = torch.empty_like(normed)
    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())

    def step():
        h.copy_(x0)
        Q.moe_rmsnorm_residual(h, None, gammas[0], 1e-6, normed)
        nin, nout = normed, normed2
        for l in range(nl):
            last = l + 1 == nl
            if fused:
                Q.moe_layer_forward_residual(d, wts[l], nin, h, ws,
                                             gamma=None if last else gammas[l + 1], eps=1e-6,
                                             normed=None if last else nout)
                nin, nout = nout, nin
            else:
                Q.moe_layer_forward(d, wts[l], normed, y, ws)
                Q.moe_rmsnorm_residual(h, y, None if last else gammas[l + 1], 1e-6,
                                       None if last else normed)

    step()
    torch.cuda.synchronize()
    ref = h.clone()
    assert bool(torch.isfinite(ref).all())

    stream = torch.cuda.current_stream(dev())
    side = torch.cuda.Stream(dev())
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        h.fill_(float("nan"))
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, ref), "replay %d differs from the eager step" % i
        step()                                   # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(h, ref)
