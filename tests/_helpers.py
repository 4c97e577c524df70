"""Shared helpers of the parity tests: device inputs from the seeded generators,
their oracle-side views, and the tolerance checks.

Tolerances (the layer's floating-point outputs): relative L2 error over the
whole compared tensor <= 1e-3 and max |y - y_oracle| <= 1e-2 * rms(y_oracle).
Dequantised weights, routing ids, offsets and permutations: bitwise.
"""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth                                  # noqa: E402
from oracle import formats as OF              # noqa: E402
from oracle import moe as OM                  # noqa: E402

REL_L2_TOL = 1e-3
MAX_ABS_TOL = 1e-2


def dev():
    return torch.device("cuda", 0)


def bf16_np(t):
    """float64 values of a bf16 tensor (any device)."""
    return OM.bf16_bits_to_float(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))


def assert_close(y, ref, what=""):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(y)), what + ": non-finite output"
    r = OM.rel_l2(y, ref)
    m = OM.max_abs_over_rms(y, ref)
    print("[parity] %s: rel_l2 %.3g max_abs/rms %.3g" % (what, r, m), flush=True)
    assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, "%s: rel_l2 %.3g (tol %g), max_abs/rms %.3g (tol %g)" % (
        what, r, REL_L2_TOL, m, MAX_ABS_TOL)
    return r, m


class ExpertCache:
    """Dequantised expert matrices for the oracle, from packed records."""

    def __init__(self, shape, record_fn):
        self.shape = shape
        self.record_fn = record_fn
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            rec = self.record_fn(e)
            self.cache[e] = OF.expert_matrices(rec, self.shape.hidden, self.shape.inter,
                                               self.shape.upgate_fmt, self.shape.down_fmt)
        return self.cache[e]


def tiny_inputs(seed=1, T=4):
    """Tiny workload: RTN-quantised experts (oracle quantiser) + given logits."""
    sh = synth.TINY
    ug, dn = synth.tiny_expert_weights(sh, seed)
    recs = []
    for e in range(sh.n_experts):
        r = np.concatenate([OF.quantize_q3s_matrix(ug[e].double().numpy()).reshape(-1),
                            OF.quantize_nl4_matrix(dn[e].double().numpy()).reshape(-1)])
        recs.append(r)
    recs = np.stack(recs)
    assert recs.shape[1] == sh.expert_bytes
    x = synth.tokens_bf16(T, sh.hidden, seed)
    logits = synth.unique_logits(T, sh.n_experts, seed)
    return sh, recs, x, logits


def real_shared_np(layer):
    ug = bf16_np(layer.shared_ug)
    dn = bf16_np(layer.shared_down)
    Is = layer.shape.shared_inter
    return ug[:Is], ug[Is:], dn


def ids_valid_topk(ids, logits, k, rel=1e-5):
    """Every selected logit >= every unselected logit - delta (near-tie check)."""
    L = np.asarray(logits, dtype=np.float64)
    delta = rel * np.abs(L).max()
    for t in range(L.shape[0]):
        sel = set(int(v) for v in ids[t])
        if len(sel) != k:
            return False
        lo = min(L[t, list(sel)])
        hi = max(L[t, e] for e in range(L.shape[1]) if e not in sel) if len(sel) < L.shape[1] else -np.inf
        if lo < hi - delta:
            return False
    return True
