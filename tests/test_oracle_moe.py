"""Pins of the oracle's layer math (CPU only).

The pages print no worked example of the layer, so each step is pinned by
what fixes it: brute force on tiny inputs (pure-Python loops over the scalar
decoders), closed forms (one-hot inputs, a single expert = a dense SwiGLU FFN,
k = E = a full softmax, constant-vector RMSNorm), library routines for the
special cases (torch fp64 SiLU and matmul, scipy softmax, torch's bf16
conversion), hand-derived values in tests/golden, and the invariants the
method guarantees (weights sum to 1; each token lands in exactly k slots).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax as scipy_softmax

from oracle import formats as F
from oracle import moe as M

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "codec_known_answers.json")))
LAYER_GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                         "micro_layer.json")))


# ---------------------------------------------------------------- bf16

@pytest.mark.parametrize("case", GOLD["bf16_rne"])
def test_bf16_known_values(case):
    assert M.bf16_rne(np.array([case["x"]]))[0] == case["r"]


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-39, 2000),
                        rng.normal(0, 1e37, 2000)]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(M.bf16_rne(x.astype(np.float64)), lib)
    bits = M.bf16_rne_bits(x.astype(np.float64))
    assert np.array_equal(M.bf16_bits_to_float(bits), lib)


def test_bf16_special_values():
    r = M.bf16_rne(np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38]))
    assert r[0] == 0.0 and r[2] == np.inf and r[3] == -np.inf and r[4] == np.inf
    assert np.isnan(M.bf16_rne(np.array([np.nan]))[0])


# ---------------------------------------------------------------- routing

def test_router_logits_closed_form():
    # one-hot token picks a column of W_r; bias adds per expert
    wr = np.arange(12.0).reshape(3, 4)        # E=3, H=4
    x = np.zeros((2, 4)); x[0, 1] = 1.0; x[1, 3] = 2.0
    b = np.array([10.0, 20.0, 30.0])
    L = M.router_logits(x, wr, b)
    assert L.tolist() == [[11.0, 25.0, 39.0], [16.0, 34.0, 52.0]]


def test_topk_bruteforce_and_fast_agree():
    rng = np.random.default_rng(32)
    L = rng.normal(size=(64, 40)).astype(np.float32).astype(np.float64)
    L[3, 5] = L[3, 9] = L[3].max() + 1      # planted exact tie at the top
    L[7, :] = 0.0                           # all equal -> lowest indices
    for k in (1, 2, 7, 40):
        a = M.topk_ids(L, k)
        assert np.array_equal(a, M.topk_ids_fast(L, k))
    a = M.topk_ids(L, 3)
    assert a[3, 0] == 5 and a[3, 1] == 9
    assert a[7].tolist() == [0, 1, 2]


def test_topk_invariants():
    rng = np.random.default_rng(33)
    L = rng.normal(size=(100, 64))
    k = 10
    ids = M.topk_ids(L, k)
    for t in range(L.shape[0]):
        sel = set(ids[t].tolist())
        assert len(sel) == k
        unsel = [L[t, e] for e in range(64) if e not in sel]
        assert min(L[t, list(sel)]) >= max(unsel)
        vals = L[t, ids[t]]
        assert np.all(np.diff(vals) <= 0)


def test_softmax_selected_closed_forms():
    L = np.array([[0.0, math.log(3.0), -50.0]])
    ids = np.array([[1, 0]])
    w = M.softmax_selected(L, ids)
    assert np.allclose(w, [[0.75, 0.25]], rtol=0, atol=1e-15)
    rng = np.random.default_rng(34)
    L = rng.normal(size=(20, 16))
    ids = M.topk_ids(L, 16)                  # k = E: the full softmax
    w = M.softmax_selected(L, ids)
    ref = np.take_along_axis(scipy_softmax(L, axis=1), ids, axis=1)
    assert np.allclose(w, ref, rtol=1e-13, atol=0)
    ids = M.topk_ids(L, 5)
    w = M.softmax_selected(L, ids)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_huge_bias_forces_expert():
    rng = np.random.default_rng(35)
    x = rng.normal(size=(50, 32)); wr = rng.normal(0, 0.02, size=(12, 32))
    b = np.zeros(12); b[7] = 1e6
    ids = M.topk_ids(M.router_logits(x, wr, b), 3)
    assert np.all(ids[:, 0] == 7)


# ---------------------------------------------------------------- permute

def test_permute_bruteforce_and_invariants():
    rng = np.random.default_rng(36)
    for T, E, k in [(1, 4, 2), (37, 16, 3), (200, 64, 10)]:
        L = rng.normal(size=(T, E))
        ids = M.topk_ids_fast(L, k)
        off, perm, inv = M.permute(ids, E)
        flat = ids.reshape(-1)
        ref = sorted(range(T * k), key=lambda f: (flat[f], f))
        assert perm.tolist() == ref
        assert off[0] == 0 and off[E] == T * k
        assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
        assert sorted(perm.tolist()) == list(range(T * k))
        assert np.array_equal(perm[inv], np.arange(T * k))
        for e in range(E):
            seg = perm[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
        toks = np.bincount(perm // k, minlength=T)
        assert np.all(toks == k)


# ---------------------------------------------------------------- FFN

def test_silu_and_swiglu_closed_form():
    assert M.silu(np.array([0.0]))[0] == 0.0
    assert abs(M.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    # one-hot x picks column 0: u = 2, g = -1  ->  a = bf16(silu(-1) * 2)
    wu = np.zeros((1, 4)); wu[0, 0] = 2.0
    wg = np.zeros((1, 4)); wg[0, 0] = -1.0
    x = np.array([[1.0, 0.0, 0.0, 0.0]])
    a = M.swiglu_act(x, wu, wg)
    assert a[0, 0] == LAYER_GOLD["swiglu_onehot"]["a"]


def test_single_expert_is_dense_swiglu_ffn():
    """E = k = 1 with no shared expert: y = W_down bf16(silu(W_gate x) * W_up x),
    computed here with torch fp64 (a separate library)."""
    rng = np.random.default_rng(37)
    H, I, T = 256, 64, 5
    wug = rng.normal(0, 0.02, size=(2 * I, H)); wd = rng.normal(0, 0.02, size=(H, I))
    rec = np.concatenate([F.quantize_q3s_matrix(wug).reshape(-1),
                          F.quantize_nl4_matrix(wd).reshape(-1)])
    up, gate, down = F.expert_matrices(rec, H, I)
    x = M.bf16_rne(rng.normal(size=(T, H)))
    out = M.layer_forward(x, 1, lambda e: (up, gate, down), 1,
                          logits=np.zeros((T, 1)))
    xt = torch.from_numpy(x)
    u = xt @ torch.from_numpy(up).T
    g = xt @ torch.from_numpy(gate).T
    a = (torch.nn.functional.silu(g) * u).to(torch.float32).to(torch.bfloat16).to(torch.float64)
    y = a @ torch.from_numpy(down).T
    assert np.allclose(out["w"], 1.0)
    # torch rounds fp64 -> fp32 -> bf16 (can double-round); compare loosely
    assert M.rel_l2(out["y"], y.numpy()) < 1e-3
    a64 = (torch.nn.functional.silu(g) * u).numpy()
    assert np.array_equal(out["a_perm"], M.bf16_rne(a64))
    assert np.allclose(out["y"], out["a_perm"] @ down.T, rtol=1e-14, atol=0)


def test_onehot_token_reads_weight_column():
    rng = np.random.default_rng(38)
    H, I = 256, 32
    wug = rng.normal(0, 0.02, size=(2 * I, H))
    wd = rng.normal(0, 0.02, size=(H, I))
    rec = np.concatenate([F.quantize_q3s_matrix(wug).reshape(-1),
                          F.quantize_nl4_matrix(wd).reshape(-1)])
    up, gate, down = F.expert_matrices(rec, H, I)
    x = np.zeros((1, H)); x[0, 17] = 1.0
    a = M.swiglu_act(x, up, gate)
    u = up[:, 17]; g = gate[:, 17]
    assert np.array_equal(a[0], M.bf16_rne(g / (1 + np.exp(-g)) * u))


def _scalar_layer(x, logits, k, records, H, I):
    """Pure-Python brute force of the whole tiny layer: scalar block decoders,
    triple loops, exhaustive top-k, direct combine by token (no permutation)."""
    T, E = len(x), len(logits[0])
    mats = [F.expert_matrices_scalar(r, H, I) for r in records]
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t][e], e))[:k]
        m = max(logits[t][e] for e in order)
        ex = [math.exp(logits[t][e] - m) for e in order]
        z = sum(ex)
        for j, e in enumerate(order):
            up, gate, down = mats[e]
            a = []
            for i in range(I):
                u = sum(up[i][h] * x[t][h] for h in range(H))
                g = sum(gate[i][h] * x[t][h] for h in range(H))
                a.append(g / (1.0 + math.exp(-g)) * u)
            a = M.bf16_rne(np.array(a)).tolist()
            for n in range(H):
                o = sum(down[n][i] * a[i] for i in range(I))
                y[t][n] += ex[j] / z * o
    return np.array(y)


def test_tiny_layer_bruteforce():
    """Scalar brute force vs the vectorised oracle on a 4-expert layer."""
    rng = np.random.default_rng(39)
    H, I, E, k, T = 256, 32, 4, 2, 2
    records = []
    for e in range(E):
        wug = rng.normal(0, 0.02, size=(2 * I, H)); wd = rng.normal(0, 0.02, size=(H, I))
        records.append(np.concatenate([F.quantize_q3s_matrix(wug).reshape(-1),
                                       F.quantize_nl4_matrix(wd).reshape(-1)]))
    x = M.bf16_rne(rng.normal(size=(T, H)))
    logits = rng.normal(size=(T, E))
    ref = _scalar_layer(x.tolist(), logits.tolist(), k, records, H, I)
    out = M.layer_forward(x, k, lambda e: F.expert_matrices(records[e], H, I), E,
                          logits=logits)
    assert np.allclose(out["y"], ref, rtol=1e-11, atol=1e-14)


def test_combine_weights_follow_slots():
    # two experts whose outputs are distinct constants; w from hand logits
    y_perm = np.array([[1.0, 1.0], [10.0, 10.0]])   # slot p=0 -> expert0, p=1 -> expert1
    # token 0 chose (expert1, expert0): f=0 -> p=1, f=1 -> p=0
    inv = np.array([1, 0])
    w = np.array([[0.75, 0.25]])
    y = M.combine(y_perm, inv, w, shared_y=np.array([[0.5, -0.5]]))
    assert y.tolist() == [[0.75 * 10 + 0.25 * 1 + 0.5, 0.75 * 10 + 0.25 * 1 - 0.5]]


def test_shared_expert_adds_with_weight_one():
    rng = np.random.default_rng(40)
    H, I = 256, 32
    x = M.bf16_rne(rng.normal(size=(3, H)))
    sh = (rng.normal(0, .02, (I, H)), rng.normal(0, .02, (I, H)), rng.normal(0, .02, (H, I)))
    zero = (np.zeros((I, H)), np.zeros((I, H)), np.zeros((H, I)))
    out = M.layer_forward(x, 1, lambda e: zero, 2, logits=rng.normal(size=(3, 2)), shared=sh)
    _, ys = M.ffn(x, *sh)
    assert np.array_equal(out["y"], ys)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector():
    c, eps = 3.0, 1e-6
    h = np.full((1, 8), c)
    gamma = np.array([1.0, 2.0, 0.5, -1.0, 1.0, 1.0, 1.0, 1.0])
    r = M.rmsnorm_bf16(h, gamma, eps)
    exp = M.bf16_rne(gamma * c / math.sqrt(c * c + eps))
    assert np.array_equal(r[0], exp)
    # scale invariance (up to eps): rmsnorm(5h) == rmsnorm(h) for large h
    rng = np.random.default_rng(41)
    h = rng.normal(size=(4, 64)) * 100
    assert np.array_equal(M.rmsnorm_bf16(h, np.ones(64), 0.0),
                          M.rmsnorm_bf16(4 * h, np.ones(64), 0.0))


def test_stack_step_is_residual():
    h = np.array([[1.0, 2.0]])
    out = M.stack_step(h, np.ones(2), 1e-6, lambda z: np.zeros_like(z))
    assert np.array_equal(out, h)


def test_stack_step_pre_norm_hand_values():
    """Pre-norm residual step h + f(bf16(gamma * h / sqrt(mean(h^2) + eps))) with
    a non-zero layer f(z) = 2 z + 1, on two rows worked out by hand:
      row 0: h = (2, 2, 2, 2): mean h^2 = 4, sqrt(4 + 1e-6) = 2.00000025, so
             h / rms = 0.999999875 each, which bf16 rounds to 1; times gamma
             (1, 0.5, 2, 1.5) -> z = (1, 0.5, 2, 1.5); f(z) = (3, 2, 5, 4);
             h + f(z) = (5, 4, 7, 6).
      row 1: h = (3, -3, 3, -3): rms = 3 (to 1e-7), h / rms -> (1, -1, 1, -1);
             z = (1, -0.5, 2, -1.5); f(z) = (3, 0, 5, -2); h + f(z) = (6, -3, 8, -5).
    A post-norm step norm(h + f(h)), the step h + f(h) without the norm, and
    a step that drops gamma or the bf16 rounding all give other values."""
    h = np.array([[2.0, 2.0, 2.0, 2.0], [3.0, -3.0, 3.0, -3.0]])
    gamma = np.array([1.0, 0.5, 2.0, 1.5])
    seen = []

    def f(z):
        seen.append(np.array(z))
        return 2.0 * z + 1.0

    out = M.stack_step(h, gamma, 1e-6, f)
    assert np.array_equal(seen[0], [[1.0, 0.5, 2.0, 1.5], [1.0, -0.5, 2.0, -1.5]])
    assert np.array_equal(out, [[5.0, 4.0, 7.0, 6.0], [6.0, -3.0, 8.0, -5.0]])
    # the layer input is rounded to bf16: a gain of 1 + 2^-9 vanishes, 1 + 2^-7 stays
    z = M.rmsnorm_bf16(np.array([[2.0, 2.0]]), np.array([1.0 + 2.0 ** -9, 1.0 + 2.0 ** -7]), 1e-6)
    assert np.array_equal(z, [[1.0, 1.0 + 2.0 ** -7]])


def test_metrics():
    ref = np.array([3.0, 4.0])
    assert M.rel_l2(ref, ref) == 0.0
    assert abs(M.rel_l2(np.array([3.0, 4.5]), ref) - 0.1) < 1e-15
    assert abs(M.max_abs_over_rms(np.array([3.0, 4.5]), ref) - 0.5 / math.sqrt(12.5)) < 1e-15


def test_oracle_pool_matches_serial_expert_ffn():
    """The process-pool evaluation of the routed experts (used for full-size
    parity) gives the serial oracle's y_perm (up to the BLAS summation order
    of a different thread count)."""
    import synth
    from oracle import formats as OF
    from tests import _oracle_pool
    from tests._helpers import bf16_np
    sh = synth.Shape(512, 128, 24, 3, 64, 2, 5)
    T, seed = 40, 5
    x = bf16_np(synth.tokens_bf16(T, sh.hidden, seed))
    L = np.random.default_rng(3).normal(size=(T, sh.n_experts))
    ids = M.topk_ids_fast(L, sh.top_k)
    offsets, perm, inv = M.permute(ids, sh.n_experts)
    get = lambda e: OF.expert_matrices(synth.expert_record(sh, seed, 0, e, mode="wide").numpy(),
                                       sh.hidden, sh.inter, sh.upgate_fmt, sh.down_fmt)
    _, ref = M.expert_ffn_perm(x, offsets, perm, sh.top_k, get)
    got = _oracle_pool.routed_outputs(sh, seed, 0, "wide", T, offsets, perm, sh.top_k)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
