"""GPU parity of the whole layer (moe_layer_forward) against the oracle.

Both regimes are covered on both sides of the switch (T <= 16: bandwidth
path; T >= 17: grouped-GEMM path), at the tiny shape (fully compared) and at
the real shape: decode batches fully compared, the 8192-token prefill on
sampled tokens (the oracle computes those tokens one by one) plus properties
that hold for every token (valid top-k ids, finite outputs).

Routing: with given logits the ids must match bit for bit.  With the router
on, GPU logits (fp32) and oracle logits (fp64) can order a near-tie
differently; the GPU's selection must then be a valid top-k within
1e-5 * max|L| and the oracle continues with it (none is expected).
"""

import dataclasses

import numpy as np
import pytest
import torch

import quantized_expert_ffn_top_amd as Q
import synth
from oracle import moe as OM
from tests._helpers import (ExpertCache, assert_close, bf16_np, dev, ids_valid_topk,
                            real_shared_np, tiny_inputs)

pytestmark = pytest.mark.gpu


def _run_layer(d, wts, x, logits=None):
    T = x.shape[0]
    y = torch.empty((T, d.hidden), dtype=torch.float32, device=dev())
    ids = torch.empty((T, d.top_k), dtype=torch.int32, device=dev())
    w = torch.empty((T, d.top_k), dtype=torch.float32, device=dev())
    ws = Q.workspace(d, T, dev())
    Q.moe_layer_forward(d, wts, x, y, ws, logits=logits, topk_ids_out=ids, topk_w_out=w)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T", [1, 4, 16, 17, 64, 300])
def test_tiny_layer(T):
    sh, recs, x, logits = tiny_inputs(seed=1, T=T)
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, 0)
    ex = torch.from_numpy(recs).to(dev())
    wts = Q.weights(ex, sh.expert_bytes)
    y, ids, w = _run_layer(d, wts, x.to(dev()), logits=logits.to(dev()))
    ref = OM.layer_forward(bf16_np(x), sh.top_k, ExpertCache(sh, lambda e: recs[e]),
                           sh.n_experts, logits=logits.double().numpy())
    assert np.array_equal(ids, ref["ids"])
    assert np.abs(w - ref["w"]).max() <= 1e-6
    assert_close(y, ref["y"], "tiny T=%d" % T)


def _real_case(T, seed, zipf_s=1.0, sample=None, sh=synth.REAL, mode="rtn"):
    if mode == "small":
        # the routed outputs of small-d experts are far below the shared
        # expert's: compare them alone
        sh = dataclasses.replace(sh, shared_inter=0)
    lay = synth.real_layer(sh, seed, 0, zipf_s=zipf_s, device=dev(), mode=mode)
    x = synth.tokens_bf16(T, sh.hidden, seed).to(dev())
    xscale = 1.0
    if mode == "small":
        # tokens 64 N(0, 1) (exact in bf16): the SwiGLU activations of
        # small-d experts then stay in fp16's normal range, which the
        # grouped-GEMM path's fp16 operands need
        xscale = 64.0
        x = (x.float() * xscale).to(torch.bfloat16)
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter, sh.upgate_fmt,
               sh.down_fmt)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    y, ids, w = _run_layer(d, wts, x)
    xs = bf16_np(x)
    L = OM.router_logits(xs, bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
    ref_ids = OM.topk_ids_fast(L, sh.top_k)
    assert ids_valid_topk(ids, L, sh.top_k)
    mism = np.where((np.sort(ids, axis=1) != np.sort(ref_ids, axis=1)).any(axis=1))[0]
    assert len(mism) <= max(1, T // 1000), "routing differs on %d tokens" % len(mism)
    rows = np.arange(T) if sample is None else np.asarray(sample)
    cache = ExpertCache(sh, lambda e: synth.expert_record(sh, seed, 0, e, mode=mode).numpy())
    ref = OM.layer_forward(xs[rows], sh.top_k, cache, sh.n_experts, logits=L[rows],
                           shared=real_shared_np(lay) if sh.shared_inter else None,
                           force_ids=ids[rows])
    # fp32 logits: their rounding error, and so the weights', grows with |x|
    assert np.abs(w[rows] - ref["w"]).max() <= 1e-5 * xscale
    assert_close(y[rows], ref["y"], "real T=%d %s" % (T, mode))
    assert np.all(np.isfinite(y))
    return y, ids


# The decoders on the whole range of their fields: every sub-scale nibble
# (-8..7, zero included) and, per block, d from four binades (subnormal or
# zero, [2^-10, 2^-9), the round-to-nearest binade, a large one) -- "wide";
# or every d in [2^-12, 2^-11), where the small table entries times d fall
# below fp16's normal range -- "small".  Both regimes of the standard formats
# (T <= 16: bandwidth kernels; T >= 17: grouped GEMMs) and every mode of the
# mixed formats.
@pytest.mark.parametrize("mode", ["wide", "small"])
@pytest.mark.parametrize("T", [1, 8, 17, 64])
def test_real_layer_full_field_range(T, mode):
    _real_case(T, seed=21, mode=mode)


@pytest.mark.parametrize("ug,dn", [(2, 3), (4, 5), (3, 3), (2, 5), (4, 3), (3, 5),
                                   (6, 3), (6, 5), (7, 3), (7, 5)],
                         ids=["q3s_nl4", "q2s_q2", "nl4_nl4", "q3s_q2", "q2s_nl4", "nl4_q2",
                              "q3k_nl4", "q3k_q2", "nl4s_nl4", "nl4s_q2"])
@pytest.mark.parametrize("mode", ["wide", "small"])
@pytest.mark.parametrize("T", [5, 40])
def test_mixed_format_layer_full_field_range(T, mode, ug, dn):
    _real_case(T, seed=22, sh=synth.Shape(512, 128, 24, 3, 64, ug, dn), mode=mode)


def _prefill_all_tokens(T, seed, zipf_s, mode="rtn", sh=synth.REAL):
    """Every output row of a prefill-sized layer against the oracle, whose
    routed experts run one at a time in a process pool (tests/_oracle_pool)."""
    import sys
    import time
    from tests import _oracle_pool
    t0 = time.time()

    def note(what):
        print("[prefill all tokens] T=%d zipf %.1f: %s, %.1f s" % (T, zipf_s, what, time.time() - t0),
              file=sys.__stderr__, flush=True)

    note("start")
    lay = synth.real_layer(sh, seed, 0, zipf_s=zipf_s, device=dev(), mode=mode)
    x = synth.tokens_bf16(T, sh.hidden, seed).to(dev())
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter, sh.upgate_fmt,
               sh.down_fmt)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    note("inputs on the GPU")
    y, ids, w = _run_layer(d, wts, x)
    note("layer done on the GPU")
    del lay.experts
    torch.cuda.empty_cache()
    xs = bf16_np(x)
    L = OM.router_logits(xs, bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
    assert ids_valid_topk(ids, L, sh.top_k)
    ref_ids = OM.topk_ids_fast(L, sh.top_k)
    flips = int((np.sort(ids, axis=1) != np.sort(ref_ids, axis=1)).any(axis=1).sum())
    assert flips <= max(1, T // 1000), "routing differs on %d tokens" % flips
    ref_w = OM.softmax_selected(L, ids.astype(np.int64))
    assert np.abs(w - ref_w).max() <= 1e-5
    offsets, perm, inv = OM.permute(ids, sh.n_experts)
    note("routing checked")
    y_perm = _oracle_pool.routed_outputs(sh, seed, 0, mode, T, offsets, perm, sh.top_k)
    _, ys = OM.ffn(xs, *real_shared_np(lay))
    ref = OM.combine(y_perm, inv, ref_w, ys)
    print("[parity] prefill T=%d zipf %.1f: %d near-tie routing flips" % (T, zipf_s, flips))
    assert_close(y, ref, "prefill all %d tokens, zipf %.1f %s" % (T, zipf_s, mode))
    # the tile mapping: every 64-row tile of every expert holds rows within the bar
    err = np.abs(y - ref).max(axis=1) / np.sqrt((ref * ref).mean())
    assert err.max() <= 1e-2


@pytest.mark.parametrize("zipf_s", [1.0, 0.0], ids=["zipf", "uniform"])
def test_real_prefill_all_tokens(zipf_s):
    _prefill_all_tokens(8192, 3, zipf_s)


@pytest.mark.parametrize("T", [1, 3, 5, 8, 16])
def test_real_decode_layer(T):
    _real_case(T, seed=2)


def test_real_decode_layer_logit_ties():
    """Given logits full of equal values through the routing inside the
    bandwidth path's up|gate kernel (E = 512, k = 10): the ids must be the
    exact top-k by (logit descending, expert ascending), on rows that take
    the threshold-and-rank selection and on rows that fall back to the
    round-based one (more than 64 logits at the threshold)."""
    sh = synth.REAL
    T, E, k = 8, sh.n_experts, sh.top_k
    rng = np.random.default_rng(11)
    L = rng.normal(size=(T, E)).astype(np.float32)
    L[1, :] = 0.25                                           # all equal
    L[2, :] = rng.integers(0, 8, size=E)                     # eight values
    L[3, [40, 7, 300, 511]] = L[3].max() + 1.0               # a four-way tie at the top
    lead = np.argsort(-L[4], kind="stable")[:12]
    L[4, lead] = L[4, lead[0]]                               # twelve equal leaders
    L[5, :] = rng.integers(0, 16, size=E) * 0.5              # sixteen values
    L[6, :] = 0.0
    L[6, ::3] = -0.0                                         # -0 ties +0
    L[6, 100] = 1.0
    L[7, :] = -np.arange(E, dtype=np.float32)                # strictly decreasing
    lay = synth.real_layer(sh, 3, 0, device=dev())
    x = synth.tokens_bf16(T, sh.hidden, 3).to(dev())
    d = Q.desc(sh.hidden, sh.inter, E, k, sh.shared_inter, sh.upgate_fmt, sh.down_fmt)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    y, ids, w = _run_layer(d, wts, x, logits=torch.from_numpy(L).to(dev()))
    L64 = L.astype(np.float64)
    assert np.array_equal(ids, OM.topk_ids(L64, k))
    assert ids[6].tolist() == [100, 0, 1, 2, 3, 4, 5, 6, 7, 8]
    cache = ExpertCache(sh, lambda e: synth.expert_record(sh, 3, 0, e).numpy())
    ref = OM.layer_forward(bf16_np(x), k, cache, E, logits=L64, shared=real_shared_np(lay))
    assert np.abs(w - ref["w"]).max() <= 1e-6
    assert_close(y, ref["y"], "logit ties T=%d" % T)


# Edge shape for both paths: I = 3 * 64 (an odd count of 64-wide K steps in
# the down projection, a partial last up|gate output tile), 24 experts (not a
# multiple of the 16-expert router tile), top-3, a 64-wide shared expert.
ODD = synth.Shape(hidden=512, inter=192, n_experts=24, top_k=3, shared_inter=64)


@pytest.mark.parametrize("T", [5, 16, 40])
def test_odd_shape_layer(T):
    _real_case(T, seed=6, sh=ODD)


# Degenerate routing: every expert selected (k = E), and a single expert (k = 1).
ALL_EXPERTS = synth.Shape(hidden=256, inter=64, n_experts=8, top_k=8, shared_inter=0)
ONE_EXPERT = synth.Shape(hidden=256, inter=128, n_experts=32, top_k=1, shared_inter=0)


@pytest.mark.parametrize("sh", [ALL_EXPERTS, ONE_EXPERT], ids=["k_eq_E", "k_1"])
@pytest.mark.parametrize("T", [3, 33])
def test_degenerate_routing_layer(T, sh):
    _real_case(T, seed=7, sh=sh)


# Limits of the descriptor: the widest hidden size (8192; its up|gate rows do
# not fit the bandwidth path's LDS staging, so small batches take the GEMM
# path too) and the most experts / largest top-k (1024, 32).
WIDE = synth.Shape(hidden=8192, inter=64, n_experts=16, top_k=2, shared_inter=64)
MANY = synth.Shape(hidden=256, inter=64, n_experts=1024, top_k=32, shared_inter=0)


@pytest.mark.parametrize("sh", [WIDE, MANY], ids=["H8192", "E1024_k32"])
@pytest.mark.parametrize("T", [2, 20])
def test_limit_shape_layer(T, sh):
    _real_case(T, seed=8, sh=sh)


# Hidden sizes of the bandwidth path's other up|gate kernel variants: the
# eight decoding waves take H/128 K groups of 128, so H = 2304 gives 3 groups
# per wave with the last waves' share short, H = 3584 four with a short share,
# H = 4096 four each (the largest hidden size whose two staged items fit LDS).
@pytest.mark.parametrize("H", [2304, 3584, 4096])
@pytest.mark.parametrize("T", [1, 7, 16])
def test_bandwidth_path_hidden_sizes(T, H):
    sh = synth.Shape(hidden=H, inter=64, n_experts=16, top_k=2, shared_inter=64)
    _real_case(T, seed=13, sh=sh)
    # the bandwidth path ran: stage 1, up|gate, down, combine (4 kernels, 5 marks)
    lay = synth.real_layer(sh, 13, 0, device=dev())
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    x = synth.tokens_bf16(T, sh.hidden, 13).to(dev())
    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(12)]
    for ev in evs:
        ev.record()
    torch.cuda.synchronize()
    n = Q.moe_layer_forward_timed(d, wts, x, y, Q.workspace(d, T, dev()), [ev.cuda_event for ev in evs])
    torch.cuda.synchronize()
    assert n == 5


@pytest.mark.parametrize("T", [17, 64])
def test_real_small_gemm_layer(T):
    _real_case(T, seed=7)


# Mixed-format layers (the 2.5-bpw / 4-bit NL up|gate and 2-bit down codecs):
# every up|gate x down pair at a small shape with a shared expert, on both
# sides of the token count where the standard formats switch kernels (these
# formats take the grouped GEMMs at every T), and an odd down K (I = 3 * 64:
# the last K period of the 2-bit rows is half).
F = synth
PAIRS = [(F.FMT_Q2S256, F.FMT_Q2_32), (F.FMT_NL4_32, F.FMT_NL4_32), (F.FMT_Q3S256, F.FMT_Q2_32),
         (F.FMT_Q2S256, F.FMT_NL4_32), (F.FMT_NL4_32, F.FMT_Q2_32),
         (F.FMT_Q3K256, F.FMT_NL4_32), (F.FMT_Q3K256, F.FMT_Q2_32),
         (F.FMT_NL4S256, F.FMT_NL4_32), (F.FMT_NL4S256, F.FMT_Q2_32)]
PAIR_IDS = ["q2s_q2", "nl4_nl4", "q3s_q2", "q2s_nl4", "nl4_q2", "q3k_nl4", "q3k_q2", "nl4s_nl4",
            "nl4s_q2"]


@pytest.mark.parametrize("ug,dn", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("T", [5, 40])
def test_mixed_format_layer(T, ug, dn):
    _real_case(T, seed=9, sh=synth.Shape(512, 128, 24, 3, 64, ug, dn))


@pytest.mark.parametrize("ug,dn", [(F.FMT_Q2S256, F.FMT_Q2_32), (F.FMT_NL4_32, F.FMT_Q2_32),
                                   (F.FMT_Q3K256, F.FMT_Q2_32), (F.FMT_NL4S256, F.FMT_Q2_32)])
def test_mixed_format_odd_down_k(ug, dn):
    _real_case(33, seed=10, sh=synth.Shape(512, 192, 24, 3, 64, ug, dn))


@pytest.mark.parametrize("ug,dn", [(F.FMT_Q2S256, F.FMT_Q2_32), (F.FMT_NL4_32, F.FMT_NL4_32),
                                   (F.FMT_Q3K256, F.FMT_NL4_32), (F.FMT_NL4S256, F.FMT_NL4_32)])
@pytest.mark.parametrize("T", [8, 64])
def test_mixed_format_real_layer(T, ug, dn):
    _real_case(T, seed=11, sh=synth.Shape(3072, 512, 512, 10, 512, ug, dn))


# The draft head's MoE layer: up|gate Q3K-256, down NL4-32, real shape with
# the shared expert, at the verify batches of two and four drafts (T = 3, 5),
# one token, and a prefill-sized chunk, on RTN and full-range fields.
@pytest.mark.parametrize("mode", ["rtn", "wide", "small"])
@pytest.mark.parametrize("T", [1, 3, 5, 64])
def test_mtp_head_layer(T, mode):
    _real_case(T, seed=31, sh=synth.MTP_HEAD, mode=mode)


def test_mtp_head_prefill_sampled():
    rng = np.random.default_rng(4)
    sample = np.sort(rng.choice(2048, size=6, replace=False))
    sample[-1] = 2047
    _real_case(2048, seed=32, sample=sample, sh=synth.MTP_HEAD)


@pytest.mark.parametrize("ug,dn", [(F.FMT_Q2S256, F.FMT_Q2_32), (F.FMT_NL4_32, F.FMT_NL4_32)])
def test_mixed_format_prefill_chunk_sampled(ug, dn):
    """9536-token chunk (the equal-size prefill batch of the mixed-format
    stack), Zipf(0.8) routing, sampled tokens including the last."""
    rng = np.random.default_rng(2)
    sample = np.sort(rng.choice(9536, size=4, replace=False))
    sample[-1] = 9535
    _real_case(9536, seed=12, zipf_s=0.8, sample=sample, sh=synth.Shape(3072, 512, 512, 10, 512, ug, dn))


def test_real_prefill_zipf_sampled():
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(8192, size=6, replace=False))
    sample[-1] = 8191                                   # the ragged end of the last tile
    _real_case(8192, seed=3, zipf_s=1.0, sample=sample)


def test_real_prefill_uniform_sampled():
    rng = np.random.default_rng(1)
    sample = np.sort(rng.choice(2048, size=5, replace=False))
    _real_case(2048, seed=3, zipf_s=0.0, sample=sample)


# The grouped-GEMM path holds the routed rows in fp16 unless its range check
# sends them to fp32: down weights scaled up (every NL4 d set to 2048) and
# tokens 4 N(0, 1) push half the rows' values past 65504 (a stays near 140),
# where fp16 would give inf; the "small" field-range cases above take the
# same fp32 form from the other side (tiles of tiny values).
@pytest.mark.parametrize("T", [40, 300])
def test_gemm_rows_beyond_fp16_take_the_fp32_form(T):
    sh = synth.Shape(512, 128, 24, 3, 64, F.FMT_Q3S256, F.FMT_NL4_32)
    seed = 41
    lay = synth.real_layer(sh, seed, 0, zipf_s=1.0, device=dev())

    def big_down(rec):
        dn = rec[sh.upgate_bytes:].view(-1, 18)
        dn[:, 0] = 0x00
        dn[:, 1] = 0x68                              # d = 2048.0
        return rec

    for e in range(sh.n_experts):
        big_down(lay.experts[e])
    x = (synth.tokens_bf16(T, sh.hidden, seed).float() * 4).to(torch.bfloat16).to(dev())
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter, sh.upgate_fmt,
               sh.down_fmt)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    y, ids, w = _run_layer(d, wts, x)
    assert np.all(np.isfinite(y))
    assert np.abs(y).max() > 65504.0 * 2          # the routed rows left fp16's range
    xs = bf16_np(x)
    L = OM.router_logits(xs, bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
    assert ids_valid_topk(ids, L, sh.top_k)
    cache = ExpertCache(sh, lambda e: big_down(synth.expert_record(sh, seed, 0, e)).numpy())
    ref = OM.layer_forward(xs, sh.top_k, cache, sh.n_experts, logits=L, shared=real_shared_np(lay),
                           force_ids=ids)
    assert_close(y, ref["y"], "rows beyond fp16 T=%d" % T)


def test_real_layer_max_tokens():
    """The largest batch the library takes (2^18 tokens, 2.6M routed slots) at
    the real shape: every token's ids are k distinct experts, its weights sum
    to 1 and its output is finite; sampled tokens (the first, the last, and
    some in between) against the oracle, routing included."""
    import sys
    T, sh, seed = 1 << 18, synth.REAL, 51
    print("[max tokens] generating", file=sys.__stderr__, flush=True)
    lay = synth.real_layer(sh, seed, 0, zipf_s=1.0, device=dev())
    x = synth.tokens_bf16(T, sh.hidden, seed).to(dev())
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    print("[max tokens] layer", file=sys.__stderr__, flush=True)
    y, ids, w = _run_layer(d, wts, x)
    print("[max tokens] checks", file=sys.__stderr__, flush=True)
    assert np.all(np.isfinite(y))
    assert ids.min() >= 0 and ids.max() < sh.n_experts
    assert (np.diff(np.sort(ids, axis=1), axis=1) > 0).all()
    assert np.abs(w.sum(axis=1) - 1.0).max() <= 1e-5
    sample = np.array([0, 1, 4097, T // 2, T - 65, T - 2, T - 1])
    xs = bf16_np(x[torch.from_numpy(sample).to(dev())])
    L = OM.router_logits(xs, bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
    assert ids_valid_topk(ids[sample], L, sh.top_k)
    cache = ExpertCache(sh, lambda e: synth.expert_record(sh, seed, 0, e).numpy())
    ref = OM.layer_forward(xs, sh.top_k, cache, sh.n_experts, logits=L, shared=real_shared_np(lay),
                           force_ids=ids[sample])
    assert np.abs(w[sample] - ref["w"]).max() <= 1e-5
    assert_close(y[sample], ref["y"], "max tokens T=%d" % T)


def test_layer_deterministic():
    sh, recs, x, logits = tiny_inputs(seed=4, T=300)
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, 0)
    ex = torch.from_numpy(recs).to(dev())
    wts = Q.weights(ex, sh.expert_bytes)
    a = _run_layer(d, wts, x.to(dev()), logits=logits.to(dev()))
    b = _run_layer(d, wts, x.to(dev()), logits=logits.to(dev()))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_stack_three_layers_teacher_forced():
    """Pre-norm residual stack (RMSNorm eps 1e-6, gamma ~ N(1, 0.1)), T = 3:
    each layer's GPU output is compared with the oracle fed the GPU's layer
    input; the end-to-end error is reported through the same tolerance."""
    sh = synth.REAL
    T, seed = 3, 4
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    h = synth.tokens_bf16(T, sh.hidden, seed).float().to(dev())
    h_ref = h.double().cpu().numpy()
    normed = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device=dev())
    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    ws = Q.workspace(d, T, dev())
    for l in range(3):
        lay = synth.real_layer(sh, seed, l, zipf_s=1.0, device=dev())
        gamma = synth.norm_gain(sh.hidden, seed, l).to(dev())
        Q.moe_rmsnorm_residual(h, None, gamma, 1e-6, normed)
        wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                        lay.shared_down)
        ids = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev())
        Q.moe_layer_forward(d, wts, normed, y, ws, topk_ids_out=ids)
        torch.cuda.synchronize()
        xin = bf16_np(normed)
        L = OM.router_logits(xin, bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
        cache = ExpertCache(sh, lambda e, l=l: synth.expert_record(sh, seed, l, e).numpy())
        ref = OM.layer_forward(xin, sh.top_k, cache, sh.n_experts, logits=L,
                               shared=real_shared_np(lay), force_ids=ids.cpu().numpy())
        assert ids_valid_topk(ids.cpu().numpy(), L, sh.top_k)
        assert_close(y.cpu().numpy(), ref["y"], "stack layer %d" % l)
        # oracle's own end-to-end stream (not teacher-forced) for the report
        h_ref = OM.stack_step(h_ref, gamma.cpu().numpy(), 1e-6,
                              lambda z: OM.layer_forward(z, sh.top_k, cache, sh.n_experts,
                                                         router_w=bf16_np(lay.router_w),
                                                         router_b=lay.router_b.cpu().numpy(),
                                                         shared=real_shared_np(lay))["y"])
        Q.moe_rmsnorm_residual(h, y, None, 1e-6, None)
    assert_close(h.cpu().numpy(), h_ref, "stack end-to-end")


def test_mixed_stack_prefill_sampled():
    """The mixed-format stack (per-layer formats of the model card, seeded
    order), one 9536-token chunk, Zipf(0.8), RMSNorm (eps 1e-6) + residual:
    layers 0..13 run in order on the GPU; on the first layer of each of the
    six (up|gate, down) format pairs, sampled tokens are compared with the
    oracle fed the GPU's layer input (teacher forcing)."""
    wl = synth.WORKLOADS["stack_prefill"]
    T, seed = wl.tokens[0], wl.seed
    fm = synth.stack_formats(seed)
    check = {}
    for l, p in enumerate(fm):
        check.setdefault(p, l)
    last = max(check.values())
    checked = set(check.values())
    assert len(checked) == 6 and last < 16
    rows = np.array([0, 4097, 9535])
    h = synth.tokens_bf16(T, synth.REAL.hidden, seed).float().to(dev())
    normed = torch.empty((T, synth.REAL.hidden), dtype=torch.bfloat16, device=dev())
    y = torch.empty((T, synth.REAL.hidden), dtype=torch.float32, device=dev())
    ids = torch.empty((T, synth.REAL.top_k), dtype=torch.int32, device=dev())
    ws = None
    for l in range(last + 1):
        sh = synth.stack_shape(seed, l)
        lay = synth.real_layer(sh, seed, l, zipf_s=wl.zipf_s, device=dev())
        gamma = synth.norm_gain(sh.hidden, seed, l).to(dev())
        d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter, sh.upgate_fmt,
                   sh.down_fmt)
        if ws is None or ws.numel() < Q.moe_workspace_size(d, T):
            ws = Q.workspace(d, T, dev())
        Q.moe_rmsnorm_residual(h, None, gamma, 1e-6, normed)
        wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                        lay.shared_down)
        Q.moe_layer_forward(d, wts, normed, y, ws, topk_ids_out=ids)
        torch.cuda.synchronize()
        if l in checked:
            xin = bf16_np(normed[rows])
            L = OM.router_logits(xin, bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
            got_ids = ids[rows].cpu().numpy()
            assert ids_valid_topk(got_ids, L, sh.top_k)
            cache = ExpertCache(sh, lambda e, l=l, sh=sh: synth.expert_record(sh, seed, l, e).numpy())
            ref = OM.layer_forward(xin, sh.top_k, cache, sh.n_experts, logits=L,
                                   shared=real_shared_np(lay), force_ids=got_ids)
            assert_close(y[rows].cpu().numpy(), ref["y"],
                         "stack layer %d formats %s" % (l, (sh.upgate_fmt, sh.down_fmt)))
        Q.moe_rmsnorm_residual(h, y, None, 1e-6, None)
        del lay, wts
    assert torch.isfinite(h).all()
