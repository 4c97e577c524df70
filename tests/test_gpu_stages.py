"""GPU parity of each stage of the layer against the oracle, through the C ABI.

Bit-exact: dequantised weights, routing ids, offsets / perm / inv_perm.
Floats: rel L2 <= 1e-3 and max abs <= 1e-2 * rms (routing weights: 1e-6).
"""

import numpy as np
import pytest
import torch

import quantized_expert_ffn_top_amd as Q
import synth
from oracle import formats as OF
from oracle import moe as OM
from tests._helpers import (ExpertCache, assert_close, bf16_np, dev, tiny_inputs)

pytestmark = pytest.mark.gpu


def _u8(arr):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).to(dev())


# ---------------------------------------------------------------- dequant

def _hand_q3s_blocks():
    blocks = []
    for d_bits in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xC000, 0x8001):
        for s in ([-8, -1, 0, 1, 7, 2, -3, 5], [7] * 8, [-8] * 8):
            blocks.append(OF.pack_q3s_block(d_bits, s, [i % 8 for i in range(256)]))
            blocks.append(OF.pack_q3s_block(d_bits, s, [7 - (i * 5) % 8 for i in range(256)]))
    return np.frombuffer(b"".join(blocks), dtype=np.uint8).reshape(-1, 104)


def test_dequant_q3s_hand_blocks_bitexact():
    raw = _hand_q3s_blocks()
    out = torch.empty(raw.shape[0] * 256, dtype=torch.float32, device=dev())
    Q.moe_dequantize(Q.MOE_FMT_Q3S256, _u8(raw), raw.shape[0] * 256, out)
    ref = OF.dequant_q3s(raw).reshape(-1).astype(np.float32)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_nl4_hand_blocks_bitexact():
    blocks = []
    for d_bits in (0x0001, 0x03FF, 0x3C00, 0x7BFF, 0xC000, 0x2800):
        blocks.append(OF.pack_nl4_block(d_bits, list(range(16)) * 2))
        blocks.append(OF.pack_nl4_block(d_bits, [15 - (i % 16) for i in range(32)]))
    raw = np.frombuffer(b"".join(blocks), dtype=np.uint8).reshape(-1, 18)
    out = torch.empty(raw.shape[0] * 32, dtype=torch.float32, device=dev())
    Q.moe_dequantize(Q.MOE_FMT_NL4_32, _u8(raw), raw.shape[0] * 32, out)
    ref = OF.dequant_nl4(raw).reshape(-1).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_dequant_q2s_hand_blocks_bitexact():
    raw = _hand_blocks(Q.MOE_FMT_Q2S256).reshape(-1, 80)
    out = torch.empty(raw.shape[0] * 256, dtype=torch.float32, device=dev())
    Q.moe_dequantize(Q.MOE_FMT_Q2S256, _u8(raw), raw.shape[0] * 256, out)
    ref = OF.dequant_q2s(raw).reshape(-1).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_dequant_q2_hand_blocks_bitexact():
    raw = _hand_blocks(Q.MOE_FMT_Q2_32).reshape(-1, 10)
    out = torch.empty(raw.shape[0] * 32, dtype=torch.float32, device=dev())
    # 14 blocks = 140 bytes: the device copy padded to a 16-byte multiple
    Q.moe_dequantize(Q.MOE_FMT_Q2_32, _padded(raw.reshape(-1)), raw.shape[0] * 32, out)
    ref = OF.dequant_q2(raw).reshape(-1).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def _dequant_padded(fmt, raw, n):
    """moe_dequantize on raw block bytes copied into a 16-byte-multiple buffer."""
    flat = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1)
    src = torch.zeros(((flat.size + 15) // 16) * 16, dtype=torch.uint8, device=dev())
    src[:flat.size] = _u8(flat)
    out = torch.empty(n, dtype=torch.float32, device=dev())
    Q.moe_dequantize(fmt, src, n, out)
    return out.cpu().numpy()


def test_dequant_q3k_hand_blocks_bitexact():
    """Every 6-bit sub-scale (-32..31) at every one of the 16 positions, with
    d from subnormal to the largest finite and negative."""
    raw = _hand_blocks(Q.MOE_FMT_Q3K256).reshape(-1, OF.Q3K_BLOCK_BYTES)
    got = _dequant_padded(Q.MOE_FMT_Q3K256, raw, raw.shape[0] * 256)
    ref = OF.dequant_q3k(raw).reshape(-1).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_nl4s_hand_blocks_bitexact():
    """Every 6-bit sub-scale at every one of the 8 positions, every table entry."""
    raw = _hand_blocks(Q.MOE_FMT_NL4S256).reshape(-1, OF.NL4S_BLOCK_BYTES)
    got = _dequant_padded(Q.MOE_FMT_NL4S256, raw, raw.shape[0] * 256)
    ref = OF.dequant_nl4s(raw).reshape(-1).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("ug,dn,mode", [(synth.FMT_Q2S256, synth.FMT_Q2_32, "full"),
                                        (synth.FMT_NL4_32, synth.FMT_NL4_32, "full"),
                                        (synth.FMT_Q3K256, synth.FMT_NL4_32, "rtn"),
                                        (synth.FMT_Q3K256, synth.FMT_Q2_32, "wide"),
                                        (synth.FMT_NL4S256, synth.FMT_NL4_32, "small"),
                                        (synth.FMT_NL4S256, synth.FMT_Q2_32, "wide")])
def test_dequant_real_mixed_experts_bitexact(ug, dn, mode):
    """Records of the mixed-format layers at real shape: every block of 8
    experts, GPU-generated, against the oracle on the CPU-regenerated bytes."""
    sh = synth.Shape(3072, 512, 512, 10, 512, ug, dn)
    for e in range(0, 512, 64):
        rec_gpu = synth.expert_record(sh, 5, 1, e, device=dev(), mode=mode)
        rec_cpu = synth.expert_record(sh, 5, 1, e, device="cpu", mode=mode).numpy()
        assert np.array_equal(rec_gpu.cpu().numpy(), rec_cpu)
        nug = sh.upgate_bytes
        for fmt, lo, hi, n in ((ug, 0, nug, 2 * sh.inter * sh.hidden),
                               (dn, nug, sh.expert_bytes, sh.hidden * sh.inter)):
            src = torch.zeros(((hi - lo + 15) // 16) * 16, dtype=torch.uint8, device=dev())
            src[:hi - lo] = rec_gpu[lo:hi]
            out = torch.empty(n, dtype=torch.float32, device=dev())
            Q.moe_dequantize(fmt, src, n, out)
            ref = OF.dequant_matrix(fmt, rec_cpu[lo:hi], 1, n).reshape(-1).astype(np.float32)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (fmt, e)


@pytest.mark.parametrize("mode", ["rtn", "full"])
def test_dequant_real_experts_bitexact(mode):
    """Every block of 24 real-shape experts (both codecs), generated on the GPU,
    against the oracle's decoder on the CPU-regenerated bytes."""
    sh = synth.REAL
    for e in range(0, 512, 22):
        rec_gpu = synth.expert_record(sh, 5, 0, e, device=dev(), mode=mode)
        rec_cpu = synth.expert_record(sh, 5, 0, e, device="cpu", mode=mode).numpy()
        assert np.array_equal(rec_gpu.cpu().numpy(), rec_cpu)       # generator is device-exact
        nug = sh.upgate_bytes
        out = torch.empty(2 * sh.inter * sh.hidden, dtype=torch.float32, device=dev())
        Q.moe_dequantize(Q.MOE_FMT_Q3S256, rec_gpu[:nug], out.numel(), out)
        ref = OF.dequant_q3s(rec_cpu[:nug].reshape(-1, 104)).reshape(-1).astype(np.float32)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), e
        # down region starts 16-byte aligned inside the record
        out2 = torch.empty(sh.hidden * sh.inter, dtype=torch.float32, device=dev())
        Q.moe_dequantize(Q.MOE_FMT_NL4_32, rec_gpu[nug:], out2.numel(), out2)
        ref2 = OF.dequant_nl4(rec_cpu[nug:].reshape(-1, 18)).reshape(-1).astype(np.float32)
        assert np.array_equal(out2.cpu().numpy().view(np.uint32), ref2.view(np.uint32)), e


# ---------------------------------------------------------------- the kernels' decoders
# moe_dequantize_path decodes with the tables, lookup addresses and fp16
# multiplies that the layer's kernels inline: the pair tables of the
# bandwidth-path kernels, the quad table and the NL4 fold of the grouped GEMM.

PATHS = [(Q.MOE_PATH_BANDWIDTH, "bandwidth"), (Q.MOE_PATH_GEMM, "gemm")]


def _fold16(w):
    """The grouped GEMM's NL4-32 down weights (its one rounding of weights):
    16 w rounded once to binary16, round to nearest even, then / 16; w is the
    oracle's exact value (16 w is exact in fp64)."""
    with np.errstate(over="ignore"):
        return (np.asarray(w, dtype=np.float64) * 16.0).astype(np.float16).astype(np.float32) * np.float32(0.0625)


def _nl4_expected(w, path):
    return _fold16(w) if path == Q.MOE_PATH_GEMM else np.asarray(w).astype(np.float32)


def _path_dequant(fmt, path, src, n):
    out = torch.empty(n, dtype=torch.float32, device=dev())
    Q.moe_dequantize_path(fmt, path, src, n, out)
    return out.cpu().numpy()


@pytest.mark.parametrize("path,name", PATHS, ids=[p[1] for p in PATHS])
def test_kernel_decoders_hand_blocks_bitexact(path, name):
    """Hand blocks through the kernels' decoders: d from the smallest subnormal
    to the largest finite value, both signs; every sub-scale; every codebook
    entry at every position."""
    raw = _hand_q3s_blocks()
    got = _path_dequant(Q.MOE_FMT_Q3S256, path, _u8(raw), raw.shape[0] * 256)
    ref = OF.dequant_q3s(raw).reshape(-1).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
    blocks = []
    for d_bits in (0x0001, 0x0155, 0x03FF, 0x0400, 0x1000, 0x3C00, 0x7BFF, 0xC000, 0x8001, 0x2800):
        blocks.append(OF.pack_nl4_block(d_bits, list(range(16)) * 2))
        blocks.append(OF.pack_nl4_block(d_bits, [15 - (i * 7) % 16 for i in range(32)]))
    raw = np.frombuffer(b"".join(blocks), dtype=np.uint8).reshape(-1, 18)
    flat = raw.reshape(-1)
    src = torch.zeros(((flat.size + 15) // 16) * 16, dtype=torch.uint8, device=dev())
    src[:flat.size] = _u8(flat)
    got = _path_dequant(Q.MOE_FMT_NL4_32, path, src, raw.shape[0] * 32)
    ref = _nl4_expected(OF.dequant_nl4(raw).reshape(-1), path)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name


@pytest.mark.parametrize("mode", ["full", "wide", "small"])
def test_kernel_decoders_real_experts_bitexact(mode):
    """Every block of 8 real-shape experts (up|gate Q3S-256, down NL4-32) with
    full-range fields (every sub-scale; d over four binades, subnormal or zero
    included; or every d below 2^-11) through the decoders of both paths."""
    sh = synth.REAL
    nug = sh.upgate_bytes
    for e in range(0, 512, 64):
        rec_gpu = synth.expert_record(sh, 7, 0, e, device=dev(), mode=mode)
        rec_cpu = synth.expert_record(sh, 7, 0, e, device="cpu", mode=mode).numpy()
        assert np.array_equal(rec_gpu.cpu().numpy(), rec_cpu)
        w_ug = OF.dequant_q3s(rec_cpu[:nug].reshape(-1, 104)).reshape(-1).astype(np.float32)
        w_dn = OF.dequant_nl4(rec_cpu[nug:].reshape(-1, 18)).reshape(-1)
        for path, name in PATHS:
            got = _path_dequant(Q.MOE_FMT_Q3S256, path, rec_gpu[:nug], w_ug.size)
            assert np.array_equal(got.view(np.uint32), w_ug.view(np.uint32)), (name, e)
            got = _path_dequant(Q.MOE_FMT_NL4_32, path, rec_gpu[nug:], w_dn.size)
            ref = _nl4_expected(w_dn, path)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (name, e)


def _hand_blocks(fmt):
    """Hand blocks of the other formats: d from the smallest subnormal to the
    largest finite value, both signs; every sub-scale at every position;
    every codebook entry."""
    blocks = []
    for d_bits in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xC000, 0x8001):
        if fmt == Q.MOE_FMT_Q2S256:
            for s in ([-8, -1, 0, 1, 7, 2, -3, 5], [7] * 8, [-8] * 8):
                blocks.append(OF.pack_q2s_block(d_bits, s, [i % 4 for i in range(256)]))
                blocks.append(OF.pack_q2s_block(d_bits, s, [3 - (i * 3) % 4 for i in range(256)]))
        elif fmt == Q.MOE_FMT_Q2_32:
            blocks.append(OF.pack_q2_block(d_bits, [i % 4 for i in range(32)]))
            blocks.append(OF.pack_q2_block(d_bits, [3 - (i * 3) % 4 for i in range(32)]))
        elif fmt == Q.MOE_FMT_Q3K256:
            for base in (-32, -16, 0, 16):
                s = [base + j for j in range(16)]
                blocks.append(OF.pack_q3k_block(d_bits, s, [i % 8 for i in range(256)]))
                blocks.append(OF.pack_q3k_block(d_bits, s[::-1], [7 - (i * 5) % 8 for i in range(256)]))
        else:
            for base in range(-32, 32, 8):
                s = [base + j for j in range(8)]
                blocks.append(OF.pack_nl4s_block(d_bits, s, [i % 16 for i in range(256)]))
                blocks.append(OF.pack_nl4s_block(d_bits, s[::-1], [15 - (i * 7) % 16 for i in range(256)]))
    return np.frombuffer(b"".join(blocks), dtype=np.uint8)


def _padded(flat):
    src = torch.zeros(((flat.size + 15) // 16) * 16, dtype=torch.uint8, device=dev())
    src[:flat.size] = _u8(flat)
    return src


def _same(got, ref, fmt):
    """Bit for bit; for Q3K-256 value for value (its two exact parts are
    summed, so a zero weight can be +0 where the oracle's product is -0)."""
    if fmt == Q.MOE_FMT_Q3K256:
        return np.array_equal(got, ref) and not np.isnan(got).any()
    return np.array_equal(got.view(np.uint32), ref.view(np.uint32))


MIXED_FMTS = [Q.MOE_FMT_Q2S256, Q.MOE_FMT_Q2_32, Q.MOE_FMT_Q3K256, Q.MOE_FMT_NL4S256]


def _q2_fp16(w):
    """The grouped GEMM's Q2-32 fragments: d (q - 2) formed in fp16, i.e. the
    exact value rounded once to binary16 (equal to it for |d| <= 32752, the
    stated bound; +-inf for code 0 beyond)."""
    with np.errstate(over="ignore"):
        return np.asarray(w, dtype=np.float64).astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("fmt", MIXED_FMTS, ids=["q2s", "q2", "q3k", "nl4s"])
def test_kernel_decoders_mixed_hand_blocks(fmt):
    """The grouped GEMM's decoders of the mixed-format and draft-head codecs
    on hand blocks, against the oracle's exact values."""
    flat = _hand_blocks(fmt)
    n = flat.size // OF.CODECS[fmt][1] * OF.CODECS[fmt][0]
    got = _path_dequant(fmt, Q.MOE_PATH_GEMM, _padded(flat), n)
    w = OF.dequant_matrix(fmt, flat, 1, n).reshape(-1)
    ref = _q2_fp16(w) if fmt == Q.MOE_FMT_Q2_32 else w.astype(np.float32)
    assert _same(got, ref, fmt)
    if fmt == Q.MOE_FMT_Q2_32:
        # within the stated bound |d| <= 32752 the fragments are the exact values
        inb = np.abs(w) <= 65504
        assert np.array_equal(got[inb].view(np.uint32), w[inb].astype(np.float32).view(np.uint32))
        assert np.isinf(got[~inb]).all() and (~inb).any()


@pytest.mark.parametrize("ug,dn,mode", [(synth.FMT_Q2S256, synth.FMT_Q2_32, "full"),
                                        (synth.FMT_NL4_32, synth.FMT_NL4_32, "wide"),
                                        (synth.FMT_Q3K256, synth.FMT_NL4_32, "wide"),
                                        (synth.FMT_Q3K256, synth.FMT_Q2_32, "small"),
                                        (synth.FMT_NL4S256, synth.FMT_NL4_32, "small"),
                                        (synth.FMT_NL4S256, synth.FMT_Q2_32, "full")])
def test_kernel_decoders_mixed_experts(ug, dn, mode):
    """Records of the mixed-format layers at real shape (every block of 4
    experts) through the decoders their grouped-GEMM modes run: NL4-32 up|gate
    through the pair table it shares with the bandwidth path's down kernel,
    NL4-32 down through the fold, the others exact."""
    sh = synth.Shape(3072, 512, 512, 10, 512, ug, dn)
    nug = sh.upgate_bytes
    for e in range(0, 512, 128):
        rec_gpu = synth.expert_record(sh, 9, 2, e, device=dev(), mode=mode)
        rec_cpu = synth.expert_record(sh, 9, 2, e, device="cpu", mode=mode).numpy()
        assert np.array_equal(rec_gpu.cpu().numpy(), rec_cpu)
        for fmt, lo, hi, n, path in (
                (ug, 0, nug, 2 * sh.inter * sh.hidden,
                 Q.MOE_PATH_BANDWIDTH if ug == synth.FMT_NL4_32 else Q.MOE_PATH_GEMM),
                (dn, nug, sh.expert_bytes, sh.hidden * sh.inter, Q.MOE_PATH_GEMM)):
            got = _path_dequant(fmt, path, _padded(rec_cpu[lo:hi]), n)
            w = OF.dequant_matrix(fmt, rec_cpu[lo:hi], 1, n).reshape(-1)
            ref = (_fold16(w) if (fmt == synth.FMT_NL4_32 and path == Q.MOE_PATH_GEMM)
                   else _q2_fp16(w) if fmt == synth.FMT_Q2_32 else w.astype(np.float32))
            assert _same(got, ref, fmt), (fmt, path, e)


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("T,sh", [(1, synth.REAL), (3, synth.REAL), (8, synth.REAL), (16, synth.REAL),
                                  (17, synth.REAL), (300, synth.REAL), (8192, synth.REAL),
                                  # expert counts off the 256-column tile, a ragged
                                  # last 128-row tile, the largest E
                                  (300, synth.Shape(512, 64, 200, 4, 0)),
                                  (129, synth.Shape(256, 64, 24, 4, 0)),
                                  (1000, synth.Shape(1024, 64, 1024, 4, 0))])
def test_router_logits(T, sh):
    x = synth.tokens_bf16(T, sh.hidden, 9).to(dev())
    wr = synth.router_weight(sh, 9, 0).to(dev())
    b = synth.zipf_bias(sh.n_experts, 1.0, 9, 0).to(dev())
    logits = torch.empty((T, sh.n_experts), dtype=torch.float32, device=dev())
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=dev())
    Q.moe_router_logits(x, wr, b, logits, ws)
    ref = OM.router_logits(bf16_np(x), bf16_np(wr), b.cpu().numpy().astype(np.float64))
    got = logits.cpu().numpy().astype(np.float64)
    # fp32 accumulation of 3072 exact products: |err| <~ 1e-5 relative to the row scale
    assert np.abs(got - ref).max() <= 2e-5 * np.abs(ref).max()


# ---------------------------------------------------------------- top-k

def _route(logits_np, k):
    T, E = logits_np.shape
    L = torch.from_numpy(logits_np.astype(np.float32)).to(dev())
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    w = torch.empty((T, k), dtype=torch.float32, device=dev())
    Q.moe_route(L, k, ids, w)
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,E,k", [(4, 16, 2), (3, 512, 10), (8192, 512, 10), (5, 1024, 32),
                                   (7, 16, 16), (2, 1, 1), (33, 100, 7)])
def test_route_bitexact(T, E, k):
    rng = np.random.default_rng(T * 1000 + E + k)
    L = rng.normal(size=(T, E)).astype(np.float32)
    if T > 2:
        L[1, :] = L[1, 0]                              # a row of ties: lowest indices win
        L[2, E // 2] = L[2, E // 3] = L[2].max() + 1   # a tie at the top
    ids, w = _route(L, k)
    ref_ids = OM.topk_ids(L.astype(np.float64), k) if T <= 64 else OM.topk_ids_fast(L.astype(np.float64), k)
    assert np.array_equal(ids, ref_ids)
    ref_w = OM.softmax_selected(L.astype(np.float64), ref_ids)
    assert np.abs(w - ref_w).max() <= 1e-6
    assert np.abs(w.sum(axis=1) - 1).max() <= 1e-6


def test_route_negative_zero_ties_positive_zero():
    L = np.zeros((1, 8), dtype=np.float32)
    L[0, 5] = -0.0
    L[0, 2] = -1.0
    ids, _ = _route(L, 3)
    assert ids[0].tolist() == [0, 1, 3]


# ---------------------------------------------------------------- permute

@pytest.mark.parametrize("T,E,k", [(1, 512, 10), (3, 512, 10), (8, 512, 10), (16, 16, 2),
                                   (17, 512, 10), (100, 16, 2), (1000, 64, 7), (8192, 512, 10)])
def test_permute_bitexact(T, E, k):
    rng = np.random.default_rng(T + 7 * E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    tid = torch.from_numpy(ids).to(dev())
    off = torch.full((E + 1,), -1, dtype=torch.int32, device=dev())
    perm = torch.full((T * k,), -1, dtype=torch.int32, device=dev())
    inv = torch.full((T * k,), -1, dtype=torch.int32, device=dev())
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=dev())
    Q.moe_permute(tid, E, off, perm, inv, ws)
    r_off, r_perm, r_inv = OM.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(perm.cpu().numpy(), r_perm)
    assert np.array_equal(inv.cpu().numpy(), r_inv)


# ---------------------------------------------------------------- expert FFN + combine

@pytest.mark.parametrize("T", [4, 16, 17, 70])
def test_expert_ffn_and_combine_tiny(T):
    sh, recs, x, logits = tiny_inputs(seed=1, T=T)
    k, E = sh.top_k, sh.n_experts
    ids = OM.topk_ids(logits.double().numpy(), k)
    off, perm, inv = OM.permute(ids, E)
    w = OM.softmax_selected(logits.double().numpy(), ids)
    d = Q.desc(sh.hidden, sh.inter, E, k, 0)
    ex = _u8(recs)
    wts = Q.weights(ex, sh.expert_bytes)
    xd = x.to(dev())
    t_off = torch.from_numpy(off.astype(np.int32)).to(dev())
    t_perm = torch.from_numpy(perm.astype(np.int32)).to(dev())
    y_perm = torch.empty((T * k, sh.hidden), dtype=torch.float32, device=dev())
    ws = Q.workspace(d, T, dev())
    Q.moe_expert_ffn(d, wts, xd, t_off, t_perm, y_perm, None, ws)
    cache = ExpertCache(sh, lambda e: recs[e])
    _, ref_yp = OM.expert_ffn_perm(bf16_np(x), off, perm, k, cache)
    assert_close(y_perm.cpu().numpy(), ref_yp, "y_perm T=%d" % T)

    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    t_inv = torch.from_numpy(inv.astype(np.int32)).to(dev())
    t_w = torch.from_numpy(w.astype(np.float32)).to(dev())
    Q.moe_combine(y_perm, t_inv, t_w, None, y)
    ref_y = OM.combine(y_perm.cpu().numpy().astype(np.float64), inv, w.astype(np.float32))
    assert np.abs(y.cpu().numpy() - ref_y).max() <= 1e-5 * np.abs(ref_y).max()


@pytest.mark.parametrize("T", [3, 40])
def test_expert_ffn_real_shape_with_shared(T):
    """Real shape, routing from the Zipf-biased router; y_perm and shared_y."""
    sh = synth.REAL
    lay = synth.real_layer(sh, 6, 0, zipf_s=1.0, device=dev())
    x = synth.tokens_bf16(T, sh.hidden, 6).to(dev())
    L = OM.router_logits(bf16_np(x), bf16_np(lay.router_w), lay.router_b.cpu().numpy().astype(np.float64))
    ids = OM.topk_ids_fast(L, sh.top_k)
    off, perm, inv = OM.permute(ids, sh.n_experts)
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    y_perm = torch.empty((T * sh.top_k, sh.hidden), dtype=torch.float32, device=dev())
    y_sh = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    ws = Q.workspace(d, T, dev())
    Q.moe_expert_ffn(d, wts, x, torch.from_numpy(off.astype(np.int32)).to(dev()),
                     torch.from_numpy(perm.astype(np.int32)).to(dev()), y_perm, y_sh, ws)
    cache = ExpertCache(sh, lambda e: synth.expert_record(sh, 6, 0, e).numpy())
    xs = bf16_np(x)
    _, ref_yp = OM.expert_ffn_perm(xs, off, perm, sh.top_k, cache)
    assert_close(y_perm.cpu().numpy(), ref_yp, "real y_perm T=%d" % T)
    from tests._helpers import real_shared_np
    _, ref_ysh = OM.ffn(xs, *real_shared_np(lay))
    assert_close(y_sh.cpu().numpy(), ref_ysh, "shared_y T=%d" % T)


@pytest.mark.parametrize("T,Is", [(17, 64), (300, 64), (17, 192), (300, 192), (8192, 192),
                                  (17, 512), (300, 512), (8192, 512)])
def test_shared_expert_dense(T, Is):
    """The shared expert on the grouped-GEMM path (the dense bf16 kernel: up|gate
    with the SwiGLU in its epilogue, then down), every output row against the
    oracle's fp64 FFN; Is = 192 leaves the last 128-output tile half full, T =
    17 and 300 leave the last 128-row tile ragged.  (Not Is = 64 at 8192
    tokens: with 64 terms per output, a 1-ulp bf16 difference of one large
    activation -- the oracle rounds silu(g) u from fp64, the kernel from fp32
    -- moves that output by more than 1% of the rms, and among 25M outputs
    such an event occurs: measured 1.7% with rel L2 7.5e-5.)"""
    sh = synth.Shape(3072, 64, 8, 1, Is)
    lay = synth.real_layer(sh, 12, 0, zipf_s=0.0, device=dev())
    x = synth.tokens_bf16(T, sh.hidden, 12).to(dev())
    ids = np.zeros((T, 1), dtype=np.int64)
    off, perm, inv = OM.permute(ids, sh.n_experts)
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    wts = Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b, lay.shared_ug,
                    lay.shared_down)
    y_perm = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    y_sh = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev())
    ws = Q.workspace(d, T, dev())
    Q.moe_expert_ffn(d, wts, x, torch.from_numpy(off.astype(np.int32)).to(dev()),
                     torch.from_numpy(perm.astype(np.int32)).to(dev()), y_perm, y_sh, ws)
    from tests._helpers import real_shared_np
    _, ref_ysh = OM.ffn(bf16_np(x), *real_shared_np(lay))
    assert_close(y_sh.cpu().numpy(), ref_ysh, "dense shared expert T=%d Is=%d" % (T, Is))


# ---------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("H", [3072, 6144, 100, 1002])
def test_rmsnorm_residual(H):
    # H = 3072 and 6144: the register-resident float4 kernels (4 and 8 float4 a
    # thread); 100: a row shorter than the workgroup; 1002 (not a multiple of 4):
    # the general kernel.
    rng = np.random.default_rng(3)
    T = 5
    h = rng.normal(size=(T, H)).astype(np.float32)
    delta = rng.normal(size=(T, H)).astype(np.float32)
    gamma = (1 + 0.1 * rng.normal(size=H)).astype(np.float32)
    th = torch.from_numpy(h).to(dev())
    normed = torch.empty((T, H), dtype=torch.bfloat16, device=dev())
    Q.moe_rmsnorm_residual(th, torch.from_numpy(delta).to(dev()), torch.from_numpy(gamma).to(dev()),
                           1e-6, normed)
    hs = h.astype(np.float64) + delta
    assert np.array_equal(th.cpu().numpy(), (h + delta).astype(np.float32))
    ref = OM.rmsnorm_bf16(th.cpu().numpy().astype(np.float64), gamma, 1e-6)
    got = bf16_np(normed)
    # fp32 vs fp64 can flip a bf16 rounding on a few elements: at most one ulp
    diff = np.abs(got - ref)
    ulp = np.abs(ref) * 2.0 ** -7
    assert np.all(diff <= ulp + 1e-30)
    assert (diff > 0).sum() <= max(5, 0.01 * diff.size)
    assert_close(got, OM.rmsnorm_bf16(hs, gamma, 1e-6), "rmsnorm")
    # no residual: the normalisation of the summed row alone gives the same bits
    normed2 = torch.empty_like(normed)
    Q.moe_rmsnorm_residual(th, None, torch.from_numpy(gamma).to(dev()), 1e-6, normed2)
    assert torch.equal(normed2, normed)
    assert np.array_equal(th.cpu().numpy(), (h + delta).astype(np.float32))
