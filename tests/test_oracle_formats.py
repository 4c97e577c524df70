"""Pins of the oracle's weight codecs (CPU only).

The pages name the codecs and their bit rates only ("Qwen3.8-Flash-Next -
Avalon GGUF" model card, "Files / Main model"), so the codecs are pinned by
construction: hand-derived byte vectors and values (tests/golden), a library
routine for binary16, the stated codebook rule recomputed with scipy, the
scalar bit-by-bit decoder against the vectorised one, exactness in fp32, and
round trips / brute-force nearest for the quantisers.
"""

import json
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import formats as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "codec_known_answers.json")))


def _hex(b):
    return bytes(b).hex()


# ---------------------------------------------------------------- layouts

@pytest.mark.parametrize("case", GOLD["q3s_index_stream"])
def test_q3s_index_stream_known_answer(case):
    q = list(case["indices_first8"]) + [0] * 248
    blk = F.pack_q3s_block(0x3C00, [1] * 8, q)
    assert _hex(blk[:3]) == case["bytes_hex"]
    assert F.unpack_q3s_block(blk)[2][:8] == case["indices_first8"]
    # vectorised packer agrees byte for byte
    v = F.pack_q3s(np.array([0x3C00]), np.ones((1, 8)), np.array([q]))
    assert _hex(v[0][:3]) == case["bytes_hex"]


@pytest.mark.parametrize("case", GOLD["q3s_subscales"])
def test_q3s_subscale_known_answer(case):
    blk = F.pack_q3s_block(0x3C00, case["s"], [0] * 256)
    assert _hex(blk[98:102]) == case["bytes_hex"]
    assert blk[102:104] == b"\x00\x00"
    assert F.unpack_q3s_block(blk)[1] == case["s"]
    d, s, q = F.unpack_q3s(np.frombuffer(blk, dtype=np.uint8)[None])
    assert s[0].tolist() == case["s"]


def test_q3s_field_offsets():
    blk = F.pack_q3s_block(0xABCD, [0] * 8, [0] * 256)
    assert len(blk) == F.Q3S_BLOCK_BYTES == 104
    assert blk[96] == 0xCD and blk[97] == 0xAB
    # sub-block j's indices occupy bytes [12j, 12j+12)
    for j in range(8):
        q = [0] * 256
        for i in range(32):
            q[32 * j + i] = 7
        b = F.pack_q3s_block(0, [0] * 8, q)
        nz = [i for i, x in enumerate(b[:96]) if x]
        assert nz == list(range(12 * j, 12 * j + 12))


@pytest.mark.parametrize("case", GOLD["nl4_index_stream"])
def test_nl4_known_answer(case):
    q = list(case["indices_first2"]) + [0] * 30
    blk = F.pack_nl4_block(0x3C00, q)
    assert len(blk) == F.NL4_BLOCK_BYTES == 18
    assert blk[0] == 0x00 and blk[1] == 0x3C
    assert "%02x" % blk[2] == case["byte0_hex"]
    assert F.unpack_nl4_block(blk)[1][:2] == case["indices_first2"]


# ---------------------------------------------------------------- binary16

@pytest.mark.parametrize("case", GOLD["fp16"])
def test_fp16_known_values(case):
    assert F.fp16_bits_to_float(int(case["bits"], 16)) == case["value"]


def test_fp16_scalar_matches_library_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    lib = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536, 1):
        v = F.fp16_bits_to_float(b)
        if np.isnan(lib[b]):
            assert v != v
        else:
            assert v == lib[b], hex(b)


# ---------------------------------------------------------------- codebooks

def _nf_rule(bits):
    n = 2 ** bits
    p = 1.0 - 1.0 / (2 * n)
    pos = norm.ppf(np.linspace(0.5, p, n // 2 + 1))[1:]
    neg = -norm.ppf(np.linspace(0.5, p, n // 2))[1:]
    v = np.concatenate([neg[::-1], [0.0], pos]) / norm.ppf(p)
    return tuple(int(x) for x in np.rint(v * 127))


def test_codebooks_follow_stated_rule():
    assert F.Q3S_CODEBOOK == _nf_rule(3)
    assert F.NL4_TABLE == _nf_rule(4)
    for book in (F.Q3S_CODEBOOK, F.NL4_TABLE):
        assert list(book) == sorted(set(book))          # sorted, distinct
        assert 0 in book and all(-128 <= c <= 127 for c in book)
        neg = sum(1 for c in book if c < 0)
        assert neg == len(book) // 2 - 1                # asymmetric


# ---------------------------------------------------------------- dequant

@pytest.mark.parametrize("case", GOLD["q3s_values"])
def test_q3s_known_values(case):
    s = [case["s"]] * 8
    q = [case["q"]] * 256
    blk = F.pack_q3s_block(int(case["d_bits"], 16), s, q)
    vals = F.dequant_q3s_block(blk)
    assert all(v == case["value"] for v in vals)
    assert np.all(F.dequant_q3s(np.frombuffer(blk, np.uint8)[None]) == case["value"])


@pytest.mark.parametrize("case", GOLD["nl4_values"])
def test_nl4_known_values(case):
    blk = F.pack_nl4_block(int(case["d_bits"], 16), [case["q"]] * 32)
    assert all(v == case["value"] for v in F.dequant_nl4_block(blk))
    assert np.all(F.dequant_nl4(np.frombuffer(blk, np.uint8)[None]) == case["value"])


def test_q3s_every_index_and_subscale_position():
    # weight i of sub-block j gets index i % 8; sub-scales differ per j
    s = [-8, -1, 0, 1, 7, 2, -3, 5]
    q = [i % 8 for i in range(256)]
    blk = F.pack_q3s_block(0x3C00, s, q)
    vals = F.dequant_q3s_block(blk)
    for i in range(256):
        assert vals[i] == s[i // 32] * F.Q3S_CODEBOOK[i % 8] / 128.0


def _random_q3s_blocks(rng, n):
    raw = rng.integers(0, 256, size=(n, 104), dtype=np.uint8)
    # d: any finite binary16 (exponent field != 31), subnormals included
    d = rng.integers(0, 65536, size=n).astype(np.uint16)
    d = np.where((d & 0x7C00) == 0x7C00, d & 0x83FF, d).astype(np.uint16)
    raw[:, 96:98] = d[:, None].view(np.uint8).reshape(n, 2)
    raw[:, 102:104] = 0
    return raw


def test_vectorised_matches_scalar_q3s():
    rng = np.random.default_rng(11)
    raw = _random_q3s_blocks(rng, 64)
    vec = F.dequant_q3s(raw)
    d, s, q = F.unpack_q3s(raw)
    for b in range(raw.shape[0]):
        db, sb, qb = F.unpack_q3s_block(raw[b])
        assert qb == q[b].tolist() and sb == s[b].tolist()
        assert F.fp16_bits_to_float(db) == d[b]
        assert F.dequant_q3s_block(raw[b]) == vec[b].tolist()


def test_vectorised_matches_scalar_nl4():
    rng = np.random.default_rng(12)
    raw = rng.integers(0, 256, size=(64, 18), dtype=np.uint8)
    raw[:, 1] &= 0x7B            # keep d finite
    vec = F.dequant_nl4(raw)
    for b in range(raw.shape[0]):
        assert F.dequant_nl4_block(raw[b]) == vec[b].tolist()


def test_dequant_is_exact_in_fp32():
    # every dequantised value (|s*c| <= 1024, 11-bit d) is a float32 value
    rng = np.random.default_rng(13)
    vals = F.dequant_q3s(_random_q3s_blocks(rng, 2000))
    assert np.array_equal(vals.astype(np.float32).astype(np.float64), vals)
    raw = rng.integers(0, 256, size=(2000, 18), dtype=np.uint8)
    raw[:, 1] &= 0x7B
    v2 = F.dequant_nl4(raw)
    assert np.array_equal(v2.astype(np.float32).astype(np.float64), v2)


def test_packers_roundtrip_fields():
    rng = np.random.default_rng(14)
    n = 50
    d = rng.integers(0, 0x7C00, size=n).astype(np.uint16)
    s = rng.integers(-8, 8, size=(n, 8))
    q = rng.integers(0, 8, size=(n, 256))
    blk = F.pack_q3s(d, s, q)
    for b in range(n):
        assert bytes(blk[b]) == F.pack_q3s_block(int(d[b]), s[b].tolist(), q[b].tolist())
    d2, s2, q2 = F.unpack_q3s(blk)
    assert np.array_equal(s2, s) and np.array_equal(q2, q)
    q4 = rng.integers(0, 16, size=(n, 32))
    b4 = F.pack_nl4(d, q4)
    for b in range(n):
        assert bytes(b4[b]) == F.pack_nl4_block(int(d[b]), q4[b].tolist())


# ---------------------------------------------------------------- quantisers

def test_q3s_quantiser_on_grid_roundtrip():
    """Blocks built on the grid (max_j s_j = 7, s_j >= 1, each sub-block holding
    an extreme codebook entry) come back bit for bit, fields recovered."""
    rng = np.random.default_rng(21)
    for _ in range(40):
        d_bits = int(rng.integers(0x1000, 0x5000))
        d = F.fp16_bits_to_float(d_bits)
        s = rng.integers(1, 8, size=8)
        s[rng.integers(0, 8)] = 7
        q = rng.integers(0, 8, size=256)
        for j in range(8):
            q[32 * j + rng.integers(0, 32)] = rng.choice([0, 7])
        blk = F.pack_q3s_block(d_bits, s.tolist(), q.tolist())
        w = np.array(F.dequant_q3s_block(blk))
        # d must be recoverable: max sigma / 7 == d exactly here
        enc = F.quantize_q3s(w[None])[0]
        assert bytes(enc) == blk


def test_q3s_quantiser_is_nearest_brute_force():
    rng = np.random.default_rng(22)
    w = rng.normal(0, 0.02, size=(30, 256))
    enc = F.quantize_q3s(w)
    for b in range(w.shape[0]):
        d_bits, s, q = F.unpack_q3s_block(enc[b])
        d = F.fp16_bits_to_float(d_bits)
        absmax = [max(abs(v) for v in w[b, 32 * j:32 * j + 32]) for j in range(8)]
        sig = [a * 128.0 / 127.0 for a in absmax]
        assert d_bits == int(np.float16(max(sig) / 7.0).view(np.uint16))
        for j in range(8):
            assert s[j] == max(-8, min(7, int(np.rint(sig[j] / d))))
        for i in range(256):
            best = min(range(8), key=lambda c: (abs(w[b, i] - d * s[i // 32] * F.Q3S_CODEBOOK[c] / 128.0), c))
            assert q[i] == best


def test_nl4_quantiser_is_nearest_brute_force():
    rng = np.random.default_rng(23)
    w = rng.normal(0, 0.02, size=(60, 32))
    enc = F.quantize_nl4(w)
    for b in range(w.shape[0]):
        d_bits, q = F.unpack_nl4_block(enc[b])
        d = F.fp16_bits_to_float(d_bits)
        assert d_bits == int(np.float16(np.abs(w[b]).max() * 128.0 / 127.0).view(np.uint16))
        for i in range(32):
            best = min(range(16), key=lambda c: (abs(w[b, i] - d * F.NL4_TABLE[c] / 128.0), c))
            assert q[i] == best


def test_quantiser_ties_go_to_lower_index():
    # a weight exactly half-way between entries 3 (0) and 4 (23/128) with d=1, s=1
    w = np.zeros((1, 256))
    w[0, 0] = 127 / 128 * 7          # forces d*7 = max sigma -> d = 1.0 when s0 = 7
    w[0, 1] = 11.5 / 128 * 7         # midpoint of 0 and 23*7/128 in sub-block 0
    enc = F.quantize_q3s(w)[0]
    d_bits, s, q = F.unpack_q3s_block(enc)
    assert d_bits == 0x3C00 and s[0] == 7
    assert q[1] == 3
    # all-zero block: d = 0, s = 0, q = 0
    d0, s0, q0 = F.unpack_q3s_block(F.quantize_q3s(np.zeros((1, 256)))[0])
    assert d0 == 0 and s0 == [0] * 8 and q0 == [0] * 256


def test_matrix_helpers_and_expert_record():
    rng = np.random.default_rng(24)
    H, I = 256, 32
    wug = rng.normal(0, 0.02, size=(2 * I, H))
    wd = rng.normal(0, 0.02, size=(H, I))
    rec = np.concatenate([F.quantize_q3s_matrix(wug).reshape(-1),
                          F.quantize_nl4_matrix(wd).reshape(-1)])
    assert rec.size == F.expert_record_bytes(H, I) == 2 * I * 104 + H * 18
    up, gate, down = F.expert_matrices(rec, H, I)
    up2, gate2, down2 = F.expert_matrices_scalar(rec, H, I)
    assert np.array_equal(up, up2) and np.array_equal(gate, gate2) and np.array_equal(down, down2)
    # quantisation error is small relative to the weights (RTN sanity)
    assert np.abs(np.concatenate([up, gate]) - wug).max() < 0.25 * np.abs(wug).max()
