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


# ---------------------------------------------------------------- the 2-bit codecs
# (mixed-format layers of the same model card: up/gate IQ2_S, down Q2_0; the
# layouts are readings, pinned by construction like the two codecs above)

@pytest.mark.parametrize("case", GOLD["q2s_index_stream"])
def test_q2s_index_stream_known_answer(case):
    q = list(case["indices_first8"]) + [0] * 248
    blk = F.pack_q2s_block(0, [0] * 8, q)
    assert _hex(blk[:2]) == case["bytes_hex"]
    assert F.unpack_q2s_block(blk)[2][:8] == case["indices_first8"]


@pytest.mark.parametrize("case", GOLD["q2s_fields"])
def test_q2s_field_offsets(case):
    blk = F.pack_q2s_block(int(case["d_bits"], 16), case["s"], [0] * 256)
    assert len(blk) == F.Q2S_BLOCK_BYTES == 80
    assert _hex(blk[64:80]) == case["bytes_64_80_hex"]
    d_bits, s, _ = F.unpack_q2s_block(blk)
    assert d_bits == int(case["d_bits"], 16) and s == case["s"]


@pytest.mark.parametrize("case", GOLD["q2s_values"])
def test_q2s_known_values(case):
    blk = F.pack_q2s_block(int(case["d_bits"], 16), [case["s"]] * 8, [case["q"]] * 256)
    assert all(v == case["value"] for v in F.dequant_q2s_block(blk))
    assert np.all(F.dequant_q2s(np.frombuffer(blk, np.uint8)[None]) == case["value"])


@pytest.mark.parametrize("case", GOLD["q2_index_stream"])
def test_q2_index_stream_known_answer(case):
    blk = F.pack_q2_block(0, list(case["indices_first4"]) + [0] * 28)
    assert len(blk) == F.Q2_BLOCK_BYTES == 10
    assert _hex(blk[2:3]) == case["byte2_hex"]


@pytest.mark.parametrize("case", GOLD["q2_values"])
def test_q2_known_values(case):
    blk = F.pack_q2_block(int(case["d_bits"], 16), [case["q"]] * 32)
    assert all(v == case["value"] for v in F.dequant_q2_block(blk))
    assert np.all(F.dequant_q2(np.frombuffer(blk, np.uint8)[None]) == case["value"])


def test_q2s_codebook_follows_stated_rule():
    assert F.Q2S_CODEBOOK == _nf_rule(2)
    book = F.Q2S_CODEBOOK
    assert list(book) == sorted(set(book)) and 0 in book
    assert sum(1 for c in book if c < 0) == len(book) // 2 - 1


def test_q2s_every_index_and_subscale_position():
    s = [-8, -1, 0, 1, 7, 2, -3, 5]
    q = [(i * 7 + i // 32) % 4 for i in range(256)]
    blk = F.pack_q2s_block(0x3C00, s, q)
    vals = F.dequant_q2s_block(blk)
    for i in range(256):
        assert vals[i] == s[i // 32] * F.Q2S_CODEBOOK[q[i]] / 128.0


def test_q2_every_position():
    q = [(5 * i + 1) % 4 for i in range(32)]
    vals = F.dequant_q2_block(F.pack_q2_block(0x3800, q))
    assert vals == [0.5 * (qi - 2) for qi in q]


def _random_q2s_blocks(rng, n):
    blk = rng.integers(0, 256, size=(n, F.Q2S_BLOCK_BYTES), dtype=np.uint8)
    blk[:, 65] = (blk[:, 65] & 0x83) | 0x20          # finite d of either sign
    return blk


def test_vectorised_matches_scalar_q2s():
    rng = np.random.default_rng(11)
    blocks = _random_q2s_blocks(rng, 40)
    vec = F.dequant_q2s(blocks)
    for b in range(len(blocks)):
        assert list(vec[b]) == F.dequant_q2s_block(bytes(blocks[b]))
        d_bits, s, q = F.unpack_q2s_block(bytes(blocks[b]))
        d2, s2, q2 = F.unpack_q2s(blocks[b][None])
        assert list(s2[0]) == s and list(q2[0]) == q


def test_vectorised_matches_scalar_q2():
    rng = np.random.default_rng(12)
    blocks = rng.integers(0, 256, size=(60, F.Q2_BLOCK_BYTES), dtype=np.uint8)
    blocks[:, 1] = (blocks[:, 1] & 0x83) | 0x28
    vec = F.dequant_q2(blocks)
    for b in range(len(blocks)):
        assert list(vec[b]) == F.dequant_q2_block(bytes(blocks[b]))


def test_2bit_dequant_is_exact_in_fp32():
    rng = np.random.default_rng(13)
    for v in F.dequant_q2s(_random_q2s_blocks(rng, 30)).ravel():
        assert float(np.float32(v)) == v
    blocks = rng.integers(0, 256, size=(30, F.Q2_BLOCK_BYTES), dtype=np.uint8)
    for v in F.dequant_q2(blocks).ravel():
        if np.isfinite(v):
            assert float(np.float32(v)) == v


def test_2bit_packers_roundtrip_fields():
    rng = np.random.default_rng(14)
    d = rng.integers(0, 0x7C00, size=5).astype(np.uint16)
    s = rng.integers(-8, 8, size=(5, 8))
    q = rng.integers(0, 4, size=(5, 256))
    vec = F.pack_q2s(d, s, q)
    for b in range(5):
        assert bytes(vec[b]) == F.pack_q2s_block(int(d[b]), list(s[b]), list(q[b]))
    q2 = rng.integers(0, 4, size=(5, 32))
    vec2 = F.pack_q2(d, q2)
    for b in range(5):
        assert bytes(vec2[b]) == F.pack_q2_block(int(d[b]), list(q2[b]))
        assert F.unpack_q2_block(bytes(vec2[b])) == (int(d[b]), list(q2[b]))


def test_q2s_quantiser_on_grid_roundtrip():
    """Weights on the grid of one block (d, s fixed; each sub-block holds the
    largest codebook entry so the rule recovers s) come back bit for bit."""
    d_bits = 0x2400
    d = float(np.uint16(d_bits).view(np.float16))
    s = [7, 3, 1, 7, 5, 2, 6, 4]
    rng = np.random.default_rng(15)
    q = rng.integers(0, 4, size=256)
    q[::32] = 3
    w = np.array([d * s[i // 32] * F.Q2S_CODEBOOK[q[i]] / 128.0 for i in range(256)])
    blk = F.quantize_q2s(w)
    d2, s2, q2 = F.unpack_q2s_block(bytes(blk))
    assert (d2, s2, q2) == (d_bits, s, list(q))


def test_q2s_quantiser_is_nearest_brute_force():
    rng = np.random.default_rng(16)
    w = rng.normal(0, 0.02, size=(6, 256))
    blks = F.quantize_q2s(w)
    for b in range(6):
        d_bits, s, q = F.unpack_q2s_block(bytes(blks[b]))
        d = F.fp16_bits_to_float(d_bits)
        for i in range(256):
            lv = [d * s[i // 32] * c / 128.0 for c in F.Q2S_CODEBOOK]
            best = min(range(4), key=lambda t: (abs(w[b, i] - lv[t]), t))
            assert q[i] == best


def test_q2_quantiser_is_nearest_brute_force():
    rng = np.random.default_rng(17)
    w = rng.normal(0, 0.02, size=(8, 32))
    blks = F.quantize_q2(w)
    for b in range(8):
        d_bits, q = F.unpack_q2_block(bytes(blks[b]))
        d = F.fp16_bits_to_float(d_bits)
        assert d_bits == int(np.float16(np.abs(w[b]).max() / 2).view(np.uint16))
        for i in range(32):
            best = min(range(4), key=lambda t: (abs(w[b, i] - d * (t - 2)), t))
            assert q[i] == best


@pytest.mark.parametrize("ug,dn", [(F.FMT_Q2S256, F.FMT_Q2_32), (F.FMT_NL4_32, F.FMT_NL4_32),
                                   (F.FMT_Q3S256, F.FMT_Q2_32)])
def test_mixed_expert_record(ug, dn):
    """Record layout for other format pairs: up|gate then down; the matrix
    helpers agree with the scalar block decoders."""
    H, I = 256, 64
    rng = np.random.default_rng(18)
    wug = rng.normal(0, 0.02, size=(2 * I, H))
    wdn = rng.normal(0, 0.02, size=(H, I))
    rec = np.concatenate([F.quantize_matrix(ug, wug).ravel(), F.quantize_matrix(dn, wdn).ravel()])
    assert rec.size == F.expert_record_bytes(H, I, ug, dn)
    a = F.expert_matrices(rec, H, I, ug, dn)
    b = F.expert_matrices_scalar(rec, H, I, ug, dn)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert np.array_equal(np.concatenate([a[0], a[1]]), F.dequant_matrix(ug, F.quantize_matrix(ug, wug), 2 * I, H))


# ---------------------------------------------------------------- the 6-bit sub-scaled codecs
# (the model card's IQ3_K and IQ4_XS up/gate names, "Files / Main model", and
# the draft head's IQ3_K experts, "MTP sidecar"; the layouts are readings,
# pinned by construction like the codecs above)

def test_q3k_and_nl4s_block_sizes_give_the_stated_bit_rates():
    assert F.Q3K_BLOCK_BYTES * 8 / 256 == 3.4375         # "3.44 bpw"
    assert F.NL4S_BLOCK_BYTES * 8 / 256 == 4.25


@pytest.mark.parametrize("case", GOLD["q3k_fields"])
def test_q3k_field_offsets(case):
    blk = F.pack_q3k_block(int(case["d_bits"], 16), case["s"], [0] * 256)
    assert len(blk) == F.Q3K_BLOCK_BYTES
    assert _hex(blk[96:110]) == case["bytes_96_110_hex"]
    d_bits, s, q = F.unpack_q3k_block(blk)
    assert d_bits == int(case["d_bits"], 16) and s == case["s"] and q == [0] * 256


@pytest.mark.parametrize("case", GOLD["q3s_index_stream"])
def test_q3k_index_stream_is_the_q3s_stream(case):
    q = list(case["indices_first8"]) + [0] * 248
    blk = F.pack_q3k_block(0, [0] * 16, q)
    assert _hex(blk[:3]) == case["bytes_hex"]
    assert F.unpack_q3k_block(blk)[2][:8] == case["indices_first8"]


@pytest.mark.parametrize("case", GOLD["q3k_values"])
def test_q3k_known_values(case):
    blk = F.pack_q3k_block(int(case["d_bits"], 16), [case["s"]] * 16, [case["q"]] * 256)
    assert all(v == case["value"] for v in F.dequant_q3k_block(blk))
    assert np.all(F.dequant_q3k(np.frombuffer(blk, np.uint8)[None]) == case["value"])


@pytest.mark.parametrize("case", GOLD["nl4s_fields"])
def test_nl4s_field_offsets(case):
    q = list(case["indices_first4"]) + [0] * 252
    blk = F.pack_nl4s_block(int(case["d_bits"], 16), case["s"], q)
    assert len(blk) == F.NL4S_BLOCK_BYTES
    assert _hex(blk[0:2]) == case["bytes_0_2_hex"]
    assert _hex(blk[128:136]) == case["bytes_128_136_hex"]
    d_bits, s, q2 = F.unpack_nl4s_block(blk)
    assert d_bits == int(case["d_bits"], 16) and s == case["s"] and q2 == q


@pytest.mark.parametrize("case", GOLD["nl4s_values"])
def test_nl4s_known_values(case):
    blk = F.pack_nl4s_block(int(case["d_bits"], 16), [case["s"]] * 8, [case["q"]] * 256)
    assert all(v == case["value"] for v in F.dequant_nl4s_block(blk))
    assert np.all(F.dequant_nl4s(np.frombuffer(blk, np.uint8)[None]) == case["value"])


def test_q3k_every_index_and_subscale_position():
    s = [-32, 31, -1, 0, 1, 17, -17, 5, -5, 9, 30, -31, 2, -2, 12, -12]
    q = [(i * 5 + i // 16) % 8 for i in range(256)]
    vals = F.dequant_q3k_block(F.pack_q3k_block(0x3C00, s, q))
    for i in range(256):
        assert vals[i] == s[i // 16] * F.Q3S_CODEBOOK[q[i]] / 128.0


def test_nl4s_every_index_and_subscale_position():
    s = [-32, 31, -1, 0, 1, 17, -17, 5]
    q = [(i * 7 + i // 32) % 16 for i in range(256)]
    vals = F.dequant_nl4s_block(F.pack_nl4s_block(0x3C00, s, q))
    for i in range(256):
        assert vals[i] == s[i // 32] * F.NL4_TABLE[q[i]] / 128.0


def _random_blocks(rng, n, nbytes, d_hi):
    blk = rng.integers(0, 256, size=(n, nbytes), dtype=np.uint8)
    blk[:, d_hi] = (blk[:, d_hi] & 0x83) | (rng.integers(0, 30, size=n, dtype=np.uint8) << 2)
    return blk                                         # finite d of either sign, subnormals included


def test_vectorised_matches_scalar_q3k_nl4s():
    rng = np.random.default_rng(21)
    for nb, d_hi, deq, deq_blk, unp_blk, unp in (
            (F.Q3K_BLOCK_BYTES, 97, F.dequant_q3k, F.dequant_q3k_block, F.unpack_q3k_block, F.unpack_q3k),
            (F.NL4S_BLOCK_BYTES, 129, F.dequant_nl4s, F.dequant_nl4s_block, F.unpack_nl4s_block,
             F.unpack_nl4s)):
        blocks = _random_blocks(rng, 40, nb, d_hi)
        vec = deq(blocks)
        for b in range(len(blocks)):
            assert list(vec[b]) == deq_blk(bytes(blocks[b]))
            _, s, q = unp_blk(bytes(blocks[b]))
            _, s2, q2 = unp(blocks[b][None])
            assert list(s2[0]) == s and list(q2[0]) == q


def test_q3k_nl4s_dequant_is_exact_in_fp32():
    rng = np.random.default_rng(22)
    for v in F.dequant_q3k(_random_blocks(rng, 30, F.Q3K_BLOCK_BYTES, 97)).ravel():
        assert float(np.float32(v)) == v
    for v in F.dequant_nl4s(_random_blocks(rng, 30, F.NL4S_BLOCK_BYTES, 129)).ravel():
        assert float(np.float32(v)) == v


def test_q3k_nl4s_packers_roundtrip_fields():
    rng = np.random.default_rng(23)
    d = rng.integers(0, 0x7C00, size=5).astype(np.uint16)
    s16 = rng.integers(-32, 32, size=(5, 16))
    s8 = rng.integers(-32, 32, size=(5, 8))
    q8 = rng.integers(0, 8, size=(5, 256))
    q16 = rng.integers(0, 16, size=(5, 256))
    v3 = F.pack_q3k(d, s16, q8)
    v4 = F.pack_nl4s(d, s8, q16)
    for b in range(5):
        assert bytes(v3[b]) == F.pack_q3k_block(int(d[b]), list(s16[b]), list(q8[b]))
        assert F.unpack_q3k_block(bytes(v3[b])) == (int(d[b]), list(s16[b]), list(q8[b]))
        assert bytes(v4[b]) == F.pack_nl4s_block(int(d[b]), list(s8[b]), list(q16[b]))
        assert F.unpack_nl4s_block(bytes(v4[b])) == (int(d[b]), list(s8[b]), list(q16[b]))


@pytest.mark.parametrize("fmt", [F.FMT_Q3K256, F.FMT_NL4S256])
def test_subscaled_quantiser_on_grid_roundtrip(fmt):
    """Weights on one block's grid (largest sub-scale 31, every sub-block
    holding the largest-magnitude entry so the rule recovers its sub-scale)
    come back bit for bit."""
    sub, book = (16, F.Q3S_CODEBOOK) if fmt == F.FMT_Q3K256 else (32, F.NL4_TABLE)
    ns = 256 // sub
    d_bits = 0x2400
    d = float(np.uint16(d_bits).view(np.float16))
    rng = np.random.default_rng(24)
    s = list(rng.integers(1, 32, size=ns))
    s[3] = 31
    q = rng.integers(0, len(book), size=256)
    q[::sub] = 0                                          # book[0] = -127: the largest magnitude
    w = np.array([d * s[i // sub] * book[q[i]] / 128.0 for i in range(256)])
    blk = F.CODECS[fmt][4](w)
    unp = F.unpack_q3k_block if fmt == F.FMT_Q3K256 else F.unpack_nl4s_block
    d2, s2, q2 = unp(bytes(blk))
    assert (d2, s2, q2) == (d_bits, [int(v) for v in s], list(q))


@pytest.mark.parametrize("fmt", [F.FMT_Q3K256, F.FMT_NL4S256])
def test_subscaled_quantiser_is_nearest_brute_force(fmt):
    sub, book = (16, F.Q3S_CODEBOOK) if fmt == F.FMT_Q3K256 else (32, F.NL4_TABLE)
    unp = F.unpack_q3k_block if fmt == F.FMT_Q3K256 else F.unpack_nl4s_block
    rng = np.random.default_rng(25)
    w = rng.normal(0, 0.02, size=(4, 256))
    blks = F.CODECS[fmt][4](w)
    for b in range(4):
        d_bits, s, q = unp(bytes(blks[b]))
        d = F.fp16_bits_to_float(d_bits)
        sigma_max = max(np.abs(w[b, j * sub:(j + 1) * sub]).max() for j in range(256 // sub)) / (127 / 128)
        assert d_bits == int(np.float16(sigma_max / 31).view(np.uint16))
        for i in range(256):
            lv = [d * s[i // sub] * c / 128.0 for c in book]
            best = min(range(len(book)), key=lambda t: (abs(w[b, i] - lv[t]), t))
            assert q[i] == best


@pytest.mark.parametrize("ug", [F.FMT_Q3K256, F.FMT_NL4S256])
def test_subscaled_expert_record(ug):
    """Records with the 6-bit sub-scaled up|gate codecs (and NL4-32 down, as
    the draft head's experts): the matrix helpers agree with the scalar block
    decoders."""
    H, I = 256, 64
    rng = np.random.default_rng(26)
    wug = rng.normal(0, 0.02, size=(2 * I, H))
    wdn = rng.normal(0, 0.02, size=(H, I))
    rec = np.concatenate([F.quantize_matrix(ug, wug).ravel(),
                          F.quantize_matrix(F.FMT_NL4_32, wdn).ravel()])
    assert rec.size == F.expert_record_bytes(H, I, ug, F.FMT_NL4_32)
    a = F.expert_matrices(rec, H, I, ug, F.FMT_NL4_32)
    b = F.expert_matrices_scalar(rec, H, I, ug, F.FMT_NL4_32)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
