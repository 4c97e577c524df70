"""Expert weight codecs of the oracle: scalar and vectorised unpack/dequant,
packers for hand-built blocks, and the round-to-nearest quantisers that build
test data.  Test infrastructure: see the package header for who may use it.

Source: "Qwen3.8-Flash-Next - Avalon GGUF" model card, "Files / Main model":
routed up/gate tensors use a 3.25-bpw type with a scale per 256-weight block
and sub-scales per 32 weights; routed down tensors use a 4-bit non-linear type
(IQ4_NL, 32-weight blocks); each expert is stored as up | gate | down,
contiguous.  The page gives names and bit rates only.  Readings taken here
(each is repeated in the repository's design notes):

Q3S-256 block (256 weights, 104 bytes = 3.25 bits per weight)
  bytes [0, 96)   256 three-bit codebook indices as one little-endian bit
                  stream: weight i occupies stream bits 3i .. 3i+2, bit 0 of
                  the stream being bit 0 of byte 0.  Sub-block j (weights
                  32j .. 32j+31) is therefore bytes [12j, 12j+12).
  bytes [96, 98)  d, IEEE binary16, little-endian.  Any finite value,
                  subnormals included.
  bytes [98, 102) eight signed 4-bit sub-scales: bytes 98..101 read as a
                  little-endian u32 V; s_j is bits 4j .. 4j+3 of V taken as a
                  two's-complement nibble, so s_j is in [-8, 7].
  bytes [102,104) reserved: writers store 0, readers ignore.
  value of weight i = d * s_{i // 32} * C3[q_i] / 128  (exact in fp32).

NL4-32 block (32 weights, 18 bytes = 4.5 bits per weight)
  bytes [0, 2)    d, IEEE binary16, little-endian.
  bytes [2, 18)   32 four-bit indices, weight i at bits 4i .. 4i+3 of the
                  little-endian stream (even i in the low nibble).
  value of weight i = d * T4[q_i] / 128  (exact in fp32).

Codebooks: sorted, distinct int8 levels placed at normal quantiles
("NF"-style), asymmetric with an exact zero: for a b-bit book with n = 2^b
entries, p = 1 - 1/(2n); the n/2 positive levels are Phi^-1 at
linspace(0.5, p, n/2 + 1)[1:], the n/2 - 1 negative levels are -Phi^-1 at
linspace(0.5, p, n/2)[1:], all divided by Phi^-1(p), times 127, rounded to
the nearest integer.  The literals below are that rule's output, frozen.

Matrix orientation: a weight matrix is stored as [out rows][in], blocks running
along the reduction (input) dimension, so one block scale serves one dot
product.  An expert record is up|gate = [2I][H] (rows 0..I-1 up, I..2I-1 gate)
in Q3S-256, then down = [H][I] in NL4-32.
"""

import numpy as np

Q3S_BLOCK_WEIGHTS = 256
Q3S_BLOCK_BYTES = 104
Q3S_SUB_WEIGHTS = 32
NL4_BLOCK_WEIGHTS = 32
NL4_BLOCK_BYTES = 18

# 8-entry codebook of the 3.25-bpw up/gate codec (value = entry / 128).
Q3S_CODEBOOK = (-127, -67, -31, 0, 23, 48, 78, 127)
# 16-entry non-linear table of the 4-bit down codec (value = entry / 128).
NL4_TABLE = (-127, -88, -66, -50, -36, -23, -11, 0, 10, 20, 31, 43, 56, 71, 91, 127)


# --------------------------------------------------------------------------
# binary16, scalar definition (IEEE 754: 1 sign, 5 exponent, 10 fraction bits)
# --------------------------------------------------------------------------

def fp16_bits_to_float(bits):
    """Value of a binary16 bit pattern, as a Python float (exact)."""
    bits = int(bits) & 0xFFFF
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * m * 2.0 ** -24
    return sign * (1024 + m) * 2.0 ** (e - 25)


# --------------------------------------------------------------------------
# scalar (pure Python) codecs: one block at a time, bit by bit
# --------------------------------------------------------------------------

def _bit_stream(data):
    """Little-endian bit stream of a byte string: list of 0/1."""
    out = []
    for byte in data:
        for b in range(8):
            out.append((byte >> b) & 1)
    return out


def unpack_q3s_block(block):
    """Fields of one 104-byte Q3S-256 block: (d_bits, s[8], q[256])."""
    block = bytes(block)
    if len(block) != Q3S_BLOCK_BYTES:
        raise ValueError("Q3S-256 block must be 104 bytes")
    bits = _bit_stream(block[0:96])
    q = []
    for i in range(Q3S_BLOCK_WEIGHTS):
        q.append(bits[3 * i] | (bits[3 * i + 1] << 1) | (bits[3 * i + 2] << 2))
    d_bits = block[96] | (block[97] << 8)
    v = block[98] | (block[99] << 8) | (block[100] << 16) | (block[101] << 24)
    s = []
    for j in range(8):
        nib = (v >> (4 * j)) & 0xF
        s.append(nib - 16 if nib >= 8 else nib)
    return d_bits, s, q


def dequant_q3s_block(block):
    """256 weight values of one Q3S-256 block (Python floats, exact)."""
    d_bits, s, q = unpack_q3s_block(block)
    d = fp16_bits_to_float(d_bits)
    return [d * s[i // Q3S_SUB_WEIGHTS] * Q3S_CODEBOOK[q[i]] / 128.0
            for i in range(Q3S_BLOCK_WEIGHTS)]


def pack_q3s_block(d_bits, s, q):
    """Bytes of one Q3S-256 block from its fields (reserved bytes zero)."""
    if len(s) != 8 or len(q) != Q3S_BLOCK_WEIGHTS:
        raise ValueError("need 8 sub-scales and 256 indices")
    stream = 0
    for i, qi in enumerate(q):
        if not 0 <= qi < 8:
            raise ValueError("index out of range")
        stream |= int(qi) << (3 * i)
    out = bytearray(stream.to_bytes(96, "little"))
    out += bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])
    v = 0
    for j, sj in enumerate(s):
        if not -8 <= sj <= 7:
            raise ValueError("sub-scale out of range")
        v |= (int(sj) & 0xF) << (4 * j)
    out += v.to_bytes(4, "little")
    out += b"\x00\x00"
    return bytes(out)


def unpack_nl4_block(block):
    """Fields of one 18-byte NL4-32 block: (d_bits, q[32])."""
    block = bytes(block)
    if len(block) != NL4_BLOCK_BYTES:
        raise ValueError("NL4-32 block must be 18 bytes")
    d_bits = block[0] | (block[1] << 8)
    bits = _bit_stream(block[2:18])
    q = []
    for i in range(NL4_BLOCK_WEIGHTS):
        q.append(bits[4 * i] | (bits[4 * i + 1] << 1) | (bits[4 * i + 2] << 2)
                 | (bits[4 * i + 3] << 3))
    return d_bits, q


def dequant_nl4_block(block):
    """32 weight values of one NL4-32 block (Python floats, exact)."""
    d_bits, q = unpack_nl4_block(block)
    d = fp16_bits_to_float(d_bits)
    return [d * NL4_TABLE[qi] / 128.0 for qi in q]


def pack_nl4_block(d_bits, q):
    """Bytes of one NL4-32 block from its fields."""
    if len(q) != NL4_BLOCK_WEIGHTS:
        raise ValueError("need 32 indices")
    stream = 0
    for i, qi in enumerate(q):
        if not 0 <= qi < 16:
            raise ValueError("index out of range")
        stream |= int(qi) << (4 * i)
    return bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF]) + stream.to_bytes(16, "little")


# --------------------------------------------------------------------------
# vectorised (NumPy) codecs; pinned bit-exactly against the scalar ones
# --------------------------------------------------------------------------

def _as_blocks(arr, nbytes):
    a = np.ascontiguousarray(arr, dtype=np.uint8)
    if a.shape[-1] != nbytes:
        a = a.reshape(a.shape[:-1] + (-1, nbytes))
    return a


def unpack_q3s(arr):
    """Vectorised Q3S-256 unpack.  arr: uint8 [..., 104] (or [..., n*104]).

    Returns (d float64 [...], s int64 [..., 8], q int64 [..., 256])."""
    a = _as_blocks(arr, Q3S_BLOCK_BYTES)
    bits = np.unpackbits(a[..., 0:96], axis=-1, bitorder="little")
    bits = bits.reshape(a.shape[:-1] + (Q3S_BLOCK_WEIGHTS, 3)).astype(np.int64)
    q = bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)
    d = np.ascontiguousarray(a[..., 96:98]).view("<f2")[..., 0].astype(np.float64)
    v = np.ascontiguousarray(a[..., 98:102]).view("<u4")[..., 0].astype(np.int64)
    s = np.stack([(v >> (4 * j)) & 0xF for j in range(8)], axis=-1)
    s = np.where(s >= 8, s - 16, s)
    return d, s, q


def dequant_q3s(arr):
    """Vectorised Q3S-256 dequant: float64 [..., 256] per block."""
    d, s, q = unpack_q3s(arr)
    c = np.asarray(Q3S_CODEBOOK, dtype=np.float64)[q]
    sw = np.repeat(s, Q3S_SUB_WEIGHTS, axis=-1).astype(np.float64)
    return d[..., None] * sw * c / 128.0


def unpack_nl4(arr):
    """Vectorised NL4-32 unpack: (d float64 [...], q int64 [..., 32])."""
    a = _as_blocks(arr, NL4_BLOCK_BYTES)
    d = np.ascontiguousarray(a[..., 0:2]).view("<f2")[..., 0].astype(np.float64)
    b = a[..., 2:18].astype(np.int64)
    q = np.stack([b & 0xF, b >> 4], axis=-1).reshape(a.shape[:-1] + (NL4_BLOCK_WEIGHTS,))
    return d, q


def dequant_nl4(arr):
    """Vectorised NL4-32 dequant: float64 [..., 32] per block."""
    d, q = unpack_nl4(arr)
    t = np.asarray(NL4_TABLE, dtype=np.float64)[q]
    return d[..., None] * t / 128.0


def dequant_q3s_matrix(raw, rows, cols):
    """Dequantise a Q3S-256 matrix stored [rows][cols] (cols % 256 == 0)."""
    nb = cols // Q3S_BLOCK_WEIGHTS
    a = np.asarray(raw, dtype=np.uint8).reshape(rows, nb, Q3S_BLOCK_BYTES)
    return dequant_q3s(a).reshape(rows, cols)


def dequant_nl4_matrix(raw, rows, cols):
    """Dequantise an NL4-32 matrix stored [rows][cols] (cols % 32 == 0)."""
    nb = cols // NL4_BLOCK_WEIGHTS
    a = np.asarray(raw, dtype=np.uint8).reshape(rows, nb, NL4_BLOCK_BYTES)
    return dequant_nl4(a).reshape(rows, cols)


def pack_q3s(d_bits, s, q):
    """Vectorised pack: d_bits uint16 [...], s int [..., 8], q int [..., 256]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    s = np.asarray(s, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    lead = d_bits.shape
    out = np.zeros(lead + (Q3S_BLOCK_BYTES,), dtype=np.uint8)
    bits = np.stack([(q >> b) & 1 for b in range(3)], axis=-1).reshape(lead + (768,))
    out[..., 0:96] = np.packbits(bits.astype(np.uint8), axis=-1, bitorder="little")
    out[..., 96:98] = d_bits[..., None].view(np.uint8).reshape(lead + (2,))
    v = np.zeros(lead, dtype=np.uint32)
    for j in range(8):
        v |= ((s[..., j] & 0xF).astype(np.uint32) << np.uint32(4 * j))
    out[..., 98:102] = v.astype("<u4")[..., None].view(np.uint8).reshape(lead + (4,))
    return out


def pack_nl4(d_bits, q):
    """Vectorised pack: d_bits uint16 [...], q int [..., 32]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    q = np.asarray(q, dtype=np.int64)
    lead = d_bits.shape
    out = np.zeros(lead + (NL4_BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0:2] = d_bits[..., None].view(np.uint8).reshape(lead + (2,))
    out[..., 2:18] = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    return out


# --------------------------------------------------------------------------
# round-to-nearest quantisers (test data only)
# --------------------------------------------------------------------------

def _fp16_rne_bits(x):
    """binary16 round-to-nearest-even bit patterns of float64 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def quantize_q3s(w):
    """Round-to-nearest Q3S-256 encoding of weights w [..., 256] (any float).

    Per block: sigma_j = absmax of sub-block j divided by max|C3|/128;
    d = fp16_RNE(max_j sigma_j / 7); s_j = clamp(round_half_even(sigma_j / d),
    -8, 7); each q_i = the codebook index minimising |w_i - d*s_j*C3[q]/128|,
    ties to the lower index.  A block whose d rounds to zero gets s = q = 0.
    Returns uint8 [..., 104]."""
    w = np.asarray(w, dtype=np.float64)
    lead = w.shape[:-1]
    sub = w.reshape(lead + (8, Q3S_SUB_WEIGHTS))
    cmax = max(abs(c) for c in Q3S_CODEBOOK) / 128.0
    sigma = np.abs(sub).max(axis=-1) / cmax
    d_bits = _fp16_rne_bits(sigma.max(axis=-1) / 7.0)
    d = d_bits.view(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(d[..., None] > 0, np.rint(sigma / d[..., None]), 0.0)
    s = np.clip(s, -8, 7).astype(np.int64)
    cands = (d[..., None, None] * s[..., None].astype(np.float64)
             * np.asarray(Q3S_CODEBOOK, dtype=np.float64) / 128.0)   # [..., 8 sub, 8 cand]
    dist = np.abs(sub[..., None] - cands[..., None, :])                # [..., 8, 32, 8]
    q = np.argmin(dist, axis=-1).reshape(lead + (Q3S_BLOCK_WEIGHTS,))
    return pack_q3s(d_bits, s, q)


def quantize_nl4(w):
    """Round-to-nearest NL4-32 encoding of weights w [..., 32].

    d = fp16_RNE(absmax / (max|T4|/128)); q_i = the table index minimising
    |w_i - d*T4[q]/128|, ties to the lower index.  Returns uint8 [..., 18]."""
    w = np.asarray(w, dtype=np.float64)
    tmax = max(abs(t) for t in NL4_TABLE) / 128.0
    d_bits = _fp16_rne_bits(np.abs(w).max(axis=-1) / tmax)
    d = d_bits.view(np.float16).astype(np.float64)
    cands = d[..., None] * np.asarray(NL4_TABLE, dtype=np.float64) / 128.0
    q = np.argmin(np.abs(w[..., None] - cands[..., None, :]), axis=-1)
    return pack_nl4(d_bits, q)


def quantize_q3s_matrix(w):
    """Quantise a matrix [rows][cols] (cols % 256 == 0) to Q3S-256 bytes
    [rows][cols/256*104]."""
    w = np.asarray(w, dtype=np.float64)
    rows, cols = w.shape
    blk = quantize_q3s(w.reshape(rows, cols // Q3S_BLOCK_WEIGHTS, Q3S_BLOCK_WEIGHTS))
    return blk.reshape(rows, -1)


def quantize_nl4_matrix(w):
    """Quantise a matrix [rows][cols] (cols % 32 == 0) to NL4-32 bytes
    [rows][cols/32*18]."""
    w = np.asarray(w, dtype=np.float64)
    rows, cols = w.shape
    blk = quantize_nl4(w.reshape(rows, cols // NL4_BLOCK_WEIGHTS, NL4_BLOCK_WEIGHTS))
    return blk.reshape(rows, -1)


# --------------------------------------------------------------------------
# expert records: up|gate (Q3S-256, [2I][H]) then down (NL4-32, [H][I])
# --------------------------------------------------------------------------

def upgate_bytes(hidden, inter):
    return 2 * inter * (hidden // Q3S_BLOCK_WEIGHTS) * Q3S_BLOCK_BYTES


def down_bytes(hidden, inter):
    return hidden * (inter // NL4_BLOCK_WEIGHTS) * NL4_BLOCK_BYTES


def expert_record_bytes(hidden, inter):
    return upgate_bytes(hidden, inter) + down_bytes(hidden, inter)


def expert_matrices(record, hidden, inter):
    """Dequantised (W_up [I][H], W_gate [I][H], W_down [H][I]) of one packed
    expert record (uint8, length >= expert_record_bytes)."""
    rec = np.asarray(record, dtype=np.uint8).reshape(-1)
    nug = upgate_bytes(hidden, inter)
    ug = dequant_q3s_matrix(rec[:nug], 2 * inter, hidden)
    dn = dequant_nl4_matrix(rec[nug:nug + down_bytes(hidden, inter)], hidden, inter)
    return ug[:inter], ug[inter:], dn


def expert_matrices_scalar(record, hidden, inter):
    """Same as expert_matrices, block by block with the scalar decoders (slow;
    for tiny shapes and sampled checks)."""
    rec = bytes(np.asarray(record, dtype=np.uint8).reshape(-1))
    nbu = hidden // Q3S_BLOCK_WEIGHTS
    ug = []
    for r in range(2 * inter):
        row = []
        for b in range(nbu):
            off = (r * nbu + b) * Q3S_BLOCK_BYTES
            row.extend(dequant_q3s_block(rec[off:off + Q3S_BLOCK_BYTES]))
        ug.append(row)
    base = upgate_bytes(hidden, inter)
    nbd = inter // NL4_BLOCK_WEIGHTS
    dn = []
    for r in range(hidden):
        row = []
        for b in range(nbd):
            off = base + (r * nbd + b) * NL4_BLOCK_BYTES
            row.extend(dequant_nl4_block(rec[off:off + NL4_BLOCK_BYTES]))
        dn.append(row)
    ug = np.array(ug, dtype=np.float64)
    return ug[:inter], ug[inter:], np.array(dn, dtype=np.float64)
