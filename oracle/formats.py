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

Two further codecs of the mixed-format layers of the same model (the model
card, "Files / Main model": up/gate IQ2_S in 20 layers, down Q2_0 in 9; the
page gives the type names only).  Readings taken here:

Q2S-256 block (256 weights, 80 bytes = 2.5 bits per weight)
  bytes [0, 64)   256 two-bit codebook indices, weight i at stream bits
                  2i .. 2i+1 (little-endian stream as above).  Sub-block j
                  is bytes [8j, 8j+8).
  bytes [64, 66)  d, binary16.
  bytes [66, 70)  eight signed 4-bit sub-scales, encoded as in Q3S-256.
  bytes [70, 80)  reserved: writers store 0, readers ignore.
  value of weight i = d * s_{i // 32} * C2[q_i] / 128  (exact in fp32).
  The sign of the sub-scale mirrors the asymmetric codebook: this is the
  "sign" of a 2-bit-plus-sign reading that fits the bit rate.

Q2-32 block (32 weights, 10 bytes = 2.5 bits per weight)
  bytes [0, 2)    d, binary16.
  bytes [2, 10)   32 two-bit q, weight i at bits 2i .. 2i+1.
  value of weight i = d * (q_i - 2)  (exact in fp32).

Two more up/gate codecs of the same model card ("Files / Main model": up/gate
IQ3_K in 10 layers, 3.44 bpw, and IQ4_XS in 1 layer; the card also puts the
draft head's experts in IQ3_K up/gate with IQ4_NL down, "MTP sidecar").  The
page gives their names and bit rates only.  Readings taken here -- each the
plainest layout that fills exactly the stated bit rate with the fields the
3.25-bpw codec has (a binary16 block scale, signed sub-scales, codebook
indices):

Q3K-256 block (256 weights, 110 bytes = 3.4375 bits per weight, "3.44")
  bytes [0, 96)   256 three-bit indices into the Q3S-256 codebook, the same
                  little-endian stream as Q3S-256.
  bytes [96, 98)  d, binary16.
  bytes [98, 110) sixteen signed 6-bit sub-scales, one per 16 weights: the 12
                  bytes read as a little-endian 96-bit number V, s_j = bits
                  6j .. 6j+5 of V as a two's-complement field, s_j in
                  [-32, 31].  (The 0.19 bpw over the 3.25-bpw codec buy twice
                  as many sub-scales with two more bits each.)
  value of weight i = d * s_{i // 16} * C3[q_i] / 128  (exact in fp32: |s c|
  <= 4064 has 12 bits, d 11).

NL4S-256 block (256 weights, 136 bytes = 4.25 bits per weight)
  bytes [0, 128)  256 four-bit indices into the NL4-32 table, weight i at
                  bits 4i .. 4i+3 of the little-endian stream (sub-block j =
                  bytes [16j, 16j+16)).
  bytes [128,130) d, binary16.
  bytes [130,136) eight signed 6-bit sub-scales, one per 32 weights, as a
                  little-endian 48-bit number (s_j = bits 6j .. 6j+5).
  value of weight i = d * s_{i // 32} * T4[q_i] / 128  (exact in fp32).

Codebooks: sorted, distinct int8 levels placed at normal quantiles
("NF"-style), asymmetric with an exact zero: for a b-bit book with n = 2^b
entries, p = 1 - 1/(2n); the n/2 positive levels are Phi^-1 at
linspace(0.5, p, n/2 + 1)[1:], the n/2 - 1 negative levels are -Phi^-1 at
linspace(0.5, p, n/2)[1:], all divided by Phi^-1(p), times 127, rounded to
the nearest integer.  The literals below are that rule's output, frozen.

Matrix orientation: a weight matrix is stored as [out rows][in], blocks running
along the reduction (input) dimension, so one block scale serves one dot
product.  An expert record is up|gate = [2I][H] (rows 0..I-1 up, I..2I-1 gate)
in Q3S-256, then down = [H][I] in NL4-32.  The mixed-format layers store
up|gate in Q3S-256, Q2S-256 or NL4-32 and down in NL4-32 or Q2-32, in the
same order.
"""

import numpy as np

Q3S_BLOCK_WEIGHTS = 256
Q3S_BLOCK_BYTES = 104
Q3S_SUB_WEIGHTS = 32
NL4_BLOCK_WEIGHTS = 32
NL4_BLOCK_BYTES = 18
Q2S_BLOCK_WEIGHTS = 256
Q2S_BLOCK_BYTES = 80
Q2S_SUB_WEIGHTS = 32
Q2_BLOCK_WEIGHTS = 32
Q2_BLOCK_BYTES = 10

# 8-entry codebook of the 3.25-bpw up/gate codec (value = entry / 128).
Q3S_CODEBOOK = (-127, -67, -31, 0, 23, 48, 78, 127)
# 16-entry non-linear table of the 4-bit down codec (value = entry / 128).
NL4_TABLE = (-127, -88, -66, -50, -36, -23, -11, 0, 10, 20, 31, 43, 56, 71, 91, 127)
# 4-entry codebook of the 2.5-bpw up/gate codec (value = entry / 128).
Q2S_CODEBOOK = (-127, 0, 54, 127)
# Format numbers (the library's moe_format values).
FMT_Q3S256, FMT_NL4_32, FMT_Q2S256, FMT_Q2_32 = 2, 3, 4, 5
FMT_Q3K256, FMT_NL4S256 = 6, 7
Q3K_BLOCK_WEIGHTS = 256
Q3K_BLOCK_BYTES = 110
Q3K_SUB_WEIGHTS = 16
NL4S_BLOCK_WEIGHTS = 256
NL4S_BLOCK_BYTES = 136
NL4S_SUB_WEIGHTS = 32


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


def _subscales(v):
    """Eight two's-complement nibbles of a u32, nibble j at bits 4j."""
    out = []
    for j in range(8):
        nib = (v >> (4 * j)) & 0xF
        out.append(nib - 16 if nib >= 8 else nib)
    return out


def unpack_q2s_block(block):
    """Fields of one 80-byte Q2S-256 block: (d_bits, s[8], q[256])."""
    block = bytes(block)
    if len(block) != Q2S_BLOCK_BYTES:
        raise ValueError("Q2S-256 block must be 80 bytes")
    bits = _bit_stream(block[0:64])
    q = [bits[2 * i] | (bits[2 * i + 1] << 1) for i in range(Q2S_BLOCK_WEIGHTS)]
    d_bits = block[64] | (block[65] << 8)
    v = block[66] | (block[67] << 8) | (block[68] << 16) | (block[69] << 24)
    return d_bits, _subscales(v), q


def dequant_q2s_block(block):
    """256 weight values of one Q2S-256 block (Python floats, exact)."""
    d_bits, s, q = unpack_q2s_block(block)
    d = fp16_bits_to_float(d_bits)
    return [d * s[i // Q2S_SUB_WEIGHTS] * Q2S_CODEBOOK[q[i]] / 128.0
            for i in range(Q2S_BLOCK_WEIGHTS)]


def pack_q2s_block(d_bits, s, q):
    """Bytes of one Q2S-256 block from its fields (reserved bytes zero)."""
    if len(s) != 8 or len(q) != Q2S_BLOCK_WEIGHTS:
        raise ValueError("need 8 sub-scales and 256 indices")
    stream = 0
    for i, qi in enumerate(q):
        if not 0 <= qi < 4:
            raise ValueError("index out of range")
        stream |= int(qi) << (2 * i)
    out = bytearray(stream.to_bytes(64, "little"))
    out += bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])
    v = 0
    for j, sj in enumerate(s):
        if not -8 <= sj <= 7:
            raise ValueError("sub-scale out of range")
        v |= (int(sj) & 0xF) << (4 * j)
    out += v.to_bytes(4, "little")
    out += bytes(10)
    return bytes(out)


def unpack_q2_block(block):
    """Fields of one 10-byte Q2-32 block: (d_bits, q[32])."""
    block = bytes(block)
    if len(block) != Q2_BLOCK_BYTES:
        raise ValueError("Q2-32 block must be 10 bytes")
    d_bits = block[0] | (block[1] << 8)
    bits = _bit_stream(block[2:10])
    return d_bits, [bits[2 * i] | (bits[2 * i + 1] << 1) for i in range(Q2_BLOCK_WEIGHTS)]


def dequant_q2_block(block):
    """32 weight values of one Q2-32 block (Python floats, exact)."""
    d_bits, q = unpack_q2_block(block)
    d = fp16_bits_to_float(d_bits)
    return [d * (qi - 2) for qi in q]


def pack_q2_block(d_bits, q):
    """Bytes of one Q2-32 block from its fields."""
    if len(q) != Q2_BLOCK_WEIGHTS:
        raise ValueError("need 32 indices")
    stream = 0
    for i, qi in enumerate(q):
        if not 0 <= qi < 4:
            raise ValueError("index out of range")
        stream |= int(qi) << (2 * i)
    return bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF]) + stream.to_bytes(8, "little")


def _subscales6(v, n):
    """n two's-complement 6-bit fields of a non-negative int, field j at
    bits 6j .. 6j+5."""
    out = []
    for j in range(n):
        f = (v >> (6 * j)) & 0x3F
        out.append(f - 64 if f >= 32 else f)
    return out


def _pack_subscales6(s, nbytes):
    v = 0
    for j, sj in enumerate(s):
        if not -32 <= sj <= 31:
            raise ValueError("sub-scale out of range")
        v |= (int(sj) & 0x3F) << (6 * j)
    return v.to_bytes(nbytes, "little")


def unpack_q3k_block(block):
    """Fields of one 110-byte Q3K-256 block: (d_bits, s[16], q[256])."""
    block = bytes(block)
    if len(block) != Q3K_BLOCK_BYTES:
        raise ValueError("Q3K-256 block must be 110 bytes")
    bits = _bit_stream(block[0:96])
    q = [bits[3 * i] | (bits[3 * i + 1] << 1) | (bits[3 * i + 2] << 2)
         for i in range(Q3K_BLOCK_WEIGHTS)]
    d_bits = block[96] | (block[97] << 8)
    return d_bits, _subscales6(int.from_bytes(block[98:110], "little"), 16), q


def dequant_q3k_block(block):
    """256 weight values of one Q3K-256 block (Python floats, exact)."""
    d_bits, s, q = unpack_q3k_block(block)
    d = fp16_bits_to_float(d_bits)
    return [d * s[i // Q3K_SUB_WEIGHTS] * Q3S_CODEBOOK[q[i]] / 128.0
            for i in range(Q3K_BLOCK_WEIGHTS)]


def pack_q3k_block(d_bits, s, q):
    """Bytes of one Q3K-256 block from its fields."""
    if len(s) != 16 or len(q) != Q3K_BLOCK_WEIGHTS:
        raise ValueError("need 16 sub-scales and 256 indices")
    stream = 0
    for i, qi in enumerate(q):
        if not 0 <= qi < 8:
            raise ValueError("index out of range")
        stream |= int(qi) << (3 * i)
    return (stream.to_bytes(96, "little") + bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])
            + _pack_subscales6(s, 12))


def unpack_nl4s_block(block):
    """Fields of one 136-byte NL4S-256 block: (d_bits, s[8], q[256])."""
    block = bytes(block)
    if len(block) != NL4S_BLOCK_BYTES:
        raise ValueError("NL4S-256 block must be 136 bytes")
    bits = _bit_stream(block[0:128])
    q = [bits[4 * i] | (bits[4 * i + 1] << 1) | (bits[4 * i + 2] << 2) | (bits[4 * i + 3] << 3)
         for i in range(NL4S_BLOCK_WEIGHTS)]
    d_bits = block[128] | (block[129] << 8)
    return d_bits, _subscales6(int.from_bytes(block[130:136], "little"), 8), q


def dequant_nl4s_block(block):
    """256 weight values of one NL4S-256 block (Python floats, exact)."""
    d_bits, s, q = unpack_nl4s_block(block)
    d = fp16_bits_to_float(d_bits)
    return [d * s[i // NL4S_SUB_WEIGHTS] * NL4_TABLE[q[i]] / 128.0
            for i in range(NL4S_BLOCK_WEIGHTS)]


def pack_nl4s_block(d_bits, s, q):
    """Bytes of one NL4S-256 block from its fields."""
    if len(s) != 8 or len(q) != NL4S_BLOCK_WEIGHTS:
        raise ValueError("need 8 sub-scales and 256 indices")
    stream = 0
    for i, qi in enumerate(q):
        if not 0 <= qi < 16:
            raise ValueError("index out of range")
        stream |= int(qi) << (4 * i)
    return (stream.to_bytes(128, "little") + bytes([d_bits & 0xFF, (d_bits >> 8) & 0xFF])
            + _pack_subscales6(s, 6))


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


def unpack_q2s(arr):
    """Vectorised Q2S-256 unpack: (d float64 [...], s int64 [..., 8],
    q int64 [..., 256])."""
    a = _as_blocks(arr, Q2S_BLOCK_BYTES)
    bits = np.unpackbits(a[..., 0:64], axis=-1, bitorder="little")
    bits = bits.reshape(a.shape[:-1] + (Q2S_BLOCK_WEIGHTS, 2)).astype(np.int64)
    q = bits[..., 0] | (bits[..., 1] << 1)
    d = np.ascontiguousarray(a[..., 64:66]).view("<f2")[..., 0].astype(np.float64)
    v = np.ascontiguousarray(a[..., 66:70]).view("<u4")[..., 0].astype(np.int64)
    s = np.stack([(v >> (4 * j)) & 0xF for j in range(8)], axis=-1)
    s = np.where(s >= 8, s - 16, s)
    return d, s, q


def dequant_q2s(arr):
    """Vectorised Q2S-256 dequant: float64 [..., 256] per block."""
    d, s, q = unpack_q2s(arr)
    c = np.asarray(Q2S_CODEBOOK, dtype=np.float64)[q]
    sw = np.repeat(s, Q2S_SUB_WEIGHTS, axis=-1).astype(np.float64)
    return d[..., None] * sw * c / 128.0


def unpack_q2(arr):
    """Vectorised Q2-32 unpack: (d float64 [...], q int64 [..., 32])."""
    a = _as_blocks(arr, Q2_BLOCK_BYTES)
    d = np.ascontiguousarray(a[..., 0:2]).view("<f2")[..., 0].astype(np.float64)
    b = a[..., 2:10].astype(np.int64)
    q = np.stack([(b >> (2 * t)) & 3 for t in range(4)], axis=-1).reshape(a.shape[:-1] + (Q2_BLOCK_WEIGHTS,))
    return d, q


def dequant_q2(arr):
    """Vectorised Q2-32 dequant: float64 [..., 32] per block."""
    d, q = unpack_q2(arr)
    return d[..., None] * (q - 2).astype(np.float64)


def _unpack_subscales6(a, n):
    """Two's-complement 6-bit fields j = 0..n-1 of little-endian byte rows a
    [..., ceil(6n/8)] (field j at bits 6j .. 6j+5)."""
    bits = np.unpackbits(a, axis=-1, bitorder="little").astype(np.int64)
    bits = bits[..., :6 * n].reshape(a.shape[:-1] + (n, 6))
    f = sum(bits[..., b] << b for b in range(6))
    return np.where(f >= 32, f - 64, f)


def unpack_q3k(arr):
    """Vectorised Q3K-256 unpack: (d float64 [...], s int64 [..., 16],
    q int64 [..., 256])."""
    a = _as_blocks(arr, Q3K_BLOCK_BYTES)
    bits = np.unpackbits(a[..., 0:96], axis=-1, bitorder="little")
    bits = bits.reshape(a.shape[:-1] + (Q3K_BLOCK_WEIGHTS, 3)).astype(np.int64)
    q = bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)
    d = np.ascontiguousarray(a[..., 96:98]).view("<f2")[..., 0].astype(np.float64)
    return d, _unpack_subscales6(a[..., 98:110], 16), q


def dequant_q3k(arr):
    """Vectorised Q3K-256 dequant: float64 [..., 256] per block."""
    d, s, q = unpack_q3k(arr)
    c = np.asarray(Q3S_CODEBOOK, dtype=np.float64)[q]
    return d[..., None] * np.repeat(s, Q3K_SUB_WEIGHTS, axis=-1) * c / 128.0


def unpack_nl4s(arr):
    """Vectorised NL4S-256 unpack: (d float64 [...], s int64 [..., 8],
    q int64 [..., 256])."""
    a = _as_blocks(arr, NL4S_BLOCK_BYTES)
    idx = a[..., 0:128].astype(np.int64)
    q = np.stack([idx & 0xF, idx >> 4], axis=-1).reshape(a.shape[:-1] + (NL4S_BLOCK_WEIGHTS,))
    d = np.ascontiguousarray(a[..., 128:130]).view("<f2")[..., 0].astype(np.float64)
    return d, _unpack_subscales6(a[..., 130:136], 8), q


def dequant_nl4s(arr):
    """Vectorised NL4S-256 dequant: float64 [..., 256] per block."""
    d, s, q = unpack_nl4s(arr)
    t = np.asarray(NL4_TABLE, dtype=np.float64)[q]
    return d[..., None] * np.repeat(s, NL4S_SUB_WEIGHTS, axis=-1) * t / 128.0


def _pack_subscales6_vec(s, nbytes):
    s = np.asarray(s, dtype=np.int64)
    f = (s & 0x3F).astype(np.uint8)
    bits = np.stack([(f >> b) & 1 for b in range(6)], axis=-1).reshape(s.shape[:-1] + (-1,))
    pad = nbytes * 8 - bits.shape[-1]
    if pad:
        bits = np.concatenate([bits, np.zeros(s.shape[:-1] + (pad,), dtype=np.uint8)], axis=-1)
    return np.packbits(bits.astype(np.uint8), axis=-1, bitorder="little")


def pack_q3k(d_bits, s, q):
    """Vectorised pack: d_bits uint16 [...], s int [..., 16], q int [..., 256]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    q = np.asarray(q, dtype=np.int64)
    lead = d_bits.shape
    out = np.zeros(lead + (Q3K_BLOCK_BYTES,), dtype=np.uint8)
    bits = np.stack([(q >> b) & 1 for b in range(3)], axis=-1).reshape(lead + (768,))
    out[..., 0:96] = np.packbits(bits.astype(np.uint8), axis=-1, bitorder="little")
    out[..., 96:98] = d_bits[..., None].view(np.uint8).reshape(lead + (2,))
    out[..., 98:110] = _pack_subscales6_vec(s, 12)
    return out


def pack_nl4s(d_bits, s, q):
    """Vectorised pack: d_bits uint16 [...], s int [..., 8], q int [..., 256]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    q = np.asarray(q, dtype=np.int64)
    lead = d_bits.shape
    out = np.zeros(lead + (NL4S_BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0:128] = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    out[..., 128:130] = d_bits[..., None].view(np.uint8).reshape(lead + (2,))
    out[..., 130:136] = _pack_subscales6_vec(s, 6)
    return out


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


def pack_q2s(d_bits, s, q):
    """Vectorised pack: d_bits uint16 [...], s int [..., 8], q int [..., 256]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    s = np.asarray(s, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    lead = d_bits.shape
    out = np.zeros(lead + (Q2S_BLOCK_BYTES,), dtype=np.uint8)
    bits = np.stack([(q >> b) & 1 for b in range(2)], axis=-1).reshape(lead + (512,))
    out[..., 0:64] = np.packbits(bits.astype(np.uint8), axis=-1, bitorder="little")
    out[..., 64:66] = d_bits[..., None].view(np.uint8).reshape(lead + (2,))
    v = np.zeros(lead, dtype=np.uint32)
    for j in range(8):
        v |= ((s[..., j] & 0xF).astype(np.uint32) << np.uint32(4 * j))
    out[..., 66:70] = v.astype("<u4")[..., None].view(np.uint8).reshape(lead + (4,))
    return out


def pack_q2(d_bits, q):
    """Vectorised pack: d_bits uint16 [...], q int [..., 32]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    q = np.asarray(q, dtype=np.int64).reshape(d_bits.shape + (8, 4))
    lead = d_bits.shape
    out = np.zeros(lead + (Q2_BLOCK_BYTES,), dtype=np.uint8)
    out[..., 0:2] = d_bits[..., None].view(np.uint8).reshape(lead + (2,))
    out[..., 2:10] = (q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)).astype(np.uint8)
    return out


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


def quantize_q2s(w):
    """Round-to-nearest Q2S-256 encoding of weights w [..., 256]: the Q3S-256
    rule with the codebook C2 (sigma_j = absmax_j / (max|C2|/128), d =
    fp16_RNE(max_j sigma_j / 7), s_j = clamp(round_half_even(sigma_j / d),
    -8, 7), q_i nearest, ties to the lower index; d = 0 gives s = q = 0).
    Returns uint8 [..., 80]."""
    w = np.asarray(w, dtype=np.float64)
    lead = w.shape[:-1]
    sub = w.reshape(lead + (8, Q2S_SUB_WEIGHTS))
    cmax = max(abs(c) for c in Q2S_CODEBOOK) / 128.0
    sigma = np.abs(sub).max(axis=-1) / cmax
    d_bits = _fp16_rne_bits(sigma.max(axis=-1) / 7.0)
    d = d_bits.view(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(d[..., None] > 0, np.rint(sigma / d[..., None]), 0.0)
    s = np.clip(s, -8, 7).astype(np.int64)
    cands = (d[..., None, None] * s[..., None].astype(np.float64)
             * np.asarray(Q2S_CODEBOOK, dtype=np.float64) / 128.0)
    dist = np.abs(sub[..., None] - cands[..., None, :])
    q = np.argmin(dist, axis=-1).reshape(lead + (Q2S_BLOCK_WEIGHTS,))
    return pack_q2s(d_bits, s, q)


def quantize_q2(w):
    """Round-to-nearest Q2-32 encoding of weights w [..., 32]: d =
    fp16_RNE(absmax / 2) (the levels are d * {-2, -1, 0, 1}); q_i = the level
    nearest w_i, ties to the lower index.  Returns uint8 [..., 10]."""
    w = np.asarray(w, dtype=np.float64)
    d_bits = _fp16_rne_bits(np.abs(w).max(axis=-1) / 2.0)
    d = d_bits.view(np.float16).astype(np.float64)
    cands = d[..., None] * np.arange(-2, 2, dtype=np.float64)
    q = np.argmin(np.abs(w[..., None] - cands[..., None, :]), axis=-1)
    return pack_q2(d_bits, q)


def _quantize_subscaled(w, sub, book):
    """Round-to-nearest for the 6-bit sub-scaled codecs: per block of
    w [..., n] with sub-blocks of `sub` weights, sigma_j = absmax_j /
    (max|book|/128); d = fp16_RNE(max_j sigma_j / 31); s_j =
    clamp(round_half_even(sigma_j / d), -32, 31); q_i = the book index
    minimising |w_i - d*s_j*book[q]/128|, ties to the lower index (d = 0 gives
    s = q = 0).  Returns (d_bits, s, q)."""
    w = np.asarray(w, dtype=np.float64)
    lead, n = w.shape[:-1], w.shape[-1]
    ns = n // sub
    subw = w.reshape(lead + (ns, sub))
    cmax = max(abs(c) for c in book) / 128.0
    sigma = np.abs(subw).max(axis=-1) / cmax
    d_bits = _fp16_rne_bits(sigma.max(axis=-1) / 31.0)
    d = d_bits.view(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(d[..., None] > 0, np.rint(sigma / d[..., None]), 0.0)
    s = np.clip(s, -32, 31).astype(np.int64)
    cands = (d[..., None, None] * s[..., None].astype(np.float64)
             * np.asarray(book, dtype=np.float64) / 128.0)
    dist = np.abs(subw[..., None] - cands[..., None, :])
    q = np.argmin(dist, axis=-1).reshape(lead + (n,))
    return d_bits, s, q


def quantize_q3k(w):
    """Round-to-nearest Q3K-256 encoding of weights w [..., 256] (16-weight
    sub-blocks, the C3 codebook).  Returns uint8 [..., 110]."""
    return pack_q3k(*_quantize_subscaled(w, Q3K_SUB_WEIGHTS, Q3S_CODEBOOK))


def quantize_nl4s(w):
    """Round-to-nearest NL4S-256 encoding of weights w [..., 256] (32-weight
    sub-blocks, the T4 table).  Returns uint8 [..., 136]."""
    return pack_nl4s(*_quantize_subscaled(w, NL4S_SUB_WEIGHTS, NL4_TABLE))


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
# any of the codecs by format number
# --------------------------------------------------------------------------

# format -> (weights per block, bytes per block, vectorised dequant,
#            scalar block dequant, round-to-nearest quantiser)
CODECS = {
    FMT_Q3S256: (Q3S_BLOCK_WEIGHTS, Q3S_BLOCK_BYTES, dequant_q3s, dequant_q3s_block, quantize_q3s),
    FMT_NL4_32: (NL4_BLOCK_WEIGHTS, NL4_BLOCK_BYTES, dequant_nl4, dequant_nl4_block, quantize_nl4),
    FMT_Q2S256: (Q2S_BLOCK_WEIGHTS, Q2S_BLOCK_BYTES, dequant_q2s, dequant_q2s_block, quantize_q2s),
    FMT_Q2_32: (Q2_BLOCK_WEIGHTS, Q2_BLOCK_BYTES, dequant_q2, dequant_q2_block, quantize_q2),
    FMT_Q3K256: (Q3K_BLOCK_WEIGHTS, Q3K_BLOCK_BYTES, dequant_q3k, dequant_q3k_block, quantize_q3k),
    FMT_NL4S256: (NL4S_BLOCK_WEIGHTS, NL4S_BLOCK_BYTES, dequant_nl4s, dequant_nl4s_block,
                  quantize_nl4s),
}
UPGATE_FORMATS = (FMT_Q3S256, FMT_Q2S256, FMT_NL4_32, FMT_Q3K256, FMT_NL4S256)
DOWN_FORMATS = (FMT_NL4_32, FMT_Q2_32)


def matrix_bytes(fmt, rows, cols):
    nw, nb = CODECS[fmt][:2]
    return rows * (cols // nw) * nb


def dequant_matrix(fmt, raw, rows, cols):
    """Dequantise a matrix stored [rows][cols] in format fmt."""
    nw, nb, deq = CODECS[fmt][:3]
    a = np.asarray(raw, dtype=np.uint8).reshape(rows, cols // nw, nb)
    return deq(a).reshape(rows, cols)


def quantize_matrix(fmt, w):
    """Round-to-nearest encoding of a matrix [rows][cols] in format fmt."""
    nw, nb, _, _, quant = CODECS[fmt]
    w = np.asarray(w, dtype=np.float64)
    rows, cols = w.shape
    return quant(w.reshape(rows, cols // nw, nw)).reshape(rows, -1)


# --------------------------------------------------------------------------
# expert records: up|gate ([2I][H]) then down ([H][I]); Q3S-256 and NL4-32
# unless other formats are given
# --------------------------------------------------------------------------

def upgate_bytes(hidden, inter, fmt=FMT_Q3S256):
    return matrix_bytes(fmt, 2 * inter, hidden)


def down_bytes(hidden, inter, fmt=FMT_NL4_32):
    return matrix_bytes(fmt, hidden, inter)


def expert_record_bytes(hidden, inter, ug_fmt=FMT_Q3S256, dn_fmt=FMT_NL4_32):
    return upgate_bytes(hidden, inter, ug_fmt) + down_bytes(hidden, inter, dn_fmt)


def expert_matrices(record, hidden, inter, ug_fmt=FMT_Q3S256, dn_fmt=FMT_NL4_32):
    """Dequantised (W_up [I][H], W_gate [I][H], W_down [H][I]) of one packed
    expert record (uint8, length >= expert_record_bytes)."""
    rec = np.asarray(record, dtype=np.uint8).reshape(-1)
    nug = upgate_bytes(hidden, inter, ug_fmt)
    ug = dequant_matrix(ug_fmt, rec[:nug], 2 * inter, hidden)
    dn = dequant_matrix(dn_fmt, rec[nug:nug + down_bytes(hidden, inter, dn_fmt)], hidden, inter)
    return ug[:inter], ug[inter:], dn


def _matrix_scalar(fmt, rec, base, rows, cols):
    nw, nb, _, deq_block, _ = CODECS[fmt]
    nbr = cols // nw
    out = []
    for r in range(rows):
        row = []
        for b in range(nbr):
            off = base + (r * nbr + b) * nb
            row.extend(deq_block(rec[off:off + nb]))
        out.append(row)
    return np.array(out, dtype=np.float64)


def expert_matrices_scalar(record, hidden, inter, ug_fmt=FMT_Q3S256, dn_fmt=FMT_NL4_32):
    """Same as expert_matrices, block by block with the scalar decoders (slow;
    for tiny shapes and sampled checks)."""
    rec = bytes(np.asarray(record, dtype=np.uint8).reshape(-1))
    ug = _matrix_scalar(ug_fmt, rec, 0, 2 * inter, hidden)
    dn = _matrix_scalar(dn_fmt, rec, upgate_bytes(hidden, inter, ug_fmt), hidden, inter)
    return ug[:inter], ug[inter:], dn
