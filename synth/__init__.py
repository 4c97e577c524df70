"""Seeded synthetic inputs for the routed MoE FFN layer.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``; imported by
neither the oracle nor the HIP library.  It holds none of the layer's
arithmetic: it draws random numbers, lays random bits into the byte fields of
the two weight codecs, and builds the per-expert router bias that sets expert
popularity.  Everything is a pure function of (seed, layer, tag), so the CPU
can regenerate any expert of a GPU-resident layer bit for bit.

Workloads (shapes of the model on the pages: 512 routed experts, 10 active,
48 layers -- "Avalon" README, opening paragraphs; prefill chunks of 8192 and
9536 tokens -- the speed tables of "Single RX 7900 XTX ..." section 5.1 and of
the "Avalon" README, "Speed"):

* tiny    H=256, E=16, k=2, I=128, no shared expert, T=4; router logits
          given (fp32 N(0,1), distinct within a row); expert weights fp32
          N(0, 0.02) to be encoded by a round-to-nearest quantiser.
* decode  H=3072, E=512, k=10, I=512, one bf16 shared expert (I_s=512),
          T in {1, 3, 8}; router W_r bf16 N(0, 0.02) [E][H] plus a per-expert
          bias giving Zipf(1.0) popularity; experts by seeded code sampling.
* stack   48 decode-shaped layers, T=3, RMSNorm gain N(1, 0.1), eps 1e-6.
* prefill T=8192, decode shapes; Zipf(1.0) bias or no bias (uniform).
* stack_prefill  48 decode-shaped layers of mixed expert formats, one
          9536-token chunk, Zipf(0.8), RMSNorm + residual between layers.
          Up|gate: 17 layers Q3S-256, 20 Q2S-256, 11 NL4-32; down: 39 NL4-32,
          9 Q2-32 (the model card's per-layer counts, "Files / Main model");
          which layer gets which format is a seeded permutation of each list
          (the page gives the counts, not the order).

Code sampling (how expert bytes are drawn at real shape): every byte of an
expert record is a counter-hash output, then the fields that must hold a
particular range are overwritten bit-wise --
  Q3S-256 block: index bytes [0,96) stay uniform random (every bit pattern is
  a valid index stream); d (bytes 96..97) = 0x2000 | 10 random bits, i.e. a
  binary16 in [2^-7, 2^-6), the scale a round-to-nearest encoding of
  N(0, 0.02) weights produces; sub-scale bytes 98..101 get nibbles 4..7
  ("rtn" mode, the range round-to-nearest gives) or any nibble ("full" and
  "wide" modes, negative and zero sub-scales included); bytes 102..103 = 0.
  NL4-32 block: d (bytes 0..1) = 0x2800 | 10 random bits, a binary16 in
  [2^-5, 2^-4); index bytes uniform random.
  Q2S-256 block (mixed-format layers): index bytes [0,64) uniform random; d
  (bytes 64..65) = 0x1C00 | 10 random bits, in [2^-8, 2^-7); sub-scale bytes
  66..69 as for Q3S-256; bytes 70..79 = 0.
  Q2-32 block: d (bytes 0..1) = 0x2400 | 10 random bits, in [2^-6, 2^-5);
  index bytes uniform random.
  Q3K-256 block (110 bytes) and NL4S-256 block (136 bytes): index bytes
  uniform random; d (bytes 96..97, resp. 128..129) in [2^-9, 2^-8); the
  6-bit sub-scale fields (bytes 98..109, resp. 130..135) in 16..31 ("rtn"
  mode) or any value (other modes).
  (Each d range is the one a round-to-nearest encoding of N(0, 0.02) weights
  gives for that codec.)  "wide" mode instead draws each block's d binade
  from four (WIDE_D_EXPONENTS: subnormal or zero, [2^-10, 2^-9), the
  round-to-nearest binade, a large one), picked by two of d's own random
  mantissa bits, so that the decoders see the whole range of the field;
  "small" mode puts every d in [2^-12, 2^-11).
The counter hash is MurmurHash3's 32-bit finaliser (fmix32, Austin Appleby,
public domain), applied twice with per-(seed, layer, expert) keys.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------

Q3S_BLOCK_BYTES = 104     # field widths of the codecs (byte layout only)
NL4_BLOCK_BYTES = 18
Q2S_BLOCK_BYTES = 80
Q2_BLOCK_BYTES = 10
Q3K_BLOCK_BYTES = 110
NL4S_BLOCK_BYTES = 136
# format number -> (weights per block, bytes per block); the numbers are the
# library's moe_format values
FMT_Q3S256, FMT_NL4_32, FMT_Q2S256, FMT_Q2_32, FMT_Q3K256, FMT_NL4S256 = 2, 3, 4, 5, 6, 7
BLOCKS = {FMT_Q3S256: (256, Q3S_BLOCK_BYTES), FMT_NL4_32: (32, NL4_BLOCK_BYTES),
          FMT_Q2S256: (256, Q2S_BLOCK_BYTES), FMT_Q2_32: (32, Q2_BLOCK_BYTES),
          FMT_Q3K256: (256, Q3K_BLOCK_BYTES), FMT_NL4S256: (256, NL4S_BLOCK_BYTES)}

# Router-bias strength.  b_e = -ZIPF_ALPHA * s * ln(rank_e).  Chosen once by
# bisection on the 8192-token prefill workload (seed 3, s = 1.0) so that the
# hottest expert receives about 100x the tokens of the coldest (of the 81,920
# slots of 8192 tokens at top-10 over 512 experts).
ZIPF_ALPHA = 0.40


@dataclass(frozen=True)
class Shape:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    shared_inter: int          # 0 = no shared expert
    upgate_fmt: int = FMT_Q3S256
    down_fmt: int = FMT_NL4_32

    @property
    def upgate_bytes(self):
        nw, nb = BLOCKS[self.upgate_fmt]
        return 2 * self.inter * (self.hidden // nw) * nb

    @property
    def down_bytes(self):
        nw, nb = BLOCKS[self.down_fmt]
        return self.hidden * (self.inter // nw) * nb

    @property
    def expert_bytes(self):
        return self.upgate_bytes + self.down_bytes


TINY = Shape(hidden=256, inter=128, n_experts=16, top_k=2, shared_inter=0)
REAL = Shape(hidden=3072, inter=512, n_experts=512, top_k=10, shared_inter=512)
# The draft head's MoE layer (model card "Qwen3.8-Flash-Next - Avalon GGUF",
# "MTP sidecar"): the main layers' shape, up|gate in the 3.44-bpw codec
# (Q3K-256 here), down in NL4-32.
MTP_HEAD = Shape(hidden=3072, inter=512, n_experts=512, top_k=10, shared_inter=512,
                 upgate_fmt=FMT_Q3K256, down_fmt=FMT_NL4_32)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    tokens: tuple
    layers: int = 1
    zipf_s: float = 1.0
    seed: int = 0
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", TINY, (4,), seed=1, zipf_s=0.0,
                     note="logits given; RTN-quantised N(0,0.02) experts"),
    "decode": Workload("decode", REAL, (1, 3, 8), seed=2),
    "stack": Workload("stack", REAL, (3,), layers=48, seed=4),
    "prefill": Workload("prefill", REAL, (8192,), seed=3),
    "prefill_uniform": Workload("prefill_uniform", REAL, (8192,), seed=3, zipf_s=0.0),
    "stack_prefill": Workload("stack_prefill", REAL, (9536,), layers=48, seed=13, zipf_s=0.8,
                              note="mixed expert formats per layer (stack_formats)"),
}


# --------------------------------------------------------------------------
# counter hash (MurmurHash3 fmix32) on int64 tensors holding 32-bit values
# --------------------------------------------------------------------------

_M32 = 0xFFFFFFFF


def _mul32(a, c):
    """(a * c) mod 2^32 for int64 tensors a < 2^32 and a constant c < 2^32,
    split in 16-bit halves so no intermediate leaves int64 range."""
    lo = a * (c & 0xFFFF)
    hi = ((a * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & _M32


def fmix32(x):
    x = x & _M32
    x = x ^ (x >> 16)
    x = _mul32(x, 0x85EBCA6B)
    x = x ^ (x >> 13)
    x = _mul32(x, 0xC2B2AE35)
    return x ^ (x >> 16)


def _fmix32_int(x):
    return int(fmix32(torch.tensor([x & _M32], dtype=torch.int64))[0])


def key(seed, layer, tag):
    """32-bit key of (seed, layer, tag)."""
    k = _fmix32_int(seed * 0x9E3779B9 + 0x7F4A7C15)
    k = _fmix32_int(k ^ (layer * 0x632BE59B + 0x1B873593))
    return _fmix32_int(k ^ (tag * 0xCC9E2D51 + 0x2545F491))


def hash_words(k1, k2, n, device="cpu", start=0):
    """n 32-bit words fmix32(fmix32(i + k1) ^ k2), i = start .. start+n-1,
    as an int64 tensor."""
    i = torch.arange(start, start + n, dtype=torch.int64, device=device)
    return fmix32(fmix32(i + k1) ^ k2)


def hash_bytes(k1, k2, nbytes, device="cpu"):
    """nbytes pseudo-random bytes (little-endian words of hash_words)."""
    nw = (nbytes + 3) // 4
    w = hash_words(k1, k2, nw, device).to(torch.int32)   # wraps to int32
    return w.view(torch.uint8)[:nbytes]


# --------------------------------------------------------------------------
# expert records by code sampling
# --------------------------------------------------------------------------

MODES = ("rtn", "full", "wide", "small")

# binary16 exponent fields of d in "wide" mode, per codec: a subnormal (or
# zero) d, d in [2^-10, 2^-9), the binade a round-to-nearest encoding of
# N(0, 0.02) weights gives, and a large binade (the largest that keeps the
# SwiGLU outputs and the down rows of N(0, 1) tokens far below 65504).
WIDE_D_EXPONENTS = {FMT_Q3S256: (0, 5, 8, 12), FMT_NL4_32: (0, 5, 10, 13),
                    FMT_Q2S256: (0, 5, 7, 12), FMT_Q2_32: (0, 5, 9, 12),
                    FMT_Q3K256: (0, 3, 6, 9), FMT_NL4S256: (0, 3, 6, 9)}
# exponent field of d in "small" mode, every codec: d in [2^-12, 2^-11), where
# d * |table entry| / 128 of the smaller entries falls below binary16's
# smallest normal
SMALL_D_EXPONENT = 3
# exponent field of d in "rtn" and "full" mode
RTN_D_EXPONENT = {FMT_Q3S256: 8, FMT_NL4_32: 10, FMT_Q2S256: 7, FMT_Q2_32: 9,
                  FMT_Q3K256: 6, FMT_NL4S256: 6}


def _set_d(hi, fmt, mode):
    """hi: uint8 view of the high byte of d (random on entry).  Keeps the two
    mantissa bits it holds and writes the exponent field: the codec's
    round-to-nearest binade, or in "wide" mode one of WIDE_D_EXPONENTS picked
    by those two mantissa bits."""
    low = hi & 0x03
    if mode == "wide":
        ex = torch.tensor(WIDE_D_EXPONENTS[fmt], dtype=torch.uint8, device=hi.device)
        hi.copy_(low | (ex[low.long()] << 2))
    elif mode == "small":
        hi.copy_(low | (SMALL_D_EXPONENT << 2))
    else:
        hi.copy_(low | (RTN_D_EXPONENT[fmt] << 2))


def _set_subscales(sb, mode):
    """sb: uint8 [n, 4] view of the eight sub-scale nibbles: 4..7 in "rtn"
    mode (the range round-to-nearest gives), any nibble (-8..7) otherwise
    ("full", "wide", "small")."""
    if mode == "rtn":
        sb.copy_((sb & 0x33) | 0x44)


def _set_subscales6(sb, n, mode):
    """sb: uint8 [blocks, ceil(6n/8)] view of n six-bit sub-scale fields
    (field j at bits 6j .. 6j+5, little-endian): in "rtn" mode each field is
    forced into 16..31 (the range round-to-nearest gives: bit 4 set, bit 5
    clear); any value (-32..31) otherwise."""
    if mode != "rtn":
        return
    nb = sb.shape[1]
    shifts = torch.arange(8, dtype=torch.uint8, device=sb.device)
    bits = ((sb[:, :, None] >> shifts) & 1).reshape(sb.shape[0], 8 * nb)
    for j in range(n):
        bits[:, 6 * j + 4] = 1
        bits[:, 6 * j + 5] = 0
    w = (bits.reshape(sb.shape[0], nb, 8).to(torch.int32) << shifts.to(torch.int32)).sum(dim=2)
    sb.copy_(w.to(torch.uint8))


def _fix_fields(fmt, raw, mode):
    """Set the d, sub-scale and reserved fields of every block of one codec."""
    if mode not in MODES:
        raise ValueError("mode must be one of %s" % (MODES,))
    blk = raw.view(-1, BLOCKS[fmt][1])
    if fmt == FMT_Q3K256:
        _set_d(blk[:, 97], fmt, mode)
        _set_subscales6(blk[:, 98:110], 16, mode)
        return
    if fmt == FMT_NL4S256:
        _set_d(blk[:, 129], fmt, mode)
        _set_subscales6(blk[:, 130:136], 8, mode)
        return
    if fmt == FMT_Q3S256:
        _set_d(blk[:, 97], fmt, mode)
        _set_subscales(blk[:, 98:102], mode)
        blk[:, 102:104] = 0
    elif fmt == FMT_Q2S256:
        _set_d(blk[:, 65], fmt, mode)
        _set_subscales(blk[:, 66:70], mode)
        blk[:, 70:80] = 0
    else:                                           # NL4-32, Q2-32: d first
        _set_d(blk[:, 1], fmt, mode)


def expert_record(shape, seed, layer, e, device="cpu", mode="rtn"):
    """Packed bytes (uint8 [expert_bytes]) of expert e of a layer."""
    k1 = key(seed, layer, 2 * e + 1)
    k2 = key(seed, layer, 2 * e + 2)
    rec = hash_bytes(k1, k2, shape.expert_bytes, device).clone()
    _fix_fields(shape.upgate_fmt, rec[:shape.upgate_bytes], mode)
    _fix_fields(shape.down_fmt, rec[shape.upgate_bytes:], mode)
    return rec


def expert_bank(shape, seed, layer, device="cpu", mode="rtn", chunk=32):
    """All E expert records of a layer: uint8 [E][expert_bytes] on `device`,
    equal byte for byte to expert_record(e) for every e.  Rows are generated
    `chunk` experts at a time to bound temporary memory."""
    E, nb = shape.n_experts, shape.expert_bytes
    nw = (nb + 3) // 4
    out = torch.empty((E, nb), dtype=torch.uint8, device=device)
    i = torch.arange(nw, dtype=torch.int64, device=device)[None, :]
    for e0 in range(0, E, chunk):
        es = range(e0, min(E, e0 + chunk))
        k1 = torch.tensor([key(seed, layer, 2 * e + 1) for e in es], dtype=torch.int64, device=device)
        k2 = torch.tensor([key(seed, layer, 2 * e + 2) for e in es], dtype=torch.int64, device=device)
        w = fmix32(fmix32(i + k1[:, None]) ^ k2[:, None]).to(torch.int32)
        rec = w.view(torch.uint8).reshape(len(es), 4 * nw)[:, :nb]
        ug = rec[:, :shape.upgate_bytes].reshape(-1, BLOCKS[shape.upgate_fmt][1])
        dn = rec[:, shape.upgate_bytes:].reshape(-1, BLOCKS[shape.down_fmt][1])
        for fmt, blk in ((shape.upgate_fmt, ug), (shape.down_fmt, dn)):
            fixed = blk.clone()
            _fix_fields(fmt, fixed.view(-1), mode)
            blk.copy_(fixed)
        out[e0:e0 + len(es)] = torch.cat([ug.reshape(len(es), -1), dn.reshape(len(es), -1)], dim=1)
        del w, rec
    return out


# --------------------------------------------------------------------------
# dense inputs
# --------------------------------------------------------------------------

def _gen(seed, layer, tag):
    g = torch.Generator(device="cpu")
    g.manual_seed(key(seed, layer, 1_000_000 + tag))
    return g


def normal_bf16(rows, cols, std, seed, layer, tag):
    """bf16 tensor [rows][cols] ~ N(0, std^2), drawn in fp32 on the CPU and
    converted by torch (round to nearest even)."""
    g = _gen(seed, layer, tag)
    return (torch.randn((rows, cols), generator=g, dtype=torch.float32) * std).to(torch.bfloat16)


def tokens_bf16(T, hidden, seed, layer=0, tag=0):
    """Activations x: bf16 [T][H] ~ N(0,1)."""
    return normal_bf16(T, hidden, 1.0, seed, layer, 10 + tag)


def unique_logits(T, E, seed, layer=0):
    """fp32 [T][E] ~ N(0,1) with all values of a row distinct (a row with a
    repeat is drawn again)."""
    g = _gen(seed, layer, 20)
    out = torch.empty((T, E), dtype=torch.float32)
    for t in range(T):
        while True:
            row = torch.randn(E, generator=g, dtype=torch.float32)
            if torch.unique(row).numel() == E:
                out[t] = row
                break
    return out


def router_weight(shape, seed, layer):
    """W_r: bf16 [E][H] ~ N(0, 0.02)."""
    return normal_bf16(shape.n_experts, shape.hidden, 0.02, seed, layer, 30)


def zipf_bias(E, s, seed, layer, alpha=ZIPF_ALPHA):
    """fp32 [E]: b_e = -alpha * s * ln(rank_e), ranks a seeded permutation
    of 1..E (so the hot experts are not the low indices that ties favour)."""
    if s == 0.0:
        return torch.zeros(E, dtype=torch.float32)
    rng = np.random.default_rng(key(seed, layer, 40))
    rank = rng.permutation(E) + 1
    return torch.from_numpy((-alpha * s * np.log(rank)).astype(np.float32))


def shared_weights(shape, seed, layer):
    """Shared expert: (up|gate bf16 [2 I_s][H], down bf16 [H][I_s]) ~ N(0, 0.02)."""
    ug = normal_bf16(2 * shape.shared_inter, shape.hidden, 0.02, seed, layer, 50)
    dn = normal_bf16(shape.hidden, shape.shared_inter, 0.02, seed, layer, 51)
    return ug, dn


def norm_gain(hidden, seed, layer):
    """RMSNorm gain gamma: fp32 [H] ~ N(1, 0.1)."""
    g = _gen(seed, layer, 60)
    return 1.0 + 0.1 * torch.randn(hidden, generator=g, dtype=torch.float32)


def tiny_expert_weights(shape, seed, layer=0):
    """fp32 N(0, 0.02) expert weights of the tiny workload, to be encoded by a
    round-to-nearest quantiser: (up|gate [E][2I][H], down [E][H][I])."""
    g = _gen(seed, layer, 70)
    ug = torch.randn((shape.n_experts, 2 * shape.inter, shape.hidden), generator=g) * 0.02
    dn = torch.randn((shape.n_experts, shape.hidden, shape.inter), generator=g) * 0.02
    return ug, dn


@dataclass
class Layer:
    """One layer's inputs (torch tensors on one device)."""
    shape: Shape
    experts: torch.Tensor                 # uint8 [E][expert_bytes]
    router_w: torch.Tensor = None         # bf16 [E][H]
    router_b: torch.Tensor = None         # fp32 [E]
    shared_ug: torch.Tensor = None        # bf16 [2 I_s][H]
    shared_down: torch.Tensor = None      # bf16 [H][I_s]
    seed: int = 0
    layer: int = 0
    extra: dict = field(default_factory=dict)


STACK_UG_FORMATS = (FMT_Q3S256,) * 17 + (FMT_Q2S256,) * 20 + (FMT_NL4_32,) * 11
STACK_DN_FORMATS = (FMT_NL4_32,) * 39 + (FMT_Q2_32,) * 9


def stack_formats(seed, layers=48):
    """(up|gate format, down format) of each layer of the mixed-format stack:
    the counts above, placed by two seeded permutations."""
    rng = np.random.default_rng(key(seed, 0, 80))
    ug = [STACK_UG_FORMATS[i] for i in rng.permutation(48)]
    dn = [STACK_DN_FORMATS[i] for i in rng.permutation(48)]
    return list(zip(ug, dn))[:layers]


def stack_shape(seed, layer):
    """Real shape with the formats of one layer of the mixed-format stack."""
    ug, dn = stack_formats(seed)[layer]
    return Shape(REAL.hidden, REAL.inter, REAL.n_experts, REAL.top_k, REAL.shared_inter, ug, dn)


def real_layer(shape, seed, layer, zipf_s=1.0, device="cpu", mode="rtn", experts=True):
    """A real-shape layer: code-sampled experts, router, Zipf bias, shared expert."""
    ex = expert_bank(shape, seed, layer, device, mode) if experts else None
    ug, dn = shared_weights(shape, seed, layer) if shape.shared_inter else (None, None)
    return Layer(shape=shape, experts=ex,
                 router_w=router_weight(shape, seed, layer).to(device),
                 router_b=zipf_bias(shape.n_experts, zipf_s, seed, layer).to(device),
                 shared_ug=None if ug is None else ug.to(device),
                 shared_down=None if dn is None else dn.to(device),
                 seed=seed, layer=layer)
