"""The routed MoE FFN layer, written out as its plain definition in fp64.
Test infrastructure: see the package header for who may use it.

Sources:
* "Avalon" README, opening paragraphs: each token is routed to 10 of 512
  experts; 48 such layers.
* "Qwen3.8-Flash-Next - Avalon GGUF" model card, "Files / Main model": a router
  and a shared expert per layer sit in the dense part; routed experts are
  packed up | gate | down.
* "Betelgeuse" post (2026-11-01): every one of the routed experts is computed
  (no gate pruning); routing is exact and checked record by record.

Readings where the pages are silent (all also listed in the design notes):
* router:      L[t][e] = sum_h x[t][h] * W_r[e][h] + b[e]; W_r stored [E][H].
* selection:   the k largest L[t][.] ordered by (value descending, expert
               index ascending); equal values go to the lower index; no
               capacity limit, no dropping.
* weights:     softmax over the k selected logits only.
* activation:  SwiGLU, a = silu(g) * u with silu(g) = g / (1 + exp(-g)),
               u = W_up x, g = W_gate x, then a is rounded to bf16 (RNE).
* down:        o = W_down a; y[t] = sum_j w[t][j] * o[t, j] + o_shared[t].
* shared:      one always-on expert, same SwiGLU FFN with bf16 weights, weight
               1.0, no gate.
* permutation: slots f = t*k + j grouped by expert with a stable counting sort
               (ascending f inside an expert); perm[p] = f, inv_perm[f] = p.
* stacking:    pre-norm residual h <- h + MoE(bf16(gamma * h / sqrt(mean(h^2)
               + eps))), h kept in fp32/fp64.
Rounding points: x is bf16 (given), a and the normed layer input are rounded
to bf16; everything else is fp64 here (fp32 on the GPU).
"""

import math

import numpy as np


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_bits_to_float(bits):
    """float64 values of bf16 bit patterns (uint16 array)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_rne(x):
    """Round float64 values to the nearest bf16 value (ties to even),
    returned as float64.  bf16 = 8 significant bits, fp32's exponent range
    (normal quantum 2^(E-7) for |x| in [2^E, 2^(E+1)), E >= -126; subnormal
    quantum 2^-133).  Values rounding past the largest finite bf16 become inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(xf)                   # |x| in [2^(e2-1), 2^e2)
    q_exp = np.maximum(e2 - 1 - 7, -133)
    q = np.ldexp(np.ones_like(xf), q_exp)
    r = np.rint(xf / q) * q               # exact scaling; rint = half-even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_rne_bits(x):
    """bf16 bit patterns (uint16) of float64 values rounded to nearest-even."""
    r = bf16_rne(x).astype(np.float32)     # bf16 values are exact in fp32
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def router_logits(x, w_r, b=None):
    """L = x W_r^T + b in fp64.  x [T][H], w_r [E][H], b [E] or None."""
    L = np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T
    if b is not None:
        L = L + np.asarray(b, dtype=np.float64)[None, :]
    return L


def topk_ids(L, k):
    """Exact top-k per row by (value descending, index ascending); pure
    Python sort, one row at a time.  Returns int64 [T][k]."""
    L = np.asarray(L)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    out = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        row = [float(v) for v in L[t]]
        out[t] = sorted(range(E), key=lambda e: (-row[e], e))[:k]
    return out


def topk_ids_fast(L, k):
    """Same selection as topk_ids, vectorised with a lexicographic sort."""
    L = np.asarray(L)
    T, E = L.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -L), axis=-1)
    return order[:, :k].astype(np.int64)


def softmax_selected(L, ids):
    """Softmax over the selected logits only (fp64).  Returns [T][k]."""
    sel = np.take_along_axis(np.asarray(L, dtype=np.float64), ids, axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


def permute(ids, n_experts):
    """Stable counting sort of the T*k slots by expert.

    Returns (offsets int64 [E+1], perm int64 [T*k], inv_perm int64 [T*k]):
    expert e owns perm[offsets[e]:offsets[e+1]], which lists its flat slot
    indices f = t*k + j in ascending order; inv_perm[perm[p]] = p."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    n = flat.size
    counts = [0] * n_experts
    for e in flat:
        counts[int(e)] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = list(offsets[:-1])
    perm = [0] * n
    for f in range(n):
        e = int(flat[f])
        perm[cursor[e]] = f
        cursor[e] += 1
    inv = [0] * n
    for p, f in enumerate(perm):
        inv[f] = p
    return (np.array(offsets, dtype=np.int64), np.array(perm, dtype=np.int64),
            np.array(inv, dtype=np.int64))


# --------------------------------------------------------------------------
# expert FFN
# --------------------------------------------------------------------------

def silu(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def swiglu_act(x_rows, w_up, w_gate):
    """a = bf16_RNE(silu(W_gate x) * (W_up x)) for each row of x ([R][H]).
    Returns [R][I] (bf16 values as float64)."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    u = x_rows @ np.asarray(w_up, dtype=np.float64).T
    g = x_rows @ np.asarray(w_gate, dtype=np.float64).T
    return bf16_rne(silu(g) * u)


def ffn(x_rows, w_up, w_gate, w_down):
    """SwiGLU expert FFN on rows of x: returns (a [R][I], o [R][H])."""
    a = swiglu_act(x_rows, w_up, w_gate)
    return a, a @ np.asarray(w_down, dtype=np.float64).T


def expert_ffn_perm(x, offsets, perm, k, get_expert):
    """Routed expert outputs in permuted order (unweighted).

    x [T][H]; offsets/perm from permute(); get_expert(e) -> (W_up, W_gate,
    W_down) as float64.  Returns (a_perm [T*k][I], y_perm [T*k][H])."""
    x = np.asarray(x, dtype=np.float64)
    n = len(perm)
    E = len(offsets) - 1
    a_perm = None
    y_perm = np.zeros((n, x.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wu, wg, wd = get_expert(e)
        toks = np.asarray(perm[lo:hi]) // k
        a, o = ffn(x[toks], wu, wg, wd)
        if a_perm is None:
            a_perm = np.zeros((n, a.shape[1]), dtype=np.float64)
        a_perm[lo:hi] = a
        y_perm[lo:hi] = o
    return a_perm, y_perm


def combine(y_perm, inv_perm, w, shared_y=None):
    """y[t] = sum_j w[t][j] * y_perm[inv_perm[t*k + j]] (+ shared_y[t])."""
    w = np.asarray(w, dtype=np.float64)
    T, k = w.shape
    y_perm = np.asarray(y_perm, dtype=np.float64)
    y = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            y[t] += w[t, j] * y_perm[int(inv_perm[t * k + j])]
    if shared_y is not None:
        y += np.asarray(shared_y, dtype=np.float64)
    return y


def layer_forward(x, k, get_expert, n_experts, logits=None, router_w=None,
                  router_b=None, shared=None, force_ids=None):
    """One routed MoE FFN layer.

    x [T][H] (bf16 values as float64); either `logits` [T][E] is given or
    router_w [E][H] (+ router_b [E]) computes them; get_expert(e) returns the
    dequantised (W_up, W_gate, W_down); shared = (W_up, W_gate, W_down) of the
    always-on expert or None.  `force_ids` [T][k] replaces the selection (used
    when a near-tie in the logits makes two valid selections differ).

    Returns a dict with logits, ids, w, offsets, perm, inv_perm, a_perm,
    y_perm, shared_a, shared_y and y (all fp64 / int64)."""
    x = np.asarray(x, dtype=np.float64)
    if logits is None:
        logits = router_logits(x, router_w, router_b)
    logits = np.asarray(logits, dtype=np.float64)
    ids = topk_ids_fast(logits, k) if force_ids is None else np.asarray(force_ids, dtype=np.int64)
    w = softmax_selected(logits, ids)
    offsets, perm, inv = permute(ids, n_experts)
    a_perm, y_perm = expert_ffn_perm(x, offsets, perm, k, get_expert)
    shared_a = shared_y = None
    if shared is not None:
        shared_a, shared_y = ffn(x, *shared)
    y = combine(y_perm, inv, w, shared_y)
    return dict(logits=logits, ids=ids, w=w, offsets=offsets, perm=perm,
                inv_perm=inv, a_perm=a_perm, y_perm=y_perm, shared_a=shared_a,
                shared_y=shared_y, y=y)


# --------------------------------------------------------------------------
# stacked layers
# --------------------------------------------------------------------------

def rmsnorm_bf16(h, gamma, eps=1e-6):
    """bf16_RNE(gamma * h / sqrt(mean(h^2) + eps)) per row, fp64 inside."""
    h = np.asarray(h, dtype=np.float64)
    r = np.sqrt((h * h).mean(axis=1, keepdims=True) + eps)
    return bf16_rne(np.asarray(gamma, dtype=np.float64)[None, :] * h / r)


def stack_step(h, gamma, eps, layer_fn):
    """One pre-norm residual step: h + layer_fn(rmsnorm_bf16(h))."""
    return np.asarray(h, dtype=np.float64) + layer_fn(rmsnorm_bf16(h, gamma, eps))


# --------------------------------------------------------------------------
# comparison metrics (tolerances of the parity tests)
# --------------------------------------------------------------------------

def rel_l2(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = math.sqrt(float((ref * ref).sum()))
    return math.sqrt(float(((y - ref) ** 2).sum())) / (den if den > 0 else 1.0)


def max_abs_over_rms(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float((ref * ref).mean()))
    return float(np.abs(y - ref).max()) / (rms if rms > 0 else 1.0)
