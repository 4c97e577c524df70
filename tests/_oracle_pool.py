"""The oracle's routed expert FFNs over a whole prefill-sized batch, one expert
at a time in a pool of worker processes.

Every worker regenerates the seeded tokens once, then for each expert it is
handed rebuilds that expert's packed record from the seeded generator,
dequantises it with the oracle's vectorised decoder, runs the oracle's SwiGLU
FFN (fp64) on the expert's token rows and returns the unweighted down rows;
nothing is cached, so memory stays at one expert per worker.  The arithmetic
is the oracle's own (oracle.formats.expert_matrices, oracle.moe.ffn); this
module only splits the experts over processes.
"""

import multiprocessing as mp
import os
import sys
import time

_STATE = {}


def _init(shape, seed, layer, mode, T):
    # one thread per worker: the workers already fill the cores, and torch
    # (the generator's counter hash) and the BLAS would each start a team of
    # OMP_NUM_THREADS threads per worker otherwise
    import torch
    torch.set_num_threads(1)
    try:
        from threadpoolctl import threadpool_limits
        _STATE["limits"] = threadpool_limits(limits=1)
    except ImportError:                                  # pragma: no cover
        pass
    import numpy as np

    import synth
    from oracle import moe as OM
    x = synth.tokens_bf16(T, shape.hidden, seed)
    _STATE.update(shape=shape, seed=seed, layer=layer, mode=mode,
                  x=OM.bf16_bits_to_float(x.view(__import__("torch").int16).numpy().view(np.uint16)))


def _expert(task):
    import synth
    from oracle import formats as OF
    from oracle import moe as OM
    e, toks = task
    sh = _STATE["shape"]
    rec = synth.expert_record(sh, _STATE["seed"], _STATE["layer"], e, mode=_STATE["mode"]).numpy()
    wu, wg, wd = OF.expert_matrices(rec, sh.hidden, sh.inter, sh.upgate_fmt, sh.down_fmt)
    _, o = OM.ffn(_STATE["x"][toks], wu, wg, wd)
    return e, o


def workers():
    """Worker count: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def routed_outputs(shape, seed, layer, mode, T, offsets, perm, k):
    """y_perm fp64 [T*k][H] (unweighted, permuted rows) of the layer whose
    tokens are synth.tokens_bf16(T, H, seed) and whose experts are
    synth.expert_record(shape, seed, layer, e, mode), for the permutation
    (offsets, perm) of the oracle's counting sort."""
    import numpy as np
    n = len(perm)
    y_perm = np.zeros((n, shape.hidden), dtype=np.float64)
    tasks = []
    for e in range(shape.n_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            tasks.append((e, np.asarray(perm[lo:hi]) // k))
    tasks.sort(key=lambda t: -len(t[1]))               # the largest groups first
    ctx = mp.get_context("spawn")
    t0 = time.time()
    nw = workers()
    with ctx.Pool(nw, initializer=_init, initargs=(shape, seed, layer, mode, T)) as pool:
        for i, (e, o) in enumerate(pool.imap_unordered(_expert, tasks, chunksize=1)):
            y_perm[int(offsets[e]):int(offsets[e + 1])] = o
            if i % 64 == 63 or i + 1 == len(tasks):
                # progress on the process's own stderr (a test runner's
                # capture does not hold it back)
                print("[oracle pool] %d of %d experts, %d workers, %.1f s" % (
                    i + 1, len(tasks), nw, time.time() - t0), file=sys.__stderr__, flush=True)
    return y_perm
