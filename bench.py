"""Benchmark of the routed, block-quantized MoE FFN layer on one MI355X.

Workload (the decode-shaped single layer at real shape): H=3072, 512 routed
experts (up|gate in the 3.25-bpw Q3S-256 codec, down in the 4-bit NL4-32
codec), top-10 with softmax over the selected logits, one always-on bf16
shared expert (I_s=512), I=512; router W_r bf16 [512][3072] plus a Zipf(1.0)
popularity bias; tokens bf16 N(0,1).  A step is one whole layer forward
(router, top-k, permutation, up|gate + SwiGLU, down, combine) over a batch of
T tokens, T = 8 for the headline value; T = 1, 3 and 5 are reported beside
it, and the 8192-token prefill chunk too (Zipf and uniform routing, the same
experts).  Decode steps rotate through 16
independently seeded layers (17.7 GB of packed experts) so the 256 MB
Infinity Cache cannot serve repeated experts; inputs are resident in HBM
before timing starts.

The roofline object is for the dominant kernel of the headline workload (the
up|gate kernel of the bandwidth path), its duration measured with HIP events
recorded by the library around that kernel on the caller's stream; its
algorithmic bytes are those of the experts the batch actually routes to.

results.stack_decode_T3 and results.stack_prefill_9536: the two 48-layer
workloads below, run inside the default line with 5 timed steps each
(--no-stacks skips them).

cpu_baseline: the CPU oracle (fp64 NumPy, dequantising from the packed bytes)
on T = 8 decode layers of the same workload, all host cores; results.cpu_oracle
adds the same sample on one thread and an expert sample of the 8192-token
prefill layer.

--stack-prefill runs the mixed-format workload instead and prints its own
JSON line: one 9536-token chunk through 48 layers whose routed experts use the
model card's per-layer formats (up|gate Q3S-256 / Q2S-256 / NL4-32, down
NL4-32 / Q2-32; seeded order), Zipf(0.8) routing, RMSNorm + residual between
layers (fused into each layer's last kernel by moe_layer_forward_residual), all
48 layers resident in HBM (about 51 GB).  A step is one pass
through the 48 layers; the roofline object is for the routed up|gate GEMMs
(MFMA-bound), their time summed over the layers of a pass.

--stack-decode runs the speculative-verify step instead (its own JSON line):
1 + K tokens (K drafts, --spec K, default 2) through 48 decode-shaped
Q3S-256 / NL4-32 layers, each independently seeded with a fresh Zipf(1.0)
bias, RMSNorm + residual between layers (fused as above), all 53 GB of
experts resident.  A
step is one 48-layer pass, captured once in a HIP graph and replayed (each
replay checked bit for bit against the eager pass, whose time is reported
beside it).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--stack-prefill | --stack-decode [--spec K]]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 matrix cores, vendor figure

# algorithmic bytes / flops (real shape: H=3072, I=512, E=512, k=10, I_s=512)
H, I, E, K, IS = 3072, 512, 512, 10, 512
UG_BYTES = 2 * I * (H // 256) * 104            # 1,277,952 packed up|gate bytes per expert
DN_BYTES = H * (I // 32) * 18                  # 884,736 packed down bytes per expert
SH_UG_BYTES = 2 * IS * H * 2                   # 6,291,456
SH_DN_BYTES = H * IS * 2                       # 3,145,728
ROUTER_BYTES = E * H * 2 + E * 4               # 3,147,776
FLOP_PER_TOKEN = K * 2 * 3 * H * I + 2 * 3 * H * IS + 2 * H * E   # 106,954,752


def stage1_bytes(T):
    """Stage 1: W_r and the shared up|gate rows read, x read, the logits, the
    shared up|gate partials (one per 256-wide K chunk) and the fp16 copy of x
    written."""
    return (ROUTER_BYTES + SH_UG_BYTES + T * H * 2 + T * E * 4 + (H // 256) * T * 2 * IS * 4
            + T * H * 2)


def upgate_bytes(T, U):
    """Up|gate kernel (bandwidth path, routing included): the logits, the packed
    up|gate of the U distinct routed experts, the tokens' fp16 rows and the
    shared partials read; a (fp16 routed, bf16 shared) written."""
    return (T * E * 4 + U * UG_BYTES + T * H * 2 + (H // 256) * T * 2 * IS * 4 + T * K * I * 2
            + T * IS * 2)


def down_bytes(T, U):
    """Down kernel: packed down of the U experts + shared down + a (routed
    fp16, shared bf16) read + unweighted outputs (permuted rows, shared) written."""
    return U * DN_BYTES + SH_DN_BYTES + T * K * I * 2 + T * IS * 2 + T * K * H * 4 + T * H * 4


def layer_bytes(T, U):
    """Whole layer: every distinct weight byte once + token in/out."""
    return U * (UG_BYTES + DN_BYTES) + SH_UG_BYTES + SH_DN_BYTES + ROUTER_BYTES + T * (H * 2 + H * 4)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=48)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--layers", type=int, default=16, help="decode layers rotated through")
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--prefill-only", action="store_true",
                   help="only the 8192-token prefill layer (profiler runs); prints its timings")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-stacks", action="store_true",
                   help="skip the two 48-layer workloads of the default run")
    p.add_argument("--host-gen", action="store_true",
                   help="build the synthetic layers on the host and copy them (profiler runs)")
    p.add_argument("--stack-prefill", action="store_true",
                   help="the 48-layer mixed-format 9536-token prefill chunk instead")
    p.add_argument("--stack-decode", action="store_true",
                   help="the 48-layer speculative-verify step instead")
    p.add_argument("--spec", type=int, default=2,
                   help="draft tokens of the verify step (tokens = 1 + spec, at most 15)")
    p.add_argument("--traffic-probe", action="store_true",
                   help="run only the workload read by rocprofv3 counter passes: decode T=8 "
                        "layers rotated as in the timed loop")
    p.add_argument("--copy-probe", action="store_true",
                   help="run only four 1 GiB device-to-device copies (the byte calibration "
                        "of the rocprofv3 traffic counters)")
    p.add_argument("--traffic-json", nargs=4,
                   metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="write profiles/traffic.json from the counter-collection CSVs of the "
                        "FETCH_SIZE and WRITE_SIZE passes over --traffic-probe and --copy-probe")
    p.add_argument("--summarize", nargs="+", metavar="CSV",
                   help="print per-(kernel, grid) tables of rocprofv3 kernel-trace or "
                        "counter-collection CSV files and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.summarize:
        for path in args.summarize:
            summarize_csv(path)
        return
    if args.traffic_json:
        write_traffic_json(*args.traffic_json)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU path); "
              "got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_expert_ffn_top_amd as Q
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_probe:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("# copy probe: 4 copies of %d bytes" % src.numel(), file=sys.stderr)
        return
    Q.load()
    if args.stack_prefill:
        stack_prefill(args, Q, synth, torch, np, dev)
        return
    if args.stack_decode:
        stack_decode(args, Q, synth, torch, np, dev)
        return
    sh = synth.REAL
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)

    t0 = time.time()
    if args.host_gen:
        # built on the host and copied: the only GPU kernels of the process are
        # then the library's and the runtime's copies (profiler runs)
        def host_layer(l):
            L = synth.real_layer(sh, 2, l, zipf_s=1.0, device="cpu")
            for f in ("experts", "router_w", "router_b", "shared_ug", "shared_down"):
                setattr(L, f, getattr(L, f).to(dev))
            return L
        layers = [host_layer(l) for l in range(args.layers)]
    else:
        layers = [synth.real_layer(sh, 2, l, zipf_s=1.0, device=dev) for l in range(args.layers)]
    wts = [Q.weights(L.experts, sh.expert_bytes, L.router_w, L.router_b, L.shared_ug,
                     L.shared_down) for L in layers]
    torch.cuda.synchronize()
    print("# generated %d layers in %.1f s" % (args.layers, time.time() - t0), file=sys.stderr)

    ws = Q.workspace(d, 8192, dev)
    stream = torch.cuda.current_stream(dev)

    def distinct_experts(T, x):
        us = []
        ids = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev)
        y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
        for l in range(args.layers):
            Q.moe_layer_forward(d, wts[l], x, y, ws, topk_ids_out=ids)
            us.append(int(torch.unique(ids).numel()))
        return us

    def time_steps(T, x, steps, warmup, nlay):
        y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
        for i in range(warmup):
            Q.moe_layer_forward(d, wts[i % nlay], x, y, ws)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            Q.moe_layer_forward(d, wts[i % nlay], x, y, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_kernels(T, x, steps, nlay, nev):
        """Per-kernel durations (ms) from events the library records between
        its kernels; averaged over `steps` calls."""
        y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        for row in evs:
            for ev in row:
                ev.record(stream)            # materialise the handles
        torch.cuda.synchronize()
        n_marks = None
        for i in range(steps):
            n_marks = Q.moe_layer_forward_timed(d, wts[i % nlay], x, y, ws,
                                                [ev.cuda_event for ev in evs[i]])
        torch.cuda.synchronize()
        dur = np.zeros(n_marks - 1)
        for row in evs:
            for j in range(n_marks - 1):
                dur[j] += row[j].elapsed_time(row[j + 1])
        return dur / steps

    if args.traffic_probe:
        x = synth.tokens_bf16(8, sh.hidden, 2, 0).to(dev)
        y = torch.empty((8, sh.hidden), dtype=torch.float32, device=dev)
        for i in range(2 * args.layers):
            Q.moe_layer_forward(d, wts[i % args.layers], x, y, ws)
        torch.cuda.synchronize()
        print("# traffic probe: %d decode layers at T=8" % (2 * args.layers), file=sys.stderr)
        return

    results = {"decode": {}, "prefill": None, "prefill_uniform": None}
    for T in (() if args.prefill_only else (1, 3, 5, 8)):
        x = synth.tokens_bf16(T, sh.hidden, 2, 0).to(dev)
        us = distinct_experts(T, x)
        ms = time_steps(T, x, args.steps, args.warmup, args.layers)
        U = float(np.mean(us))
        lb = layer_bytes(T, U)
        kd = time_kernels(T, x, max(args.layers, 16), args.layers, 8)
        names = ["stage1", "upgate", "down", "combine"]
        kern = {}
        for nm, t in zip(names, kd):
            kern[nm] = {"us": round(t * 1e3, 2)}
        for nm, b, j in (("stage1", stage1_bytes(T), 0), ("upgate", upgate_bytes(T, U), 1),
                         ("down", down_bytes(T, U), 2)):
            kern[nm]["GBps"] = round(b / (kd[j] * 1e-3) / 1e9, 1)
            kern[nm]["hbm_frac"] = round(b / (kd[j] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        results["decode"][T] = {
            "tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "distinct_experts_mean": U, "layer_bytes": int(lb),
            "layer_GBps": round(lb / (ms * 1e-3) / 1e9, 1),
            "layer_hbm_frac": round(lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels": kern, "_kd": kd, "_U": U,
        }
        print("# decode T=%d: %.4f ms/step, U=%.1f, %.0f GB/s layer, kernels %s" % (
            T, ms, U, lb / (ms * 1e-3) / 1e9, kern), file=sys.stderr)

    pre_sample = None
    if not args.no_prefill:
        Tp = 8192
        x = synth.tokens_bf16(Tp, sh.hidden, 3, 0).to(dev)
        L0 = layers[0]
        # the same experts and router with the Zipf bias (wts[0]) and with none
        # (uniform routing)
        w_uni = Q.weights(L0.experts, sh.expert_bytes, L0.router_w, torch.zeros_like(L0.router_b),
                          L0.shared_ug, L0.shared_down)
        for key, wl in (("prefill", wts), ("prefill_uniform", [w_uni])):
            saved = wts[0]
            wts[0] = wl[0]
            ms = time_steps(Tp, x, args.prefill_steps, 2, 1)
            kd = time_kernels(Tp, x, 4, 1, 12)
            wts[0] = saved
            names = ["router_shared_upgate", "topk_and_f16", "permute", "shared_down", "upgate",
                     "down", "down_fp32_if_needed", "combine"]
            flops = FLOP_PER_TOKEN * Tp
            ug_flops = 2.0 * Tp * K * 2 * I * H
            dn_flops = 2.0 * Tp * K * I * H
            kern = {nm: {"us": round(t * 1e3, 1)} for nm, t in zip(names, kd)}
            kern["upgate"]["TFLOPs"] = round(ug_flops / (kd[4] * 1e-3) / 1e12, 1)
            kern["down"]["TFLOPs"] = round(dn_flops / ((kd[5] + kd[6]) * 1e-3) / 1e12, 1)
            results[key] = {
                "tokens": Tp, "routing": "Zipf(1.0)" if key == "prefill" else "uniform",
                "tokens_per_s": round(Tp / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
                "algorithmic_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                "kernels": kern,
            }
            print("# %s T=%d: %.3f ms, %.1f TFLOP/s, kernels %s" % (
                key, Tp, ms, flops / (ms * 1e-3) / 1e12, kern), file=sys.stderr)
        if not args.no_cpu and not args.prefill_only:
            ids = torch.empty((Tp, sh.top_k), dtype=torch.int32, device=dev)
            y = torch.empty((Tp, sh.hidden), dtype=torch.float32, device=dev)
            Q.moe_layer_forward(d, wts[0], x, y, ws, topk_ids_out=ids)
            torch.cuda.synchronize()
            pre_sample = (L0, x, ids)

    if args.prefill_only:
        print(json.dumps({"prefill": results["prefill"], "prefill_uniform": results["prefill_uniform"]}))
        return
    # roofline of the dominant kernel of the headline workload (decode T=8)
    dec8 = results["decode"][8]
    kd8, U8 = dec8.pop("_kd"), dec8.pop("_U")
    for T in (1, 3, 5):
        results["decode"][T].pop("_kd")
        results["decode"][T].pop("_U")
    ub = upgate_bytes(8, U8)
    ach = ub / (kd8[1] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_for("k_upgate_dec", ub),
            "kernel": "k_upgate_dec (routed up|gate + SwiGLU, T=8)",
            "bytes_per_launch": int(ub), "us_per_launch": round(kd8[1] * 1e3, 2)}

    cpu = None if args.no_cpu else cpu_baseline(layers, sh)
    if not args.no_cpu:
        results["cpu_oracle"] = {"decode_T8_all_cores": cpu,
                                 "decode_T8_one_thread": cpu_baseline(layers, sh, min_s=6.0, threads=1)}
        if pre_sample is not None:
            results["cpu_oracle"]["prefill_8192_expert_sample"] = cpu_baseline_prefill(*pre_sample, sh)

    ms8 = dec8["ms_per_step"]
    line = {
        "metric": "MoE-layer tokens/s (decode, T=8)", "value": dec8["tokens_per_s"],
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms8, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "q3s/nl4 weights, fp16/bf16 mfma, fp32 accumulate", "data": "synthetic",
        "config": {"workload": "decode-shaped MoE layer: H=3072, E=512 routed (Q3S-256 up|gate, "
                               "NL4-32 down), top-10 + 1 shared bf16 expert, I=512, T=8 tokens, "
                               "Zipf(1.0) routing, 16 rotating layers",
                   "tokens": 8, "layers_rotated": args.layers},
        "roofline": roof, "cpu_baseline": cpu, "results": results,
    }
    if not args.no_stacks:
        # the two 48-layer workloads, with fewer steps, inside this line: the
        # speculative-verify step (T = 3, graph replay) and the mixed-format
        # 9536-token prefill chunk; the decode layers are freed first
        import argparse as _ap
        del layers, wts
        pre_sample = None
        torch.cuda.empty_cache()
        sargs = _ap.Namespace(**vars(args))
        sargs.steps, sargs.warmup, sargs.spec = 5, 1, 2
        for key, fn in (("stack_decode_T3", stack_decode), ("stack_prefill_9536", stack_prefill)):
            sl = fn(sargs, Q, synth, torch, np, dev, emit=False)
            results[key] = {"metric": sl["metric"], "value": sl["value"], "unit": sl["unit"],
                            "ms_per_step": sl["ms_per_step"], "steps": sl["steps"],
                            "workload": sl["config"]["workload"], "roofline": sl["roofline"],
                            "results": sl["results"]}
            del sl
            torch.cuda.empty_cache()
    print(json.dumps(line))


def stack_prefill(args, Q, synth, torch, np, dev, emit=True):
    """48 mixed-format layers, one 9536-token chunk (see the module header)."""
    wl = synth.WORKLOADS["stack_prefill"]
    T, seed, nl = wl.tokens[0], wl.seed, wl.layers
    t0 = time.time()
    layers, descs, wts, gammas = [], [], [], []
    for l in range(nl):
        sh = synth.stack_shape(seed, l)
        lay = synth.real_layer(sh, seed, l, zipf_s=wl.zipf_s, device=dev)
        layers.append(lay)
        descs.append(Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter,
                            sh.upgate_fmt, sh.down_fmt))
        wts.append(Q.weights(lay.experts, sh.expert_bytes, lay.router_w, lay.router_b,
                             lay.shared_ug, lay.shared_down))
        gammas.append(synth.norm_gain(sh.hidden, seed, l).to(dev))
    torch.cuda.synchronize()
    gb = sum(L.experts.numel() for L in layers) / 1e9
    print("# stack: generated %d layers (%.1f GB of packed experts) in %.1f s" % (
        nl, gb, time.time() - t0), file=sys.stderr)
    ws = torch.zeros(max(Q.moe_workspace_size(dd, T) for dd in descs), dtype=torch.uint8, device=dev)
    x0 = synth.tokens_bf16(T, H, seed).float().to(dev)
    h = torch.empty_like(x0)
    normed = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    normed2 = torch.empty_like(normed)

    def one_pass(timed_events=None):
        # h += MoE_l(norm_l(h)): the layer call adds its output to h and writes
        # the next layer's normalised input (two buffers in turn); the pass
        # with per-kernel events runs the unfused pair of calls instead
        h.copy_(x0)
        marks = []
        Q.moe_rmsnorm_residual(h, None, gammas[0], 1e-6, normed)
        nin, nout = normed, normed2
        for l in range(nl):
            last = l + 1 == nl
            if timed_events is None:
                Q.moe_layer_forward_residual(descs[l], wts[l], nin, h, ws,
                                             gamma=None if last else gammas[l + 1], eps=1e-6,
                                             normed=None if last else nout)
                nin, nout = nout, nin
            else:
                marks.append(Q.moe_layer_forward_timed(descs[l], wts[l], normed, y, ws,
                                                       [ev.cuda_event for ev in timed_events[l]]))
                Q.moe_rmsnorm_residual(h, y, None if last else gammas[l + 1], 1e-6,
                                       None if last else normed)
        return marks

    for _ in range(max(1, args.warmup // 8)):
        one_pass()
    torch.cuda.synchronize()
    steps = max(1, args.steps // 16)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert bool(torch.isfinite(h).all())

    # per-kernel times of one pass, grouped by the layer's up|gate and down formats
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(12)] for _ in range(nl)]
    for row in evs:
        for ev in row:
            ev.record(stream)
    torch.cuda.synchronize()
    marks = one_pass(evs)
    torch.cuda.synchronize()
    names = ["router_shared_upgate", "topk_and_f16", "permute", "shared_down", "upgate", "down",
             "down_fp32_if_needed", "combine"]
    fmt_name = {2: "q3s256", 3: "nl4_32", 4: "q2s256", 5: "q2_32", 6: "q3k256", 7: "nl4s256"}
    ug_t, dn_t, ug_by, dn_by, tot = {}, {}, {}, {}, {}
    for l in range(nl):
        dur = [evs[l][j].elapsed_time(evs[l][j + 1]) for j in range(marks[l] - 1)]
        for nm, t in zip(names, dur):
            tot[nm] = tot.get(nm, 0.0) + t
        u, dn = descs[l].upgate_fmt, descs[l].down_fmt
        ug_t.setdefault(fmt_name[u], []).append(dur[4])
        dn_t.setdefault(fmt_name[dn], []).append(dur[5] + dur[6])
    ug_flops = 2.0 * T * K * 2 * I * H            # per layer
    dn_flops = 2.0 * T * K * I * H
    per_fmt = {"upgate": {f: {"layers": len(v), "us_mean": round(1e3 * np.mean(v), 1),
                               "TFLOPs": round(ug_flops / (np.mean(v) * 1e-3) / 1e12, 1)}
                          for f, v in ug_t.items()},
               "down": {f: {"layers": len(v), "us_mean": round(1e3 * np.mean(v), 1),
                             "TFLOPs": round(dn_flops / (np.mean(v) * 1e-3) / 1e12, 1)}
                        for f, v in dn_t.items()}}
    ug_sum = sum(sum(v) for v in ug_t.values())
    ach = ug_flops * nl / (ug_sum * 1e-3) / 1e12
    flops = FLOP_PER_TOKEN * T * nl
    line = {
        "metric": "MoE-stack prefill tokens/s (48 mixed-format layers, one 9536-token chunk)",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": max(1, args.warmup // 8), "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "q3s/q2s/nl4/q2 weights, fp16/bf16 mfma, fp32 accumulate", "data": "synthetic",
        "config": {"workload": "48 MoE layers H=3072, E=512 (top-10) + 1 shared bf16 expert, "
                               "I=512, per-layer expert formats, 9536 tokens, Zipf(0.8), "
                               "RMSNorm + residual", "tokens": T, "layers": nl,
                   "packed_expert_GB": round(gb, 2)},
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "k_gemm routed up|gate (Q3S / Q2S / NL4 modes), summed over a pass"},
        "cpu_baseline": None,
        "results": {"algorithmic_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                    "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                    "kernel_ms_per_pass": {k: round(v, 3) for k, v in tot.items()},
                    "per_format": per_fmt},
    }
    print("# stack prefill: %.2f ms per 48-layer pass, per format %s" % (ms, per_fmt), file=sys.stderr)
    if emit:
        print(json.dumps(line))
    return line


def stack_decode(args, Q, synth, torch, np, dev, emit=True):
    """48 decode-shaped layers, 1 + spec tokens per step (see the module header)."""
    wl = synth.WORKLOADS["stack"]
    seed, nl = wl.seed, wl.layers
    if not 0 <= args.spec <= 15:
        sys.exit("--spec must be in [0, 15] (the bandwidth path takes up to 16 tokens)")
    T = 1 + args.spec
    sh = synth.REAL
    t0 = time.time()
    layers = [synth.real_layer(sh, seed, l, zipf_s=wl.zipf_s, device=dev) for l in range(nl)]
    wts = [Q.weights(L.experts, sh.expert_bytes, L.router_w, L.router_b, L.shared_ug, L.shared_down)
           for L in layers]
    gammas = [synth.norm_gain(sh.hidden, seed, l).to(dev) for l in range(nl)]
    torch.cuda.synchronize()
    gb = sum(L.experts.numel() for L in layers) / 1e9
    print("# stack decode: generated %d layers (%.1f GB of packed experts) in %.1f s" % (
        nl, gb, time.time() - t0), file=sys.stderr)
    d = Q.desc(sh.hidden, sh.inter, sh.n_experts, sh.top_k, sh.shared_inter)
    ws = Q.workspace(d, T, dev)
    x0 = synth.tokens_bf16(T, H, seed).float().to(dev)
    h = torch.empty_like(x0)
    normed = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    normed2 = torch.empty_like(normed)

    def one_pass(count=False):
        # h += MoE_l(norm_l(h)): the layer call adds its output to h and writes
        # the next layer's normalised input (two buffers in turn)
        h.copy_(x0)
        us = []
        Q.moe_rmsnorm_residual(h, None, gammas[0], 1e-6, normed)
        nin, nout = normed, normed2
        for l in range(nl):
            last = l + 1 == nl
            Q.moe_layer_forward_residual(d, wts[l], nin, h, ws, gamma=None if last else gammas[l + 1],
                                         eps=1e-6, normed=None if last else nout,
                                         topk_ids_out=ids if count else None)
            if count:
                us.append(int(torch.unique(ids).numel()))
            nin, nout = nout, nin
        return us

    us = one_pass(count=True)
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    h_eager = h.clone()
    steps = max(1, args.steps)

    def timed(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_eager = timed(one_pass)
    # the whole step (48 layers of 4 launches each, the last one carrying the
    # residual add and the next norm, plus the first norm) captured once
    # in a HIP graph and replayed; every replay is checked against the eager
    # pass (the kernels are deterministic)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        one_pass()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        one_pass()
    for _ in range(3):
        h.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(h, h_eager):
            sys.exit("graph replay differs from the eager step")
    ms = timed(graph.replay)
    assert bool(torch.isfinite(h).all())
    U = float(np.mean(us))
    step_bytes = sum(layer_bytes(T, u) for u in us)
    line = {
        "metric": "speculative-verify step tokens/s (48 decode layers, %d tokens)" % T,
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "q3s/nl4 weights, fp16/bf16 mfma, fp32 accumulate", "data": "synthetic",
        "config": {"workload": "48 MoE layers H=3072, E=512 (Q3S-256 up|gate, NL4-32 down), top-10 "
                               "+ 1 shared bf16 expert, I=512, %d tokens (1 + %d drafts), Zipf(1.0) "
                               "per layer, RMSNorm + residual" % (T, T - 1), "tokens": T, "layers": nl,
                   "packed_expert_GB": round(gb, 2)},
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole step (all kernels of the 48 layers), algorithmic bytes"},
        "cpu_baseline": None,
        "results": {"distinct_experts_mean": U, "step_bytes": int(step_bytes),
                    "us_per_layer": round(ms * 1e3 / nl, 2), "graph_replay": True,
                    "ms_per_step_eager": round(ms_eager, 4)},
    }
    print("# stack decode: %.3f ms per 48-layer step (graph replay; eager %.3f ms), U = %.1f, "
          "%.0f GB/s" % (ms, ms_eager, U, step_bytes / (ms * 1e-3) / 1e9), file=sys.stderr)
    if emit:
        print(json.dumps(line))
    return line


def summarize_csv(path):
    """Group a rocprofv3 CSV by (kernel, grid size): dispatch count and mean /
    min / max duration (kernel trace), or mean value per counter (counter
    collection).  Kernels of the library only, plus the runtime's copy kernel."""
    import collections
    import csv
    rows = list(csv.DictReader(open(path)))
    if not rows:
        print("%s: empty" % path)
        return
    cols = rows[0].keys()
    gcols = [c for c in cols if c.startswith("Grid_Size")]

    def short(name):
        name = name.split("(")[0]
        return name.replace("void ", "").replace("moe::", "")

    def keep(name):
        return "moe::" in name or "copyBuffer" in name

    def grid(r):
        g = 1
        for c in gcols:
            g *= max(int(float(r[c])), 1)
        return g

    print("### %s" % os.path.basename(path))
    if "Counter_Name" in cols:
        agg = collections.defaultdict(list)
        for r in rows:
            if keep(r["Kernel_Name"]):
                agg[(short(r["Kernel_Name"]), grid(r), r["Counter_Name"])].append(
                    float(r["Counter_Value"]))
        print("| kernel | grid (work-items) | counter | dispatches | mean per dispatch |")
        print("|---|---|---|---|---|")
        for (k, g, c), v in sorted(agg.items()):
            print("| %s | %d | %s | %d | %.6g |" % (k, g, c, len(v), sum(v) / len(v)))
    else:
        # every kernel of a layer forward is tagged with the batch of the layer:
        # the token count T of the combine kernel that ends it (its grid holds
        # ceil(H / 1024) blocks of 256 per token)
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        tag = [None] * len(rows)
        nxt = None
        for i in range(len(rows) - 1, -1, -1):
            if "k_combine" in rows[i]["Kernel_Name"]:
                nxt = grid(rows[i]) // (256 * ((H + 1023) // 1024))
            tag[i] = nxt
        agg = collections.defaultdict(list)
        for r, t in zip(rows, tag):
            if keep(r["Kernel_Name"]):
                agg[(short(r["Kernel_Name"]), grid(r), t)].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print("| kernel | grid (work-items) | layer T | dispatches | mean us | min us | max us |")
        print("|---|---|---|---|---|---|---|")
        for (k, g, t), v in sorted(agg.items(), key=lambda kv: (kv[0][0], kv[0][1], kv[0][2] or 0)):
            print("| %s | %d | %s | %d | %.2f | %.2f | %.2f |" % (k, g, t if t else "-", len(v),
                                                                 sum(v) / len(v), min(v), max(v)))
    print()


def counter_means(path, counter, count=False):
    """Mean per dispatch of `counter` (summed over its rows within a dispatch),
    per kernel name, from a rocprofv3 counter-collection CSV (count: the
    number of dispatches instead)."""
    import collections
    import csv
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("moe::", "")
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    return {k: (len(v) if count else sum(v) / len(v)) for k, v in out.items()}


TRAFFIC_SOURCES = ["moe_common.hpp", "moe_decoders.hpp", "moe_kernels.hpp", "moe_kernels_decode.hip"]


def write_traffic_json(fetch_csv, write_csv, cfetch_csv, cwrite_csv):
    """HBM bytes per launch of the three decode kernels from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a 1 GiB device copy (1,048,576 KiB read and written)."""
    fetch, write = counter_means(fetch_csv, "FETCH_SIZE"), counter_means(write_csv, "WRITE_SIZE")
    ndisp = {k: n for k, n in counter_means(fetch_csv, "FETCH_SIZE", count=True).items()}
    ndisp = {kern: next((n for k, n in ndisp.items() if k.startswith(kern)), 0)
             for kern in ("k_dec_stage1", "k_upgate_dec", "k_down_dec")}
    cf = [v for k, v in counter_means(cfetch_csv, "FETCH_SIZE").items() if "copyBuffer" in k]
    cw = [v for k, v in counter_means(cwrite_csv, "WRITE_SIZE").items() if "copyBuffer" in k]
    ff, wf = 1048576.0 / max(cf), 1048576.0 / max(cw)
    sha = source_digest(TRAFFIC_SOURCES)
    out = {}
    for kern in ("k_dec_stage1", "k_upgate_dec", "k_down_dec"):
        fk = [v for k, v in fetch.items() if k.startswith(kern)]
        wk = [v for k, v in write.items() if k.startswith(kern)]
        if not fk or not wk:
            continue
        out[kern] = {
            "sources": TRAFFIC_SOURCES, "sources_sha256": sha,
            "hbm_bytes_per_launch": int(round((fk[0] * ff + wk[0] * wf) * 1024)),
            "fetch_kib_per_dispatch": round(fk[0], 2), "write_kib_per_dispatch": round(wk[0], 2),
            "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
            "workload": "decode layer, T=8 tokens, %d launches over %d rotating layers "
                        "(bench.py --traffic-probe --host-gen --layers %d)" % (
                            ndisp[kern], ndisp[kern] // 2, ndisp[kern] // 2)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote %s: %s" % (path, {k: v["hbm_bytes_per_launch"] for k, v in out.items()}))


def source_digest(files):
    """sha256 over the named kernel sources, in order (the kernel's identity)."""
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "quantized_expert_ffn_top_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_for(kernel, algo_bytes):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[kernel]
        sha = source_digest(rec["sources"])
    except (OSError, KeyError, ValueError):
        return None
    if sha != rec.get("sources_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(layers, sh, min_s=10.0, threads=None):
    """The oracle as it stands, on decode layers of the workload (T = 8 tokens
    each, layer after layer until at least `min_s` seconds of CPU work), with
    the BLAS on `threads` threads (default: every core the process may use)."""
    import numpy as np
    import torch

    import synth
    from oracle import formats as OF
    from oracle import moe as OM
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                                     # pragma: no cover
        threadpool_limits = None
    cores = threads or len(os.sched_getaffinity(0))
    T = 8
    x = synth.tokens_bf16(T, sh.hidden, 2, 0)

    def bf(t):
        return OM.bf16_bits_to_float(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))

    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    t0 = time.time()
    done = 0
    try:
        for layer in layers:
            cache = {}

            def get(e, layer=layer, cache=cache):
                if e not in cache:
                    cache[e] = OF.expert_matrices(layer.experts[e].cpu().numpy(), sh.hidden,
                                                  sh.inter)
                return cache[e]

            ug = bf(layer.shared_ug)
            shared = (ug[:sh.shared_inter], ug[sh.shared_inter:], bf(layer.shared_down))
            OM.layer_forward(bf(x), sh.top_k, get, sh.n_experts, router_w=bf(layer.router_w),
                             router_b=layer.router_b.cpu().numpy().astype(np.float64),
                             shared=shared)
            done += 1
            if time.time() - t0 >= min_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.time() - t0
    return {"value": round(done * T / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d decode layers of the workload, T=8 tokens each (router, top-k, ~60 "
                      "routed experts dequantised from their packed bytes, shared expert), "
                      "fp64 NumPy, %.1f s" % (done, dt)}


def cpu_baseline_prefill(layer, x, ids, sh, min_s=10.0):
    """The oracle on an expert sample of the 8192-token prefill layer: experts
    taken in id order, each dequantised from its packed bytes and run (SwiGLU
    FFN, fp64) on all of its routed rows, until at least `min_s` seconds; the
    router, top-k and shared expert are not in the sample.  tokens/s = the
    rows processed / k / time."""
    import numpy as np
    import torch

    from oracle import formats as OF
    from oracle import moe as OM
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                                     # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    xs = OM.bf16_bits_to_float(x.detach().cpu().view(torch.int16).numpy().view(np.uint16))
    ids = ids.cpu().numpy()
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    t0 = time.time()
    rows = experts = 0
    try:
        for e in range(sh.n_experts):
            toks = np.nonzero((ids == e).any(axis=1))[0]
            if len(toks) == 0:
                continue
            wu, wg, wd = OF.expert_matrices(layer.experts[e].cpu().numpy(), sh.hidden, sh.inter)
            OM.ffn(xs[toks], wu, wg, wd)
            rows += len(toks)
            experts += 1
            if time.time() - t0 >= min_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.time() - t0
    return {"value": round(rows / sh.top_k / dt, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": "routed experts of the 8192-token prefill layer in id order, each "
                      "dequantised and run on all its rows: %d experts, %d rows (of %d), "
                      "fp64 NumPy, %.1f s" % (experts, rows, ids.size, dt)}


if __name__ == "__main__":
    main()
