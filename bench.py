"""Benchmark: triangle attention forward + backward on one MI355X.

One step is the whole hot path on one batch of resident synthetic input: the forward
(bias conversion + attention kernel) and the backward (bias conversion, the query-tile kernel
for dq and the correction D, the key-tile-parallel kernel for dk, dv and the dbias partials, the
ordered sum of the dbias partials).  W untimed warm-up steps, then exactly K timed steps
bracketed by torch.cuda.synchronize().

Throughput is credited with the method's FLOP convention: 4*B*N^3*H*d for the forward
(Q K^T and P V) and 2.5x that for the backward (five products), whatever the kernels
actually execute.  The roofline object reports the dominant kernel, the backward's
key-tile-parallel kernel, credited with the four products it runs (S and dP recomputed, dV,
dK: 8*B*N^3*H*d), against the published dense bf16 MFMA peak, with its duration from HIP
events recorded on the launch stream around that kernel (the backward's MAIN stage, one
launch) in every timed step.

Prints one JSON line.  Only one GPU is used: --gpus above 1 exits with a message.

With --op trimul the same contract covers the triangle multiplication core instead: a step is
the forward and backward of both directions (outgoing, incoming) at the trimul workload,
credited with 2*B*N^3*C flop per forward product and twice that per backward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "triangle-attn fwd+bwd TFLOPS & % bf16 MFMA peak at N=768 H=4 d=32, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak (2.5 PFLOP/s)
HEADLINE = "n768_h4_d32"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_main_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "triangle_attention_amd", "csrc", "tri_attn.hip")
TRIMUL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "trimul_traffic.json")
TRIMUL_SRC = os.path.join(ROOT, "triangle_attention_amd", "csrc", "tri_mul.hip")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=30, help="untimed steps; the GPU needs about 30 to reach its steady clock")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-residual", action="store_true", help="uncompensated backward correction")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle CPU-baseline budget (0 = skip)")
    ap.add_argument("--cpu-protocol", nargs="*", default=None, metavar="WORKLOAD",
                    help="only time the FP64 oracle on whole workloads (all five by default), forward and "
                         "backward apart, and print one JSON line per workload")
    ap.add_argument("--graph", action="store_true",
                    help="also time the whole fwd+bwd step captured in one HIP graph (small-N launch latency)")
    ap.add_argument("--op", choices=("attention", "trimul"), default="attention")
    ap.add_argument("--trimul-workload", default="trimul_n768_c128")
    ap.add_argument("--trimul-layout", choices=("channels_first", "channels_last"), default="channels_first")
    ap.add_argument("--trimul-direct", action="store_true",
                    help="channels last without a workspace (the in-place kernel instead of the layout change)")
    return ap.parse_args()


def _src_hash(path: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic(bytes_alg: float, path: str = TRAFFIC_FILE, src: str = KERNEL_SRC, key: str | None = None):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter runs,
    valid only while the kernel source is the one the counters were taken on."""
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != _src_hash(src):
        return None
    if key is not None:
        t = t.get(key) or {}
    return t.get("hbm_bytes_per_launch")


def cpu_info() -> dict:
    """The host the oracle runs on: CPU model, usable cores, BLAS library and its thread count."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                blas = f"{d.get('internal_api')} {d.get('version')}"
                threads = max(threads or 0, int(d.get("num_threads", 1)))
    except Exception:
        pass
    host = len(os.sched_getaffinity(0))
    return {"cpu_model": model, "host_cores": host, "blas": blas, "blas_threads": threads or host}


def cpu_baseline(w, inp, budget_s: float):
    """The FP64 oracle as it stands, slice by slice (all heads), forward then backward, until the
    budget is spent; forward and backward timed apart.  The backward of a slice recomputes its
    forward, as the oracle is written."""
    import oracle
    from tri_synth import bf16_bits_to_f64
    info = cpu_info()
    x = {n: bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "bias", "dO")}
    m = inp["key_mask"]
    t_f = t_b = 0.0
    done = 0
    t0 = time.perf_counter()
    for i in range(w.N):
        for h in range(w.H):
            mrow = None if m is None else m[0, i]
            a = time.perf_counter()
            oracle.slice_forward64(x["q"][0, i, h], x["k"][0, i, h], x["v"][0, i, h], x["bias"][0, h], mrow)
            b = time.perf_counter()
            oracle.slice_backward64(x["q"][0, i, h], x["k"][0, i, h], x["v"][0, i, h], x["bias"][0, h],
                                    x["dO"][0, i, h], mrow)
            t_f += b - a
            t_b += time.perf_counter() - b
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    per = w.N * w.N * w.H * w.D * done  # score elements x d of the sample
    f_fwd, f_bwd = 4.0 * per, 10.0 * per
    return {"value": (f_fwd + f_bwd) / (t_f + t_b) / 1e12, "unit": "TFLOP/s", "cores": int(info["blas_threads"]),
            "kind": "oracle",
            "sample": f"{done} of {w.N} slices x {w.H} heads of {w.name}, forward then backward in FP64 "
                      f"({t_f + t_b:.1f} s)",
            "fwd_tflops": f_fwd / t_f / 1e12, "bwd_tflops": f_bwd / t_b / 1e12, **info}


def cpu_protocol(names):
    """The oracle on whole workloads, forward and backward timed apart: median of three runs for
    the small workloads, one run for crop 768.  One JSON line per workload."""
    import statistics
    import oracle
    from tri_synth import WORKLOADS, bf16_bits_to_f64, workload_inputs
    info = cpu_info()
    for name in names:
        w = WORKLOADS[name]
        inp = workload_inputs(w)
        x = {n: bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "bias", "dO")}
        m = inp["key_mask"]
        runs = 1 if w.N >= 768 else 3
        tf, tb = [], []
        for _ in range(runs):
            a = time.perf_counter()
            oracle.forward64(x["q"], x["k"], x["v"], x["bias"], m)
            b = time.perf_counter()
            oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], m)
            tf.append(b - a)
            tb.append(time.perf_counter() - b)
        f, b_ = statistics.median(tf), statistics.median(tb)
        print(json.dumps({"workload": name, "runs": runs, "t_fwd_s": round(f, 3), "t_bwd_s": round(b_, 3),
                          "fwd_gflops": round(w.flops_fwd / f / 1e9, 2), "bwd_gflops": round(w.flops_bwd / b_ / 1e9, 2),
                          "fwd_bwd_s": round(f + b_, 3), **info}), flush=True)


def trimul_cpu_baseline(a64, b64, dx64, budget_s: float):
    """The FP64 trimul oracle as it stands, both directions fwd+bwd, one channel at a time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    B, N, _, C = a64.shape
    t0 = time.perf_counter()
    done = 0
    for c in range(C):
        sl = (Ellipsis, slice(c, c + 1))
        for direction in ("outgoing", "incoming"):
            oracle.tri_mul_forward64(a64[sl], b64[sl], direction)
            oracle.tri_mul_backward64(a64[sl], b64[sl], dx64[sl], direction)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 12.0 * B * N ** 3 * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {C} channels, both directions fwd+bwd in FP64 ({dt:.1f} s)"}


def main_trimul(args):
    import torch
    import triangle_attention_amd as ta
    from tri_synth import TRIMUL_WORKLOADS, bf16_bits_to_f64, make_pair_inputs

    w = TRIMUL_WORKLOADS[args.trimul_workload]
    B, N, C = w["B"], w["N"], w["C"]
    inp = make_pair_inputs(B, N, C, seed=w["seed"])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    first = args.trimul_layout == "channels_first"

    def dt(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return t.permute(0, 3, 1, 2).contiguous() if first else t

    a, b, dx = dt(inp["a"]), dt(inp["b"]), dt(inp["dx"])
    outs = {d: [torch.empty_like(a) for _ in range(3)] for d in ("outgoing", "incoming")}
    lay = ta.TRI_MUL_LAYOUTS[args.trimul_layout]
    nws = 0 if args.trimul_direct else ta.tri_mul_workspace_bytes(lay, B, N, C)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    stream = torch.cuda.current_stream()

    def mk(direction, fwd):
        d = ta.TRI_MUL_DIRECTIONS[direction]
        x, da, db = outs[direction]

        def call():
            sh = torch.cuda.current_stream().cuda_stream
            st = (ta.tri_mul_fwd(d, lay, B, N, C, a, b, x, ws, nws, stream=sh) if fwd
                  else ta.tri_mul_bwd(d, lay, B, N, C, a, b, dx, da, db, ws, nws, stream=sh))
            if st:
                raise ta.TriAttnError(st, "tri_mul")
        return call

    calls = [mk("outgoing", True), mk("outgoing", False), mk("incoming", True), mk("incoming", False)]
    names = ["out_fwd", "out_bwd", "in_fwd", "in_bwd"]
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for n_, c in enumerate(calls):
            c()
            ev[s][n_ + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = ev[0][0].elapsed_time(ev[-1][-1]) / args.steps
    stage_ms = {names[n_]: float(np.mean([ev[s][n_].elapsed_time(ev[s][n_ + 1]) for s in range(args.steps)]))
                for n_ in range(len(calls))}
    prod = 2.0 * B * N ** 3 * C  # flop of one product (one forward; a backward runs two)
    flops = 2 * (prod + 2 * prod)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # dominant kernel: one product launch (the forward call is one launch); its algorithmic
    # HBM bytes are the two operands read once and the output written once
    launch_ms = 0.5 * (stage_ms["out_fwd"] + stage_ms["in_fwd"])
    alg_bytes = 3.0 * B * N * N * C * 2
    gbs = alg_bytes / (launch_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(gbs / 8000.0, 4),
                # the committed counter runs cover the 768 x 128 workload only
                "traffic": (_traffic(None, TRIMUL_TRAFFIC_FILE, TRIMUL_SRC, key=f"{args.trimul_layout}_fwd")
                            if args.trimul_workload == "trimul_n768_c128" else None),
                "kernel": f"tri_mul {'channels-first' if first else 'channels-last'} product (one launch)",
                "per_launch_bytes": alg_bytes, "per_launch_flop": prod, "avg_launch_ms": round(launch_ms, 4),
                "mfma_tflops": round(prod / (launch_ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(prod / (launch_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    graph = None
    if args.graph:  # the step's four calls captured once and replayed (small-N launch latency)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in calls:
                c()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        g_ms = e0.elapsed_time(e1) / args.steps
        graph = {"ms_per_step": round(g_ms, 4), "value": round(flops / (g_ms * 1e-3) / 1e12, 2),
                 "unit": "TFLOP/s", "eager_ms_per_step": round(ms_per_step, 4)}
    cpu = None
    if args.cpu_seconds > 0:
        a64, b64, dx64 = (bf16_bits_to_f64(inp[n]) for n in ("a", "b", "dx"))
        cpu = trimul_cpu_baseline(a64, b64, dx64, args.cpu_seconds)
    out = {
        "metric": "triangle-multiplication core fwd+bwd TFLOPS (outgoing + incoming), 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.trimul_workload, "B": B, "N": N, "C": C, "layout": args.trimul_layout,
                   "channels_last_path": None if first else ("direct" if ws is None else "workspace")},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {k_: round(v_, 4) for k_, v_ in stage_ms.items()},
        "wall_s_timed_region": round(wall, 4), "roofline": roofline, "cpu_baseline": cpu,
    }
    if graph is not None:
        out["graph"] = graph
    print(json.dumps(out), flush=True)


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    if args.cpu_protocol is not None:
        cpu_protocol(args.cpu_protocol or ["n64_h4_d16", "n384_h4_d32", "n640_h4_d16_mask64", "n768_h4_d32",
                                           "n768_h4_d16_bias4"])
        return
    if args.op == "trimul":
        main_trimul(args)
        return

    import torch
    import triangle_attention_amd as ta
    from tri_synth import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    inp = workload_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dt(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, bias, dO = (dt(inp[n]) for n in ("q", "k", "v", "bias", "dO"))
    mask = None if inp["key_mask"] is None else torch.from_numpy(inp["key_mask"]).to(dev)
    B, N, H, D = w.B, w.N, w.H, w.D
    o = torch.empty_like(q)
    res = None if args.no_residual else torch.empty_like(q)
    lse = torch.empty((B, N, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dbias = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    fws = torch.empty(ta.tri_attn_fwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device=dev)
    bws = torch.empty(ta.tri_attn_bwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # each call enqueues on the stream current at call time (the capture stream under --graph)
    def fwd(stage):
        st = ta.tri_attn_fwd_stages(stage, B, N, H, D, q, k, v, bias, mask, o, lse, res, fws, fws.numel(),
                                    torch.cuda.current_stream().cuda_stream)
        if st:
            raise ta.TriAttnError(st, "tri_attn_fwd_stages")

    def bwd(stage):
        st = ta.tri_attn_bwd_stages(stage, B, N, H, D, q, k, v, bias, mask, o, lse, res, dO, dq, dk, dv, dbias,
                                    bws, bws.numel(), torch.cuda.current_stream().cuda_stream)
        if st:
            raise ta.TriAttnError(st, "tri_attn_bwd_stages")

    calls = [lambda: fwd(ta.STAGE_PREP), lambda: fwd(ta.STAGE_MAIN), lambda: bwd(ta.STAGE_PREP),
             lambda: bwd(ta.STAGE_MAIN), lambda: bwd(ta.STAGE_FINAL)]
    names = ["fwd_prep", "fwd_main", "bwd_prep", "bwd_main", "bwd_final"]

    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for n_, c in enumerate(calls):
            c()
            ev[s][n_ + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = ev[0][0].elapsed_time(ev[-1][-1])
    stage_ms = {names[n_]: float(np.mean([ev[s][n_].elapsed_time(ev[s][n_ + 1]) for s in range(args.steps)]))
                for n_ in range(len(calls))}
    ms_per_step = total_ms / args.steps
    flops = w.flops_fwd + w.flops_bwd
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    bwd_main_ms = stage_ms["bwd_main"]
    kernel_flop = 0.8 * w.flops_bwd  # four of the backward's five products
    achieved = kernel_flop / (bwd_main_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                # the committed counter runs cover the headline workload only
                "traffic": _traffic(None) if w.name == HEADLINE else None,
                "kernel": "bwd_kernel (key-tile-parallel backward: S, dP, dV, dK products)",
                "per_launch_flop": kernel_flop, "avg_launch_ms": round(bwd_main_ms, 4)}

    graph = None
    if args.graph:
        # the same five calls captured once and replayed; no memset nodes are involved (the
        # kernels write every byte they later read)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in calls:
                c()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        g_ms = e0.elapsed_time(e1) / args.steps
        graph = {"ms_per_step": round(g_ms, 4), "value": round(flops / (g_ms * 1e-3) / 1e12, 2),
                 "unit": "TFLOP/s", "eager_ms_per_step": round(ms_per_step, 4)}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, inp, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "N": N, "H": H, "D": D, "mask_tail": w.mask_tail,
                   "bias_std": w.bias_std, "residual_compensation": not args.no_residual},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {k_: round(v_, 4) for k_, v_ in stage_ms.items()},
        "wall_s_timed_region": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if graph is not None:
        out["graph"] = graph
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
