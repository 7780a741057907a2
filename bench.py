"""Benchmark: triangle attention forward + backward on one MI355X.

One step is the whole hot path on one batch of resident synthetic input: the forward
(bias conversion + attention kernel) and the backward (bias conversion + correction D,
the key-tile-parallel kernel, ordered sums of the dq / dbias partials).  W untimed
warm-up steps, then exactly K timed steps bracketed by torch.cuda.synchronize().

Throughput is credited with the method's FLOP convention: 4*B*N^3*H*d for the forward
(Q K^T and P V) and 2.5x that for the backward (five products), whatever the kernels
actually execute.  The roofline object reports the dominant kernel (the backward main
kernel) against the published dense bf16 MFMA peak, with its duration from HIP events
recorded on the launch stream around that kernel in every timed step.

Prints one JSON line.  Only one GPU is used: --gpus above 1 exits with a message.
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


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=30, help="untimed steps; the GPU needs about 30 to reach its steady clock")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-residual", action="store_true", help="uncompensated backward correction")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle CPU-baseline budget (0 = skip)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the whole fwd+bwd step captured in one HIP graph (small-N launch latency)")
    return ap.parse_args()


def _src_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def _traffic(bytes_alg: float):
    """HBM bytes per launch of the backward main kernel from committed rocprofv3 counter runs,
    valid only while the kernel source is the one the counters were taken on."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != _src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, budget_s: float):
    """The FP64 oracle as it stands, fwd+bwd slice by slice (all heads), until the budget is spent."""
    import oracle
    from tri_synth import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    x = {n: bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "bias", "dO")}
    m = inp["key_mask"]
    t0 = time.perf_counter()
    done = 0
    for i in range(w.N):
        for h in range(w.H):
            mrow = None if m is None else m[0, i]
            oracle.slice_forward64(x["q"][0, i, h], x["k"][0, i, h], x["v"][0, i, h], x["bias"][0, h], mrow)
            oracle.slice_backward64(x["q"][0, i, h], x["k"][0, i, h], x["v"][0, i, h], x["bias"][0, h],
                                    x["dO"][0, i, h], mrow)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 14.0 * w.N * w.N * w.H * w.D * done  # fwd (4) + bwd (10) per score element
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.N} slices x {w.H} heads of {w.name}, fwd+bwd in FP64 ({dt:.1f} s)"}


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

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
    achieved = w.flops_bwd / (bwd_main_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": _traffic(None),
                "kernel": "bwd_kernel (key-tile-parallel backward: S, dP, dV, dK, dQ products)",
                "per_launch_flop": w.flops_bwd, "avg_launch_ms": round(bwd_main_ms, 4)}

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
