"""Forward + backward captured in one HIP graph (the small-N latency path).

The library makes only kernel launches on the caller's stream (no allocation, no memset, no
host synchronisation), so a caller can capture a whole step and replay it.  Each replay must
reproduce the eager results bit for bit; eager work and synchronisation run between the
replays, as a capturing caller would interleave them.
"""
import numpy as np
import pytest
import torch

from tri_synth import WORKLOADS, make_inputs, workload_inputs

from ._util import mask_dev, to_dev

pytestmark = pytest.mark.gpu

OUTS = ("o", "lse", "res", "dq", "dk", "dv", "dbias")


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _check_graph_replays(inp, against_oracle=False):
    import triangle_attention_amd as ta
    q, k, v, bias, dO = (to_dev(inp[n]) for n in ("q", "k", "v", "bias", "dO"))
    m = mask_dev(inp["key_mask"])
    B, N, H, _, D = q.shape
    dev = q.device
    out = dict(o=torch.empty_like(q), res=torch.empty_like(q),
               lse=torch.empty((B, N, H, N), dtype=torch.float32, device=dev),
               dq=torch.empty_like(q), dk=torch.empty_like(q), dv=torch.empty_like(q),
               dbias=torch.empty((B, H, N, N), dtype=torch.float32, device=dev))
    fws = torch.empty(ta.tri_attn_fwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device=dev)
    bws = torch.empty(ta.tri_attn_bwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device=dev)

    def step():
        sh = torch.cuda.current_stream().cuda_stream
        st = ta.tri_attn_fwd(B, N, H, D, q, k, v, bias, m, out["o"], out["lse"], out["res"], fws, fws.numel(), sh)
        assert st == 0, st
        st = ta.tri_attn_bwd(B, N, H, D, q, k, v, bias, m, out["o"], out["lse"], out["res"], dO, out["dq"],
                             out["dk"], out["dv"], out["dbias"], bws, bws.numel(), sh)
        assert st == 0, st

    step()
    torch.cuda.synchronize()
    ref = {n: out[n].clone() for n in OUTS}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    scratch = torch.zeros(1 << 20, device=dev)
    for rep in range(3):
        for n in OUTS:  # poison the outputs so that a replay that skips a write shows up
            out[n].view(torch.uint8).fill_(0x7F)
        g.replay()
        scratch.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        for n in OUTS:
            assert torch.equal(_bits(out[n]), _bits(ref[n])), (rep, n)
        if against_oracle:  # each replay's outputs against the FP64 oracle, element by element
            _oracle_check(inp, out, f"graph replay {rep}")


def _oracle_check(inp, out, label):
    import oracle
    from ._util import (TOL_GRAD_RRMSE, TOL_LSE_MAXABS, TOL_O_MAXABS, TOL_O_RRMSE, f64, inputs64, maxabs,
                        rrmse)
    x = inputs64(inp)
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"])
    g64 = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"])
    o = f64(out["o"])
    errs = dict(o_maxabs=maxabs(o, o64), o=rrmse(o, o64), lse=maxabs(f64(out["lse"]), lse64))
    for n, ref in zip(("dq", "dk", "dv", "dbias"), g64):
        errs[n] = rrmse(f64(out[n]), ref)
    print(label, {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o_maxabs"] <= TOL_O_MAXABS and errs["o"] <= TOL_O_RRMSE and errs["lse"] <= TOL_LSE_MAXABS, errs
    for n in ("dq", "dk", "dv", "dbias"):
        assert errs[n] <= TOL_GRAD_RRMSE, (n, errs)


def test_graph_replay_small():
    # the launch-bound workload the graph path is for; replays also checked against the oracle
    _check_graph_replays(workload_inputs(WORKLOADS["n64_h4_d16"]), against_oracle=True)


def test_graph_replay_masked_ragged():
    inp = make_inputs(1, 200, 2, 32, seed=77, bias_std=2.0)
    rng = np.random.default_rng(78)
    msk = (rng.random((1, 200, 200)) > 0.3).astype(np.uint8)
    msk[:, :, 5] = 1
    inp["key_mask"] = msk
    _check_graph_replays(inp, against_oracle=True)


def test_graph_replay_chunked_backward():
    # N = 900: two query chunks in two launches plus the dK/dV chunk sum, all inside the graph
    inp = make_inputs(1, 900, 1, 16, seed=79, bias_std=2.0)
    rng = np.random.default_rng(80)
    msk = (rng.random((1, 900, 900)) > 0.3).astype(np.uint8)
    msk[:, :, 899] = 1
    inp["key_mask"] = msk
    _check_graph_replays(inp)


def test_graph_replay_tri_mul():
    """The triangle multiplication core (both directions, forward and backward, channels first and
    channels last through the workspace) captured in one graph: replays reproduce eager results."""
    import triangle_attention_amd as ta
    from tri_synth import make_pair_inputs

    B, N, C = 1, 64, 32
    inp = make_pair_inputs(B, N, C, seed=64)
    base = {n: to_dev(inp[n]) for n in ("a", "b", "dx")}
    runs = []
    for layout in ("channels_first", "channels_last"):
        t = {n: (v.permute(0, 3, 1, 2).contiguous() if layout == "channels_first" else v) for n, v in base.items()}
        lay = ta.TRI_MUL_LAYOUTS[layout]
        nws = ta.tri_mul_workspace_bytes(lay, B, N, C)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=t["a"].device) if nws else None
        outs = {d: [torch.empty_like(t["a"]) for _ in range(3)] for d in ("outgoing", "incoming")}
        runs.append((lay, t, ws, nws, outs))

    def step():
        sh = torch.cuda.current_stream().cuda_stream
        for lay, t, ws, nws, outs in runs:
            for d, (x, da, db) in outs.items():
                dd = ta.TRI_MUL_DIRECTIONS[d]
                assert ta.tri_mul_fwd(dd, lay, B, N, C, t["a"], t["b"], x, ws, nws, stream=sh) == 0
                assert ta.tri_mul_bwd(dd, lay, B, N, C, t["a"], t["b"], t["dx"], da, db, ws, nws, stream=sh) == 0

    step()
    torch.cuda.synchronize()
    ref = [[o.clone() for d in outs for o in outs[d]] for _, _, _, _, outs in runs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for _, _, _, _, outs in runs:
            for d in outs:
                for o in outs[d]:
                    o.view(torch.uint8).fill_(0x7F)
        g.replay()
        torch.cuda.synchronize()
        for r, (_, _, _, _, outs) in zip(ref, runs):
            got = [o for d in outs for o in outs[d]]
            for a_, b_ in zip(got, r):
                assert torch.equal(a_.view(torch.int16), b_.view(torch.int16)), rep
