"""GPU parity: the HIP path through the C ABI against the FP64 oracle on identical bf16 inputs.

Bounds (stated for this path): forward max-abs(o) <= 2e-2 and rel-RMSE(o) <= 1e-2;
rel-RMSE <= 3e-2 for dq, dk, dv and dbias.  Internal extra check: lse max-abs <= 1e-4.
Method: "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
Optimized Triangle Attention Kernel" (arXiv 2610.05854), Abstract.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import WORKLOADS, make_inputs, workload_inputs

from ._util import (TOL_GRAD_RRMSE, TOL_LSE_MAXABS, TOL_O_MAXABS, TOL_O_RRMSE, f64, inputs64, maxabs, rrmse,
                    run_gpu)

pytestmark = pytest.mark.gpu


def _check_full(inp, out, label):
    x = inputs64(inp)
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"])
    dq64, dk64, dv64, db64 = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"])
    o = f64(out["o"])
    errs = dict(o_maxabs=maxabs(o, o64), o=rrmse(o, o64), lse=maxabs(f64(out["lse"]), lse64),
                dq=rrmse(f64(out["dq"]), dq64), dk=rrmse(f64(out["dk"]), dk64), dv=rrmse(f64(out["dv"]), dv64),
                dbias=rrmse(f64(out["dbias"]), db64))
    print(label, {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o_maxabs"] <= TOL_O_MAXABS, (label, errs)
    assert errs["o"] <= TOL_O_RRMSE, (label, errs)
    assert errs["lse"] <= TOL_LSE_MAXABS, (label, errs)
    for g in ("dq", "dk", "dv", "dbias"):
        assert errs[g] <= TOL_GRAD_RRMSE, (label, g, errs)
    return errs


# small shapes: several tiles and ragged tails in both the query and the key direction
SMALL = [
    # (B, N, H, D, mask_kind)
    (1, 1, 1, 16, None),
    (1, 2, 2, 32, None),
    (1, 37, 2, 32, None),
    (2, 64, 3, 16, None),
    (1, 100, 2, 16, "random"),
    (1, 130, 1, 32, "tail"),
    (1, 200, 2, 32, "random"),
    (1, 257, 1, 16, None),
    (1, 450, 1, 32, "random"),  # four query steps; the last key block's upper half lies past N
]


def _small_inputs(B, N, H, D, mask_kind, seed):
    inp = make_inputs(B, N, H, D, seed=seed, bias_std=2.0)
    if mask_kind == "random":
        rng = np.random.default_rng(seed + 7)
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, rng.integers(0, N)] = 1  # every slice keeps at least one key
        inp["key_mask"] = m
    elif mask_kind == "tail":
        m = np.ones((B, N, N), dtype=np.uint8)
        m[:, :, N - max(1, N // 5):] = 0
        inp["key_mask"] = m
    return inp


@pytest.mark.parametrize("B,N,H,D,mask_kind", SMALL)
def test_small_shapes_elementwise(B, N, H, D, mask_kind):
    print(f"case B={B} N={N} H={H} D={D} mask={mask_kind}", flush=True)
    inp = _small_inputs(B, N, H, D, mask_kind, seed=1000 + N * 7 + D)
    out = run_gpu(inp)
    _check_full(inp, out, f"B{B}N{N}H{H}D{D}{mask_kind}")
    if mask_kind is not None:
        # masked keys receive exactly zero gradient: dk, dv rows and dbias columns (tail mask: all slices)
        m = inp["key_mask"]
        dk, dv = f64(out["dk"]), f64(out["dv"])
        sel = np.broadcast_to((m == 0)[:, :, None, :, None], dk.shape)
        assert np.abs(dk[sel]).max(initial=0.0) == 0.0
        assert np.abs(dv[sel]).max(initial=0.0) == 0.0
        if mask_kind == "tail":
            db = f64(out["dbias"])
            assert np.abs(db[..., N - max(1, N // 5):]).max() == 0.0


def test_small_shape_n1_closed_form():
    # N = 1: o = v exactly, dv = dO exactly, dq = dk = dbias = 0
    inp = make_inputs(1, 1, 3, 32, seed=5)
    out = run_gpu(inp)
    assert torch.equal(out["o"].cpu(), torch.from_numpy(inp["v"].view(np.int16)).view(torch.bfloat16))
    assert torch.equal(out["dv"].cpu(), torch.from_numpy(inp["dO"].view(np.int16)).view(torch.bfloat16))
    # dS = P (dP - D) with P = 1: dP and D are the same dot product dO.v summed in two FP32
    # orders (MFMA vs. the correction formed in the dQ kernel), so they agree to a few ulps of |dO.v|
    assert float(out["dq"].float().abs().max()) < 1e-5
    assert float(out["dk"].float().abs().max()) < 1e-5
    assert float(out["dbias"].abs().max()) < 1e-5


def test_residual_bound_and_gain():
    inp = make_inputs(1, 96, 2, 32, seed=77)
    out = run_gpu(inp)
    x = inputs64(inp)
    o64, _ = oracle.forward64(x["q"], x["k"], x["v"], x["bias"])
    o, r = f64(out["o"]), f64(out["res"])
    # |r| is at most half a bf16 ulp of o (r is the rounding error of o, itself rounded)
    ulp = np.ldexp(1.0, np.frexp(np.abs(o))[1] - 8)
    assert np.all(np.abs(r) <= 0.5 * ulp + 1e-30)
    assert rrmse(o + r, o64) < rrmse(o, o64)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_sampled_parity(name):
    """Full-size workloads at the benchmark's launch configuration: sampled slices element by
    element against the oracle, sampled dbias rows (each a sum over all slices), and the
    invariants that hold at any size."""
    w = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    inp = workload_inputs(w)
    out = run_gpu(inp)
    x = inputs64(inp)
    rng = np.random.default_rng(w.seed)
    slices = sorted(rng.choice(w.N, size=3, replace=False).tolist() + [0, w.N - 1])
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"], slices=slices)
    dq64, dk64, dv64, _ = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"], slices=slices)
    sl = (slice(None), slices)
    o = f64(out["o"])[sl]
    errs = dict(o_maxabs=maxabs(o, o64[sl]), o=rrmse(o, o64[sl]), lse=maxabs(f64(out["lse"])[sl], lse64[sl]),
                dq=rrmse(f64(out["dq"])[sl], dq64[sl]), dk=rrmse(f64(out["dk"])[sl], dk64[sl]),
                dv=rrmse(f64(out["dv"])[sl], dv64[sl]))
    rows = [(0, int(h), int(j)) for h, j in zip(rng.integers(0, w.H, 6), rng.integers(0, w.N, 6))]
    rows += [(0, 0, 0), (0, w.H - 1, w.N - 1)]
    db64 = oracle.dbias_rows64(x["q"], x["k"], x["v"], x["bias"], x["dO"], rows, x["key_mask"])
    db = f64(out["dbias"])
    errs["dbias"] = rrmse(np.stack([db[b, h, j] for b, h, j in rows]), db64)
    print(name, {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o_maxabs"] <= TOL_O_MAXABS and errs["o"] <= TOL_O_RRMSE and errs["lse"] <= TOL_LSE_MAXABS, errs
    for g in ("dq", "dk", "dv", "dbias"):
        assert errs[g] <= TOL_GRAD_RRMSE, (g, errs)
    # invariants at full size: sum_k dbias = 0 and sum_k dk = 0 (softmax shift invariance)
    assert float(out["dbias"].sum(-1).abs().max()) <= 1e-3 * float(out["dbias"].abs().max()) * w.N ** 0.5
    if w.mask_tail:
        assert float(out["dbias"][..., w.N - w.mask_tail:].abs().max()) == 0.0
        assert float(out["dk"][:, :, :, w.N - w.mask_tail:].float().abs().max()) == 0.0
        assert float(out["dv"][:, :, :, w.N - w.mask_tail:].float().abs().max()) == 0.0


# backward past six 128-query steps: query chunks as equal as possible, whose dK / dV partials are
# summed in FP32 (N = 900: 4 + 4 steps; N = 1100: 5 + 4; N = 2048: 6 + 5 + 5); sampled
# slices element by element, sampled dbias rows, the invariants, and a bitwise repeat
@pytest.mark.parametrize("B,N,H,D,masked", [(1, 900, 2, 32, False), (1, 1100, 1, 16, True), (1, 2048, 1, 16, True)])
def test_chunked_backward_long_crops(B, N, H, D, masked):
    import triangle_attention_amd as ta
    print(f"chunked backward B={B} N={N} H={H} D={D} masked={masked}", flush=True)
    assert N > 768 and ta.tri_attn_bwd_workspace_bytes(B, N, H, D) > 0
    inp = make_inputs(B, N, H, D, seed=7 * N + D, bias_std=2.0)
    rng = np.random.default_rng(N + 5)
    if masked:
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, N - 1] = 1
        m[:, :, N - 40:N - 8] = 0  # fully masked keys inside the last key block
        inp["key_mask"] = m
    out = run_gpu(inp)
    again = run_gpu(inp)
    for n in ("o", "lse", "dq", "dk", "dv", "dbias"):
        assert torch.equal(out[n], again[n]), n
    x = inputs64(inp)
    # slices from the first and the last query chunk, and the last slice
    slices = sorted(set(rng.choice(N, size=2, replace=False).tolist() + [0, N - 1]))
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"], slices=slices)
    dq64, dk64, dv64, _ = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"], slices=slices)
    sl = (slice(None), slices)
    o = f64(out["o"])[sl]
    errs = dict(o_maxabs=maxabs(o, o64[sl]), o=rrmse(o, o64[sl]), lse=maxabs(f64(out["lse"])[sl], lse64[sl]),
                dq=rrmse(f64(out["dq"])[sl], dq64[sl]), dk=rrmse(f64(out["dk"])[sl], dk64[sl]),
                dv=rrmse(f64(out["dv"])[sl], dv64[sl]))
    # dbias rows of queries in every chunk (rows 0..767 first chunk, 768.. the next ones)
    js = [0, 767, 768, N - 1] + rng.integers(0, N, 3).tolist()
    rows = [(0, int(rng.integers(0, H)), int(j)) for j in js]
    db64 = oracle.dbias_rows64(x["q"], x["k"], x["v"], x["bias"], x["dO"], rows, x["key_mask"])
    db = f64(out["dbias"])
    errs["dbias"] = rrmse(np.stack([db[b, h, j] for b, h, j in rows]), db64)
    print(f"N={N}", {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o_maxabs"] <= TOL_O_MAXABS and errs["o"] <= TOL_O_RRMSE and errs["lse"] <= TOL_LSE_MAXABS, errs
    for g in ("dq", "dk", "dv", "dbias"):
        assert errs[g] <= TOL_GRAD_RRMSE, (g, errs)
    # per-row element checks of dk / dv keep a dropped chunk from hiding in the RMS over slices
    for i in slices:
        for g, ref in (("dk", dk64), ("dv", dv64)):
            got, want = f64(out[g])[0, i], ref[0, i]
            assert rrmse(got, want) <= TOL_GRAD_RRMSE, (g, i)
    assert float(out["dbias"].sum(-1).abs().max()) <= 1e-3 * float(out["dbias"].abs().max()) * N ** 0.5
    if masked:
        assert float(out["dbias"][..., N - 40:N - 8].abs().max()) == 0.0
        assert float(out["dk"][:, :, :, N - 40:N - 8].float().abs().max()) == 0.0
        assert float(out["dv"][:, :, :, N - 40:N - 8].float().abs().max()) == 0.0


# forward alone on crops past the backward's limit (inference), up to its maximum N = 4096:
# sampled slices, element by element
@pytest.mark.parametrize("B,N,H,D,masked", [(1, 2100, 1, 16, True), (1, 2304, 1, 32, False), (1, 4096, 1, 16, False)])
def test_forward_only_long_crops(B, N, H, D, masked):
    import triangle_attention_amd as ta
    from tri_synth import bf16_bits_to_f64
    from ._util import mask_dev, to_dev
    print(f"forward only B={B} N={N} H={H} D={D} masked={masked}", flush=True)
    inp = make_inputs(B, N, H, D, seed=N + D, bias_std=2.0)
    if masked:
        rng = np.random.default_rng(N)
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, 0] = 1
        inp["key_mask"] = m
    q, k, v, bias = (to_dev(inp[n]) for n in ("q", "k", "v", "bias"))
    o, lse, res = ta.forward(q, k, v, bias, mask_dev(inp["key_mask"]))
    torch.cuda.synchronize()
    assert ta.tri_attn_bwd_workspace_bytes(B, N, H, D) == 0  # no backward at this N
    o_, lse_ = f64(o), f64(lse)
    rng = np.random.default_rng(N + 1)
    for i in sorted(set(rng.integers(0, N, 2).tolist() + [N - 1])):
        for h in range(H):
            mrow = None if inp["key_mask"] is None else inp["key_mask"][0, i]
            o64, l64, _ = oracle.slice_forward64(bf16_bits_to_f64(inp["q"][0, i, h]), bf16_bits_to_f64(inp["k"][0, i, h]),
                                                 bf16_bits_to_f64(inp["v"][0, i, h]), bf16_bits_to_f64(inp["bias"][0, h]),
                                                 mrow)
            e = dict(o_maxabs=maxabs(o_[0, i, h], o64), o=rrmse(o_[0, i, h], o64), lse=maxabs(lse_[0, i, h], l64))
            print(f"  slice {i} head {h}", {k_: f"{v_:.2e}" for k_, v_ in e.items()}, flush=True)
            assert e["o_maxabs"] <= TOL_O_MAXABS and e["o"] <= TOL_O_RRMSE and e["lse"] <= TOL_LSE_MAXABS, e


def test_autograd_chunked_backward():
    """The autograd function past N = 768 returns the C entry points' results bit for bit."""
    import triangle_attention_amd as ta
    from ._util import mask_dev, to_dev
    B, N, H, D = 1, 800, 1, 32
    print(f"autograd chunked B={B} N={N} H={H} D={D}", flush=True)
    inp = make_inputs(B, N, H, D, seed=81, bias_std=2.0)
    ref = run_gpu(inp)
    q, k, v = (to_dev(inp[n]).requires_grad_(True) for n in ("q", "k", "v"))
    bias = to_dev(inp["bias"]).requires_grad_(True)
    o = ta.triangle_attention(q, k, v, bias, mask_dev(inp["key_mask"]))
    o.backward(to_dev(inp["dO"]))
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ref["o"])
    for n, t in (("dq", q), ("dk", k), ("dv", v)):
        assert torch.equal(t.grad, ref[n]), n
    assert torch.equal(bias.grad, ref["dbias"].to(torch.bfloat16))
