"""Accuracy sweep in the pages' evaluation shape: crops {384, 640, 768} x head dims {16, 32},
bf16 inputs, against the FP64 oracle, with and without the output-residual compensation
("TurboPairFormer ...", arXiv 2610.05854, Abstract: accuracy on crops 384/640/768 and head
dims 16/32, the residual lowering the backward error, bitwise-identical repeated calls).

Each case runs the full-size problem on the GPU and compares sampled slices element by element
(o, dq, dk, dv) and sampled dbias rows (each a sum over every slice) with the oracle.  It checks
the bounds, that the compensated backward is not worse on dbias (the gradient that sees the
correction D most directly), and that three calls agree bit for bit.  The table is printed
(`pytest -s`); its figures are quoted where the design notes discuss accuracy.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import make_inputs

from ._util import TOL_GRAD_RRMSE, TOL_O_RRMSE, f64, inputs64, rrmse, run_gpu

pytestmark = pytest.mark.gpu

CASES = [(384, 16), (384, 32), (640, 16), (640, 32), (768, 16), (768, 32)]
SEEDS = 3
H = 4
RESULTS = {}  # (N, D, seed index) -> (errors with residual, errors without)


def _references(x, slices, rows):
    o64, _ = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], None, slices=slices)
    dq64, dk64, dv64, _ = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], None, slices=slices)
    db64 = oracle.dbias_rows64(x["q"], x["k"], x["v"], x["bias"], x["dO"], rows, None)
    sl = (slice(None), slices)
    return dict(o=o64[sl], dq=dq64[sl], dk=dk64[sl], dv=dv64[sl], dbias=db64)


def _errors(out, ref, slices, rows):
    sl = (slice(None), slices)
    db = f64(out["dbias"])
    errs = {n: rrmse(f64(out[n])[sl], ref[n]) for n in ("o", "dq", "dk", "dv")}
    errs["dbias"] = rrmse(np.stack([db[b, h, j] for b, h, j in rows]), ref["dbias"])
    return errs


@pytest.mark.parametrize("rep", range(SEEDS))
@pytest.mark.parametrize("N,D", CASES)
def test_sweep_case(N, D, rep):
    seed = 1000 * (CASES.index((N, D)) + 1) + 17 * rep
    print(f"sweep N={N} d={D} seed={seed}", flush=True)
    inp = make_inputs(1, N, H, D, seed=seed, bias_std=1.0)
    x = inputs64(inp)
    rng = np.random.default_rng(seed + 1)
    slices = sorted(rng.choice(N, size=2, replace=False).tolist() + [N - 1])
    rows = [(0, int(h), int(j)) for h, j in zip(rng.integers(0, H, 4), rng.integers(0, N, 4))]

    comp = run_gpu(inp, residual=True)
    plain = run_gpu(inp, residual=False)
    ref = _references(x, slices, rows)
    e_c = _errors(comp, ref, slices, rows)
    e_p = _errors(plain, ref, slices, rows)
    print(f"N={N} d={D} with residual   " + " ".join(f"{k}={v:.3e}" for k, v in e_c.items()), flush=True)
    print(f"N={N} d={D} without residual " + " ".join(f"{k}={v:.3e}" for k, v in e_p.items()), flush=True)
    print(f"N={N} d={D} dbias error change with the residual: {100 * (e_c['dbias'] / e_p['dbias'] - 1):+.1f}%",
          flush=True)

    RESULTS[(N, D, rep)] = (e_c, e_p)
    assert e_c["o"] <= TOL_O_RRMSE
    for g in ("dq", "dk", "dv", "dbias"):
        assert e_c[g] <= TOL_GRAD_RRMSE and e_p[g] <= TOL_GRAD_RRMSE, (g, e_c, e_p)
    assert e_c["dbias"] <= e_p["dbias"], (e_c, e_p)

    # repeated calls: bitwise identical
    for _ in range(2):
        again = run_gpu(inp, residual=True)
        for n in ("o", "lse", "res", "dq", "dk", "dv", "dbias"):
            a, b = comp[n], again[n]
            va = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
            vb = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
            assert torch.equal(va, vb), n


def test_sweep_summary():
    """Mean rel-RMSE per gradient over the seeds of each case, with and without the residual
    (printed with -s); the compensated dbias error must be lower on average in every case."""
    if not RESULTS:
        pytest.skip("run together with the sweep cases")
    for N, D in CASES:
        runs = [RESULTS[k] for k in RESULTS if k[:2] == (N, D)]
        if not runs:
            continue
        mean = {side: {g: float(np.mean([r[side][g] for r in runs])) for g in ("dq", "dk", "dv", "dbias")}
                for side in (0, 1)}
        red = 100 * (mean[0]["dbias"] / mean[1]["dbias"] - 1)
        print(f"N={N} d={D} seeds={len(runs)} with r " + " ".join(f"{g}={v:.3e}" for g, v in mean[0].items())
              + " | without r " + " ".join(f"{g}={v:.3e}" for g, v in mean[1].items())
              + f" | dbias {red:+.1f}%", flush=True)
        assert mean[0]["dbias"] < mean[1]["dbias"], (N, D, mean)
