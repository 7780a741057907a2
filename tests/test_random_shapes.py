"""GPU parity on seeded random small shapes: batch 1-2, N 1-259, 1-3 heads, d 16 or 32, a key
mask on a random tail in about 40% of the cases, bias std 0.5, 1 or 4, against the FP64 oracle
on every slice.

Bounds as in test_parity.py: forward max-abs(o) and rel-RMSE(o), lse, every gradient's rel-RMSE.
Method: TurboPairFormer (arXiv 2610.05854), Abstract.
"""
import numpy as np
import pytest

import oracle
from tri_synth import make_inputs

from ._util import (TOL_GRAD_RRMSE, TOL_LSE_MAXABS, TOL_O_MAXABS, TOL_O_RRMSE, f64, inputs64, maxabs, rrmse,
                    run_gpu)

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 3)); N = int(rng.integers(1, 260)); H = int(rng.integers(1, 4))
        D = int(rng.choice([16, 32]))
        tail = int(rng.integers(0, N)) if rng.random() < 0.4 else 0
        bstd = float(rng.choice([0.5, 1.0, 4.0]))
        out.append((B, N, H, D, tail, bstd, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("B,N,H,D,tail,bstd,seed", _cases())
def test_random_shape(B, N, H, D, tail, bstd, seed):
    label = f"B={B} N={N} H={H} D={D} tail={tail} bias_std={bstd} seed={seed}"
    print(label, flush=True)
    inp = make_inputs(B, N, H, D, bias_std=bstd, mask_tail=tail, seed=seed)
    out = run_gpu(inp)
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
