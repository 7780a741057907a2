"""GPU parity of the triangle multiplication core (include/tri_mul.h) against the FP64 oracle.

Definition (kongchang.com article on fast_trimul, section "什么是三角乘法更新"; reading in
``oracle/tri_mul_oracle.py``): outgoing x[i,j,c] = sum_k a[i,k,c] b[j,k,c], incoming
x[i,j,c] = sum_k a[k,i,c] b[k,j,c], and the gradients da, db.

Bound, from the arithmetic (exact bf16 products, FP32 sums of at most N <= 1024 terms, one
final rounding to bf16): every element within 2^-8 |ref| + 2^-13 sum_k |a||b| of the FP64
value (half an ulp of bf16 is 2^-9 relative; n u_fp32 <= 2^-14), and rel-RMSE <= 3e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import TRIMUL_WORKLOADS, bf16_bits_to_f64, make_pair_inputs

from ._util import f64, rrmse, to_dev

pytestmark = pytest.mark.gpu

TOL_RRMSE = 3e-3


def _bits(t):
    return t.view(torch.int16)


def _run(ta, a, b, dx, direction):
    B, N, _, C = a.shape
    d = ta.TRI_MUL_DIRECTIONS[direction]
    x, da, db = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    assert ta.tri_mul_fwd(d, B, N, C, a, b, x) == 0
    assert ta.tri_mul_bwd(d, B, N, C, a, b, dx, da, db) == 0
    torch.cuda.synchronize()
    return dict(x=x, da=da, db=db)


def _bound_check(name, got, ref, absref):
    err = np.abs(got - ref)
    lim = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * absref
    worst = float((err / np.maximum(lim, 1e-300)).max())
    e = rrmse(got, ref)
    print(f"  {name}: rel-RMSE {e:.3e}, worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0, (name, worst)
    assert e <= TOL_RRMSE, (name, e)


def _check(inp, direction, channels=None):
    import triangle_attention_amd as ta
    dev = {n: to_dev(inp[n]) for n in ("a", "b", "dx")}
    out = _run(ta, dev["a"], dev["b"], dev["dx"], direction)
    x64 = {n: bf16_bits_to_f64(inp[n]) for n in ("a", "b", "dx")}
    if channels is not None:  # channels are independent: check a subset at large sizes
        x64 = {n: v[..., channels] for n, v in x64.items()}
    a, b, dx = x64["a"], x64["b"], x64["dx"]
    ref = dict(x=oracle.tri_mul_forward64(a, b, direction))
    ref["da"], ref["db"] = oracle.tri_mul_backward64(a, b, dx, direction)
    absx = oracle.tri_mul_forward64(np.abs(a), np.abs(b), direction)
    absda, absdb = oracle.tri_mul_backward64(np.abs(a), np.abs(b), np.abs(dx), direction)
    absref = dict(x=absx, da=absda, db=absdb)
    for n in ("x", "da", "db"):
        got = f64(out[n])
        if channels is not None:
            got = got[..., channels]
        _bound_check(n, got, ref[n], absref[n])
    return dev, out


SMALL = [
    # (B, N, C): one tile, ragged rows/columns/reduction, several tiles and channel groups
    (1, 1, 8),
    (1, 5, 16),
    (2, 37, 8),
    (1, 64, 24),
    (1, 100, 32),
    (1, 130, 16),
    (2, 200, 8),
]


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("B,N,C", SMALL)
def test_tri_mul_parity_small(B, N, C, direction):
    print(f"tri_mul {direction} B={B} N={N} C={C}", flush=True)
    inp = make_pair_inputs(B, N, C, seed=7 * N + C)
    _check(inp, direction)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_tri_mul_parity_full_size_sampled_channels(direction):
    w = TRIMUL_WORKLOADS["trimul_n768_c128"]
    print(f"tri_mul {direction} full size {w}", flush=True)
    inp = make_pair_inputs(w["B"], w["N"], w["C"], seed=w["seed"])
    # one channel from each of four channel groups, including the last channel
    _check(inp, direction, channels=[0, 45, 90, 127])


def test_tri_mul_deterministic_and_autograd():
    import triangle_attention_amd as ta
    inp = make_pair_inputs(1, 150, 32, seed=99)
    a, b, dx = (to_dev(inp[n]) for n in ("a", "b", "dx"))
    for direction in ("outgoing", "incoming"):
        first = _run(ta, a, b, dx, direction)
        for _ in range(2):
            again = _run(ta, a, b, dx, direction)
            for n in ("x", "da", "db"):
                assert torch.equal(_bits(again[n]), _bits(first[n])), (direction, n)
        al, bl = a.clone().requires_grad_(True), b.clone().requires_grad_(True)
        x = ta.triangle_multiplication(al, bl, direction)
        x.backward(dx)
        torch.cuda.synchronize()
        assert torch.equal(_bits(x.detach()), _bits(first["x"]))
        assert torch.equal(_bits(al.grad), _bits(first["da"]))
        assert torch.equal(_bits(bl.grad), _bits(first["db"]))
