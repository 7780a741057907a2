"""GPU parity of the triangle multiplication core (include/tri_mul.h) against the FP64 oracle,
in both layouts (channels last [B, N, N, C] and channels first [B, C, N, N]).

Definition (kongchang.com article on fast_trimul, section "什么是三角乘法更新"; reading in
``oracle/tri_mul_oracle.py``): outgoing x[i,j,c] = sum_k a[i,k,c] b[j,k,c], incoming
x[i,j,c] = sum_k a[k,i,c] b[k,j,c], and the gradients da, db.

Bound, from the arithmetic (exact bf16 products, FP32 sums of at most N <= 1024 terms, one
final rounding to bf16): every element within 2^-8 |ref| + 2^-13 sum_k |a||b| of the FP64
value (the rounding to bf16 errs by at most its unit roundoff, 2^-8 relative; the FP32 sum by
at most n u_fp32 sum|ab| <= 2^-14 sum|ab|, taken twice), and rel-RMSE <= 3e-3.
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


def cf(t):  # channels last -> channels first
    return t.permute(0, 3, 1, 2).contiguous()


def cl(t):  # channels first -> channels last
    return t.permute(0, 2, 3, 1).contiguous()


def _run(ta, a, b, dx, direction, layout="channels_last", workspace=False):
    """a, b, dx channels last; returns channels-last outputs computed in `layout` (channels last:
    through the workspace path if `workspace`, else the in-place kernel)."""
    B, N, _, C = a.shape
    d, lay = ta.TRI_MUL_DIRECTIONS[direction], ta.TRI_MUL_LAYOUTS[layout]
    if layout == "channels_first":
        a, b, dx = cf(a), cf(b), cf(dx)
    x, da, db = torch.empty_like(a), torch.empty_like(a), torch.empty_like(a)
    nws = ta.tri_mul_workspace_bytes(lay, B, N, C) if workspace else 0
    ws = torch.empty(nws, dtype=torch.uint8, device=a.device) if nws else None
    assert ta.tri_mul_fwd(d, lay, B, N, C, a, b, x, ws, nws) == 0
    assert ta.tri_mul_bwd(d, lay, B, N, C, a, b, dx, da, db, ws, nws) == 0
    torch.cuda.synchronize()
    out = dict(x=x, da=da, db=db)
    return {n: cl(v) for n, v in out.items()} if layout == "channels_first" else out


def _bound_check(name, got, ref, absref):
    err = np.abs(got - ref)
    lim = 2.0 ** -8 * np.abs(ref) + 2.0 ** -13 * absref
    worst = float((err / np.maximum(lim, 1e-300)).max())
    e = rrmse(got, ref)
    print(f"  {name}: rel-RMSE {e:.3e}, worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0, (name, worst)
    assert e <= TOL_RRMSE, (name, e)


def _check(inp, direction, channels=None, layout="channels_last"):
    import triangle_attention_amd as ta
    dev = {n: to_dev(inp[n]) for n in ("a", "b", "dx")}
    out = _run(ta, dev["a"], dev["b"], dev["dx"], direction, layout)
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
    print(f"tri_mul channels_last {direction} B={B} N={N} C={C}", flush=True)
    inp = make_pair_inputs(B, N, C, seed=7 * N + C)
    _check(inp, direction)


# channels first: N a multiple of 8 (one 128 x 128 tile, ragged tiles, several tiles; any C)
SMALL_CF = [(1, 8, 3), (1, 40, 8), (2, 136, 5), (1, 200, 4), (1, 264, 2)]


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("B,N,C", SMALL_CF)
def test_tri_mul_parity_small_channels_first(B, N, C, direction):
    print(f"tri_mul channels_first {direction} B={B} N={N} C={C}", flush=True)
    inp = make_pair_inputs(B, N, C, seed=11 * N + C)
    _check(inp, direction, layout="channels_first")


@pytest.mark.parametrize("layout", ["channels_last", "channels_first"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_tri_mul_parity_full_size_sampled_channels(direction, layout):
    w = TRIMUL_WORKLOADS["trimul_n768_c128"]
    print(f"tri_mul {layout} {direction} full size {w}", flush=True)
    inp = make_pair_inputs(w["B"], w["N"], w["C"], seed=w["seed"])
    # one channel from each of four channel groups, including the last channel
    _check(inp, direction, channels=[0, 45, 90, 127], layout=layout)


@pytest.mark.parametrize("B,N,C", [(1, 136, 16), (2, 72, 24), (1, 264, 8)])
def test_tri_mul_layouts_agree_bitwise(B, N, C):
    # every path adds the same 16-term products in the same ascending order per element
    import triangle_attention_amd as ta
    inp = make_pair_inputs(B, N, C, seed=5 + N)
    a, b, dx = (to_dev(inp[n]) for n in ("a", "b", "dx"))
    for direction in ("outgoing", "incoming"):
        last = _run(ta, a, b, dx, direction, "channels_last")
        staged = _run(ta, a, b, dx, direction, "channels_last", workspace=True)
        first = _run(ta, a, b, dx, direction, "channels_first")
        for n in ("x", "da", "db"):
            assert torch.equal(_bits(last[n]), _bits(first[n])), (direction, n)
            assert torch.equal(_bits(staged[n]), _bits(first[n])), (direction, n, "workspace")


def test_tri_mul_deterministic_and_autograd():
    import triangle_attention_amd as ta
    inp = make_pair_inputs(1, 152, 32, seed=99)  # N a multiple of 8 (channels first)
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
        # channels first through the autograd wrapper
        ref = _run(ta, a, b, dx, direction, "channels_first")
        al, bl = cf(a).requires_grad_(True), cf(b).requires_grad_(True)
        x = ta.triangle_multiplication(al, bl, direction, layout="channels_first")
        x.backward(cf(dx))
        torch.cuda.synchronize()
        assert torch.equal(_bits(cl(x.detach())), _bits(ref["x"]))
        assert torch.equal(_bits(cl(al.grad)), _bits(ref["da"]))
        assert torch.equal(_bits(cl(bl.grad)), _bits(ref["db"]))
