"""GPU parity of the triangle multiplication's input gating (include/tri_mul.h) against the FP64
oracle, and of the gated chain: gate -> product -> backward through both.

Gating (kongchang.com article on fast_trimul, section "什么是三角乘法更新"; reading in
``oracle/tri_mul_oracle.py``): a = sigmoid(g) * p * mask.  Bound per element, from the
arithmetic: one rounding to bf16 (unit roundoff 2^-8, relative) on top of FP32 sigmoid and
products (a few units of 2^-24, relative; 2^-16 allowed): (2^-8 + 2^-16) |ref| + 2^-24.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import bf16_bits_to_f64, make_pair_inputs

from ._util import f64, rrmse, to_dev

pytestmark = pytest.mark.gpu


def _cl(t):  # channels first -> channels last
    return t.permute(0, 2, 3, 1).contiguous()


def _bound(name, got, ref):
    err = np.abs(got - ref)
    worst = float((err / ((2.0 ** -8 + 2.0 ** -16) * np.abs(ref) + 2.0 ** -24)).max())
    print(f"  {name}: rel-RMSE {rrmse(got, ref):.3e}, worst err/bound {worst:.3f}", flush=True)
    assert worst <= 1.0, (name, worst)


CASES = [
    # (B, N, C, masked, layout)
    (1, 8, 8, False, "channels_first"),
    (2, 40, 16, True, "channels_first"),
    (1, 136, 24, True, "channels_first"),
    (1, 200, 72, False, "channels_first"),
    (1, 37, 8, True, "channels_last"),
    (2, 64, 32, False, "channels_last"),
]


@pytest.mark.parametrize("B,N,C,masked,layout", CASES)
def test_gate_parity(B, N, C, masked, layout):
    import triangle_attention_amd as ta
    print(f"gate {layout} B={B} N={N} C={C} masked={masked}", flush=True)
    inp = make_pair_inputs(B, N, C, seed=3 * N + C, scale=2.0)  # a -> g, b -> p, dx -> da (channels last)
    rng = np.random.default_rng(N)
    m = (rng.random((B, N, N)) > 0.3).astype(np.uint8) if masked else None
    g, p, da_cl = (to_dev(inp[n]) for n in ("a", "b", "dx"))
    mdev = None if m is None else torch.from_numpy(m).cuda()
    lay = ta.TRI_MUL_LAYOUTS[layout]
    first = layout == "channels_first"
    a = torch.empty((B, C, N, N) if first else (B, N, N, C), dtype=torch.bfloat16, device="cuda")
    da = da_cl.permute(0, 3, 1, 2).contiguous() if first else da_cl
    dg, dp = torch.empty_like(g), torch.empty_like(p)
    assert ta.tri_mul_gate_fwd(lay, B, N, C, g, p, mdev, a) == 0
    assert ta.tri_mul_gate_bwd(lay, B, N, C, g, p, mdev, da, dg, dp) == 0
    torch.cuda.synchronize()
    g64, p64, da64 = (bf16_bits_to_f64(inp[n]) for n in ("a", "b", "dx"))
    _bound("a", f64(_cl(a) if first else a), oracle.gate_forward64(g64, p64, m))
    dg64, dp64 = oracle.gate_backward64(g64, p64, da64, m)
    _bound("dg", f64(dg), dg64)
    _bound("dp", f64(dp), dp64)
    if m is not None:  # dropped pair entries are exact zeros in every channel
        a_cl = _cl(a) if first else a
        assert torch.count_nonzero(a_cl[torch.from_numpy(m == 0).cuda()]) == 0


def test_gated_chain_through_the_product():
    """gated_operand -> triangle_multiplication (channels first) -> backward, against the FP64
    chain; the GPU rounds the gated operands to bf16 before the product, so the bound is the
    product's plus that rounding (rel-RMSE <= 6e-3)."""
    import triangle_attention_amd as ta
    B, N, C = 1, 72, 16
    ga_in = make_pair_inputs(B, N, C, seed=71, scale=2.0)
    gb_in = make_pair_inputs(B, N, C, seed=72, scale=2.0)
    rng = np.random.default_rng(73)
    m = (rng.random((B, N, N)) > 0.2).astype(np.uint8)
    mdev = torch.from_numpy(m).cuda()
    ga, pa, dx_cl = (to_dev(ga_in[n]) for n in ("a", "b", "dx"))
    gb, pb = to_dev(gb_in["a"]), to_dev(gb_in["b"])
    for t in (ga, pa, gb, pb):
        t.requires_grad_(True)
    for direction in ("outgoing", "incoming"):
        for t in (ga, pa, gb, pb):
            t.grad = None
        a = ta.gated_operand(ga, pa, mdev)
        b = ta.gated_operand(gb, pb, mdev)
        x = ta.triangle_multiplication(a, b, direction, layout="channels_first")
        x.backward(dx_cl.permute(0, 3, 1, 2).contiguous())
        torch.cuda.synchronize()
        G = {n: bf16_bits_to_f64(v) for n, v in (("ga", ga_in["a"]), ("pa", ga_in["b"]), ("gb", gb_in["a"]),
                                                 ("pb", gb_in["b"]), ("dx", ga_in["dx"]))}
        a64 = oracle.gate_forward64(G["ga"], G["pa"], m)
        b64 = oracle.gate_forward64(G["gb"], G["pb"], m)
        x64 = oracle.tri_mul_forward64(a64, b64, direction)
        da64, db64 = oracle.tri_mul_backward64(a64, b64, G["dx"], direction)
        dga64, dpa64 = oracle.gate_backward64(G["ga"], G["pa"], da64, m)
        dgb64, dpb64 = oracle.gate_backward64(G["gb"], G["pb"], db64, m)
        errs = dict(x=rrmse(f64(_cl(x.detach())), x64), dga=rrmse(f64(ga.grad), dga64),
                    dpa=rrmse(f64(pa.grad), dpa64), dgb=rrmse(f64(gb.grad), dgb64), dpb=rrmse(f64(pb.grad), dpb64))
        print(f"  gated chain {direction}", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        assert max(errs.values()) <= 6e-3, (direction, errs)
