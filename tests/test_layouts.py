"""Token layouts: the pair layout [B, N, N, H, D] read in place, attending along the second
pair index (starting node) or along the first with the second fixed (ending node), with no
transposed copy.

Every kernel runs the same work in the same order in each layout, so on the same values the
outputs must equal the slice-major path's bit for bit; the parity tests pin that path to the
FP64 oracle.  One ending-node case is also compared with the oracle directly, on the pair
tensor's values re-indexed on the CPU.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import make_inputs

from ._util import TOL_GRAD_RRMSE, TOL_O_RRMSE, f64, inputs64, mask_dev, rrmse, to_dev

pytestmark = pytest.mark.gpu

TOK = ("q", "k", "v", "dO")


# slice-major t[b, i, h, j, c] <-> pair layouts
def to_pair_start(t):  # P[b, i, j, h, c] = t[b, i, h, j, c]
    return t.permute(0, 1, 3, 2, 4).contiguous()


def from_pair_start(p):
    return p.permute(0, 1, 3, 2, 4)


def to_pair_end(t):  # E[b, j, i, h, c] = t[b, i, h, j, c]
    return t.permute(0, 3, 1, 2, 4).contiguous()


def from_pair_end(e):
    return e.permute(0, 2, 3, 1, 4)


CONV = {"pair_start": (to_pair_start, from_pair_start), "pair_end": (to_pair_end, from_pair_end)}


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _inputs(B, N, H, D, masked, seed):
    inp = make_inputs(B, N, H, D, seed=seed, bias_std=2.0)
    if masked:
        rng = np.random.default_rng(seed + 1)
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, rng.integers(0, N)] = 1
        inp["key_mask"] = m
    return inp


def _run(ta, dev, layout, residual):
    o, lse, res = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], residual, layout=layout)
    dq, dk, dv, dbias = ta.backward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], o, lse, res, dev["dO"],
                                    layout=layout)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, res=res, dq=dq, dk=dk, dv=dv, dbias=dbias)


CASES = [
    # (B, N, H, D, masked, residual)
    (1, 64, 4, 16, False, True),
    (2, 37, 3, 32, True, True),
    (1, 200, 2, 32, True, False),
    (1, 450, 1, 16, False, True),
    (1, 384, 4, 32, True, True),
    (1, 640, 2, 16, True, True),   # five query steps
    (1, 768, 2, 32, False, True),  # six query steps: the largest backward instantiation
    (1, 900, 1, 16, True, True),   # two query chunks of four steps each
    (1, 800, 1, 32, True, True),   # two query chunks of four and three steps
    (1, 1664, 1, 32, False, True), # three query chunks of five, four and four steps
]


@pytest.mark.parametrize("layout", ["pair_start", "pair_end"])
@pytest.mark.parametrize("B,N,H,D,masked,residual", CASES)
def test_layout_bitwise(layout, B, N, H, D, masked, residual):
    import triangle_attention_amd as ta
    print(f"layout={layout} B={B} N={N} H={H} D={D} masked={masked} residual={residual}", flush=True)
    inp = _inputs(B, N, H, D, masked, seed=100 * N + H)
    base = {n: to_dev(inp[n]) for n in TOK + ("bias",)}
    base["mask"] = mask_dev(inp["key_mask"])
    ref = _run(ta, base, "slice_head", residual)

    to, back = CONV[layout]
    dev = {n: to(base[n]) for n in TOK}
    dev["bias"], dev["mask"] = base["bias"], base["mask"]
    out = _run(ta, dev, layout, residual)
    for n in ("o", "res", "dq", "dk", "dv"):
        if ref[n] is None:
            assert out[n] is None
            continue
        assert torch.equal(_bits(back(out[n]).contiguous()), _bits(ref[n])), n
    for n in ("lse", "dbias"):
        assert torch.equal(_bits(out[n]), _bits(ref[n])), n


def test_ending_node_against_oracle():
    """Ending node on a pair tensor: slice = second pair index, tokens = first pair index."""
    import triangle_attention_amd as ta
    B, N, H, D = 1, 70, 2, 32
    rng = np.random.default_rng(4242)
    # pair-layout tensors [B, N(first index), N(second index), H, D] as bf16 bit patterns
    inp = make_inputs(B, N, H, D, seed=4243, bias_std=2.0)  # slice-major draws, re-used as raw values
    pair = {n: np.ascontiguousarray(inp[n].reshape(B, N, N, H, D)) for n in TOK}
    mask = (rng.random((B, N, N)) > 0.25).astype(np.uint8)  # [b, slice, key]
    mask[:, :, 3] = 1
    dev = {n: to_dev(pair[n]) for n in TOK}
    dev["bias"], dev["mask"] = to_dev(inp["bias"]), mask_dev(mask)
    out = _run(ta, dev, "pair_end", True)

    # the oracle's slice-major view: t[b, s, h, a, c] = pair[b, a, s, h, c]
    sm = {n: np.ascontiguousarray(pair[n].transpose(0, 2, 3, 1, 4)) for n in TOK}
    sm["bias"], sm["key_mask"] = inp["bias"], mask
    x = inputs64(sm)
    o64, _ = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"])
    dq64, dk64, dv64, db64 = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"])
    back = from_pair_end
    errs = dict(o=rrmse(f64(back(out["o"])), o64), dq=rrmse(f64(back(out["dq"])), dq64),
                dk=rrmse(f64(back(out["dk"])), dk64), dv=rrmse(f64(back(out["dv"])), dv64),
                dbias=rrmse(f64(out["dbias"]), db64))
    print("ending node vs oracle", {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o"] <= TOL_O_RRMSE, errs
    for g in ("dq", "dk", "dv", "dbias"):
        assert errs[g] <= TOL_GRAD_RRMSE, (g, errs)


def test_autograd_pair_end():
    import triangle_attention_amd as ta
    B, N, H, D = 1, 96, 2, 16
    inp = _inputs(B, N, H, D, True, seed=31)
    base = {n: to_dev(inp[n]) for n in TOK + ("bias",)}
    m = mask_dev(inp["key_mask"])
    ref = _run(ta, dict(base, mask=m), "slice_head", True)
    leaves = {n: to_pair_end(base[n]).requires_grad_(True) for n in ("q", "k", "v")}
    bias = base["bias"].clone().requires_grad_(True)
    o = ta.triangle_attention(leaves["q"], leaves["k"], leaves["v"], bias, m, layout="pair_end")
    o.backward(to_pair_end(base["dO"]))
    torch.cuda.synchronize()
    assert torch.equal(_bits(from_pair_end(o.detach()).contiguous()), _bits(ref["o"]))
    for n in ("q", "k", "v"):
        assert torch.equal(_bits(from_pair_end(leaves[n].grad).contiguous()), _bits(ref["d" + n])), n
    assert torch.equal(_bits(bias.grad), _bits(ref["dbias"].to(torch.bfloat16)))
