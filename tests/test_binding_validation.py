"""The Python binding rejects tensors the C entry points would misread (CPU, no GPU needed).

The C ABI takes raw device pointers in a fixed layout (include/tri_attn.h, include/tri_mul.h),
so a strided view, another dtype, a host tensor or a wrong shape must be refused before any
call: each case below raises ValueError naming the offending argument.
"""
import pytest
import torch

import triangle_attention_amd as ta

B, N, H, D = 2, 6, 3, 16


def _tok(dtype=torch.bfloat16, shape=(B, N, H, N, D)):
    return torch.zeros(shape, dtype=dtype)


def _args(**over):
    a = dict(q=_tok(), k=_tok(), v=_tok(), bias=torch.zeros((B, H, N, N), dtype=torch.bfloat16),
             key_mask=torch.ones((B, N, N), dtype=torch.uint8))
    a.update(over)
    return a


def _fwd(**over):
    a = _args(**over)
    return ta.forward(a["q"], a["k"], a["v"], a["bias"], a["key_mask"])


@pytest.mark.parametrize("name,value,match", [
    ("q", _tok().permute(0, 1, 3, 2, 4).contiguous().permute(0, 1, 3, 2, 4), "contiguous"),
    ("k", _tok(torch.float32), "dtype"),
    ("v", _tok(shape=(B, N, H, N + 1, D)), "shape"),
    ("bias", torch.zeros((B, H, N, N + 1), dtype=torch.bfloat16), "shape"),
    ("bias", torch.zeros((B, H, N, N), dtype=torch.float32), "dtype"),
    ("bias", torch.zeros((B, H, N, N), dtype=torch.bfloat16).transpose(2, 3), "contiguous"),
    ("key_mask", torch.ones((B, N, N), dtype=torch.int32), "dtype"),
    ("key_mask", torch.ones((1, N, N), dtype=torch.uint8), "shape"),
])
def test_forward_rejects(name, value, match):
    with pytest.raises(ValueError, match=match):
        _fwd(**{name: value})
    with pytest.raises(ValueError, match=name):
        _fwd(**{name: value})


def test_permuted_pair_view_is_rejected():
    # the usual way to get [B, N, H, N, D] from a pair tensor [B, N, N, H, D] is a permuted view;
    # it must be made contiguous (or passed with layout="pair_start") rather than misread
    pair = torch.zeros((B, N, N, H, D), dtype=torch.bfloat16)
    view = pair.permute(0, 1, 3, 2, 4)
    with pytest.raises(ValueError, match="q must be contiguous"):
        _fwd(q=view)


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="q must be on a GPU"):
        _fwd()


def test_bool_mask_and_no_mask_pass_the_checks():
    # a bool mask (one byte per entry, 1 = keep) and no mask are accepted; the host tensors then
    # fail on the device check, not on the mask
    with pytest.raises(ValueError, match="on a GPU"):
        _fwd(key_mask=torch.ones((B, N, N), dtype=torch.bool))
    with pytest.raises(ValueError, match="on a GPU"):
        _fwd(key_mask=None)


def test_head_dim_and_layout():
    with pytest.raises(ValueError, match="head dimension"):
        _fwd(q=_tok(shape=(B, N, H, N, 8)), k=_tok(shape=(B, N, H, N, 8)), v=_tok(shape=(B, N, H, N, 8)))
    with pytest.raises(ValueError, match="layout"):
        ta.forward(_tok(), _tok(), _tok(), torch.zeros((B, H, N, N), dtype=torch.bfloat16), layout="nope")
    with pytest.raises(ValueError, match="equal slice and token"):
        _fwd(q=_tok(shape=(B, N, H, N + 2, D)))


@pytest.mark.parametrize("name,value,match", [
    ("o", _tok(torch.float32), "dtype"),
    ("lse", torch.zeros((B, N, H, N), dtype=torch.bfloat16), "dtype"),
    ("lse", torch.zeros((B, N, H, N + 1), dtype=torch.float32), "shape"),
    ("residual", _tok(shape=(B, N, H, N, 32)), "shape"),
    ("dO", _tok().transpose(3, 4).contiguous().transpose(3, 4), "contiguous"),
])
def test_backward_rejects(name, value, match):
    a = _args()
    b = dict(o=_tok(), lse=torch.zeros((B, N, H, N), dtype=torch.float32), residual=_tok(), dO=_tok())
    b[name] = value
    with pytest.raises(ValueError, match=match):
        ta.backward(a["q"], a["k"], a["v"], a["bias"], a["key_mask"], b["o"], b["lse"], b["residual"], b["dO"])


def test_tri_mul_rejects():
    a = torch.zeros((1, 8, 8, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="b must have shape"):
        ta.triangle_multiplication(a, torch.zeros((1, 8, 8, 8), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="a must have dtype"):
        ta.triangle_multiplication(a.float(), a)
    with pytest.raises(ValueError, match="contiguous"):
        ta.triangle_multiplication(a.transpose(1, 2), a)
    with pytest.raises(ValueError, match="on a GPU"):
        ta.triangle_multiplication(a, a)
    with pytest.raises(ValueError, match="mask must have shape"):
        ta.gated_operand(a, a, torch.ones((1, 8, 7), dtype=torch.uint8))
