"""The allocation-free forward (tri_attn_fwd_noalloc, scratch inside the library) against the
workspace forward (tri_attn_fwd) through the C ABI.

Both run the same kernels on the same inputs, so o, lse and the residual must agree bit for bit.
Two calls in a row on one GPU, the second with a smaller input, check that the shared scratch
array carries nothing from one call into the next.
"""
import numpy as np
import pytest
import torch

from tri_synth import make_inputs

from ._util import mask_dev, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _case(B, N, H, D, masked, seed):
    inp = make_inputs(B, N, H, D, seed=seed, bias_std=2.0)
    if masked:
        rng = np.random.default_rng(seed)
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, 0] = 1
        m[0, 1] = 0  # one slice with every key masked
        inp["key_mask"] = m
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "bias")}
    t["mask"] = mask_dev(inp["key_mask"])
    return t


def _outputs(q, B, N, H):
    o = torch.empty_like(q)
    res = torch.empty_like(q)
    lse = torch.empty((B, N, H, N), dtype=torch.float32, device=q.device)
    for x in (o, res, lse):
        x.view(torch.uint8).fill_(0x7F)  # poisoned: a skipped write shows up
    return o, lse, res


def test_noalloc_forward_matches_workspace_forward():
    import triangle_attention_amd as ta
    # the headline shape (9.4 MB of scratch), then a smaller masked, ragged one
    cases = [(1, 768, 4, 32, False, 11), (2, 200, 3, 16, True, 12)]
    for B, N, H, D, masked, seed in cases:
        print(f"noalloc forward B={B} N={N} H={H} D={D} masked={masked}", flush=True)
        t = _case(B, N, H, D, masked, seed)
        q, k, v, bias, m = t["q"], t["k"], t["v"], t["bias"], t["mask"]
        ref = _outputs(q, B, N, H)
        ws = torch.empty(ta.tri_attn_fwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device=q.device)
        assert ta.tri_attn_fwd(B, N, H, D, q, k, v, bias, m, *ref, ws, ws.numel()) == 0
        got = _outputs(q, B, N, H)
        assert ta.tri_attn_fwd_noalloc(B, N, H, D, q, k, v, bias, m, *got) == 0
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "res"), got, ref):
            assert torch.equal(_bits(a), _bits(b)), (N, name)
        assert torch.isfinite(got[1]).float().mean() > 0.9


def test_noalloc_forward_rejects_oversized_shape():
    import triangle_attention_amd as ta
    B, N, H, D = 1, 768, 29, 16  # 29 heads at N = 768 need more than the 64 MiB of scratch
    q = torch.zeros((B, N, H, N, D), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((B, H, N, N), dtype=torch.bfloat16, device="cuda")
    o, lse, res = _outputs(q, B, N, H)
    assert ta.tri_attn_fwd_noalloc(B, N, H, D, q, q, q, bias, None, o, lse, res) == 6  # SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert (o.view(torch.uint8) == 0x7F).all()  # nothing was launched
