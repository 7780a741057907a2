"""Shared helpers for the GPU tests: move seeded bf16 inputs to the device, run the HIP
path through the C ABI, and compare with the FP64 oracle."""
from __future__ import annotations

import numpy as np
import torch

from tri_synth import bf16_bits_to_f64

# Bounds stated for this path: forward max-abs(o) <= 2e-2, rel-RMSE(o) <= 1e-2 and
# rel-RMSE <= 3e-2 for each gradient, all against the FP64 oracle.
TOL_O_MAXABS = 2e-2
TOL_O_RRMSE = 1e-2
TOL_GRAD_RRMSE = 3e-2
TOL_LSE_MAXABS = 1e-4  # internal check: FP32 logsumexp of exact bf16 products


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def mask_dev(m, device="cuda"):
    return None if m is None else torch.from_numpy(np.ascontiguousarray(m)).to(device)


def f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def rrmse(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.sqrt((ref ** 2).sum())
    return float(np.sqrt(((x - ref) ** 2).sum()) / max(den, 1e-300))


def maxabs(x, ref) -> float:
    return float(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64)).max())


def inputs64(inp: dict) -> dict:
    out = {n: bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "bias", "dO")}
    out["key_mask"] = inp["key_mask"]
    return out


def run_gpu(inp: dict, residual=True):
    """Forward + backward through the C entry points; returns a dict of torch tensors."""
    import triangle_attention_amd as ta
    q, k, v, bias, dO = (to_dev(inp[n]) for n in ("q", "k", "v", "bias", "dO"))
    m = mask_dev(inp["key_mask"])
    o, lse, res = ta.forward(q, k, v, bias, m, residual_compensation=residual)
    dq, dk, dv, dbias = ta.backward(q, k, v, bias, m, o, lse, res, dO)
    torch.cuda.synchronize()
    return dict(o=o, lse=lse, res=res, dq=dq, dk=dk, dv=dv, dbias=dbias)
