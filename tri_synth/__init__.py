"""Seeded synthetic inputs for starting-node triangle attention.

This module is shared by the CPU oracle's tests and the GPU path's tests and
benchmark.  It holds no arithmetic of the method: it only draws normal
variates, rounds them to bfloat16 and builds key-padding masks, so that both
sides see bit-identical inputs.

Workloads follow the evaluation grid of "TurboPairFormer: Fast and Stable
Protein Folding Model Training with an Optimized Triangle Attention Kernel"
(arXiv 2610.05854), Abstract: bf16 inputs, crop sizes 384/640/768, head
dimensions 16 and 32.  The pages name no dataset; these synthetic tensors are
the workload.

Layout (all row-major, contiguous):
  q, k, v, dO : [B, N, H, N, D]   index [b, i, h, j, c]  (i = slice, j = token)
  bias        : [B, H, N, N]      index [b, h, j, k], shared by every slice i
  key_mask    : [B, N, N] uint8   index [b, i, k], 1 = keep, 0 = masked
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "f32_to_bf16_bits", "bf16_bits_to_f64", "make_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int
    D: int
    bias_std: float = 1.0
    mask_tail: int = 0  # number of trailing keys masked in every slice
    seed: int = 0

    @property
    def flops_fwd(self) -> float:
        # two dense contractions (Q K^T and P V) of depth D per score element
        return 4.0 * self.B * self.N ** 3 * self.H * self.D

    @property
    def flops_bwd(self) -> float:
        # five contractions (S, dP, dV, dK, dQ): 2.5x the forward
        return 2.5 * self.flops_fwd


# The synthetic workloads: tiny latency case, crop 384, masked crop 640, crop 768 at both head
# dims (the d=16 one with a wide bias to stress softmax), and a crop of 1024, past the 768
# queries one backward work-group covers (its backward runs in two query chunks).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("n64_h4_d16", 1, 64, 4, 16, seed=1),
        Workload("n384_h4_d32", 1, 384, 4, 32, seed=2),
        Workload("n640_h4_d16_mask64", 1, 640, 4, 16, mask_tail=64, seed=3),
        Workload("n768_h4_d32", 1, 768, 4, 32, seed=4),
        Workload("n768_h4_d16_bias4", 1, 768, 4, 16, bias_std=4.0, seed=5),
        Workload("n1024_h4_d32", 1, 1024, 4, 32, seed=6),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def make_inputs(B: int, N: int, H: int, D: int, *, bias_std: float = 1.0, mask_tail: int = 0,
                seed: int = 0, with_mask: bool | None = None) -> dict:
    """Draw q, k, v, bias, dO in that order from PCG64(seed), standard normal float32, then RNE to bf16.

    Returns a dict of uint16 bf16 bit arrays ('q','k','v','bias','dO') and 'key_mask' (uint8 or None).
    bias is multiplied by bias_std in float32 before rounding.  The mask keeps keys k < N - mask_tail.
    """
    rng = np.random.default_rng(seed)
    shp = (B, N, H, N, D)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = f32_to_bf16_bits(rng.standard_normal(shp, dtype=np.float32))
    bias = rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(bias_std)
    out["bias"] = f32_to_bf16_bits(bias)
    out["dO"] = f32_to_bf16_bits(rng.standard_normal(shp, dtype=np.float32))
    if with_mask is None:
        with_mask = mask_tail > 0
    if with_mask:
        m = np.ones((B, N, N), dtype=np.uint8)
        if mask_tail > 0:
            m[:, :, N - mask_tail:] = 0
        out["key_mask"] = m
    else:
        out["key_mask"] = None
    return out


def workload_inputs(w: Workload) -> dict:
    return make_inputs(w.B, w.N, w.H, w.D, bias_std=w.bias_std, mask_tail=w.mask_tail, seed=w.seed)


def make_pair_inputs(B: int, N: int, C: int, *, seed: int = 0, scale: float = 1.0) -> dict:
    """Pair tensors for the triangle multiplication core: a, b, dx drawn in that order from
    PCG64(seed), standard normal float32 times `scale`, then RNE to bf16; uint16 bit arrays of
    shape [B, N, N, C] (channels last)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("a", "b", "dx"):
        out[name] = f32_to_bf16_bits(rng.standard_normal((B, N, N, C), dtype=np.float32) * np.float32(scale))
    return out


# triangle multiplication workloads: the crop of the attention headline with AlphaFold3's
# hidden width of the multiplicative update (128 channels), and a small case
TRIMUL_WORKLOADS = {
    "trimul_n768_c128": dict(B=1, N=768, C=128, seed=2024),
    "trimul_n64_c128": dict(B=1, N=64, C=128, seed=2025),
}
