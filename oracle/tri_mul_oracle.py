"""FP64 CPU oracle for the triangle multiplication core (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may use it; the
GPU product path never calls it and shares no code with it.

Source: the kongchang.com article on fast_trimul, section "什么是三角乘法更新" (what the
triangle multiplicative update is).  The update lets each residue pair (i, j) gather
information through a third residue k.  Along the rows or the columns of the N x N pair
representation, it combines elementwise gating, an outer product and a reduction over one
index.  TurboPairFormer's Abstract places triangle multiplication kernels next to its
attention kernel in the OpenFold3 step.

Reading taken here (the pages print no formula): the cubic core of the update, for pair
tensors a, b of shape [B, N, N, C] (channels last) that already carry their gating:
  outgoing ("rows"):    x[b,i,j,c] = sum_k a[b,i,k,c] * b[b,j,k,c]
  incoming ("columns"): x[b,i,j,c] = sum_k a[b,k,i,c] * b[b,k,j,c]
Each channel is an independent product of two N x N matrices, so the definition below is
a per-channel matrix product in float64.  The gradients follow from x being bilinear in
(a, b): for a loss with gradient dx,
  outgoing: da[i,k,c] = sum_j dx[i,j,c] b[j,k,c],   db[j,k,c] = sum_i dx[i,j,c] a[i,k,c]
  incoming: da[k,i,c] = sum_j dx[i,j,c] b[k,j,c],   db[k,j,c] = sum_i dx[i,j,c] a[k,i,c]
"""
from __future__ import annotations

import numpy as np

DIRECTIONS = ("outgoing", "incoming")


def _check(direction: str):
    if direction not in DIRECTIONS:
        raise ValueError(f"direction must be one of {DIRECTIONS}")


def _channel_major(t: np.ndarray) -> np.ndarray:
    """[B, N, N, C] -> [B, C, N, N] float64 (each channel as a plain matrix)."""
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64).transpose(0, 3, 1, 2))


def _pair_major(t: np.ndarray) -> np.ndarray:
    """[B, C, N, N] -> [B, N, N, C]."""
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1))


def tri_mul_forward64(a: np.ndarray, b: np.ndarray, direction: str = "outgoing") -> np.ndarray:
    """x per the definition above; a, b: [B, N, N, C] (any real dtype); returns float64."""
    _check(direction)
    A, Bm = _channel_major(a), _channel_major(b)
    if direction == "outgoing":
        X = A @ Bm.transpose(0, 1, 3, 2)   # X_c = A_c B_c^T: rows i of A, rows j of B, k shared
    else:
        X = A.transpose(0, 1, 3, 2) @ Bm   # X_c = A_c^T B_c: columns i of A, columns j of B
    return _pair_major(X)


def tri_mul_backward64(a: np.ndarray, b: np.ndarray, dx: np.ndarray, direction: str = "outgoing"):
    """(da, db) for upstream gradient dx; all [B, N, N, C]; returns float64."""
    _check(direction)
    A, Bm, dX = _channel_major(a), _channel_major(b), _channel_major(dx)
    if direction == "outgoing":
        dA = dX @ Bm                        # da[i,k] = sum_j dx[i,j] b[j,k]
        dB = dX.transpose(0, 1, 3, 2) @ A   # db[j,k] = sum_i dx[i,j] a[i,k]
    else:
        dA = Bm @ dX.transpose(0, 1, 3, 2)  # da[k,i] = sum_j b[k,j] dx[i,j]
        dB = A @ dX                         # db[k,j] = sum_i a[k,i] dx[i,j]
    return _pair_major(dA), _pair_major(dB)


def tri_mul_loops64(a: np.ndarray, b: np.ndarray, direction: str = "outgoing") -> np.ndarray:
    """The same definition as explicit loops over (b, i, j, k, c); for tiny inputs only."""
    _check(direction)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    Bn, N, _, C = a.shape
    x = np.zeros((Bn, N, N, C))
    for bb in range(Bn):
        for i in range(N):
            for j in range(N):
                for c in range(C):
                    s = 0.0
                    for k in range(N):
                        if direction == "outgoing":
                            s += a[bb, i, k, c] * b[bb, j, k, c]
                        else:
                            s += a[bb, k, i, c] * b[bb, k, j, c]
                    x[bb, i, j, c] = s
    return x


# ---------------------------------------------------------------------------- input gating
# The same section of the article names elementwise gating as the update's first step.  The
# plainest reading, as in AlphaFold-family models: each operand of the product is a projection
# of the pair representation gated elementwise by the sigmoid of another projection, and pair
# entries outside the pair mask contribute nothing:
#   a[b,i,j,c] = sigmoid(g[b,i,j,c]) * p[b,i,j,c] * mask[b,i,j]
def _sigmoid64(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gate_forward64(g, p, mask=None):
    """a = sigmoid(g) * p (* mask[..., None]); g, p: [B, N, N, C]; mask: [B, N, N] or None."""
    a = _sigmoid64(g) * np.asarray(p, dtype=np.float64)
    if mask is not None:
        a = a * np.asarray(mask, dtype=np.float64)[..., None]
    return a


def gate_backward64(g, p, da, mask=None):
    """(dg, dp) for upstream gradient da: dp = da * sigmoid(g) * m, dg = da * p * m * s (1 - s)."""
    s = _sigmoid64(g)
    m = 1.0 if mask is None else np.asarray(mask, dtype=np.float64)[..., None]
    da = np.asarray(da, dtype=np.float64) * m
    return da * np.asarray(p, dtype=np.float64) * s * (1.0 - s), da * s
