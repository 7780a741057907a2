"""Plain, slow FP64 reference for triangle attention (starting node), forward and backward.

Test infrastructure only (see the package docstring): nothing in the GPU path
imports this module.

Conventions (all arrays float64 unless stated):
  q, k, v, dO : [B, N, H, N, d]   index [b, i, h, j, c]
  bias        : [B, H, N, N]      index [b, h, j, k]; the same bias serves every slice i
  key_mask    : [B, N, N] uint8   index [b, i, k]; 1 keeps key k of slice i, 0 masks it
  lse         : [B, N, H, N]      natural-log logsumexp of each score row
  dbias       : [B, H, N, N]

The score of slice (b, i, h) is
    s[j, k] = alpha * sum_c q[j, c] k[k, c] + bias[b, h, j, k] + m[k],
    m[k] = -1e9 if key k of slice i is masked else 0,  alpha = d ** -0.5,
the forward is o = softmax_k(s) v, and the backward is the vector-Jacobian
product of L = sum(dO * o) with respect to q, k, v and the shared bias.
Following the TurboPairFormer abstract (arXiv 2610.05854), the bias gradient
of one slice is the score gradient dS of that slice, and because the bias is
shared, dbias is the sum of dS over all slices i.
"""
from __future__ import annotations

import numpy as np

MASK_NEG = -1e9  # additive score term for a masked key


def _alpha(d: int) -> float:
    return 1.0 / np.sqrt(d)


def slice_forward64(qs, ks, vs, bias_h, mask_row=None):
    """One attention slice.

    qs, ks, vs: [N, d]; bias_h: [N, N] (query j, key k); mask_row: [N] (1 keep) or None.
    Returns (o [N, d], lse [N], p [N, N]).
    """
    alpha = _alpha(qs.shape[1])
    s = alpha * (qs @ ks.T) + bias_h
    if mask_row is not None:
        s = s + np.where(np.asarray(mask_row) == 0, MASK_NEG, 0.0)[None, :]
    # softmax over keys, after subtracting each row's maximum
    row_max = s.max(axis=1, keepdims=True)
    e = np.exp(s - row_max)
    row_sum = e.sum(axis=1, keepdims=True)
    p = e / row_sum
    lse = row_max[:, 0] + np.log(row_sum[:, 0])
    o = p @ vs
    return o, lse, p


def slice_backward64(qs, ks, vs, bias_h, dOs, mask_row=None):
    """Gradients of L = sum(dO * o) for one slice.

    Returns (dq, dk, dv, ds) with ds = dL/ds the score gradient [N, N]; the
    slice's contribution to dbias is ds itself (the bias enters s with weight 1).
    """
    alpha = _alpha(qs.shape[1])
    o, _, p = slice_forward64(qs, ks, vs, bias_h, mask_row)
    # softmax backward correction: D[j] = sum_c dO[j,c] o[j,c] = sum_k p[j,k] dp[j,k]
    D = (dOs * o).sum(axis=1)
    dp = dOs @ vs.T                    # dL/dp[j,k] = sum_c dO[j,c] v[k,c]
    ds = p * (dp - D[:, None])         # softmax Jacobian applied row by row
    dv = p.T @ dOs                     # o = p v
    dq = alpha * (ds @ ks)             # s = alpha q k^T + ...
    dk = alpha * (ds.T @ qs)
    return dq, dk, dv, ds


def _as64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def forward64(q, k, v, bias, key_mask=None, slices=None):
    """Forward over all slices (or only the slice indices in ``slices``).

    Returns (o, lse) with full shapes [B,N,H,N,d] and [B,N,H,N]; entries of
    slices not computed are left as NaN.
    """
    q, k, v, bias = _as64(q), _as64(k), _as64(v), _as64(bias)
    B, N, H, _, d = q.shape
    o = np.full(q.shape, np.nan)
    lse = np.full((B, N, H, N), np.nan)
    for b in range(B):
        for i in (range(N) if slices is None else slices):
            mrow = None if key_mask is None else key_mask[b, i]
            for h in range(H):
                o[b, i, h], lse[b, i, h], _ = slice_forward64(q[b, i, h], k[b, i, h], v[b, i, h],
                                                              bias[b, h], mrow)
    return o, lse


def backward64(q, k, v, bias, dO, key_mask=None, slices=None):
    """Backward over all slices: returns (dq, dk, dv, dbias).

    dbias[b,h] is accumulated over slices i in ascending order.  With
    ``slices`` given, only those slices are computed (dq/dk/dv elsewhere NaN)
    and dbias is returned as None, since it needs every slice.
    """
    q, k, v, bias, dO = _as64(q), _as64(k), _as64(v), _as64(bias), _as64(dO)
    B, N, H, _, d = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(q.shape, np.nan)
    dv = np.full(q.shape, np.nan)
    dbias = np.zeros((B, H, N, N)) if slices is None else None
    for b in range(B):
        for i in (range(N) if slices is None else slices):
            mrow = None if key_mask is None else key_mask[b, i]
            for h in range(H):
                gq, gk, gv, ds = slice_backward64(q[b, i, h], k[b, i, h], v[b, i, h], bias[b, h],
                                                  dO[b, i, h], mrow)
                dq[b, i, h], dk[b, i, h], dv[b, i, h] = gq, gk, gv
                if dbias is not None:
                    dbias[b, h] += ds
    return dq, dk, dv, dbias


def dbias_rows64(q, k, v, bias, dO, rows, key_mask=None):
    """dbias[b, h, j, :] for the (b, h, j) triples in ``rows``, summed over every slice i.

    The same definition as ``backward64`` restricted to one query row: row j of
    slice i needs only q[b,i,h,j], all keys and values of the slice and dO[b,i,h,j].
    Returns an array [len(rows), N].
    """
    q, k, v, bias, dO = _as64(q), _as64(k), _as64(v), _as64(bias), _as64(dO)
    B, N, H, _, d = q.shape
    alpha = _alpha(d)
    out = np.zeros((len(rows), N))
    for r, (b, h, j) in enumerate(rows):
        for i in range(N):
            s = alpha * (k[b, i, h] @ q[b, i, h, j]) + bias[b, h, j]
            if key_mask is not None:
                s = s + np.where(key_mask[b, i] == 0, MASK_NEG, 0.0)
            e = np.exp(s - s.max())
            p = e / e.sum()
            o = p @ v[b, i, h]
            D = dO[b, i, h, j] @ o
            dp = v[b, i, h] @ dO[b, i, h, j]
            out[r] += p * (dp - D)
    return out
