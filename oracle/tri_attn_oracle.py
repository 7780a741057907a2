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
    s[j, k] = alpha * sum_c q[j, c] k[k, c] + bias[b, h, j, k] + m[k],  alpha = d ** -0.5,
the forward is o = softmax_k(s) v, and the backward is the vector-Jacobian
product of L = sum(dO * o) with respect to q, k, v and the shared bias.
Following the TurboPairFormer abstract (arXiv 2610.05854), the bias gradient
of one slice is the score gradient dS of that slice, and because the bias is
shared, dbias is the sum of dS over all slices i.

Key mask.  The workloads describe the mask as an additive -1e9 on the score of
a masked key.  That term stands for leaving the key out: whenever a row keeps
a key with a finite score, exp(-1e9 + O(1)) is exactly 0 in float64 and the
result is the same as with m[k] = -inf.  The oracle therefore writes m[k] =
-inf, which also settles the case the -1e9 form leaves open: a row with no key
of finite score (every key of its slice masked, or every key carrying a -inf
bias) attends to nothing, so its output is 0, its lse is +inf (the value whose
exp(s - lse) gives zero probability) and it contributes no gradient.  Bias
values are finite or -inf.
"""
from __future__ import annotations

import numpy as np

MASK_NEG = -1e9  # additive score term for a masked key, as the workloads state it (see above)


def _alpha(d: int) -> float:
    return 1.0 / np.sqrt(d)


def slice_forward64(qs, ks, vs, bias_h, mask_row=None):
    """One attention slice.

    qs, ks, vs: [N, d]; bias_h: [N, N] (query j, key k); mask_row: [N] (1 keep) or None.
    Returns (o [N, d], lse [N], p [N, N]).
    """
    alpha = _alpha(qs.shape[1])
    s = _scores(alpha, qs, ks, bias_h, mask_row)
    p, lse = _softmax_rows(s)
    o = p @ vs
    return o, lse, p


def _scores(alpha, qs, ks, bias_h, mask_row):
    """s[j, k] = alpha q[j].k[k] + bias[j, k], with masked keys left out (-inf)."""
    s = alpha * (qs @ ks.T) + bias_h
    if mask_row is not None:
        s = np.where(np.asarray(mask_row)[None, :] == 0, -np.inf, s)
    return s


def _softmax_rows(s):
    """Softmax over keys of each row of s, after subtracting the row's maximum, and the row's
    logsumexp.  A row with no finite score attends to nothing: p = 0 and lse = +inf."""
    row_max = s.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(row_max)
    shift = np.where(empty, 0.0, row_max)
    e = np.exp(s - shift)
    row_sum = e.sum(axis=-1, keepdims=True)
    p = np.where(empty, 0.0, e / np.where(empty, 1.0, row_sum))
    lse = np.where(empty, np.inf, shift + np.log(np.where(empty, 1.0, row_sum)))
    return p, lse[..., 0]


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
            mrow = None if key_mask is None else key_mask[b, i]
            s = _scores(alpha, q[b, i, h, j][None, :], k[b, i, h], bias[b, h, j][None, :], mrow)[0]
            p, _ = _softmax_rows(s)
            o = p @ v[b, i, h]
            D = dO[b, i, h, j] @ o
            dp = v[b, i, h] @ dO[b, i, h, j]
            out[r] += p * (dp - D)
    return out
