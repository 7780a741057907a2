"""Pins for the FP64 oracle, each independent of the oracle's own arithmetic.

Each test checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, torch's library attention routine
with autograd (float64, CPU), or central finite differences.  Together they
fail on the plausible slips: a dropped bias or mask term, a transposed bias,
alpha applied to the bias, the mask applied on the query axis, a wrong sign in
the softmax correction, dbias summed over the wrong axis.

Method: "TurboPairFormer: Fast and Stable Protein Folding Model Training with
an Optimized Triangle Attention Kernel" (arXiv 2610.05854), Abstract: a pair
bias shared across attention slices, whose gradient is a reduction over
slices, and the softmax backward correction.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tri_synth import bf16_bits_to_f64, make_inputs


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _case(B=1, N=5, H=2, d=4, seed=0, mask=False, bias_scale=1.0):
    rng = np.random.default_rng(seed)
    q, k, v, dO = (_rand(rng, B, N, H, N, d) for _ in range(4))
    bias = _rand(rng, B, H, N, N, scale=bias_scale)
    key_mask = None
    if mask:
        key_mask = (rng.random((B, N, N)) > 0.35).astype(np.uint8)
        key_mask[:, :, 0] = 1  # every slice keeps at least one key
    return q, k, v, bias, dO, key_mask


# ---------------------------------------------------------------- closed forms

def test_softmax_rows_sum_to_one():
    q, k, v, bias, dO, m = _case(N=7, d=4, mask=True, bias_scale=4.0)
    for i in range(7):
        _, _, p = oracle.slice_forward64(q[0, i, 1], k[0, i, 1], v[0, i, 1], bias[0, 1], m[0, i])
        assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-13
        assert (p >= 0).all()


def test_uniform_attention_closed_form():
    # q = 0 and bias = 0: every score is 0, so o is the mean of the values and lse = ln N
    q, k, v, bias, dO, _ = _case(N=6, d=4)
    q[:] = 0.0
    bias[:] = 0.0
    o, lse = oracle.forward64(q, k, v, bias)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=3, keepdims=True), o.shape), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(6), rtol=0, atol=1e-14)


def test_single_token_closed_form():
    # N = 1: softmax over one key is 1, so o = v, dv = dO and every other gradient is 0
    q, k, v, bias, dO, _ = _case(N=1, H=3, d=4)
    o, lse = oracle.forward64(q, k, v, bias)
    np.testing.assert_array_equal(o, v)
    s = (q * k).sum(-1) / 2.0 + bias[:, None, :, 0, :]  # alpha = 1/2 at d = 4
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-14)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO)
    np.testing.assert_array_equal(dv, dO)
    # dp - D is zero up to round-off (two summation orders of the same dot product)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14 and np.abs(db).max() < 1e-14


def test_two_key_sigmoid_closed_form():
    # N = 2 keys: p[j,0] = sigmoid(s0 - s1); o = v1 + p0 (v0 - v1); dbias[j,0] = p0 p1 dO.(v0 - v1)
    rng = np.random.default_rng(3)
    q, k, v, dO = (rng.standard_normal((1, 2, 1, 2, 3)) for _ in range(4))
    bias = rng.standard_normal((1, 1, 2, 2))
    o, _ = oracle.forward64(q, k, v, bias)
    _, _, _, db = oracle.backward64(q, k, v, bias, dO)
    alpha = 1.0 / math.sqrt(3.0)
    want_db = np.zeros((2, 2))
    for i in range(2):
        for j in range(2):
            s0 = alpha * q[0, i, 0, j] @ k[0, i, 0, 0] + bias[0, 0, j, 0]
            s1 = alpha * q[0, i, 0, j] @ k[0, i, 0, 1] + bias[0, 0, j, 1]
            p0 = 1.0 / (1.0 + math.exp(s1 - s0))
            p1 = 1.0 - p0
            dv01 = v[0, i, 0, 0] - v[0, i, 0, 1]
            np.testing.assert_allclose(o[0, i, 0, j], v[0, i, 0, 1] + p0 * dv01, atol=1e-14)
            g = p0 * p1 * (dO[0, i, 0, j] @ dv01)
            want_db[j] += [g, -g]
    np.testing.assert_allclose(db[0, 0], want_db, atol=1e-14)


def test_zero_and_linear_in_dO():
    q, k, v, bias, dO, m = _case(N=5, d=4, mask=True)
    z = oracle.backward64(q, k, v, bias, np.zeros_like(dO), m)
    for g in z:
        assert np.abs(g).max() == 0
    rng = np.random.default_rng(7)
    dO2 = rng.standard_normal(dO.shape)
    g1 = oracle.backward64(q, k, v, bias, dO, m)
    g2 = oracle.backward64(q, k, v, bias, dO2, m)
    g12 = oracle.backward64(q, k, v, bias, 2.0 * dO - 3.0 * dO2, m)
    for a, b, c in zip(g1, g2, g12):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- mask semantics

def test_mask_equals_key_deletion():
    # Masking key k of slice i must act as if the key were not there, for that slice only.
    q, k, v, bias, dO, _ = _case(N=6, H=2, d=4, seed=11)
    keep = np.array([1, 0, 1, 1, 0, 1], dtype=np.uint8)
    m = np.ones((1, 6, 6), dtype=np.uint8)
    m[0, 2] = keep  # only slice 2 masks keys 1 and 4
    o, lse = oracle.forward64(q, k, v, bias, m)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    kept = np.flatnonzero(keep)
    for h in range(2):
        o_r, lse_r, _ = oracle.slice_forward64(q[0, 2, h], k[0, 2, h][kept], v[0, 2, h][kept], bias[0, h][:, kept])
        np.testing.assert_allclose(o[0, 2, h], o_r, atol=1e-13)
        np.testing.assert_allclose(lse[0, 2, h], lse_r, atol=1e-12)
        gq, gk, gv, ds = oracle.slice_backward64(q[0, 2, h], k[0, 2, h][kept], v[0, 2, h][kept],
                                                 bias[0, h][:, kept], dO[0, 2, h])
        np.testing.assert_allclose(dq[0, 2, h], gq, atol=1e-13)
        np.testing.assert_allclose(dk[0, 2, h][kept], gk, atol=1e-13)
        np.testing.assert_allclose(dv[0, 2, h][kept], gv, atol=1e-13)
        assert np.abs(dk[0, 2, h][[1, 4]]).max() == 0.0
        assert np.abs(dv[0, 2, h][[1, 4]]).max() == 0.0
    # the unmasked slices still use keys 1 and 4
    o_nm, _ = oracle.forward64(q, k, v, bias)
    np.testing.assert_allclose(o[0, 3], o_nm[0, 3], atol=0)


def test_tail_mask_zero_columns_in_dbias():
    q, k, v, bias, dO, _ = _case(N=6, H=2, d=4, seed=5)
    m = np.ones((1, 6, 6), dtype=np.uint8)
    m[:, :, 4:] = 0  # the last two keys of every slice
    _, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    assert np.abs(db[..., 4:]).max() == 0.0
    assert np.abs(dk[..., 4:, :]).max() == 0.0 and np.abs(dv[..., 4:, :]).max() == 0.0


def _sdpa_slices(q, k, v, bias, dO, m, slices, b):
    """Per-slice torch float64 attention with autograd over the listed slices of batch entry b:
    returns o, dq, dk, dv of those slices and the sum of their bias gradients."""
    B, N, H, _, d = q.shape
    outs, db = {}, np.zeros((H, N, N))
    for i in slices:
        t = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)  # noqa: E731
        tq, tk, tv, tb = t(q[b, i]), t(k[b, i]), t(v[b, i]), t(bias[b])
        madd = torch.where(torch.tensor(m[b, i] == 0)[None, None, :], -1e9, 0.0).double()
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tb + madd, scale=1.0 / math.sqrt(d))
        o.backward(torch.tensor(dO[b, i]))
        outs[i] = (o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())
        db += tb.grad.numpy()
    return outs, db


def test_fully_masked_slices_attend_to_nothing():
    # Slices whose every key is masked (padded residues of a cropped batch): output 0, lse = +inf,
    # no gradient, and dbias is the sum over the remaining slices only.  The remaining slices are
    # checked against torch's library attention with autograd, slice by slice.
    q, k, v, bias, dO, m = _case(B=2, N=6, H=2, d=4, seed=61, mask=True)
    empty = {0: [1, 4], 1: [5]}
    for b, sl in empty.items():
        m[b, sl] = 0
    o, lse = oracle.forward64(q, k, v, bias, m)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    for b, sl in empty.items():
        assert np.abs(o[b, sl]).max() == 0.0
        assert np.isposinf(lse[b, sl]).all()
        for g in (dq, dk, dv):
            assert np.abs(g[b, sl]).max() == 0.0
        rest = [i for i in range(6) if i not in sl]
        assert np.isfinite(lse[b, rest]).all()
        ref, db_ref = _sdpa_slices(q, k, v, bias, dO, m, rest, b)
        for i in rest:
            for got, want in zip((o[b, i], dq[b, i], dk[b, i], dv[b, i]), ref[i]):
                np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(db[b], db_ref, rtol=1e-10, atol=1e-11)
    # the same rows through the row-restricted dbias
    rows = [(0, 1, 2), (1, 0, 5)]
    got = oracle.dbias_rows64(q, k, v, bias, dO, rows, m)
    for r, (b, h, j) in enumerate(rows):
        np.testing.assert_allclose(got[r], db[b, h, j], atol=1e-13)


def test_row_with_only_minus_inf_bias_attends_to_nothing():
    # A query row whose keys all carry a -inf bias has no finite score: o = 0, lse = +inf, and the
    # row adds nothing to any gradient.  So every gradient equals that of the same problem with the
    # row's bias made finite and its output gradient set to zero (which also adds nothing).
    q, k, v, bias, dO, m = _case(B=1, N=5, H=2, d=4, seed=71)
    j, h = 3, 1
    bias_inf = bias.copy()
    bias_inf[0, h, j, :] = -np.inf
    o, lse = oracle.forward64(q, k, v, bias_inf)
    assert np.abs(o[0, :, h, j]).max() == 0.0 and np.isposinf(lse[0, :, h, j]).all()
    assert np.isfinite(lse[0, :, 0]).all()
    g_inf = oracle.backward64(q, k, v, bias_inf, dO)
    dO0 = dO.copy()
    dO0[0, :, h, j] = 0.0
    g_ref = oracle.backward64(q, k, v, bias, dO0)
    for a, b_ in zip(g_inf, g_ref):
        np.testing.assert_allclose(a, b_, rtol=1e-12, atol=1e-13)
    # a -inf bias on some keys only: those keys get exactly zero probability (key deletion)
    bias_part = bias.copy()
    bias_part[0, h, :, [0, 2]] = -np.inf
    o_p, _ = oracle.forward64(q, k, v, bias_part)
    keep = [1, 3, 4]
    for i in range(5):
        o_r, _, _ = oracle.slice_forward64(q[0, i, h], k[0, i, h][keep], v[0, i, h][keep], bias[0, h][:, keep])
        np.testing.assert_allclose(o_p[0, i, h], o_r, atol=1e-13)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("mask", [False, True])
def test_gradient_invariants(mask):
    q, k, v, bias, dO, m = _case(N=7, H=2, d=4, seed=21, mask=mask, bias_scale=2.0)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    # softmax is invariant to adding a constant along k: sum_k dbias = 0, sum_k dk = 0
    assert np.abs(db.sum(axis=-1)).max() < 1e-12
    assert np.abs(dk.sum(axis=3)).max() < 1e-12
    # sum_k p = 1 gives sum_k dv[k] = sum_j dO[j]
    np.testing.assert_allclose(dv.sum(axis=3), dO.sum(axis=3), atol=1e-12)
    # scaling q and k together: sum q.dq = sum k.dk in every slice
    np.testing.assert_allclose((q * dq).sum(axis=(3, 4)), (k * dk).sum(axis=(3, 4)), atol=1e-12)


def test_slice_permutation_equivariance():
    q, k, v, bias, dO, m = _case(N=5, H=2, d=4, seed=8, mask=True)
    perm = np.array([3, 0, 4, 1, 2])
    o, lse = oracle.forward64(q, k, v, bias, m)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    P = lambda x: x[:, perm]  # noqa: E731
    o_p, _ = oracle.forward64(P(q), P(k), P(v), bias, m[:, perm])
    dq_p, dk_p, dv_p, db_p = oracle.backward64(P(q), P(k), P(v), bias, P(dO), m[:, perm])
    np.testing.assert_allclose(o_p, P(o), atol=1e-14)
    np.testing.assert_allclose(dq_p, P(dq), atol=1e-14)
    np.testing.assert_allclose(dk_p, P(dk), atol=1e-14)
    np.testing.assert_allclose(dv_p, P(dv), atol=1e-14)
    np.testing.assert_allclose(db_p, db, atol=1e-12)  # only the summation order changes


def test_key_permutation_invariance():
    q, k, v, bias, dO, m = _case(N=5, H=2, d=4, seed=9, mask=True)
    perm = np.array([2, 4, 0, 3, 1])
    o, lse = oracle.forward64(q, k, v, bias, m)
    _, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    kp = k[:, :, :, perm]
    vp = v[:, :, :, perm]
    bp = bias[..., perm]
    mp = m[..., perm]
    o2, lse2 = oracle.forward64(q, kp, vp, bp, mp)
    _, dk2, dv2, db2 = oracle.backward64(q, kp, vp, bp, dO, mp)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    np.testing.assert_allclose(dk2, dk[:, :, :, perm], atol=1e-13)
    np.testing.assert_allclose(dv2, dv[:, :, :, perm], atol=1e-13)
    np.testing.assert_allclose(db2, db[..., perm], atol=1e-13)


# ---------------------------------------------------------------- library routine + autograd

def _torch_reference(q, k, v, bias, dO, m):
    """torch's scaled_dot_product_attention in float64 with autograd; bias is one shared leaf."""
    B, N, H, _, d = q.shape
    t = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)  # noqa: E731
    tq, tk, tv, tb = t(q), t(k), t(v), t(bias)
    madd = torch.zeros((B, N, 1, 1, N), dtype=torch.float64)
    if m is not None:
        madd = torch.where(torch.tensor(m == 0)[:, :, None, None, :], -1e9, 0.0).double()
    # [B, N(slice), H, Nq, Nk] additive mask: the shared bias broadcast over slices plus the key mask
    attn = tb[:, None] + madd
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn, scale=1.0 / math.sqrt(d))
    o.backward(torch.tensor(dO, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), tb.grad.numpy()


@pytest.mark.parametrize("mask", [False, True])
@pytest.mark.parametrize("B,N,H,d", [(1, 6, 2, 4), (1, 9, 3, 8), (1, 17, 2, 16), (2, 6, 2, 4), (2, 9, 3, 8)])
def test_matches_torch_sdpa_autograd(B, N, H, d, mask):
    # B = 2 draws a different bias and key mask for each batch entry, so a batch-index slip in the
    # oracle (bias[0] or key_mask[0] used for b = 1) fails here
    q, k, v, bias, dO, m = _case(B=B, N=N, H=H, d=d, seed=N * 10 + d + 1000 * (B - 1), mask=mask, bias_scale=2.0)
    if B > 1:
        assert np.abs(bias[1] - bias[0]).max() > 0.5
        assert m is None or (m[1] != m[0]).any()
    ro, rdq, rdk, rdv, rdb = _torch_reference(q, k, v, bias, dO, m)
    o, _ = oracle.forward64(q, k, v, bias, m)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dq, rdq, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, rdk, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, rdv, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(db, rdb, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("B", [1, 2])
def test_dbias_is_slice_sum_of_per_slice_bias_gradients(B):
    # Give every slice its own bias leaf [B, N(slice), H, N, N]; their gradients summed over slices
    # must equal the oracle's shared-bias gradient (per batch entry, with per-batch bias and mask).
    q, k, v, bias, dO, m = _case(B=B, N=6, H=2, d=4, seed=31, mask=True)
    B, N, H, _, d = q.shape
    per = torch.tensor(np.broadcast_to(bias[:, None], (B, N, H, N, N)).copy(), requires_grad=True)
    madd = torch.where(torch.tensor(m == 0)[:, :, None, None, :], -1e9, 0.0).double()
    o = F.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                       attn_mask=per + madd, scale=1.0 / math.sqrt(d))
    o.backward(torch.tensor(dO))
    _, _, _, db = oracle.backward64(q, k, v, bias, dO, m)
    np.testing.assert_allclose(db, per.grad.numpy().sum(axis=1), rtol=1e-10, atol=1e-11)


def test_lse_from_library_probabilities():
    # SDPA with v = identity returns the probability matrix; lse[j] = s[j,k] - log p[j,k] for every k.
    rng = np.random.default_rng(4)
    N, d = 7, 4
    qs, ks = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    b = rng.standard_normal((N, N)) * 3
    p = F.scaled_dot_product_attention(torch.tensor(qs)[None], torch.tensor(ks)[None],
                                       torch.eye(N, dtype=torch.float64)[None],
                                       attn_mask=torch.tensor(b)[None], scale=0.5)[0].numpy()
    _, lse, _ = oracle.slice_forward64(qs, ks, rng.standard_normal((N, d)), b)
    s = 0.5 * qs @ ks.T + b
    np.testing.assert_allclose(lse[:, None] * np.ones((1, N)), s - np.log(p), atol=1e-12)


# ---------------------------------------------------------------- finite differences

def _loss(q, k, v, bias, dO, m):
    o, _ = oracle.forward64(q, k, v, bias, m)
    return float((o * dO).sum())


@pytest.mark.parametrize("B,N,d,mask", [(1, 2, 2, False), (1, 3, 4, True), (1, 5, 2, True), (1, 5, 4, False),
                                         (2, 3, 2, True), (2, 4, 2, False)])
def test_central_finite_differences(B, N, d, mask):
    q, k, v, bias, dO, m = _case(B=B, N=N, H=2, d=d, seed=100 + N * d + B, mask=mask)
    dq, dk, dv, db = oracle.backward64(q, k, v, bias, dO, m)
    eps = 1e-6
    rng = np.random.default_rng(0)
    for x, g in ((q, dq), (k, dk), (v, dv), (bias, db)):
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 24), replace=False)
        for t in idx:
            old = flat[t]
            flat[t] = old + eps
            lp = _loss(q, k, v, bias, dO, m)
            flat[t] = old - eps
            lm = _loss(q, k, v, bias, dO, m)
            flat[t] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g.reshape(-1)[t]) < 1e-7 * max(1.0, abs(fd)), (t, fd, g.reshape(-1)[t])


# ---------------------------------------------------------------- row-restricted dbias

def test_dbias_rows_match_full():
    q, k, v, bias, dO, m = _case(N=6, H=2, d=4, seed=41, mask=True)
    _, _, _, db = oracle.backward64(q, k, v, bias, dO, m)
    rows = [(0, 0, 0), (0, 1, 3), (0, 1, 5)]
    got = oracle.dbias_rows64(q, k, v, bias, dO, rows, m)
    for r, (b, h, j) in enumerate(rows):
        np.testing.assert_allclose(got[r], db[b, h, j], atol=1e-13)


def test_slice_subset_matches_full():
    q, k, v, bias, dO, m = _case(N=6, H=2, d=4, seed=42, mask=True)
    o, lse = oracle.forward64(q, k, v, bias, m)
    o2, lse2 = oracle.forward64(q, k, v, bias, m, slices=[1, 4])
    np.testing.assert_array_equal(o2[:, [1, 4]], o[:, [1, 4]])
    assert np.isnan(o2[:, 0]).all()
    dq, dk, dv, _ = oracle.backward64(q, k, v, bias, dO, m)
    dq2, dk2, dv2, db2 = oracle.backward64(q, k, v, bias, dO, m, slices=[2])
    assert db2 is None
    np.testing.assert_array_equal(dq2[:, 2], dq[:, 2])
    np.testing.assert_array_equal(dk2[:, 2], dk[:, 2])
    np.testing.assert_array_equal(dv2[:, 2], dv[:, 2])


# ---------------------------------------------------------------- input generator

def test_bf16_inputs_roundtrip_and_determinism():
    a = make_inputs(1, 8, 2, 16, seed=3, mask_tail=2)
    b = make_inputs(1, 8, 2, 16, seed=3, mask_tail=2)
    for name in ("q", "k", "v", "bias", "dO"):
        np.testing.assert_array_equal(a[name], b[name])
    x = bf16_bits_to_f64(a["q"])
    # bf16 values have at most 8 significant bits
    mant = np.frexp(x)[0] * 256
    assert np.all(mant == np.round(mant))
    assert a["key_mask"][0, :, 6:].max() == 0 and a["key_mask"][0, :, :6].min() == 1
    # ties round to even: 1 + 2^-8 (exactly half an ulp) rounds down to 1
    from tri_synth import f32_to_bf16_bits
    assert f32_to_bf16_bits(np.array([1.0 + 2 ** -8], dtype=np.float32))[0] == 0x3F80
    assert f32_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8], dtype=np.float32))[0] == 0x3F82
