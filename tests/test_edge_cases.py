"""GPU edge cases against the FP64 oracle, through the C ABI.

- Rows with no key of finite score (fully masked slices of a padded batch, queries whose every
  key carries a -inf bias) attend to nothing: o = 0, lse = +inf, no gradient.
- Slices that keep exactly one key: probability 1, o = v bit for bit, gradients that vanish in
  exact arithmetic stay within the dot-product rounding bound.
- -inf and very large bias values; finite bias magnitudes above 65504 are clamped alike in
  both passes (include/tri_attn.h).
- Backward shapes whose last key block has a 32-key half entirely past N without query chunks
  (five and six 128-query steps), and the chunked instances (three-step chunks, six-step
  chunks at d = 32).
- Workspace poisoning: the kernels read only workspace bytes they wrote in the same call.

Method: "TurboPairFormer: Fast and Stable Protein Folding Model Training with an Optimized
Triangle Attention Kernel" (arXiv 2610.05854), Abstract.  Bounds as in test_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from tri_synth import f32_to_bf16_bits, make_inputs

from ._util import (TOL_GRAD_RRMSE, TOL_LSE_MAXABS, TOL_O_MAXABS, TOL_O_RRMSE, f64, inputs64, mask_dev, maxabs,
                    rrmse, run_gpu, to_dev)

pytestmark = pytest.mark.gpu


def _full_oracle(inp, bias64=None):
    x = inputs64(inp)
    if bias64 is not None:
        x["bias"] = bias64
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"])
    g64 = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"])
    return o64, lse64, g64


def _check_against(out, o64, lse64, g64, label):
    """Element-wise bounds where the oracle's lse is finite; +inf lse (rows that attend to nothing)
    must be +inf on the GPU too, with exactly zero output and residual."""
    o, lse = f64(out["o"]), f64(out["lse"])
    for n in ("o", "lse", "dq", "dk", "dv", "dbias"):
        assert not torch.isnan(out[n].float()).any(), (label, n)
    inf_rows = np.isposinf(lse64)
    assert np.array_equal(np.isposinf(lse), inf_rows), label
    assert np.abs(o[inf_rows]).max(initial=0.0) == 0.0, label
    if out["res"] is not None:
        assert np.abs(f64(out["res"])[inf_rows]).max(initial=0.0) == 0.0, label
    fin = ~inf_rows
    dq64, dk64, dv64, db64 = g64
    # lse bound: the internal 1e-4 plus a few FP32 ulps of |lse| itself, which matters only for
    # rows whose bias is near the 65504 clamp (the FP32 ulp there is 2^-8)
    lse_err = np.abs(lse[fin] - lse64[fin]) - 2.0 ** -20 * np.abs(lse64[fin])
    errs = dict(o_maxabs=maxabs(o, o64), o=rrmse(o, o64), lse=float(lse_err.max(initial=0.0)),
                dq=rrmse(f64(out["dq"]), dq64), dk=rrmse(f64(out["dk"]), dk64), dv=rrmse(f64(out["dv"]), dv64),
                dbias=rrmse(f64(out["dbias"]), db64))
    print(label, {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o_maxabs"] <= TOL_O_MAXABS and errs["o"] <= TOL_O_RRMSE, (label, errs)
    assert errs["lse"] <= TOL_LSE_MAXABS, (label, errs)
    for g in ("dq", "dk", "dv", "dbias"):
        assert errs[g] <= TOL_GRAD_RRMSE, (label, g, errs)
    return errs


@pytest.mark.parametrize("B,N,H,D", [(2, 100, 2, 32), (2, 130, 1, 16)])
def test_fully_masked_slices(B, N, H, D):
    """Padded residues: every key of some slices masked.  Those slices output 0 with lse = +inf and
    get exactly zero dq, dk, dv; dbias sums only the other slices (checked against the oracle)."""
    print(f"fully masked slices B={B} N={N} H={H} D={D}", flush=True)
    inp = make_inputs(B, N, H, D, seed=300 + N + D, bias_std=2.0)
    rng = np.random.default_rng(N)
    m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
    m[:, :, 3] = 1
    dead = {0: [0, 17, N - 1], 1: list(range(40, 48))}
    for b, sl in dead.items():
        m[b, sl] = 0
    inp["key_mask"] = m
    out = run_gpu(inp)
    o64, lse64, g64 = _full_oracle(inp)
    _check_against(out, o64, lse64, g64, f"dead-slices N={N} D={D}")
    for b, sl in dead.items():
        assert torch.isposinf(out["lse"][b, sl]).all()
        for n in ("o", "res", "dq", "dk", "dv"):
            assert float(out[n][b, sl].float().abs().max()) == 0.0, n


@pytest.mark.parametrize("N,D", [(150, 32), (287, 32), (200, 16)])
def test_one_kept_key_per_slice(N, D):
    """Every slice keeps exactly one key (a different one per slice), with a wide bias.  Each
    query's probability is then exactly 1 on that key: o equals its v row bit for bit, lse is
    its score, dv is the sum of dO over the queries.  dS = dP - D is zero in exact arithmetic,
    where dP and D are the same dot product dO.v summed in two FP32 orders, so dq, dk and dbias
    are rounding noise, bounded by the standard dot-product error bounds: D's own sum of d terms
    (d eps S) and the product's sum of -D and d terms of magnitude up to 2S ((d + 1) eps 2S),
    |dP - D| <= 4 d eps S with S = sum_c |dO_c v_c| and eps = 2^-24, per query; times alpha
    max|k| for dq (one key per query), alpha max|q| summed over the queries for dk, and summed
    over the slices for dbias."""
    B, H = 1, 2
    print(f"one kept key per slice N={N} D={D}", flush=True)
    inp = make_inputs(B, N, H, D, seed=500 + N + D, bias_std=4.0)
    rng = np.random.default_rng(N + D)
    kept = rng.integers(0, N, size=N)
    m = np.zeros((B, N, N), dtype=np.uint8)
    m[0, np.arange(N), kept] = 1
    inp["key_mask"] = m
    out = run_gpu(inp)
    x = inputs64(inp)
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], m)
    _, _, dv64, _ = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], m)
    v = x["v"][0]                                             # [N(slice), H, N(key), D]
    o = f64(out["o"])[0]
    for i in range(N):
        assert np.array_equal(o[i], np.broadcast_to(v[i, :, kept[i]][:, None, :], o[i].shape)), i
    assert maxabs(f64(out["lse"]), lse64) <= TOL_LSE_MAXABS
    assert rrmse(f64(out["dv"]), dv64) <= TOL_GRAD_RRMSE
    alpha = D ** -0.5
    eps = 2.0 ** -24
    dO = x["dO"][0]                                           # [N, H, N(query), D]
    vk = np.stack([v[i, :, kept[i]] for i in range(N)])      # [N, H, D]: the kept key's v row
    dsb = 4 * D * eps * np.abs(dO * vk[:, :, None, :]).sum(-1)  # [N, H, N(query)]: |dS| bound
    kk = np.stack([x["k"][0][i, :, kept[i]] for i in range(N)])  # [N, H, D]
    dq_b = alpha * dsb.max() * np.abs(kk).max()
    dk_b = alpha * dsb.sum(-1).max() * np.abs(x["q"]).max()
    db_b = dsb.sum(0).max()
    print(f"  bounds dq {dq_b:.2e} dk {dk_b:.2e} dbias {db_b:.2e}; "
          f"max |dq| {float(out['dq'].float().abs().max()):.2e} |dk| {float(out['dk'].float().abs().max()):.2e} "
          f"|dbias| {float(out['dbias'].abs().max()):.2e}", flush=True)
    # dq and dk are rounded to bf16 (at most 2^-9 relative); dbias adds N FP32 terms
    assert float(out["dq"].float().abs().max()) <= dq_b * (1 + 2 ** -8)
    assert float(out["dk"].float().abs().max()) <= dk_b * (1 + 2 ** -8)
    assert float(out["dbias"].abs().max()) <= db_b * (1 + 2 ** -10)


@pytest.mark.parametrize("D", [16, 32])
def test_minus_inf_and_large_bias(D):
    """Queries whose first key tile (64 keys and more) carries a -inf or bf16-lowest bias, queries
    with a -inf bias on every key, and finite bias values beyond fp16's range."""
    B, N, H = 1, 200, 2
    print(f"-inf / large bias N={N} D={D}", flush=True)
    inp = make_inputs(B, N, H, D, seed=500 + D, bias_std=2.0)
    bias = inp["bias"].copy()
    ninf = f32_to_bf16_bits(np.array([-np.inf], dtype=np.float32))[0]
    lowest = np.uint16(0xFF7F)  # bf16 lowest finite value, about -3.39e38
    big = f32_to_bf16_bits(np.array([1.0e5, -1.0e5], dtype=np.float32))
    bias[0, 0, 0:10, 0:80] = ninf        # a -inf prefix longer than one 64-key tile
    bias[0, 1, 0:6, 0:130] = lowest       # the idiom bias = finfo.min on a key prefix
    bias[0, 0, 20, :] = ninf               # a query with no finite score: attends to nothing
    bias[0, 1, 50, :] = ninf
    bias[0, 0, 60:70, 5] = big[0]          # one dominant key (+1e5): the output is that key's value
    bias[0, 1, 80:90, 100:150] = big[1]    # -1e5: those keys get zero probability
    inp["bias"] = bias
    out = run_gpu(inp)
    # finite magnitudes above 65504 are clamped in both passes (the library's contract), so the
    # reference is the oracle on the clamped bias; for these values the probabilities, and so o
    # and every gradient, are also those of the unclamped bias (only lse moves, on rows 60..69)
    o64, lse64, g64 = _full_oracle(inp, _clamped_bias64(inp))
    _check_against(out, o64, lse64, g64, f"bias-extremes D={D}")
    o64_raw, _ = oracle.forward64(*(inputs64(inp)[n] for n in ("q", "k", "v", "bias")))
    assert maxabs(f64(out["o"]), o64_raw) <= TOL_O_MAXABS
    assert torch.isposinf(out["lse"][0, :, 0, 20]).all() and torch.isposinf(out["lse"][0, :, 1, 50]).all()
    assert float(out["dbias"][0, 0, 20].abs().max()) == 0.0


def _clamped_bias64(inp):
    """The bias in float64 with finite values clamped to [-65504, 65504] (65504 itself is not a
    bf16 value, so the clamped problem is handed to the oracle in float64)."""
    b64 = inputs64(inp)["bias"]
    fin = np.isfinite(b64)
    return np.where(fin, np.clip(np.where(fin, b64, 0.0), -65504.0, 65504.0), b64)


def test_bias_clamp_is_the_same_in_both_passes():
    """Two different bias values above 65504 in one row: the library computes the attention of
    the clamped bias (65504 for both), in the forward and in the backward alike."""
    B, N, H, D = 1, 96, 1, 32
    inp = make_inputs(B, N, H, D, seed=611, bias_std=1.0)
    bias = inp["bias"].copy()
    vals = f32_to_bf16_bits(np.array([7.0e4, 1.0e5, 3.0e38], dtype=np.float32))
    bias[0, 0, 10, 3], bias[0, 0, 10, 40], bias[0, 0, 11, 7] = vals
    bias[0, 0, 11, 8] = vals[1]
    inp["bias"] = bias
    out = run_gpu(inp)
    o64, lse64, g64 = _full_oracle(inp, _clamped_bias64(inp))
    _check_against(out, o64, lse64, g64, "bias-clamp")


# Backward without query chunks whose last 64-key block has its upper 32-key half entirely past
# N: N = 580 (five 128-query steps, ten key blocks) and N = 705 (six steps, twelve key blocks;
# with a mask at d = 16 this is the instance with the most registers).
@pytest.mark.parametrize("N,D,masked", [(580, 16, False), (580, 32, True), (705, 16, True), (705, 32, False),
                                        (705, 32, True), (580, 16, True)])
def test_unchunked_key_half_past_n(N, D, masked):
    B, H = 1, 1
    print(f"unchunked tail N={N} D={D} masked={masked}", flush=True)
    inp = make_inputs(B, N, H, D, seed=900 + N + D + masked, bias_std=2.0)
    rng = np.random.default_rng(N + D)
    if masked:
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, 1] = 1
        inp["key_mask"] = m
    out = run_gpu(inp)
    _sampled_check(inp, out, rng, f"N={N} D={D} masked={masked}", n_slices=3)


def _sampled_check(inp, out, rng, label, n_slices):
    x = inputs64(inp)
    B, N, H, _, D = x["q"].shape
    slices = sorted(set(rng.choice(N, size=n_slices, replace=False).tolist() + [0, N - 1]))
    o64, lse64 = oracle.forward64(x["q"], x["k"], x["v"], x["bias"], x["key_mask"], slices=slices)
    dq64, dk64, dv64, _ = oracle.backward64(x["q"], x["k"], x["v"], x["bias"], x["dO"], x["key_mask"], slices=slices)
    sl = (slice(None), slices)
    o = f64(out["o"])[sl]
    errs = dict(o_maxabs=maxabs(o, o64[sl]), o=rrmse(o, o64[sl]), lse=maxabs(f64(out["lse"])[sl], lse64[sl]))
    for g, ref in (("dq", dq64), ("dk", dk64), ("dv", dv64)):
        errs[g] = rrmse(f64(out[g])[sl], ref[sl])
        # per slice, so that one wrong key block cannot hide in the RMS over slices
        for i in slices:
            assert rrmse(f64(out[g])[:, i], ref[:, i]) <= TOL_GRAD_RRMSE, (label, g, i)
    js = [0, N - 1, 127, 128] + rng.integers(0, N, 3).tolist()
    rows = [(0, int(rng.integers(0, H)), int(j)) for j in js if j < N]
    db64 = oracle.dbias_rows64(x["q"], x["k"], x["v"], x["bias"], x["dO"], rows, x["key_mask"])
    db = f64(out["dbias"])
    errs["dbias"] = rrmse(np.stack([db[b, h, j] for b, h, j in rows]), db64)
    print(label, {k: f"{v:.3e}" for k, v in errs.items()}, flush=True)
    assert errs["o_maxabs"] <= TOL_O_MAXABS and errs["o"] <= TOL_O_RRMSE and errs["lse"] <= TOL_LSE_MAXABS, errs
    for g in ("dq", "dk", "dv", "dbias"):
        assert errs[g] <= TOL_GRAD_RRMSE, (label, g, errs)


# Chunked backward instances: N = 800 runs chunks of 4 + 3 steps (the three-step chunked instance),
# N = 2048 at d = 32 runs 6 + 5 + 5 (six-step chunks at d = 32).
@pytest.mark.parametrize("N,D", [(800, 16), (800, 32), (2048, 32)])
def test_chunked_instances(N, D):
    import triangle_attention_amd as ta
    B, H = 1, 1
    print(f"chunked instance N={N} D={D}", flush=True)
    assert ta.tri_attn_bwd_workspace_bytes(B, N, H, D) > 0
    inp = make_inputs(B, N, H, D, seed=1700 + N + D, bias_std=2.0)
    out = run_gpu(inp)
    _sampled_check(inp, out, np.random.default_rng(N * D), f"chunked N={N} D={D}", n_slices=2)


@pytest.mark.parametrize("B,N,H,D,masked", [(2, 200, 2, 32, True), (1, 130, 3, 16, False), (1, 800, 1, 16, True)])
def test_workspace_poison(B, N, H, D, masked):
    """Results with a workspace filled with 0xFF bytes (NaN patterns) before every call equal, bit
    for bit, those with a zeroed workspace: no kernel reads workspace it did not write."""
    import triangle_attention_amd as ta
    print(f"workspace poison B={B} N={N} H={H} D={D} masked={masked}", flush=True)
    inp = make_inputs(B, N, H, D, seed=2200 + N, bias_std=2.0)
    if masked:
        rng = np.random.default_rng(N)
        m = (rng.random((B, N, N)) > 0.3).astype(np.uint8)
        m[:, :, 0] = 1
        inp["key_mask"] = m
    q, k, v, bias, dO = (to_dev(inp[n]) for n in ("q", "k", "v", "bias", "dO"))
    msk = mask_dev(inp["key_mask"])
    fws = torch.empty(ta.tri_attn_fwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device="cuda")
    bws = torch.empty(ta.tri_attn_bwd_workspace_bytes(B, N, H, D), dtype=torch.uint8, device="cuda")

    def call(fill):
        o, res, dq, dk, dv = (torch.empty_like(q) for _ in range(5))
        lse = torch.empty((B, N, H, N), dtype=torch.float32, device="cuda")
        dbias = torch.empty((B, H, N, N), dtype=torch.float32, device="cuda")
        fws.fill_(fill)
        assert ta.tri_attn_fwd(B, N, H, D, q, k, v, bias, msk, o, lse, res, fws, fws.numel()) == 0
        bws.fill_(fill)
        assert ta.tri_attn_bwd(B, N, H, D, q, k, v, bias, msk, o, lse, res, dO, dq, dk, dv, dbias, bws,
                               bws.numel()) == 0
        torch.cuda.synchronize()
        return dict(o=o, lse=lse, res=res, dq=dq, dk=dk, dv=dv, dbias=dbias)

    clean = call(0)
    dirty = call(0xFF)
    for n in clean:
        a, b = clean[n], dirty[n]
        bits = (lambda t: t.view(torch.int32)) if a.dtype == torch.float32 else (lambda t: t.view(torch.int16))
        assert torch.equal(bits(a), bits(b)), n
