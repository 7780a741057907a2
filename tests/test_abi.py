"""The C ABI of libtriattn.so: exported symbols and synchronous argument validation.

These tests run without a GPU.  Every call below is built to fail validation
(the library validates every argument before touching the HIP runtime), so the fake
integer pointers are never dereferenced and nothing is launched.
"""
import os
import re

import pytest

import triangle_attention_amd as ta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUCCESS, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, LAUNCH, SCRATCH_LIMIT = range(7)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ta.LIB_PATH):
        ta.build()
    return ta.load_library()


def _declared_functions():
    names = set()
    for h in ("tri_attn.h", "tri_mul.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"\b(tri_(?:attn|mul)_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"tri_attn_fwd", "tri_attn_bwd", "tri_attn_fwd_workspace_bytes", "tri_attn_bwd_workspace_bytes",
            "tri_attn_status_string", "tri_attn_fwd_ex", "tri_attn_bwd_ex", "tri_mul_fwd", "tri_mul_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in [(SUCCESS, "SUCCESS"), (INVALID, "INVALID_VALUE"), (UNSUPPORTED, "UNSUPPORTED"),
                       (MISALIGNED, "MISALIGNED"), (WORKSPACE, "WORKSPACE"), (LAUNCH, "LAUNCH"),
                       (SCRATCH_LIMIT, "SCRATCH_LIMIT")]:
        assert ta.tri_attn_status_string(code).endswith(name)
    assert "UNKNOWN" in ta.tri_attn_status_string(1234)


def test_workspace_sizes(lib):
    for B, N, H, D in [(1, 1, 1, 16), (1, 64, 4, 16), (2, 100, 3, 32), (1, 768, 4, 32)]:
        f = ta.tri_attn_fwd_workspace_bytes(B, N, H, D)
        b = ta.tri_attn_bwd_workspace_bytes(B, N, H, D)
        assert f > 0 and b > 0 and f % 256 == 0 and b % 256 == 0
        # the backward holds the pair bias twice (fp16 column blocks, FP32 tiles), the row
        # statistics (16 bytes per query) and one FP32 pair-bias partial per slice group
        assert b >= B * H * N * N * (2 + 4 + 4) + B * N * H * N * 16
    for bad in [(0, 8, 1, 16), (1, 0, 1, 16), (1, 8, 0, 16), (1, 8, 1, 64), (1, 4097, 1, 16)]:
        assert ta.tri_attn_fwd_workspace_bytes(*bad) == 0
        assert ta.tri_attn_bwd_workspace_bytes(*bad) == 0
    # the forward alone reaches TRI_ATTN_FWD_MAX_N; the backward stops at TRI_ATTN_MAX_N
    assert ta.TRI_ATTN_MAX_N == 2048 and ta.TRI_ATTN_FWD_MAX_N == 4096
    assert ta.tri_attn_fwd_workspace_bytes(1, 2049, 1, 16) > 0
    assert ta.tri_attn_fwd_workspace_bytes(1, 4096, 4, 32) > 0
    assert ta.tri_attn_bwd_workspace_bytes(1, 2049, 1, 16) == 0
    assert ta.tri_attn_bwd_workspace_bytes(1, 2048, 1, 16) > 0
    # past six 128-query steps the backward runs in query chunks and adds FP32 dK / dV partials
    # per chunk: two chunks at N = 769, three at N = 2048
    for N, nqc in [(769, 2), (1536, 2), (1537, 3), (2048, 3)]:
        b = ta.tri_attn_bwd_workspace_bytes(1, N, 2, 32)
        assert b >= 2 * N * N * (2 + 4 + 4) + 2 * nqc * N * 2 * N * 32 * 4, N
    assert ta.tri_attn_bwd_workspace_bytes(1, 768, 4, 32) > ta.tri_attn_bwd_workspace_bytes(1, 384, 4, 32)


# fake, well-separated, 16-byte-aligned device addresses; never dereferenced
def _ptrs(n, base=1 << 40, step=1 << 32):
    return [base + i * step for i in range(n)]


def _fwd(shape=(1, 64, 4, 16), ptrs=None, mask=None, res=True, ws=None, wsb=None):
    p = ptrs or _ptrs(8)
    q, k, v, bias, o, lse, r, w = p
    wsb = ta.tri_attn_fwd_workspace_bytes(*shape) if wsb is None else wsb
    return ta.tri_attn_fwd(*shape, q, k, v, bias, mask, o, lse, r if res else None, w if ws is None else ws, wsb, 0)


def _bwd(shape=(1, 64, 4, 16), ptrs=None, mask=None, ws=None, wsb=None):
    p = ptrs or _ptrs(14)
    q, k, v, bias, o, lse, r, dO, dq, dk, dv, db, w = p[:13]
    wsb = ta.tri_attn_bwd_workspace_bytes(*shape) if wsb is None else wsb
    return ta.tri_attn_bwd(*shape, q, k, v, bias, mask, o, lse, r, dO, dq, dk, dv, db, w if ws is None else ws, wsb, 0)


def test_fwd_validation(lib):
    assert _fwd(shape=(0, 64, 4, 16)) == INVALID
    assert _fwd(shape=(1, 0, 4, 16)) == INVALID
    assert _fwd(shape=(1, 64, 0, 16)) == INVALID
    assert _fwd(shape=(1, 64, 4, 64)) == UNSUPPORTED
    assert _fwd(shape=(1, 64, 4, 8)) == UNSUPPORTED
    assert _fwd(shape=(1, 4097, 4, 16)) == UNSUPPORTED
    assert _fwd(shape=(1, 2049, 4, 16), wsb=16) == WORKSPACE  # a forward-only crop past the backward's limit
    for idx in range(6):  # q, k, v, bias, o, lse are required
        p = _ptrs(8)
        p[idx] = 0
        assert _fwd(ptrs=p) == INVALID, idx
    p = _ptrs(8)
    p[4] = p[0] + 64  # o overlaps q
    assert _fwd(ptrs=p) == INVALID
    p = _ptrs(8)
    p[7] = p[1]  # workspace overlaps k
    assert _fwd(ptrs=p) == INVALID
    for idx in (0, 1, 2, 3, 4, 5, 6, 7):
        p = _ptrs(8)
        p[idx] += 8
        assert _fwd(ptrs=p) == MISALIGNED, idx
    assert _fwd(ws=0) == WORKSPACE
    assert _fwd(wsb=ta.tri_attn_fwd_workspace_bytes(1, 64, 4, 16) - 256) == WORKSPACE
    # the mask may have any alignment; with everything else valid except the workspace size
    assert _fwd(mask=(1 << 40) + 13 * (1 << 32) + 3, wsb=16) == WORKSPACE


def test_bwd_validation(lib):
    assert _bwd(shape=(1, 64, 4, 48)) == UNSUPPORTED
    assert _bwd(shape=(1, 2049, 4, 16), wsb=1 << 40) == UNSUPPORTED
    # a chunked backward (N past 768) checks its larger workspace
    assert _bwd(shape=(1, 769, 4, 16), wsb=ta.tri_attn_bwd_workspace_bytes(1, 768, 4, 16)) == WORKSPACE
    assert _bwd(shape=(2, 0, 4, 16)) == INVALID
    for idx in (0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 11):  # every tensor except the residual is required
        p = _ptrs(14)
        p[idx] = 0
        assert _bwd(ptrs=p) == INVALID, idx
    p = _ptrs(14)
    p[11] = p[3]  # dbias aliases bias
    assert _bwd(ptrs=p) == INVALID
    p = _ptrs(14)
    p[9] = p[8] + 32  # dk overlaps dq
    assert _bwd(ptrs=p) == INVALID
    p = _ptrs(14)
    p[6] = 0  # no residual: uncompensated correction, still only the workspace is wrong
    assert _bwd(ptrs=p, wsb=64) == WORKSPACE
    p = _ptrs(14)
    p[10] += 4
    assert _bwd(ptrs=p) == MISALIGNED
    assert _bwd(wsb=ta.tri_attn_bwd_workspace_bytes(1, 64, 4, 16) - 1) == WORKSPACE
    assert _bwd(ws=0) == WORKSPACE


def _fwd_ex(layout, shape=(1, 64, 4, 16), stages=7, wsb=None):
    q, k, v, bias, o, lse, r, w = _ptrs(8)
    wsb = ta.tri_attn_fwd_workspace_bytes(*shape) if wsb is None else wsb
    return ta.tri_attn_fwd_ex(stages, layout, *shape, q, k, v, bias, None, o, lse, r, w, wsb, 0)


def _bwd_ex(layout, shape=(1, 64, 4, 16), stages=7, wsb=None):
    q, k, v, bias, o, lse, r, dO, dq, dk, dv, db, w = _ptrs(13)
    wsb = ta.tri_attn_bwd_workspace_bytes(*shape) if wsb is None else wsb
    return ta.tri_attn_bwd_ex(stages, layout, *shape, q, k, v, bias, None, o, lse, r, dO, dq, dk, dv, db, w, wsb, 0)


def test_layout_validation(lib):
    assert ta.LAYOUTS == {"slice_head": 0, "pair_start": 1, "pair_end": 2}
    for f in (_fwd_ex, _bwd_ex):
        for bad in (-1, 3, 1 << 20):
            assert f(bad) == INVALID, (f, bad)
        assert f(0, stages=8) == INVALID
        # every known layout passes validation up to the (too small) workspace
        for layout in ta.LAYOUTS.values():
            assert f(layout, wsb=16) == WORKSPACE, (f, layout)
        # the ending-node layout at N=768: a slice's rows span N*H*D*2 bytes each, 32-bit offsets
        # reach H=32 (768 padded rows x 768*32*32*2 bytes < 2^31) but not H=64
        assert f(2, shape=(1, 768, 32, 32), wsb=16) == WORKSPACE
        assert f(2, shape=(1, 768, 64, 32)) == UNSUPPORTED
        assert f(1, shape=(1, 768, 64, 32), wsb=16) == WORKSPACE  # pair_start rows are H*D apart
        assert f(0, shape=(1, 768, 64, 32), wsb=16) == WORKSPACE


def test_tri_mul_validation(lib):
    a, b, x, dx, da, db = _ptrs(6)
    ws = _ptrs(1, base=1 << 46)[0]
    fwd = lambda d, B, N, C, lay=0, **k: ta.tri_mul_fwd(d, lay, B, N, C, k.get("a", a), k.get("b", b),
                                                          k.get("x", x), k.get("ws"), k.get("wsb", 0), stream=0)
    bwd = lambda d, B, N, C, lay=0, **k: ta.tri_mul_bwd(d, lay, B, N, C, k.get("a", a), k.get("b", b),
                                                          k.get("dx", dx), k.get("da", da), k.get("db", db),
                                                          k.get("ws"), k.get("wsb", 0), stream=0)
    assert ta.TRI_MUL_LAYOUTS == {"channels_last": 0, "channels_first": 1}
    for f in (fwd, bwd):
        assert f(2, 1, 64, 32) == INVALID          # unknown direction
        assert f(-1, 1, 64, 32) == INVALID
        assert f(0, 1, 64, 32, lay=2) == INVALID   # unknown layout
        assert f(0, 0, 64, 32) == INVALID
        assert f(0, 1, 0, 32) == INVALID
        assert f(1, 1, 64, 0) == INVALID
        assert f(0, 1, 64, 12) == UNSUPPORTED      # channels last: C a multiple of 8
        assert f(0, 1, 60, 16, lay=1) == UNSUPPORTED  # channels first: N a multiple of 8
        assert f(0, 1, 64, 1032) == UNSUPPORTED
        assert f(1, 1, 1025, 32) == UNSUPPORTED
        assert f(0, 1, 64, 32, a=0) == INVALID
        assert f(0, 1, 64, 32, a=a + 8) == MISALIGNED
        assert f(0, 1, 64, 12, lay=1, a=a + 8) == MISALIGNED  # channels first accepts any C
    # channels last: the workspace holds five channels-first tensors; too small is an error,
    # overlapping a tensor is invalid, and N not a multiple of 8 needs none
    need = ta.tri_mul_workspace_bytes(0, 1, 64, 32)
    assert need >= 5 * 64 * 64 * 32 * 2 and need % 256 == 0
    assert ta.tri_mul_workspace_bytes(1, 1, 64, 32) == 0
    assert ta.tri_mul_workspace_bytes(0, 1, 60, 32) == 0
    assert ta.tri_mul_workspace_bytes(0, 1, 64, 12) == 0
    for f in (fwd, bwd):
        assert f(0, 1, 64, 32, ws=ws, wsb=need - 256) == WORKSPACE
        assert f(0, 1, 64, 32, ws=a, wsb=need) == INVALID
        assert f(0, 1, 64, 32, ws=ws + 8, wsb=need) == MISALIGNED
    assert fwd(0, 1, 64, 32, x=a + 64) == INVALID  # output overlaps an input
    assert bwd(0, 1, 64, 32, db=da + 1024) == INVALID
    assert bwd(1, 1, 64, 32, da=dx) == INVALID
    assert bwd(0, 1, 64, 32, dx=0) == INVALID


def test_tri_mul_gate_validation(lib):
    g, p, a, da, dg, dp = _ptrs(6)
    fwd = lambda lay, B, N, C, **k: ta.tri_mul_gate_fwd(lay, B, N, C, k.get("g", g), k.get("p", p), k.get("m"),
                                                          k.get("a", a), stream=0)
    bwd = lambda lay, B, N, C, **k: ta.tri_mul_gate_bwd(lay, B, N, C, k.get("g", g), k.get("p", p), k.get("m"),
                                                          k.get("da", da), k.get("dg", dg), k.get("dp", dp), stream=0)
    for f in (fwd, bwd):
        assert f(2, 1, 64, 32) == INVALID
        assert f(0, 0, 64, 32) == INVALID
        assert f(0, 1, 64, 12) == UNSUPPORTED     # C a multiple of 8
        assert f(1, 1, 60, 16) == UNSUPPORTED     # channels first: N a multiple of 8
        assert f(0, 1, 1025, 16) == UNSUPPORTED
        assert f(0, 1, 64, 32, g=0) == INVALID
        assert f(0, 1, 64, 32, p=p + 8) == MISALIGNED
    assert fwd(0, 1, 64, 32, a=g + 64) == INVALID
    assert bwd(0, 1, 64, 32, dg=dp) == INVALID
    assert bwd(0, 1, 64, 32, dp=da + 32) == INVALID


def test_noalloc_forward_validation(lib):
    """The allocation-free forward rejects, before any HIP call, what tri_attn_fwd rejects, and
    shapes whose prepared bias exceeds the library's scratch array."""
    assert ta.tri_attn_noalloc_scratch_bytes() == 64 << 20
    P = 1 << 20  # fake, 16-byte aligned; never dereferenced
    args = lambda B, N, H, D, q=P: (B, N, H, D, q, P, P, P, None, P, P, P, 0)  # noqa: E731
    assert ta.tri_attn_fwd_noalloc(*args(0, 8, 1, 16)) == INVALID
    assert ta.tri_attn_fwd_noalloc(*args(1, 8, 1, 64)) == UNSUPPORTED
    assert ta.tri_attn_fwd_noalloc(*args(1, 8, 1, 16, q=0)) == INVALID
    # N = 768: 2359296 bytes of prepared bias per (batch, head); 28 fit in 64 MiB, 29 do not
    assert ta.tri_attn_fwd_workspace_bytes(1, 768, 28, 32) <= 64 << 20 < ta.tri_attn_fwd_workspace_bytes(1, 768, 29, 32)
    assert ta.tri_attn_fwd_noalloc(*args(1, 768, 29, 32)) == SCRATCH_LIMIT
    assert ta.tri_attn_fwd_workspace_bytes(2, 1024, 8, 16) == 64 << 20  # exactly full: accepted
    assert ta.tri_attn_fwd_noalloc(*args(2, 1024, 9, 16)) == SCRATCH_LIMIT
