"""Python binding of libtriattn.so: gfx950 triangle attention (starting node), forward + backward.

The C entry points of ``include/tri_attn.h`` are exposed under the same names; the
binding only marshals arguments (tensor pointers, sizes, the current HIP stream).  Every
step of the computation runs in the HIP library.  If the library is not built, every
call raises: there is no fallback implementation.

Method: "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
Optimized Triangle Attention Kernel" (arXiv 2610.05854), Abstract.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIB_PATH, build  # noqa: F401

__all__ = [
    "TriAttnError", "load_library", "tri_attn_status_string", "tri_attn_fwd_workspace_bytes",
    "tri_attn_bwd_workspace_bytes", "tri_attn_fwd", "tri_attn_bwd", "tri_attn_fwd_stages", "tri_attn_bwd_stages",
    "tri_attn_fwd_ex", "tri_attn_bwd_ex", "tri_attn_fwd_noalloc", "tri_attn_noalloc_scratch_bytes",
    "triangle_attention", "TRI_ATTN_MAX_N", "TRI_ATTN_FWD_MAX_N", "LAYOUTS",
    "tri_mul_fwd", "tri_mul_bwd", "tri_mul_workspace_bytes", "tri_mul_gate_fwd", "tri_mul_gate_bwd",
    "triangle_multiplication", "gated_operand", "TRI_MUL_DIRECTIONS", "TRI_MUL_LAYOUTS",
    "TRI_MUL_MAX_N",
]

TRI_ATTN_MAX_N = 2048       # backward (and a forward that feeds it)
TRI_ATTN_FWD_MAX_N = 4096   # forward alone
TRI_MUL_MAX_N = 1024
TRI_MUL_DIRECTIONS = {"outgoing": 0, "incoming": 1}
TRI_MUL_LAYOUTS = {"channels_last": 0, "channels_first": 1}
_lib = None


class TriAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {tri_attn_status_string(status)} ({status})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libtriattn.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.tri_attn_status_string.argtypes = [ctypes.c_int]
    lib.tri_attn_status_string.restype = ctypes.c_char_p
    for name in ("tri_attn_fwd_workspace_bytes", "tri_attn_bwd_workspace_bytes"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, i64]
        f.restype = sz
    lib.tri_attn_fwd.argtypes = [i64, i64, i64, i64] + [vp] * 8 + [vp, sz, vp]
    lib.tri_attn_fwd.restype = ctypes.c_int
    lib.tri_attn_bwd.argtypes = [i64, i64, i64, i64] + [vp] * 13 + [vp, sz, vp]
    lib.tri_attn_bwd.restype = ctypes.c_int
    lib.tri_attn_fwd_stages.argtypes = [ctypes.c_uint] + lib.tri_attn_fwd.argtypes
    lib.tri_attn_fwd_stages.restype = ctypes.c_int
    lib.tri_attn_bwd_stages.argtypes = [ctypes.c_uint] + lib.tri_attn_bwd.argtypes
    lib.tri_attn_bwd_stages.restype = ctypes.c_int
    lib.tri_attn_fwd_ex.argtypes = [ctypes.c_uint, ctypes.c_int] + lib.tri_attn_fwd.argtypes
    lib.tri_attn_fwd_ex.restype = ctypes.c_int
    lib.tri_attn_bwd_ex.argtypes = [ctypes.c_uint, ctypes.c_int] + lib.tri_attn_bwd.argtypes
    lib.tri_attn_bwd_ex.restype = ctypes.c_int
    lib.tri_attn_noalloc_scratch_bytes.argtypes = []
    lib.tri_attn_noalloc_scratch_bytes.restype = sz
    lib.tri_attn_fwd_noalloc.argtypes = [i64, i64, i64, i64] + [vp] * 8 + [vp]
    lib.tri_attn_fwd_noalloc.restype = ctypes.c_int
    lib.tri_mul_gate_fwd.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.tri_mul_gate_fwd.restype = ctypes.c_int
    lib.tri_mul_gate_bwd.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.tri_mul_gate_bwd.restype = ctypes.c_int
    lib.tri_mul_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64]
    lib.tri_mul_workspace_bytes.restype = sz
    lib.tri_mul_fwd.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.tri_mul_fwd.restype = ctypes.c_int
    lib.tri_mul_bwd.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tri_mul_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def tri_attn_status_string(status: int) -> str:
    return load_library().tri_attn_status_string(int(status)).decode()


def tri_attn_fwd_workspace_bytes(B: int, N: int, H: int, D: int) -> int:
    return int(load_library().tri_attn_fwd_workspace_bytes(B, N, H, D))


def tri_attn_bwd_workspace_bytes(B: int, N: int, H: int, D: int) -> int:
    return int(load_library().tri_attn_bwd_workspace_bytes(B, N, H, D))


def tri_attn_fwd(B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, workspace, workspace_bytes,
                 stream=None) -> int:
    """Marshal to the C entry point; returns the status code (0 = success)."""
    return int(load_library().tri_attn_fwd(B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(key_mask),
                                           _ptr(o), _ptr(lse), _ptr(residual), _ptr(workspace),
                                           int(workspace_bytes), _stream(stream)))


def tri_attn_bwd(B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, dO, dq, dk, dv, dbias, workspace,
                 workspace_bytes, stream=None) -> int:
    """Marshal to the C entry point; returns the status code (0 = success)."""
    return int(load_library().tri_attn_bwd(B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(key_mask),
                                           _ptr(o), _ptr(lse), _ptr(residual), _ptr(dO), _ptr(dq), _ptr(dk),
                                           _ptr(dv), _ptr(dbias), _ptr(workspace), int(workspace_bytes),
                                           _stream(stream)))


def tri_attn_noalloc_scratch_bytes() -> int:
    return int(load_library().tri_attn_noalloc_scratch_bytes())


def tri_attn_fwd_noalloc(B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, stream=None) -> int:
    """Marshal to the allocation-free forward (scratch inside the library); returns the status code."""
    return int(load_library().tri_attn_fwd_noalloc(B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                                   _ptr(key_mask), _ptr(o), _ptr(lse), _ptr(residual),
                                                   _stream(stream)))


STAGE_PREP, STAGE_MAIN, STAGE_FINAL, STAGE_ALL = 1, 2, 4, 7


def tri_attn_fwd_stages(stages, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, workspace, workspace_bytes,
                        stream=None) -> int:
    return int(load_library().tri_attn_fwd_stages(stages, B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                                  _ptr(key_mask), _ptr(o), _ptr(lse), _ptr(residual),
                                                  _ptr(workspace), int(workspace_bytes), _stream(stream)))


def tri_attn_bwd_stages(stages, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, dO, dq, dk, dv, dbias,
                        workspace, workspace_bytes, stream=None) -> int:
    return int(load_library().tri_attn_bwd_stages(stages, B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                                  _ptr(key_mask), _ptr(o), _ptr(lse), _ptr(residual), _ptr(dO),
                                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace),
                                                  int(workspace_bytes), _stream(stream)))


# token-tensor layouts of tri_attn_fwd_ex / tri_attn_bwd_ex (tri_attn_layout)
LAYOUTS = {"slice_head": 0, "pair_start": 1, "pair_end": 2}


def tri_attn_fwd_ex(stages, layout, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, workspace,
                    workspace_bytes, stream=None) -> int:
    return int(load_library().tri_attn_fwd_ex(stages, layout, B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                              _ptr(key_mask), _ptr(o), _ptr(lse), _ptr(residual),
                                              _ptr(workspace), int(workspace_bytes), _stream(stream)))


def tri_attn_bwd_ex(stages, layout, B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, dO, dq, dk, dv, dbias,
                    workspace, workspace_bytes, stream=None) -> int:
    return int(load_library().tri_attn_bwd_ex(stages, layout, B, N, H, D, _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                              _ptr(key_mask), _ptr(o), _ptr(lse), _ptr(residual), _ptr(dO),
                                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace),
                                              int(workspace_bytes), _stream(stream)))


def tri_mul_gate_fwd(layout, B, N, C, g, p, mask, a, stream=None) -> int:
    """Marshal to the C entry point (include/tri_mul.h); returns the status code."""
    return int(load_library().tri_mul_gate_fwd(layout, B, N, C, _ptr(g), _ptr(p), _ptr(mask), _ptr(a),
                                               _stream(stream)))


def tri_mul_gate_bwd(layout, B, N, C, g, p, mask, da, dg, dp, stream=None) -> int:
    """Marshal to the C entry point (include/tri_mul.h); returns the status code."""
    return int(load_library().tri_mul_gate_bwd(layout, B, N, C, _ptr(g), _ptr(p), _ptr(mask), _ptr(da), _ptr(dg),
                                               _ptr(dp), _stream(stream)))


def tri_mul_workspace_bytes(layout, B, N, C) -> int:
    return int(load_library().tri_mul_workspace_bytes(layout, B, N, C))


def tri_mul_fwd(direction, layout, B, N, C, a, b, x, workspace=None, workspace_bytes=0, stream=None) -> int:
    """Marshal to the C entry point (include/tri_mul.h); returns the status code."""
    return int(load_library().tri_mul_fwd(direction, layout, B, N, C, _ptr(a), _ptr(b), _ptr(x), _ptr(workspace),
                                          int(workspace_bytes), _stream(stream)))


def tri_mul_bwd(direction, layout, B, N, C, a, b, dx, da, db, workspace=None, workspace_bytes=0,
                stream=None) -> int:
    """Marshal to the C entry point (include/tri_mul.h); returns the status code."""
    return int(load_library().tri_mul_bwd(direction, layout, B, N, C, _ptr(a), _ptr(b), _ptr(dx), _ptr(da),
                                          _ptr(db), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def _check(status: int, where: str):
    if status != 0:
        raise TriAttnError(status, where)


def _shape(q, layout="slice_head"):
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if not isinstance(q, torch.Tensor) or q.dim() != 5:
        raise ValueError("q must be a 5-dimensional tensor")
    if layout == "slice_head":
        B, N, H, N2, D = q.shape
    else:
        B, N, N2, H, D = q.shape
    if N2 != N:
        raise ValueError("q must have equal slice and token extents")
    return B, N, H, D


def _require(t, name, shape, dtypes):
    """Raise ValueError unless t is a contiguous tensor of one of `dtypes` with exactly `shape`.
    The C entry points read raw memory in the documented layout, so a view with other strides or
    another dtype would be misread, not rejected."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (strides {t.stride()}); call .contiguous() first")


def _one_gpu(named):
    """Raise ValueError unless every tensor of `named` ((name, tensor) pairs, None skipped) is on
    the GPU of the first one."""
    named = [(n, t) for n, t in named if t is not None]
    dev = named[0][1].device
    for n, t in named:
        if not t.is_cuda:
            raise ValueError(f"{n} must be on a GPU, got device {t.device}")
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, {named[0][0]} on {dev}: all tensors must be on one GPU")


_BF16 = (torch.bfloat16,)
_MASK = (torch.uint8, torch.bool)


def _check_inputs(q, k, v, bias, key_mask, layout, more=()):
    B, N, H, D = _shape(q, layout)
    if D not in (16, 32):
        raise ValueError(f"head dimension must be 16 or 32, got {D}")
    tok = tuple(q.shape)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _require(t, n, tok, _BF16)
    _require(bias, "bias", (B, H, N, N), _BF16)
    if key_mask is not None:
        _require(key_mask, "key_mask", (B, N, N), _MASK)
    for n, t, shape, dtypes in more:
        if t is not None:
            _require(t, n, shape, dtypes)
    _one_gpu([("q", q), ("k", k), ("v", v), ("bias", bias), ("key_mask", key_mask)] + [(m[0], m[1]) for m in more])
    return B, N, H, D


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def forward(q, k, v, bias, key_mask=None, residual_compensation=True, layout="slice_head"):
    """Returns (o, lse, residual-or-None).  q, k, v: contiguous bf16 laid out as `layout` names
    (see triangle_attention); bias: contiguous bf16 [B, H, N, N]; key_mask: contiguous uint8 (or
    bool) [B, N, N] or None; all on one GPU.  Anything else raises ValueError before any call."""
    B, N, H, D = _check_inputs(q, k, v, bias, key_mask, layout)
    o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty((B, N, H, N), dtype=torch.float32, device=q.device)
    res = torch.empty(q.shape, dtype=q.dtype, device=q.device) if residual_compensation else None
    nws = tri_attn_fwd_workspace_bytes(B, N, H, D)
    ws = _workspace(nws, q.device)
    _check(tri_attn_fwd_ex(STAGE_ALL, LAYOUTS[layout], B, N, H, D, q, k, v, bias, key_mask, o, lse, res, ws,
                           ws.numel()), "tri_attn_fwd_ex")
    return o, lse, res


def backward(q, k, v, bias, key_mask, o, lse, residual, dO, layout="slice_head"):
    """Returns (dq, dk, dv, dbias) with dbias in float32.  The inputs follow forward(); o,
    residual (or None) and dO have q's shape and dtype, lse is float32 [B, N, H, N]."""
    B, N, H, D = _shape(q, layout)
    dev, tok = q.device, tuple(q.shape)
    _check_inputs(q, k, v, bias, key_mask, layout,
                  more=(("o", o, tok, _BF16), ("lse", lse, (B, N, H, N), (torch.float32,)),
                        ("residual", residual, tok, _BF16), ("dO", dO, tok, _BF16)))
    dq, dk, dv = (torch.empty(tok, dtype=q.dtype, device=dev) for _ in range(3))
    dbias = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    nws = tri_attn_bwd_workspace_bytes(B, N, H, D)
    ws = _workspace(nws, dev)
    _check(tri_attn_bwd_ex(STAGE_ALL, LAYOUTS[layout], B, N, H, D, q, k, v, bias, key_mask, o, lse, residual, dO,
                           dq, dk, dv, dbias, ws, ws.numel()), "tri_attn_bwd_ex")
    return dq, dk, dv, dbias


class _TriAttnFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, bias, key_mask, residual_compensation, layout):
        o, lse, res = forward(q, k, v, bias, key_mask, residual_compensation, layout)
        ctx.save_for_backward(q, k, v, bias, o, lse, res, key_mask)
        ctx.layout = layout
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, bias, o, lse, res, key_mask = ctx.saved_tensors
        dq, dk, dv, dbias = backward(q, k, v, bias, key_mask, o, lse, res, dO.contiguous(), ctx.layout)
        return dq, dk, dv, dbias.to(bias.dtype), None, None, None


def triangle_attention(q, k, v, bias, key_mask=None, residual_compensation=True, layout="slice_head"):
    """Triangle attention, differentiable in q, k, v and the shared bias.

    layout "slice_head": q, k, v bf16 [B, N, H, N, D], index [b, i, h, j, c] (starting node).
    layout "pair_start": q, k, v bf16 [B, N, N, H, D] (the pair layout), index [b, i, j, h, c]:
        attention along the second pair index (starting node).
    layout "pair_end": the same pair layout, index [b, j, i, h, c]: attention along the first
        pair index for each fixed second index (ending node), with no transposed copy.
    bias: bf16 [B, H, N, N] indexed [b, h, query, key] and key_mask: uint8 [B, N, N] indexed
    [b, slice, key], in the orientation of the attended axis, or None.
    """
    return _TriAttnFn.apply(q, k, v, bias, key_mask, residual_compensation, layout)


def _mul_shape(a, b, direction, layout):
    if direction not in TRI_MUL_DIRECTIONS:
        raise ValueError(f"direction must be one of {sorted(TRI_MUL_DIRECTIONS)}")
    if layout not in TRI_MUL_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(TRI_MUL_LAYOUTS)}")
    if not isinstance(a, torch.Tensor) or a.dim() != 4:
        raise ValueError("a must be a 4-dimensional tensor")
    if layout == "channels_last":
        B, N, N2, C = a.shape
    else:
        B, C, N, N2 = a.shape
    if N2 != N:
        raise ValueError("the two pair indices must have equal extents")
    _require(a, "a", tuple(a.shape), _BF16)
    _require(b, "b", tuple(a.shape), _BF16)
    _one_gpu([("a", a), ("b", b)])
    return B, N, C


def _mul_workspace(layout, B, N, C, device):
    n = tri_mul_workspace_bytes(TRI_MUL_LAYOUTS[layout], B, N, C)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


class _TriMulFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a, b, direction, layout):
        B, N, C = _mul_shape(a, b, direction, layout)
        x = torch.empty(a.shape, dtype=a.dtype, device=a.device)
        ws = _mul_workspace(layout, B, N, C, a.device)
        _check(tri_mul_fwd(TRI_MUL_DIRECTIONS[direction], TRI_MUL_LAYOUTS[layout], B, N, C, a, b, x, ws,
                           0 if ws is None else ws.numel()), "tri_mul_fwd")
        ctx.save_for_backward(a, b)
        ctx.direction, ctx.layout, ctx.shape = direction, layout, (B, N, C)
        return x

    @staticmethod
    def backward(ctx, dx):
        a, b = ctx.saved_tensors
        B, N, C = ctx.shape
        dx = dx.contiguous()
        _require(dx, "dx", tuple(a.shape), _BF16)
        _one_gpu([("a", a), ("dx", dx)])
        da, db = (torch.empty(a.shape, dtype=a.dtype, device=a.device) for _ in range(2))
        ws = _mul_workspace(ctx.layout, B, N, C, a.device)
        _check(tri_mul_bwd(TRI_MUL_DIRECTIONS[ctx.direction], TRI_MUL_LAYOUTS[ctx.layout], B, N, C, a, b,
                           dx, da, db, ws, 0 if ws is None else ws.numel()), "tri_mul_bwd")
        return da, db, None, None


def triangle_multiplication(a, b, direction="outgoing", layout="channels_last"):
    """Cubic core of the triangle multiplicative update, differentiable in a and b.

    outgoing: x[b,i,j,c] = sum_k a[b,i,k,c] b[b,j,k,c];  incoming: x[b,i,j,c] = sum_k a[b,k,i,c] b[b,k,j,c].
    layout "channels_last": a, b contiguous bf16 [B, N, N, C] (C a multiple of 8);
    layout "channels_first": [B, C, N, N] (N a multiple of 8), the faster form.
    """
    return _TriMulFn.apply(a, b, direction, layout)


class _GateFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, g, p, mask, layout):
        if not isinstance(g, torch.Tensor) or g.dim() != 4 or g.shape[1] != g.shape[2]:
            raise ValueError("g must be channels-last [B, N, N, C]")
        B, N, _, C = g.shape
        _require(g, "g", tuple(g.shape), _BF16)
        _require(p, "p", tuple(g.shape), _BF16)
        if mask is not None:
            _require(mask, "mask", (B, N, N), _MASK)
        _one_gpu([("g", g), ("p", p), ("mask", mask)])
        lay = TRI_MUL_LAYOUTS[layout]
        a = torch.empty((B, C, N, N) if lay == 1 else (B, N, N, C), dtype=g.dtype, device=g.device)
        _check(tri_mul_gate_fwd(lay, B, N, C, g, p, mask, a), "tri_mul_gate_fwd")
        ctx.save_for_backward(g, p, mask)
        ctx.lay = lay
        return a

    @staticmethod
    def backward(ctx, da):
        g, p, mask = ctx.saved_tensors
        B, N, _, C = g.shape
        da = da.contiguous()
        _require(da, "da", (B, C, N, N) if ctx.lay == 1 else (B, N, N, C), _BF16)
        _one_gpu([("g", g), ("da", da)])
        dg, dp = (torch.empty(g.shape, dtype=g.dtype, device=g.device) for _ in range(2))
        _check(tri_mul_gate_bwd(ctx.lay, B, N, C, g, p, mask, da, dg, dp), "tri_mul_gate_bwd")
        return dg, dp, None, None


def gated_operand(g, p, mask=None, layout="channels_first"):
    """a = sigmoid(g) * p * mask, differentiable in g and p: the gated operand of the triangle
    multiplication, from channels-last projections g, p [B, N, N, C] (bf16) and an optional
    uint8 pair mask [B, N, N]; returned in `layout` (channels first [B, C, N, N] by default,
    ready for triangle_multiplication(..., layout="channels_first"))."""
    return _GateFn.apply(g, p, mask, layout)
