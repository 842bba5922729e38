"""Tensor-parallel sharded linear layer Y = X W on one MI355X (gfx950).

Thin torch binding over the C interface of libtp_amd.so (include/tp.h):
it reads data pointers, shapes and strides of torch tensors, passes the
current HIP stream, and calls the library. Every step of the computation
runs in the library's HIP kernels; this module computes nothing itself.

Shard layouts accepted for weights and inputs:
  * 2-D tensors: the logical full matrix; shard s is its s-th contiguous block
    of columns (column split) or rows (row split);
  * 3-D tensors [N, r, c]: shard-major storage, block s = t[s].
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (TP_ACT_GELU, TP_ACT_NONE, TP_BF16, TP_F32, TP_SPLIT_COLS, TP_SPLIT_ROWS, TP_SPLIT_TOKENS,
                   TpError, TpMatrix, status_string)

__all__ = [
    "col_linear",
    "row_linear",
    "reduce_partials",
    "mlp",
    "mlp_workspace_bytes",
    "mlp_noalloc",
    "mlp_noalloc_max_scratch",
    "col_linear_backward",
    "row_linear_backward",
    "mlp_backward",
    "mlp_backward_workspace_bytes",
    "attention",
    "sp_layernorm",
    "TpError",
    "library",
    "version",
]

_ACTS = {"none": TP_ACT_NONE, "gelu": TP_ACT_GELU}
_AXES = {"rows": TP_SPLIT_ROWS, "cols": TP_SPLIT_COLS, "tokens": TP_SPLIT_TOKENS}


def library() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    return _lib.load()


def version() -> int:
    return int(library().tp_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TP_F32
    if t.dtype == torch.bfloat16:
        return TP_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _require_gpu(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if t.dim() >= 1 and t.numel() > 0 and t.stride(-1) != 1:
            raise ValueError("the last dimension must be contiguous (stride 1)")


def _full(t: torch.Tensor) -> TpMatrix:
    """A 2-D tensor as one row-major matrix."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    return _lib.matrix(t.data_ptr(), _dtype_code(t), t.shape[0], t.shape[1], max(t.stride(0), t.shape[1]), 0)


def _blocks(t: torch.Tensor, rows: int, cols: int) -> TpMatrix:
    """A 2-D logical matrix, or a 3-D shard-major stack whose logical shape is (rows, cols)."""
    if t.dim() == 2:
        return _full(t)
    if t.dim() != 3:
        raise ValueError("expected a 2-D matrix or a 3-D shard-major stack")
    ld = max(t.stride(1), t.shape[2])
    stride = t.stride(0) if t.shape[0] > 1 else max(1, (t.shape[1] - 1) * ld + t.shape[2])
    return _lib.matrix(t.data_ptr(), _dtype_code(t), rows, cols, ld, stride)


def _check_stack(t: torch.Tensor, s0: int, ns: int) -> None:
    """A shard-major stack [blocks, r, c] must hold block s for every executed shard s (block s = t[s])."""
    if t.dim() == 3 and t.shape[0] < s0 + ns:
        raise ValueError(f"shard-major stack holds {t.shape[0]} blocks, shards up to {s0 + ns - 1} are executed")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def col_linear(x: torch.Tensor, w: torch.Tensor, n: int, s0: int = 0, ns: int | None = None, act: str = "none",
               out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
               partitioned: bool = False) -> torch.Tensor:
    """Column-parallel linear: Y_j = act(X W_{s0+j}) for the executed shards.

    w: [K, Nout] (shard s = columns s*Nout/n ...) or shard-major [n, K, Nout/n].
    Returns Y [M, ns*Nout/n] (concatenated), or [ns, M, Nout/n] if partitioned.
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w)
    k = x.shape[1]
    _check_stack(w, s0, ns)
    nout = w.shape[1] if w.dim() == 2 else n * w.shape[2]
    width = nout // n if n > 0 else 0
    od = out_dtype or (out.dtype if out is not None else x.dtype)
    if out is None:
        shape = (ns, x.shape[0], width) if partitioned else (x.shape[0], ns * width)
        out = torch.empty(shape, dtype=od, device=x.device)
    _require_gpu(out)
    if out.dim() == 3:
        ym = _lib.matrix(out.data_ptr(), _dtype_code(out), out.shape[1], ns * width,
                         max(out.stride(1), out.shape[2]),
                         out.stride(0) if out.shape[0] > 1 else max(1, (out.shape[1] - 1) * out.stride(1) + width))
    else:
        ym = _full(out)
    xm = _full(x)
    wm = _blocks(w, k, nout)
    st = library().tp_col_linear(ctypes.byref(xm), ctypes.byref(wm), n, s0, ns, _ACTS[act], ctypes.byref(ym),
                                 ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_col_linear")
    return out


def row_linear(x: torch.Tensor, w: torch.Tensor, n: int, s0: int = 0, ns: int | None = None,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-parallel partial products P_j = X_{s0+j} W_{s0+j} (fp32), returned as [ns, M, Nout].

    x: [M, K] (shard s = columns s*K/n ...) or shard-major [n, M, K/n].
    w: [K, Nout] (shard s = rows s*K/n ...) or shard-major [n, K/n, Nout].
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w)
    _check_stack(x, s0, ns)
    _check_stack(w, s0, ns)
    m = x.shape[0] if x.dim() == 2 else x.shape[1]
    k = x.shape[1] if x.dim() == 2 else n * x.shape[2]
    nout = w.shape[1] if w.dim() == 2 else w.shape[2]
    if out is None:
        out = torch.empty((ns, m, nout), dtype=torch.float32, device=x.device)
    _require_gpu(out)
    xm = _blocks(x, m, k)
    wm = _blocks(w, k, nout)
    pm = _lib.matrix(out.data_ptr(), _dtype_code(out), m, nout, max(out.stride(1), nout),
                     out.stride(0) if out.shape[0] > 1 else 0)
    st = library().tp_row_linear(ctypes.byref(xm), ctypes.byref(wm), n, s0, ns, ctypes.byref(pm),
                                 ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_row_linear")
    return out


def reduce_partials(p: torch.Tensor, axis: str = "rows", out: torch.Tensor | None = None,
                    out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Combine shard outputs p [n, R, C]: sum (axis="rows"), concatenation of columns (axis="cols")
    or token shards stacked in order (axis="tokens", [n*R, C])."""
    _require_gpu(p)
    n, r, c = p.shape
    if out is None:
        shape = {"rows": (r, c), "cols": (r, n * c), "tokens": (n * r, c)}[axis]
        out = torch.empty(shape, dtype=out_dtype, device=p.device)
    _require_gpu(out)
    pm = _lib.matrix(p.data_ptr(), _dtype_code(p), r, c, max(p.stride(1), c), p.stride(0) if n > 1 else 0)
    ym = _full(out)
    st = library().tp_reduce_partials(ctypes.byref(pm), n, _AXES[axis], ctypes.byref(ym),
                                      ctypes.c_void_p(_stream(p)))
    _lib.check(st, "tp_reduce_partials")
    return out


def _mlp_mats(x, w1, w2, n):
    d = x.shape[1]
    f = w1.shape[1] if w1.dim() == 2 else n * w1.shape[2]
    dout = w2.shape[1] if w2.dim() == 2 else w2.shape[2]
    return _full(x), _blocks(w1, d, f), _blocks(w2, f, dout), dout


def mlp_workspace_bytes(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, n: int, s0: int = 0,
                        ns: int | None = None, act: str = "gelu") -> int:
    """Device scratch that mlp() needs for these operands (query of the library)."""
    ns = n - s0 if ns is None else ns
    _check_stack(w1, s0, ns)
    _check_stack(w2, s0, ns)
    xm, w1m, w2m, dout = _mlp_mats(x, w1, w2, n)
    ym = _lib.matrix(0, TP_F32, x.shape[0], dout, dout, 0)
    size = ctypes.c_size_t(0)
    st = library().tp_mlp(ctypes.byref(xm), ctypes.byref(w1m), ctypes.byref(w2m), n, s0, ns, _ACTS[act], None,
                          ctypes.byref(size), ctypes.byref(ym), None)
    _lib.check(st, "tp_mlp(workspace query)")
    return int(size.value)


def mlp(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, n: int, s0: int = 0, ns: int | None = None,
        act: str = "gelu", out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Megatron MLP pair: Y = sum_s act(X W1_s) W2_s over the executed shards, fp32 [M, Dout].

    w1: [d, F] or shard-major [n, d, F/n]; w2: [F, Dout] or shard-major [n, F/n, Dout].
    workspace: optional uint8 device tensor of at least mlp_workspace_bytes(...) bytes.
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w1, w2)
    xm, w1m, w2m, dout = _mlp_mats(x, w1, w2, n)
    if out is None:
        out = torch.empty((x.shape[0], dout), dtype=torch.float32, device=x.device)
    _require_gpu(out)
    need = mlp_workspace_bytes(x, w1, w2, n, s0, ns, act)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ym = _full(out)
    size = ctypes.c_size_t(workspace.numel())
    st = library().tp_mlp(ctypes.byref(xm), ctypes.byref(w1m), ctypes.byref(w2m), n, s0, ns, _ACTS[act],
                          ctypes.c_void_p(workspace.data_ptr()), ctypes.byref(size), ctypes.byref(ym),
                          ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_mlp")
    return out


def mlp_noalloc(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, n: int, s0: int = 0,
                ns: int | None = None, act: str = "gelu", out: torch.Tensor | None = None) -> torch.Tensor:
    """tp_mlp_noalloc: the MLP pair with the library's built-in per-GPU scratch instead of a workspace.

    Raises TpError (TP_ERR_TOO_LARGE) when the shapes need more than mlp_noalloc_max_scratch() bytes.
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w1, w2)
    xm, w1m, w2m, dout = _mlp_mats(x, w1, w2, n)
    if out is None:
        out = torch.empty((x.shape[0], dout), dtype=torch.float32, device=x.device)
    _require_gpu(out)
    ym = _full(out)
    st = library().tp_mlp_noalloc(ctypes.byref(xm), ctypes.byref(w1m), ctypes.byref(w2m), n, s0, ns, _ACTS[act],
                                  ctypes.byref(ym), ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_mlp_noalloc")
    return out


def mlp_noalloc_max_scratch() -> int:
    """Bytes of the per-GPU scratch array mlp_noalloc uses."""
    return int(library().tp_mlp_noalloc_max_scratch())


# ----------------------------------------------------------------------------- backward passes


def _ref(t):
    return ctypes.byref(t) if t is not None else None


def _out(spec, shape3, shape2, partitioned, dtype, device):
    """An output tensor: the one given, a new one (spec True), or None (spec False/None)."""
    if spec is None or spec is False:
        return None
    if isinstance(spec, torch.Tensor):
        return spec
    return torch.empty(shape3 if partitioned else shape2, dtype=dtype, device=device)


def col_linear_backward(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, n: int, s0: int = 0,
                        ns: int | None = None, dx_partials=True, dw=True, dw_dtype: torch.dtype = torch.float32,
                        partitioned_dw: bool = False):
    """Backward of col_linear (no activation): returns (P, dW).

    dy: [M, ns*Nout/n] or partitioned [ns, M, Nout/n].
    P: fp32 [ns, M, K] with P_j = dY_j W_{s0+j}^T; dX is their sum (reduce_partials).
    dW: [K, ns*Nout/n] (or [ns, K, Nout/n] if partitioned_dw) with dW_j = X^T dY_j.
    Pass False to skip an output or a tensor to write into.
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w, dy)
    _check_stack(w, s0, ns)
    m, k = x.shape
    nout = w.shape[1] if w.dim() == 2 else n * w.shape[2]
    width = nout // n if n > 0 else 0
    p = _out(dx_partials, (ns, m, k), None, True, torch.float32, x.device)
    g = _out(dw, (ns, k, width), (k, ns * width), partitioned_dw, dw_dtype, x.device)
    pm = None if p is None else _lib.matrix(p.data_ptr(), TP_F32, m, k, max(p.stride(1), k),
                                            p.stride(0) if p.shape[0] > 1 else 0)
    gm = None if g is None else _blocks(g, k, ns * width)
    st = library().tp_col_linear_backward(ctypes.byref(_full(x)), ctypes.byref(_blocks(w, k, nout)),
                                          ctypes.byref(_blocks(dy, m, ns * width)), n, s0, ns, _ref(pm), _ref(gm),
                                          ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_col_linear_backward")
    return p, g


def row_linear_backward(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, n: int, s0: int = 0,
                        ns: int | None = None, dx=True, dw=True, dx_dtype: torch.dtype = torch.float32,
                        dw_dtype: torch.dtype = torch.float32, partitioned: bool = False):
    """Backward of row_linear: returns (dX, dW) for the executed shards.

    dX: [M, ns*K/n] (or [ns, M, K/n] if partitioned) with dX_j = dY W_{s0+j}^T.
    dW: [ns*K/n, Nout] (or [ns, K/n, Nout] if partitioned) with dW_j = X_{s0+j}^T dY.
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w, dy)
    _check_stack(x, s0, ns)
    _check_stack(w, s0, ns)
    m = x.shape[0] if x.dim() == 2 else x.shape[1]
    k = x.shape[1] if x.dim() == 2 else n * x.shape[2]
    nout = w.shape[1] if w.dim() == 2 else w.shape[2]
    kb = k // n if n > 0 else 0
    a = _out(dx, (ns, m, kb), (m, ns * kb), partitioned, dx_dtype, x.device)
    g = _out(dw, (ns, kb, nout), (ns * kb, nout), partitioned, dw_dtype, x.device)
    am = None if a is None else _blocks(a, m, ns * kb)
    gm = None if g is None else _blocks(g, ns * kb, nout)
    st = library().tp_row_linear_backward(ctypes.byref(_blocks(x, m, k)), ctypes.byref(_blocks(w, k, nout)),
                                          ctypes.byref(_full(dy)), n, s0, ns, _ref(am), _ref(gm),
                                          ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_row_linear_backward")
    return a, g


def _mlp_bwd_mats(x, w1, w2, dy, n, ns, dx, dw1, dw2):
    xm, w1m, w2m, dout = _mlp_mats(x, w1, w2, n)
    m, d = x.shape
    f = w1.shape[1] if w1.dim() == 2 else n * w1.shape[2]
    width = f // n if n > 0 else 0
    am = None if dx is None else _full(dx)
    g1 = None if dw1 is None else _blocks(dw1, d, ns * width)
    g2 = None if dw2 is None else _blocks(dw2, ns * width, dout)
    return xm, w1m, w2m, _full(dy), am, g1, g2


def mlp_backward_workspace_bytes(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, dy: torch.Tensor, n: int,
                                 s0: int = 0, ns: int | None = None, act: str = "gelu", dx: bool = True,
                                 dw1: bool = True, dw2: bool = True) -> int:
    """Device scratch that mlp_backward() needs for these operands and requested gradients."""
    ns = n - s0 if ns is None else ns
    _check_stack(w1, s0, ns)
    _check_stack(w2, s0, ns)
    m, d = x.shape
    f = w1.shape[1] if w1.dim() == 2 else n * w1.shape[2]
    dout = w2.shape[1] if w2.dim() == 2 else w2.shape[2]
    width = f // n if n > 0 else 0
    xm, w1m, w2m, dout = _mlp_mats(x, w1, w2, n)
    am = _lib.matrix(0, TP_F32, m, d, d, 0) if dx else None
    g1 = _lib.matrix(0, TP_F32, d, ns * width, ns * width, 0) if dw1 else None
    g2 = _lib.matrix(0, TP_F32, ns * width, dout, dout, 0) if dw2 else None
    size = ctypes.c_size_t(0)
    st = library().tp_mlp_backward(ctypes.byref(xm), ctypes.byref(w1m), ctypes.byref(w2m), ctypes.byref(_full(dy)),
                                   n, s0, ns, _ACTS[act], None, ctypes.byref(size), _ref(am), _ref(g1), _ref(g2),
                                   None)
    _lib.check(st, "tp_mlp_backward(workspace query)")
    return int(size.value)


def mlp_backward(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, dy: torch.Tensor, n: int, s0: int = 0,
                 ns: int | None = None, act: str = "gelu", dx=True, dw1=True, dw2=True,
                 dw_dtype: torch.dtype = torch.float32, workspace: torch.Tensor | None = None):
    """Backward of mlp(): returns (dX fp32 [M, d], dW1 [d, ns*F/n], dW2 [ns*F/n, Dout]).

    Pass False to skip a gradient or a tensor to write into (dW1/dW2 may be
    shard-major stacks [ns, d, F/n] / [ns, F/n, Dout]).
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(x, w1, w2, dy)
    m, d = x.shape
    f = w1.shape[1] if w1.dim() == 2 else n * w1.shape[2]
    dout = w2.shape[1] if w2.dim() == 2 else w2.shape[2]
    width = f // n if n > 0 else 0
    a = _out(dx, None, (m, d), False, torch.float32, x.device)
    g1 = _out(dw1, None, (d, ns * width), False, dw_dtype, x.device)
    g2 = _out(dw2, None, (ns * width, dout), False, dw_dtype, x.device)
    need = mlp_backward_workspace_bytes(x, w1, w2, dy, n, s0, ns, act, a is not None, g1 is not None,
                                        g2 is not None)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    xm, w1m, w2m, dym, am, g1m, g2m = _mlp_bwd_mats(x, w1, w2, dy, n, ns, a, g1, g2)
    size = ctypes.c_size_t(workspace.numel())
    st = library().tp_mlp_backward(ctypes.byref(xm), ctypes.byref(w1m), ctypes.byref(w2m), ctypes.byref(dym), n,
                                   s0, ns, _ACTS[act], ctypes.c_void_p(workspace.data_ptr()), ctypes.byref(size),
                                   _ref(am), _ref(g1m), _ref(g2m), ctypes.c_void_p(_stream(x)))
    _lib.check(st, "tp_mlp_backward")
    return a, g1, g2


# ----------------------------------------------------------------------------- attention per head subset


def attention(qkv: torch.Tensor, n: int, heads: int, kv_heads: int, head_dim: int, seq_len: int,
              causal: bool = True, s0: int = 0, ns: int | None = None, out: torch.Tensor | None = None,
              partitioned: bool = False) -> torch.Tensor:
    """Attention of the executed shards' heads (tp_attention).

    qkv: [M, ns*(hq + 2 hkv)*head_dim] (column-parallel QKV output) or partitioned
    [ns, M, (hq + 2 hkv)*head_dim]. Returns [M, ns*hq*head_dim] (or [ns, M, hq*head_dim]).
    """
    ns = n - s0 if ns is None else ns
    _require_gpu(qkv)
    hq = heads // n if n > 0 else 0
    hkv = (kv_heads // n if kv_heads >= n else 1) if n > 0 else 0
    blk = (hq + 2 * hkv) * head_dim
    m = qkv.shape[0] if qkv.dim() == 2 else qkv.shape[1]
    oblk = hq * head_dim
    if out is None:
        shape = (ns, m, oblk) if partitioned else (m, ns * oblk)
        out = torch.empty(shape, dtype=qkv.dtype, device=qkv.device)
    _require_gpu(out)
    qm = _blocks(qkv, m, ns * blk)
    am = _blocks(out, m, ns * oblk)
    st = library().tp_attention(ctypes.byref(qm), n, s0, ns, heads, kv_heads, head_dim, seq_len, int(bool(causal)),
                                ctypes.byref(am), ctypes.c_void_p(_stream(qkv)))
    _lib.check(st, "tp_attention")
    return out


# ----------------------------------------------------------------------------- sequence parallelism


def sp_layernorm(p: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, n: int, s0: int = 0,
                 ns: int | None = None, residual: torch.Tensor | None = None, keep: torch.Tensor | None = None,
                 p_drop: float = 0.0, eps: float = 1e-5, out: torch.Tensor | None = None,
                 out_dtype: torch.dtype | None = None, residual_out: bool | torch.Tensor = False,
                 partitioned: bool = False):
    """Reduce-scatter, dropout, residual add and LayerNorm on token shards s0 .. s0+ns-1 (tp_sp_layernorm).

    p: fp32 partials [t, M, d] (row_linear's output; summed in order) or [M, d].
    residual, out, residual_out: [ns*M/n, d], or [ns, M/n, d] when partitioned.
    keep: uint8 0/1 [ns*M/n, d] (contiguous), or None for no dropout.
    Returns y, or (y, x) when residual_out is set (x = the pre-norm sum, fp32).
    """
    ns = n - s0 if ns is None else ns
    p3 = p if p.dim() == 3 else p.unsqueeze(0)
    _require_gpu(p3, gamma, beta)
    t, m, d = p3.shape
    rows = ns * (m // n) if n > 0 else 0
    shape = (ns, rows // ns if ns > 0 else 0, d) if partitioned else (rows, d)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype or torch.float32, device=p.device)
    x1 = None
    if isinstance(residual_out, torch.Tensor):
        x1 = residual_out
    elif residual_out:
        x1 = torch.empty(shape, dtype=torch.float32, device=p.device)
    for a in (out, x1, residual):
        if a is not None:
            _require_gpu(a)
    if keep is not None:
        _require_gpu(keep)
        if keep.dtype != torch.uint8 or not keep.is_contiguous() or keep.numel() != rows * d:
            raise ValueError("keep must be a contiguous uint8 tensor of ns*M/n x d elements")
    if not (gamma.dtype == beta.dtype == torch.float32 and gamma.is_contiguous() and beta.is_contiguous()):
        raise ValueError("gamma and beta must be contiguous float32 vectors")
    if gamma.numel() != d or beta.numel() != d:
        raise ValueError(f"gamma and beta must hold {d} elements")
    pm = _lib.matrix(p3.data_ptr(), _dtype_code(p3), m, d,
                     max(p3.stride(1), d), p3.stride(0) if t > 1 else 0)
    ym = _blocks(out, rows, d)
    rm = _blocks(residual, rows, d) if residual is not None else None
    xm = _blocks(x1, rows, d) if x1 is not None else None
    st = library().tp_sp_layernorm(ctypes.byref(pm), t, _ref(rm),
                                   ctypes.c_void_p(keep.data_ptr() if keep is not None else 0), float(p_drop),
                                   ctypes.c_void_p(gamma.data_ptr()), ctypes.c_void_p(beta.data_ptr()), float(eps),
                                   n, s0, ns, _ref(xm), ctypes.byref(ym), ctypes.c_void_p(_stream(p3)))
    _lib.check(st, "tp_sp_layernorm")
    return (out, x1) if x1 is not None else out
