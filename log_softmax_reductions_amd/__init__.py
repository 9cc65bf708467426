"""MI355X-native max-shifted log-sum-exp engine: Python binding of liblse.so.

Each function has the name of the C entry point it calls and does argument
marshalling only: it checks that tensors are fp32, contiguous and on the GPU,
allocates outputs / workspaces with torch when the caller passes none, and
enqueues the library call on torch's current stream.  All arithmetic runs in
the HIP kernels of liblse.so; there is no CPU path, and a missing library
raises ImportError on first use.

  lse_reduce_axis0(x)           logsumexp over dim 0 of an (R, ...) tensor
  lse_reduce_axis(x, dim)       logsumexp over any dim (strided views accepted)
  log_softmax_axis(x, dim)      log_softmax over any dim (strided views accepted)
  log_softmax_rows(x)           log_softmax over the last dim of a 2-D tensor
                                (rows may be ld apart: column slices accepted)
  softmax_rows(x)               softmax over the last dim of a 2-D tensor
  lse_rows_partial(x, chunk)    (max, sum) pair per (row, chunk)
  lse_rows_merge(partials)      row logsumexp from the pairs
  fused_conv_gn_act_lse(...)    conv3x3 -> GroupNorm -> tanh -> hardswish ->
                                residual -> logsumexp over channels
"""
from __future__ import annotations

import contextlib
import ctypes
import math

from . import _lib
from ._lib import LseError  # noqa: F401

__all__ = [
    "lse_reduce_axis0", "lse_reduce_axis", "log_softmax_axis", "softmax_rows", "log_softmax_rows",
    "log_softmax_rows_noalloc",
    "log_softmax_rows_workspace_bytes",
    "log_softmax_rows_plan", "lse_testing_set_spin_limit", "lse_testing_set_chain_path",
    "lse_testing_set_rows_reread", "lse_rows_num_chunks", "lse_rows_partial",
    "lse_rows_merge", "fused_conv_gn_act_lse", "fused_conv_gn_act_lse_workspace_bytes",
    "lse_abi_version", "LseError", "lse_axis_workspace_bytes",
]


def _stream(stream):
    """The HIP stream handle: the given torch stream's, else the current stream
    of the current device (callers run inside _on, so the tensors' GPU)."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:  # the handle without building a Stream object
            return ctypes.c_void_p(raw(torch._C._cuda_getDevice()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _dev(t, name, contiguous=True):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32 (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ptr_or_null(t, name):
    return None if t is None else _dev(t, name)


def _on(*ts):
    """Context that makes the tensors' GPU the current device, so the library
    launches on the device that holds the memory; all tensors (None skipped)
    must be on that one GPU."""
    import torch
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one GPU (got {sorted(map(str, devs))})")
    d = devs.pop() if devs else None
    if d is None or d.type != "cuda":
        raise ValueError(f"tensors must be on the GPU (got {d})")
    if d.index is None or d.index == torch.cuda.current_device():
        return contextlib.nullcontext()  # already current: no device switch
    return torch.cuda.device(d)


def _numel(t, n, name):
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements (got {t.numel()})")


def _workspace(nbytes, device, ws, stream=None):
    """The caller's workspace, or a new one from torch's allocator.  A new one
    is allocated on the current stream; when the call runs on another stream
    it is recorded there, so the allocator does not reuse it before that
    stream's kernels are done."""
    import torch
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if stream is not None:
            ws.record_stream(stream)
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws, ws.numel() * ws.element_size()


def lse_abi_version() -> int:
    return int(_lib.load().lse_abi_version())


def lse_axis_workspace_bytes(outer: int, R: int, inner: int, log_softmax: bool = False) -> int:
    """Workspace bytes of the axis calls on these sizes (0: none needed)."""
    return int(_lib.load().lse_axis_workspace_bytes(outer, R, inner, 1 if log_softmax else 0))


def _ws_ptr(ws):
    return None if ws is None else ctypes.c_void_p(ws.data_ptr())


def lse_reduce_axis0(x, out=None, ws=None, stream=None):
    """out[...] = logsumexp over dim 0 of x (shape x.shape[1:]).  Few outputs
    over many planes take a workspace (`ws`, or a new one from torch's
    allocator)."""
    import torch
    lib = _lib.load()
    if x.dim() == 0:
        raise ValueError("x must have at least one dimension")
    R = x.shape[0]
    inner = math.prod(x.shape[1:]) if R > 0 else 0
    if out is None:
        out = torch.empty(x.shape[1:], dtype=torch.float32, device=x.device)
    if out.numel() != inner:
        raise ValueError("out has the wrong number of elements")
    with _on(x, out, ws):
        ws, ws_bytes = _workspace(lse_axis_workspace_bytes(1, R, inner), x.device, ws, stream)
        _lib.check(lib.lse_reduce_axis0_ws(_dev(x, "x"), _dev(out, "out"), R, inner, _ws_ptr(ws),
                                           ws_bytes, _stream(stream)), "lse_reduce_axis0")
    return out


def _axis_view(x, dim):
    """(outer, R, inner) of contiguous x reduced over `dim`."""
    d = dim % x.dim()
    outer = 1
    for n in x.shape[:d]:
        outer *= n
    inner = 1
    for n in x.shape[d + 1:]:
        inner *= n
    return d, outer, x.shape[d], inner


def _collapse(shape, strides, name):
    """Stride of the dims of `shape` merged into one run, or None when they
    do not merge (size-1 dims are ignored; an empty or all-size-1 set merges
    to stride 0)."""
    dims = [(n, st) for n, st in zip(shape, strides) if n != 1]
    for (n0, s0), (n1, s1) in zip(dims, dims[1:]):
        if s0 != s1 * n1:
            return None
    return dims[-1][1] if dims else 0


def _strided_axis(t, d, name):
    """(outer_stride, r_stride) of t viewed as (outer, R, inner) around dim d,
    the inner run contiguous.  Raises ValueError for layouts the strided
    entry points cannot express (no silent copy is made)."""
    shape, strides = tuple(t.shape), tuple(t.stride())
    inner_st = _collapse(shape[d + 1:], strides[d + 1:], name)
    if inner_st not in (0, 1):
        raise ValueError(f"{name}: the dims after the reduced one must form one contiguous run")
    outer_st = _collapse(shape[:d], strides[:d], name)
    if outer_st is None:
        raise ValueError(f"{name}: the dims before the reduced one must merge into one stride")
    return outer_st, strides[d]


def lse_reduce_axis(x, dim, out=None, ws=None, stream=None):
    """logsumexp over `dim` of an fp32 GPU tensor (dim removed).  x and out
    may be strided views whose dims after `dim` form one contiguous run and
    whose dims before it merge into one stride.  Few outputs over many planes
    take a workspace (`ws`, or a new one from torch's allocator)."""
    import torch
    lib = _lib.load()
    d, outer, R, inner = _axis_view(x, dim)
    shape = tuple(x.shape[:d]) + tuple(x.shape[d + 1:])
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must have shape {shape}")
    xso, xsr = _strided_axis(x, d, "x")
    oso, _ = _strided_axis(out.unsqueeze(d), d, "out")
    with _on(x, out, ws):
        ws, ws_bytes = _workspace(lse_axis_workspace_bytes(outer, R, inner), x.device, ws, stream)
        _lib.check(lib.lse_reduce_axis_strided_ws(_dev(x, "x", False), _dev(out, "out", False),
                                                  outer, R, inner, xso, xsr, oso, _ws_ptr(ws),
                                                  ws_bytes, _stream(stream)),
                   "lse_reduce_axis")
    return out


def log_softmax_axis(x, dim, y=None, ws=None, stream=None):
    """log_softmax over `dim` of an fp32 GPU tensor; x and y may be strided
    views as for lse_reduce_axis (a new y is contiguous).  Few outputs over
    many planes, and long last-axis rows, take a workspace (`ws`, or a new
    one from torch's allocator)."""
    import torch
    lib = _lib.load()
    d, outer, R, inner = _axis_view(x, dim)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    if y.shape != x.shape:
        raise ValueError("y must have x's shape")
    xso, xsr = _strided_axis(x, d, "x")
    yso, ysr = _strided_axis(y, d, "y")
    with _on(x, y, ws):
        ws, ws_bytes = _workspace(lse_axis_workspace_bytes(outer, R, inner, True), x.device, ws,
                                  stream)
        _lib.check(lib.log_softmax_axis_strided_ws(_dev(x, "x", False), _dev(y, "y", False),
                                                   outer, R, inner, xso, xsr, yso, ysr,
                                                   _ws_ptr(ws), ws_bytes, _stream(stream)),
                   "log_softmax_axis")
    return y


def _ld(t, name):
    """Row pitch of a 2-D tensor whose rows are contiguous."""
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: each row must be contiguous (stride 1 along dim 1)")
    return t.stride(0) if rows > 1 else cols


def _rows_call(fn, name, x, y, ws, stream):
    import torch
    lib = _lib.load()
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, cols)")
    rows, cols = x.shape
    if y is None:
        y = torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    if y.shape != x.shape:
        raise ValueError("y must have x's shape")
    ldx, ldy = _ld(x, "x"), _ld(y, "y")
    with _on(x, y, ws):
        ws, ws_bytes = _workspace(log_softmax_rows_workspace_bytes(rows, cols), x.device, ws,
                                  stream)
        _lib.check(getattr(lib, fn)(_dev(x, "x", False), _dev(y, "y", False), rows, cols, ldx,
                                    ldy, None if ws is None else ctypes.c_void_p(ws.data_ptr()),
                                    ws_bytes, _stream(stream)), name)
    return y


def log_softmax_rows_noalloc(x, y, stream=None):
    """log_softmax_rows with the library's static device scratch instead of a
    workspace: x and y are contiguous 2-D fp32 tensors on one GPU (y given:
    the call allocates nothing)."""
    lib = _lib.load()
    if x.dim() != 2 or y.shape != x.shape:
        raise ValueError("x must be 2-D (rows, cols) and y the same shape")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise ValueError("log_softmax_rows_noalloc takes contiguous x and y")
    rows, cols = x.shape
    with _on(x, y):
        _lib.check(lib.log_softmax_rows_noalloc(_dev(x, "x", False), _dev(y, "y", False), rows,
                                                cols, _stream(stream)),
                   "log_softmax_rows_noalloc")
    return y


def softmax_rows(x, y=None, ws=None, stream=None):
    """y = softmax(x, dim=-1) for a 2-D fp32 GPU tensor x whose rows are
    contiguous (rows may be any pitch apart)."""
    return _rows_call("softmax_rows_strided", "softmax_rows", x, y, ws, stream)


def log_softmax_rows_workspace_bytes(rows: int, cols: int) -> int:
    return int(_lib.load().log_softmax_rows_workspace_bytes(rows, cols))


def log_softmax_rows_plan(cols: int):
    """(nchunks, chunk): workgroups per row and columns per workgroup."""
    n, c = ctypes.c_int64(), ctypes.c_int64()
    _lib.check(_lib.load().log_softmax_rows_plan(cols, ctypes.byref(n), ctypes.byref(c)),
               "log_softmax_rows_plan")
    return n.value, c.value


def lse_testing_set_spin_limit(polls: int) -> None:
    """Test hook (include/lse_testing.h): the poll limit of the split rows' and
    the conv chain's cross-workgroup waits, for calls this thread enqueues."""
    _lib.load().lse_testing_set_spin_limit(int(polls))


def lse_testing_set_chain_path(path: int) -> None:
    """Test hook (include/lse_testing.h): 0 automatic, 1 fused, 2 statistics +
    recomputing apply, 3 statistics + staged apply, for calls this thread
    enqueues (and for the workspace size it queries)."""
    _lib.check(_lib.load().lse_testing_set_chain_path(int(path)), "lse_testing_set_chain_path")


def lse_testing_set_rows_reread(enable: bool) -> None:
    """Test hook (include/lse_testing.h): split rows through the re-read kernel
    (chunks read again for the write) instead of the register-resident one."""
    _lib.load().lse_testing_set_rows_reread(1 if enable else 0)


def log_softmax_rows(x, y=None, ws=None, stream=None):
    """y = log_softmax(x, dim=-1) for a 2-D fp32 GPU tensor x whose rows are
    contiguous (rows may be any pitch apart)."""
    return _rows_call("log_softmax_rows_strided", "log_softmax_rows", x, y, ws, stream)


def lse_rows_num_chunks(cols: int, chunk: int) -> int:
    return int(_lib.load().lse_rows_num_chunks(cols, chunk))


def lse_rows_partial(x, chunk: int, partials=None, stream=None):
    """(rows, nchunks, 2) float32 tensor of (m, s) pairs per chunk of each row."""
    import torch
    lib = _lib.load()
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, cols)")
    rows, cols = x.shape
    k = lse_rows_num_chunks(cols, chunk)
    if k < 1:
        raise ValueError("invalid cols / chunk")
    if partials is None:
        partials = torch.empty((rows, k, 2), dtype=torch.float32, device=x.device)
    if partials.numel() != rows * k * 2:
        raise ValueError("partials has the wrong size")
    with _on(x, partials):
        _lib.check(lib.lse_rows_partial(_dev(x, "x"), rows, cols, chunk,
                                        _dev(partials, "partials"), _stream(stream)),
                   "lse_rows_partial")
    return partials


def lse_rows_merge(partials, row_lse=None, stream=None):
    """(rows,) row logsumexp from a (rows, nchunks, 2) tensor of pairs."""
    import torch
    lib = _lib.load()
    if partials.dim() != 3 or partials.shape[2] != 2:
        raise ValueError("partials must be (rows, nchunks, 2)")
    rows, k, _ = partials.shape
    if row_lse is None:
        row_lse = torch.empty(rows, dtype=torch.float32, device=partials.device)
    _numel(row_lse, rows, "row_lse")
    with _on(partials, row_lse):
        _lib.check(lib.lse_rows_merge(_dev(partials, "partials"), rows, k,
                                      _dev(row_lse, "row_lse"), _stream(stream)),
                   "lse_rows_merge")
    return row_lse


def fused_conv_gn_act_lse_workspace_bytes(N, Cin, H, W, Cout, K, groups) -> int:
    return int(_lib.load().fused_conv_gn_act_lse_workspace_bytes(N, Cin, H, W, Cout, K, groups))


def fused_conv_gn_act_lse(x, w, b, gamma, beta, groups: int, eps: float = 1e-5, out=None,
                          ws=None, stream=None):
    """(N, 1, Ho, Wo) = logsumexp_c(conv + hardswish(tanh(GroupNorm(conv))))."""
    import torch
    lib = _lib.load()
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("x must be (N, Cin, H, W) and w (Cout, Cin, K, K)")
    N, Cin, H, W = x.shape
    Cout, Cin2, K, K2 = w.shape
    if Cin2 != Cin or K2 != K:
        raise ValueError("w does not match x")
    Ho, Wo = H - K + 1, W - K + 1
    for t, name in ((b, "b"), (gamma, "gamma"), (beta, "beta")):
        _numel(t, Cout, name)
    if out is None:
        out = torch.empty((N, 1, Ho, Wo), dtype=torch.float32, device=x.device)
    if Ho > 0 and Wo > 0:
        _numel(out, N * Ho * Wo, "out")
    with _on(x, w, b, gamma, beta, out, ws):
        ws, ws_bytes = _workspace(
            fused_conv_gn_act_lse_workspace_bytes(N, Cin, H, W, Cout, K, groups), x.device, ws,
            stream)
        _lib.check(lib.fused_conv_gn_act_lse(
            _dev(x, "x"), _dev(w, "w"), _ptr_or_null(b, "b"), _ptr_or_null(gamma, "gamma"),
            _ptr_or_null(beta, "beta"), N, Cin, H, W, Cout, K, groups, float(eps),
            _dev(out, "out"), None if ws is None else ctypes.c_void_p(ws.data_ptr()), ws_bytes,
            _stream(stream)), "fused_conv_gn_act_lse")
    return out
