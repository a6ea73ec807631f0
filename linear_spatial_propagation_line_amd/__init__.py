"""GSPN 2D line-scan propagation on MI355X (gfx950).

Thin ctypes binding over ``libgspn.so`` (built from ``csrc/`` by
``python -m linear_spatial_propagation_line_amd.build``). It only marshals
arguments: every step of the propagation runs in the library's HIP kernels,
and there is no fallback -- a missing library raises.

    out = propagate(x, (l0, l1, l2), lam, u, dirs=ALL, group_rows=0)

computes, for every plane of the [B, C, H, W] tensors, the sum over the
selected scan directions of u * h_d, where h_d is the line scan
h_s = w_s h_{s-1} + lam * x with tridiagonal, row-normalised sigmoid weights
(CSDN page on GSPN, sections 方法 and 如何设计一个高效的传播层). The C ABI and its
argument rules are documented in include/gspn.h.
"""
from __future__ import annotations

import ctypes
import os

T2B, B2T, L2R, R2L, ALL = 1, 2, 4, 8, 15
GSPN_F32, GSPN_BF16 = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgspn.so")

_STATUS = ["GSPN_OK", "GSPN_E_NULL", "GSPN_E_SHAPE", "GSPN_E_DIRMASK", "GSPN_E_GROUP",
           "GSPN_E_DTYPE", "GSPN_E_ALIGN", "GSPN_E_ALIAS", "GSPN_E_NOMEM", "GSPN_E_HIP",
           "GSPN_E_WORKSPACE"]
STATUS = {name: i for i, name in enumerate(_STATUS)}

_lib = None


class GspnError(RuntimeError):
    """A gspn_* call returned a non-zero status."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = _STATUS[status] if 0 <= status < len(_STATUS) else str(status)
        self.detail = detail
        super().__init__(f"{self.name}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded libgspn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_spatial_propagation_line_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        logits_t = ctypes.POINTER(ctypes.c_void_p)
        common = [vp, logits_t, vp, vp, i64, i64, i64, i64, u32, i64, ctypes.c_int, vp]
        L.gspn_propagate.argtypes = common + [vp]
        L.gspn_propagate.restype = ctypes.c_int
        L.gspn_propagate_ws.argtypes = common + [vp, ctypes.c_size_t, vp]
        L.gspn_propagate_ws.restype = ctypes.c_int
        L.gspn_propagate_noalloc.argtypes = common + [vp]
        L.gspn_propagate_noalloc.restype = ctypes.c_int
        L.gspn_noalloc_scratch_bytes.argtypes = []
        L.gspn_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.gspn_workspace_bytes.argtypes = [i64, i64, i64, i64, u32, i64, ctypes.c_int]
        L.gspn_workspace_bytes.restype = ctypes.c_size_t
        L.gspn_plan_name.argtypes = [i64, i64, i64, i64, u32, i64, ctypes.c_int]
        L.gspn_plan_name.restype = ctypes.c_char_p
        L.gspn_status_str.argtypes = [ctypes.c_int]
        L.gspn_status_str.restype = ctypes.c_char_p
        L.gspn_last_error.argtypes = []
        L.gspn_last_error.restype = ctypes.c_char_p
        L.gspn_trace_events.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.gspn_trace_events.restype = None
        L.gspn_trace_count.argtypes = []
        L.gspn_trace_count.restype = ctypes.c_int
        L.gspn_trace_kernel.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]
        L.gspn_trace_kernel.restype = ctypes.c_char_p
        L.gspn_abi_version.argtypes = []
        L.gspn_abi_version.restype = ctypes.c_int
        bcommon = [vp, logits_t, vp, vp, vp, i64, i64, i64, i64, u32, i64, ctypes.c_int,
                   vp, logits_t, vp, vp]
        L.gspn_propagate_backward.argtypes = bcommon + [vp]
        L.gspn_propagate_backward.restype = ctypes.c_int
        L.gspn_propagate_backward_ws.argtypes = bcommon + [vp, ctypes.c_size_t, vp]
        L.gspn_propagate_backward_ws.restype = ctypes.c_int
        L.gspn_backward_workspace_bytes.argtypes = [i64, i64, i64, i64, u32, i64, ctypes.c_int]
        L.gspn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.gspn_backward_plan_name.argtypes = [i64, i64, i64, i64, u32, i64, ctypes.c_int]
        L.gspn_backward_plan_name.restype = ctypes.c_char_p
        L.gspn_propagate_shared_ws.argtypes = [vp, logits_t, i64, vp, vp, i64, i64, i64, i64, u32,
                                               i64, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
        L.gspn_propagate_shared_ws.restype = ctypes.c_int
        L.gspn_propagate_backward_shared_ws.argtypes = [
            vp, logits_t, i64, vp, vp, vp, i64, i64, i64, i64, u32, i64, ctypes.c_int,
            vp, logits_t, vp, vp, vp, ctypes.c_size_t, vp]
        L.gspn_propagate_backward_shared_ws.restype = ctypes.c_int
        L.gspn_backward_workspace_bytes_shared.argtypes = [i64, i64, i64, i64, i64, u32, i64,
                                                           ctypes.c_int]
        L.gspn_backward_workspace_bytes_shared.restype = ctypes.c_size_t
        L.gspn_propagate_dirs_ws.argtypes = [vp, logits_t, vp, vp, i64, vp, i64, i64, i64, i64,
                                             u32, i64, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
        L.gspn_propagate_dirs_ws.restype = ctypes.c_int
        L.gspn_workspace_bytes_dirs.argtypes = [i64, i64, i64, i64, u32, i64, ctypes.c_int]
        L.gspn_workspace_bytes_dirs.restype = ctypes.c_size_t
        L.gspn_propagate_backward_dirs_ws.argtypes = [
            vp, logits_t, vp, vp, i64, vp, vp, i64, i64, i64, i64, u32, i64, ctypes.c_int, vp,
            logits_t, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.gspn_propagate_backward_dirs_ws.restype = ctypes.c_int
        L.gspn_backward_workspace_bytes_dirs.argtypes = [i64, i64, i64, i64, u32, i64,
                                                         ctypes.c_int]
        L.gspn_backward_workspace_bytes_dirs.restype = ctypes.c_size_t
        outs5_t = ctypes.POINTER(ctypes.c_void_p)
        L.gspn_prologue.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                    vp, outs5_t, vp]
        L.gspn_prologue.restype = ctypes.c_int
        L.gspn_module_ws.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, i64, i64, u32, i64,
                                     ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
        L.gspn_module_ws.restype = ctypes.c_int
        L.gspn_module_workspace_bytes.argtypes = [i64, i64, i64, i64, u32, i64, ctypes.c_int]
        L.gspn_module_workspace_bytes.restype = ctypes.c_size_t
        _lib = L
    return _lib


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return GSPN_F32
    if t.dtype == torch.bfloat16:
        return GSPN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _check(status: int) -> None:
    if status != 0:
        raise GspnError(status, lib().gspn_last_error().decode())


def _check_out(out, shape, dtype, device, what="out"):
    """A caller-supplied output must be a contiguous tensor of the given
    shape and dtype on the inputs' device: the library writes exactly that
    many bytes through its pointer."""
    import torch
    if not isinstance(out, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if out.device != device:
        raise TypeError(f"{what} must be on {device}, not {out.device}")
    if out.dtype != dtype or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{what} must be {dtype} {tuple(shape)}, "
                         f"not {out.dtype} {tuple(out.shape)}")
    if not out.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _check_workspace(ws, device):
    """A caller-supplied workspace must be a contiguous uint8 tensor on the
    inputs' device; the library checks its size and alignment."""
    import torch
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if ws.device != device:
        raise TypeError(f"workspace must be on {device}, not {ws.device}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")


def workspace_bytes(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32) -> int:
    return int(lib().gspn_workspace_bytes(B, C, H, W, dirs, group_rows, dtype))


def plan_name(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32) -> str:
    return lib().gspn_plan_name(B, C, H, W, dirs, group_rows, dtype).decode()


def _check_tensors(x, logits, others):
    """Contiguous GPU tensors of x's dtype; logits may have fewer channels
    (shared by groups of channels). Returns B, C, H, W, logit channels."""
    import torch
    if x.dim() != 4:
        raise ValueError("inputs must be [B, C, H, W]")
    B, C, H, W = x.shape
    cl = logits[0].shape[1] if logits[0].dim() == 4 else -1
    for t in (x,) + tuple(logits) + tuple(others):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.device != x.device:
            raise TypeError("all inputs must be torch tensors on x's GPU device")
        if t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError("inputs must be contiguous tensors of one dtype")
    for t in others:
        if t.shape != x.shape:
            raise ValueError("x, lambda, u (and grad_out) must have one shape")
    for t in logits:
        if tuple(t.shape) != (B, cl, H, W):
            raise ValueError("logits must be [B, Cl, H, W] with Cl dividing C")
    return B, C, H, W, cl


def propagate(x, logits, lam, u, dirs: int = ALL, group_rows: int = 0, out=None,
              workspace=None, stream=None):
    """out = sum_{d in dirs} u * h_d for contiguous [B, C, H, W] device tensors
    of one dtype (float32 or bfloat16). ``logits`` = (l0, l1, l2) for the
    neighbours at orthogonal offsets -1, 0, +1, each [B, C, H, W] or
    [B, Cl, H, W] (shared by groups of C / Cl channels). Work is enqueued on
    ``stream`` (default: torch's current stream of x's device)."""
    import torch
    l0, l1, l2 = logits
    B, C, H, W, cl = _check_tensors(x, (l0, l1, l2), (lam, u))
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, x.shape, x.dtype, x.device)
    _check_workspace(workspace, x.device)
    L = lib()
    need = int(L.gspn_workspace_bytes(B, C, H, W, dirs, group_rows, dt))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lg = (ctypes.c_void_p * 3)(l0.data_ptr(), l1.data_ptr(), l2.data_ptr())
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.gspn_propagate_shared_ws(x.data_ptr(), lg, cl, lam.data_ptr(), u.data_ptr(), B, C,
                                      H, W, dirs, group_rows, dt, out.data_ptr(), ws_ptr, ws_len,
                                      sptr))
    return out


def workspace_bytes_dirs(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32) -> int:
    return int(lib().gspn_workspace_bytes_dirs(B, C, H, W, dirs, group_rows, dtype))


def propagate_dirs(x, logits, lam, u, merge=None, dirs: int = ALL, group_rows: int = 0,
                   out=None, workspace=None, stream=None):
    """Per-direction parameters with a per-channel merger:
    out = sum_{d in dirs} merge[d, c] * u[d] * h_d, where h_d scans x with
    lam[d] and the logits' slice d. ``x`` is a contiguous [B, C, H, W] device
    tensor; ``logits`` = (l0, l1, l2), ``lam`` and ``u`` are contiguous
    [4, B, C, H, W] tensors of x's dtype, slice d for direction d (top->bottom,
    bottom->top, left->right, right->left); ``merge`` is a contiguous float32
    [4, C] device tensor, or None for all ones."""
    import torch
    l0, l1, l2 = logits
    if x.dim() != 4:
        raise ValueError("x must be [B, C, H, W]")
    B, C, H, W = x.shape
    for t in (x, l0, l1, l2, lam, u):
        if not isinstance(t, torch.Tensor) or t.device != x.device or t.device.type != "cuda":
            raise TypeError("all inputs must be torch tensors on x's GPU device")
        if t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError("inputs must be contiguous tensors of one dtype")
    for t in (l0, l1, l2, lam, u):
        if tuple(t.shape) != (4, B, C, H, W):
            raise ValueError("per-direction tensors must be [4, B, C, H, W]")
    mptr = None
    if merge is not None:
        if (merge.dtype != torch.float32 or merge.device != x.device or not merge.is_contiguous()
                or tuple(merge.shape) != (4, C)):
            raise ValueError("merge must be a contiguous float32 [4, C] tensor on x's device")
        mptr = merge.data_ptr()
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, x.shape, x.dtype, x.device)
    _check_workspace(workspace, x.device)
    L = lib()
    need = int(L.gspn_workspace_bytes_dirs(B, C, H, W, dirs, group_rows, dt))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lg = (ctypes.c_void_p * 3)(l0.data_ptr(), l1.data_ptr(), l2.data_ptr())
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.gspn_propagate_dirs_ws(x.data_ptr(), lg, lam.data_ptr(), u.data_ptr(),
                                    B * C * H * W, mptr, B, C, H, W, dirs, group_rows, dt,
                                    out.data_ptr(), ws_ptr, ws_len, sptr))
    return out


PARAM_NAMES = ("l0", "l1", "l2", "lam", "u")


def _check_prologue(x_in, w_r, b_r, w_p, b_p):
    import torch
    if x_in.dim() != 4:
        raise ValueError("x_in must be [B, Cin, H, W]")
    B, Cin, H, W = x_in.shape
    if w_r.dim() != 2 or w_r.shape[1] != Cin:
        raise ValueError("w_reduce must be [C, Cin]")
    C = w_r.shape[0]
    shapes = [(w_r, (C, Cin)), (b_r, (C,)), (w_p, (5 * C, C)), (b_p, (5 * C,))]
    for t in [x_in] + [t for t, _ in shapes]:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.device != x_in.device or t.device.type != "cuda":
            raise TypeError("all prologue tensors must be on x_in's GPU device")
        if t.dtype != x_in.dtype or not t.is_contiguous():
            raise ValueError("prologue tensors must be contiguous and of x_in's dtype")
    for t, shp in shapes:
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"prologue weight of shape {tuple(t.shape)}, expected {shp}")
    return B, Cin, C, H, W


def prologue(x_in, w_reduce, b_reduce, w_params, b_params, outs=None, stream=None) -> dict:
    """The module prologue's 1x1 convolutions: x = w_reduce x_in + b_reduce,
    then l0, l1, l2, lam, u = the five C-row blocks of w_params x + b_params.
    ``x_in`` [B, Cin, H, W]; ``w_reduce`` [C, Cin]; ``w_params`` [5C, C];
    biases [C] / [5C] or None; contiguous device tensors of one dtype. Returns
    {"x", "l0", "l1", "l2", "lam", "u"}, each [B, C, H, W]."""
    import torch
    B, Cin, C, H, W = _check_prologue(x_in, w_reduce, b_reduce, w_params, b_params)
    if outs is None:
        outs = {k: torch.empty((B, C, H, W), dtype=x_in.dtype, device=x_in.device)
                for k in ("x",) + PARAM_NAMES}
    for k in ("x",) + PARAM_NAMES:
        if k not in outs:
            raise ValueError(f"outs is missing {k!r}")
        _check_out(outs[k], (B, C, H, W), x_in.dtype, x_in.device, f"outs[{k!r}]")
    if stream is None:
        stream = torch.cuda.current_stream(x_in.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    po = (ctypes.c_void_p * 5)(*[outs[k].data_ptr() for k in PARAM_NAMES])
    L = lib()
    _check(L.gspn_prologue(x_in.data_ptr(), Cin, w_reduce.data_ptr(),
                           None if b_reduce is None else b_reduce.data_ptr(),
                           w_params.data_ptr(), None if b_params is None else b_params.data_ptr(),
                           B, C, H, W, _dtype_code(x_in), outs["x"].data_ptr(), po, sptr))
    return outs


def module_workspace_bytes(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32) -> int:
    return int(lib().gspn_module_workspace_bytes(B, C, H, W, dirs, group_rows, dtype))


def module(x_in, w_reduce, b_reduce, w_params, b_params, dirs: int = ALL, group_rows: int = 0,
           out=None, workspace=None, stream=None):
    """The GSPN unit: the prologue's convolutions, then the propagation of
    their outputs; returns out = sum_{d in dirs} u * h_d, [B, C, H, W]."""
    import torch
    B, Cin, C, H, W = _check_prologue(x_in, w_reduce, b_reduce, w_params, b_params)
    dt = _dtype_code(x_in)
    if out is None:
        out = torch.empty((B, C, H, W), dtype=x_in.dtype, device=x_in.device)
    _check_out(out, (B, C, H, W), x_in.dtype, x_in.device)
    _check_workspace(workspace, x_in.device)
    L = lib()
    need = int(L.gspn_module_workspace_bytes(B, C, H, W, dirs, group_rows, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x_in.device)
    if stream is None:
        stream = torch.cuda.current_stream(x_in.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _check(L.gspn_module_ws(x_in.data_ptr(), Cin, w_reduce.data_ptr(),
                            None if b_reduce is None else b_reduce.data_ptr(),
                            w_params.data_ptr(), None if b_params is None else b_params.data_ptr(),
                            B, C, H, W, dirs, group_rows, dt, out.data_ptr(),
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            sptr))
    return out


def propagate_alloc(x, logits, lam, u, dirs: int = ALL, group_rows: int = 0, out=None,
                    stream=None):
    """Same as propagate() but lets the library take its workspace with
    hipMallocAsync on the stream (the plain gspn_propagate entry point)."""
    import torch
    l0, l1, l2 = logits
    B, C, H, W, cl = _check_tensors(x, (l0, l1, l2), (lam, u))
    if cl != C:
        raise ValueError("the allocating entry point takes unshared logits")
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, x.shape, x.dtype, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lg = (ctypes.c_void_p * 3)(l0.data_ptr(), l1.data_ptr(), l2.data_ptr())
    _check(lib().gspn_propagate(x.data_ptr(), lg, lam.data_ptr(), u.data_ptr(), B, C, H, W,
                                dirs, group_rows, dt, out.data_ptr(), sptr))
    return out


def noalloc_scratch_bytes() -> int:
    """Size of gspn_propagate_noalloc's per-device scratch array."""
    return int(lib().gspn_noalloc_scratch_bytes())


def propagate_noalloc(x, logits, lam, u, dirs: int = ALL, group_rows: int = 0, out=None,
                      stream=None):
    """Same as propagate() through the entry point that allocates nothing
    (gspn_propagate_noalloc): scratch comes from the library's static
    per-device array, so problems whose workspace exceeds
    noalloc_scratch_bytes() raise GSPN_E_WORKSPACE, and calls that overlap in
    time on one device race. ``out`` must be supplied by callers that cannot
    allocate."""
    import torch
    l0, l1, l2 = logits
    B, C, H, W, cl = _check_tensors(x, (l0, l1, l2), (lam, u))
    if cl != C:
        raise ValueError("the no-allocation entry point takes unshared logits")
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, x.shape, x.dtype, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lg = (ctypes.c_void_p * 3)(l0.data_ptr(), l1.data_ptr(), l2.data_ptr())
    _check(lib().gspn_propagate_noalloc(x.data_ptr(), lg, lam.data_ptr(), u.data_ptr(), B, C, H,
                                        W, dirs, group_rows, dt, out.data_ptr(), sptr))
    return out


def backward_workspace_bytes(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32,
                             logit_channels=None) -> int:
    cl = C if logit_channels is None else logit_channels
    return int(lib().gspn_backward_workspace_bytes_shared(B, C, H, W, cl, dirs, group_rows, dtype))


def backward_plan_name(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32) -> str:
    return lib().gspn_backward_plan_name(B, C, H, W, dirs, group_rows, dtype).decode()


GRAD_NAMES = ("x", "l0", "l1", "l2", "lam", "u")


def backward_workspace_bytes_dirs(B, C, H, W, dirs=ALL, group_rows=0, dtype=GSPN_F32) -> int:
    return int(lib().gspn_backward_workspace_bytes_dirs(B, C, H, W, dirs, group_rows, dtype))


def propagate_backward_dirs(x, logits, lam, u, grad_out, merge=None, dirs: int = ALL,
                            group_rows: int = 0, grads=None, workspace=None, stream=None) -> dict:
    """Gradients of the per-direction layer of propagate_dirs(), given
    ``grad_out`` = dL/dout [B, C, H, W]: a dict with "x" [B, C, H, W]; "l0",
    "l1", "l2", "lam", "u" [4, B, C, H, W] (slice d = direction d, zero
    outside ``dirs``); "merge" float32 [4, C] (the merge weights' gradient;
    of an all-ones merger when ``merge`` is None). ``grads`` may supply the
    tensors."""
    import torch
    l0, l1, l2 = logits
    if x.dim() != 4:
        raise ValueError("x must be [B, C, H, W]")
    B, C, H, W = x.shape
    for t in (x, l0, l1, l2, lam, u, grad_out):
        if not isinstance(t, torch.Tensor) or t.device != x.device or t.device.type != "cuda":
            raise TypeError("all inputs must be torch tensors on x's GPU device")
        if t.dtype != x.dtype or not t.is_contiguous():
            raise ValueError("inputs must be contiguous tensors of one dtype")
    for t in (l0, l1, l2, lam, u):
        if tuple(t.shape) != (4, B, C, H, W):
            raise ValueError("per-direction tensors must be [4, B, C, H, W]")
    if tuple(grad_out.shape) != (B, C, H, W):
        raise ValueError("grad_out must be [B, C, H, W]")
    mptr = None
    if merge is not None:
        if (merge.dtype != torch.float32 or merge.device != x.device or not merge.is_contiguous()
                or tuple(merge.shape) != (4, C)):
            raise ValueError("merge must be a contiguous float32 [4, C] tensor on x's device")
        mptr = merge.data_ptr()
    dt = _dtype_code(x)
    if grads is None:
        grads = {"x": torch.empty_like(x)}
        for k in ("l0", "l1", "l2", "lam", "u"):
            grads[k] = torch.empty_like(lam)
        grads["merge"] = torch.empty((4, C), dtype=torch.float32, device=x.device)
    for k in ("x", "l0", "l1", "l2", "lam", "u"):
        t = grads[k]
        like = x if k == "x" else lam
        if t.shape != like.shape or t.dtype != x.dtype or not t.is_contiguous() or t.device != x.device:
            raise ValueError("gradient tensors must match the inputs")
    gm = grads.get("merge")
    if gm is not None and (gm.dtype != torch.float32 or tuple(gm.shape) != (4, C)
                           or not gm.is_contiguous() or gm.device != x.device):
        raise ValueError("the merge gradient must be a contiguous float32 [4, C] tensor")
    _check_workspace(workspace, x.device)
    L = lib()
    need = int(L.gspn_backward_workspace_bytes_dirs(B, C, H, W, dirs, group_rows, dt))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lg = (ctypes.c_void_p * 3)(l0.data_ptr(), l1.data_ptr(), l2.data_ptr())
    dlg = (ctypes.c_void_p * 3)(grads["l0"].data_ptr(), grads["l1"].data_ptr(),
                                grads["l2"].data_ptr())
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.gspn_propagate_backward_dirs_ws(
        x.data_ptr(), lg, lam.data_ptr(), u.data_ptr(), B * C * H * W, mptr, grad_out.data_ptr(),
        B, C, H, W, dirs, group_rows, dt, grads["x"].data_ptr(), dlg, grads["lam"].data_ptr(),
        grads["u"].data_ptr(), gm.data_ptr() if gm is not None else None, ws_ptr, ws_len, sptr))
    return grads


def propagate_backward(x, logits, lam, u, grad_out, dirs: int = ALL, group_rows: int = 0,
                       grads=None, workspace=None, stream=None, alloc: bool = False) -> dict:
    """Gradients of a loss with respect to every input of propagate(), given
    ``grad_out`` = dL/dout: a dict ``{"x", "l0", "l1", "l2", "lam", "u"}`` of
    tensors shaped and typed like the inputs (``grads`` may supply them).
    ``alloc=True`` lets the library take its own workspace (the plain
    gspn_propagate_backward entry point)."""
    import torch
    l0, l1, l2 = logits
    B, C, H, W, cl = _check_tensors(x, (l0, l1, l2), (lam, u, grad_out))
    dt = _dtype_code(x)
    if grads is None:
        grads = {k: torch.empty_like(l0 if k in ("l0", "l1", "l2") else x) for k in GRAD_NAMES}
    for k in GRAD_NAMES:
        t = grads[k]
        like = l0 if k in ("l0", "l1", "l2") else x
        if t.shape != like.shape or t.dtype != x.dtype or not t.is_contiguous() or t.device != x.device:
            raise ValueError("gradient tensors must match the inputs")
    L = lib()
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    lg = (ctypes.c_void_p * 3)(l0.data_ptr(), l1.data_ptr(), l2.data_ptr())
    dlg = (ctypes.c_void_p * 3)(grads["l0"].data_ptr(), grads["l1"].data_ptr(),
                                grads["l2"].data_ptr())
    args = (x.data_ptr(), lg, lam.data_ptr(), u.data_ptr(), grad_out.data_ptr(), B, C, H, W,
            dirs, group_rows, dt, grads["x"].data_ptr(), dlg, grads["lam"].data_ptr(),
            grads["u"].data_ptr())
    if alloc:
        if cl != C:
            raise ValueError("the allocating backward entry point takes unshared logits")
        _check(L.gspn_propagate_backward(*args, sptr))
        return grads
    _check_workspace(workspace, x.device)
    need = int(L.gspn_backward_workspace_bytes_shared(B, C, H, W, cl, dirs, group_rows, dt))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.gspn_propagate_backward_shared_ws(args[0], args[1], cl, *args[2:], ws_ptr, ws_len,
                                               sptr))
    return grads
