"""fp64 CPU oracle of the GSPN 2D line-scan propagation.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the product package
(``linear_spatial_propagation_line_amd``) never does, and shares no code with
it. The arithmetic lives in ``gspn_oracle.c`` (plain C, fp64); this module only
builds it with gcc and marshals numpy arrays.

What it computes, and the readings of open points, are documented at the top of
``gspn_oracle.c`` (CSDN page on GSPN, sections 方法, 稳定性-上下文条件 and
如何设计一个高效的传播层; aitntnews page, section 传播层的关键实现).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gspn_oracle.c")
_LIB = os.path.join(_HERE, "libgspn_oracle.so")

ORC_F64, ORC_F32, ORC_BF16 = 0, 1, 2
T2B, B2T, L2R, R2L = 1, 2, 4, 8

_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, no fast-math). Returns the .so path."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, src, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building if needed) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    f = lib.gspn_oracle_propagate
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    f.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                  ctypes.c_uint32, i64, vp, ctypes.c_int]
    f.restype = ctypes.c_int
    if hasattr(lib, "gspn_oracle_propagate_shared"):
        f2 = lib.gspn_oracle_propagate_shared
        f2.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                       ctypes.c_uint32, i64, vp, ctypes.c_int]
        f2.restype = ctypes.c_int
        b2 = lib.gspn_oracle_backward_shared
        b2.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                       ctypes.c_uint32, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        b2.restype = ctypes.c_int
    if hasattr(lib, "gspn_oracle_propagate_dirs"):
        f3 = lib.gspn_oracle_propagate_dirs
        f3.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, vp,
                       ctypes.c_uint32, i64, vp, ctypes.c_int]
        f3.restype = ctypes.c_int
    if hasattr(lib, "gspn_oracle_backward_dirs"):
        b3 = lib.gspn_oracle_backward_dirs
        b3.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, vp,
                       ctypes.c_uint32, i64, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        b3.restype = ctypes.c_int
    if hasattr(lib, "gspn_oracle_prologue"):
        f4 = lib.gspn_oracle_prologue
        f4.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp,
                       ctypes.c_int]
        f4.restype = ctypes.c_int
    if hasattr(lib, "gspn_oracle_round"):
        f5 = lib.gspn_oracle_round
        f5.argtypes = [vp, ctypes.c_int, i64, vp]
        f5.restype = ctypes.c_int
    if hasattr(lib, "gspn_oracle_backward"):
        b = lib.gspn_oracle_backward
        b.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                      ctypes.c_uint32, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        b.restype = ctypes.c_int
    return lib


def _as_input(a: np.ndarray, shape) -> tuple[np.ndarray, int]:
    a = np.ascontiguousarray(a)
    if a.shape != tuple(shape):
        raise ValueError(f"shape {a.shape} != {tuple(shape)}")
    if a.dtype == np.float64:
        return a, ORC_F64
    if a.dtype == np.float32:
        return a, ORC_F32
    if a.dtype == np.uint16:      # bf16 bit patterns
        return a, ORC_BF16
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _gather(x, logits, others):
    """Validate shapes and a common dtype; returns (arrays, dtype code, shape,
    logit channel count). Logits may have fewer channels than x (shared)."""
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("inputs must be [B, C, H, W]")
    shape = x.shape
    lg0 = np.asarray(logits[0])
    if lg0.ndim != 4:
        raise ValueError("logits must be [B, Cl, H, W]")
    cl = lg0.shape[1]
    lshape = (shape[0], cl, shape[2], shape[3])
    arrs, dts = [], set()
    for a, shp in [(x, shape)] + [(lg, lshape) for lg in logits] + [(o, shape) for o in others]:
        a2, dt = _as_input(np.asarray(a), shp)
        arrs.append(a2)
        dts.add(dt)
    if len(dts) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    return arrs, dts.pop(), shape, cl


def propagate(x, l0, l1, l2, lam, u, dirs: int = 15, group_rows: int = 0,
              nthreads: int | None = None, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """y = sum over directions in ``dirs`` of u * h_d, as float64 [B, C, H, W].

    Inputs are numpy arrays of one dtype: float64, float32, or uint16 holding
    bf16 bit patterns. ``l0, l1, l2`` are the logits of the neighbours at
    orthogonal offsets -1, 0, +1: [B, C, H, W], or [B, Cl, H, W] with Cl
    dividing C for logits shared by groups of C / Cl channels (channel c uses
    logit channel c // (C // Cl)).
    """
    arrs, dt, shape, cl = _gather(x, (l0, l1, l2), (lam, u))
    out = np.empty(shape, dtype=np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    L = lib if lib is not None else load()
    B, C, H, W = shape
    rc = L.gspn_oracle_propagate_shared(*[a.ctypes.data for a in arrs], dt, B, C, H, W, cl,
                                        int(dirs), int(group_rows), out.ctypes.data,
                                        int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def propagate_dirs(x, l0, l1, l2, lam, u, merge=None, dirs: int = 15, group_rows: int = 0,
                   nthreads: int | None = None, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Per-direction parameters with a per-channel merger, as float64
    [B, C, H, W]: y = sum over d in ``dirs`` of merge[d, c] * u[d] * h_d, where
    h_d is direction d's scan of x with lam[d] and logits l0[d], l1[d], l2[d].

    ``x`` is [B, C, H, W]; ``l0, l1, l2, lam, u`` are [4, B, C, H, W] (one slice
    per direction: top->bottom, bottom->top, left->right, right->left), all of
    one dtype as in ``propagate``. ``merge`` is [4, C] (converted to float64)
    or None for all ones.
    """
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("x must be [B, C, H, W]")
    shape = x.shape
    dshape = (4,) + tuple(shape)
    arrs, dts = [], set()
    for a, shp in [(x, shape)] + [(t, dshape) for t in (l0, l1, l2, lam, u)]:
        a2, dt = _as_input(np.asarray(a), shp)
        arrs.append(a2)
        dts.add(dt)
    if len(dts) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    dt = dts.pop()
    B, C, H, W = shape
    m = None
    if merge is not None:
        m = np.ascontiguousarray(merge, dtype=np.float64)
        if m.shape != (4, C):
            raise ValueError(f"merge must be [4, {C}]")
    out = np.empty(shape, dtype=np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    L = lib if lib is not None else load()
    rc = L.gspn_oracle_propagate_dirs(*[a.ctypes.data for a in arrs], dt, B, C, H, W,
                                      B * C * H * W, None if m is None else m.ctypes.data,
                                      int(dirs), int(group_rows), out.ctypes.data,
                                      int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def _gather_dirs(x, params, merge):
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("x must be [B, C, H, W]")
    shape = x.shape
    dshape = (4,) + tuple(shape)
    arrs, dts = [], set()
    for a, shp in [(x, shape)] + [(t, dshape) for t in params]:
        a2, dt = _as_input(np.asarray(a), shp)
        arrs.append(a2)
        dts.add(dt)
    if len(dts) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    m = None
    if merge is not None:
        m = np.ascontiguousarray(merge, dtype=np.float64)
        if m.shape != (4, shape[1]):
            raise ValueError(f"merge must be [4, {shape[1]}]")
    return arrs, dts.pop(), shape, m


def backward_dirs(x, l0, l1, l2, lam, u, gy, merge=None, dirs: int = 15, group_rows: int = 0,
                  nthreads: int | None = None, lib: ctypes.CDLL | None = None) -> dict:
    """Gradients of the per-direction layer of ``propagate_dirs`` (CSDN page
    on GSPN, section 反向传播; reading R15 in gspn_oracle.c), given ``gy`` =
    dL/dy [B, C, H, W] in the inputs' dtype. Returns float64 arrays: "x"
    [B, C, H, W]; "l0", "l1", "l2", "lam", "u" [4, B, C, H, W] (slice d =
    direction d, zero outside ``dirs``); "merge" [4, C], the gradient of the
    merge weights (of an all-ones merger when ``merge`` is None)."""
    x = np.asarray(x)
    arrs, dt, shape, m = _gather_dirs(x, (l0, l1, l2, lam, u), merge)
    g2, gdt = _as_input(np.asarray(gy), shape)
    if gdt != dt:
        raise TypeError("gy must have the inputs' dtype")
    B, C, H, W = shape
    dshape = (4,) + tuple(shape)
    outs = {"x": np.empty(shape, dtype=np.float64)}
    for k in ("l0", "l1", "l2", "lam", "u"):
        outs[k] = np.empty(dshape, dtype=np.float64)
    outs["merge"] = np.empty((4, C), dtype=np.float64)
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    L = lib if lib is not None else load()
    rc = L.gspn_oracle_backward_dirs(*[a.ctypes.data for a in arrs], g2.ctypes.data, dt,
                                     B, C, H, W, B * C * H * W,
                                     None if m is None else m.ctypes.data, int(dirs),
                                     int(group_rows),
                                     *[outs[k].ctypes.data for k in ("x", "l0", "l1", "l2",
                                                                     "lam", "u", "merge")],
                                     int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return outs


PARAM_NAMES = ("l0", "l1", "l2", "lam", "u")


def prologue(x_in, w_r, b_r, w_p, b_p, nthreads: int | None = None,
             lib: ctypes.CDLL | None = None) -> dict:
    """The module prologue's 1x1 convolutions (reading R16 in gspn_oracle.c).

    ``x_in`` [B, Cin, H, W]; ``w_r`` [C, Cin]; ``b_r`` [C] or None; ``w_p``
    [5C, C] (output channel t * C + c for t = l0, l1, l2, lam, u); ``b_p``
    [5C] or None; all of one dtype as in ``propagate``. Returns float64
    arrays: "x" (exact), "xr" (x rounded to the storage type) and "l0", "l1",
    "l2", "lam", "u", each [B, C, H, W], computed from "xr"."""
    x_in = np.asarray(x_in)
    if x_in.ndim != 4:
        raise ValueError("x_in must be [B, Cin, H, W]")
    B, Cin, H, W = x_in.shape
    C = np.asarray(w_r).shape[0]
    arrs, dts = [], set()
    for a, shp in ((x_in, (B, Cin, H, W)), (w_r, (C, Cin)), (b_r, (C,)), (w_p, (5 * C, C)),
                   (b_p, (5 * C,))):
        if a is None:
            arrs.append(None)
            continue
        a2, dt = _as_input(np.asarray(a), shp)
        arrs.append(a2)
        dts.add(dt)
    if len(dts) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    dt = dts.pop()
    x = np.empty((B, C, H, W))
    xr = np.empty((B, C, H, W))
    p = np.empty((5, B, C, H, W))
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    L = lib if lib is not None else load()
    ptr = [None if a is None else a.ctypes.data for a in arrs]
    rc = L.gspn_oracle_prologue(ptr[0], dt, B, Cin, C, H, W, ptr[1], ptr[2], ptr[3], ptr[4],
                                x.ctypes.data, xr.ctypes.data, p.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out = {"x": x, "xr": xr}
    for t, name in enumerate(PARAM_NAMES):
        out[name] = p[t]
    return out


def round_to(a, dtype: str, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """float64 values rounded to "f32" or "bf16" (nearest, ties to even), as
    float64; the rounding the prologue applies to x."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty_like(a)
    dt = {"f64": ORC_F64, "f32": ORC_F32, "bf16": ORC_BF16}[dtype]
    L = lib if lib is not None else load()
    if L.gspn_oracle_round(a.ctypes.data, dt, a.size, out.ctypes.data) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


GRAD_NAMES = ("x", "l0", "l1", "l2", "lam", "u")


def backward(x, l0, l1, l2, lam, u, gy, dirs: int = 15, group_rows: int = 0,
             nthreads: int | None = None, lib: ctypes.CDLL | None = None) -> dict:
    """Gradients of a loss L with respect to every input of ``propagate``,
    given ``gy`` = dL/dy (same shape and dtype as x). Returns a dict
    ``{"x", "l0", "l1", "l2", "lam", "u"}`` of float64 arrays shaped like the
    corresponding inputs (CSDN page on GSPN, section 反向传播; the logit
    gradients are taken through the sigmoid and the normalisation, and a
    shared logit's gradient is the sum over the channels that use it)."""
    arrs, dt, shape, cl = _gather(x, (l0, l1, l2), (lam, u, gy))
    # argument order of the C function: x, l0, l1, l2, lam, u, gy
    B, C, H, W = shape
    lshape = (B, cl, H, W)
    outs = {k: np.empty(lshape if k in ("l0", "l1", "l2") else shape, dtype=np.float64)
            for k in GRAD_NAMES}
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    L = lib if lib is not None else load()
    rc = L.gspn_oracle_backward_shared(*[a.ctypes.data for a in arrs], dt, B, C, H, W, cl,
                                       int(dirs), int(group_rows),
                                       *[outs[k].ctypes.data for k in GRAD_NAMES],
                                       int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return outs
