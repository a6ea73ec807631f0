#!/usr/bin/env python3
"""Throughput of the GSPN 2D line-scan propagation on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1] [--backward]

One step = one full propagation (all selected scan directions, fused merge)
over one batch of seeded synthetic inputs already resident in HBM. Prints ONE
JSON line:
  value     elem-steps/s = B*C*H*W*dirs*K / (time of K steps)
  roofline  the launches of one step (one kernel, or the three-kernel
            pipeline of large planes): compulsory bytes Q_min = 7 s per pixel
            / their time (HIP events recorded around each launch on its
            stream inside the timed region; the step time for a pipeline
            whose launches overlap on two streams), against the 8 TB/s HBM
            peak; traffic = HBM bytes per step from the committed rocprofv3
            counter summary when it was taken on the current kernel sources
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
            workload on this host's cores (rank 0, N = 1 only)
With --backward a step is one backward pass instead (gradients of x, lambda,
the three logits and u for a seeded dL/dout), with Q_min = 13 s per pixel
(seven tensors read, six written). Per-direction workloads (own lambda,
logits and u per direction, per-channel merge weights) have
Q_min = (2 + 5 * dirs) s per pixel: x, each direction's five tensors, out.
Module workloads (*_mod) time the whole unit, the prologue's 1x1
convolutions and the propagation, with Q_min = (Cin / C + 1) s per pixel
(x_in read, out written); with --prologue a step is the prologue alone and
the metric is its TFLOP/s, the roofline bound being MFMA or HBM, whichever
the kernel's flops and bytes make the longer.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GSPN propagated elem-steps/s (B·C·H·W·dirs) + achieved HBM GB/s vs peak"
METRIC_BWD = "GSPN backward elem-steps/s (B·C·H·W·dirs) + achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
METRIC_PRO = "GSPN module prologue (1x1 convolutions on MFMA) TFLOP/s"
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}    # dense, MI355X
DEFAULT_WORKLOAD = "t2i_2048x1024"
CSRC = os.path.join(ROOT, "linear_spatial_propagation_line_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# kernel source of each plan; the counter figures of a plan stay valid while
# these files are unchanged
PLAN_SOURCES = {
    "plane16": ("gspn_plane.hip", "gspn_device.hpp"),
    "plane64": ("gspn_plane.hip", "gspn_device.hpp"),
    "band": ("gspn_band.hip", "gspn_device.hpp"),
    "tpipe": ("gspn_tpipe.hip", "gspn_quad.hpp", "gspn_device.hpp"),
    "stream": ("gspn_stream.hip", "gspn_device.hpp"),
    "tpipe_t": ("gspn_tpipe.hip", "gspn_quad.hpp", "gspn_dirs.hip", "gspn_device.hpp"),
    "large": ("gspn_dirs.hip", "gspn_stream.hip", "gspn_device.hpp"),
    "bwd_plane16": ("gspn_bwd_plane.hip", "gspn_device.hpp"),
    "bwd_plane64": ("gspn_bwd_plane.hip", "gspn_device.hpp"),
    "bwd_stream": ("gspn_bwd_stream.hip", "gspn_device.hpp"),
    "bwd_band": ("gspn_bwd_band.hip", "gspn_device.hpp"),
    "bwd_tpipe": ("gspn_bwd_tpipe.hip", "gspn_quad.hpp", "gspn_device.hpp"),
    "bwd_tpipe_t": ("gspn_bwd_tpipe.hip", "gspn_quad.hpp", "gspn_dirs.hip", "gspn_device.hpp"),
    "bwd_dirs": ("gspn_bwd_stream.hip", "gspn_dirs.hip", "gspn_device.hpp"),
    "dirs": ("gspn_dirs.hip", "gspn_device.hpp"),
    "prologue": ("gspn_prologue.hip", "gspn_mfma.hpp", "gspn_device.hpp"),
    "module": ("gspn_prologue.hip", "gspn_fused.hip", "gspn_mfma.hpp", "gspn_plane.hip",
               "gspn_band.hip", "gspn_tpipe.hip", "gspn_quad.hpp", "gspn_stream.hip",
               "gspn_device.hpp"),
}


def source_digest(plan: str) -> str:
    """sha256 over the kernel sources of `plan`; counter figures are only
    reported when they were taken on exactly these sources."""
    h = hashlib.sha256()
    for name in PLAN_SOURCES[plan]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class Hip:
    """Just the HIP event calls the benchmark needs."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                               ctypes.c_void_p, ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.L.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
        return arr

    def elapsed_ms(self, a, b) -> float:
        self.L.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for e in arr:
            self.L.hipEventDestroy(e)


def design_bytes(kernel: str, planes: int, w, first: bool = True, last: bool = True) -> float:
    """HBM bytes one launch of `kernel` over `planes` planes moves by design
    (every tensor it touches read or written once). `first` / `last`: the
    launch's place among the direction passes of one call (per-direction
    kernels only).

    Per pixel, with s = bytes per stored element:
      plane_kernel16/64, plane_pc_kernel (all directions on chip): x, lambda, l0, l1, l2, u
          read once, out written once -> 7 s
      stream_kernel (one launch per direction, fp32 accumulator between
          them): 5 s inputs + 4 (accumulator read or write, counted once);
          the u read / out write of the last direction are not included
      band_kernel (local groups; vertical phase, then horizontal phase that
          reads the plane again): 2 * 5 s inputs + s (u) + s (out)
      tpipe (column-major copy = lambda*x in fp32 + 3 logits):
          tp_vfwd  5 s inputs + (4 + 3 s) copy write + 4/8 checkpoints
          tp_hpair 2 (4 + 3 s) copy reads + 2 * 4/4 checkpoints + 4 sum write
          tp_vbwd  5 s inputs + 4/8 checkpoints + 4 sum read + s (u) + s (out)
          (planes wider than 1024 take a checkpoint every 4 rows: 4/4)
          (shared logits, Cl < C: the logit part of the copy is 3 s Cl/C, made
          by tp_lgcopy over the B * Cl logit planes: 6 s per logit pixel)
    Backward pass:
      bplane_kernel16/64: x, lambda, l0, l1, l2, u, grad_out read once, six
          gradients written -> 13 s (the second read of five inputs in the
          gradient phase comes from L2)
      bwd_fwd  5 s inputs + 4 state write + 4 running sum of h
      bwd_adj  5 s (u, grad_out, logits) + 4 state read + 16 accumulator
          write + 16 accumulator read (a middle direction; approximate)
      bwd_transpose  seven inputs read and written (2 * 7 s), or, over 5x the
          planes, the fp32 accumulators (2 * 4)
      bwd_finish  5 * 4 accumulators + 3 s (x, lambda, grad_out) + 6 s out
      bwd_reduce_logits (shared logits): three fp32 per-channel gradients
          read, three shared gradients written (Cl / C of a tensor each)
      bband_kernel (local groups): seven inputs read in the vertical and again
          in the horizontal rounds, five fp32 partial sums written and read
          back, six gradients written -> 20 s + 40
      backward pipeline for large planes (states and error terms of the first
      sweep of an axis stored as fp32 pairs, 8 bytes per pixel; the
      column-major copy = lambda x and u gy in fp32 + 3 logits):
          bt_vA  7 s inputs + 8 states + (8 + 3 s) copy write
          bt_hA  (8 + 3 s) copy read + 8 states
          bt_hB  (8 + 3 s) copy read + 8 states read + 20 horizontal parts
          bt_vB  7 s inputs + 8 states read + 20 horizontal parts + 6 s out
          (no horizontal direction: no copy, no parts, no bt_hA / bt_hB)
      backward of the per-direction layer (each direction a single-direction
      bwd_fwd / bwd_adj pair on its own tensors, see bwd_dirs_path_bytes for
      the whole path):
          bwd_dirs_zero  one gradient slice of an unselected direction (s)
          bwd_dirs_store_dx  the fp32 sum read, dx written (4 + s)
          bwd_dirs_tr  one tensor read and written transposed (2 s), counted
          per plane and tensor
          bwd_dirs_tr_acc  the transposed fp32 sum of dx read and written
          row-major (8)
          bwd_dirs_merge  the fp64 partials that bwd_adj leaves, 4 per plane
          (8 bytes each; the products u gy h are summed inside bwd_adj,
          which reads all three anyway)
    Per-direction parameters, planes up to 64 x 64 (one wavefront per plane,
    the four directions in turn):
      dir_plane  x read once, each selected direction's five tensors read once,
          out written once: (2 + 5 dirs) s
    Per-direction parameters, larger planes (one pass per direction;
    horizontal directions run over transposed copies):
      dir_vert  x and the direction's lambda, l0, l1, l2, u read (6 s), the
          fp32 accumulator read unless first (4), then the accumulator
          written (4) or, by the last pass, out (s)
      dir_tr_in  one tensor read and written transposed (2 s), counted per
          plane and tensor
      dir_tr_acc  the fp32 sum of the horizontal passes read (4) and written
          back row-major (4), or as out (s) when no vertical direction follows
    Module prologue (counted per pixel of B images: `planes` is B here):
      prologue_reduce  x_in read (Cin s), x written (C s)
      prologue_params  x read (C s), five parameter tensors written (5 C s)
      tp_t_in / tp_t_out, btp_t_in / btp_t_out  the forward and backward
          pipelines on transposed copies: one tensor read and written
          transposed (2 s), counted per plane and tensor
      fused_unit (small planes: the parameter product fused with the scan,
          counted per pixel of the B * C planes): x read (s), out written (s);
          the parameters never leave the chip
      (the weights, read once from HBM, are left out)
    """
    s = 4 if w.dtype == "f32" else 2
    px = planes * w.H * w.W
    hz = bool(w.dirs & 12)
    sh = w.cl / w.C   # shared logits: the logit copy is made once per logit plane
    ckv = (4 / 4 if w.W > 1024 else 4 / 8) if w.dirs & 1 else 0   # vertical checkpoints
    per = {
        "plane_kernel16": 7 * s,
        "plane_kernel64": 7 * s,
        "plane_pc_kernel": 7 * s,
        "stream_kernel": 5 * s + 4,
        "band_kernel": 12 * s,
        "tp_vfwd": 5 * s + (4 + 3 * s * sh if hz else 0) + ckv,
        "tp_hpair": 2 * (4 + 3 * s * sh) + 2.0 + 4,
        "tp_lgcopy": 6 * s * (w.B * w.C) / max(planes, 1) * sh,
        "tp_vbwd": 5 * s + ckv + (4 if hz else 0) + 2 * s,
        "bplane_kernel16": 13 * s,
        "bplane_kernel64": 13 * s,
        "bwd_fwd": 5 * s + 8,
        "bwd_adj": 5 * s + 4 + 32,
        "bwd_transpose": 2 * 7 * s if planes == w.B * w.C else 2 * 4,
        "bwd_finish": 20 + 9 * s,
        "bband_kernel": 20 * s + 40,
        "bwd_dirs_zero": s,
        "bwd_dirs_store_dx": 4 + s,
        "bwd_dirs_tr": 2 * s,
        "bwd_dirs_tr_acc": 8,
        "bwd_dirs_merge": 4 * 8 / (w.H * w.W),
        "bt_vA": 7 * s + 8 + (8 + 3 * s if hz else 0),
        "bt_hA": 8 + 3 * s + 8,
        "bt_hB": 8 + 3 * s + 8 + 20,
        "bt_vB": 7 * s + 8 + (20 if hz else 0) + 6 * s,
        "bwd_reduce_logits": 12 + 3 * s * w.cl / w.C,
        "dir_plane": (2 + 5 * w.ndirs) * s,
        "dir_vert": 6 * s + (0 if first else 4) + (s if last else 4),
        "dir_tr_in": 2 * s,
        "dir_tr_acc": 4 + (4 if w.dirs & 3 else s),
        "prologue_reduce": (w.prologue_cin + w.C) * s,
        "prologue_params": 6 * w.C * s,
        "fused_unit": 2 * s,
        "tp_t_in": 2 * s,
        "tp_t_out": 2 * s,
        "btp_t_in": 2 * s,
        "btp_t_out": 2 * s,
    }[kernel]
    return per * px


def bwd_dirs_path_bytes(w) -> float:
    """Design bytes per pixel of the per-direction backward: x and grad_out
    transposed (2 * 2 s) and, per horizontal direction, its five tensors in
    and its five gradients back (2 * 10 s), the fp32 sum of dx back (8); per
    direction the forward scan (5 s in, 4 states out), the reverse scan (u,
    grad_out, three logits, x and lambda read: 7 s; states 4; the dx sum read
    and written: 8; five gradients written: 5 s); the merge gradients come
    out of the reverse scan, whose per-plane partials are too few to count."""
    s = 4 if w.dtype == "f32" else 2
    nh = bin(w.dirs & 12).count("1")
    per_dir = (5 * s + 4) + (12 * s + 12)
    return (4 * s if nh else 0) + nh * (20 * s) + (8 if nh else 0) + w.ndirs * per_dir


def qmin_per_pixel(w, bwd: bool) -> float:
    """Compulsory HBM bytes per pixel: x, lambda, u (and grad_out) read once,
    out (or the gradients) written once, plus the logits (and their
    gradients) at Cl / C of a tensor each when they are shared. Per-direction
    parameters: x, each selected direction's lambda, l0, l1, l2 and u read
    once, out written once; backward: x, grad_out and the directions' five
    tensors read, dx and the directions' five gradients written."""
    s = 4 if w.dtype == "f32" else 2
    if w.per_direction:
        if bwd:
            return (3 + 10 * w.ndirs) * s
        return (2 + 5 * w.ndirs) * s
    if w.prologue_cin:
        if bwd:
            raise ValueError("no backward pass for the module prologue")
        return (w.prologue_cin / w.C + 1) * s
    share = w.cl / w.C
    return (7 + 6 * share) * s if bwd else (4 + 3 * share) * s


def input_sets(w, bwd: bool) -> int:
    """Input sets the timed loop rotates through: small problems use several
    so that it does not run out of the 256 MB last-level cache."""
    set_bytes = int(qmin_per_pixel(w, bwd) * w.pixels)
    return int(max(1, min(8, -(-1024 ** 3 // set_bytes))))


def counter_traffic(plan: str, workload: str, digest: str):
    """HBM bytes per step (the launches of one step) from
    profiles/<plan>__<workload>__pmc.txt, or None when absent or taken on
    other kernel sources."""
    path = os.path.join(PROFILES, f"{plan}__{workload}__pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_step"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp_dev, w, planes: int, grad_out=None):
    """The oracle as it stands on the first `planes` planes of the same
    device-resident inputs, all host cores (its backward pass when grad_out
    is given). Returns the timing record and (planes, the oracle's result),
    which the caller holds the timed output to."""
    import numpy as np
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))
    planes = max(1, min(planes, w.B * w.C))

    def host(t):
        # planes are contiguous in [B, C, H, W]; take the first `planes` of them
        t = t.reshape(-1, w.H, w.W)[:planes].cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16).reshape(1, planes, w.H, w.W)
        return t.numpy().reshape(1, planes, w.H, w.W)

    # shared logits: whole channel groups, and the logit planes they read
    g = w.C // w.cl
    if g > 1 and planes > g:
        planes = planes // g * g

    def host_logits(t):
        nlp = (planes + g - 1) // g
        t = t.reshape(-1, w.H, w.W)[:nlp].cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16).reshape(1, nlp, w.H, w.W)
        return t.numpy().reshape(1, nlp, w.H, w.W)

    def host_dirs(t):
        # [4, B, C, H, W]: the first `planes` planes of every direction
        t = t.reshape(4, -1, w.H, w.W)[:, :planes].cpu().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16).numpy().view(np.uint16)
        else:
            t = t.numpy()
        return t.reshape(4, 1, planes, w.H, w.W)

    threads = min(cores, planes)
    if w.per_direction and grad_out is not None:
        merge = inp_dev["merge"].cpu().numpy()[:, np.arange(planes) % w.C]
        args = [host(inp_dev["x"])] + [host_dirs(inp_dev[k]) for k in ("l0", "l1", "l2",
                                                                         "lam", "u")]
        t0 = time.perf_counter()
        ref = oracle.backward_dirs(*args, host(grad_out), merge=merge, dirs=w.dirs,
                                   group_rows=w.group_rows, nthreads=threads)
        dt = time.perf_counter() - t0
        steps = planes * w.H * w.W * w.ndirs
        return {"value": steps / dt, "unit": "elem-steps/s", "cores": threads, "kind": "oracle",
                "sample": f"per-direction backward, first {planes} of {w.B * w.C} planes "
                          f"({w.H}x{w.W}, {w.ndirs} dirs), {steps} elem-steps in {dt:.2f} s"}, \
            (planes, ref)
    if w.per_direction:
        # sample plane p is channel p % C of the merge weights
        merge = inp_dev["merge"].cpu().numpy()[:, np.arange(planes) % w.C]
        args = [host(inp_dev["x"])] + [host_dirs(inp_dev[k]) for k in ("l0", "l1", "l2",
                                                                         "lam", "u")]
        t0 = time.perf_counter()
        ref = oracle.propagate_dirs(*args, merge=merge, dirs=w.dirs, group_rows=w.group_rows,
                                    nthreads=threads)
        dt = time.perf_counter() - t0
        steps = planes * w.H * w.W * w.ndirs
        return {"value": steps / dt, "unit": "elem-steps/s", "cores": threads, "kind": "oracle",
                "sample": f"per-direction, first {planes} of {w.B * w.C} planes ({w.H}x{w.W}, "
                          f"{w.ndirs} dirs), {steps} elem-steps in {dt:.2f} s"}, (planes, ref)
    arrs = [host(inp_dev["x"])] + [host_logits(inp_dev[k]) for k in ("l0", "l1", "l2")] + \
        [host(inp_dev[k]) for k in ("lam", "u")]
    t0 = time.perf_counter()
    if grad_out is None:
        ref = oracle.propagate(*arrs, dirs=w.dirs, group_rows=w.group_rows, nthreads=threads)
    else:
        ref = oracle.backward(*arrs, host(grad_out), dirs=w.dirs, group_rows=w.group_rows,
                              nthreads=threads)
    dt = time.perf_counter() - t0
    steps = planes * w.H * w.W * w.ndirs
    what = "backward " if grad_out is not None else ""
    return {"value": steps / dt, "unit": "elem-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}first {planes} of {w.B * w.C} planes ({w.H}x{w.W}, {w.ndirs} dirs), "
                      f"{steps} elem-steps in {dt:.2f} s"}, (planes, ref)


def timed_output_parity(out, ref, planes: int, w, bwd: bool) -> dict:
    """The timed output's first `planes` planes against the oracle's result
    on them (forward: out; backward: every gradient of the sampled planes,
    the per-direction merge-weight gradient aside, which sums over every
    plane)."""
    import numpy as np

    def host(t, lead=()):
        return t.detach().float().reshape(*lead, -1, w.H, w.W).cpu().numpy()

    if not bwd:
        got = host(out)[:planes]
        return parity_of_sample(got, ref.reshape(-1, w.H, w.W)[:planes], w.dtype)
    worst = {"planes": planes, "scaled_error": 0.0, "ok": True}
    for k in ("x", "l0", "l1", "l2", "lam", "u"):
        o = np.asarray(ref[k])
        if w.per_direction and k != "x":
            gk = host(out[k], (4,))[:, :planes].reshape(-1, w.H, w.W)
            o = o.reshape(4, -1, w.H, w.W)[:, :planes].reshape(-1, w.H, w.W)
        else:
            n = o.reshape(-1, w.H, w.W).shape[0]
            gk = host(out[k])[:n]
            o = o.reshape(-1, w.H, w.W)
        p = parity_of_sample(gk, o, w.dtype)
        worst["rtol"] = p["rtol"]
        worst[k] = p["scaled_error"]
        worst["scaled_error"] = max(worst["scaled_error"], p["scaled_error"])
        worst["ok"] = worst["ok"] and p["ok"]
    return worst


def prologue_work(w, B=None, H=None):
    """(flops, algorithmic bytes) of the prologue: two products over B*H*W
    pixels, C x Cin then 5C x C, and x_in read, x and five parameter
    tensors written, the weights and biases read once."""
    s = 4 if w.dtype == "f32" else 2
    B = w.B if B is None else B
    H = w.H if H is None else H
    px = B * H * w.W
    cin, c = w.prologue_cin, w.C
    flops = 2.0 * px * c * (cin + 5 * c)
    nbytes = (px * (cin + 6 * c) + c * cin + 5 * c * c + 6 * c) * s
    return flops, nbytes


def cpu_baseline_module(inp_dev, w, seconds: float, prologue_only: bool):
    """The oracle's prologue (and, for the whole unit, its propagation) on the
    first image's first rows, sized for about `seconds` on all host cores."""
    import numpy as np
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))
    macs_per_row = w.W * w.C * (w.prologue_cin + 5 * w.C)
    rows = int(max(1, min(w.H, seconds * 1.5e8 * cores / macs_per_row)))

    def host(t):
        t = t.cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    x_in = host(inp_dev["x_in"][:1, :, :rows])
    wts = [host(inp_dev[k]) for k in ("w_r", "b_r", "w_p", "b_p")]
    t0 = time.perf_counter()
    pro = oracle.prologue(x_in, *wts, nthreads=cores)
    t_pro = time.perf_counter() - t0
    flops, _ = prologue_work(w, B=1, H=rows)
    sample = f"first image, rows 0..{rows - 1} of {w.H} ({rows}x{w.W} pixels, Cin {w.prologue_cin}, C {w.C})"
    if prologue_only:
        return {"value": flops / t_pro / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"prologue, {sample}, {t_pro:.2f} s"}, None
    p = {k: oracle.round_to(pro[k], w.dtype) for k in ("l0", "l1", "l2", "lam", "u")}
    t0 = time.perf_counter()
    ref = oracle.propagate(pro["xr"], p["l0"], p["l1"], p["l2"], p["lam"], p["u"], dirs=w.dirs,
                           group_rows=w.group_rows, nthreads=cores)
    t_prop = time.perf_counter() - t0
    steps = w.C * rows * w.W * w.ndirs
    res = {"value": steps / (t_pro + t_prop), "unit": "elem-steps/s", "cores": cores,
           "kind": "oracle",
           "sample": f"prologue + propagation, {sample}, {steps} elem-steps in "
                     f"{t_pro:.2f} + {t_prop:.2f} s"}
    # the unit's output of the first image is comparable when the sample
    # holds its whole planes
    return res, (ref if rows == w.H else None)


STREAM_KINDS = ("read", "write", "copy")


def stream_ceiling(torch, L, reps: int = 5, nbytes: int = 4 << 30, variants=None) -> dict:
    """The library's hand-written HBM stream kernels (gspn_bench_stream:
    16-byte accesses, grid-stride, every CU filled) over `nbytes` buffers,
    each variant timed with events over `reps` passes after one warm pass.
    Returns the best rate of each kind in GB/s (copy counts its read and
    its write) and every variant's rate."""
    L.gspn_bench_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.gspn_bench_stream.restype = ctypes.c_int
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    variants = variants or [(k, nt, bpc) for k in range(3) for nt in (0, 1) for bpc in (1, 2, 4, 8)]
    res = {"bytes": nbytes, "variants": {}}
    for kind, nt, bpc in variants:
        def run():
            rc = L.gspn_bench_stream(kind, nt, src.data_ptr(), dst.data_ptr(), nbytes, bpc,
                                     stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"gspn_bench_stream returned {rc}")
        run()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        moved = nbytes * (2 if kind == 2 else 1)
        gbs = moved / (ms * 1e-3) / 1e9
        name = STREAM_KINDS[kind]
        res["variants"][f"{name}{'_nt' if nt else ''}_b{bpc}"] = round(gbs, 1)
        res[f"{name}_gbs"] = round(max(res.get(f"{name}_gbs", 0.0), gbs), 1)
    del src, dst
    torch.cuda.empty_cache()
    return res


def handshake_latency(torch, L, rounds: int = 20000) -> dict:
    """Round trips of a flag between two workgroups through device memory
    (gspn_bench_handshake), for partner workgroups at several distances in
    the dispatch order (workgroups are dealt to the XCDs in turn, so 8 apart
    is the same XCD on an 8-XCD part). Microseconds per round trip."""
    L.gspn_bench_handshake.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    L.gspn_bench_handshake.restype = ctypes.c_int
    L.gspn_bench_wall_clock_khz.restype = ctypes.c_int
    khz = L.gspn_bench_wall_clock_khz()
    flags = torch.zeros(512, dtype=torch.uint8, device="cuda")
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    abort = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    stream = torch.cuda.current_stream()
    res = {"wall_clock_khz": khz, "rounds": rounds}
    for partner in (1, 8, 16, 64):
        flags.zero_()
        out.zero_()
        rc = L.gspn_bench_handshake(flags.data_ptr(), abort.data_ptr(), rounds, 1 << 20, partner,
                                    out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gspn_bench_handshake returned {rc}")
        torch.cuda.synchronize()
        ticks, missed, polls, missed_b = (int(v) for v in out.cpu())
        res[f"partner_{partner}"] = {
            "us_per_round_trip": ticks / max(khz, 1) * 1e3 / rounds if khz else None,
            "polls_per_round_trip": polls / rounds, "gave_up": missed + missed_b}
    return res


def calibrate(torch, reps: int) -> int:
    """The hand-written read / write / copy stream kernels on 4 GiB buffers,
    torch's own copy and sum for comparison, and the cross-workgroup
    handshake latency; one JSON line."""
    import linear_spatial_propagation_line_amd as g
    res = {"stream_kernels": stream_ceiling(torch, g.lib(), reps=max(reps, 3)),
           "handshake": handshake_latency(torch, g.lib())}
    n = 1 << 30                      # float32 elements = 4 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for name, fn, nbytes in (("torch_copy", lambda: dst.copy_(src), 8 * n),
                             ("torch_sum", lambda: src.sum(), 4 * n)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"{name}_gbs"] = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps(res), flush=True)
    return 0


def strip_prototype(torch, steps: int) -> int:
    """The other schedule for large planes, measured: the top->bottom scan
    with each 2048 x 1024 plane split over 32 one-wavefront workgroups that
    exchange halo states through device memory every K rows
    (gspn_bench_strip_t2b), at several slab sizes (planes in flight), against
    the library's own top->bottom propagation (one workgroup per plane) on the
    same inputs. Every output is compared with the library's; one JSON line."""
    import linear_spatial_propagation_line_amd as g
    from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_inputs
    L = g.lib()
    L.gspn_bench_strip_work_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.gspn_bench_strip_work_bytes.restype = ctypes.c_size_t
    L.gspn_bench_strip_fail_offset.argtypes = [ctypes.c_int, ctypes.c_int]
    L.gspn_bench_strip_fail_offset.restype = ctypes.c_size_t
    L.gspn_bench_strip_t2b.argtypes = [ctypes.c_void_p] * 2 + [ctypes.POINTER(ctypes.c_void_p)] + \
        [ctypes.c_void_p] * 2 + [ctypes.c_int64] + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.gspn_bench_strip_t2b.restype = ctypes.c_int
    w = WORKLOADS["t2i_2048x1024"]
    d = make_inputs(w, device="cuda")
    B, C, H, W = d["x"].shape
    planes = B * C
    lg = (ctypes.c_void_p * 3)(*(d[k].data_ptr() for k in ("l0", "l1", "l2")))
    stream = torch.cuda.current_stream()
    abort = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    steps = max(steps, 2)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ref = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], dirs=g.T2B)
    lib_ms = timed(lambda: g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                       dirs=g.T2B, out=ref))
    res = {"workload": w.name, "planes": planes, "H": H, "W": W, "direction": "top->bottom",
           "library_ms": lib_ms, "library_plan": g.plan_name(B, C, H, W, g.T2B, 0, 1),
           "prototype": []}
    out = torch.empty_like(ref)
    S = 32
    for K in (16, 8):
        for pf in (8, 32, 64, 128, 256):
            nbytes = L.gspn_bench_strip_work_bytes(S, K, pf)
            work = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device="cuda")
            wp = (work.data_ptr() + 255) // 256 * 256
            fail_at = L.gspn_bench_strip_fail_offset(S, pf)

            def run():
                work.zero_()
                rc = L.gspn_bench_strip_t2b(d["x"].data_ptr(), d["lam"].data_ptr(), lg,
                                            d["u"].data_ptr(), out.data_ptr(), planes, H, W, S, K,
                                            pf, wp, nbytes, abort.data_ptr(), 1 << 20,
                                            stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"gspn_bench_strip_t2b returned {rc}")
            print(f"[strip] K={K} pf={pf}", flush=True)
            ms = timed(run)
            fail = int(work.view(torch.uint8)[wp - work.data_ptr() + fail_at:][:4].view(torch.int32)[0])
            err = float(((out.float() - ref.float()).abs() /
                         (ref.float().abs() + ref.float().pow(2).mean().sqrt())).max())
            res["prototype"].append({"K": K, "planes_in_flight": pf, "workgroups": pf * S,
                                     "ms": ms, "vs_library": ms / lib_ms, "gave_up": fail,
                                     "scaled_diff_vs_library": err})
    print(json.dumps(res), flush=True)
    return 0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_per_core_rate(seconds: float = 1.0) -> dict:
    """The oracle on one thread over planes of the 56x56 classification
    workload (4 directions, fp32): its per-core rate on this host."""
    import numpy as np
    import torch

    import oracle
    from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS["cls_56x56"]
    planes = max(1, int(seconds * 2.0e7 / (w.H * w.W * w.ndirs)))
    inp = make_inputs(w, seed=4242, B=1, C=planes)
    arrs = [inp[k].numpy() for k in ("x", "l0", "l1", "l2", "lam", "u")]
    t0 = time.perf_counter()
    oracle.propagate(*arrs, dirs=w.dirs, group_rows=w.group_rows, nthreads=1)
    dt = time.perf_counter() - t0
    steps = planes * w.H * w.W * w.ndirs
    del torch, np
    return {"value": steps / dt, "unit": "elem-steps/s", "threads": 1,
            "sample": f"{planes} planes of 56x56 fp32, 4 dirs, {steps} elem-steps in {dt:.2f} s"}


def parity_of_sample(got, ref, dtype: str) -> dict:
    """Scaled error max |g - o| / (|o| + rms(o)) of the timed output's sample
    planes against the oracle's, per plane, with the rms over the sample."""
    import numpy as np
    rtol = 1e-5 if dtype == "f32" else 1e-2
    rms = float(np.sqrt(np.mean([np.mean(r * r) for r in ref]))) if len(ref) else 0.0
    worst = 0.0
    for gp, rp in zip(got, ref):
        err = np.max(np.abs(gp.astype(np.float64) - rp) / (np.abs(rp) + rms + 1e-300))
        worst = max(worst, float(err))
    return {"planes": len(ref), "scaled_error": worst, "rtol": rtol, "ok": bool(worst <= rtol)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="rough wall time of the CPU oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the stream-kernel bandwidth ceiling measured after the timed steps")
    ap.add_argument("--no-step-sample", action="store_true",
                    help="skip the extra sample of >= 50 steps taken for the median and min "
                         "when fewer steps are timed (profiling runs)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (all six gradients) instead of the forward")
    ap.add_argument("--prologue", action="store_true",
                    help="module workloads: time the prologue's 1x1 convolutions alone")
    ap.add_argument("--calibrate", action="store_true",
                    help="time a plain device copy and a read-only reduction of known size "
                         "(the reference points for HBM bandwidth and for counter scaling)")
    ap.add_argument("--strip-prototype", action="store_true",
                    help="time the split-line prototype (top->bottom over strips of 32 "
                         "workgroups per plane) against the library's top->bottom scan")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the propagation shards by independent (b, c) "
              f"planes with no collective, so --gpus {args.gpus} is not run here.",
              file=sys.stderr)
        return 2

    import torch

    if args.strip_prototype:
        return strip_prototype(torch, args.steps)
    if args.calibrate:
        return calibrate(torch, args.steps)

    import linear_spatial_propagation_line_amd as g
    from linear_spatial_propagation_line_amd.inputs import (WORKLOADS, make_grad_out, make_inputs,
                                                            make_prologue_inputs)

    w = WORKLOADS[args.workload]
    bwd = args.backward
    mod = w.prologue_cin > 0
    pro_only = args.prologue
    if bwd and mod:
        print("no backward pass for the module prologue", file=sys.stderr)
        return 2
    if pro_only and not mod:
        print("--prologue needs a module workload (*_mod)", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    dt_code = g.GSPN_F32 if w.dtype == "f32" else g.GSPN_BF16
    if bwd and w.per_direction:
        plan = "bwd_dirs"
    elif bwd:
        plan = g.backward_plan_name(w.B, w.C, w.H, w.W, w.dirs, w.group_rows, dt_code)
    elif w.per_direction:
        plan = "dirs"
    elif mod:
        plan = "prologue" if pro_only else "module"
    else:
        plan = g.plan_name(w.B, w.C, w.H, w.W, w.dirs, w.group_rows, dt_code)

    per_px = qmin_per_pixel(w, bwd)
    set_bytes = int(per_px * w.pixels)
    nsets = input_sets(w, bwd)
    sets = []
    for i in range(nsets):
        seed = 1000 + w.index + 17 * i
        if mod:
            big = set_bytes > 1 << 30
            st = make_prologue_inputs(w, seed=seed + 2000, device=dev if big else "cpu")
            sets.append({k: v.to(dev) for k, v in st.items()})
            continue
        if set_bytes > 1 << 30:
            st = make_inputs(w, seed=seed, device=dev)
            if bwd:
                st["gy"] = make_grad_out(w, seed=seed + 1000, device=dev)
        else:
            st = {k: v.to(dev) for k, v in make_inputs(w, seed=seed).items()}
            if bwd:
                st["gy"] = make_grad_out(w, seed=seed + 1000).to(dev)
        sets.append(st)
    if bwd and w.per_direction:
        outs = []
        for st in sets:
            o = {k: torch.empty_like(st["lam"]) for k in g.PARAM_NAMES}
            o["x"] = torch.empty_like(st["x"])
            o["merge"] = torch.empty((4, w.C), dtype=torch.float32, device=dev)
            outs.append(o)
        ws_bytes = g.backward_workspace_bytes_dirs(w.B, w.C, w.H, w.W, w.dirs, w.group_rows,
                                                   dt_code)
    elif bwd:
        outs = [{k: torch.empty_like(st[k] if k in ("l0", "l1", "l2") else st["x"])
                 for k in g.GRAD_NAMES} for st in sets]
        ws_bytes = g.backward_workspace_bytes(w.B, w.C, w.H, w.W, w.dirs, w.group_rows, dt_code,
                                              logit_channels=w.cl)
    elif mod:
        shape = (w.B, w.C, w.H, w.W)
        if pro_only:
            outs = [{k: torch.empty(shape, dtype=w.torch_dtype, device=dev)
                     for k in ("x",) + g.PARAM_NAMES} for _ in sets]
            ws_bytes = 0
        else:
            outs = [torch.empty(shape, dtype=w.torch_dtype, device=dev) for _ in sets]
            ws_bytes = g.module_workspace_bytes(w.B, w.C, w.H, w.W, w.dirs, w.group_rows, dt_code)
    else:
        outs = [torch.empty_like(st["x"]) for st in sets]
        wsb = g.workspace_bytes_dirs if w.per_direction else g.workspace_bytes
        ws_bytes = wsb(w.B, w.C, w.H, w.W, w.dirs, w.group_rows, dt_code)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        st = sets[i % nsets]
        if bwd and w.per_direction:
            g.propagate_backward_dirs(st["x"], (st["l0"], st["l1"], st["l2"]), st["lam"], st["u"],
                                      st["gy"], merge=st["merge"], dirs=w.dirs,
                                      group_rows=w.group_rows, grads=outs[i % nsets],
                                      workspace=ws if ws_bytes else None, stream=stream)
        elif bwd:
            g.propagate_backward(st["x"], (st["l0"], st["l1"], st["l2"]), st["lam"], st["u"],
                                 st["gy"], dirs=w.dirs, group_rows=w.group_rows,
                                 grads=outs[i % nsets], workspace=ws if ws_bytes else None,
                                 stream=stream)
        elif mod and pro_only:
            g.prologue(st["x_in"], st["w_r"], st["b_r"], st["w_p"], st["b_p"],
                       outs=outs[i % nsets], stream=stream)
        elif mod:
            g.module(st["x_in"], st["w_r"], st["b_r"], st["w_p"], st["b_p"], dirs=w.dirs,
                     group_rows=w.group_rows, out=outs[i % nsets], workspace=ws, stream=stream)
        elif w.per_direction:
            g.propagate_dirs(st["x"], (st["l0"], st["l1"], st["l2"]), st["lam"], st["u"],
                             merge=st["merge"], dirs=w.dirs, group_rows=w.group_rows,
                             out=outs[i % nsets], workspace=ws if ws_bytes else None,
                             stream=stream)
        else:
            g.propagate(st["x"], (st["l0"], st["l1"], st["l2"]), st["lam"], st["u"],
                        dirs=w.dirs, group_rows=w.group_rows, out=outs[i % nsets],
                        workspace=ws if ws_bytes else None, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    hip = Hip()
    L = g.lib()
    max_launch = 64   # launches traced per step (two plane groups double a chain)
    evs = [hip.events(2 * max_launch) for _ in range(args.steps)]
    # step boundaries: events on the caller's stream, into which every launch
    # of a step (also those on helper streams) is joined
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    sev[0].record(stream)
    wall0 = time.perf_counter()
    counts = []
    for k in range(args.steps):
        L.gspn_trace_events(evs[k], max_launch)
        step(k)
        counts.append(L.gspn_trace_count())
        sev[k + 1].record(stream)
    L.gspn_trace_events(None, 0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = sev[0].elapsed_time(sev[-1])
    ms_per_step = ms_total / args.steps
    step_ms = sorted(sev[k].elapsed_time(sev[k + 1]) for k in range(args.steps))

    def med(v):
        n = len(v)
        return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])

    step_stats = {"steps": args.steps, "median_ms": med(step_ms), "min_ms": step_ms[0],
                  "mean_ms": ms_per_step, "max_ms": step_ms[-1]}
    if args.steps < 50 and not args.no_step_sample:
        # a further sample of at least 50 steps and about a second, after the
        # timed region, for the median and min of the step time
        n_more = int(min(2000, max(50, 1000.0 / max(ms_per_step, 1e-3))))
        mev = [torch.cuda.Event(enable_timing=True) for _ in range(n_more + 1)]
        mev[0].record(stream)
        for k in range(n_more):
            step(args.steps + k)
            mev[k + 1].record(stream)
        torch.cuda.synchronize()
        more = sorted(mev[k].elapsed_time(mev[k + 1]) for k in range(n_more))
        step_stats["extra_sample"] = {"steps": n_more, "median_ms": med(more),
                                      "min_ms": more[0],
                                      "mean_ms": mev[0].elapsed_time(mev[-1]) / n_more}

    nl = min(counts[0], max_launch)
    launches = []
    for i in range(nl):
        np_ = ctypes.c_int64()
        name = L.gspn_trace_kernel(i, ctypes.byref(np_))
        launches.append((name.decode() if name else "?", int(np_.value)))
    per_launch = [0.0] * nl
    for k in range(args.steps):
        for i in range(nl):
            per_launch[i] += hip.elapsed_ms(evs[k][2 * i], evs[k][2 * i + 1])
    per_launch = [t / args.steps for t in per_launch]
    for e in evs:
        hip.destroy(e)
    # per kernel: summed launch time and design bytes (launches of one kernel
    # may run on two streams; each is timed on its own stream)
    kt, kb = {}, {}
    passes = [i for i, (name, _) in enumerate(launches) if name == "dir_vert"]
    for i, ((name, np_), t) in enumerate(zip(launches, per_launch)):
        kt[name] = kt.get(name, 0.0) + t
        first, last = (i == passes[0], i == passes[-1]) if i in passes else (True, True)
        kb[name] = kb.get(name, 0.0) + design_bytes(name, np_, w, first=first, last=last)
    path_bytes = sum(kb.values())
    if bwd and w.per_direction:
        # the transposes of this path move tensors the trace does not tell
        # apart: the path's design bytes are counted as a whole
        path_bytes = bwd_dirs_path_bytes(w) * w.pixels
    # Roofline unit: the launches of one step. A single launch is timed by its
    # own events; a pipeline of several launches (overlapping on two streams)
    # by the step time. Algorithmic bytes: the compulsory Q_min = 7 s per
    # pixel (five inputs and u read once, out written once), 13 s for the
    # backward pass (seven tensors read, six gradients written), (2 + 5 dirs) s
    # with per-direction parameters.
    q_min = int(per_px * w.pixels)
    if nl == 1:
        unit_name, unit_ms = launches[0][0], per_launch[0]
    else:
        unit_name = "+".join(dict.fromkeys(n for n, _ in launches))
        unit_ms = ms_per_step
    achieved = q_min / (unit_ms * 1e-3) / 1e9
    traffic = counter_traffic(plan, w.name, source_digest(plan))

    value = w.elem_steps * args.steps / (ms_total * 1e-3)
    ceiling = None if args.no_ceiling else stream_ceiling(
        torch, L, reps=5, variants=[(2, nt, bpc) for nt in (0, 1) for bpc in (1, 2, 4)] +
        [(0, 1, 2), (1, 1, 2)])
    roofline = {"bound": "hbm", "kernel": unit_name, "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic,
                "traffic_counter": "FETCH_SIZE * 2 + WRITE_SIZE per step (bytes between L2 and "
                                   "the memory fabric; last-level-cache hits included, so an "
                                   "upper bound on HBM bytes)",
                "algorithmic_bytes_per_step": q_min, "unit_ms": unit_ms}
    if ceiling:
        roofline["ceiling_gbs"] = ceiling["copy_gbs"]
        roofline["frac_of_ceiling"] = achieved / ceiling["copy_gbs"]
        roofline["ceiling"] = "hand-written 16-byte copy kernel over 4 GiB (gspn_bench_stream), " \
                              "read + write bytes; read-only %.0f, write-only %.0f GB/s" % (
                                  ceiling["read_gbs"], ceiling["write_gbs"])
    if mod and not pro_only:
        # the whole unit: its products' flops against the MFMA peak, its
        # compulsory bytes (x_in read, out written) against HBM; the bound is
        # whichever takes the longer at peak
        flops, _ = prologue_work(w)
        peak = MFMA_PEAK_TFLOPS[w.dtype]
        if flops / (peak * 1e12) >= q_min / (HBM_PEAK_GBS * 1e9):
            ach = flops / (unit_ms * 1e-3) / 1e12
            roofline.update({"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                             "frac": ach / peak, "algorithmic_flops_per_step": flops,
                             "hbm_qmin_gbs": achieved})
            for k in ("ceiling_gbs", "frac_of_ceiling", "ceiling"):
                roofline.pop(k, None)
    if pro_only:
        # the prologue's two products: bound by MFMA or by HBM, whichever its
        # flops and bytes make the longer at peak
        flops, nbytes = prologue_work(w)
        peak = MFMA_PEAK_TFLOPS[w.dtype]
        value = flops / (ms_per_step * 1e-3) / 1e12
        if flops / (peak * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9):
            ach = flops / (unit_ms * 1e-3) / 1e12
            roofline = {"bound": "mfma", "kernel": unit_name, "achieved": ach, "peak": peak,
                        "unit": "TFLOP/s", "frac": ach / peak, "traffic": traffic,
                        "algorithmic_flops_per_step": flops, "unit_ms": unit_ms}
        else:
            ach = nbytes / (unit_ms * 1e-3) / 1e9
            roofline = {"bound": "hbm", "kernel": unit_name, "achieved": ach,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                        "traffic": traffic, "algorithmic_bytes_per_step": nbytes,
                        "unit_ms": unit_ms}
        roofline["flops_per_step"] = flops
        roofline["mfma_tflops"] = flops / (unit_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC_PRO if pro_only else (METRIC_BWD if bwd else METRIC),
        "value": value,
        "unit": "TFLOP/s" if pro_only else "elem-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if (mod and w.dtype == "bf16") else "f32",
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": w.name, "B": w.B, "C": w.C, "H": w.H, "W": w.W,
                   "dirs": w.dirs, "group_rows": w.group_rows, "storage": w.dtype,
                   "logit_channels": w.cl, "per_direction": w.per_direction,
                   "prologue_cin": w.prologue_cin,
                   "plan": plan, "launches_per_step": counts[0],
                   "launches": [f"{n}[{p}]" for n, p in launches],
                   "launch_ms": [round(t, 4) for t in per_launch],
                   "kernel_ms": {k: round(v, 4) for k, v in kt.items()},
                   "path_design_bytes": path_bytes,
                   "path_design_gbs": path_bytes / (ms_per_step * 1e-3) / 1e9,
                   "path_qmin_bytes": q_min,
                   "host_wall_s": round(wall, 3), "input_sets": nsets},
        "roofline": roofline,
        "step_stats": step_stats,
    }
    if not args.no_cpu_baseline and mod:
        cb, ref = cpu_baseline_module(sets[0], w, args.cpu_seconds, pro_only)
        if ref is not None:
            # outs[0]: set 0's unit output from the last timed step that used it
            cb["parity"] = parity_of_sample(outs[0][:1].float().reshape(-1, w.H, w.W).cpu().numpy(),
                                            ref.reshape(-1, w.H, w.W), w.dtype)
        else:
            cb["parity"] = {"checked": False,
                            "why": "the CPU sample is a band of rows, not whole planes"}
        cb["cpu_model"] = cpu_model()
        result["cpu_baseline"] = cb
    elif not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        # the oracle runs roughly 1.5e7 - 3.5e7 elem-steps/s per core forward
        # and 0.6e6 - 3e6 backward (large planes at the low end)
        rate = 6e5 if bwd else 2.5e7
        planes = int(args.cpu_seconds * rate * cores / (w.H * w.W * w.ndirs)) + 1
        cb, (np_s, ref) = cpu_baseline(sets[0], w, planes,
                                       grad_out=sets[0]["gy"] if bwd else None)
        # outs[0] holds set 0's result from the last timed step that used it
        cb["parity"] = timed_output_parity(outs[0], ref, np_s, w, bwd)
        cb["cpu_model"] = cpu_model()
        cb["per_core"] = oracle_per_core_rate()
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
