"""Helpers for comparing the HIP path with the fp64 oracle.

Parity criterion (per element): |g - o| <= rtol * (|o| + rms(o)), where o is
the oracle output, rms is taken over the whole compared tensor (outputs are
roughly zero-mean, so a purely relative bound is meaningless near zero), and
rtol = 1e-5 for float32 storage, 1e-2 for bfloat16 storage with fp32
accumulation.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

RTOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def to_oracle_array(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def oracle_y(inp: dict, dirs: int, G: int, nthreads=None) -> np.ndarray:
    arrs = [to_oracle_array(inp[k]) for k in ("x", "l0", "l1", "l2", "lam", "u")]
    return oracle.propagate(*arrs, dirs=dirs, group_rows=G, nthreads=nthreads)


def scaled_error(got: torch.Tensor, ref: np.ndarray) -> float:
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(g - ref) / (np.abs(ref) + rms + 1e-300)))


def assert_parity(got: torch.Tensor, ref: np.ndarray, what: str = "") -> float:
    rtol = RTOL[got.dtype]
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.detach().float().cpu().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = scaled_error(got, ref)
    assert err <= rtol, f"{what}: scaled error {err:.3e} > {rtol:.0e}"
    return err
