"""Helpers for comparing the HIP path with the fp64 oracle.

Parity criterion (per element): |g - o| <= rtol * (|o| + rms(o)), where o is
the oracle output, rms is taken over the whole compared tensor (outputs are
roughly zero-mean, so a purely relative bound is meaningless near zero), and
rtol = 1e-5 for float32 storage, 1e-2 for bfloat16 storage with fp32
accumulation (fp32 scans longer than 2048 steps: see rtol_for).

Gradients (backward pass) use the same bound per tensor, with one more term
in the scale: 1e-3 of the largest rms among the six gradient tensors of the
call. It only matters for a tensor that is (nearly) zero everywhere -- the
logit gradients of a one-pixel-wide line, or under Theorem 1 -- where the
oracle's own fp64 rounding (~1e-16) would otherwise set the scale.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

RTOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def rtol_for(dtype, shape) -> float:
    """The dtype's bound; for fp32 scans longer than 2048 steps, a bound that
    grows with the scan length. The recurrence rounds each step (weights
    that sum to 1 only to within an ulp, three FMAs), so the relative error
    can grow linearly with the number of steps n, up to about n * 2^-24.
    Measured errors grow at about a thirteenth of that (4e-5 at 9000 steps);
    the bound n * 2^-26 (1.3e-4 at 9000 steps) keeps a margin of about 3 over
    them, so a kernel that rounds markedly worse still fails. Every workload
    scans at most 2048 steps and keeps the plain bound."""
    base = RTOL[dtype]
    n = max(shape[-2], shape[-1])
    if dtype == torch.float32 and n > 2048:
        return max(base, n * 2.0 ** -26)
    return base


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
    rtol = rtol_for(got.dtype, got.shape)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.detach().float().cpu().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = scaled_error(got, ref)
    assert err <= rtol, f"{what}: scaled error {err:.3e} > {rtol:.0e}"
    return err


GRAD_NAMES = ("x", "l0", "l1", "l2", "lam", "u")


def oracle_grads(inp: dict, gy: torch.Tensor, dirs: int, G: int, nthreads=None) -> dict:
    arrs = [to_oracle_array(inp[k]) for k in ("x", "l0", "l1", "l2", "lam", "u")]
    return oracle.backward(*arrs, to_oracle_array(gy), dirs=dirs, group_rows=G,
                           nthreads=nthreads)


def assert_grad_parity(got: dict, ref: dict, what: str = "", names=GRAD_NAMES) -> float:
    """Every gradient tensor in ``names`` within the dtype's bound; returns the
    worst scaled error."""
    floor = 1e-3 * max(float(np.sqrt(np.mean(ref[k] * ref[k]))) for k in ref)
    worst = 0.0
    for k in names:
        g_t = got[k]
        rtol = rtol_for(g_t.dtype, g_t.shape)
        assert tuple(g_t.shape) == ref[k].shape, (k, g_t.shape, ref[k].shape)
        g = g_t.detach().float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g)), f"{what} d{k}: non-finite gradient"
        o = ref[k]
        rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
        err = float(np.max(np.abs(g - o) / (np.abs(o) + rms + floor + 1e-300))) if o.size else 0.0
        assert err <= rtol, f"{what} d{k}: scaled error {err:.3e} > {rtol:.0e}"
        worst = max(worst, err)
    return worst
