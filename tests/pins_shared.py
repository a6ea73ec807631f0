"""Pins for channel-shared logits in the fp64 oracle (CSDN page on GSPN,
section 局限性: the speed test sets the weights' feature dimension to 1).

With logits [B, Cl, H, W], channel c uses logit channel c // (C // Cl):
  * forward: the result equals the unshared oracle run on logits repeated
    over each group of C // Cl consecutive channels -- numpy.repeat builds
    that input, independently of the oracle's index mapping;
  * backward: x, lambda and u gradients equal the repeated run's, and each
    shared logit gradient is the sum over its group of the repeated run's
    per-channel gradients (chain rule for a shared parameter);
  * backward, independently of both: central finite differences of the
    shared forward with respect to a shared logit.
Every check takes ``prop`` / ``bwd`` with the signatures of
``oracle.propagate`` / ``oracle.backward``.
"""
from __future__ import annotations

import numpy as np

import oracle
from pins import ALL, B2T, L2R, T2B, _close

CASES = [((2, 4, 5, 6), 1, 0), ((1, 4, 6, 5), 2, 0), ((1, 6, 5, 5), 3, 2), ((2, 2, 4, 4), 2, 0)]


def _shared_inputs(rng, shape, cl):
    B, C, H, W = shape
    x = rng.standard_normal(shape)
    lam = rng.uniform(0.2, 1.0, shape)
    u = rng.uniform(-1.0, 1.0, shape)
    lg = [rng.standard_normal((B, cl, H, W)) * 1.5 for _ in range(3)]
    return x, lg, lam, u


def check_shared_forward(prop):
    rng = np.random.default_rng(43)
    for shape, cl, G in CASES:
        x, lg, lam, u = _shared_inputs(rng, shape, cl)
        rep = [np.repeat(l, shape[1] // cl, axis=1) for l in lg]
        for dirs in (ALL, T2B, L2R, B2T | L2R):
            got = prop(x, *lg, lam, u, dirs=dirs, group_rows=G, nthreads=2)
            want = oracle.propagate(x, *rep, lam, u, dirs=dirs, group_rows=G, nthreads=1)
            assert np.array_equal(got, want), f"shared forward {shape} Cl={cl} dirs={dirs}"


def check_shared_backward_sum(bwd):
    rng = np.random.default_rng(47)
    for shape, cl, G in CASES:
        x, lg, lam, u = _shared_inputs(rng, shape, cl)
        gy = rng.standard_normal(shape)
        g = shape[1] // cl
        rep = [np.repeat(l, g, axis=1) for l in lg]
        got = bwd(x, *lg, lam, u, gy, dirs=ALL, group_rows=G, nthreads=2)
        want = oracle.backward(x, *rep, lam, u, gy, dirs=ALL, group_rows=G, nthreads=1)
        for k in ("x", "lam", "u"):
            assert np.array_equal(got[k], want[k]), f"shared backward d{k} {shape} Cl={cl}"
        B, C, H, W = shape
        for k in ("l0", "l1", "l2"):
            summed = want[k].reshape(B, cl, g, H, W).sum(axis=2)
            assert got[k].shape == (B, cl, H, W)
            _close(got[k], summed, 1e-13, f"shared backward d{k} {shape} Cl={cl}")


def check_shared_finite_difference(bwd):
    rng = np.random.default_rng(53)
    eps = 1e-6
    shape, cl, G = (1, 4, 4, 5), 2, 0
    x, lg, lam, u = _shared_inputs(rng, shape, cl)
    gy = rng.standard_normal(shape)
    got = bwd(x, *lg, lam, u, gy, dirs=ALL, group_rows=G, nthreads=1)
    B, C, H, W = shape
    for k in range(3):
        fd = np.zeros_like(lg[k])
        for idx in np.ndindex(lg[k].shape):
            lp = [l.copy() for l in lg]
            lm = [l.copy() for l in lg]
            lp[k][idx] += eps
            lm[k][idx] -= eps
            yp = oracle.propagate(x, *lp, lam, u, dirs=ALL, group_rows=G, nthreads=1)
            ym = oracle.propagate(x, *lm, lam, u, dirs=ALL, group_rows=G, nthreads=1)
            fd[idx] = ((yp - ym) * gy).sum() / (2 * eps)
        tol = 2e-6 * (np.abs(fd) + np.sqrt(np.mean(fd * fd))) + 1e-8
        err = np.abs(got[f"l{k}"] - fd)
        assert np.all(err <= tol), f"shared finite difference dl{k}: max error {err.max():.3e}"


SHARED_CHECKS = [check_shared_forward]
SHARED_BWD_CHECKS = [check_shared_backward_sum, check_shared_finite_difference]
