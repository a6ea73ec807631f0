"""Pins for the backward pass of the fp64 oracle (CSDN page
"GSPN——在convolution基础上并行序列建模", section 反向传播): checks that tie the
gradients to mathematics other than the oracle's own backward code.

Every ``check_*`` takes ``bwd`` -- a callable with the signature of
``oracle.backward`` -- and raises AssertionError on a mismatch, so the same
checks run against the real oracle and against planted mistakes.

  * central finite differences of the (separately pinned) forward oracle,
    for every input, direction subset and local grouping on tiny planes;
  * the linear part in closed form: y = u (.) sum_d G_d x with the explicit G
    of section 方法, so dL/dx = sum_d G_d^T (u (.) gy) -- a numpy transpose,
    independent of the oracle's adjoint loop; and lambda dL/dlambda = x dL/dx;
  * dL/du = gy (.) sum_d h_d, with h_d from the forward oracle;
  * Theorem 1 (section 稳定性-上下文条件): with lambda x = 1 every predecessor
    of a pixel holds the same h, so no weight can change y: the logit
    gradients vanish;
  * one-hot middle weight (w = I): dL/dx is lambda times the reversed prefix
    sum of u gy along the scan, per local group (numpy.cumsum);
  * hand-derived exact gradients in tests/golden/hand_backward.txt.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
from pins import ALL, B2T, GOLDEN, L2R, R2L, T2B, _close, _inputs, gmatrix_of, load_golden

NAMES = ("x", "l0", "l1", "l2", "lam", "u")


def _fwd(args, dirs, G):
    return oracle.propagate(*args, dirs=dirs, group_rows=G, nthreads=1)


def check_bwd_golden(bwd):
    """Hand-derived exact gradients (tests/golden/hand_backward.txt)."""
    for case in load_golden(os.path.join(GOLDEN, "hand_backward.txt")):
        got = bwd(*case["inputs"], case["gy"], dirs=case["dirs"], group_rows=case["G"],
                  nthreads=1)
        for key, name in (("dx", "x"), ("dl0", "l0"), ("dl1", "l1"), ("dl2", "l2"),
                          ("dlam", "lam"), ("du", "u")):
            assert np.allclose(got[name], case[key], rtol=1e-13, atol=1e-13), \
                f"golden {case['name']} {key}: got {got[name][0, 0]} want {case[key][0, 0]}"


def check_bwd_finite_difference(bwd):
    """Central differences of L = sum(gy * y) through the forward oracle; every
    perturbed copy is one plane of a single batched forward call."""
    rng = np.random.default_rng(23)
    eps = 1e-6
    cases = [((4, 5), 0, (ALL, T2B, B2T, L2R, R2L)), ((5, 3), 0, (ALL,)),
             ((6, 6), 2, (ALL, T2B, R2L)), ((5, 5), 3, (ALL,)), ((1, 4), 0, (ALL,)),
             ((3, 1), 0, (ALL,)), ((2, 2), 0, (ALL,))]
    for (H, W), G, masks in cases:
        shape = (1, 1, H, W)
        args = list(_inputs(rng, shape))
        gy = rng.standard_normal(shape)
        n = H * W
        for dirs in masks:
            got = bwd(*args, gy, dirs=dirs, group_rows=G, nthreads=1)
            for t, name in enumerate(NAMES):
                # planes 2i / 2i+1: element i of input t moved by +eps / -eps
                batch = [np.repeat(a, 2 * n, axis=0) for a in args]
                flat = batch[t].reshape(2 * n, n)
                for i in range(n):
                    flat[2 * i, i] += eps
                    flat[2 * i + 1, i] -= eps
                y = _fwd(batch, dirs, G)
                L = (y * gy).reshape(2 * n, n).sum(axis=1)
                fd = ((L[0::2] - L[1::2]) / (2 * eps)).reshape(shape)
                # truncation error ~eps^2, rounding of L ~1e-16 |L| / eps
                tol = 2e-6 * (np.abs(fd) + np.sqrt(np.mean(fd * fd))) + 1e-8
                err = np.abs(got[name] - fd)
                assert np.all(err <= tol), \
                    f"finite difference d{name} shape={(H, W)} dirs={dirs} G={G}: " \
                    f"max error {err.max():.3e}"


def check_bwd_gmatrix_transpose(bwd):
    """dL/dx = sum_d G_d^T (u gy) with the explicit G (lambda inside G), and
    lambda dL/dlambda = x dL/dx."""
    rng = np.random.default_rng(29)
    for (H, W), G in [((4, 5), 0), ((5, 4), 0), ((6, 6), 2), ((5, 7), 3), ((1, 3), 0),
                      ((3, 1), 0)]:
        shape = (1, 2, H, W)
        x, l0, l1, l2, lam, u = _inputs(rng, shape)
        gy = rng.standard_normal(shape)
        for dirs in (ALL, T2B, B2T, L2R, R2L):
            got = bwd(x, l0, l1, l2, lam, u, gy, dirs=dirs, group_rows=G, nthreads=1)
            want = np.zeros(shape)
            for c in range(2):
                lg = [l0[0, c], l1[0, c], l2[0, c]]
                ug = (u * gy)[0, c]
                for d in range(4):
                    if not dirs & (1 << d):
                        continue
                    Gm, lines = gmatrix_of(H, W, lg, lam[0, c], d, G)
                    vec = np.array([ug[p] for line in lines for p in line])
                    back = Gm.T @ vec
                    k = 0
                    for line in lines:
                        for p in line:
                            want[0, c][p] += back[k]
                            k += 1
            _close(got["x"], want, 1e-12, f"G^T dx shape={(H, W)} dirs={dirs} G={G}")
            _close(lam * got["lam"], x * got["x"], 1e-12, "lambda dlam = x dx")


def check_bwd_du(bwd):
    """dL/du = gy (.) sum_d h_d, h_d from the forward oracle with u = 1."""
    rng = np.random.default_rng(31)
    for (H, W), G in [((5, 6), 0), ((6, 5), 2), ((1, 1), 0)]:
        shape = (2, 1, H, W)
        x, l0, l1, l2, lam, u = _inputs(rng, shape)
        gy = rng.standard_normal(shape)
        for dirs in (ALL, B2T | L2R):
            got = bwd(x, l0, l1, l2, lam, u, gy, dirs=dirs, group_rows=G, nthreads=1)
            hsum = _fwd((x, l0, l1, l2, lam, np.ones(shape)), dirs, G)
            _close(got["u"], gy * hsum, 1e-13, f"du shape={(H, W)} dirs={dirs}")


def check_bwd_invariant(bwd):
    """lambda x = 1: all predecessors of a pixel hold the same h (Theorem 1),
    so the weights cannot move y and every logit gradient is zero."""
    rng = np.random.default_rng(37)
    for (H, W), G in [((6, 7), 0), ((8, 8), 3), ((1, 5), 0)]:
        shape = (1, 2, H, W)
        one = np.ones(shape)
        l0, l1, l2 = (rng.standard_normal(shape) * 2 for _ in range(3))
        u = rng.uniform(-1, 1, shape)
        gy = rng.standard_normal(shape)
        got = bwd(one, l0, l1, l2, one, u, gy, dirs=ALL, group_rows=G, nthreads=1)
        scale = np.max(np.abs(got["x"]))
        for k in ("l0", "l1", "l2"):
            assert np.max(np.abs(got[k])) <= 1e-12 * scale, f"invariant d{k} G={G}"


def check_bwd_onehot(bwd):
    """w = I (l0 = l2 = -inf): each direction is a prefix sum, whose adjoint is
    the reversed prefix sum of u gy along the scan, restarted per group."""
    rng = np.random.default_rng(41)
    shape = (1, 2, 6, 7)
    x = rng.standard_normal(shape)
    lam = rng.uniform(-1, 1, shape)
    l1 = rng.standard_normal(shape)
    u = rng.uniform(-1, 1, shape)
    gy = rng.standard_normal(shape)
    ninf = np.full(shape, -np.inf)
    ug = u * gy

    def rev_cumsum(a, axis, G):
        n = a.shape[axis]
        out = np.zeros_like(a)
        starts = range(0, n, G) if G else [0]
        for s0 in starts:
            s1 = min(n, s0 + G) if G else n
            blk = np.take(a, range(s0, s1), axis=axis)
            r = np.flip(np.cumsum(np.flip(blk, axis), axis=axis), axis)
            idx = [slice(None)] * a.ndim
            idx[axis] = slice(s0, s1)
            out[tuple(idx)] = r
        return out

    for G in (0, 3):
        for bit, axis, rev in ((T2B, 2, False), (B2T, 2, True), (L2R, 3, False),
                               (R2L, 3, True)):
            got = bwd(x, ninf, l1, ninf, lam, u, gy, dirs=bit, group_rows=G, nthreads=1)
            # adjoint of a forward prefix sum is a suffix sum and vice versa
            e = _prefix(ug, axis, G) if rev else rev_cumsum(ug, axis, G)
            _close(got["x"], lam * e, 1e-13, f"one-hot dx dirs={bit} G={G}")
            # the single live link always has weight 1 (zero up to rounding);
            # the dead ones have sigmoid slope 0 exactly
            scale = np.max(np.abs(got["x"]))
            assert np.max(np.abs(got["l1"])) <= 1e-13 * scale, f"one-hot dl1 dirs={bit}"
            assert np.all(got["l0"] == 0) and np.all(got["l2"] == 0), f"one-hot dl0/dl2 dirs={bit}"


def _prefix(a, axis, G):
    """forward prefix sum along axis, restarted at every block of G (0: none)"""
    n = a.shape[axis]
    out = np.zeros_like(a)
    starts = range(0, n, G) if G else [0]
    for s0 in starts:
        s1 = min(n, s0 + G) if G else n
        idx = [slice(None)] * a.ndim
        idx[axis] = slice(s0, s1)
        out[tuple(idx)] = np.cumsum(a[tuple(idx)], axis=axis)
    return out


ALL_BWD_CHECKS = [check_bwd_golden, check_bwd_finite_difference, check_bwd_gmatrix_transpose,
                  check_bwd_du, check_bwd_invariant, check_bwd_onehot]
