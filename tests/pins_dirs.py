"""Pins for per-direction parameters and the per-channel merger in the fp64
oracle (aitntnews page, sections 二维线性传播 and GSPN架构; CSDN page, section
GSPN模块的设计): direction d scans x with its own lambda_d and logits, gates
with its own u_d, and the directions are merged as y = sum_d m[d, c] u_d h_d.

  * explicit G matrices, one per direction built by numpy from that
    direction's logits and lambda, independent of the oracle's loops;
  * Theorem 1 per direction: with x = 1, lambda_d = a_d, u_d = b_d (constants
    that differ between directions) and any logits, direction d's state at a
    pixel is a_d times the number of steps taken so far in its group, so
    y = sum_d m[d, c] a_d b_d count_d -- a closed form;
  * four identical parameter sets with unit merge weights reproduce the
    shared-parameter oracle bit for bit.
Every check takes ``prop`` with the signature of ``oracle.propagate_dirs``.
"""
from __future__ import annotations

import numpy as np

import oracle
from pins import ALL, B2T, L2R, R2L, T2B, _close, gmatrix_plane

DIR_BITS = (T2B, B2T, L2R, R2L)


def _dir_inputs(rng, shape):
    """x [B, C, H, W]; l0, l1, l2, lam, u [4, B, C, H, W]; merge [4, C]."""
    x = rng.standard_normal(shape)
    dshape = (4,) + tuple(shape)
    lg = [rng.standard_normal(dshape) * 1.5 for _ in range(3)]
    lam = rng.uniform(0.2, 1.0, dshape)
    u = rng.uniform(-1.0, 1.0, dshape)
    merge = rng.uniform(-1.0, 1.0, (4, shape[1]))
    return x, lg, lam, u, merge


def gmatrix_dirs_reference(x, lg, lam, u, merge, dirs, G):
    """y = sum_d merge[d, c] u_d * (G_d vec(x)) from explicit per-direction
    G matrices; float64 [B, C, H, W]."""
    B, C, H, W = x.shape
    y = np.zeros((B, C, H, W))
    for b in range(B):
        for c in range(C):
            for d in range(4):
                if not dirs & (1 << d):
                    continue
                lgd = [lg[k][d, b, c] for k in range(3)]
                m = 1.0 if merge is None else merge[d, c]
                y[b, c] += m * u[d, b, c] * gmatrix_plane(x[b, c], lgd, lam[d, b, c], d, G)
    return y


def check_dirs_gmatrix(prop):
    """Oracle == explicit per-direction G matrices, with and without merge
    weights, every direction alone and together, global and local."""
    rng = np.random.default_rng(71)
    cases = [((1, 2, 5, 4), 0), ((1, 3, 4, 5), 0), ((1, 2, 1, 3), 0), ((1, 2, 3, 1), 0),
             ((1, 2, 6, 6), 2), ((2, 2, 5, 7), 3)]
    for shape, G in cases:
        x, lg, lam, u, merge = _dir_inputs(rng, shape)
        for dirs in (T2B, B2T, L2R, R2L, T2B | L2R, ALL):
            for m in (merge, None):
                ref = gmatrix_dirs_reference(x, lg, lam, u, m, dirs, G)
                got = prop(x, *lg, lam, u, merge=m, dirs=dirs, group_rows=G, nthreads=1)
                _close(got, ref, 1e-12, f"per-direction G-matrix shape={shape} dirs={dirs} G={G}")


def _steps_in_group(d, H, W, G):
    """Steps taken by direction d's scan at every pixel, counted from the
    start of its local group (1 at the first pixel of a group)."""
    n_s = H if d < 2 else W
    cnt = np.zeros(n_s)
    k = 0
    for s in range(n_s):
        p = s if d in (0, 2) else n_s - 1 - s
        prev = p - 1 if d in (0, 2) else p + 1
        k = 1 if s == 0 or (G > 0 and p // G != prev // G) else k + 1
        cnt[p] = k
    return np.broadcast_to(cnt[:, None], (H, W)) if d < 2 else np.broadcast_to(cnt[None, :], (H, W))


def check_dirs_invariant(prop):
    """Theorem 1 per direction, with per-direction constants a_d (lambda) and
    b_d (u) and per-channel merge weights: a closed form at every pixel."""
    rng = np.random.default_rng(73)
    a = np.array([0.5, 2.0, -1.25, 3.0])
    bgate = np.array([1.5, -0.75, 0.25, 2.5])
    for (H, W, G) in [(6, 5, 0), (5, 8, 0), (7, 7, 3), (1, 4, 0), (4, 1, 2)]:
        shape = (1, 3, H, W)
        dshape = (4,) + shape
        x = np.ones(shape)
        lg = [rng.standard_normal(dshape) * 2 for _ in range(3)]
        lam = np.broadcast_to(a[:, None, None, None, None], dshape).copy()
        u = np.broadcast_to(bgate[:, None, None, None, None], dshape).copy()
        merge = rng.uniform(-1.0, 1.0, (4, 3))
        for dirs in (T2B, R2L, B2T | L2R, ALL):
            got = prop(x, *lg, lam, u, merge=merge, dirs=dirs, group_rows=G, nthreads=1)
            ref = np.zeros(shape)
            for d in range(4):
                if dirs & (1 << d):
                    steps = _steps_in_group(d, H, W, G)
                    for c in range(3):
                        ref[0, c] += merge[d, c] * a[d] * bgate[d] * steps
            _close(got, ref, 1e-12, f"per-direction invariant H={H} W={W} G={G} dirs={dirs}")


def check_dirs_equal_sets(prop):
    """Four copies of one parameter set, unit merge weights (explicit and
    omitted): the shared-parameter oracle's result, bit for bit."""
    rng = np.random.default_rng(79)
    for shape, G in [((2, 3, 6, 5), 0), ((1, 2, 7, 9), 3)]:
        x = rng.standard_normal(shape)
        l0, l1, l2 = (rng.standard_normal(shape) for _ in range(3))
        lam = rng.uniform(0.2, 1.0, shape)
        u = rng.uniform(-1.0, 1.0, shape)
        rep = [np.stack([t] * 4) for t in (l0, l1, l2, lam, u)]
        for dirs in (ALL, B2T | R2L):
            ref = oracle.propagate(x, l0, l1, l2, lam, u, dirs=dirs, group_rows=G, nthreads=1)
            for m in (None, np.ones((4, shape[1]))):
                got = prop(x, *rep, merge=m, dirs=dirs, group_rows=G, nthreads=1)
                assert np.array_equal(got, ref), f"equal sets differ from the shared oracle {shape}"


ALL_DIRS_CHECKS = [check_dirs_gmatrix, check_dirs_invariant, check_dirs_equal_sets]
