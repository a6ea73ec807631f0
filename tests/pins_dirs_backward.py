"""Pins for the backward pass of the per-direction layer in the fp64 oracle
(CSDN page on GSPN, section 反向传播; per-direction sets and a merger: aitntnews
page, section GSPN架构; reading R15).

  * central finite differences of the per-direction forward oracle, on
    sampled entries of every input, every direction slice and the merge
    weights, global and local;
  * four equal direction sets with an all-ones merger give, summed over the
    directions, the gradients of the shared layer (whose backward is pinned
    on its own), and the same dx;
  * the merge gradient of direction d is sum(gy * y_d), y_d the single
    direction's forward output (its definition, evaluated by the forward
    oracle), and directions outside the mask get exact zeros.
Every check takes ``bwd`` with the signature of ``oracle.backward_dirs``.
"""
from __future__ import annotations

import numpy as np

import oracle
from pins import _close

PNAMES = ("l0", "l1", "l2", "lam", "u")


def _case(seed, B, C, H, W):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C, H, W))
    params = [rng.standard_normal((4, B, C, H, W)) for _ in range(5)]
    gy = rng.standard_normal((B, C, H, W))
    merge = rng.uniform(-1.5, 1.5, (4, C))
    return x, params, gy, merge


def _loss(x, params, gy, merge, dirs, G):
    y = oracle.propagate_dirs(x, *params, merge=merge, dirs=dirs, group_rows=G, nthreads=1)
    return float((gy * y).sum())


def check_finite_differences(bwd):
    """Every gradient kind against central differences of the forward, on
    sampled entries of each direction slice (eps 1e-6 in fp64)."""
    eps = 1e-6
    for seed, (B, C, H, W), dirs, G in [(201, (1, 2, 5, 4), 15, 0), (202, (2, 1, 4, 6), 15, 3),
                                        (203, (1, 2, 3, 5), 9, 0)]:
        x, params, gy, merge = _case(seed, B, C, H, W)
        g = bwd(x, *params, gy, merge=merge, dirs=dirs, group_rows=G, nthreads=1)
        rng = np.random.default_rng(seed + 50)
        worst = 0.0
        # x
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd = (_loss(xp, params, gy, merge, dirs, G) - _loss(xm, params, gy, merge, dirs, G)) / (2 * eps)
            worst = max(worst, abs(g["x"][idx] - fd) / (1 + abs(fd)))
        # each parameter kind, each direction slice
        for k, name in enumerate(PNAMES):
            for d in range(4):
                idx = (d,) + tuple(int(rng.integers(0, n)) for n in x.shape)
                pp = [p.copy() for p in params]
                pm = [p.copy() for p in params]
                pp[k][idx] += eps
                pm[k][idx] -= eps
                fd = (_loss(x, pp, gy, merge, dirs, G) - _loss(x, pm, gy, merge, dirs, G)) / (2 * eps)
                worst = max(worst, abs(g[name][idx] - fd) / (1 + abs(fd)))
        # the merge weights
        for d in range(4):
            for c in range(C):
                mp, mm = merge.copy(), merge.copy()
                mp[d, c] += eps
                mm[d, c] -= eps
                fd = (_loss(x, params, gy, mp, dirs, G) - _loss(x, params, gy, mm, dirs, G)) / (2 * eps)
                worst = max(worst, abs(g["merge"][d, c] - fd) / (1 + abs(fd)))
        assert worst < 1e-6, f"finite differences: worst scaled error {worst:.2e} (dirs {dirs}, G {G})"


def check_equal_sets_reduce_to_shared(bwd):
    """Four copies of one set, all-ones merger: the per-direction gradients
    summed over the directions are the shared layer's, dx is the same."""
    rng = np.random.default_rng(211)
    B, C, H, W = 2, 2, 5, 6
    x = rng.standard_normal((B, C, H, W))
    one = [rng.standard_normal((B, C, H, W)) for _ in range(5)]
    gy = rng.standard_normal((B, C, H, W))
    for dirs, G in [(15, 0), (15, 2), (6, 0)]:
        params = [np.broadcast_to(t, (4,) + t.shape).copy() for t in one]
        g = bwd(x, *params, gy, merge=None, dirs=dirs, group_rows=G, nthreads=2)
        ref = oracle.backward(x, *one, gy, dirs=dirs, group_rows=G, nthreads=2)
        _close(g["x"], ref["x"], 1e-12, f"equal sets dx (dirs {dirs}, G {G})")
        for name in PNAMES:
            _close(g[name].sum(axis=0), ref[name], 1e-12,
                   f"equal sets d{name} summed over directions (dirs {dirs}, G {G})")


def check_merge_gradient_and_unused_directions(bwd):
    """dmerge[d, c] = sum over images and pixels of gy * y_d (y_d: the single
    direction's forward with u_d and a unit merger); directions outside the
    mask have zero gradients everywhere."""
    B, C, H, W = 2, 3, 4, 5
    x, params, gy, merge = _case(221, B, C, H, W)
    for dirs, G in [(15, 0), (10, 3)]:
        g = bwd(x, *params, gy, merge=merge, dirs=dirs, group_rows=G, nthreads=2)
        for d in range(4):
            if dirs & (1 << d):
                unit = np.zeros((4, C))
                unit[d] = 1.0
                y_d = oracle.propagate_dirs(x, *params, merge=unit, dirs=1 << d, group_rows=G,
                                            nthreads=1)
                want = (gy * y_d).sum(axis=(0, 2, 3))
                _close(g["merge"][d], want, 1e-12, f"dmerge of direction {d} (G {G})")
            else:
                for name in PNAMES:
                    assert not np.any(g[name][d]), f"direction {d} outside the mask has d{name}"
                assert not np.any(g["merge"][d]), f"direction {d} outside the mask has dmerge"


ALL_DIRS_BACKWARD_CHECKS = [check_finite_differences, check_equal_sets_reduce_to_shared,
                            check_merge_gradient_and_unused_directions]
