"""Pins for the fp64 oracle: checks that tie it to what the pages and plain
mathematics fix, not to itself.

Every ``check_*`` takes ``prop`` -- a callable with the signature of
``oracle.propagate`` -- and raises AssertionError on a mismatch, so the same
checks run against the real oracle (tests/test_oracle_pins.py) and against
deliberately broken copies of it (tests/test_oracle_mutants.py).

Pins (CSDN page "GSPN——在convolution基础上并行序列建模"):
  * explicit lower-triangular G (section 方法): H = G X with
    G_ij = (w_i w_{i-1} ... w_{j+1}) lambda_j, G_ii = lambda_i, built here with
    numpy matrix products from the tridiagonal w of section
    如何设计一个高效的传播层 -- independent code from the oracle's loop;
  * Theorem 1 (section 稳定性-上下文条件): with row-stochastic w and
    lambda x = 1, u = 1, h at scan step s equals s + 1;
  * one-hot middle weight (w = I exactly) reduces the recurrence to a per-line
    prefix sum, i.e. numpy.cumsum, bitwise;
  * hand-derived exact examples in tests/golden/hand_examples.txt;
  * symmetries of the four scan directions, linearity, mask additivity and
    the local-group restart (section GSPN模块的设计).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

T2B, B2T, L2R, R2L = 1, 2, 4, 8
ALL = 15


def _sig(v):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


# ---------------------------------------------------------------------------
# explicit G matrix (numpy, float64), one plane, one direction
# ---------------------------------------------------------------------------
def _line_pixels(d, H, W, s):
    """(row, col) of the n_o pixels that scan step s of direction d visits."""
    if d == 0:
        return [(s, o) for o in range(W)]
    if d == 1:
        return [(H - 1 - s, o) for o in range(W)]
    if d == 2:
        return [(o, s) for o in range(H)]
    return [(o, W - 1 - s) for o in range(H)]


def _abs_pos(d, H, W, s):
    return [s, H - 1 - s, s, W - 1 - s][d]


def _step_matrix(d, H, W, s, lg):
    """Tridiagonal w_s: row o holds the weights of pixel o of line s for the
    previous line's o-1, o, o+1 (in-range only), sigmoid then row-normalised."""
    pix = _line_pixels(d, H, W, s)
    n = len(pix)
    w = np.zeros((n, n))
    for o, (r, c) in enumerate(pix):
        ks = [k for k in range(3) if 0 <= o + k - 1 < n]
        sig = {k: _sig(lg[k][r, c]) for k in ks}
        tot = sum(sig.values())
        for k in ks:
            w[o, o + k - 1] = sig[k] / tot
    return w


def gmatrix_plane(x, lg, lam, d, G):
    """h for one plane and direction via the unrolled form H = G X."""
    H, W = x.shape
    Gm, lines = gmatrix_of(H, W, lg, lam, d, G)
    n_o = len(lines[0])
    X = np.array([x[p] for line in lines for p in line])
    Hv = Gm @ X
    h = np.zeros((H, W))
    for i, line in enumerate(lines):
        for o, p in enumerate(line):
            h[p] = Hv[i * n_o + o]
    return h


def gmatrix_of(H, W, lg, lam, d, G):
    """The explicit block lower-triangular G of one plane and direction (rows
    and columns in scan order: line by line, orthogonal index fastest) and
    the (row, col) pixels of each line."""
    n_s = H if d < 2 else W
    n_o = W if d < 2 else H
    ws = [_step_matrix(d, H, W, s, lg) for s in range(n_s)]
    lines = [_line_pixels(d, H, W, s) for s in range(n_s)]
    block = [(_abs_pos(d, H, W, s) // G) if G > 0 else 0 for s in range(n_s)]
    Gm = np.zeros((n_s * n_o, n_s * n_o))
    for i in range(n_s):
        for j in range(i + 1):
            if block[i] != block[j]:
                continue
            prod = np.eye(n_o)
            for r in range(j + 1, i + 1):     # w_i w_{i-1} ... w_{j+1}
                prod = ws[r] @ prod
            lam_j = np.diag([lam[p] for p in lines[j]])
            Gm[i * n_o:(i + 1) * n_o, j * n_o:(j + 1) * n_o] = prod @ lam_j
    return Gm, lines


def gmatrix_reference(x, l0, l1, l2, lam, u, dirs, G):
    """y = sum_d u * h_d from explicit G matrices; float64 [B, C, H, W]."""
    B, C, H, W = x.shape
    y = np.zeros((B, C, H, W))
    for b in range(B):
        for c in range(C):
            lg = [l0[b, c], l1[b, c], l2[b, c]]
            for d in range(4):
                if dirs & (1 << d):
                    y[b, c] += u[b, c] * gmatrix_plane(x[b, c], lg, lam[b, c], d, G)
    return y


# ---------------------------------------------------------------------------
def _rand(rng, shape, kind="normal"):
    if kind == "normal":
        return rng.standard_normal(shape)
    return rng.uniform(-1.0, 1.0, shape)


def _inputs(rng, shape):
    x = _rand(rng, shape)
    lam = rng.uniform(0.2, 1.0, shape)
    u = _rand(rng, shape, "uniform")
    l0, l1, l2 = (_rand(rng, shape) * 1.5 for _ in range(3))
    return x, l0, l1, l2, lam, u


def _close(a, b, rtol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = np.abs(b) + np.sqrt(np.mean(b * b)) + 1e-300
    err = np.max(np.abs(a - b) / scale)
    assert err <= rtol, f"{what}: max scaled error {err:.3e} > {rtol:.1e}"


# ---------------------------------------------------------------------------
def check_gmatrix(prop):
    """Oracle == explicit G matrix on tiny planes, every direction, global and
    local, including single-row / single-column planes."""
    rng = np.random.default_rng(7)
    cases = [((1, 2, 5, 4), 0), ((1, 2, 4, 5), 0), ((1, 1, 1, 3), 0),
             ((1, 1, 3, 1), 0), ((1, 1, 6, 6), 2), ((1, 1, 6, 6), 4),
             ((2, 1, 5, 7), 3), ((1, 1, 2, 2), 0)]
    for shape, G in cases:
        args = _inputs(rng, shape)
        for dirs in (T2B, B2T, L2R, R2L, ALL):
            ref = gmatrix_reference(*args, dirs, G)
            got = prop(*args, dirs=dirs, group_rows=G, nthreads=1)
            _close(got, ref, 1e-12, f"G-matrix shape={shape} dirs={dirs} G={G}")


def check_invariant(prop):
    """Theorem 1: row-stochastic w with lambda x = 1 and u = 1 gives h = s + 1
    at scan step s (counted from the start of the local group)."""
    rng = np.random.default_rng(11)
    for (H, W, G) in [(7, 5, 0), (5, 9, 0), (8, 8, 3), (1, 4, 0), (4, 1, 0)]:
        shape = (1, 2, H, W)
        one = np.ones(shape)
        l0, l1, l2 = (rng.standard_normal(shape) * 2 for _ in range(3))
        for d, bit in enumerate((T2B, B2T, L2R, R2L)):
            y = prop(one, l0, l1, l2, one, one, dirs=bit, group_rows=G, nthreads=1)
            n_s = H if d < 2 else W
            exp_line = np.zeros(n_s)
            count = 0
            for s in range(n_s):
                p = [s, n_s - 1 - s, s, n_s - 1 - s][d]
                prevp = [s - 1, n_s - s, s - 1, n_s - s][d]
                if s == 0 or (G > 0 and p // G != prevp // G):
                    count = 0
                count += 1
                exp_line[p] = count
            exp = exp_line[:, None] if d < 2 else exp_line[None, :]
            exp = np.broadcast_to(exp, (H, W))
            assert np.allclose(y[0, 0], exp, rtol=1e-12, atol=0), \
                f"invariant d={d} H={H} W={W} G={G}"
            assert np.allclose(y[0, 1], exp, rtol=1e-12, atol=0)
        if G == 0:
            y = prop(one, l0, l1, l2, one, one, dirs=ALL, group_rows=0, nthreads=1)
            assert np.allclose(y, H + W + 2, rtol=1e-12, atol=0), "4-dir invariant"


def check_onehot_cumsum(prop):
    """l0 = l2 = -inf gives w = I exactly, so h is numpy.cumsum of lambda x
    along the scan axis (reversed for bottom->top and right->left), bitwise."""
    rng = np.random.default_rng(13)
    shape = (2, 3, 6, 9)
    x = rng.standard_normal(shape)
    lam = rng.uniform(-1, 1, shape)
    l1 = rng.standard_normal(shape)
    ninf = np.full(shape, -np.inf)
    one = np.ones(shape)
    bx = lam * x
    want = {
        T2B: np.cumsum(bx, axis=2),
        B2T: np.flip(np.cumsum(np.flip(bx, 2), axis=2), 2),
        L2R: np.cumsum(bx, axis=3),
        R2L: np.flip(np.cumsum(np.flip(bx, 3), axis=3), 3),
    }
    for bit, ref in want.items():
        got = prop(x, ninf, l1, ninf, lam, one, dirs=bit, group_rows=0, nthreads=2)
        assert np.array_equal(got, ref), f"one-hot cumsum dirs={bit}"


def check_golden(prop):
    """Hand-derived exact examples (tests/golden/hand_examples.txt)."""
    for case in load_golden(os.path.join(GOLDEN, "hand_examples.txt")):
        got = prop(*case["inputs"], dirs=case["dirs"], group_rows=case["G"], nthreads=1)
        want = case["y"]
        assert np.allclose(got, want, rtol=1e-13, atol=1e-13), \
            f"golden case {case['name']}: got {got[0, 0]} want {want[0, 0]}"


def check_symmetries(prop):
    """Direction conventions relative to each other: bottom->top is the
    vertical flip of top->bottom, left->right the transpose of top->bottom,
    right->left the horizontal flip of left->right. Also linearity in x,
    additivity over the direction mask, local == global on each group strip,
    and G >= n == global."""
    rng = np.random.default_rng(17)
    shape = (1, 2, 7, 6)
    x, l0, l1, l2, lam, u = _inputs(rng, shape)
    args = (x, l0, l1, l2, lam, u)

    def P(a, dirs, G=0):
        return prop(*a, dirs=dirs, group_rows=G, nthreads=1)

    fh = lambda t: np.ascontiguousarray(np.flip(t, 2))
    fw = lambda t: np.ascontiguousarray(np.flip(t, 3))
    tr = lambda t: np.ascontiguousarray(np.swapaxes(t, 2, 3))
    _close(P(args, B2T), fh(P([fh(a) for a in args], T2B)), 1e-13, "B2T = flipH T2B flipH")
    _close(P(args, L2R), tr(P([tr(a) for a in args], T2B)), 1e-13, "L2R = T T2B T")
    _close(P(args, R2L), fw(P([fw(a) for a in args], L2R)), 1e-13, "R2L = flipW L2R flipW")

    x2 = rng.standard_normal(shape)
    lin = P((2.5 * x - 1.5 * x2, l0, l1, l2, lam, u), ALL)
    _close(lin, 2.5 * P(args, ALL) - 1.5 * P((x2, l0, l1, l2, lam, u), ALL), 1e-12, "linearity")

    parts = sum(P(args, b) for b in (T2B, B2T, L2R, R2L))
    _close(P(args, ALL), parts, 1e-13, "mask additivity")

    # local: vertical scans with G = 3 equal global scans run on each strip
    G = 3
    for bit in (T2B, B2T):
        full = P(args, bit, G)
        for r0 in range(0, shape[2], G):
            sl = [np.ascontiguousarray(a[:, :, r0:r0 + G, :]) for a in args]
            _close(full[:, :, r0:r0 + G, :], P(sl, bit), 1e-13, f"local strip rows dirs={bit}")
    for bit in (L2R, R2L):
        full = P(args, bit, G)
        for c0 in range(0, shape[3], G):
            sl = [np.ascontiguousarray(a[:, :, :, c0:c0 + G]) for a in args]
            _close(full[:, :, :, c0:c0 + G], P(sl, bit), 1e-13, f"local strip cols dirs={bit}")
    _close(P(args, ALL, 7), P(args, ALL, 0), 1e-15, "G >= n is global")
    _close(P(args, ALL, 100), P(args, ALL, 0), 1e-15, "G >> n is global")


ALL_CHECKS = [check_golden, check_gmatrix, check_invariant, check_onehot_cumsum,
              check_symmetries]


# ---------------------------------------------------------------------------
# golden file parser
# ---------------------------------------------------------------------------
_SYMS = {"inf": math.inf, "-inf": -math.inf, "ln3": math.log(3.0),
         "-ln3": -math.log(3.0)}


def _num(tok):
    if tok in _SYMS:
        return _SYMS[tok]
    if "/" in tok:
        a, b = tok.split("/")
        return float(a) / float(b)
    return float(tok)


def load_golden(path):
    """Parse the hand-example file: blocks separated by blank lines; lines
    'key: v v v ; v v v' (rows split by ';'), '#' starts a comment."""
    cases = []
    cur = {}
    with open(path, encoding="utf-8") as f:
        for raw in f:
            if raw.lstrip().startswith("#"):
                continue
            line = raw.split("#", 1)[0].strip()
            if not line:
                if cur:
                    cases.append(cur)
                    cur = {}
                continue
            key, val = [t.strip() for t in line.split(":", 1)]
            cur[key] = val
    if cur:
        cases.append(cur)
    out = []
    for c in cases:
        H, W = (int(t) for t in c["shape"].split())

        def grid(v, H=H, W=W):
            if v.strip().split() and len(v.split(";")) == 1 and len(v.split()) == 1:
                return np.full((1, 1, H, W), _num(v.strip()))
            rows = [[_num(t) for t in r.split()] for r in v.split(";")]
            a = np.array(rows, dtype=np.float64)
            assert a.shape == (H, W), (c["name"], a.shape)
            return a.reshape(1, 1, H, W)
        inputs = tuple(grid(c[k]) for k in ("x", "l0", "l1", "l2", "lam", "u"))
        case = {"name": c["name"], "dirs": int(c["dirs"]), "G": int(c["G"]),
                "inputs": inputs, "y": grid(c["y"])}
        # backward examples also give gy and the six gradients
        for k in ("gy", "dx", "dl0", "dl1", "dl2", "dlam", "du"):
            if k in c:
                case[k] = grid(c[k])
        out.append(case)
    return out
