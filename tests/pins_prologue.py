"""Pins for the module prologue in the fp64 oracle (aitntnews page, section
GSPN架构: a shared 1x1 convolution reduces the channels, three independent 1x1
convolutions produce the propagation parameters).

  * a 1x1 convolution is what torch.nn.functional.conv2d computes with a
    1x1 kernel: x and the five parameter tensors against conv2d in float64;
  * the x the parameter convolutions read is x rounded to the storage type:
    every value representable in it, no representable neighbour closer, ties
    to an even last bit (checked for bf16 from the bit patterns);
  * identity weights give exact copies and multiples.
Every check takes ``prol`` with the signature of ``oracle.prologue``.
"""
from __future__ import annotations

import numpy as np
import torch

from pins import _close

NAMES = ("l0", "l1", "l2", "lam", "u")


def conv1x1(x, w, b):
    """torch's conv2d with a 1x1 kernel, float64."""
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float64))[:, :, None, None]
    bt = None if b is None else torch.from_numpy(np.ascontiguousarray(b, dtype=np.float64))
    return torch.nn.functional.conv2d(xt, wt, bt).numpy()


def _params_ref(xr, w_p, b_p):
    p = conv1x1(xr, w_p, b_p)
    C = xr.shape[1]
    return {n: p[:, t * C:(t + 1) * C] for t, n in enumerate(NAMES)}


def _to_bf16_bits(a):
    """float64 -> bf16 bit patterns by truncation (exact for the small
    integers and dyadic values the checks draw)."""
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _from_bf16_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_conv2d(prol):
    """fp64 and fp32 storage: x, its rounding and the parameters against
    conv2d, with and without biases, Cin != C."""
    rng = np.random.default_rng(101)
    for (B, Cin, C, H, W) in [(2, 5, 3, 4, 6), (1, 3, 4, 1, 7), (1, 8, 8, 3, 3)]:
        x_in = rng.standard_normal((B, Cin, H, W))
        w_r = rng.standard_normal((C, Cin)) / np.sqrt(Cin)
        b_r = rng.standard_normal(C)
        w_p = rng.standard_normal((5 * C, C)) / np.sqrt(C)
        b_p = rng.standard_normal(5 * C)
        for dt in (np.float64, np.float32):
            args = [a.astype(dt) for a in (x_in, w_r, b_r, w_p, b_p)]
            for bias in (True, False):
                br, bp = (args[2], args[4]) if bias else (None, None)
                got = prol(args[0], args[1], br, args[3], bp, nthreads=2)
                ref_x = conv1x1(args[0], args[1], br)
                _close(got["x"], ref_x, 1e-12, f"prologue x {dt.__name__}")
                want_xr = ref_x if dt is np.float64 else ref_x.astype(np.float32).astype(np.float64)
                _close(got["xr"], want_xr, 1e-12, f"prologue rounded x {dt.__name__}")
                ref_p = _params_ref(got["xr"], args[3], bp)
                for n in NAMES:
                    _close(got[n], ref_p[n], 1e-12, f"prologue {n} {dt.__name__}")


def check_bf16_rounding(prol):
    """bf16 storage: the rounded x is bf16-representable, nearest to the
    exact x, ties to an even last bit; the parameters are conv2d of it."""
    rng = np.random.default_rng(103)
    B, Cin, C, H, W = 2, 6, 4, 5, 5
    # small dyadic values: exact in bf16, so the exact x is known to fp64
    x_in = rng.integers(-64, 65, (B, Cin, H, W)) / 16.0
    w_r = rng.integers(-32, 33, (C, Cin)) / 8.0
    b_r = rng.integers(-8, 9, C) / 4.0
    w_p = rng.integers(-16, 17, (5 * C, C)) / 16.0
    b_p = rng.integers(-8, 9, 5 * C) / 8.0
    bits = [_to_bf16_bits(a) for a in (x_in, w_r, b_r, w_p, b_p)]
    got = prol(*bits, nthreads=1)
    x = got["x"]
    _close(x, conv1x1(x_in, w_r, b_r), 1e-12, "bf16 prologue x")
    xr = got["xr"]
    rb = _to_bf16_bits(xr)
    assert np.array_equal(_from_bf16_bits(rb), xr), "rounded x is not bf16-representable"
    nz = xr != 0
    mag = rb & 0x7FFF
    up = _from_bf16_bits((rb & 0x8000) | (mag + 1))
    down = _from_bf16_bits((rb & 0x8000) | np.maximum(mag, 1) - 1)
    d0 = np.abs(x - xr)
    assert np.all(d0[nz] <= np.abs(x - up)[nz]), "a larger bf16 neighbour is closer"
    assert np.all(d0[nz] <= np.abs(x - down)[nz]), "a smaller bf16 neighbour is closer"
    tie = nz & ((d0 == np.abs(x - up)) | (d0 == np.abs(x - down)))
    assert np.all(rb[tie] & 1 == 0), "tie not rounded to an even last bit"
    assert tie.any() and (d0 > 0).any(), "the draw exercised no rounding"
    ref_p = _params_ref(xr, w_p, b_p)
    for n in NAMES:
        _close(got[n], ref_p[n], 1e-12, f"bf16 prologue {n}")


def check_identity(prol):
    """W_r = I without bias copies x_in; parameter weights that are multiples
    of I give exact multiples of x."""
    rng = np.random.default_rng(107)
    C = 4
    x_in = rng.standard_normal((2, C, 3, 5))
    eye = np.eye(C)
    w_p = np.concatenate([eye, 2 * eye, -eye, 0 * eye, 0.5 * eye])
    got = prol(x_in, eye, None, w_p, None, nthreads=1)
    assert np.array_equal(got["x"], x_in)
    for n, f in zip(NAMES, (1.0, 2.0, -1.0, 0.0, 0.5)):
        assert np.array_equal(got[n], f * x_in), f"identity prologue {n}"


ALL_PROLOGUE_CHECKS = [check_conv2d, check_bf16_rounding, check_identity]
