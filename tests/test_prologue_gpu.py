"""The module prologue (MFMA 1x1 convolutions) and the whole unit on the GPU
against the fp64 oracle, through the C ABI (needs an MI355X)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import linear_spatial_propagation_line_amd as g
import oracle
from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_prologue_inputs
from parity import assert_parity, to_oracle_array

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {torch.float32: "f32", torch.bfloat16: "bf16"}


def oracle_prologue(inp, bias=True):
    arrs = [to_oracle_array(inp[k]) for k in ("x_in", "w_r")]
    arrs.append(to_oracle_array(inp["b_r"]) if bias else None)
    arrs.append(to_oracle_array(inp["w_p"]))
    arrs.append(to_oracle_array(inp["b_p"]) if bias else None)
    return oracle.prologue(*arrs)


def gpu_prologue(inp, bias=True):
    d = {k: v.to(DEV) for k, v in inp.items()}
    out = g.prologue(d["x_in"], d["w_r"], d["b_r"] if bias else None, d["w_p"],
                     d["b_p"] if bias else None)
    torch.cuda.synchronize()
    return out


# (B, Cin, C, H, W): ragged M (C and 5C not multiples of 128), ragged K (Cin,
# C not multiples of 32), ragged N (H*W not a multiple of 128 or of the
# 16-byte run), a single pixel, single channels, K above one tile, C above
# one M tile
SHAPES = [(1, 1, 1, 1, 1), (2, 3, 5, 7, 9), (1, 37, 20, 9, 15), (1, 64, 96, 16, 16),
          (2, 96, 96, 56, 56), (1, 40, 130, 3, 50), (1, 300, 33, 8, 8), (3, 16, 8, 1, 129)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prologue_shapes(shape, dtype):
    B, Cin, C, H, W = shape
    print(f"[prologue] shape={shape} dtype={dtype}", flush=True)
    inp = make_prologue_inputs(None, seed=11 + Cin + C, B=B, Cin=Cin, C=C, H=H, W=W,
                               dtype=DT[dtype])
    for bias in (True, False):
        got = gpu_prologue(inp, bias)
        ref = oracle_prologue(inp, bias)
        assert_parity(got["x"], ref["x"], f"prologue x {shape} bias={bias}")
        for k in g.PARAM_NAMES:
            assert_parity(got[k], ref[k], f"prologue {k} {shape} bias={bias}")


def test_prologue_wide_channels():
    """C = Cin = 1152 (the DiT-XL/2 width): K spans 36 tiles, 5C 45 M tiles."""
    inp = make_prologue_inputs("dit_16x16_mod", B=1)
    got = gpu_prologue(inp)
    ref = oracle_prologue(inp)
    assert_parity(got["x"], ref["x"], "prologue x C=1152")
    for k in g.PARAM_NAMES:
        assert_parity(got[k], ref[k], f"prologue {k} C=1152")


def test_prologue_identity_is_exact():
    """Identity weights, no bias: x copies x_in and the parameters are exact
    multiples of it, bit for bit (every product is exact, one term per sum)."""
    for dtype in (torch.float32, torch.bfloat16):
        C = 40
        x_in = torch.randn(2, C, 9, 11).to(dtype).to(DEV)
        eye = torch.eye(C)
        w_p = torch.cat([eye, 2 * eye, -eye, 0 * eye, 0.5 * eye]).to(dtype).to(DEV)
        out = g.prologue(x_in, eye.to(dtype).to(DEV), None, w_p, None)
        torch.cuda.synchronize()
        assert torch.equal(out["x"], x_in)
        for k, f in zip(g.PARAM_NAMES, (1.0, 2.0, -1.0, 0.0, 0.5)):
            assert torch.equal(out[k], (f * x_in.float()).to(dtype)), k


def oracle_module(inp, dirs, G, dtype):
    pro = oracle_prologue(inp)
    p = {k: oracle.round_to(pro[k], DT[dtype]) for k in g.PARAM_NAMES}
    return oracle.propagate(pro["xr"], p["l0"], p["l1"], p["l2"], p["lam"], p["u"], dirs=dirs,
                            group_rows=G)


# (B, Cin, C, H, W, G): propagation plans plane16, plane64, band, stream, tpipe
MODULE_CASES = [(2, 24, 16, 16, 16, 0), (1, 40, 12, 56, 56, 0), (1, 16, 8, 128, 128, 8),
                (1, 9, 6, 65, 80, 0), (1, 32, 4, 130, 96, 0)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", MODULE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_module(case, dtype):
    B, Cin, C, H, W, G = case
    inp = make_prologue_inputs(None, seed=7 + H, B=B, Cin=Cin, C=C, H=H, W=W, dtype=DT[dtype])
    d = {k: v.to(DEV) for k, v in inp.items()}
    for dirs in (15, g.T2B | g.R2L):
        out = g.module(d["x_in"], d["w_r"], d["b_r"], d["w_p"], d["b_p"], dirs=dirs,
                       group_rows=G)
        torch.cuda.synchronize()
        assert_parity(out, oracle_module(inp, dirs, G, dtype), f"module {case} dirs={dirs}")


def test_module_errors():
    inp = make_prologue_inputs(None, seed=1, B=1, Cin=8, C=4, H=8, W=8, dtype="f32")
    d = {k: v.to(DEV) for k, v in inp.items()}
    with pytest.raises(ValueError):
        g.prologue(d["x_in"], d["w_r"][:, :3].contiguous(), None, d["w_p"], None)
    with pytest.raises(ValueError):
        g.prologue(d["x_in"], d["w_r"], None, d["w_p"][:19].contiguous(), None)
    with pytest.raises(g.GspnError):
        g.module(d["x_in"], d["w_r"], None, d["w_p"], None,
                 workspace=torch.empty(16, dtype=torch.uint8, device=DEV))


def test_t2i_module_full_size_sampled():
    """The 2048x1024 unit with Cin = C = 320 in bf16 at full size, as the
    benchmark runs it: the prologue's outputs on sampled pixel rows against
    the oracle prologue, and the propagation of sampled channel planes of
    those outputs against the oracle propagation."""
    w = WORKLOADS["t2i_2048x1024_mod"]
    d = make_prologue_inputs(w, device=DEV)
    pro = g.prologue(d["x_in"], d["w_r"], d["b_r"], d["w_p"], d["b_p"])
    out = g.propagate(pro["x"], (pro["l0"], pro["l1"], pro["l2"]), pro["lam"], pro["u"],
                      dirs=w.dirs)
    full = g.module(d["x_in"], d["w_r"], d["b_r"], d["w_p"], d["b_p"], dirs=w.dirs)
    torch.cuda.synchronize()
    assert torch.equal(out, full), "module differs from prologue + propagate"
    rows = [0, 1023, 2047]
    sub = {k: v.cpu() for k, v in d.items()}
    sub["x_in"] = sub["x_in"][:, :, rows]
    ref = oracle_prologue(sub)
    for k in ("x",) + g.PARAM_NAMES:
        assert_parity(pro[k][:, :, rows], ref[k], f"t2i prologue {k} rows {rows}")
    for c in (0, 211):
        arrs = [to_oracle_array(pro[k][:, c:c + 1]) for k in ("x", "l0", "l1", "l2", "lam", "u")]
        assert_parity(out[:, c:c + 1], oracle.propagate(*arrs, dirs=w.dirs), f"t2i module plane {c}")
