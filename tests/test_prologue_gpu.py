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


@pytest.mark.parametrize("shape", [(2, 512, 96, 16, 16), (75, 512, 384, 16, 16),
                                   (1, 1152, 1152, 16, 16)],
                         ids=lambda s: "x".join(map(str, s)))
def test_prologue_whole_tiles_direct_to_lds(shape, monkeypatch):
    """bf16 products of whole tiles with K above the pixel-stationary
    kernel's reach load their K stages straight into LDS: the first shape's
    first product takes M tiles of 96 rows, the second's of 128, the third
    (DiT width) both products. Same sums
    in the same order as the register-staged kernel: the same bits, and the
    oracle's bound."""
    B, Cin, C, H, W = shape
    inp = make_prologue_inputs(None, seed=5 + C, B=B, Cin=Cin, C=C, H=H, W=W, dtype="bf16")
    monkeypatch.delenv("GSPN_GEMM_LDS", raising=False)
    got = gpu_prologue(inp)
    monkeypatch.setenv("GSPN_GEMM_LDS", "0")
    reg = gpu_prologue(inp)
    for k in ("x",) + tuple(g.PARAM_NAMES):
        assert torch.equal(got[k].view(torch.int16), reg[k].view(torch.int16)), f"{shape} {k}"
    if B <= 2:
        ref = oracle_prologue(inp)
        assert_parity(got["x"], ref["x"], f"x {shape}")
        for k in g.PARAM_NAMES:
            assert_parity(got[k], ref[k], f"{k} {shape}")


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


# (B, Cin, C, H, W, G) that take the fused path (bf16, H, W <= 16, H W a
# multiple of 8, C a multiple of 64): full and partial planes, one-pixel-wide
# lines, local groups, several channel groups and K steps
FUSED_CASES = [(2, 24, 64, 16, 16, 0), (1, 40, 128, 8, 8, 0), (3, 64, 64, 16, 12, 3),
               (1, 20, 64, 4, 2, 0), (1, 64, 192, 16, 1, 0), (2, 96, 64, 12, 16, 5),
               (1, 7, 256, 2, 4, 0)]


def _module(d, dirs, G, bias=True, force=None, monkeypatch=None):
    if force:
        monkeypatch.setenv("GSPN_FORCE_MODULE", force)
    else:
        monkeypatch.delenv("GSPN_FORCE_MODULE", raising=False)
    out = g.module(d["x_in"], d["w_r"], d["b_r"] if bias else None, d["w_p"],
                   d["b_p"] if bias else None, dirs=dirs, group_rows=G)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fused_unit(case, monkeypatch):
    """The fused parameter product + scan against the oracle's prologue,
    rounding and propagation, and against the unfused two-step path: the
    same products in the same order, so the same bits."""
    B, Cin, C, H, W, G = case
    print(f"[fused] case={case}", flush=True)
    inp = make_prologue_inputs(None, seed=31 + C + H, B=B, Cin=Cin, C=C, H=H, W=W, dtype="bf16")
    d = {k: v.to(DEV) for k, v in inp.items()}
    for dirs in (15, g.T2B | g.R2L, g.L2R):
        for bias in (True, False):
            fused = _module(d, dirs, G, bias, monkeypatch=monkeypatch)
            plain = _module(d, dirs, G, bias, force="unfused", monkeypatch=monkeypatch)
            sub = dict(inp)
            if not bias:
                sub = {k: v for k, v in inp.items()}
                sub["b_r"] = torch.zeros_like(inp["b_r"])
                sub["b_p"] = torch.zeros_like(inp["b_p"])
            assert_parity(fused, oracle_module(sub, dirs, G, torch.bfloat16),
                          f"fused {case} dirs={dirs} bias={bias}")
            assert torch.equal(fused, plain), f"fused and unfused paths differ: {case} {dirs}"


def test_fused_unit_takes_the_fused_path(monkeypatch):
    """The launches of a fused call: the first product, then the fused kernel
    (no parameter product, no separate propagation)."""
    import bench
    monkeypatch.delenv("GSPN_FORCE_MODULE", raising=False)
    inp = make_prologue_inputs(None, seed=3, B=1, Cin=16, C=64, H=16, W=16, dtype="bf16")
    d = {k: v.to(DEV) for k, v in inp.items()}
    L = g.lib()
    hip = bench.Hip()
    evs = hip.events(16)
    L.gspn_trace_events(evs, 8)
    g.module(d["x_in"], d["w_r"], d["b_r"], d["w_p"], d["b_p"])
    torch.cuda.synchronize()
    L.gspn_trace_events(None, 0)
    names = [L.gspn_trace_kernel(i, None).decode() for i in range(L.gspn_trace_count())]
    hip.destroy(evs)
    assert names == ["prologue_reduce", "fused_unit"], names


def test_dit_unit_full_size_fused(monkeypatch):
    """The DiT-XL/2 unit (32 x 1152 x 16 x 16, bf16) at full size through the
    fused path, as the benchmark runs it: image 0 against the oracle, the
    whole output against the unfused path bit for bit."""
    monkeypatch.delenv("GSPN_FORCE_MODULE", raising=False)
    w = WORKLOADS["dit_16x16_mod"]
    d = make_prologue_inputs(w, device=DEV)
    fused = _module(d, w.dirs, 0, monkeypatch=monkeypatch)
    plain = _module(d, w.dirs, 0, force="unfused", monkeypatch=monkeypatch)
    assert torch.equal(fused, plain)
    sub = {k: v.cpu() for k, v in d.items()}
    sub["x_in"] = sub["x_in"][:1]
    assert_parity(fused[:1], oracle_module(sub, w.dirs, 0, torch.bfloat16), "DiT unit image 0")


def _extreme_unit(B, Cin, C, H, W, seed, base, outside):
    """A unit whose logits all lie near ``base`` (spread of a few units), and
    with ``outside``, base + 40 for each neighbour outside the plane (l0 on
    row 0 and column 0, l2 on row H - 1 and column W - 1): x channels 0 and
    1 carry those border indicators, the logit rows of W_p weight them by 40."""
    gen = torch.Generator().manual_seed(seed)
    uni = lambda *s: 2.0 * torch.rand(*s, generator=gen, dtype=torch.float64) - 1.0
    x_in = uni(B, Cin, H, W)
    r = torch.arange(H).view(H, 1)
    c = torch.arange(W).view(1, W)
    x_in[:, 0] = ((r == 0) | (c == 0)).double()
    x_in[:, 1] = ((r == H - 1) | (c == W - 1)).double()
    w_r = torch.zeros(C, Cin, dtype=torch.float64)
    for i in range(C):
        w_r[i, i if i < Cin else 2 + i % (Cin - 2)] = 1.0
    w_p = torch.zeros(5 * C, C, dtype=torch.float64)
    b_p = torch.zeros(5 * C, dtype=torch.float64)
    for t in range(5):
        w_p[t * C:(t + 1) * C, 2:] = uni(C, C - 2) * (4.0 if t < 3 else 0.5) / (C - 2) ** 0.5
    b_p[:3 * C] = base
    b_p[3 * C:4 * C] = 0.5
    b_p[4 * C:] = 1.0
    if outside:
        w_p[0:C, 0] = 40.0
        w_p[2 * C:3 * C, 1] = 40.0
    bf = torch.bfloat16
    return {"x_in": x_in.to(bf), "w_r": w_r.to(bf), "b_r": torch.zeros(C, dtype=bf),
            "w_p": w_p.to(bf), "b_p": b_p.to(bf)}


def oracle_module_clamped(inp, dirs, G):
    """The unit as the kernels form it: the bf16 logits clamped below at -40."""
    pro = oracle_prologue(inp)
    p = {k: oracle.round_to(pro[k], "bf16") for k in g.PARAM_NAMES}
    for k in ("l0", "l1", "l2"):
        p[k] = np.maximum(p[k], -40.0)
    return oracle.propagate(pro["xr"], p["l0"], p["l1"], p["l2"], p["lam"], p["u"], dirs=dirs,
                            group_rows=G)


@pytest.mark.parametrize("recipe", [(-30.0, False), (-30.0, True), (-60.0, False)],
                         ids=["shallow", "outside", "deep"])
@pytest.mark.parametrize("case", [(2, 16, 64, 16, 16), (1, 16, 64, 16, 12), (1, 8, 64, 8, 8)],
                         ids=lambda c: "x".join(map(str, c)))
def test_fused_unit_extreme_logits(case, recipe, monkeypatch):
    """Logits near -30 give weights far from uniform (they follow the logits'
    differences); with +10 on the neighbours outside the plane, border pixels
    hold nearly all their interior weight on a neighbour that edge lanes
    drop. Near -60 the weights are those of the logits clamped at -40. Against
    the oracle, and bit for bit against the unfused path."""
    B, Cin, C, H, W = case
    base, outside = recipe
    inp = _extreme_unit(B, Cin, C, H, W, 40 + H + W, base, outside)
    d = {k: v.to(DEV) for k, v in inp.items()}
    for dirs in (15, g.T2B | g.R2L, g.L2R):
        fused = _module(d, dirs, 0, monkeypatch=monkeypatch)
        plain = _module(d, dirs, 0, force="unfused", monkeypatch=monkeypatch)
        ref = oracle_module_clamped(inp, dirs, 0)
        if base > -35.0:   # nothing clamped: the exact unit
            ref_exact = oracle_module(inp, dirs, 0, torch.bfloat16)
            assert np.array_equal(ref, ref_exact)
        assert_parity(fused, ref, f"fused extreme {case} dirs={dirs}")
        assert torch.equal(fused, plain), f"fused and unfused paths differ: {case} {dirs}"
