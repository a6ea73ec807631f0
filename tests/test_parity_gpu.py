"""HIP path vs the fp64 oracle, element by element, on the same seeded inputs
(needs an MI355X). Every call goes through the C ABI via the binding."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import linear_spatial_propagation_line_amd as g
from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_inputs
from parity import assert_parity, oracle_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(inp, dirs, G, **kw):
    d = {k: v.to(DEV) for k, v in inp.items()}
    out = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                      dirs=dirs, group_rows=G, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["tiny_16x16_t2b", "cls_56x56", "dit_16x16",
                                  "local_128x128_g8"])
def test_workload_full_size(name):
    w = WORKLOADS[name]
    print(f"[parity] {name} plan={g.plan_name(w.B, w.C, w.H, w.W, w.dirs, w.group_rows, 0 if w.dtype == 'f32' else 1)}", flush=True)
    inp = make_inputs(w)
    out = run(inp, w.dirs, w.group_rows)
    err = assert_parity(out, oracle_y(inp, w.dirs, w.group_rows), name)
    print(f"[parity] {name} scaled error {err:.3e}", flush=True)


def test_t2i_full_size_sampled_planes():
    """The 2048x1024x320 bf16 workload at full size, in the launch
    configuration the benchmark times; the oracle checks sampled planes."""
    w = WORKLOADS["t2i_2048x1024"]
    print("[parity] t2i full size, generating on device", flush=True)
    d = make_inputs(w, device=DEV)
    out = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                      dirs=w.dirs, group_rows=w.group_rows)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # the two plane groups of the pipeline (two streams) meet at 159 / 160
    for c in (0, 137, 159, 160, 319):
        inp = {k: v[:, c:c + 1].cpu() for k, v in d.items()}
        err = assert_parity(out[:, c:c + 1], oracle_y(inp, w.dirs, 0), f"t2i plane {c}")
        print(f"[parity] t2i plane {c} scaled error {err:.3e}", flush=True)


@pytest.mark.parametrize("shape,plan", [((1, 320, 1024, 2048), "tpipe"),
                                        ((1, 64, 2048, 2048), "tpipe"),
                                        ((1, 320, 2047, 1023), "large")],
                         ids=["portrait_1024x2048", "square_2048x2048", "odd_2047x1023"])
def test_large_planes_off_the_pipeline_full_size(shape, plan):
    """Latents of the text-to-image size in other orientations and sizes
    (the pages' model runs at arbitrary resolution): planes wider than 1024
    take the pipeline with its 1024-thread row sweeps, odd sides the
    transposed-copy passes. Sampled planes at full size, both plane groups
    where there are two."""
    B, C, H, W = shape
    assert g.plan_name(B, C, H, W, 15, 0, 1) == plan
    print(f"[parity] {shape} plan={plan}, generating on device", flush=True)
    d = make_inputs(WORKLOADS["t2i_2048x1024"], device=DEV, B=B, C=C, H=H, W=W)
    out = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], dirs=15)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    for c in sorted({0, C // 2 - 1, C // 2, C - 1}):
        inp = {k: v[:, c:c + 1].cpu() for k, v in d.items()}
        err = assert_parity(out[:, c:c + 1], oracle_y(inp, 15, 0), f"{shape} plane {c}")
        print(f"[parity] {shape} plane {c} scaled error {err:.3e}", flush=True)


SHAPES = [
    (1, 1, 1, 1), (1, 3, 1, 7), (2, 2, 7, 1), (1, 5, 16, 16), (3, 3, 13, 11),
    (1, 2, 17, 16), (2, 3, 64, 64), (1, 3, 63, 61), (1, 2, 65, 64), (1, 2, 64, 65),
    (1, 1, 100, 300), (1, 2, 300, 100), (1, 1, 1, 1000), (1, 1, 777, 1), (1, 1, 3, 9000),
    (1, 1, 5000, 2),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(shape, dtype):
    B, C, H, W = shape
    base = WORKLOADS["cls_56x56"]
    w = base if dtype == torch.float32 else WORKLOADS["dit_16x16"]
    inp = make_inputs(w, seed=hash(shape) % 10000, B=B, C=C, H=H, W=W)
    for G in (0, 3):
        out = run(inp, 15, G)
        assert_parity(out, oracle_y(inp, 15, G), f"{shape} G={G}")


@pytest.mark.parametrize("shape", [(1, 6, 16, 16), (2, 2, 40, 24), (1, 2, 96, 80)],
                         ids=["plane16", "plane64", "stream"])
def test_every_direction_mask(shape):
    B, C, H, W = shape
    inp = make_inputs("cls_56x56", seed=21, B=B, C=C, H=H, W=W)
    for mask in range(1, 16):
        out = run(inp, mask, 0)
        assert_parity(out, oracle_y(inp, mask, 0), f"{shape} mask={mask}")


@pytest.mark.parametrize("shape", [(1, 4, 16, 16), (1, 2, 48, 40), (1, 2, 130, 70)])
@pytest.mark.parametrize("G", [1, 2, 5, 8, 16, 1000])
def test_local_groups(shape, G):
    B, C, H, W = shape
    inp = make_inputs("local_128x128_g8", seed=31 + G, B=B, C=C, H=H, W=W)
    out = run(inp, 15, G)
    assert_parity(out, oracle_y(inp, 15, G), f"{shape} G={G}")


@pytest.mark.parametrize("C,cl", [(5, 5), (4, 1), (300, 300)], ids=["C5", "C4_Cl1", "C300"])
@pytest.mark.parametrize("G", [0, 5])
def test_plane64_fp32_producer_consumer(monkeypatch, C, cl, G):
    """fp32 planes of 64 x 64 take the producer / consumer kernel: every
    direction subset against the oracle (sampled planes when there are more
    planes than CUs, so that each workgroup runs several groups), and the
    same bits as the one-role kernel."""
    inp = make_inputs("cls_56x56", seed=C + G, B=2, C=C, H=64, W=64)
    if cl != C:
        inp = {k: (v[:, :cl].contiguous() if k in ("l0", "l1", "l2") else v)
               for k, v in inp.items()}
    for mask in (15, 1, 8, 6):
        monkeypatch.delenv("GSPN_PLANE_PC", raising=False)
        out = run(inp, mask, G)
        monkeypatch.setenv("GSPN_PLANE_PC", "0")
        one = run(inp, mask, G)
        assert torch.equal(out, one), f"C={C} Cl={cl} G={G} mask={mask}"
        planes = [0, 1, C - 1] if C > 8 else list(range(C))
        for c in planes:
            sub = {k: v[:, c:c + 1] if v.shape[1] == C else v for k, v in inp.items()}
            assert_parity(out[:, c:c + 1], oracle_y(sub, mask, G), f"C={C} plane {c} mask={mask}")


@pytest.mark.parametrize("plan,shape", [("plane", (1, 3, 16, 16)), ("plane", (1, 2, 56, 56)),
                                        ("band", (1, 2, 66, 40)), ("tpipe", (1, 2, 66, 40)),
                                        ("tpipe_t", (1, 2, 40, 130)), ("large", (1, 3, 65, 67)),
                                        ("stream", (1, 2, 66, 40))],
                         ids=lambda v: v if isinstance(v, str) else "x".join(map(str, v)))
def test_bf16_store_rounds_to_nearest_even(force_plan, plan, shape):
    """With a restart at every step (G = 1) the state is lambda * x, exact in
    fp32 for bf16 inputs (16 significant bits at most), and with u = 1 and one
    direction the stored output is that product rounded once to bf16: it must
    be the nearest bf16 value, ties to even, bit for bit. Random mantissas
    give about one tie in 256 products."""
    force_plan(plan)
    B, C, H, W = shape
    gen = torch.Generator().manual_seed(H * W + C)
    def rnd():
        m = 1.0 + torch.rand(shape, generator=gen, dtype=torch.float64)
        e = torch.randint(-20, 20, shape, generator=gen).to(torch.float64)
        sgn = torch.where(torch.rand(shape, generator=gen) < 0.5, -1.0, 1.0).to(torch.float64)
        return (sgn * m * torch.exp2(e)).to(torch.bfloat16)
    x, lam = rnd(), rnd()
    lg = [torch.randn(shape, generator=gen).to(torch.bfloat16) for _ in range(3)]
    u = torch.ones(shape, dtype=torch.bfloat16)
    want = (lam.float() * x.float()).to(torch.bfloat16)
    d = [t.to(DEV) for t in (x, *lg, lam, u)]
    for mask in (1, 4):
        assert g.plan_name(B, C, H, W, mask, 1, 1).startswith(plan)
        out = g.propagate(d[0], (d[1], d[2], d[3]), d[4], d[5], dirs=mask, group_rows=1)
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), \
            f"{plan} {shape} mask={mask}: {(got != want).sum().item()} elements differ"


@pytest.mark.parametrize("shape", [(2, 3, 16, 16), (1, 2, 56, 56), (1, 2, 200, 150)])
def test_row_stochastic_invariant(shape):
    """lambda = x = u = 1: y = H + W + 2 everywhere (Theorem 1)."""
    B, C, H, W = shape
    inp = make_inputs("cls_56x56", seed=5, B=B, C=C, H=H, W=W)
    for k in ("x", "lam", "u"):
        inp[k] = torch.ones_like(inp[k])
    out = run(inp, 15, 0)
    assert torch.allclose(out.cpu(), torch.full(shape, float(H + W + 2)), rtol=2e-6, atol=0)


@pytest.mark.parametrize("shape", [(1, 2, 16, 16), (1, 2, 50, 60), (1, 1, 150, 90)])
def test_one_hot_middle_weight(shape):
    """l0 = l2 = -inf: w = I, so the scan is a per-line prefix sum."""
    B, C, H, W = shape
    inp = make_inputs("cls_56x56", seed=9, B=B, C=C, H=H, W=W)
    inp["l0"] = torch.full(shape, -float("inf"))
    inp["l2"] = torch.full(shape, -float("inf"))
    for mask in (1, 2, 4, 8, 15):
        out = run(inp, mask, 0)
        assert_parity(out, oracle_y(inp, mask, 0), f"one-hot {shape} mask={mask}")


@pytest.mark.parametrize("shape,dtype", [((4, 8, 56, 56), torch.float32),
                                         ((2, 16, 16, 16), torch.bfloat16),
                                         ((1, 3, 300, 200), torch.bfloat16),
                                         ((1, 4, 96, 300), torch.float32),
                                         ((1, 4, 128, 300), torch.bfloat16)])
def test_deterministic(shape, dtype):
    """Bitwise-identical repeats (no atomics; catches LDS races between
    steps, e.g. with idle threads in a partly filled workgroup)."""
    B, C, H, W = shape
    w = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(w, seed=2, B=B, C=C, H=H, W=W)
    a = run(inp, 15, 0)
    for mask in (15, 1, 8):
        ref = run(inp, mask, 0)
        for _ in range(3):
            assert torch.equal(run(inp, mask, 0), ref)
    assert torch.equal(run(inp, 15, 0), a)


def test_alloc_entry_point_matches_workspace_entry_point():
    inp = {k: v.to(DEV) for k, v in make_inputs("cls_56x56", seed=4, B=1, C=3, H=130, W=90).items()}
    args = (inp["x"], (inp["l0"], inp["l1"], inp["l2"]), inp["lam"], inp["u"])
    a = g.propagate(*args, dirs=15, group_rows=0)
    b = g.propagate_alloc(*args, dirs=15, group_rows=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_side_stream():
    inp = {k: v.to(DEV) for k, v in make_inputs("dit_16x16", seed=6, B=2, C=8).items()}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = g.propagate(inp["x"], (inp["l0"], inp["l1"], inp["l2"]), inp["lam"], inp["u"])
    s.synchronize()
    ref = oracle_y({k: v.cpu() for k, v in inp.items()}, 15, 0)
    assert_parity(out, ref, "side stream")


def test_binding_rejects_mismatched_tensors():
    x = torch.zeros(1, 1, 4, 4, device=DEV)
    y = torch.zeros(1, 1, 4, 5, device=DEV)
    with pytest.raises(ValueError):
        g.propagate(x, (x, x, x), x, y)
    with pytest.raises(g.GspnError) as ei:
        g.propagate(x, (x, x, x), x, x, dirs=0)
    assert ei.value.name == "GSPN_E_DIRMASK"


FORCED_SHAPES = [(1, 2, 2, 2), (1, 2, 8, 8), (2, 3, 16, 32), (1, 2, 66, 40), (1, 1, 130, 96),
                 (1, 2, 40, 130), (2, 1, 48, 1024), (1, 1, 2048, 64),
                 # wider than 1024: 1024-thread row sweeps, 4-row chunks (H % 4 == 2
                 # leaves a ragged last chunk)
                 (1, 2, 10, 1026), (2, 1, 34, 1500), (1, 1, 64, 2048)]


@pytest.fixture
def force_plan(monkeypatch):
    def _set(name):
        monkeypatch.setenv("GSPN_FORCE_PLAN", name)
    return _set


@pytest.mark.parametrize("plan", ["tpipe", "stream"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", FORCED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forced_plan(force_plan, plan, shape, dtype):
    """Each large-plane path on small and odd-sized planes, every direction
    subset family, global and local."""
    force_plan(plan)
    B, C, H, W = shape
    assert g.plan_name(B, C, H, W, 15, 0, 0 if dtype == torch.float32 else 1) == plan
    w = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(w, seed=(H * 31 + W) % 997, B=B, C=C, H=H, W=W)
    for mask in (15, 1, 2, 3, 4, 8, 12, 5, 10):
        for G in ((0, 3, 8) if mask == 15 else (0,)):
            out = run(inp, mask, G)
            assert_parity(out, oracle_y(inp, mask, G), f"{plan} {shape} mask={mask} G={G}")


# the pipeline on transposed copies: every shape whose transpose the pipeline
# takes (W <= 2048, H <= 1024, both even)
TPIPE_T_SHAPES = [(1, 2, 2, 2), (1, 2, 8, 8), (2, 3, 16, 32), (1, 2, 66, 40), (1, 1, 130, 96),
                  (1, 2, 40, 130), (2, 1, 48, 1024), (1, 1, 64, 2048)]
# the transposed-copy passes: planes above 64 x 64, odd sides included
LARGE_SHAPES = [(1, 2, 66, 40), (1, 1, 130, 96), (1, 2, 40, 130), (1, 3, 65, 67),
                (1, 1, 129, 33), (2, 1, 97, 255), (1, 1, 3, 300)]


@pytest.mark.parametrize("plan,shape", [("tpipe_t", s) for s in TPIPE_T_SHAPES] +
                         [("large", s) for s in LARGE_SHAPES],
                         ids=lambda v: v if isinstance(v, str) else "x".join(map(str, v)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_forced_large_plane_plans(force_plan, plan, shape, dtype):
    """The plans for large planes the pipeline does not take, forced on small
    and odd planes: every direction-subset family, global and local."""
    force_plan(plan)
    B, C, H, W = shape
    assert g.plan_name(B, C, H, W, 15, 0, 0 if dtype == torch.float32 else 1) == plan
    w = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(w, seed=(H * 37 + W) % 997, B=B, C=C, H=H, W=W)
    for mask in (15, 1, 2, 3, 4, 8, 12, 5, 10):
        for G in ((0, 3, 8) if mask == 15 else (0,)):
            out = run(inp, mask, G)
            assert_parity(out, oracle_y(inp, mask, G), f"{plan} {shape} mask={mask} G={G}")


@pytest.mark.parametrize("plan", ["tpipe_t", "large"])
def test_large_plane_plans_shared_logits(force_plan, plan):
    """Logits shared by groups of channels on the large-plane plans (the
    transposed-copy passes hand them to the streaming path)."""
    force_plan(plan)
    B, C, H, W = 2, 4, 66, 130
    inp = make_inputs("dit_16x16", seed=77, B=B, C=C, H=H, W=W)
    for k in ("l0", "l1", "l2"):
        inp[k] = inp[k][:, :2].contiguous()    # two logit channels shared by pairs
    out = run(inp, 15, 0)
    assert_parity(out, oracle_y(inp, 15, 0), f"{plan} shared logits")


BAND_SHAPES = [(1, 2, 72, 40), (2, 1, 128, 128), (1, 1, 100, 70), (1, 2, 66, 130),
               (1, 1, 160, 96), (1, 1, 8, 300)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", BAND_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_band_plan(force_plan, shape, dtype):
    """Band-resident local plan: group sizes 1..16 (ragged last bands included),
    every direction-mask family."""
    force_plan("band")
    B, C, H, W = shape
    w = "local_128x128_g8" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(w, seed=(H * 7 + W) % 991, B=B, C=C, H=H, W=W)
    for G in (1, 2, 3, 5, 8, 13, 16):
        assert g.plan_name(B, C, H, W, 15, G, 0 if dtype == torch.float32 else 1) == "band"
        masks = (15, 1, 2, 4, 8, 3, 12, 5, 10) if G in (3, 8) else (15,)
        for mask in masks:
            out = run(inp, mask, G)
            assert_parity(out, oracle_y(inp, mask, G), f"band {shape} mask={mask} G={G}")


def _offset_view(t, off):
    """A contiguous copy of t that starts `off` elements into its allocation."""
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=DEV)
    v = buf[off:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape,G,plan", [
    ((1, 3, 16, 16), 0, "plane16"), ((1, 2, 56, 56), 0, "plane64"),
    ((1, 2, 128, 128), 8, "band"), ((1, 1, 96, 64), 16, "band"),
    ((1, 2, 130, 96), 0, "tpipe"), ((1, 1, 65, 80), 0, "stream")],
    ids=["plane16", "plane64", "band8", "band16", "tpipe", "stream"])
@pytest.mark.parametrize("off", [1, 2, 3])
def test_element_offset_views(shape, G, plan, dtype, off):
    """Tensors that start 1-3 elements into their allocation (naturally
    aligned, but not to the 8- or 16-byte vectors the fast paths use) take
    the element-wise code and still match the oracle."""
    B, C, H, W = shape
    dt = 0 if dtype == torch.float32 else 1
    assert g.plan_name(B, C, H, W, 15, G, dt) == plan
    w = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(w, seed=17 + off, B=B, C=C, H=H, W=W)
    d = {k: _offset_view(v.to(DEV), off) for k, v in inp.items()}
    out = _offset_view(torch.zeros(shape, dtype=dtype, device=DEV), off)
    g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], dirs=15, group_rows=G,
                out=out)
    torch.cuda.synchronize()
    assert_parity(out, oracle_y(inp, 15, G), f"{plan} offset {off}")


@pytest.mark.parametrize("plan", ["tpipe", "tpipe_t"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_pipeline_plane_groups(force_plan, monkeypatch, plan, dtype):
    """The pipelines with one to four plane groups on their own streams
    (GSPN_TPIPE_GROUPS): each group count matches the oracle, and all of them
    give the same bits, since every plane is computed the same way whichever
    group and stream it runs in. 11 planes put group boundaries inside an
    image."""
    force_plan(plan)
    w = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(w, seed=611, B=1, C=11, H=34, W=66)
    for mask, G in ((15, 0), (15, 3), (3, 0), (12, 0)):
        ref = oracle_y(inp, mask, G)
        outs = []
        for n in (1, 2, 3, 4):
            monkeypatch.setenv("GSPN_TPIPE_GROUPS", str(n))
            print(f"[parity] {plan} groups={n} mask={mask} G={G}", flush=True)
            outs.append(run(inp, mask, G))
            assert_parity(outs[-1], ref, f"{plan} groups={n} mask={mask} G={G}")
        for o in outs[1:]:
            assert torch.equal(o, outs[0])
