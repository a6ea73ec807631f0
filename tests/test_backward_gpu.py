"""Backward pass on the GPU vs the fp64 oracle's backward, gradient by
gradient, on the same seeded inputs (needs an MI355X). Every call goes
through the C ABI via the binding."""
from __future__ import annotations

import pytest
import torch

import linear_spatial_propagation_line_amd as g
from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_grad_out, make_inputs
from parity import GRAD_NAMES, assert_grad_parity, oracle_grads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_bwd(inp, gy, dirs, G, **kw):
    d = {k: v.to(DEV) for k, v in inp.items()}
    grads = g.propagate_backward(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                 gy.to(DEV), dirs=dirs, group_rows=G, **kw)
    torch.cuda.synchronize()
    return grads


def case(name, seed, **shape):
    return make_inputs(name, seed=seed, **shape), make_grad_out(name, seed=seed + 7, **shape)


@pytest.mark.parametrize("name,planes", [("tiny_16x16_t2b", None), ("cls_56x56", (8, 96)),
                                         ("dit_16x16", (4, 1152)),
                                         ("local_128x128_g8", (2, 192))])
def test_workload_shapes(name, planes):
    """The workloads' plane shapes, dtypes, direction sets and groups (fewer
    planes than the benchmark: the fp64 oracle backward is slow)."""
    w = WORKLOADS[name]
    B, C = planes if planes else (w.B, w.C)
    print(f"[bwd] {name} B={B} C={C} plan={g.backward_plan_name(B, C, w.H, w.W, w.dirs, w.group_rows, 0 if w.dtype == 'f32' else 1)}", flush=True)
    inp, gy = case(name, 5, B=B, C=C)
    got = run_bwd(inp, gy, w.dirs, w.group_rows)
    err = assert_grad_parity(got, oracle_grads(inp, gy, w.dirs, w.group_rows), name)
    print(f"[bwd] {name} worst scaled error {err:.3e}", flush=True)


SHAPES = [(1, 1, 1, 1), (1, 2, 1, 7), (1, 2, 7, 1), (1, 3, 16, 16), (2, 2, 13, 11),
          (1, 2, 17, 16), (1, 2, 64, 64), (1, 2, 65, 64), (1, 1, 100, 300), (1, 1, 300, 100),
          (1, 1, 1, 1000), (1, 1, 777, 1), (1, 1, 1030, 40), (1, 1, 3, 9000), (1, 1, 5000, 2)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(shape, dtype):
    B, C, H, W = shape
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, hash(shape) % 10000, B=B, C=C, H=H, W=W)
    for G in (0, 3):
        got = run_bwd(inp, gy, 15, G)
        assert_grad_parity(got, oracle_grads(inp, gy, 15, G), f"{shape} G={G}")


@pytest.mark.parametrize("shape", [(1, 3, 16, 16), (1, 2, 40, 24), (1, 2, 96, 80)])
def test_every_direction_mask(shape):
    B, C, H, W = shape
    inp, gy = case("cls_56x56", 21, B=B, C=C, H=H, W=W)
    for mask in range(1, 16):
        got = run_bwd(inp, gy, mask, 0)
        assert_grad_parity(got, oracle_grads(inp, gy, mask, 0), f"{shape} mask={mask}")


@pytest.mark.parametrize("shape", [(1, 4, 16, 16), (1, 2, 48, 40), (1, 2, 130, 70)])
@pytest.mark.parametrize("G", [1, 2, 5, 8, 16, 1000])
def test_local_groups(shape, G):
    B, C, H, W = shape
    inp, gy = case("local_128x128_g8", 33 + G, B=B, C=C, H=H, W=W)
    got = run_bwd(inp, gy, 15, G)
    assert_grad_parity(got, oracle_grads(inp, gy, 15, G), f"{shape} G={G}")


@pytest.mark.parametrize("shape", [(1, 2, 16, 16), (1, 2, 56, 56), (1, 1, 150, 90)])
def test_invariant_zero_logit_gradients(shape):
    """Theorem 1: with lambda x = 1 every predecessor of a pixel holds the same
    state, so the logit gradients vanish. In fp32 the neighbouring states still
    differ by rounding (sum_k w_k is 1 only to ~1 ulp), so the logit gradients
    are bounded by a few ulps of e * h instead of compared with the oracle's
    zeros; the other gradients are compared as usual."""
    B, C, H, W = shape
    inp, gy = case("cls_56x56", 8, B=B, C=C, H=H, W=W)
    inp["x"] = torch.ones_like(inp["x"])
    inp["lam"] = torch.ones_like(inp["lam"])
    got = run_bwd(inp, gy, 15, 0)
    assert_grad_parity(got, oracle_grads(inp, gy, 15, 0), f"invariant {shape}",
                       names=("x", "lam", "u"))
    e_max = got["x"].abs().max().item()          # lambda = 1: dx = sum_d e_d
    h_max = float(H + W + 2)                     # sum_d h_d under Theorem 1
    for k in ("l0", "l1", "l2"):
        assert got[k].abs().max().item() <= 1e-5 * e_max * h_max, k


def test_alloc_entry_point_matches_workspace_entry_point():
    inp, gy = case("cls_56x56", 4, B=1, C=3, H=70, W=90)
    a = run_bwd(inp, gy, 15, 0)
    b = run_bwd(inp, gy, 15, 0, alloc=True)
    for k in GRAD_NAMES:
        assert torch.equal(a[k], b[k]), k


def test_deterministic():
    inp, gy = case("cls_56x56", 9, B=2, C=4, H=56, W=56)
    a = run_bwd(inp, gy, 15, 0)
    for _ in range(2):
        b = run_bwd(inp, gy, 15, 0)
        for k in GRAD_NAMES:
            assert torch.equal(a[k], b[k]), k


def test_binding_rejects_aliased_gradients():
    x = torch.zeros(1, 1, 4, 4, device=DEV)
    t = [torch.zeros_like(x) for _ in range(6)]
    grads = dict(zip(GRAD_NAMES, t))
    grads["u"] = grads["x"]
    with pytest.raises(g.GspnError) as ei:
        g.propagate_backward(x, (t[0], t[1], t[2]), t[3], t[4], t[5], grads=grads)
    assert ei.value.name == "GSPN_E_ALIAS"


@pytest.fixture
def force_bwd_plan(monkeypatch):
    def _set(name):
        monkeypatch.setenv("GSPN_FORCE_BWD_PLAN", name)
    return _set


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 3, 16, 16), (2, 2, 13, 11), (1, 2, 40, 24),
                                   (1, 1, 64, 64), (1, 2, 1, 9)],
                         ids=lambda s: "x".join(map(str, s)))
def test_streaming_path_on_small_planes(force_bwd_plan, shape, dtype):
    """The general backward path forced onto shapes the plane-resident path
    normally takes, every direction subset family, global and local."""
    force_bwd_plan("stream")
    B, C, H, W = shape
    assert g.backward_plan_name(B, C, H, W) == "bwd_stream"
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, 50 + H, B=B, C=C, H=H, W=W)
    for mask in (15, 1, 2, 4, 8, 5, 10):
        for G in ((0, 3) if mask == 15 else (0,)):
            got = run_bwd(inp, gy, mask, G)
            assert_grad_parity(got, oracle_grads(inp, gy, mask, G),
                               f"stream {shape} mask={mask} G={G}")


def _offset_view(t, off):
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=DEV)
    v = buf[off:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 3, 16, 16), (1, 2, 56, 56), (1, 1, 70, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_element_offset_views(shape, dtype):
    """Tensors starting 1 element into their allocation take the element-wise
    loads and stores and still match the oracle."""
    B, C, H, W = shape
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, 61, B=B, C=C, H=H, W=W)
    d = {k: _offset_view(v.to(DEV), 1) for k, v in inp.items()}
    gyd = _offset_view(gy.to(DEV), 1)
    grads = {k: _offset_view(torch.zeros(shape, dtype=dtype, device=DEV), 1) for k in GRAD_NAMES}
    g.propagate_backward(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], gyd,
                         grads=grads)
    torch.cuda.synchronize()
    assert_grad_parity(grads, oracle_grads(inp, gy, 15, 0), f"offset {shape}")


def test_plane_path_matches_streaming_path(force_bwd_plan):
    """Both backward paths on the same classification-stage planes agree to
    the fp32 bound (they round differently, so not bitwise)."""
    inp, gy = case("cls_56x56", 71, B=2, C=8)
    a = run_bwd(inp, gy, 15, 0)
    force_bwd_plan("stream")
    b = run_bwd(inp, gy, 15, 0)
    ref = {k: a[k].double().cpu().numpy() for k in GRAD_NAMES}
    assert_grad_parity(b, ref, "plane vs stream")


def test_t2i_full_size_sampled_planes():
    """The 2048x1024x320 bf16 workload at full size, as the benchmark runs it;
    the fp64 oracle checks sampled planes."""
    w = WORKLOADS["t2i_2048x1024"]
    print("[bwd] t2i full size, generating on device", flush=True)
    d = make_inputs(w, device=DEV)
    gy = make_grad_out(w, device=DEV)
    grads = g.propagate_backward(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], gy,
                                 dirs=w.dirs, group_rows=w.group_rows)
    torch.cuda.synchronize()
    for c in (0, 211):
        inp = {k: v[:, c:c + 1].cpu() for k, v in d.items()}
        got = {k: v[:, c:c + 1] for k, v in grads.items()}
        err = assert_grad_parity(got, oracle_grads(inp, gy[:, c:c + 1].cpu(), w.dirs, 0),
                                 f"t2i plane {c}")
        print(f"[bwd] t2i plane {c} worst scaled error {err:.3e}", flush=True)


def test_portrait_full_size_sampled_planes():
    """The text-to-image latent in portrait orientation (1024 x 2048 x 320
    bf16): wider than the backward pipeline's row sweeps, so it runs the
    pipeline on transposed copies; sampled planes of both plane groups."""
    w = WORKLOADS["t2i_2048x1024"]
    B, C, H, W = 1, 320, 1024, 2048
    assert g.backward_plan_name(B, C, H, W, w.dirs, 0, 1) == "bwd_tpipe_t"
    print("[bwd] portrait full size, generating on device", flush=True)
    d = make_inputs(w, device=DEV, B=B, C=C, H=H, W=W)
    gy = make_grad_out(w, device=DEV, B=B, C=C, H=H, W=W)
    grads = g.propagate_backward(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], gy,
                                 dirs=w.dirs, group_rows=0)
    torch.cuda.synchronize()
    for c in (0, 159, 160, 319):
        inp = {k: v[:, c:c + 1].cpu() for k, v in d.items()}
        got = {k: v[:, c:c + 1] for k, v in grads.items()}
        err = assert_grad_parity(got, oracle_grads(inp, gy[:, c:c + 1].cpu(), w.dirs, 0),
                                 f"portrait plane {c}")
        print(f"[bwd] portrait plane {c} worst scaled error {err:.3e}", flush=True)


def test_local_full_size():
    w = WORKLOADS["local_128x128_g8"]
    inp, gy = make_inputs(w), make_grad_out(w)
    got = run_bwd(inp, gy, w.dirs, w.group_rows)
    err = assert_grad_parity(got, oracle_grads(inp, gy, w.dirs, w.group_rows), w.name)
    print(f"[bwd] {w.name} full size worst scaled error {err:.3e}", flush=True)


BAND_SHAPES = [(1, 2, 72, 40), (2, 1, 128, 128), (1, 1, 100, 70), (1, 2, 66, 130),
               (1, 1, 8, 200), (1, 1, 256, 24), (1, 1, 24, 300), (1, 1, 512, 16)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", BAND_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_band_path(force_bwd_plan, shape, dtype):
    """Band-resident backward for local groups 1..8 (ragged last bands
    included) and every direction-mask family."""
    force_bwd_plan("band")
    B, C, H, W = shape
    name = "local_128x128_g8" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, (H * 7 + W) % 991, B=B, C=C, H=H, W=W)
    for G in (1, 2, 3, 5, 8):
        assert g.backward_plan_name(B, C, H, W, 15, G, 0 if dtype == torch.float32 else 1) == "bwd_band"
        masks = (15, 1, 2, 4, 8, 3, 12, 5, 10) if G in (3, 8) else (15,)
        for mask in masks:
            got = run_bwd(inp, gy, mask, G)
            assert_grad_parity(got, oracle_grads(inp, gy, mask, G),
                               f"band {shape} mask={mask} G={G}")


PIPE_SHAPES = [(1, 2, 66, 40), (2, 1, 130, 96), (1, 1, 96, 130), (1, 1, 2, 2), (1, 1, 2, 70),
               (1, 1, 70, 2), (1, 2, 18, 22), (1, 1, 250, 34), (1, 1, 34, 250)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", PIPE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_pipeline_path(force_bwd_plan, shape, dtype):
    """Large-plane backward pipeline forced onto small even planes: one row
    or column pair, rows not a multiple of the 4-row group of the horizontal
    parts, prefetch rings longer than the plane; every direction-mask family,
    global and local groups (a restart line on either side of a pair)."""
    force_bwd_plan("tpipe")
    B, C, H, W = shape
    assert g.backward_plan_name(B, C, H, W) == "bwd_tpipe"
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, 90 + H + W, B=B, C=C, H=H, W=W)
    for G in (0, 1, 3, 8):
        masks = (15, 1, 2, 4, 8, 3, 12, 5, 10) if G in (0, 3) else (15,)
        for mask in masks:
            got = run_bwd(inp, gy, mask, G)
            assert_grad_parity(got, oracle_grads(inp, gy, mask, G),
                               f"pipeline {shape} mask={mask} G={G}")


PIPE_T_SHAPES = [(1, 2, 40, 66), (2, 1, 96, 130), (1, 1, 2, 2), (1, 1, 70, 2), (1, 1, 2, 70),
                 (1, 2, 22, 18), (1, 1, 34, 250), (1, 1, 30, 1100)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", PIPE_T_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_transposed_pipeline_path(force_bwd_plan, shape, dtype):
    """The backward pipeline on transposed copies (the plan of planes wider
    than its row sweeps take), forced onto small even planes: every
    direction-mask family (the mask's axes swap for the transposed planes),
    global and local groups."""
    force_bwd_plan("tpipe_t")
    B, C, H, W = shape
    assert g.backward_plan_name(B, C, H, W) == "bwd_tpipe_t"
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, 70 + H + 3 * W, B=B, C=C, H=H, W=W)
    for G in (0, 1, 3, 8):
        masks = (15, 1, 2, 4, 8, 3, 12, 5, 10) if G in (0, 3) else (15,)
        for mask in masks:
            got = run_bwd(inp, gy, mask, G)
            assert_grad_parity(got, oracle_grads(inp, gy, mask, G),
                               f"transposed pipeline {shape} mask={mask} G={G}")


def test_pipeline_matches_streaming_path(force_bwd_plan):
    """Both large-plane backward paths on the same bf16 planes agree to the
    bf16 bound (they round differently)."""
    inp, gy = case("t2i_2048x1024", 93, B=1, C=3, H=256, W=192)
    force_bwd_plan("tpipe")
    a = run_bwd(inp, gy, 15, 0)
    force_bwd_plan("stream")
    b = run_bwd(inp, gy, 15, 0)
    ref = {k: a[k].double().cpu().numpy() for k in GRAD_NAMES}
    assert_grad_parity(b, ref, "pipeline vs stream")


@pytest.mark.parametrize("plan,shape", [("tpipe", (1, 11, 34, 66)), ("tpipe_t", (1, 11, 66, 34))],
                         ids=lambda v: v if isinstance(v, str) else "x".join(map(str, v)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_pipeline_plane_groups(force_bwd_plan, monkeypatch, plan, shape, dtype):
    """The backward pipelines with one to four plane groups on their own
    streams (GSPN_TPIPE_GROUPS): each group count matches the oracle, and all
    of them give the same bits. 11 planes put group boundaries inside an
    image."""
    force_bwd_plan(plan)
    B, C, H, W = shape
    assert g.backward_plan_name(B, C, H, W) == "bwd_" + plan
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    inp, gy = case(name, 612, B=B, C=C, H=H, W=W)
    for mask, G in ((15, 0), (15, 3), (5, 0)):
        ref = oracle_grads(inp, gy, mask, G)
        first = None
        for n in (1, 2, 3, 4):
            monkeypatch.setenv("GSPN_TPIPE_GROUPS", str(n))
            print(f"[parity] bwd_{plan} groups={n} mask={mask} G={G}", flush=True)
            got = run_bwd(inp, gy, mask, G)
            assert_grad_parity(got, ref, f"bwd_{plan} groups={n} mask={mask} G={G}")
            if first is None:
                first = got
            for k in GRAD_NAMES:
                assert torch.equal(got[k], first[k]), (k, n)
