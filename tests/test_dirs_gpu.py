"""Per-direction parameters with a per-channel merger on the GPU against the
fp64 oracle (needs an MI355X). Every case goes through the C ABI
(gspn_propagate_dirs_ws, via the binding or directly)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import linear_spatial_propagation_line_amd as g
import oracle
from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_inputs
from parity import assert_parity, oracle_y, to_oracle_array

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("l0", "l1", "l2", "lam", "u")


def dirs_case(shape, dtype, seed):
    name = "cls_56x56_pd" if dtype == torch.float32 else "t2i_2048x1024_pd"
    B, C, H, W = shape
    return make_inputs(name, seed=seed, B=B, C=C, H=H, W=W)


def oracle_dirs(inp, dirs, G, merge=True):
    arrs = [to_oracle_array(inp["x"])] + [to_oracle_array(inp[k]) for k in KEYS]
    m = inp["merge"].double().cpu().numpy() if merge else None
    return oracle.propagate_dirs(*arrs, merge=m, dirs=dirs, group_rows=G)


def run_dirs(inp, dirs, G, merge=True, **kw):
    d = {k: v.to(DEV) for k, v in inp.items()}
    out = g.propagate_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                           merge=d["merge"] if merge else None, dirs=dirs, group_rows=G, **kw)
    torch.cuda.synchronize()
    return out


# shapes that reach every launch configuration: vertical passes with 1, 2, 4
# and 8 columns per thread, horizontal passes with 1, 2, 4 and 8 rows per
# thread, 16-byte runs and element runs (widths that no run length divides),
# single rows and columns, ragged last wavefronts
SHAPES = [(1, 1, 1, 1), (1, 2, 1, 7), (1, 2, 7, 1), (2, 3, 16, 16), (2, 2, 13, 11),
          (1, 3, 56, 56), (1, 2, 65, 64), (1, 2, 64, 72), (1, 1, 100, 300), (1, 1, 300, 100),
          (1, 1, 1030, 40), (1, 1, 40, 1030), (1, 1, 2050, 24), (1, 1, 24, 2050),
          (1, 1, 4100, 16), (1, 1, 16, 4100), (1, 1, 3, 8192), (1, 1, 8192, 3)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(shape, dtype):
    print(f"[dirs] shape={shape} dtype={dtype}", flush=True)
    for G in (0, 3):
        inp = dirs_case(shape, dtype, 31 + shape[2] + shape[3])
        out = run_dirs(inp, 15, G)
        assert_parity(out, oracle_dirs(inp, 15, G), f"dirs {shape} G={G}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_every_mask(dtype):
    shape = (2, 3, 24, 40)
    inp = dirs_case(shape, dtype, 5)
    for mask in range(1, 16):
        for merge in (True, False):
            out = run_dirs(inp, mask, 0, merge=merge)
            assert_parity(out, oracle_dirs(inp, mask, 0, merge=merge),
                          f"dirs mask={mask} merge={merge}")


@pytest.mark.parametrize("G", [1, 2, 5, 8, 16, 1000])
@pytest.mark.parametrize("shape", [(1, 2, 37, 45), (1, 2, 36, 44), (1, 2, 70, 66)],
                         ids=["small", "small-runs", "large"])
def test_local_groups(G, shape):
    """Local groups on the one-wavefront path (element loads, and 4-column
    runs) and on the large-plane path."""
    for dtype in (torch.float32, torch.bfloat16):
        inp = dirs_case(shape, dtype, 11 + G)
        assert_parity(run_dirs(inp, 15, G), oracle_dirs(inp, 15, G), f"dirs G={G}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_plane_groups(dtype, monkeypatch):
    """Planes wider than 64 (the plane-group path): more planes than compute
    units (and fewer than twice as many) split into plane groups on their own
    streams; 300 planes of 100 channels put the group boundary inside an
    image. Three groups are forced on 10 planes as well, over every mask
    family."""
    inp = dirs_case((3, 100, 8, 66), dtype, 93)
    for G in (0, 4):
        assert_parity(run_dirs(inp, 15, G), oracle_dirs(inp, 15, G), f"dirs 300 planes G={G}")
    monkeypatch.setenv("GSPN_TPIPE_GROUPS", "3")
    inp = dirs_case((2, 5, 9, 70), dtype, 94)
    for mask in (15, 12, 3, 4, 1):
        assert_parity(run_dirs(inp, mask, 0), oracle_dirs(inp, mask, 0),
                      f"dirs three groups mask={mask}")


def test_stride_zero_is_the_shared_layer():
    """dir_stride = 0 and no merge weights through the C ABI: every direction
    reads the same [B, C, H, W] tensors, so the result is the shared layer's,
    checked against the shared-parameter oracle."""
    for dtype, name in ((torch.float32, "cls_56x56"), (torch.bfloat16, "dit_16x16")):
        inp = make_inputs(name, seed=3, B=2, C=3, H=30, W=20)
        d = {k: v.to(DEV) for k, v in inp.items()}
        out = torch.empty_like(d["x"])
        B, C, H, W = d["x"].shape
        dt = g.GSPN_F32 if dtype == torch.float32 else g.GSPN_BF16
        ws = torch.empty(g.workspace_bytes_dirs(B, C, H, W, 15, 0, dt), dtype=torch.uint8,
                         device=DEV)
        lg = (ctypes.c_void_p * 3)(d["l0"].data_ptr(), d["l1"].data_ptr(), d["l2"].data_ptr())
        st = g.lib().gspn_propagate_dirs_ws(
            d["x"].data_ptr(), lg, d["lam"].data_ptr(), d["u"].data_ptr(), 0, None, B, C, H, W,
            15, 0, dt, out.data_ptr(), ws.data_ptr(), ws.numel(),
            torch.cuda.current_stream().cuda_stream)
        assert st == 0, g.lib().gspn_last_error()
        torch.cuda.synchronize()
        assert_parity(out, oracle_y(inp, 15, 0), f"dirs stride 0 {dtype}")


def test_merge_weights_are_per_channel_and_direction():
    """Zero merge weights except one (direction, channel) pair: out is that
    direction's gated scan in that channel and exactly zero elsewhere."""
    shape = (2, 3, 20, 28)
    inp = dirs_case(shape, torch.float32, 9)
    for d, c in ((0, 0), (1, 2), (2, 1), (3, 2)):
        m = torch.zeros(4, 3)
        m[d, c] = 1.0
        inp["merge"] = m
        out = run_dirs(inp, 15, 0).cpu()
        assert torch.count_nonzero(out[:, [k for k in range(3) if k != c]]) == 0
        assert_parity(out, oracle_dirs(inp, 15, 0), f"dirs single merge weight {d},{c}")


def test_offset_views_take_the_element_path():
    """Tensors that start one element into their allocation (no aligned
    vector runs) give the oracle's result too."""
    for shape, dtype in [((1, 2, 40, 1032), torch.float32), ((1, 2, 40, 1032), torch.bfloat16),
                         ((1, 2, 20, 36), torch.float32), ((1, 2, 20, 36), torch.bfloat16)]:
        inp = dirs_case(shape, dtype, 21)
        d = {}
        for k, v in inp.items():
            if k == "merge":
                d[k] = v.to(DEV)
                continue
            buf = torch.zeros(v.numel() + 1, dtype=v.dtype, device=DEV)
            buf[1:].copy_(v.reshape(-1).to(DEV))
            d[k] = buf[1:].view(v.shape)
        out = torch.zeros(shape[0] * shape[1] * shape[2] * shape[3] + 1, dtype=dtype,
                          device=DEV)[1:].view(shape)
        g.propagate_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                         merge=d["merge"], out=out)
        torch.cuda.synchronize()
        assert_parity(out, oracle_dirs(inp, 15, 0), f"dirs offset views {dtype}")


def test_deterministic():
    inp = dirs_case((2, 4, 70, 90), torch.bfloat16, 13)
    a = run_dirs(inp, 15, 0)
    b = run_dirs(inp, 15, 0)
    assert torch.equal(a, b)


def test_binding_errors():
    inp = dirs_case((1, 2, 8, 8), torch.float32, 1)
    d = {k: v.to(DEV) for k, v in inp.items()}
    with pytest.raises(ValueError):
        g.propagate_dirs(d["x"], (d["l0"][0], d["l1"], d["l2"]), d["lam"], d["u"])
    with pytest.raises(ValueError):
        g.propagate_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                         merge=d["merge"][:, :1].contiguous())
    with pytest.raises(g.GspnError):
        g.propagate_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                         out=d["lam"][2])   # out is direction 2's lambda


def test_cls_pd_full_size():
    """The 64x96x56x56 fp32 per-direction workload at full size."""
    w = WORKLOADS["cls_56x56_pd"]
    inp = make_inputs(w)
    out = run_dirs(inp, w.dirs, w.group_rows)
    err = assert_parity(out, oracle_dirs(inp, w.dirs, w.group_rows), w.name)
    print(f"[dirs] {w.name} scaled error {err:.3e}", flush=True)


def test_t2i_pd_full_size_sampled_planes():
    """The 2048x1024x320 bf16 per-direction workload at full size, as the
    benchmark runs it; the oracle checks sampled planes."""
    w = WORKLOADS["t2i_2048x1024_pd"]
    d = make_inputs(w, device=DEV)
    out = g.propagate_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                           merge=d["merge"], dirs=w.dirs)
    torch.cuda.synchronize()
    for c in (0, 177, 319):
        inp = {"x": d["x"][:, c:c + 1].cpu(), "merge": d["merge"][:, c:c + 1].cpu()}
        for k in KEYS:
            inp[k] = d[k][:, :, c:c + 1].contiguous().cpu()
        assert_parity(out[:, c:c + 1], oracle_dirs(inp, w.dirs, 0), f"t2i pd plane {c}")
