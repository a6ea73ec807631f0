"""Backward pass of the per-direction layer on the GPU against the fp64
oracle's (needs an MI355X). Every case goes through the C ABI
(gspn_propagate_backward_dirs_ws, via the binding)."""
from __future__ import annotations

import pytest
import torch

import linear_spatial_propagation_line_amd as g
import oracle
from linear_spatial_propagation_line_amd.inputs import WORKLOADS, make_grad_out, make_inputs
from parity import assert_grad_parity, to_oracle_array

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("l0", "l1", "l2", "lam", "u")
NAMES = ("x",) + KEYS + ("merge",)


def case(shape, dtype, seed):
    name = "cls_56x56_pd" if dtype == torch.float32 else "t2i_2048x1024_pd"
    B, C, H, W = shape
    return (make_inputs(name, seed=seed, B=B, C=C, H=H, W=W),
            make_grad_out(name, seed=seed + 5, B=B, C=C, H=H, W=W))


def oracle_bwd(inp, gy, dirs, G, merge=True):
    arrs = [to_oracle_array(inp["x"])] + [to_oracle_array(inp[k]) for k in KEYS]
    m = inp["merge"].double().cpu().numpy() if merge else None
    return oracle.backward_dirs(*arrs, to_oracle_array(gy), merge=m, dirs=dirs, group_rows=G)


def run_bwd(inp, gy, dirs, G, merge=True):
    d = {k: v.to(DEV) for k, v in inp.items()}
    grads = g.propagate_backward_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                      gy.to(DEV), merge=d["merge"] if merge else None, dirs=dirs,
                                      group_rows=G)
    torch.cuda.synchronize()
    return grads


# single pixels, single rows and columns, ragged planes, both scan axes longer
SHAPES = [(1, 1, 1, 1), (1, 2, 1, 7), (1, 2, 7, 1), (2, 3, 16, 16), (2, 2, 13, 11),
          (1, 3, 56, 56), (1, 1, 70, 40), (1, 1, 40, 70), (1, 1, 130, 96)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_edge_shapes(shape, dtype):
    print(f"[dirs bwd] shape={shape} dtype={dtype}", flush=True)
    for G in (0, 3):
        inp, gy = case(shape, dtype, 41 + shape[2] + shape[3])
        got = run_bwd(inp, gy, 15, G)
        assert_grad_parity(got, oracle_bwd(inp, gy, 15, G), f"dirs backward {shape} G={G}",
                           names=NAMES)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_every_mask_family(dtype):
    """Single directions, one axis, mixed pairs and triples; with and without
    a merger (directions outside the mask get zero gradients)."""
    inp, gy = case((2, 2, 24, 20), dtype, 77)
    for mask in (1, 2, 4, 8, 3, 12, 5, 10, 6, 9, 7, 14, 15):
        for merge in ((True, False) if mask in (15, 6) else (True,)):
            got = run_bwd(inp, gy, mask, 0, merge)
            assert_grad_parity(got, oracle_bwd(inp, gy, mask, 0, merge),
                               f"dirs backward mask={mask} merge={merge}", names=NAMES)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_plane_groups(dtype, monkeypatch):
    """Planes wider than 64 (the plane-group path): more planes than compute
    units (and fewer than twice as many) split into plane groups on their own
    streams; 300 planes of 100 channels put the group boundary inside an
    image. Three groups are forced on 10 planes as well (boundaries at planes
    3 and 6)."""
    inp, gy = case((3, 100, 8, 66), dtype, 91)
    for G in (0, 4):
        assert_grad_parity(run_bwd(inp, gy, 15, G), oracle_bwd(inp, gy, 15, G),
                           f"dirs backward, 300 planes, G={G}", names=NAMES)
    monkeypatch.setenv("GSPN_TPIPE_GROUPS", "3")
    inp, gy = case((2, 5, 9, 70), dtype, 92)
    for mask in (15, 12, 3):
        assert_grad_parity(run_bwd(inp, gy, mask, 0), oracle_bwd(inp, gy, mask, 0),
                           f"dirs backward, three groups, mask={mask}", names=NAMES)


def test_classification_workload_shape():
    """The classification stage's plane shape and dtype (fewer planes than
    the benchmark: the fp64 oracle is slow)."""
    w = WORKLOADS["cls_56x56_pd"]
    inp = make_inputs(w, seed=9, B=2, C=24)
    gy = make_grad_out(w, seed=10, B=2, C=24)
    got = run_bwd(inp, gy, w.dirs, w.group_rows)
    err = assert_grad_parity(got, oracle_bwd(inp, gy, w.dirs, w.group_rows), w.name, names=NAMES)
    print(f"[dirs bwd] {w.name} worst scaled error {err:.3e}", flush=True)


def test_t2i_full_size_sampled_planes():
    """The 2048x1024x320 bf16 per-direction workload at full size; the
    oracle checks sampled channels (their planes and merge gradients)."""
    w = WORKLOADS["t2i_2048x1024_pd"]
    print("[dirs bwd] t2i full size, generating on device", flush=True)
    d = make_inputs(w, device=DEV)
    gy = make_grad_out(w, device=DEV)
    grads = g.propagate_backward_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], gy,
                                      merge=d["merge"], dirs=w.dirs)
    torch.cuda.synchronize()
    for c in (0, 211):
        inp = {"x": d["x"][:, c:c + 1].cpu(), "merge": d["merge"][:, c:c + 1].cpu()}
        for k in KEYS:
            inp[k] = d[k][:, :, c:c + 1].contiguous().cpu()
        got = {"x": grads["x"][:, c:c + 1], "merge": grads["merge"][:, c:c + 1]}
        for k in KEYS:
            got[k] = grads[k][:, :, c:c + 1]
        ref = oracle_bwd(inp, gy[:, c:c + 1].cpu(), w.dirs, 0)
        err = assert_grad_parity(got, ref, f"t2i per-direction channel {c}", names=NAMES)
        print(f"[dirs bwd] t2i channel {c} worst scaled error {err:.3e}", flush=True)


def _offset(v):
    """A copy of v on the GPU that starts one element into its allocation."""
    buf = torch.zeros(v.numel() + 1, dtype=v.dtype, device=DEV)
    buf[1:].copy_(v.reshape(-1).to(DEV))
    return buf[1:].view(v.shape)


def test_offset_views_take_the_element_path():
    """Inputs and gradients that start one element into their allocations
    (no aligned vector runs, per-element transposes) give the oracle's
    gradients too."""
    for shape, dtype in [((1, 2, 40, 70), torch.float32), ((1, 2, 40, 70), torch.bfloat16),
                         ((1, 2, 20, 36), torch.float32), ((1, 2, 20, 36), torch.bfloat16)]:
        inp, gy = case(shape, dtype, 23)
        d = {k: (v.to(DEV) if k == "merge" else _offset(v)) for k, v in inp.items()}
        grads = {"x": _offset(torch.zeros_like(inp["x"]))}
        for k in KEYS:
            grads[k] = _offset(torch.zeros_like(inp["lam"]))
        grads["merge"] = _offset(torch.zeros((4, shape[1]), dtype=torch.float32))
        got = g.propagate_backward_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                        _offset(gy), merge=d["merge"], dirs=15, grads=grads)
        torch.cuda.synchronize()
        assert_grad_parity(got, oracle_bwd(inp, gy, 15, 0), f"dirs backward offset views {dtype}",
                           names=NAMES)


def test_deterministic():
    """Two calls give bitwise equal gradients, the merge gradients included
    (fixed reduction trees, no atomics), with and without plane groups."""
    for shape in [(3, 100, 8, 66), (3, 100, 12, 12)]:
        inp, gy = case(shape, torch.bfloat16, 27)
        a = run_bwd(inp, gy, 15, 0)
        b = run_bwd(inp, gy, 15, 0)
        for k in NAMES:
            assert torch.equal(a[k], b[k]), (shape, k)


def test_binding_rejects_aliased_gradients():
    inp, gy = case((1, 2, 8, 8), torch.float32, 5)
    d = {k: v.to(DEV) for k, v in inp.items()}
    grads = {"x": torch.empty_like(d["x"])}
    for k in KEYS:
        grads[k] = torch.empty_like(d["lam"])
    grads["merge"] = torch.empty((4, 2), device=DEV)
    grads["u"] = grads["lam"]
    with pytest.raises(g.GspnError) as ei:
        g.propagate_backward_dirs(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                  gy.to(DEV), merge=d["merge"], grads=grads)
    assert ei.value.name == "GSPN_E_ALIAS"


def test_empty_batch_gives_zero_merge_gradients():
    """B = 0 through the C ABI (real, non-null buffers): the merge gradients
    are empty sums, written as zeros."""
    import ctypes
    inp, gy = case((1, 3, 8, 8), torch.float32, 6)
    d = {k: v.to(DEV) for k, v in inp.items()}
    gyd = gy.to(DEV)
    gm = torch.full((4, 3), 7.0, device=DEV)
    outs = {k: torch.empty_like(d["lam"]) for k in KEYS}
    gx = torch.empty_like(d["x"])
    L = g.lib()
    lg = (ctypes.c_void_p * 3)(d["l0"].data_ptr(), d["l1"].data_ptr(), d["l2"].data_ptr())
    dlg = (ctypes.c_void_p * 3)(outs["l0"].data_ptr(), outs["l1"].data_ptr(), outs["l2"].data_ptr())
    st = L.gspn_propagate_backward_dirs_ws(
        d["x"].data_ptr(), lg, d["lam"].data_ptr(), d["u"].data_ptr(), 3 * 64,
        d["merge"].data_ptr(), gyd.data_ptr(), 0, 3, 8, 8, 15, 0, 0, gx.data_ptr(), dlg,
        outs["lam"].data_ptr(), outs["u"].data_ptr(), gm.data_ptr(), None, 0,
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.count_nonzero(gm).item() == 0
