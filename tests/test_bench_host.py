"""Host-side pieces of bench.py (no GPU): input-set sizing, compulsory bytes
and per-kernel design bytes for every workload and kernel name the library
traces."""
import re

import pytest

import bench
from linear_spatial_propagation_line_amd.inputs import WORKLOADS

KERNELS = ["plane_kernel16", "plane_kernel64", "plane_pc_kernel", "stream_kernel", "band_kernel", "tp_vfwd",
           "tp_hpair", "tp_vbwd", "tp_lgcopy", "bplane_kernel16", "bplane_kernel64", "bwd_fwd",
           "bwd_adj", "bwd_transpose", "bwd_finish", "bband_kernel", "bwd_reduce_logits",
           "dir_plane", "dir_vert", "dir_tr_in", "dir_tr_acc", "prologue_reduce", "prologue_params",
           "bt_vA", "bt_hA", "bt_hB", "bt_vB", "bwd_dirs_zero", "bwd_dirs_store_dx", "bwd_dirs_tr",
           "bwd_dirs_tr_acc", "bwd_dirs_merge", "fused_unit", "tp_t_in", "tp_t_out"]


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("bwd", [False, True])
def test_input_sets_and_qmin(name, bwd):
    w = WORKLOADS[name]
    s = 4 if w.dtype == "f32" else 2
    if w.prologue_cin and bwd:
        with pytest.raises(ValueError):
            bench.qmin_per_pixel(w, bwd)
        return
    if w.per_direction:
        # forward: x and the directions' five tensors in, out; backward: x,
        # grad_out and the five tensors in, dx and the five gradients out
        want = ((3 + 10 * w.ndirs) if bwd else (2 + 5 * w.ndirs)) * s
        assert bench.qmin_per_pixel(w, bwd) == want
    elif w.prologue_cin:
        assert bench.qmin_per_pixel(w, bwd) == (w.prologue_cin / w.C + 1) * s
    n = bench.input_sets(w, bwd)
    assert isinstance(n, int) and 1 <= n <= 8
    q = bench.qmin_per_pixel(w, bwd)
    if w.per_direction or w.prologue_cin:
        return
    if w.cl == w.C:
        assert q == (13 if bwd else 7) * s
    else:
        assert (4 if not bwd else 7) * s < q < (7 if not bwd else 13) * s


@pytest.mark.parametrize("kernel", KERNELS)
def test_design_bytes_known(kernel):
    for w in WORKLOADS.values():
        assert bench.design_bytes(kernel, w.B * w.C, w) > 0


def test_direction_passes_sum_to_their_design():
    """Per-direction layer, four directions: x and the horizontal directions'
    ten tensors transposed (11 tensors read and written), four passes that
    each read their six tensors, the accumulator written by the first, read
    and written by the next two and read by the last, which writes out, and
    the horizontal sum transposed back (fp32 read and write)."""
    w = WORKLOADS["t2i_2048x1024_pd"]
    s = 2
    planes = w.B * w.C
    tot = bench.design_bytes("dir_tr_in", planes * 11, w)
    for i in range(4):
        tot += bench.design_bytes("dir_vert", planes, w, first=i == 0, last=i == 3)
    tot += bench.design_bytes("dir_tr_acc", planes, w)
    assert tot == w.pixels * (22 * s + 4 * 6 * s + 4 + 8 + 8 + 4 + s + 8)
    assert bench.qmin_per_pixel(w, False) == 22 * s


def test_every_traced_kernel_name_has_design_bytes():
    """Each kernel name a launcher hands to the tracer (directly, or through
    the pipeline's launch helper) is one design_bytes knows."""
    import glob
    import os
    names = set()
    for f in glob.glob(os.path.join(bench.CSRC, "*.hip")):
        text = open(f, encoding="utf-8").read()
        for call in re.findall(r"tr->before\(([^;]*)\);", text):
            names |= set(re.findall(r'"(\w+)"', call))
        for call in re.findall(r"launch\(k\d, \w+, ([^;]*)\)", text):
            names |= set(re.findall(r'"(\w+)"', call))
    assert {"plane_kernel64", "tp_vfwd", "bwd_adj", "tp_lgcopy"} <= names, names
    for n in names:
        assert n in KERNELS, f"traced kernel {n} missing from the list"


def test_prologue_work():
    """Flops and bytes of the prologue on the 2048x1024 unit: two products of
    2 * pixels * C * (Cin + 5C) flops; x_in read, six tensors written."""
    w = WORKLOADS["t2i_2048x1024_mod"]
    flops, nbytes = bench.prologue_work(w)
    px = 2048 * 1024
    assert flops == 2.0 * px * 320 * (320 + 1600)
    assert nbytes == (px * (320 + 6 * 320) + 320 * 320 + 5 * 320 * 320 + 6 * 320) * 2
    # at MI355X peaks the bf16 products take less time than the bytes
    assert flops / 2500e12 < nbytes / 8000e9
    wd = WORKLOADS["dit_16x16_mod"]
    f2, b2 = bench.prologue_work(wd)
    assert f2 / 2500e12 > b2 / 8000e9     # C = 1152: MFMA-bound


def test_per_direction_backward_path_bytes():
    """Four directions, bf16: x and grad_out transposed, ten tensors through
    each horizontal direction's transposes, the dx sum back; per direction
    the scan pair (the merge partials ride along in the reverse scan)."""
    w = WORKLOADS["t2i_2048x1024_pd"]
    s = 2
    per_dir = (5 * s + 4) + (12 * s + 12)
    assert bench.bwd_dirs_path_bytes(w) == 4 * s + 2 * 20 * s + 8 + 4 * per_dir


def test_parity_of_sample_catches_a_planted_error():
    """The bench's in-run check of the timed output: equal planes pass, one
    element off by more than the dtype's bound fails."""
    import numpy as np
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 8, 8))
    got = ref.astype(np.float32)
    p = bench.parity_of_sample(got, ref, "f32")
    assert p["ok"] and p["planes"] == 3 and p["scaled_error"] < 1e-6
    bad = got.copy()
    bad[1, 2, 3] += 1e-2
    assert not bench.parity_of_sample(bad, ref, "f32")["ok"]
    assert bench.parity_of_sample(bad, ref, "bf16")["ok"]


def test_timed_output_parity_forward_and_backward():
    import numpy as np
    import torch
    w = WORKLOADS["cls_56x56"]
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((1, 4, w.H, w.W))
    out = torch.zeros((w.B, w.C, w.H, w.W))
    out.reshape(-1, w.H, w.W)[:4] = torch.from_numpy(ref[0]).float()
    assert bench.timed_output_parity(out, ref, 4, w, False)["ok"]
    out.reshape(-1, w.H, w.W)[3, 0, 0] += 1.0
    assert not bench.timed_output_parity(out, ref, 4, w, False)["ok"]
    grads = {k: torch.zeros((w.B, w.C, w.H, w.W)) for k in ("x", "l0", "l1", "l2", "lam", "u")}
    refs = {k: rng.standard_normal((1, 2, w.H, w.W)) for k in grads}
    for k in grads:
        grads[k].reshape(-1, w.H, w.W)[:2] = torch.from_numpy(refs[k][0]).float()
    p = bench.timed_output_parity(grads, refs, 2, w, True)
    assert p["ok"] and p["planes"] == 2


def test_cpu_model_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
