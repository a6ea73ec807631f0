"""Host-side pieces of bench.py (no GPU): input-set sizing, compulsory bytes
and per-kernel design bytes for every workload and kernel name the library
traces."""
import re

import pytest

import bench
from linear_spatial_propagation_line_amd.inputs import WORKLOADS

KERNELS = ["plane_kernel16", "plane_kernel64", "stream_kernel", "band_kernel", "tp_vfwd",
           "tp_hpair", "tp_vbwd", "tp_lgcopy", "bplane_kernel16", "bplane_kernel64", "bwd_fwd",
           "bwd_adj", "bwd_transpose", "bwd_finish", "bband_kernel", "bwd_reduce_logits"]


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("bwd", [False, True])
def test_input_sets_and_qmin(name, bwd):
    w = WORKLOADS[name]
    n = bench.input_sets(w, bwd)
    assert isinstance(n, int) and 1 <= n <= 8
    s = 4 if w.dtype == "f32" else 2
    q = bench.qmin_per_pixel(w, bwd)
    if w.cl == w.C:
        assert q == (13 if bwd else 7) * s
    else:
        assert (4 if not bwd else 7) * s < q < (7 if not bwd else 13) * s


@pytest.mark.parametrize("kernel", KERNELS)
def test_design_bytes_known(kernel):
    for w in WORKLOADS.values():
        assert bench.design_bytes(kernel, w.B * w.C, w) > 0


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
