"""The split-line prototype (gspn_bench_strip_t2b): a top->bottom scan whose
lines are split over several one-wavefront workgroups that exchange halo
states through device memory. It is a measurement of another schedule, not a
plan of the library; these tests check that what it measures is the same
propagation: its output equals the library's top->bottom propagation to the
bf16 bound, on ragged row blocks, several strips and slab sizes, and more
planes than are in flight."""
import ctypes

import pytest
import torch

import linear_spatial_propagation_line_amd as g
from linear_spatial_propagation_line_amd.inputs import make_inputs

from parity import assert_parity, oracle_y

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def L():
    lib = g.lib()
    lib.gspn_bench_strip_work_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.gspn_bench_strip_work_bytes.restype = ctypes.c_size_t
    lib.gspn_bench_strip_fail_offset.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.gspn_bench_strip_fail_offset.restype = ctypes.c_size_t
    lib.gspn_bench_strip_t2b.argtypes = [ctypes.c_void_p] * 2 + [ctypes.POINTER(ctypes.c_void_p)] + \
        [ctypes.c_void_p] * 2 + [ctypes.c_int64] + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.gspn_bench_strip_t2b.restype = ctypes.c_int
    return lib


def run_strip(L, d, S, K, pf):
    B, C, H, W = d["x"].shape
    out = torch.full_like(d["x"], float("nan"))
    nbytes = L.gspn_bench_strip_work_bytes(S, K, pf)
    work = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device=DEV)
    wp = (work.data_ptr() + 255) // 256 * 256
    abort = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    lg = (ctypes.c_void_p * 3)(*(d[k].data_ptr() for k in ("l0", "l1", "l2")))
    print(f"[strip] shape={(B, C, H, W)} S={S} K={K} pf={pf}", flush=True)
    rc = L.gspn_bench_strip_t2b(d["x"].data_ptr(), d["lam"].data_ptr(), lg, d["u"].data_ptr(),
                                out.data_ptr(), B * C, H, W, S, K, pf, wp, nbytes,
                                abort.data_ptr(), 1 << 20, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    off = wp - work.data_ptr() + L.gspn_bench_strip_fail_offset(S, pf)
    fail = int(work.view(torch.uint8)[off:off + 4].view(torch.int32)[0])
    assert fail == 0, "a wait gave up"
    return out


# (B, C, H, W), strips, halo K, planes in flight: W / S + 2K <= 64, W / S >= K
CASES = [((1, 3, 100, 64), 4, 8, 3), ((1, 3, 100, 64), 4, 16, 2), ((2, 3, 37, 96), 3, 16, 4),
         ((1, 5, 64, 256), 8, 16, 2), ((1, 2, 17, 1024), 32, 16, 2), ((1, 4, 40, 1024), 32, 8, 1)]


@pytest.mark.parametrize("shape,S,K,pf", CASES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_strip_prototype_matches_oracle(L, shape, S, K, pf):
    B, C, H, W = shape
    cpu = make_inputs("dit_16x16", seed=(H * 13 + W + S) % 997, B=B, C=C, H=H, W=W)
    d = {k: v.to(DEV) for k, v in cpu.items()}
    out = run_strip(L, d, S, K, pf)
    assert torch.isfinite(out.float()).all()
    assert_parity(out, oracle_y(cpu, g.T2B, 0), f"strip {shape} S={S} K={K} pf={pf}")


def test_strip_prototype_rejects_what_it_cannot_run(L):
    d = {k: v.to(DEV) for k, v in make_inputs("dit_16x16", seed=5, B=1, C=2, H=8, W=64).items()}
    lg = (ctypes.c_void_p * 3)(*(d[k].data_ptr() for k in ("l0", "l1", "l2")))
    work = torch.zeros(1 << 16, dtype=torch.int32, device=DEV)
    wp = (work.data_ptr() + 255) // 256 * 256
    abort = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    s = torch.cuda.current_stream().cuda_stream
    out = torch.empty_like(d["x"])

    def call(S, K, pf, nbytes=1 << 17):
        return L.gspn_bench_strip_t2b(d["x"].data_ptr(), d["lam"].data_ptr(), lg, d["u"].data_ptr(),
                                      out.data_ptr(), 2, 8, 64, S, K, pf, wp, nbytes,
                                      abort.data_ptr(), 1 << 20, s)
    assert call(3, 8, 1) == 1           # W not a multiple of S
    assert call(1, 8, 1) == 1           # one strip: 64 + 2 * 8 > 64 lanes
    assert call(8, 16, 1) == 1          # strips narrower than the halo
    assert call(4, 12, 1) == 1          # K neither 8 nor 16
    assert call(4, 8, 1, nbytes=16) == 1   # work too small
    assert call(4, 8, 1 << 20) == 1     # more workgroups than can be resident
