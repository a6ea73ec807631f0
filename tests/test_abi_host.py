"""Host-only checks of the C ABI (no GPU needed: no call here reaches a HIP
API). The library must load, export every function include/gspn.h declares,
and reject bad arguments with the documented status before touching HIP."""
import ctypes
import os
import re

import pytest

import linear_spatial_propagation_line_amd as g

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(g.LIB_PATH):
        from linear_spatial_propagation_line_amd import build
        build.build()
    return g.lib()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(gspn_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 7, names
    assert "gspn_bench_stream" in names and "gspn_propagate_noalloc" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def test_abi_version(L):
    assert L.gspn_abi_version() == 1


def test_status_strings(L):
    for i in range(11):
        s = L.gspn_status_str(i).decode()
        assert s.startswith(g._STATUS[i])


# fake, well-aligned device addresses: validation never dereferences them
BASE = 1 << 40
SZ = 1 << 32


def call(L, x=BASE, lg=(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ), lam=BASE + 4 * SZ,
         u=BASE + 5 * SZ, B=1, C=1, H=8, W=8, mask=15, G=0, dt=0, out=BASE + 6 * SZ,
         ws=None, ws_bytes=0, use_ws=False):
    arr = None if lg is None else (ctypes.c_void_p * 3)(*lg)
    if use_ws:
        return L.gspn_propagate_ws(x, arr, lam, u, B, C, H, W, mask, G, dt, out, ws, ws_bytes, None)
    return L.gspn_propagate(x, arr, lam, u, B, C, H, W, mask, G, dt, out, None)


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), "GSPN_E_NULL"),
    (dict(lg=None), "GSPN_E_NULL"),
    (dict(lg=(BASE + SZ, None, BASE + 3 * SZ)), "GSPN_E_NULL"),
    (dict(out=None), "GSPN_E_NULL"),
    (dict(H=0), "GSPN_E_SHAPE"),
    (dict(W=-3), "GSPN_E_SHAPE"),
    (dict(B=-1), "GSPN_E_SHAPE"),
    (dict(H=1 << 31), "GSPN_E_SHAPE"),
    (dict(H=20000, W=100), "GSPN_E_SHAPE"),      # orthogonal length above the limit
    (dict(mask=0), "GSPN_E_DIRMASK"),
    (dict(mask=16), "GSPN_E_DIRMASK"),
    (dict(G=-1), "GSPN_E_GROUP"),
    (dict(dt=2), "GSPN_E_DTYPE"),
    (dict(x=BASE + 2), "GSPN_E_ALIGN"),
    (dict(dt=1, u=BASE + 5 * SZ + 1), "GSPN_E_ALIGN"),
    (dict(out=BASE + 8), "GSPN_E_ALIAS"),          # overlaps x
    (dict(out=BASE + 5 * SZ + 64), "GSPN_E_ALIAS"),  # overlaps u
])
def test_rejects_bad_arguments(L, kw, status, use_ws):
    assert call(L, use_ws=use_ws, **kw) == g.STATUS[status]
    assert L.gspn_last_error().decode() != ""


def test_empty_batch_is_ok_without_gpu(L):
    assert call(L, B=0) == 0
    assert call(L, C=0, use_ws=True) == 0


def test_workspace_checks(L, monkeypatch):
    monkeypatch.setenv("GSPN_FORCE_PLAN", "stream")
    need = L.gspn_workspace_bytes(2, 3, 300, 200, 15, 0, 0)
    assert need == 2 * 3 * 300 * 200 * 4
    assert call(L, B=2, C=3, H=300, W=200, use_ws=True) == g.STATUS["GSPN_E_WORKSPACE"]
    assert call(L, B=2, C=3, H=300, W=200, use_ws=True, ws=BASE + 7 * SZ,
                ws_bytes=need - 1) == g.STATUS["GSPN_E_WORKSPACE"]
    assert call(L, B=2, C=3, H=300, W=200, use_ws=True, ws=BASE + 7 * SZ + 16,
                ws_bytes=need) == g.STATUS["GSPN_E_ALIGN"]
    assert call(L, B=2, C=3, H=300, W=200, use_ws=True, ws=BASE + 6 * SZ,
                ws_bytes=need) == g.STATUS["GSPN_E_ALIAS"]


def test_workspace_and_plans(L, monkeypatch):
    assert g.workspace_bytes(64, 96, 56, 56) == 0
    assert g.plan_name(64, 96, 56, 56) == "plane64"
    assert g.plan_name(32, 1152, 16, 16, dtype=1) == "plane16"
    assert g.plan_name(1, 1, 16, 17) == "plane64"
    assert g.plan_name(1, 1, 65, 8) == "stream"          # odd H: no pair kernels
    assert g.plan_name(1, 320, 2048, 1024, dtype=1) == "tpipe"
    assert g.plan_name(16, 192, 128, 128, group_rows=8) == "band"
    assert g.plan_name(16, 192, 128, 128, group_rows=0) == "tpipe"
    assert g.plan_name(16, 192, 128, 128, group_rows=17) == "tpipe"   # groups above 16
    assert g.plan_name(1, 1, 512, 512, group_rows=8) == "tpipe"       # y_V too big for LDS
    assert g.plan_name(1, 1, 100, 2048) == "tpipe"        # W above 1024: 1024-thread row sweeps
    assert g.plan_name(1, 320, 1024, 2048, dtype=1) == "tpipe"     # the portrait latent
    assert g.plan_name(1, 1, 2048, 2048, dtype=1) == "tpipe"
    assert g.plan_name(1, 1, 100, 2050) == "large"        # W above 2048: transposed copies
    assert g.plan_name(1, 1, 2050, 100) == "large"        # H above 2048
    assert g.plan_name(1, 4, 2047, 1023, dtype=1) == "large"  # odd sides: transposed copies
    assert g.plan_name(1, 1, 3001, 9, dtype=1) == "stream"    # small plane, odd
    assert g.plan_name(1, 1, 20000, 4) == "invalid"
    assert g.workspace_bytes(1, 2, 100, 100) > 0
    assert g.plan_name(1, 1, 0, 5) == "invalid"
    assert g.workspace_bytes(1, 1, 0, 5) == 0
    monkeypatch.setenv("GSPN_FORCE_PLAN", "stream")
    assert g.plan_name(1, 2, 8, 8) == "stream"
    assert g.workspace_bytes(1, 2, 100, 100, dirs=g.T2B) == 0
    monkeypatch.setenv("GSPN_FORCE_PLAN", "tpipe")
    assert g.plan_name(1, 2, 8, 8) == "tpipe"
    assert g.plan_name(1, 2, 7, 8) == "plane16"           # tpipe needs even sizes


def bcall(L, lg=(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ), gy=BASE + 6 * SZ,
          outs=(BASE + 7 * SZ, BASE + 8 * SZ, BASE + 9 * SZ, BASE + 10 * SZ, BASE + 11 * SZ,
                BASE + 12 * SZ), B=1, C=1, H=8, W=8, mask=15, G=0, dt=0, ws=None, ws_bytes=0,
          use_ws=False):
    arr = (ctypes.c_void_p * 3)(*lg)
    dlg = None if outs[1] is None and outs[2] is None and outs[3] is None else \
        (ctypes.c_void_p * 3)(*outs[1:4])
    args = (BASE, arr, BASE + 4 * SZ, BASE + 5 * SZ, gy, B, C, H, W, mask, G, dt, outs[0], dlg,
            outs[4], outs[5])
    if use_ws:
        return L.gspn_propagate_backward_ws(*args, ws, ws_bytes, None)
    return L.gspn_propagate_backward(*args, None)


@pytest.fixture(scope="module")
def LB(L):
    g.lib()   # sets the backward argtypes
    return L


O = BASE + 7 * SZ


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(gy=None), "GSPN_E_NULL"),
    (dict(outs=(None, O + SZ, O + 2 * SZ, O + 3 * SZ, O + 4 * SZ, O + 5 * SZ)), "GSPN_E_NULL"),
    (dict(outs=(O, None, None, None, O + 4 * SZ, O + 5 * SZ)), "GSPN_E_NULL"),
    (dict(outs=(O, O + SZ, None, O + 3 * SZ, O + 4 * SZ, O + 5 * SZ)), "GSPN_E_NULL"),
    (dict(H=0), "GSPN_E_SHAPE"),
    (dict(mask=0), "GSPN_E_DIRMASK"),
    (dict(G=-2), "GSPN_E_GROUP"),
    (dict(dt=7), "GSPN_E_DTYPE"),
    (dict(gy=BASE + 6 * SZ + 2), "GSPN_E_ALIGN"),
    (dict(outs=(O + 1, O + SZ, O + 2 * SZ, O + 3 * SZ, O + 4 * SZ, O + 5 * SZ), dt=1), "GSPN_E_ALIGN"),
    (dict(outs=(BASE + 8, O + SZ, O + 2 * SZ, O + 3 * SZ, O + 4 * SZ, O + 5 * SZ)), "GSPN_E_ALIAS"),
    (dict(outs=(O, O + SZ, O + 2 * SZ, O + 3 * SZ, O + 4 * SZ, BASE + 6 * SZ)), "GSPN_E_ALIAS"),
    (dict(outs=(O, O + SZ, O + 2 * SZ, O + 3 * SZ, O + 4 * SZ, O + 16)), "GSPN_E_ALIAS"),
])
def test_backward_rejects_bad_arguments(LB, kw, status, use_ws):
    assert bcall(LB, use_ws=use_ws, **kw) == g.STATUS[status]
    assert LB.gspn_last_error().decode() != ""


def test_backward_workspace_checks(LB, monkeypatch):
    monkeypatch.setenv("GSPN_FORCE_BWD_PLAN", "stream")
    need = g.backward_workspace_bytes(2, 3, 30, 20)
    px = 2 * 3 * 30 * 20
    r256 = lambda v: (v + 255) // 256 * 256
    # states, 5 accumulators, and for horizontal directions 7 transposed
    # inputs and 5 transposed accumulators (regions 256-byte aligned)
    assert need == r256(r256(r256(r256(px * 4) + 5 * px * 4) + 7 * px * 4) + 5 * px * 4)
    assert g.backward_workspace_bytes(2, 3, 30, 20, dirs=g.T2B) == r256(px * 4)
    assert g.backward_workspace_bytes(2, 3, 30, 20, dirs=g.T2B | g.B2T) == \
        r256(r256(px * 4) + 5 * px * 4)
    assert g.backward_workspace_bytes(2, 3, 30, 20, dirs=g.L2R, dtype=g.GSPN_BF16) == \
        r256(r256(r256(r256(px * 4) + 5 * px * 4) + 7 * px * 2) + 5 * px * 4)
    assert g.backward_workspace_bytes(1, 1, 0, 20) == 0
    assert bcall(LB, B=2, C=3, H=30, W=20, use_ws=True) == g.STATUS["GSPN_E_WORKSPACE"]
    assert bcall(LB, B=2, C=3, H=30, W=20, use_ws=True, ws=BASE + 13 * SZ,
                 ws_bytes=need - 1) == g.STATUS["GSPN_E_WORKSPACE"]
    assert bcall(LB, B=2, C=3, H=30, W=20, use_ws=True, ws=BASE + 13 * SZ + 16,
                 ws_bytes=need) == g.STATUS["GSPN_E_ALIGN"]
    assert bcall(LB, B=2, C=3, H=30, W=20, use_ws=True, ws=BASE + 12 * SZ,
                 ws_bytes=need) == g.STATUS["GSPN_E_ALIAS"]
    assert bcall(LB, B=0, use_ws=True) == 0
    assert bcall(LB, C=0) == 0


def test_backward_plans(LB, monkeypatch):
    assert g.backward_plan_name(64, 96, 56, 56) == "bwd_plane64"
    assert g.backward_plan_name(32, 1152, 16, 16, dtype=1) == "bwd_plane16"
    assert g.backward_plan_name(1, 1, 65, 8) == "bwd_stream"
    assert g.backward_plan_name(1, 320, 2048, 1024, dtype=1) == "bwd_tpipe"
    assert g.backward_plan_name(1, 1, 0, 4) == "invalid"
    assert g.backward_plan_name(16, 192, 128, 128, group_rows=8) == "bwd_band"
    assert g.backward_plan_name(16, 192, 128, 128, group_rows=9) == "bwd_tpipe"
    assert g.backward_plan_name(1, 1, 600, 100, group_rows=4) == "bwd_tpipe"   # H > 512
    # the pipeline: both sides even, H <= 2048, W <= 1024; wider planes whose
    # transpose fits take it on transposed copies
    assert g.backward_plan_name(1, 1, 2050, 100) == "bwd_stream"
    assert g.backward_plan_name(1, 1, 100, 1026) == "bwd_tpipe_t"
    assert g.backward_plan_name(1, 320, 1024, 2048, dtype=1) == "bwd_tpipe_t"
    assert g.backward_plan_name(1, 1, 1026, 1026) == "bwd_stream"    # transpose too wide too
    assert g.backward_plan_name(1, 1, 100, 2050) == "bwd_stream"
    assert g.backward_plan_name(1, 1, 100, 1025) == "bwd_stream"
    assert g.backward_plan_name(1, 1, 2048, 2) == "bwd_tpipe"
    assert g.backward_workspace_bytes(2, 3, 128, 128, group_rows=8) == 5 * 6 * 128 * 128 * 4
    assert g.backward_workspace_bytes(2, 3, 128, 128, dirs=g.T2B, group_rows=8) == 0
    assert g.backward_workspace_bytes(64, 96, 56, 56) == 0
    monkeypatch.setenv("GSPN_FORCE_BWD_PLAN", "stream")
    assert g.backward_plan_name(64, 96, 56, 56) == "bwd_stream"
    assert g.backward_workspace_bytes(1, 2, 8, 8, dirs=g.T2B | g.B2T) == 6 * 2 * 64 * 4
    monkeypatch.setenv("GSPN_FORCE_BWD_PLAN", "tpipe")
    assert g.backward_plan_name(64, 96, 56, 56) == "bwd_tpipe"
    assert g.backward_plan_name(1, 1, 65, 8) == "bwd_stream"
    monkeypatch.setenv("GSPN_FORCE_BWD_PLAN", "tpipe_t")
    assert g.backward_plan_name(1, 2, 66, 40) == "bwd_tpipe_t"
    # shared logits: the transposed pipeline is not taken, the streaming path is
    monkeypatch.delenv("GSPN_FORCE_BWD_PLAN")
    shared = g.backward_workspace_bytes(1, 4, 100, 1026, logit_channels=2)
    monkeypatch.setenv("GSPN_FORCE_BWD_PLAN", "stream")
    assert shared == g.backward_workspace_bytes(1, 4, 100, 1026, logit_channels=2) > 0


def _al(v):
    return (v + 255) // 256 * 256


def _stream_ws(planes, H, W, dirs, es):
    px = planes * H * W
    hz = bool(dirs & 12)
    accs = hz or bin(dirs).count("1") > 1
    return (_al(px * 4) + _al(5 * px * 4 if accs else 0) + _al(7 * px * es if hz else 0)
            + _al(5 * px * 4 if hz else 0))


def _pipe_ws(planes, H, W, dirs, es):
    """The pipeline's regions: states of the two first sweeps (8 bytes a
    pixel each), the column-major copy in column quads (rows padded to 16,
    columns to a multiple of 4), the five fp32 horizontal parts in tiles of
    4 rows x 4 columns."""
    px = planes * H * W
    hz = bool(dirs & 12)
    Hp, ng, nq = (H + 15) // 16 * 16, (H + 3) // 4, (W // 2 + 1) // 2
    cp = planes * 4 * ((W + 3) // 4) * Hp
    if not hz:
        return _al(px * 8)
    return (_al(px * 8) + 2 * _al(cp * 4) + _al(3 * cp * es) + _al(px * 8)
            + _al(5 * planes * ng * nq * 16 * 4))


@pytest.mark.parametrize("shape", [(1, 2, 130, 96), (3, 1, 66, 1024), (1, 1, 2048, 2), (1, 1, 66, 6)])
@pytest.mark.parametrize("dirs", [15, 3, 12, 1])
@pytest.mark.parametrize("dtype", [0, 1])
def test_backward_pipeline_workspace(shape, dirs, dtype):
    """The pipeline asks for the larger of its own regions and the streaming
    path's, which serves calls whose tensors start at odd element offsets."""
    B, C, H, W = shape
    es = 4 if dtype == 0 else 2
    assert g.backward_plan_name(B, C, H, W, dirs, 0, dtype) == "bwd_tpipe"
    want = max(_pipe_ws(B * C, H, W, dirs, es), _stream_ws(B * C, H, W, dirs, es))
    assert g.backward_workspace_bytes(B, C, H, W, dirs, 0, dtype) == want


@pytest.mark.parametrize("cl", [0, -1, 3])
def test_shared_logit_channels_must_divide(LB, cl):
    lg = (ctypes.c_void_p * 3)(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ)
    st = LB.gspn_propagate_shared_ws(BASE, lg, cl, BASE + 4 * SZ, BASE + 5 * SZ, 1, 4, 8, 8, 15,
                                     0, 0, BASE + 6 * SZ, None, 0, None)
    assert st == g.STATUS["GSPN_E_SHAPE"]
    dlg = (ctypes.c_void_p * 3)(BASE + 8 * SZ, BASE + 9 * SZ, BASE + 10 * SZ)
    st = LB.gspn_propagate_backward_shared_ws(BASE, lg, cl, BASE + 4 * SZ, BASE + 5 * SZ,
                                              BASE + 6 * SZ, 1, 4, 8, 8, 15, 0, 0, BASE + 7 * SZ,
                                              dlg, BASE + 11 * SZ, BASE + 12 * SZ, None, 0, None)
    assert st == g.STATUS["GSPN_E_SHAPE"]
    assert LB.gspn_backward_workspace_bytes_shared(1, 4, 8, 8, cl, 15, 0, 0) == 0


def test_shared_workspace(LB):
    px = 2 * 4 * 56 * 56
    # plane-resident backward: no plan workspace, only the per-channel logit gradients
    assert g.backward_workspace_bytes(2, 4, 56, 56, logit_channels=1) == 3 * px * 4
    assert g.backward_workspace_bytes(2, 4, 56, 56, logit_channels=4) == 0
    assert g.backward_workspace_bytes(2, 4, 56, 56, logit_channels=2) == 3 * px * 4


def test_shared_aliasing_uses_logit_size(LB):
    # out placed right after one shared logit plane: no overlap with Cl = 1.
    # The shape needs a workspace and none is given, so the call that passes
    # the aliasing check stops at the workspace check and launches nothing.
    lg = (ctypes.c_void_p * 3)(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ)
    out = BASE + SZ + 100 * 100 * 4      # one 100x100 fp32 logit plane after l0
    st = LB.gspn_propagate_shared_ws(BASE, lg, 1, BASE + 4 * SZ, BASE + 5 * SZ, 1, 4, 100, 100,
                                     15, 0, 0, out, None, 0, None)
    assert st == g.STATUS["GSPN_E_WORKSPACE"]
    st = LB.gspn_propagate_shared_ws(BASE, lg, 4, BASE + 4 * SZ, BASE + 5 * SZ, 1, 4, 100, 100,
                                     15, 0, 0, out, None, 0, None)
    assert st == g.STATUS["GSPN_E_ALIAS"]


# ---- per-direction parameters (gspn_propagate_dirs_ws) ----------------------
# Every call below either fails validation or needs a workspace that it does
# not get, so none reaches a launch.
# (planes above 64 x 64: the calls need a workspace, and stop without one)
DP = 2 * 3 * 100 * 80         # elements of one [2, 3, 100, 80] tensor


def dcall(L, x=BASE, lg=(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ), lam=BASE + 4 * SZ,
          u=BASE + 5 * SZ, stride=DP, merge=BASE + 8 * SZ, B=2, C=3, H=100, W=80, mask=15, G=0,
          dt=0, out=BASE + 6 * SZ, ws=None, ws_bytes=0):
    arr = None if lg is None else (ctypes.c_void_p * 3)(*lg)
    return L.gspn_propagate_dirs_ws(x, arr, lam, u, stride, merge, B, C, H, W, mask, G, dt, out,
                                    ws, ws_bytes, None)


def test_dirs_workspace_bytes(L):
    # fp32 sums (transposed, row-major) and transposed x plus five tensors per
    # horizontal direction; DP * 4 and DP * 2 are multiples of 256 here
    assert L.gspn_workspace_bytes_dirs(2, 3, 100, 80, 15, 0, 0) == DP * 4 * (2 + 11)
    assert L.gspn_workspace_bytes_dirs(2, 3, 100, 80, g.L2R | g.R2L, 0, 1) == DP * (4 + 2 * 11)
    assert L.gspn_workspace_bytes_dirs(2, 3, 100, 80, g.R2L, 0, 0) == DP * 4 * (1 + 6)
    assert L.gspn_workspace_bytes_dirs(2, 3, 100, 80, g.T2B | g.B2T, 0, 0) == DP * 4
    assert L.gspn_workspace_bytes_dirs(2, 3, 100, 80, g.B2T, 0, 1) == 0
    assert L.gspn_workspace_bytes_dirs(1, 1, 9000, 16, 15, 0, 0) == 0     # above the limit
    assert g.workspace_bytes_dirs(2, 3, 100, 80) == DP * 4 * 13
    # planes up to 64 x 64: one wavefront per plane, no workspace
    for H, W in [(20, 16), (64, 64), (1, 64), (64, 1), (56, 56)]:
        assert L.gspn_workspace_bytes_dirs(2, 3, H, W, 15, 0, 0) == 0
    assert L.gspn_workspace_bytes_dirs(1, 1, 65, 64, 15, 0, 0) > 0
    assert L.gspn_workspace_bytes_dirs(1, 1, 64, 65, 15, 0, 1) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), "GSPN_E_NULL"),
    (dict(lg=None), "GSPN_E_NULL"),
    (dict(u=None), "GSPN_E_NULL"),
    (dict(stride=-1), "GSPN_E_SHAPE"),
    (dict(stride=DP - 1), "GSPN_E_SHAPE"),         # directions would overlap
    (dict(stride=1 << 62), "GSPN_E_SHAPE"),
    (dict(H=8200, W=4), "GSPN_E_SHAPE"),          # above the per-direction limit
    (dict(mask=0), "GSPN_E_DIRMASK"),
    (dict(G=-2), "GSPN_E_GROUP"),
    (dict(dt=3), "GSPN_E_DTYPE"),
    (dict(merge=BASE + 8 * SZ + 2), "GSPN_E_ALIGN"),
    (dict(dt=1, lam=BASE + 4 * SZ + 1), "GSPN_E_ALIGN"),
    # out inside direction 2's lambda (element offset 2 * stride)
    (dict(out=BASE + 4 * SZ + 2 * DP * 4 + 64), "GSPN_E_ALIAS"),
    (dict(out=BASE + 8 * SZ - 64), "GSPN_E_ALIAS"),   # out runs into the merge weights
    (dict(out=BASE + 8), "GSPN_E_ALIAS"),            # overlaps x
])
def test_dirs_rejects_bad_arguments(L, kw, status):
    assert dcall(L, **kw) == g.STATUS[status]
    assert L.gspn_last_error().decode() != ""


def test_dirs_aliasing_only_for_selected_directions(L):
    # out exactly on direction 2's lambda, but direction 2 is not selected:
    # the call passes the aliasing check and stops at the missing workspace
    out = BASE + 4 * SZ + 2 * DP * 4
    assert dcall(L, out=out, mask=g.T2B | g.R2L) == g.STATUS["GSPN_E_WORKSPACE"]
    # stride 0: every direction reads the same tensors, no overlap among them
    assert dcall(L, stride=0) == g.STATUS["GSPN_E_WORKSPACE"]
    assert dcall(L, merge=None) == g.STATUS["GSPN_E_WORKSPACE"]


def test_dirs_workspace_checks(L):
    need = L.gspn_workspace_bytes_dirs(2, 3, 100, 80, 15, 0, 0)
    assert dcall(L, ws=BASE + 7 * SZ, ws_bytes=need - 1) == g.STATUS["GSPN_E_WORKSPACE"]
    assert dcall(L, ws=BASE + 7 * SZ + 16, ws_bytes=need) == g.STATUS["GSPN_E_ALIGN"]
    # the workspace inside direction 3's u
    assert dcall(L, ws=BASE + 5 * SZ + 3 * DP * 4, ws_bytes=need) == g.STATUS["GSPN_E_ALIAS"]
    assert dcall(L, ws=BASE + 6 * SZ, ws_bytes=need) == g.STATUS["GSPN_E_ALIAS"]   # out


def test_dirs_empty_batch_is_ok_without_gpu(L):
    assert dcall(L, B=0) == 0


# ---- per-direction backward (gspn_propagate_backward_dirs_ws) ------------------
def bdcall(L, x=BASE, lg=(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ), lam=BASE + 4 * SZ,
           u=BASE + 5 * SZ, stride=DP, merge=BASE + 8 * SZ, gy=BASE + 9 * SZ, B=2, C=3, H=100,
           W=80, mask=15, G=0, dt=0, gx=BASE + 10 * SZ,
           glg=(BASE + 11 * SZ, BASE + 12 * SZ, BASE + 13 * SZ), glam=BASE + 14 * SZ,
           gu=BASE + 15 * SZ, gm=BASE + 16 * SZ, ws=None, ws_bytes=0):
    arr = None if lg is None else (ctypes.c_void_p * 3)(*lg)
    garr = None if glg is None else (ctypes.c_void_p * 3)(*glg)
    return L.gspn_propagate_backward_dirs_ws(x, arr, lam, u, stride, merge, gy, B, C, H, W, mask,
                                             G, dt, gx, garr, glam, gu, gm, ws, ws_bytes, None)


def test_backward_dirs_workspace_bytes(L):
    # stored states and the fp32 sum for grad_x; with a horizontal direction
    # also transposed x and grad_out, five inputs and five gradients of one
    # direction, and a transposed fp32 sum (DP * 4 and DP * 2 are multiples
    # of 256 here); last the fp64 merge partials, 4 per plane (6 planes:
    # 192 bytes, one 256-byte block)
    assert L.gspn_backward_workspace_bytes_dirs(2, 3, 100, 80, 15, 0, 0) == DP * 4 * 15 + 256
    assert L.gspn_backward_workspace_bytes_dirs(2, 3, 100, 80, 15, 0, 1) == \
        DP * (4 * 3 + 2 * 12) + 256
    assert L.gspn_backward_workspace_bytes_dirs(2, 3, 100, 80, g.T2B | g.B2T, 0, 1) == \
        DP * 4 * 2 + 256
    assert L.gspn_backward_workspace_bytes_dirs(1, 1, 9000, 16, 15, 0, 0) == 0   # above the limit
    assert g.backward_workspace_bytes_dirs(2, 3, 100, 80, g.L2R) == DP * 4 * 15 + 256
    # 40 planes: 1280 bytes of partials
    DP40 = 8 * 5 * 20 * 80
    assert L.gspn_backward_workspace_bytes_dirs(8, 5, 20, 80, g.T2B, 0, 0) == DP40 * 4 * 2 + 1280


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), "GSPN_E_NULL"),
    (dict(lg=None), "GSPN_E_NULL"),
    (dict(gy=None), "GSPN_E_NULL"),
    (dict(gx=None), "GSPN_E_NULL"),
    (dict(glg=(BASE + 11 * SZ, None, BASE + 13 * SZ)), "GSPN_E_NULL"),
    (dict(stride=DP - 1), "GSPN_E_SHAPE"),
    (dict(H=8200, W=4), "GSPN_E_SHAPE"),
    (dict(mask=0), "GSPN_E_DIRMASK"),
    (dict(G=-1), "GSPN_E_GROUP"),
    (dict(dt=3), "GSPN_E_DTYPE"),
    (dict(gm=BASE + 16 * SZ + 2), "GSPN_E_ALIGN"),
    (dict(dt=1, glam=BASE + 14 * SZ + 1), "GSPN_E_ALIGN"),
    (dict(gx=BASE), "GSPN_E_ALIAS"),                                  # grad_x on x
    (dict(glam=BASE + 5 * SZ + DP * 4), "GSPN_E_ALIAS"),              # on direction 1's u
    (dict(gm=BASE + 8 * SZ + 4), "GSPN_E_ALIAS"),                     # on the merge weights
    (dict(gu=BASE + 14 * SZ + 3 * DP * 4), "GSPN_E_ALIAS"),           # inside grad_lambda's slices
])
def test_backward_dirs_rejects_bad_arguments(L, kw, status):
    assert bdcall(L, **kw) == g.STATUS[status]
    assert L.gspn_last_error().decode() != ""


def test_backward_dirs_workspace_checks(L):
    need = L.gspn_backward_workspace_bytes_dirs(2, 3, 100, 80, 15, 0, 0)
    assert bdcall(L) == g.STATUS["GSPN_E_WORKSPACE"]
    assert bdcall(L, ws=BASE + 17 * SZ, ws_bytes=need - 1) == g.STATUS["GSPN_E_WORKSPACE"]
    assert bdcall(L, ws=BASE + 17 * SZ + 16, ws_bytes=need) == g.STATUS["GSPN_E_ALIGN"]
    assert bdcall(L, ws=BASE + 9 * SZ, ws_bytes=need) == g.STATUS["GSPN_E_ALIAS"]    # grad_out
    assert bdcall(L, ws=BASE + 15 * SZ, ws_bytes=need) == g.STATUS["GSPN_E_ALIAS"]   # grad_u
    # without a merger and without the merge gradient the pointers may be NULL
    assert bdcall(L, merge=None, gm=None) == g.STATUS["GSPN_E_WORKSPACE"]


def test_backward_dirs_empty_batch_is_ok_without_gpu(L):
    assert bdcall(L, B=0, gm=None) == 0


# ---- module prologue (gspn_prologue, gspn_module_ws) -------------------------
# fake addresses again; every call fails validation or has B = 0
PB, PCIN, PC, PH, PW = 2, 6, 4, 5, 7


def pcall(L, x_in=BASE, cin=PCIN, w_r=BASE + SZ, b_r=BASE + 2 * SZ, w_p=BASE + 3 * SZ,
          b_p=BASE + 4 * SZ, B=PB, C=PC, H=PH, W=PW, dt=0, x_out=BASE + 5 * SZ,
          p_out=(BASE + 6 * SZ, BASE + 7 * SZ, BASE + 8 * SZ, BASE + 9 * SZ, BASE + 10 * SZ)):
    arr = None if p_out is None else (ctypes.c_void_p * 5)(*p_out)
    return L.gspn_prologue(x_in, cin, w_r, b_r, w_p, b_p, B, C, H, W, dt, x_out, arr, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x_in=None), "GSPN_E_NULL"),
    (dict(w_p=None), "GSPN_E_NULL"),
    (dict(p_out=None), "GSPN_E_NULL"),
    (dict(p_out=(BASE + 6 * SZ, None, BASE + 8 * SZ, BASE + 9 * SZ, BASE + 10 * SZ)), "GSPN_E_NULL"),
    (dict(dt=4), "GSPN_E_DTYPE"),
    (dict(cin=0), "GSPN_E_SHAPE"),
    (dict(C=0), "GSPN_E_SHAPE"),
    (dict(B=70000), "GSPN_E_SHAPE"),
    (dict(H=1 << 16, W=1 << 16), "GSPN_E_SHAPE"),
    (dict(w_r=BASE + SZ + 2), "GSPN_E_ALIGN"),
    (dict(dt=1, x_out=BASE + 5 * SZ + 1), "GSPN_E_ALIGN"),
    (dict(x_out=BASE + 16), "GSPN_E_ALIAS"),                      # inside x_in
    (dict(x_out=BASE + 3 * SZ + 8), "GSPN_E_ALIAS"),              # inside w_params
    (dict(p_out=(BASE + 5 * SZ + 64, BASE + 7 * SZ, BASE + 8 * SZ, BASE + 9 * SZ,
                 BASE + 10 * SZ)), "GSPN_E_ALIAS"),               # l0 inside x_out
])
def test_prologue_rejects_bad_arguments(L, kw, status):
    assert pcall(L, **kw) == g.STATUS[status]
    assert L.gspn_last_error().decode() != ""


def test_prologue_empty_batch_and_null_biases(L):
    assert pcall(L, B=0) == 0
    assert pcall(L, B=0, b_r=None, b_p=None) == 0


def test_module_workspace(L):
    px = PB * PC * PH * PW
    tb = (px * 4 + 255) // 256 * 256
    assert L.gspn_module_workspace_bytes(PB, PC, PH, PW, 15, 0, 0) == 6 * tb   # plane plan
    assert L.gspn_module_workspace_bytes(PB, PC, PH, PW, 0, 0, 0) == 0        # bad mask
    need = L.gspn_module_workspace_bytes(PB, PC, 300, 200, 15, 0, 1)
    assert need > 6 * PB * PC * 300 * 200 * 2
    assert g.module_workspace_bytes(PB, PC, PH, PW) == 6 * tb
    st = L.gspn_module_ws(BASE, PCIN, BASE + SZ, None, BASE + 3 * SZ, None, PB, PC, PH, PW, 15,
                          0, 0, BASE + 5 * SZ, BASE + 7 * SZ, 6 * tb - 1, None)
    assert st == g.STATUS["GSPN_E_WORKSPACE"]
    st = L.gspn_module_ws(BASE, PCIN, BASE + SZ, None, BASE + 3 * SZ, None, PB, PC, PH, PW, 15,
                          0, 0, BASE + 7 * SZ + 64, BASE + 7 * SZ, 6 * tb, None)
    assert st == g.STATUS["GSPN_E_ALIAS"]      # out inside the workspace
    st = L.gspn_module_ws(BASE, PCIN, BASE + SZ, None, BASE + 3 * SZ, None, PB, PC, PH, PW, 15,
                          0, 0, BASE + 5 * SZ, BASE + 16, 6 * tb, None)
    assert st == g.STATUS["GSPN_E_ALIGN"]      # workspace not 256-byte aligned
    st = L.gspn_module_ws(BASE, PCIN, BASE + SZ, None, BASE + 3 * SZ, None, PB, PC, PH, PW, 15,
                          0, 0, BASE + 5 * SZ, BASE + 256, 6 * tb, None)
    assert st == g.STATUS["GSPN_E_ALIAS"]      # workspace inside x_in
    st = L.gspn_module_ws(BASE, PCIN, BASE + SZ, None, BASE + 3 * SZ, None, 0, PC, PH, PW, 15,
                          0, 0, BASE + 5 * SZ, BASE + 7 * SZ, 6 * tb, None)
    assert st == 0


def call_noalloc(L, x=BASE, lg=(BASE + SZ, BASE + 2 * SZ, BASE + 3 * SZ), lam=BASE + 4 * SZ,
                 u=BASE + 5 * SZ, B=1, C=1, H=8, W=8, mask=15, G=0, dt=0, out=BASE + 6 * SZ):
    arr = None if lg is None else (ctypes.c_void_p * 3)(*lg)
    return L.gspn_propagate_noalloc(x, arr, lam, u, B, C, H, W, mask, G, dt, out, None)


def test_noalloc_validation_before_any_hip_call(L):
    """The allocation-free entry point validates like gspn_propagate and
    rejects, before touching HIP, a problem whose scratch exceeds its static
    per-device array."""
    assert L.gspn_noalloc_scratch_bytes() == 64 << 20
    assert call_noalloc(L, x=None) == g.STATUS["GSPN_E_NULL"]
    assert call_noalloc(L, mask=0) == g.STATUS["GSPN_E_DIRMASK"]
    assert call_noalloc(L, out=BASE + 8) == g.STATUS["GSPN_E_ALIAS"]
    assert call_noalloc(L, B=0) == 0
    # 320 planes of 2048 x 1024: the pipeline's workspace is gigabytes
    assert L.gspn_workspace_bytes(1, 320, 2048, 1024, 15, 0, 1) > 64 << 20
    assert call_noalloc(L, B=1, C=320, H=2048, W=1024, dt=1) == g.STATUS["GSPN_E_WORKSPACE"]
    assert "64" in L.gspn_last_error().decode() or "67108864" in L.gspn_last_error().decode()
