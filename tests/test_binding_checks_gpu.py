"""The binding checks caller-supplied outputs and workspaces before it hands
their pointers to the C ABI: a tensor of the wrong shape, dtype, layout or
device, or a workspace that is not a uint8 tensor on the inputs' device,
raises before anything is launched (needs a GPU for the device tensors)."""
from __future__ import annotations

import pytest
import torch

import linear_spatial_propagation_line_amd as g
from linear_spatial_propagation_line_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def inp():
    d = make_inputs("cls_56x56", seed=5, B=1, C=2, H=40, W=24)
    return {k: v.to(DEV) for k, v in d.items()}


def bad_outs(x):
    return [
        (torch.empty(x.shape, dtype=torch.bfloat16, device=DEV), ValueError),   # dtype
        (torch.empty((1, 2, 40, 23), dtype=x.dtype, device=DEV), ValueError),   # shape
        (torch.empty((1, 2, 24, 40), dtype=x.dtype, device=DEV).transpose(2, 3), ValueError),
        (torch.empty(x.shape, dtype=x.dtype), TypeError),                       # host memory
        ("not a tensor", TypeError),
    ]


def bad_workspaces():
    return [(torch.empty(1 << 20, dtype=torch.uint8), TypeError),               # host memory
            (torch.empty(1 << 18, dtype=torch.float32, device=DEV), ValueError),
            (torch.empty(1 << 21, dtype=torch.uint8, device=DEV)[::2], ValueError)]


def test_propagate_checks_out_and_workspace(inp):
    lg = (inp["l0"], inp["l1"], inp["l2"])
    for out, exc in bad_outs(inp["x"]):
        with pytest.raises(exc):
            g.propagate(inp["x"], lg, inp["lam"], inp["u"], out=out)
        with pytest.raises(exc):
            g.propagate_alloc(inp["x"], lg, inp["lam"], inp["u"], out=out)
        with pytest.raises(exc):
            g.propagate_noalloc(inp["x"], lg, inp["lam"], inp["u"], out=out)
    for ws, exc in bad_workspaces():
        with pytest.raises(exc):
            g.propagate(inp["x"], lg, inp["lam"], inp["u"], workspace=ws)
    # an input on another device type is refused as before
    with pytest.raises(TypeError):
        g.propagate(inp["x"], lg, inp["lam"].cpu(), inp["u"])


def test_propagate_dirs_checks_out_and_workspace(inp):
    d4 = {k: torch.stack([inp[k]] * 4) for k in ("l0", "l1", "l2", "lam", "u")}
    lg = (d4["l0"], d4["l1"], d4["l2"])
    for out, exc in bad_outs(inp["x"]):
        with pytest.raises(exc):
            g.propagate_dirs(inp["x"], lg, d4["lam"], d4["u"], out=out)
    for ws, exc in bad_workspaces():
        with pytest.raises(exc):
            g.propagate_dirs(inp["x"], lg, d4["lam"], d4["u"], workspace=ws)


def test_backward_checks_workspace(inp):
    lg = (inp["l0"], inp["l1"], inp["l2"])
    gy = torch.randn_like(inp["x"])
    for ws, exc in bad_workspaces():
        with pytest.raises(exc):
            g.propagate_backward(inp["x"], lg, inp["lam"], inp["u"], gy, workspace=ws)


def test_prologue_and_module_check_outputs():
    B, Cin, C, H, W = 1, 3, 2, 8, 8
    x_in = torch.randn(B, Cin, H, W, device=DEV)
    w_r = torch.randn(C, Cin, device=DEV)
    w_p = torch.randn(5 * C, C, device=DEV)
    good = {k: torch.empty((B, C, H, W), device=DEV) for k in ("x",) + g.PARAM_NAMES}
    for k in ("x", "lam"):
        for bad, exc in [(torch.empty((B, C, H, W + 1), device=DEV), ValueError),
                         (torch.empty((B, C, H, W)), TypeError),
                         (torch.empty((B, C, H, W), dtype=torch.bfloat16, device=DEV), ValueError)]:
            outs = dict(good)
            outs[k] = bad
            with pytest.raises(exc):
                g.prologue(x_in, w_r, None, w_p, None, outs=outs)
    with pytest.raises(ValueError):
        g.prologue(x_in, w_r, None, w_p, None, outs={"x": good["x"]})
    for out, exc in [(torch.empty((B, C, H, W), dtype=torch.bfloat16, device=DEV), ValueError),
                     (torch.empty((B, C + 1, H, W), device=DEV), ValueError),
                     (torch.empty((B, C, H, W)), TypeError)]:
        with pytest.raises(exc):
            g.module(x_in, w_r, None, w_p, None, out=out)
    for ws, exc in bad_workspaces():
        with pytest.raises(exc):
            g.module(x_in, w_r, None, w_p, None, workspace=ws)
