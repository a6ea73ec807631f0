"""Weights from very negative logits, against the fp64 oracle (needs an
MI355X). The weights are sigmoid(l_k) normalised over the in-range
neighbours (CSDN page, section 如何设计一个高效的传播层), so they follow the
logits' differences as well as their level: with every logit near -30 they
are far from uniform although each sigmoid is below 1e-13.

The kernels form the weights from logits clamped below at -40 (sigmoid(-40)
is about 4e-18), which keeps the product form of the normalisation finite in
fp32. These tests pin both sides of that contract:
  * shallow: every logit in [-39.5, -20] (nothing clamped): the exact
    weights, against the oracle on the logits as given; with "outside", each
    neighbour outside the plane gets the logit +10, so at the border the
    interior weights go almost all to a neighbour that edge lanes drop, and
    renormalising them must still give the in-range weights;
  * deep: every logit in [-70, -50]: the weights of the clamped logits
    (uniform), against the oracle on logits clamped at -40.
Every plan is forced in turn on a plane it takes; forward and backward."""
from __future__ import annotations

import pytest
import torch

import linear_spatial_propagation_line_amd as g
from linear_spatial_propagation_line_amd.inputs import make_grad_out, make_inputs
from parity import assert_grad_parity, assert_parity, oracle_grads, oracle_y

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LOGIT_FLOOR = -40.0
RECIPES = {"shallow": (-39.5, -20.0, False), "outside": (-39.5, -20.0, True),
           "deep": (-70.0, -50.0, False)}


def extreme(inp, seed, recipe):
    """(inputs for the GPU, the same with the logits the kernels use)."""
    lo, hi, outside = RECIPES[recipe]
    gen = torch.Generator().manual_seed(seed)
    gpu = dict(inp)
    for k in ("l0", "l1", "l2"):
        t = lo + (hi - lo) * torch.rand(inp[k].shape, generator=gen, dtype=torch.float64)
        if outside and k == "l0":
            t[..., :, 0] = 10.0      # vertical scans: column c - 1 at c = 0
            t[..., 0, :] = 10.0      # horizontal scans: row r - 1 at r = 0
        if outside and k == "l2":
            t[..., :, -1] = 10.0
            t[..., -1, :] = 10.0
        gpu[k] = t.to(inp[k].dtype)
    ref = dict(gpu)
    for k in ("l0", "l1", "l2"):
        ref[k] = torch.clamp(gpu[k], min=LOGIT_FLOOR)
    if recipe != "deep":
        assert all(torch.equal(ref[k], gpu[k]) for k in ("l0", "l1", "l2"))
    return gpu, ref


FWD_CASES = [("plane", (2, 3, 16, 16), 0), ("plane", (1, 2, 56, 56), 0),
             ("plane", (1, 2, 40, 64), 5), ("band", (1, 2, 66, 40), 8),
             ("tpipe", (1, 2, 66, 40), 0), ("tpipe_t", (1, 2, 40, 130), 0),
             ("large", (1, 3, 65, 67), 0), ("stream", (1, 2, 66, 40), 3)]


@pytest.fixture
def env(monkeypatch):
    return monkeypatch.setenv


@pytest.mark.parametrize("recipe", list(RECIPES))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("plan,shape,G", FWD_CASES,
                         ids=lambda v: v if isinstance(v, str) else "x".join(map(str, v))
                         if isinstance(v, tuple) else f"G{v}")
def test_forward(env, plan, shape, G, dtype, recipe):
    env("GSPN_FORCE_PLAN", plan)
    B, C, H, W = shape
    dt = 0 if dtype == torch.float32 else 1
    got_plan = g.plan_name(B, C, H, W, 15, G, dt)
    assert got_plan.startswith(plan), got_plan
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    gpu, ref = extreme(make_inputs(name, seed=H + W, B=B, C=C, H=H, W=W), 5 + H, recipe)
    d = {k: v.to(DEV) for k, v in gpu.items()}
    for mask in (15, 1, 8):
        out = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                          dirs=mask, group_rows=G)
        torch.cuda.synchronize()
        assert_parity(out, oracle_y(ref, mask, G), f"{got_plan} {shape} mask={mask}")


BWD_CASES = [("plane", (2, 3, 16, 16), 0), ("plane", (1, 2, 56, 56), 0),
             ("band", (1, 2, 66, 40), 8), ("tpipe", (1, 2, 66, 40), 0),
             ("stream", (1, 2, 66, 40), 3)]


@pytest.mark.parametrize("recipe", ["shallow", "outside"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("plan,shape,G", BWD_CASES,
                         ids=lambda v: v if isinstance(v, str) else "x".join(map(str, v))
                         if isinstance(v, tuple) else f"G{v}")
def test_backward(env, plan, shape, G, dtype, recipe):
    """(Gradients of clamped logits are not those of the logits as given,
    so the deep recipe has no backward counterpart.)"""
    env("GSPN_FORCE_BWD_PLAN", plan)
    B, C, H, W = shape
    dt = 0 if dtype == torch.float32 else 1
    got_plan = g.backward_plan_name(B, C, H, W, 15, G, dt)
    assert got_plan.startswith("bwd_" + plan), got_plan
    name = "cls_56x56" if dtype == torch.float32 else "dit_16x16"
    gpu, _ = extreme(make_inputs(name, seed=H + 2 * W, B=B, C=C, H=H, W=W), 9 + W, recipe)
    gy = make_grad_out(name, seed=H + 3, B=B, C=C, H=H, W=W)
    d = {k: v.to(DEV) for k, v in gpu.items()}
    grads = g.propagate_backward(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                 gy.to(DEV), dirs=15, group_rows=G)
    torch.cuda.synchronize()
    assert_grad_parity(grads, oracle_grads(gpu, gy, 15, G), f"{got_plan} {shape}")
