"""Channel-shared logits on the GPU (logits [B, Cl, H, W], channel c reads
logit channel c // (C // Cl)) against the fp64 oracle, forward and backward,
through every plan (needs an MI355X)."""
from __future__ import annotations

import pytest
import torch

import linear_spatial_propagation_line_amd as g
from linear_spatial_propagation_line_amd.inputs import make_grad_out, make_inputs
from parity import assert_grad_parity, assert_parity, oracle_grads, oracle_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (shape, G, forward plan, backward plan)
CASES = [
    ((2, 4, 16, 16), 0, "plane16", "bwd_plane16"),
    ((1, 4, 56, 56), 0, "plane64", "bwd_plane64"),
    ((1, 4, 128, 128), 8, "band", "bwd_band"),
    ((1, 6, 100, 70), 5, "band", "bwd_band"),
    ((1, 4, 130, 96), 0, "tpipe", "bwd_tpipe"),
    ((1, 4, 66, 40), 20, "tpipe", "bwd_tpipe"),
    ((1, 4, 65, 80), 0, "stream", "bwd_stream"),
]


def shared_case(shape, cl, dtype, seed):
    B, C, H, W = shape
    name = "local_128x128_g8" if dtype == torch.float32 else "dit_16x16"
    inp = make_inputs(name, seed=seed, B=B, C=C, H=H, W=W)
    for k in ("l0", "l1", "l2"):
        inp[k] = inp[k][:, :cl].contiguous()
    gy = make_grad_out(name, seed=seed + 3, B=B, C=C, H=H, W=W)
    return inp, gy


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("cl", [1, 2])
@pytest.mark.parametrize("shape,G,fplan,bplan", CASES, ids=[c[2] + "-" + "x".join(map(str, c[0]))
                                                          for c in CASES])
def test_shared_logits(shape, G, fplan, bplan, cl, dtype):
    B, C, H, W = shape
    dt = 0 if dtype == torch.float32 else 1
    assert g.plan_name(B, C, H, W, 15, G, dt) == fplan
    assert g.backward_plan_name(B, C, H, W, 15, G, dt) == bplan
    inp, gy = shared_case(shape, cl, dtype, 90 + H + cl)
    d = {k: v.to(DEV) for k, v in inp.items()}
    out = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"], dirs=15,
                      group_rows=G)
    grads = g.propagate_backward(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"],
                                 gy.to(DEV), dirs=15, group_rows=G)
    torch.cuda.synchronize()
    assert grads["l0"].shape == (B, cl, H, W)
    assert_parity(out, oracle_y(inp, 15, G), f"shared forward {shape} Cl={cl}")
    assert_grad_parity(grads, oracle_grads(inp, gy, 15, G), f"shared backward {shape} Cl={cl}")


def test_shared_equals_repeated_unshared():
    """Shared logits give the same output, bit for bit, as the unshared call
    on logits repeated over each channel group."""
    shape, cl = (2, 6, 56, 56), 3
    inp, _ = shared_case(shape, cl, torch.float32, 7)
    d = {k: v.to(DEV) for k, v in inp.items()}
    rep = [d[k].repeat_interleave(shape[1] // cl, dim=1).contiguous() for k in ("l0", "l1", "l2")]
    a = g.propagate(d["x"], (d["l0"], d["l1"], d["l2"]), d["lam"], d["u"])
    b = g.propagate(d["x"], tuple(rep), d["lam"], d["u"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_t2i_shared_full_size_sampled_planes():
    """The 2048x1024x320 bf16 workload with one logit channel shared by all
    320 channels, at full size as the benchmark runs it, forward and
    backward; the oracle checks sampled planes (with their logit plane)."""
    from linear_spatial_propagation_line_amd.inputs import WORKLOADS
    w = WORKLOADS["t2i_2048x1024_cl1"]
    d = make_inputs(w, device=DEV)
    gy = make_grad_out(w, device=DEV)
    assert d["l0"].shape == (1, 1, 2048, 1024)
    lg = (d["l0"], d["l1"], d["l2"])
    out = g.propagate(d["x"], lg, d["lam"], d["u"], dirs=w.dirs)
    grads = g.propagate_backward(d["x"], lg, d["lam"], d["u"], gy, dirs=w.dirs)
    torch.cuda.synchronize()
    for c in (0, 255):
        inp = {k: (v if k in ("l0", "l1", "l2") else v[:, c:c + 1]).cpu() for k, v in d.items()}
        assert_parity(out[:, c:c + 1], oracle_y(inp, w.dirs, 0), f"t2i shared plane {c}")
        got = {k: v[:, c:c + 1] for k, v in grads.items() if k not in ("l0", "l1", "l2")}
        ref = oracle_grads(inp, gy[:, c:c + 1].cpu(), w.dirs, 0)
        ref = {k: ref[k] for k in got}
        assert_grad_parity(got, ref, f"t2i shared plane {c}", names=tuple(got))


def test_t2i_shared_logit_grads_full_size_sum_property():
    """Full-size shared logit gradients of the 2048x1024x320 one-logit-plane
    workload, which the oracle cannot take at this size (each sums all 320
    channels). A shared logit's gradient is the sum over the channels that
    read it, so it must equal the channel sum of the unshared call's logit
    gradients on logits repeated over the channels -- a call that the other
    tests check against the oracle. That call runs on the same values widened
    to fp32 storage (exact), so its per-channel gradients carry no bf16
    rounding into the sum. The x, lambda and u gradients must equal the
    unshared bf16 call's bit for bit: sharing changes only where the logits
    are read from."""
    from linear_spatial_propagation_line_amd.inputs import WORKLOADS
    w = WORKLOADS["t2i_2048x1024_cl1"]
    d = make_inputs(w, device=DEV)
    gy = make_grad_out(w, device=DEV)
    lg = (d["l0"], d["l1"], d["l2"])
    shared = g.propagate_backward(d["x"], lg, d["lam"], d["u"], gy, dirs=w.dirs)
    rep = tuple(t.expand(-1, w.C, -1, -1).contiguous() for t in lg)
    full = g.propagate_backward(d["x"], rep, d["lam"], d["u"], gy, dirs=w.dirs)
    torch.cuda.synchronize()
    for k in ("x", "lam", "u"):
        assert torch.equal(shared[k], full[k]), f"d{k} differs from the unshared call"
    del full
    f32 = {k: v.float() for k, v in d.items() if k not in ("l0", "l1", "l2")}
    rep = tuple(t.float() for t in rep)
    full = g.propagate_backward(f32["x"], rep, f32["lam"], f32["u"], gy.float(), dirs=w.dirs)
    torch.cuda.synchronize()
    for k in ("l0", "l1", "l2"):
        ref = full[k].sum(dim=1, keepdim=True).double().cpu().numpy()
        assert_parity(shared[k], ref, f"shared d{k} vs channel sum")
