"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random tensors; it holds none of the propagation's
arithmetic. Both the HIP path and the CPU oracle consume the tensors it makes.

Workloads (the pages' settings, with synthetic data in place of ImageNet,
DiT latents and SD-XL text-to-image latents, which need datasets and trained
weights):
  tiny_16x16_t2b     B=1,  C=4,    16x16,     fp32, top->bottom only, global
  cls_56x56          B=64, C=96,   56x56,     fp32, 4 directions, global
                     (first stage of a Swin-like classifier; aitntnews page,
                     section GSPN架构)
  dit_16x16          B=32, C=1152, 16x16,     bf16, 4 directions, global
                     (DiT-XL/2 latent of a 256x256 image: /8 VAE, patch 2)
  local_128x128_g8   B=16, C=192,  128x128,   fp32, 4 directions, groups of 8
  t2i_2048x1024      B=1,  C=320,  2048x1024, bf16, 4 directions, global
                     (16Kx8K text-to-image latent, /8 VAE; aitntnews page,
                     section 文本到图像生成)
  t2i_2048x1024_cl1  the same with one logit channel shared by all 320
                     channels (the speed-test setting of the CSDN page,
                     section 局限性: the weights' feature dimension set to 1)
  cls_56x56_pd       cls_56x56 with one set of (lambda, logits, u) per scan
  t2i_2048x1024_pd   direction and per-channel merge weights (aitntnews page,
                     sections 二维线性传播 and GSPN架构; CSDN page, section
                     GSPN模块的设计)
  cls_56x56_mod      the whole unit: the prologue's 1x1 convolutions produce
  dit_16x16_mod      x, the logits, lambda and u from an input of Cin = C
  t2i_2048x1024_mod  channels (aitntnews page, section GSPN架构), then the
                     propagation
  t2i_1024x2048      the text-to-image latent in portrait orientation and
  t2i_2047x1023      with odd sides (the pages' model runs at arbitrary
                     resolution: aitntnews page, section 文本到图像生成)

Draw order is x, lambda, u, l0, l1, l2, each drawn in float32 from one
generator seeded with 1000 + k (k = 1..8 in the order above) and then cast
(round-to-nearest-even) to the storage type. Per-direction workloads draw
lambda, u and the logits as [4, B, C, H, W] (slice d for direction d) in the
same order, then merge weights [4, C] from U(-1, 1), kept in float32. Module
workloads draw, from one generator seeded 3000 + k, x_in ~ N(0, 1)
[B, Cin, H, W], w_reduce [C, Cin] normal with standard deviation Cin^-1/2,
b_reduce [C] with standard deviation 0.1, w_params [5C, C] with standard
deviation C^-1/2, b_params [5C] with 0.1, in that order, each
cast to the storage type (weights scaled so that x and the parameters stay
near unit variance). The output gradient of the
backward pass (make_grad_out) is N(0, 1) from a generator seeded with
2000 + k, cast the same way.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based position in the table above (seed = 1000 + index)
    B: int
    C: int
    H: int
    W: int
    dtype: str          # "f32" or "bf16"
    dirs: int           # bit mask: 1 T->B, 2 B->T, 4 L->R, 8 R->L
    group_rows: int     # 0 = global
    logits: tuple       # distribution spec
    x: tuple
    lam: tuple
    u: tuple
    logit_channels: int = 0   # 0: one logit channel per channel (unshared)
    per_direction: bool = False   # own (lambda, logits, u) per direction + merge weights
    prologue_cin: int = 0         # > 0: the whole unit, prologue from Cin channels

    @property
    def cl(self) -> int:
        return self.logit_channels or self.C

    @property
    def pixels(self) -> int:
        return self.B * self.C * self.H * self.W

    @property
    def ndirs(self) -> int:
        return bin(self.dirs).count("1")

    @property
    def elem_steps(self) -> int:
        return self.pixels * self.ndirs

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    def with_planes(self, B: int | None = None, C: int | None = None) -> "Workload":
        return replace(self, B=self.B if B is None else B, C=self.C if C is None else C)


NORMAL1 = ("normal", 1.0)
SIG_NORMAL = ("sigmoid_normal", 1.0)

WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_16x16_t2b", 1, 1, 4, 16, 16, F32, 1, 0,
                 NORMAL1, ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0)),
        Workload("cls_56x56", 2, 64, 96, 56, 56, F32, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL),
        Workload("dit_16x16", 3, 32, 1152, 16, 16, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL),
        Workload("local_128x128_g8", 4, 16, 192, 128, 128, F32, 15, 8,
                 ("normal", 2.0), NORMAL1, ("uniform", 0.0, 1.0), ("uniform", 0.0, 1.0)),
        Workload("t2i_2048x1024", 5, 1, 320, 2048, 1024, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL),
        Workload("t2i_2048x1024_cl1", 6, 1, 320, 2048, 1024, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL, logit_channels=1),
        Workload("cls_56x56_pd", 7, 64, 96, 56, 56, F32, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL, per_direction=True),
        Workload("t2i_2048x1024_pd", 8, 1, 320, 2048, 1024, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL, per_direction=True),
        Workload("cls_56x56_mod", 9, 64, 96, 56, 56, F32, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL, prologue_cin=96),
        Workload("dit_16x16_mod", 10, 32, 1152, 16, 16, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL, prologue_cin=1152),
        Workload("t2i_2048x1024_mod", 11, 1, 320, 2048, 1024, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL, prologue_cin=320),
        Workload("t2i_1024x2048", 12, 1, 320, 1024, 2048, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL),
        Workload("t2i_2047x1023", 13, 1, 320, 2047, 1023, BF16, 15, 0,
                 NORMAL1, NORMAL1, SIG_NORMAL, SIG_NORMAL),
    ]
}


def _draw(spec, shape, gen, device):
    kind = spec[0]
    if kind == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * spec[1]
    if kind == "sigmoid_normal":
        return torch.sigmoid(torch.randn(shape, generator=gen, device=device,
                                         dtype=torch.float32) * spec[1])
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        return torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * (hi - lo) + lo
    raise ValueError(kind)


def make_inputs(w: Workload | str, seed: int | None = None, device="cpu",
                B: int | None = None, C: int | None = None, H: int | None = None,
                W: int | None = None) -> dict:
    """Tensors x, lam, u of shape [B, C, H, W] and l0, l1, l2 of shape
    [B, Cl, H, W] (Cl = C unless the workload shares logits) in the
    workload's storage dtype on ``device``. Per-direction workloads give
    lam, u, l0, l1, l2 of shape [4, B, C, H, W] and merge weights "merge"
    [4, C] in float32. Shape overrides keep the distributions."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    shape = (B or w.B, C or w.C, H or w.H, W or w.W)
    lshape = (shape[0], w.logit_channels or shape[1], shape[2], shape[3])
    if seed is None:
        seed = 1000 + w.index
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for name, spec in (("x", w.x), ("lam", w.lam), ("u", w.u),
                       ("l0", w.logits), ("l1", w.logits), ("l2", w.logits)):
        shp = lshape if name in ("l0", "l1", "l2") else shape
        if w.per_direction and name != "x":
            shp = (4,) + tuple(shp)
        out[name] = _draw(spec, shp, gen, device).to(w.torch_dtype)
    if w.per_direction:
        out["merge"] = _draw(("uniform", -1.0, 1.0), (4, shape[1]), gen, device)
    return out


def make_prologue_inputs(w: Workload | str | None = None, seed: int | None = None,
                         device="cpu", B: int | None = None, Cin: int | None = None,
                         C: int | None = None, H: int | None = None, W: int | None = None,
                         dtype: str | None = None) -> dict:
    """Input and weights of the module prologue: "x_in" [B, Cin, H, W],
    "w_r" [C, Cin], "b_r" [C], "w_p" [5C, C], "b_p" [5C] in the storage dtype
    (the workload's, or ``dtype``) on ``device``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = B or w.B
    Cin = Cin or w.prologue_cin
    C = C or w.C
    H = H or w.H
    W = W or w.W
    tdt = {F32: torch.float32, BF16: torch.bfloat16}[dtype or w.dtype]
    if seed is None:
        seed = 3000 + (w.index if w is not None else 0)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(shape, std):
        return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std).to(tdt)

    return {"x_in": normal((B, Cin, H, W), 1.0),
            "w_r": normal((C, Cin), Cin ** -0.5),
            "b_r": normal((C,), 0.1),
            "w_p": normal((5 * C, C), C ** -0.5),
            "b_p": normal((5 * C,), 0.1)}


def make_grad_out(w: Workload | str, seed: int | None = None, device="cpu",
                  B: int | None = None, C: int | None = None, H: int | None = None,
                  W: int | None = None) -> torch.Tensor:
    """dL/dout for the backward pass: N(0, 1) in the workload's storage dtype."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    shape = (B or w.B, C or w.C, H or w.H, W or w.W)
    if seed is None:
        seed = 2000 + w.index
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(w.torch_dtype)
