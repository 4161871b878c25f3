"""Seeded synthetic workloads for the MoE expert path.

This module is the one piece shared by the HIP path's callers and the oracle's
callers: it only draws random tensors in a fixed order.  It contains none of
the method's arithmetic (no routing, no scores, no GEMMs) and imports neither
the HIP binding nor the oracle.

Shapes follow the MoE configurations the MegaMoE page's workloads stand for
(DeepSeek-V3 with mock data on that page; the sizes here are fixed recipes).
Every tensor is drawn as fp32 N(0,1) from one ``torch.Generator`` seeded with
``seed``, in the order x -> router weight (or logits) -> bias -> w1 -> w2 -> dy,
scaled by its standard deviation and, where bf16, rounded to nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    n_groups: int = 1
    topk_groups: int = 1
    score: str = "softmax"          # "softmax" | "sigmoid"
    renorm: bool = False            # softmax router: renormalise the selected probs
    scale: float = 1.0              # sigmoid router: scale after normalising
    aux_coeff: float = 0.01
    x_std: float = 1.0
    wr_std: float = 0.02
    w_std: float = 0.02
    bias_std: Optional[float] = None
    logits: Optional[str] = None    # None: router weight; "zipf" / "normal": logits supplied
    route: str = "learned"          # "learned" | "even" (forced round-robin experts)
    # intermediates of the expert path: "bf16", or "split" (hi + lo bf16
    # pairs) for the layers whose outputs are large enough (|y| or |dW| of
    # order 10) that one bf16 rounding exceeds the absolute error budget
    precision: str = "bf16"
    backward: bool = True
    description: str = ""

    @property
    def M(self) -> int:
        return self.T * self.k

    def gemm_flops(self, backward: Optional[bool] = None) -> int:
        """Algorithmic grouped-GEMM flops: 6*M*H*I forward, 12*M*H*I backward."""
        bwd = self.backward if backward is None else backward
        f = 6 * self.M * self.H * self.I
        return f + (12 * self.M * self.H * self.I if bwd else 0)


WORKLOADS = {
    "tiny": Workload(
        "tiny", T=256, H=128, I=64, E=8, k=2, score="softmax", renorm=False,
        x_std=1.0, description="Tiny MoE fwd+bwd, top-2 softmax, no groups"),
    "few_large": Workload(
        "few_large", T=8192, H=4096, I=14336, E=8, k=2, score="softmax", renorm=True,
        x_std=1.0, backward=False, precision="split",
        description="Few-large-experts MoE fwd, top-2 softmax renorm"),
    "fine_grained": Workload(
        "fine_grained", T=16384, H=2048, I=768, E=128, k=8, score="softmax", renorm=True,
        x_std=1.0, precision="split", description="Fine-grained MoE fwd+bwd, top-8 softmax renorm"),
    "deepseek_v3": Workload(
        "deepseek_v3", T=8192, H=7168, I=2048, E=256, k=8, n_groups=8, topk_groups=4,
        score="sigmoid", scale=2.5, x_std=0.02, bias_std=0.1,
        description="DeepSeek-V3-style group-limited MoE fwd+bwd, sigmoid + bias, scale 2.5"),
    "skewed": Workload(
        "skewed", T=8192, H=7168, I=2048, E=256, k=8, n_groups=8, topk_groups=4,
        score="sigmoid", scale=2.5, x_std=0.02, logits="zipf",
        description="DeepSeek-V3 shapes, Zipf(1.2) logits, ~20% dead experts"),
    "uniform": Workload(
        "uniform", T=8192, H=7168, I=2048, E=256, k=8, n_groups=8, topk_groups=4,
        score="sigmoid", scale=2.5, x_std=0.02, logits="normal",
        description="DeepSeek-V3 shapes, i.i.d. N(0,1) logits (balanced routing)"),
    # test shapes: several GEMM tiles and ragged tails, small enough for the oracle
    "ep8_share": Workload(
        "ep8_share", T=8192, H=7168, I=2048, E=32, k=8, score="sigmoid", scale=2.5, x_std=0.02,
        route="even",
        description="one GPU's share of DeepSeek-V3 under EP8: 32 local experts, 65536 rows "
                    "split evenly (even routing)"),
    "mid_softmax": Workload(
        "mid_softmax", T=600, H=256, I=192, E=16, k=4, score="softmax", renorm=True,
        x_std=1.0, description="parity shape, softmax renorm"),
    "mid_sigmoid": Workload(
        "mid_sigmoid", T=500, H=384, I=320, E=32, k=6, n_groups=4, topk_groups=2,
        score="sigmoid", scale=2.5, x_std=1.0, bias_std=0.1,
        description="parity shape, sigmoid + bias, group-limited"),
    "mid_even": Workload(
        "mid_even", T=530, H=256, I=192, E=24, k=4, n_groups=4, topk_groups=2,
        score="sigmoid", scale=2.5, x_std=1.0, bias_std=0.1, route="even",
        description="parity shape, even forced routing (sigmoid, groups ignored)"),
    "even_softmax": Workload(
        "even_softmax", T=333, H=128, I=128, E=8, k=2, score="softmax", renorm=False,
        x_std=1.0, route="even",
        description="parity shape, even forced routing, softmax without renorm"),
    "mid_split": Workload(
        "mid_split", T=600, H=256, I=192, E=16, k=4, score="softmax", renorm=True,
        x_std=1.0, precision="split", description="parity shape, split intermediates"),
    "mid_sigmoid_split": Workload(
        "mid_sigmoid_split", T=500, H=384, I=320, E=32, k=6, n_groups=4, topk_groups=2,
        score="sigmoid", scale=2.5, x_std=1.0, bias_std=0.1, precision="split",
        description="parity shape, sigmoid + bias, group-limited, split intermediates"),
    "mid_skewed": Workload(
        "mid_skewed", T=700, H=256, I=128, E=64, k=4, n_groups=8, topk_groups=4,
        score="sigmoid", scale=2.5, x_std=1.0, logits="zipf",
        description="parity shape, Zipf logits with dead experts"),
}

_CHUNK = 1 << 27  # elements per randn call for big tensors (bounds the fp32 temporary)


def _randn(shape, std: float, dtype, gen: torch.Generator, device) -> torch.Tensor:
    """fp32 N(0,1) * std, cast (round-to-nearest-even) to dtype; drawn in chunks
    along dim 0 so the fp32 temporary stays bounded."""
    out = torch.empty(shape, dtype=dtype, device=device)
    if out.numel() == 0:
        return out
    rows = shape[0]
    per_row = out.numel() // rows
    step = max(1, _CHUNK // max(per_row, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        out[r0:r1].copy_(tmp)
        del tmp
    return out


def _zipf_logits(T: int, E: int, gen: torch.Generator, device) -> torch.Tensor:
    """Skewed-routing logits: a seeded permutation marks 20% of the experts dead
    (logit -30); the others get ranks r = 1.. and logit = -1.2 ln r + Gumbel(0,1),
    so popularity follows Zipf(1.2) under Gumbel-top-k sampling."""
    perm = torch.randperm(E, generator=gen, device=device)
    n_dead = int(round(0.2 * E))
    rank = torch.empty(E, dtype=torch.float32, device=device)
    rank[perm] = torch.arange(1, E + 1, dtype=torch.float32, device=device)
    u = torch.rand((T, E), generator=gen, device=device, dtype=torch.float32)
    u = u.clamp_(min=1e-12, max=1.0 - 1e-7)
    gumbel = -torch.log(-torch.log(u))
    base = -1.2 * torch.log(rank)
    logits = base.unsqueeze(0) + gumbel
    dead = perm[E - n_dead:]
    logits[:, dead] = -30.0
    return logits.contiguous()


def make_inputs(w: Workload | str, device="cpu", seed: int = 0, with_dy: Optional[bool] = None,
                T: Optional[int] = None) -> dict:
    """Draw the workload's tensors.  Returns a dict with x [T,H] bf16, Wr [E,H] fp32
    (or None), logits [T,E] fp32 (or None), bias [E] fp32 (or None), w1 [E,2I,H]
    bf16, w2 [E,H,I] bf16 and dy [T,H] bf16 (or None).  ``T`` overrides the token
    count (same recipe, fewer or more tokens)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if T is not None:
        w = dataclasses.replace(w, T=T)
    if with_dy is None:
        with_dy = w.backward
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {"workload": w}
    out["x"] = _randn((w.T, w.H), w.x_std, torch.bfloat16, gen, device)
    if w.logits is None:
        out["Wr"] = _randn((w.E, w.H), w.wr_std, torch.float32, gen, device)
        out["logits"] = None
    elif w.logits == "zipf":
        out["Wr"] = None
        out["logits"] = _zipf_logits(w.T, w.E, gen, device)
    elif w.logits == "normal":
        out["Wr"] = None
        out["logits"] = _randn((w.T, w.E), 1.0, torch.float32, gen, device)
    else:
        raise ValueError(w.logits)
    out["bias"] = (_randn((w.E,), w.bias_std, torch.float32, gen, device)
                   if w.bias_std is not None else None)
    out["w1"] = _randn((w.E, 2 * w.I, w.H), w.w_std, torch.bfloat16, gen, device)
    out["w2"] = _randn((w.E, w.H, w.I), w.w_std, torch.bfloat16, gen, device)
    out["dy"] = _randn((w.T, w.H), 1.0, torch.bfloat16, gen, device) if with_dy else None
    return out


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def describe(w: Workload) -> str:
    return (f"{w.name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} G={w.n_groups} "
            f"kg={w.topk_groups} {w.score}" + (" renorm" if w.renorm else "")
            + (" split" if w.precision == "split" else "")
            + (f" scale={w.scale}" if w.score == "sigmoid" else ""))
