"""torch.autograd binding of the whole layer: MoEFunction runs moe_forward in
its forward and moe_backward in its backward, and nothing else.

The MegaMoE page ("Design: two stages + weight modules") keeps the split of
the layer into its weight-owning stages at the Python / autograd level; here
the autograd node covers the one-call forms, and the stage entry points stay
available in ``ops`` for callers that hook each weight separately.

Arguments are marshalled only: tensors go to the library as device pointers
on the current stream.  The one conversion is at the layer's edge: the
incoming gradient of y is rounded to bf16, the dtype moe_backward takes dy in.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import ops


class MoEFunction(torch.autograd.Function):
    """(y, aux) = MoE(x, Wr, bias, w1, w2) for one moe_config.

    x [T,H] bf16, Wr [E,H] fp32 router weight, bias [E] fp32 selection-only
    bias or None, w1 [E,2I,H] and w2 [E,H,I] bf16.  y [T,H] fp32, aux [1]
    fp32.  Gradients: x, Wr, w1, w2 (the library's fp32 results, which
    autograd casts to each input's dtype); bias and the selection carry none.
    """

    @staticmethod
    def forward(ctx, x, Wr, bias, w1, w2, cfg: ops.MoeConfig):
        dev = x.device
        saved = ops.alloc_saved(cfg, dev)
        y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
        aux = torch.empty((1,), dtype=torch.float32, device=dev)
        ops.moe_forward(cfg, x, Wr, bias, w1, w2, y, aux, saved, ops.workspace(cfg, "fwd", dev))
        ctx.cfg = cfg
        ctx.saved = saved
        ctx.save_for_backward(x, Wr, w1, w2)
        return y, aux

    @staticmethod
    def backward(ctx, dy: Optional[torch.Tensor], d_aux: Optional[torch.Tensor]):
        x, Wr, w1, w2 = ctx.saved_tensors
        cfg = ctx.cfg
        dev = x.device
        if dy is None:
            dy = torch.zeros((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
        dy = dy.to(torch.bfloat16).contiguous()
        if d_aux is not None:
            d_aux = d_aux.to(torch.float32).contiguous()
        dx = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
        dlogits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
        dWr = torch.empty((cfg.E, cfg.H), dtype=torch.float32, device=dev) if Wr is not None else None
        dW1 = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.float32, device=dev)
        dW2 = torch.empty((cfg.E, cfg.H, cfg.I), dtype=torch.float32, device=dev)
        ops.moe_backward(cfg, ctx.saved, x, Wr, w1, w2, dy, d_aux, dx, dlogits, dWr, dW1, dW2,
                         ops.workspace(cfg, "bwd", dev))
        ctx.saved = None
        return dx, dWr, None, dW1, dW2, None


def moe(x, Wr, bias, w1, w2, cfg: ops.MoeConfig):
    """Functional form: (y, aux) = MoEFunction.apply(x, Wr, bias, w1, w2, cfg)."""
    return MoEFunction.apply(x, Wr, bias, w1, w2, cfg)
