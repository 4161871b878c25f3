"""An independent, differentiable fp64 formulation of the MoE expert path, on
the CPU, used only to pin the oracle's hand-derived backward (the oracle loops
per token; this one evaluates every expert on every token and masks with a
dense [T,E] combine-weight matrix, then lets torch.autograd differentiate).

Routing indices and counts are inputs: the selection carries no gradient.
"""
from __future__ import annotations

import torch


def dense_loss(x, w1, w2, idx, dy, *, score, renorm, scale, coeff, d_aux, counts,
               Wr=None, logits=None):
    """Loss = sum(y * dy) + d_aux * aux, everything in float64.

    x [T,H], w1 [E,2I,H], w2 [E,H,I], Wr [E,H] (or logits [T,E]), idx [T,k] int64,
    counts [E].  Returns (loss, y, aux, logits)."""
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    k = idx.shape[1]
    if logits is None:
        logits = x @ Wr.t()
    if score == "softmax":
        p = torch.softmax(logits, dim=-1)
        psel = torch.gather(p, 1, idx)
        w = psel / psel.sum(-1, keepdim=True) if renorm else psel
        probs = p
    else:
        s = torch.sigmoid(logits)
        ssel = torch.gather(s, 1, idx)
        w = scale * ssel / ssel.sum(-1, keepdim=True)
        probs = s / s.sum(-1, keepdim=True)
    comb = torch.zeros(T, E, dtype=x.dtype).scatter_add(1, idx, w)
    h = torch.einsum("th,enh->ten", x, w1)
    g, u = h[..., :I], h[..., I:]
    a = torch.nn.functional.silu(g) * u
    o = torch.einsum("tei,ehi->teh", a, w2)
    y = torch.einsum("te,teh->th", comb, o)
    if T > 0:
        aux = coeff * E / (k * T * T) * (counts.to(x.dtype) * probs.sum(0)).sum()
    else:
        aux = torch.zeros((), dtype=x.dtype)
    loss = (y * dy).sum() + d_aux * aux
    return loss, y, aux, logits
