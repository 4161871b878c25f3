"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, and measure errors in fp64.

Nothing from the HIP path ever feeds the oracle: the oracle computes its own
logits, routing and values from the generated inputs.  Where the HIP path's
routing is compared it is compared against the oracle's, and tokens whose
fp32 selection is a near-tie (within the logit error of an fp32 projection)
are the only ones allowed to differ.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from grouped_gemm_expert_amd import inputs

SCORE = {"softmax": 0, "sigmoid": 1}

# error bounds for floating-point outputs (max abs, relative Frobenius)
FWD_TOL = (2e-2, 1e-2)
GRAD_TOL = (3e-2, 1.5e-2)
# the MXFP8 forward against the oracle's MXFP8 forward: both quantise the same
# bf16 inputs the same way, so only fp32 accumulation and rare one-step code
# flips of a (from the kernel's fp32 SwiGLU value) separate them
MX_FWD_TOL = (2e-2, 1e-3)
# the MXFP8 backward against the oracle's MXFP8 backward: as for the forward,
# only fp32 accumulation and rare one-step code flips (of dh, quantised from
# the kernel's fp32 SwiGLU backward) separate them; measured relative
# Frobenius errors stay below 2e-3
MX_GRAD_TOL = (3e-2, 5e-3)


def say(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return inputs.bf16_bits(t)


def errors(got, ref):
    """(max abs error, relative Frobenius error) in fp64."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    d = g - r
    mx = float(np.abs(d).max()) if d.size else 0.0
    nr = float(np.linalg.norm(r))
    fro = float(np.linalg.norm(d)) / nr if nr > 0 else float(np.linalg.norm(d))
    return mx, fro


def assert_close(name, got, ref, tol):
    mx, fro = errors(got, ref)
    say(f"{name}: max_abs={mx:.3e} rel_fro={fro:.3e} (bounds {tol[0]:.1e}/{tol[1]:.1e})")
    assert mx <= tol[0] and fro <= tol[1], (name, mx, fro)
    return mx, fro


def to_device(d: dict, device="cuda") -> dict:
    out = {}
    for k, v in d.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


# ------------------------------------------------------------- HIP path ----

def run_hip(w: inputs.Workload, d: dict, *, backward=True, dw_dtype=torch.float32,
            dw_accumulate=False, dW_init=None, d_aux=1.0, logits_in=None):
    """Forward (+ backward) through moe_forward / moe_backward.  d holds the
    workload tensors on the GPU.  With `logits_in` (fp32 [T,E]) the forward
    routes on those logits (router weight not used) while the backward still
    takes the router weight, so dx includes the router path and dWr is formed.
    Returns GPU tensors."""
    from grouped_gemm_expert_amd import ops
    dev = d["x"].device
    cfg = ops.config_from_workload(w)
    saved = ops.alloc_saved(cfg, dev)
    Wr_fwd = d["Wr"]
    if logits_in is not None:
        saved["logits"].copy_(logits_in)
        Wr_fwd = None
    elif d["logits"] is not None:
        saved["logits"].copy_(d["logits"])
    y = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    wsf = ops.workspace(cfg, "fwd", dev)
    ops.moe_forward(cfg, d["x"], Wr_fwd, d["bias"], d["w1"], d["w2"], y, aux, saved, wsf)
    out = dict(y=y, aux=aux, saved=saved, cfg=cfg)
    if not backward:
        return out
    wsb = ops.workspace(cfg, "bwd", dev)
    dx = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
    dl = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    dWr = torch.empty((w.E, w.H), dtype=torch.float32, device=dev) if d["Wr"] is not None else None
    if dW_init is not None:
        dW1, dW2 = dW_init[0].clone(), dW_init[1].clone()
    else:
        dW1 = torch.empty((w.E, 2 * w.I, w.H), dtype=dw_dtype, device=dev)
        dW2 = torch.empty((w.E, w.H, w.I), dtype=dw_dtype, device=dev)
    da = torch.full((1,), d_aux, dtype=torch.float32, device=dev)
    ops.moe_backward(cfg, saved, d["x"], d["Wr"], d["w1"], d["w2"], d["dy"], da, dx, dl, dWr,
                     dW1, dW2, wsb, dw_accumulate=dw_accumulate)
    out.update(dx=dx, dlogits=dl, dWr=dWr, dW1=dW1, dW2=dW2)
    return out


# ---------------------------------------------------------------- oracle ----

def oracle_route(w: inputs.Workload, dc: dict):
    """Oracle logits (double) and routing from the generated inputs."""
    X = bits(dc["x"])
    if dc["Wr"] is not None:
        l64 = oracle.logits(X, dc["Wr"].numpy())
    else:
        l64 = dc["logits"].double().numpy()
    bias = None if dc["bias"] is None else dc["bias"].numpy()
    r = oracle.route(l64, score=SCORE[w.score], k=w.k, n_groups=w.n_groups,
                     topk_groups=w.topk_groups, bias=bias, renorm=w.renorm, scale=w.scale,
                     coeff=w.aux_coeff, route_mode=w.route)
    return l64, r


def projection_error_bound(x: torch.Tensor, Wr: torch.Tensor) -> np.ndarray:
    """Worst-case error of an fp32-accumulated x . Wr^T: H * 2^-24 * sum|x Wr|."""
    ax = x.double().abs().numpy()
    aw = Wr.double().abs().numpy()
    return (x.shape[1] * 2.0 ** -24) * (ax @ aw.T) + 1e-30


def routing_valid_under_perturbation(w: inputs.Workload, l64: np.ndarray, bias, idx_gpu,
                                     eps_logit: np.ndarray) -> np.ndarray:
    """For each token: is the GPU's chosen expert set the oracle's top-k of
    some selection scores within the logit error bound of the oracle's?  The
    witness pushes the GPU-chosen experts up by the bound and the others down."""
    l32 = l64.astype(np.float32)
    S = oracle.selection_scores(l32, SCORE[w.score], bias).astype(np.float64)
    dS = eps_logit * (0.25 if w.score == "sigmoid" else 1.0) + 2 * np.spacing(np.abs(S))
    chosen = np.zeros_like(S, bool)
    np.put_along_axis(chosen, idx_gpu.astype(np.int64), True, axis=1)
    S_w = np.where(chosen, S + dS, S - dS).astype(np.float32)
    idx_w = oracle.topk(S_w, w.k, w.n_groups, w.topk_groups)
    return (np.sort(idx_w, 1) == np.sort(idx_gpu, 1)).all(1)


def oracle_forward_backward(w: inputs.Workload, dc: dict, r: dict, l64: np.ndarray,
                            toks=None, backward=True, d_aux=1.0):
    X, W1, W2 = bits(dc["x"]), bits(dc["w1"]), bits(dc["w2"])
    y = oracle.forward(X, W1, W2, r["idx"], r["w"], toks=toks)
    out = dict(y=y)
    if backward:
        DY = bits(dc["dy"])
        Wr = None if dc["Wr"] is None else dc["Wr"].numpy()
        dx, dl = oracle.backward_tokens(X, Wr, l64, W1, W2, r["idx"], r["counts"], DY,
                                        score=SCORE[w.score], renorm=w.renorm, scale=w.scale,
                                        coeff=w.aux_coeff, d_aux=d_aux, toks=toks)
        out.update(dx=dx, dlogits=dl)
        if toks is None:
            dW1, dW2 = oracle.weight_grads(X, W1, W2, r["idx"], r["w"], DY)
            out.update(dW1=dW1, dW2=dW2)
            if dc["Wr"] is not None:
                out["dWr"] = oracle.router_weight_grad(X, dl)
    return out
