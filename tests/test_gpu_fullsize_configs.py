"""Parity at the full sizes of the other configurations of the benchmark
suite (the DeepSeek-V3-style one is covered by test_gpu_fullsize.py), run
through moe_forward / moe_backward the way bench.py launches them (weight
gradients accumulated in fp32 into zeros):
  - few_large     T=8192 H=4096 I=14336 E=8, top-2 softmax, renormalised
                  (a forward workload)
  - fine_grained  T=16384 H=2048 I=768 E=128, top-8 softmax, renormalised
  - skewed        the DeepSeek-V3 shapes with Zipf(1.2) logits supplied
                  (about 20% of the experts get no token, one more than 10%)
The oracle cannot run these layers whole, so it checks what it can compute one
output at a time:
  - the routing of every token: bit-exact given the same fp32 logits, else
    (router projection on the GPU) explained by the projection's rounding;
  - aux, and y of sampled tokens;
  - with the backward: dx and dlogits of sampled tokens, sampled dW1 / dW2
    elements of the two busiest experts, and exact zeros in the weight
    gradients of experts without tokens;
  - the same layers through the MXFP8 path against the oracle's MXFP8
    forward and backward.
Only the experts the samples touch are copied to the host, into full-shape
zero arrays (np.zeros maps untouched pages lazily) or compact arrays."""
import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_expert_amd import inputs
from tests import harness as hz

pytestmark = pytest.mark.gpu

N_TOK = 4      # sampled tokens
N_EL = 12      # sampled dW elements per weight and expert


def _sparse_full(d, experts):
    """Full-shape host bf16 bits of w1 / w2 holding only the listed experts."""
    ex = torch.as_tensor(np.asarray(experts), device="cuda")
    w1 = np.zeros(tuple(d["w1"].shape), np.uint16)
    w2 = np.zeros(tuple(d["w2"].shape), np.uint16)
    w1[np.asarray(experts)] = hz.bits(d["w1"].index_select(0, ex))
    w2[np.asarray(experts)] = hz.bits(d["w2"].index_select(0, ex))
    return w1, w2


@pytest.fixture(scope="module", params=["few_large", "fine_grained", "skewed"])
def run(request):
    w = inputs.WORKLOADS[request.param]
    hz.say(f"fullsize {w.name}: generating {inputs.describe(w)} on the GPU")
    d = inputs.make_inputs(w, device="cuda", seed=0)
    hz.say(f"fullsize {w.name}: moe_forward" + (" + moe_backward" if w.backward else ""))
    dW_init = None
    if w.backward:
        dW_init = (torch.zeros((w.E, 2 * w.I, w.H), device="cuda"),
                   torch.zeros((w.E, w.H, w.I), device="cuda"))
    out = hz.run_hip(w, d, backward=w.backward, dw_accumulate=True, dW_init=dW_init)
    torch.cuda.synchronize()
    hz.say(f"fullsize {w.name}: oracle logits and routing")
    X = hz.bits(d["x"])
    Wr = None if d["Wr"] is None else d["Wr"].cpu().numpy()
    bias = None if d["bias"] is None else d["bias"].cpu().numpy()
    l64 = oracle.logits(X, Wr) if Wr is not None else d["logits"].double().cpu().numpy()
    r = oracle.route(l64, score=hz.SCORE[w.score], k=w.k, n_groups=w.n_groups,
                     topk_groups=w.topk_groups, bias=bias, renorm=w.renorm, scale=w.scale,
                     coeff=w.aux_coeff, route_mode=w.route)
    idx_gpu = out["saved"]["topk_idx"].cpu().numpy()
    same = (idx_gpu == r["idx"]).all(1)
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(np.nonzero(same)[0], size=N_TOK, replace=False))
    yield dict(w=w, d=d, out=out, X=X, Wr=Wr, bias=bias, l64=l64, r=r, idx_gpu=idx_gpu,
               same=same, toks=toks)
    del out, d
    torch.cuda.empty_cache()


def test_fullsize_config_routing(run):
    w, r, same = run["w"], run["r"], run["same"]
    hz.say(f"fullsize {w.name} routing: identical on {int(same.sum())} of {w.T} tokens")
    if run["Wr"] is None:       # the same fp32 logits on both sides: bit-exact
        assert same.all()
    else:
        assert same.mean() >= 0.99
        bad = ~same
        if bad.any():
            xb = run["d"]["x"][torch.as_tensor(np.nonzero(bad)[0], device="cuda")].cpu().float()
            eps = hz.projection_error_bound(xb, torch.from_numpy(run["Wr"]))
            ok = hz.routing_valid_under_perturbation(w, run["l64"][bad], run["bias"],
                                                     run["idx_gpu"][bad], eps)
            assert ok.all()
    counts_gpu = run["out"]["saved"]["counts"].cpu().numpy()
    if same.all():
        assert np.array_equal(counts_gpu, r["counts"])
    aux_g = float(run["out"]["aux"].cpu())
    assert abs(aux_g - r["aux"]) <= 1e-3 * abs(r["aux"]) + 1e-9, (aux_g, r["aux"])
    if w.name == "skewed":      # the load the configuration asks for
        assert (r["counts"] == 0).mean() >= 0.15
        assert r["counts"].max() > 0.10 * w.T * w.k


def test_fullsize_config_sampled_tokens(run):
    w, r, toks = run["w"], run["r"], run["toks"]
    ex = np.unique(r["idx"][toks])
    hz.say(f"fullsize {w.name} tokens {toks.tolist()}: {len(ex)} experts to the host")
    W1s, W2s = _sparse_full(run["d"], ex)
    tk = torch.as_tensor(toks, device="cuda")
    y_ref = oracle.forward(run["X"], W1s, W2s, r["idx"], r["w"], toks=toks)
    hz.assert_close(f"fullsize {w.name} y", run["out"]["y"][tk].cpu().numpy(), y_ref, hz.FWD_TOL)
    if not w.backward:
        return
    DY = hz.bits(run["d"]["dy"])
    dx_ref, dl_ref = oracle.backward_tokens(run["X"], run["Wr"], run["l64"], W1s, W2s, r["idx"],
                                            r["counts"], DY, score=hz.SCORE[w.score],
                                            renorm=w.renorm, scale=w.scale, coeff=w.aux_coeff,
                                            d_aux=1.0, toks=toks)
    hz.assert_close(f"fullsize {w.name} dx", run["out"]["dx"][tk].cpu().numpy(), dx_ref,
                    hz.GRAD_TOL)
    hz.assert_close(f"fullsize {w.name} dlogits", run["out"]["dlogits"][tk].cpu().numpy(),
                    dl_ref, hz.GRAD_TOL)


def test_fullsize_config_weight_grads(run):
    w, r = run["w"], run["r"]
    if not w.backward:
        pytest.skip(f"{w.name} is a forward workload")
    counts = r["counts"]
    ex = np.argsort(-counts, kind="stable")[:2]          # the two busiest experts
    hz.say(f"fullsize {w.name} dW: experts {ex.tolist()} with {counts[ex].tolist()} rows")
    W1s, W2s = _sparse_full(run["d"], ex)
    DY = hz.bits(run["d"]["dy"])
    rng = np.random.default_rng(2)
    which, ee, rr, cc = [], [], [], []
    for e in ex:
        for wh, nr, nc in ((1, 2 * w.I, w.H), (2, w.H, w.I)):
            which += [wh] * N_EL
            ee += [int(e)] * N_EL
            rr += rng.integers(0, nr, N_EL).tolist()
            cc += rng.integers(0, nc, N_EL).tolist()
    which, ee, rr, cc = (np.array(v, np.int32) for v in (which, ee, rr, cc))
    ref = oracle.weight_grad_elements(run["X"], W1s, W2s, r["idx"], r["w"], DY, which, ee, rr, cc)
    for wh, name in ((1, "dW1"), (2, "dW2")):
        dW = run["out"][name]
        sel = which == wh
        e_, r_, c_ = ee[sel], rr[sel], cc[sel]
        # indices checked on the host: the gather below does not check them
        assert (e_ < dW.shape[0]).all() and (r_ < dW.shape[1]).all() and (c_ < dW.shape[2]).all()
        got = dW[torch.as_tensor(e_, device="cuda"), torch.as_tensor(r_, device="cuda"),
                 torch.as_tensor(c_, device="cuda")].cpu().numpy()
        hz.assert_close(f"fullsize {w.name} {name} elements", got, ref[sel], hz.GRAD_TOL)
    empty = np.nonzero(counts == 0)[0]
    if len(empty):
        ez = torch.as_tensor(empty[:4], device="cuda")
        for name in ("dW1", "dW2"):
            assert float(run["out"][name].index_select(0, ez).abs().max().cpu()) == 0.0


# ---------------------------------------------------------------- MXFP8 ----
# The same configurations through the MXFP8 path (weight cache with the
# forward and transposed forms), on the same inputs, against the oracle's
# MXFP8 forward (sampled tokens) and backward (dx, dlogits of two sampled
# tokens; sampled dW elements of the busiest expert).

def _compact(d, experts):
    ex = torch.as_tensor(np.asarray(experts), device="cuda")
    return hz.bits(d["w1"].index_select(0, ex)), hz.bits(d["w2"].index_select(0, ex))


def _remap(idx, experts):
    m = np.full(int(idx.max()) + 1, -1, np.int32)
    m[np.asarray(experts)] = np.arange(len(experts), dtype=np.int32)
    return m[idx]


@pytest.fixture(scope="module")
def runmx(run):
    from grouped_gemm_expert_amd import ops
    w, d = run["w"], run["d"]
    cfg = ops.config_from_workload(w)
    hz.say(f"fullsize {w.name} mx: quantising the weights")
    cache = ops.MxWeightCache(backward=w.backward)
    cache.get(d["w1"], d["w2"])
    saved = ops.alloc_saved(cfg)
    if d["logits"] is not None:
        saved["logits"].copy_(d["logits"])
    y = torch.empty((w.T, w.H), device="cuda")
    aux = torch.empty((1,), device="cuda")
    hz.say(f"fullsize {w.name} mx: moe_forward_mx" + (" + moe_backward_mx" if w.backward else ""))
    ops.moe_forward_mx(cfg, d["x"], d["Wr"], d["bias"], cache.w1_mx, cache.w2_mx, y, aux, saved,
                       ops.workspace(cfg, "fwd"))
    out = dict(saved=saved, y=y)
    if w.backward:
        dx = torch.empty((w.T, w.H), device="cuda")
        dl = torch.empty((w.T, w.E), device="cuda")
        dWr = torch.empty((w.E, w.H), device="cuda") if d["Wr"] is not None else None
        dW1 = torch.zeros((w.E, 2 * w.I, w.H), device="cuda")
        dW2 = torch.zeros((w.E, w.H, w.I), device="cuda")
        d_aux = torch.ones((1,), device="cuda")
        ops.moe_backward_mx(cfg, saved, d["x"], d["Wr"], cache.w1t_mx, cache.w2t_mx, d["dy"],
                            d_aux, dx, dl, dWr, dW1, dW2, ops.workspace(cfg, "bwd"),
                            dw_accumulate=True)
        out.update(dx=dx, dl=dl, dW1=dW1, dW2=dW2)
    torch.cuda.synchronize()
    yield out
    del out, cache
    torch.cuda.empty_cache()


def test_fullsize_config_mx_forward(run, runmx):
    """y of sampled tokens against the oracle's MXFP8 forward.  The MFMA adds
    each group of 8 products in a fixed-point window (about 13 bits below the
    group's largest product) and the group sums in fp32, so an output of
    GEMM2 is within (2^-10 + (I/8 + 1) 2^-24) * sum_i |a_i w2[h, i]| of the
    exact sum of its MX products; at few-large's I = 14336 and |y| ~ 11 that
    exceeds the fixed MX tolerance.  Each element is held to that bound
    (summed over the token's slots with their weights) plus the forward's
    absolute bound, and the whole to the forward's relative bound."""
    w, r, toks = run["w"], run["r"], run["toks"]
    assert np.array_equal(runmx["saved"]["topk_idx"].cpu().numpy(), run["idx_gpu"])
    ex = np.unique(r["idx"][toks])
    W1c, W2c = _compact(run["d"], ex)
    ops_o = oracle.MxOperands(run["X"][toks], W1c, W2c)
    idx_c = _remap(r["idx"][toks], ex)
    wt = r["w"][toks]
    y_ref = oracle.mx_forward(ops_o, idx_c, wt)
    y_gpu = runmx["y"][torch.as_tensor(toks, device="cuda")].cpu().numpy().astype(np.float64)
    # sum_i |a_i w2[e, h, i]| per slot, from the oracle's MX a and MX w2
    k = idx_c.shape[1]
    _, _, _, aq, as_, _ = oracle.mx_expert_rows(ops_o, idx_c, np.arange(len(toks) * k))
    A = np.abs(oracle.mx_dequantize(aq, as_)).astype(np.float32)          # [n*k, I]
    win = 2.0 ** -10 + (w.I / 8 + 1) * 2.0 ** -24
    bound = np.zeros_like(y_ref)
    for c_e in range(len(ex)):
        rows = slice(c_e * w.H, (c_e + 1) * w.H)
        W2 = np.abs(oracle.mx_dequantize(ops_o.w2q[rows], ops_o.w2s[rows])).astype(np.float32)
        for p in range(len(toks)):
            for j in range(k):
                if idx_c[p, j] == c_e:
                    bound[p] += wt[p, j] * win * (W2 @ A[p * k + j]).astype(np.float64)
    err = np.abs(y_gpu - y_ref)
    hz.say(f"fullsize {w.name} mx y: max_abs={err.max():.3e}, largest share of the window "
           f"bound {float((err / (bound + hz.FWD_TOL[0])).max()):.3f}")
    assert (err <= bound + hz.FWD_TOL[0]).all()
    rel = np.linalg.norm(y_gpu - y_ref) / np.linalg.norm(y_ref)
    assert rel <= hz.FWD_TOL[1], rel


def test_fullsize_config_mx_backward(run, runmx):
    w, r = run["w"], run["r"]
    if not w.backward:
        pytest.skip(f"{w.name} is a forward workload")
    toks = run["toks"][:2]
    ex = np.unique(r["idx"][toks])
    W1c, W2c = _compact(run["d"], ex)
    DY = hz.bits(run["d"]["dy"])
    ops_o = oracle.MxBackwardOperands.from_experts(run["X"], DY, w.E, ex, W1c, W2c)
    dx_ref, dl_ref = oracle.mx_backward_tokens(ops_o, run["Wr"], run["l64"], r["idx"],
                                               r["counts"], r["w"], score=hz.SCORE[w.score],
                                               renorm=w.renorm, scale=w.scale,
                                               coeff=w.aux_coeff, d_aux=1.0, toks=toks)
    tk = torch.as_tensor(toks, device="cuda")
    hz.assert_close(f"fullsize {w.name} mx dx", runmx["dx"][tk].cpu().numpy(), dx_ref,
                    hz.MX_GRAD_TOL)
    hz.assert_close(f"fullsize {w.name} mx dlogits", runmx["dl"][tk].cpu().numpy(), dl_ref,
                    hz.MX_GRAD_TOL)
    e = int(np.argmax(r["counts"]))                      # the busiest expert
    W1c, W2c = _compact(run["d"], [e])
    ops_w = oracle.MxBackwardOperands.from_experts(run["X"], DY, w.E, np.array([e]), W1c, W2c)
    rng = np.random.default_rng(3)
    which, ee, rr, cc = [], [], [], []
    for wh, nr, nc in ((1, 2 * w.I, w.H), (2, w.H, w.I)):
        which += [wh] * N_EL
        ee += [e] * N_EL
        rr += rng.integers(0, nr, N_EL).tolist()
        cc += rng.integers(0, nc, N_EL).tolist()
    which, ee, rr, cc = (np.array(v, np.int32) for v in (which, ee, rr, cc))
    ref = oracle.mx_weight_grad_elements(ops_w, run["X"], DY, r["idx"], r["w"], which, ee, rr, cc)
    for wh, name in ((1, "dW1"), (2, "dW2")):
        sel = which == wh
        dW = runmx[name]
        e_, r_, c_ = ee[sel], rr[sel], cc[sel]
        assert (e_ < dW.shape[0]).all() and (r_ < dW.shape[1]).all() and (c_ < dW.shape[2]).all()
        got = dW[torch.as_tensor(e_, device="cuda"), torch.as_tensor(r_, device="cuda"),
                 torch.as_tensor(c_, device="cuda")].cpu().numpy()
        hz.assert_close(f"fullsize {w.name} mx {name} elements", got, ref[sel], hz.MX_GRAD_TOL)
