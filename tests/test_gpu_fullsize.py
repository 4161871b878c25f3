"""Parity at the full DeepSeek-V3-style size (T=8192, H=7168, I=2048, E=256 in
8 groups, top-4 groups, top-8 sigmoid + bias, scale 2.5), in the launch
configuration the benchmark times: moe_forward from the router weight, then
moe_backward accumulating into zeroed fp32 weight gradients; and the MXFP8
forward and backward on the same inputs.  The oracle cannot run the whole
layer at this size, so it is checked on outputs it computes one by one,
chosen to reach every tile the kernels compute:
  - routing of every token (bit-exact on all tokens whose fp32 selection is
    not a near-tie under the projection's rounding),
  - y, dx and dlogits of tokens whose slots are the first and last sorted row
    of every active expert and of 256-row tiles inside them,
  - whole weight-gradient lines of every active expert: a dW1 row in every
    256-row band and a dW2 column in every 256-column band (together they
    reach every 256 x 256 output tile), and exact zeros for every expert
    without rows,
  - the MX forward's y, dx and dlogits on fewer of those tokens, and whole MX
    dW lines of three experts, against the oracle's MXFP8 path.
Only the experts the samples touch are copied to the host: into full-shape
zero arrays (np.zeros maps untouched pages lazily, so only those experts take
memory) for the oracle calls that index experts by their ids, and into
compact arrays with remapped expert ids elsewhere."""
import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_expert_amd import inputs
from tests import harness as hz

pytestmark = pytest.mark.gpu

N_TOK = (64, 32)   # tile-edge tokens: at most, at least
N_TOK_MX = 16      # tokens of the MXFP8 forward check


@pytest.fixture(scope="module")
def ds():
    from grouped_gemm_expert_amd import ops
    w = inputs.WORKLOADS["deepseek_v3"]
    hz.say(f"fullsize: generating {inputs.describe(w)} on the GPU")
    d = inputs.make_inputs(w, device="cuda", seed=0)
    cfg = ops.config_from_workload(w)
    saved = ops.alloc_saved(cfg)
    y = torch.empty((w.T, w.H), device="cuda")
    aux = torch.empty((1,), device="cuda")
    wsf = ops.workspace(cfg, "fwd")
    wsb = ops.workspace(cfg, "bwd")
    dx = torch.empty((w.T, w.H), device="cuda")
    dl = torch.empty((w.T, w.E), device="cuda")
    dWr = torch.empty((w.E, w.H), device="cuda")
    dW1 = torch.zeros((w.E, 2 * w.I, w.H), device="cuda")
    dW2 = torch.zeros((w.E, w.H, w.I), device="cuda")
    d_aux = torch.ones((1,), device="cuda")
    hz.say("fullsize: moe_forward + moe_backward")
    ops.moe_forward(cfg, d["x"], d["Wr"], d["bias"], d["w1"], d["w2"], y, aux, saved, wsf)
    ops.moe_backward(cfg, saved, d["x"], d["Wr"], d["w1"], d["w2"], d["dy"], d_aux, dx, dl, dWr,
                     dW1, dW2, wsb, dw_accumulate=True)
    torch.cuda.synchronize()
    hz.say("fullsize: oracle logits and routing")
    X = hz.bits(d["x"])
    Wr = d["Wr"].cpu().numpy()
    bias = d["bias"].cpu().numpy()
    l64 = oracle.logits(X, Wr)
    r = oracle.route(l64, score=hz.SCORE[w.score], k=w.k, n_groups=w.n_groups,
                     topk_groups=w.topk_groups, bias=bias, renorm=w.renorm, scale=w.scale,
                     coeff=w.aux_coeff, route_mode=w.route)
    idx_gpu = saved["topk_idx"].cpu().numpy()
    same = (idx_gpu == r["idx"]).all(1)
    rng = np.random.default_rng(1)
    toks = hz.tile_edge_tokens(r, w.k, N_TOK[0], N_TOK[1], rng, allowed=same)
    toks_mx = toks[np.unique(np.linspace(0, len(toks) - 1, N_TOK_MX).round().astype(int))]
    return dict(w=w, d=d, cfg=cfg, saved=saved, y=y, aux=aux, dx=dx, dl=dl, dW1=dW1, dW2=dW2,
                X=X, Wr=Wr, bias=bias, l64=l64, r=r, idx_gpu=idx_gpu, same=same, toks=toks,
                toks_mx=toks_mx)


def _sparse_full(d, experts):
    """Full-shape host bf16 bits of w1 / w2 holding only the listed experts."""
    w1 = np.zeros(tuple(d["w1"].shape), np.uint16)
    w2 = np.zeros(tuple(d["w2"].shape), np.uint16)
    c1, c2 = _compact(d, experts)
    w1[np.asarray(experts)] = c1
    w2[np.asarray(experts)] = c2
    return w1, w2


def _compact(d, experts):
    """Host bf16 bits of w1 / w2 for the listed experts only."""
    ex = torch.as_tensor(np.asarray(experts), device="cuda")
    return hz.bits(d["w1"].index_select(0, ex)), hz.bits(d["w2"].index_select(0, ex))


def _remap(idx, experts):
    m = np.full(int(idx.max()) + 1, -1, np.int32)
    m[np.asarray(experts)] = np.arange(len(experts), dtype=np.int32)
    return m[idx]


def test_fullsize_routing(ds):
    w, r = ds["w"], ds["r"]
    hz.say(f"fullsize routing: identical on {int(ds['same'].sum())} of {w.T} tokens")
    assert ds["same"].mean() >= 0.99
    bad = ~ds["same"]
    if bad.any():   # the rest must be a valid top-k within the projection's error bound
        eps = hz.projection_error_bound(ds["d"]["x"][torch.as_tensor(np.nonzero(bad)[0], device="cuda")].cpu().float(),
                                        torch.from_numpy(ds["Wr"]))
        ok = hz.routing_valid_under_perturbation(w, ds["l64"][bad], ds["bias"], ds["idx_gpu"][bad], eps)
        assert ok.all()
    aux_g = float(ds["aux"].cpu())
    assert abs(aux_g - r["aux"]) <= 1e-3 * abs(r["aux"]) + 1e-9, (aux_g, r["aux"])


def test_fullsize_sampled_tokens(ds):
    w, r, toks = ds["w"], ds["r"], ds["toks"]
    ex = np.unique(r["idx"][toks])
    hz.say(f"fullsize tokens {toks.tolist()}: {len(ex)} experts to the host")
    W1s, W2s = _sparse_full(ds["d"], ex)
    DY = hz.bits(ds["d"]["dy"])
    y_ref = oracle.forward(ds["X"], W1s, W2s, r["idx"], r["w"], toks=toks)
    hz.assert_close("fullsize y", ds["y"][torch.as_tensor(toks, device="cuda")].cpu().numpy(),
                    y_ref, hz.FWD_TOL)
    dx_ref, dl_ref = oracle.backward_tokens(ds["X"], ds["Wr"], ds["l64"], W1s, W2s, r["idx"],
                                            r["counts"], DY, score=hz.SCORE[w.score],
                                            renorm=w.renorm, scale=w.scale, coeff=w.aux_coeff,
                                            d_aux=1.0, toks=toks)
    tk = torch.as_tensor(toks, device="cuda")
    hz.assert_close("fullsize dx", ds["dx"][tk].cpu().numpy(), dx_ref, hz.GRAD_TOL)
    hz.assert_close("fullsize dlogits", ds["dl"][tk].cpu().numpy(), dl_ref, hz.GRAD_TOL)


def test_fullsize_weight_grad_lines(ds):
    """Whole dW lines of every active expert, reaching all its 256 x 256 output
    tiles, and exact zeros for every expert without rows."""
    w, r = ds["w"], ds["r"]
    counts = r["counts"]
    active = np.nonzero(counts)[0]
    which, ee, rr = hz.weight_grad_line_spec(active, w.I, np.random.default_rng(2))
    hz.say(f"fullsize dW: {len(which)} lines over {len(active)} active experts "
           f"({counts[active].tolist()} rows)")
    DY = hz.bits(ds["d"]["dy"])
    ref = hz.oracle_lines(ds["d"], ds["X"], DY, r, which, ee, rr)
    got = hz.gather_lines(ds["dW1"], ds["dW2"], which, ee, rr)
    for wh, name in ((1, "dW1"), (2, "dW2")):
        sel = which == wh
        hz.assert_close(f"fullsize {name} lines", got[sel], ref[sel], hz.GRAD_TOL)
    empty = np.nonzero(counts == 0)[0]
    for e in empty.tolist():
        for dW in (ds["dW1"], ds["dW2"]):
            assert float(dW[e].abs().max().cpu()) == 0.0, e
    hz.say(f"fullsize: {len(empty)} experts without rows have exact-zero dW")


@pytest.fixture(scope="module")
def dsmx(ds):
    """The MXFP8 forward and backward on the same inputs, in the benchmark's
    launch configuration (router weight, fp32 weight gradients accumulated
    into zeros)."""
    from grouped_gemm_expert_amd import ops
    w, d, cfg = ds["w"], ds["d"], ds["cfg"]
    hz.say("fullsize mx: quantising the weights (forward and transposed forms)")
    cache = ops.MxWeightCache(backward=True)
    cache.get(d["w1"], d["w2"])
    saved = ops.alloc_saved(cfg)
    y = torch.empty((w.T, w.H), device="cuda")
    aux = torch.empty((1,), device="cuda")
    hz.say("fullsize mx: moe_forward_mx + moe_backward_mx")
    ops.moe_forward_mx(cfg, d["x"], d["Wr"], d["bias"], cache.w1_mx, cache.w2_mx, y, aux, saved,
                       ops.workspace(cfg, "fwd"))
    dx = torch.empty((w.T, w.H), device="cuda")
    dl = torch.empty((w.T, w.E), device="cuda")
    dWr = torch.empty((w.E, w.H), device="cuda")
    dW1 = torch.zeros((w.E, 2 * w.I, w.H), device="cuda")
    dW2 = torch.zeros((w.E, w.H, w.I), device="cuda")
    d_aux = torch.ones((1,), device="cuda")
    ops.moe_backward_mx(cfg, saved, d["x"], d["Wr"], cache.w1t_mx, cache.w2t_mx, d["dy"], d_aux,
                        dx, dl, dWr, dW1, dW2, ops.workspace(cfg, "bwd"), dw_accumulate=True)
    torch.cuda.synchronize()
    return dict(saved=saved, y=y, dx=dx, dl=dl, dW1=dW1, dW2=dW2)


def test_fullsize_mx_forward_sampled_tokens(ds, dsmx):
    """y of tile-edge tokens against the oracle's MXFP8 forward, per element
    within the block-scaled MFMA's summation-window bound (see
    harness.assert_mx_y_within_window)."""
    w, r, toks = ds["w"], ds["r"], ds["toks_mx"]
    d = ds["d"]
    assert np.array_equal(dsmx["saved"]["topk_idx"].cpu().numpy(), ds["idx_gpu"])
    ex = np.unique(r["idx"][toks])
    W1c, W2c = _compact(d, ex)
    hz.say(f"fullsize mx: oracle on tokens {toks.tolist()}")
    y_gpu = dsmx["y"][torch.as_tensor(toks, device="cuda")].cpu().numpy()
    hz.assert_mx_y_within_window("fullsize mx y", w.I, ds["X"][toks], W1c, W2c,
                                 _remap(r["idx"][toks], ex), r["w"][toks], y_gpu)


def test_fullsize_mx_backward_sampled_tokens(ds, dsmx):
    """dx and dlogits of two tokens against the oracle's MXFP8 backward, with
    operands that hold only the experts those tokens use (the router part
    needs every logit, so the expert ids are kept)."""
    w, r = ds["w"], ds["r"]
    toks = ds["toks_mx"][::max(1, len(ds["toks_mx"]) // 4)][:4]
    ex = np.unique(r["idx"][toks])
    hz.say(f"fullsize mx backward tokens {toks.tolist()}: quantising {len(ex)} experts")
    W1c, W2c = _compact(ds["d"], ex)
    DY = hz.bits(ds["d"]["dy"])
    ops_o = oracle.MxBackwardOperands.from_experts(ds["X"], DY, w.E, ex, W1c, W2c)
    del W1c, W2c
    dx_ref, dl_ref = oracle.mx_backward_tokens(ops_o, ds["Wr"], ds["l64"], r["idx"], r["counts"],
                                               r["w"], score=hz.SCORE[w.score], renorm=w.renorm,
                                               scale=w.scale, coeff=w.aux_coeff, d_aux=1.0,
                                               toks=toks)
    tk = torch.as_tensor(toks, device="cuda")
    hz.assert_close("fullsize mx dx", dsmx["dx"][tk].cpu().numpy(), dx_ref, hz.MX_GRAD_TOL)
    hz.assert_close("fullsize mx dlogits", dsmx["dl"][tk].cpu().numpy(), dl_ref, hz.MX_GRAD_TOL)


def test_fullsize_mx_backward_weight_grad_lines(ds, dsmx):
    """Whole MX dW lines (a dW1 row in every 256-row band, a dW2 column in every
    256-column band) of the busiest, a median and the least busy active
    expert, against the oracle's MXFP8 backward."""
    w, r = ds["w"], ds["r"]
    counts = r["counts"]
    active = np.nonzero(counts)[0]
    by = active[np.argsort(-counts[active], kind="stable")]
    experts = np.unique([by[0], by[len(by) // 2], by[-1]])
    hz.say(f"fullsize mx dW lines: experts {experts.tolist()} with {counts[experts].tolist()} rows")
    W1c, W2c = _compact(ds["d"], experts)
    DY = hz.bits(ds["d"]["dy"])
    ops_o = oracle.MxBackwardOperands.from_experts(ds["X"], DY, w.E, experts, W1c, W2c)
    which, ee, rr = hz.weight_grad_line_spec(experts, w.I, np.random.default_rng(3))
    ref, mag = oracle.mx_weight_grad_lines(ops_o, ds["X"], DY, r["idx"], r["w"], which, ee, rr,
                                           with_magnitude=True)
    got = hz.gather_lines(dsmx["dW1"], dsmx["dW2"], which, ee, rr)
    for wh, name in ((1, "dW1"), (2, "dW2")):
        sel = which == wh
        hz.assert_mx_lines_within_window(f"fullsize mx {name} lines", got[sel], ref[sel],
                                         mag[sel], counts[ee[sel]])
