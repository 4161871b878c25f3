"""GPU parity of the MXFP8 backward (page "MegaMoE", "Expert precision": the
mxfp8 mode runs both expert stages, and both weight gradients, in MXFP8):

  - moe_mx_quantize_t (the transposed weights of the cache) against the
    oracle's quantiser of the transposes, bit for bit;
  - moe_backward_mx after moe_forward_mx against the oracle's MXFP8
    backward on the same bf16 inputs: dx and dlogits of every token, dW1 and
    dW2 on sampled elements (every expert, empty ones included), dWr from
    the oracle's own dlogits;
  - the two stages against the one call, accumulate mode and bf16 weight
    gradients, no tokens, and every token on one expert.

Both sides quantise the same bf16 operands the same way (dy along H, dh along
2I, and for the weight gradients the operands along their routed rows, in
32-row blocks from each expert's first row).  What separates them is the
block-scaled MFMA's accumulation window (each output within 2^-10 of the sum
of its absolute products, see the forward's tests), and the rare one-code
flips that follow when a value the kernel rounds to bf16 (h, a, dh) lies
within that error of a rounding boundary.
"""
import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_expert_amd import inputs
from tests import harness as hz
from tests.test_gpu_e2e import _wl

pytestmark = pytest.mark.gpu

N_EL = 600     # sampled elements per weight gradient


def _bf16_bits_of(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------- transposed weights ----

QT = [(4, 64, 128), (3, 96, 192), (2, 384, 320), (5, 32, 64), (1, 2048, 7168 // 8)]


@pytest.mark.parametrize("B,R,C", QT)
def test_mx_quantize_t_bit_exact(B, R, C):
    from grouped_gemm_expert_amd import ops
    hz.say(f"mx quantize_t batches={B} R={R} C={C}")
    rng = np.random.default_rng(B * 1000 + R + C)
    v = np.ldexp(rng.uniform(1, 2, (B, R, C)), rng.integers(-20, 6, (B, R, C)))
    v *= rng.choice([-1.0, 1.0], (B, R, C))
    v[rng.random((B, R, C)) < 0.05] = 0.0
    v[rng.random((B, R, C)) < 0.02] = -0.0        # negative zeros keep their sign
    v[:, :32, :C // 2] = 0.0                      # whole zero blocks
    sub = v[:, -32:, -8:]                         # blocks of bf16 subnormals
    sub[...] = np.ldexp(rng.uniform(1, 2, sub.shape), rng.integers(-133, -126, sub.shape))
    src = _bf16_bits_of(v.astype(np.float32))
    dev = torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).cuda()
    buf = ops.mx_alloc(B * C, R)
    buf.fill_(0xAB)
    ops.moe_mx_quantize_t(dev, buf)
    torch.cuda.synchronize()
    codes, scales = ops.mx_views(buf, B * C, R)
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    ref_c, ref_s = oracle.mx_quantize(np.ascontiguousarray(src.transpose(0, 2, 1)).reshape(B * C, R))
    assert np.array_equal(codes[:, :R], ref_c)
    assert np.array_equal(scales[:, :R // 32], ref_s)
    assert not codes[:, R:].any() and not scales[:, R // 32:].any()


QB = [(4, 64, 128), (3, 96, 192), (2, 384, 320), (5, 32, 64), (2, 64, 160), (1, 2048, 896)]


@pytest.mark.parametrize("B,R,C", QB)
def test_mx_quantize_both_bit_exact(B, R, C):
    """Both cache forms from one read: the row form along C equals
    moe_mx_quantize's and the oracle's, the transposed form along R equals
    moe_mx_quantize_t's (where it takes the shape) and the oracle's; ragged
    128-groups in R and C, zero blocks, negative zeros and subnormals."""
    from grouped_gemm_expert_amd import ops
    hz.say(f"mx quantize_both batches={B} R={R} C={C}")
    rng = np.random.default_rng(B * 7 + R + 3 * C)
    v = np.ldexp(rng.uniform(1, 2, (B, R, C)), rng.integers(-20, 6, (B, R, C)))
    v *= rng.choice([-1.0, 1.0], (B, R, C))
    v[rng.random((B, R, C)) < 0.05] = 0.0
    v[rng.random((B, R, C)) < 0.02] = -0.0
    v[:, :32, :32] = 0.0
    sub = v[:, -32:, -8:]
    sub[...] = np.ldexp(rng.uniform(1, 2, sub.shape), rng.integers(-133, -126, sub.shape))
    src = _bf16_bits_of(v.astype(np.float32))
    dev = torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).cuda()
    f = ops.mx_alloc(B * R, C)
    t = ops.mx_alloc(B * C, R)
    f.fill_(0xAB)
    t.fill_(0xCD)
    ops.moe_mx_quantize_both(dev, f, t)
    torch.cuda.synchronize()
    # the row form along C
    c_f, s_f = ops.mx_views(f, B * R, C)
    ref_c, ref_s = oracle.mx_quantize(src.reshape(B * R, C))
    c_f, s_f = c_f.cpu().numpy(), s_f.cpu().numpy()
    assert np.array_equal(c_f[:, :C], ref_c) and np.array_equal(s_f[:, :C // 32], ref_s)
    assert not c_f[:, C:].any() and not s_f[:, C // 32:].any()
    f2 = ops.mx_alloc(B * R, C)
    f2.fill_(0xAB)
    ops.moe_mx_quantize(dev, f2)
    # the transposed form along R
    c_t, s_t = ops.mx_views(t, B * C, R)
    ref_c, ref_s = oracle.mx_quantize(np.ascontiguousarray(src.transpose(0, 2, 1)).reshape(B * C, R))
    c_t, s_t = c_t.cpu().numpy(), s_t.cpu().numpy()
    assert np.array_equal(c_t[:, :R], ref_c) and np.array_equal(s_t[:, :R // 32], ref_s)
    assert not c_t[:, R:].any() and not s_t[:, R // 32:].any()
    torch.cuda.synchronize()
    # the whole buffers equal the separate quantisers' (scale padding included)
    assert torch.equal(f[:f2.numel()], f2)
    if C % 64 == 0:
        t2 = ops.mx_alloc(B * C, R)
        t2.fill_(0xCD)
        ops.moe_mx_quantize_t(dev, t2)
        torch.cuda.synchronize()
        assert torch.equal(t, t2)


def test_mx_weight_cache_backward_forms():
    from grouped_gemm_expert_amd import ops
    w = inputs.WORKLOADS["mid_sigmoid"]
    d = hz.to_device(inputs.make_inputs(w))
    cache = ops.MxWeightCache(backward=True)
    cache.get(d["w1"], d["w2"])
    torch.cuda.synchronize()
    E, H, I = w.E, w.H, w.I
    for buf, src, rows, K in ((cache.w1_mx, d["w1"], E * 2 * I, H), (cache.w2_mx, d["w2"], E * H, I)):
        c, s = ops.mx_views(buf, rows, K)
        ref_c, ref_s = oracle.mx_quantize(hz.bits(src).reshape(rows, K))
        assert np.array_equal(c.cpu().numpy()[:, :K], ref_c)
        assert np.array_equal(s.cpu().numpy()[:, :K // 32], ref_s)
    for buf, src, rows, K in ((cache.w2t_mx, d["w2"], E * I, H), (cache.w1t_mx, d["w1"], E * H, 2 * I)):
        c, s = ops.mx_views(buf, rows, K)
        ref_c, ref_s = oracle.mx_quantize(np.ascontiguousarray(hz.bits(src).transpose(0, 2, 1)).reshape(rows, K))
        assert np.array_equal(c.cpu().numpy()[:, :K], ref_c)
        assert np.array_equal(s.cpu().numpy()[:, :K // 32], ref_s)


# ----------------------------------------------------------------- backward ----

def _route(w, dc):
    """Oracle routing on the fp32 logits both sides route on."""
    if dc["Wr"] is not None:
        l64 = oracle.logits(hz.bits(dc["x"]), dc["Wr"].numpy())
        l32 = l64.astype(np.float32)
    else:
        l32 = dc["logits"].numpy()
        l64 = dc["logits"].double().numpy()
    bias = None if dc["bias"] is None else dc["bias"].numpy()
    r = oracle.route(l64, score=hz.SCORE[w.score], k=w.k, n_groups=w.n_groups,
                     topk_groups=w.topk_groups, bias=bias, renorm=w.renorm, scale=w.scale,
                     coeff=w.aux_coeff, logits32=l32, route_mode=w.route)
    return l32, l64, r


def _run_mx_bwd(w, d, l32, staged=False, dw_dtype=torch.float32, dw_accumulate=False,
                dW_init=None, d_aux=1.0):
    """moe_forward_mx (routing on l32), then the MX backward."""
    from grouped_gemm_expert_amd import ops
    cfg = ops.config_from_workload(w)
    saved = ops.alloc_saved(cfg)
    saved["logits"].copy_(torch.from_numpy(l32).cuda())
    y = torch.empty((w.T, w.H), device="cuda")
    aux = torch.empty((1,), device="cuda")
    wsf = ops.workspace(cfg, "fwd")
    wsb = ops.workspace(cfg, "bwd")
    cache = ops.MxWeightCache(backward=True)
    cache.get(d["w1"], d["w2"])
    ops.moe_forward_mx(cfg, d["x"], None, d["bias"], cache.w1_mx, cache.w2_mx, y, aux, saved, wsf)
    dx = torch.full((w.T, w.H), float("nan"), device="cuda")
    dl = torch.full((w.T, w.E), float("nan"), device="cuda")
    dWr = torch.full((w.E, w.H), float("nan"), device="cuda") if d["Wr"] is not None else None
    if dW_init is not None:
        dW1, dW2 = dW_init[0].clone(), dW_init[1].clone()
    else:
        dW1 = torch.full((w.E, 2 * w.I, w.H), float("nan"), dtype=dw_dtype, device="cuda")
        dW2 = torch.full((w.E, w.H, w.I), float("nan"), dtype=dw_dtype, device="cuda")
    da = torch.full((1,), d_aux, device="cuda")
    if staged:
        ops.moe_stage2_backward_mx(cfg, saved, cache.w2t_mx, d["dy"], dW2, wsb,
                                   dw_accumulate=dw_accumulate)
        ops.moe_stage1_backward_mx(cfg, saved, d["x"], d["Wr"], cache.w1t_mx, da, dx, dl, dWr,
                                   dW1, wsb, dw_accumulate=dw_accumulate)
    else:
        ops.moe_backward_mx(cfg, saved, d["x"], d["Wr"], cache.w1t_mx, cache.w2t_mx, d["dy"], da,
                            dx, dl, dWr, dW1, dW2, wsb, dw_accumulate=dw_accumulate)
    torch.cuda.synchronize()
    return dict(y=y, aux=aux, saved=saved, dx=dx, dlogits=dl, dWr=dWr, dW1=dW1, dW2=dW2)


def _sample_elements(w, rng, n=N_EL):
    which, ee, rr, cc = [], [], [], []
    for wh, nr, nc in ((1, 2 * w.I, w.H), (2, w.H, w.I)):
        which += [wh] * n
        ee += rng.integers(0, w.E, n).tolist()
        rr += rng.integers(0, nr, n).tolist()
        cc += rng.integers(0, nc, n).tolist()
    return tuple(np.array(v, np.int32) for v in (which, ee, rr, cc))


def _gather_dw(got, which, ee, rr, cc):
    out = np.empty(len(which))
    for wh, name in ((1, "dW1"), (2, "dW2")):
        sel = which == wh
        dW = got[name]
        e_, r_, c_ = ee[sel], rr[sel], cc[sel]
        # indices checked on the host: the gather below does not check them
        assert (e_ < dW.shape[0]).all() and (r_ < dW.shape[1]).all() and (c_ < dW.shape[2]).all()
        out[sel] = dW[torch.as_tensor(e_, device="cuda"), torch.as_tensor(r_, device="cuda"),
                      torch.as_tensor(c_, device="cuda")].float().cpu().numpy()
    return out


def _check_against_oracle(w, dc, got, r, l64, seed=0, d_aux=1.0):
    X, W1, W2, DY = hz.bits(dc["x"]), hz.bits(dc["w1"]), hz.bits(dc["w2"]), hz.bits(dc["dy"])
    sv = got["saved"]
    assert np.array_equal(sv["topk_idx"].cpu().numpy(), r["idx"])
    ops_o = oracle.MxBackwardOperands(X, W1, W2, DY)
    Wr = None if dc["Wr"] is None else dc["Wr"].numpy()
    dx_ref, dl_ref = oracle.mx_backward_tokens(ops_o, Wr, l64, r["idx"], r["counts"], r["w"],
                                               score=hz.SCORE[w.score], renorm=w.renorm,
                                               scale=w.scale, coeff=w.aux_coeff, d_aux=d_aux)
    hz.assert_close(f"{w.name} mx dx", got["dx"].cpu().numpy(), dx_ref, hz.MX_GRAD_TOL)
    hz.assert_close(f"{w.name} mx dlogits", got["dlogits"].cpu().numpy(), dl_ref, hz.MX_GRAD_TOL)
    if got["dWr"] is not None:
        hz.assert_close(f"{w.name} mx dWr", got["dWr"].cpu().numpy(),
                        oracle.router_weight_grad(X, dl_ref), hz.MX_GRAD_TOL)
    which, ee, rr, cc = _sample_elements(w, np.random.default_rng(seed))
    ref = oracle.mx_weight_grad_elements(ops_o, X, DY, r["idx"], r["w"], which, ee, rr, cc)
    g = _gather_dw(got, which, ee, rr, cc)
    for wh, name in ((1, "dW1"), (2, "dW2")):
        sel = which == wh
        hz.assert_close(f"{w.name} mx {name} elements", g[sel], ref[sel], hz.MX_GRAD_TOL)
    # the MX backward really quantises: it is not the bf16 backward
    dx_bf, _ = oracle.backward_tokens(X, Wr, l64, W1, W2, r["idx"], r["counts"], DY,
                                      score=hz.SCORE[w.score], renorm=w.renorm, scale=w.scale,
                                      coeff=w.aux_coeff, d_aux=d_aux)
    _, fro = hz.errors(got["dx"].cpu().numpy(), dx_bf)
    hz.say(f"{w.name} mx dx vs exact bf16 backward: rel_fro={fro:.3e}")
    assert fro > 1e-3


MX_BWD = ["tiny", "mid_softmax", "mid_sigmoid", "mid_skewed", "mid_even"]


@pytest.mark.parametrize("name", MX_BWD)
def test_mx_backward_matches_oracle(name):
    w = inputs.WORKLOADS[name]
    hz.say(f"mx backward {inputs.describe(w)}")
    dc = inputs.make_inputs(w)
    d = hz.to_device(dc)
    l32, l64, r = _route(w, dc)
    got = _run_mx_bwd(w, d, l32)
    _check_against_oracle(w, dc, got, r, l64)


def test_mx_backward_padded_hidden():
    """H = 320 and I = 192: both contraction dimensions padded to 128 in the MX
    matrices (x, dy and the transposed w2 along H; a and dh along I, 2I)."""
    w = _wl("mid_sigmoid", H=320, I=192, T=300)
    hz.say(f"mx backward padded {inputs.describe(w)}")
    dc = inputs.make_inputs(w, seed=9)
    d = hz.to_device(dc)
    l32, l64, r = _route(w, dc)
    got = _run_mx_bwd(w, d, l32)
    X, W1, W2 = hz.bits(dc["x"]), hz.bits(dc["w1"]), hz.bits(dc["w2"])
    y_ref = oracle.mx_forward(oracle.MxOperands(X, W1, W2), r["idx"], r["w"])
    hz.assert_close("padded mx y", got["y"].cpu().numpy(), y_ref, hz.FWD_TOL)  # as the MX forward tests
    _check_against_oracle(w, dc, got, r, l64, seed=2)


def test_mx_backward_two_stages_equal_one_call():
    w = inputs.WORKLOADS["mid_sigmoid"]
    hz.say(f"mx backward stages {inputs.describe(w)}")
    dc = inputs.make_inputs(w, seed=5)
    d = hz.to_device(dc)
    l32, _, _ = _route(w, dc)
    a = _run_mx_bwd(w, d, l32)
    b = _run_mx_bwd(w, d, l32, staged=True)
    for k in ("dx", "dlogits", "dWr", "dW1", "dW2"):
        assert torch.equal(a[k], b[k]), k


def test_mx_backward_accumulate_and_bf16_weight_grads():
    w = inputs.WORKLOADS["mid_skewed"]
    hz.say(f"mx dW modes {inputs.describe(w)}")
    dc = inputs.make_inputs(w, seed=3)
    d = hz.to_device(dc)
    l32, _, _ = _route(w, dc)
    base = _run_mx_bwd(w, d, l32)
    g = torch.Generator(device="cpu").manual_seed(11)
    init1 = torch.randn((w.E, 2 * w.I, w.H), generator=g).cuda()
    init2 = torch.randn((w.E, w.H, w.I), generator=g).cuda()
    acc = _run_mx_bwd(w, d, l32, dw_accumulate=True, dW_init=(init1, init2))
    counts = base["saved"]["counts"].cpu().numpy()
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) > 0
    assert not base["dW1"][empty].any() and not base["dW2"][empty].any()
    assert torch.equal(acc["dW1"][empty], init1[empty])
    assert torch.equal(acc["dW2"][empty], init2[empty])
    hz.assert_close("mx dW1 accumulate", (acc["dW1"] - init1).cpu().numpy(),
                    base["dW1"].cpu().numpy(), (1e-5, 1e-5))
    hz.assert_close("mx dW2 accumulate", (acc["dW2"] - init2).cpu().numpy(),
                    base["dW2"].cpu().numpy(), (1e-5, 1e-5))
    b16 = _run_mx_bwd(w, d, l32, dw_dtype=torch.bfloat16)
    for k in ("dW1", "dW2"):
        ref = base[k].cpu().numpy()
        got = b16[k].float().cpu().numpy()
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-12), k


def test_mx_backward_hot_expert():
    """Every token's first choice on expert 3: most experts empty (exact zero
    weight gradients), one expert with every token (many 128-row chunks)."""
    w = _wl("mid_skewed", E=16, k=2, n_groups=1, topk_groups=1, T=400)
    hz.say(f"mx backward hot expert {inputs.describe(w)}")
    dc = inputs.make_inputs(w, seed=2)
    lg = torch.full((w.T, w.E), -20.0)
    lg[:, 3] = 5.0
    lg[:, 7] = 1.0 + 0.01 * torch.arange(w.T) / w.T
    dc["logits"] = lg
    d = hz.to_device(dc)
    l32, l64, r = _route(w, dc)
    got = _run_mx_bwd(w, d, l32)
    empty = np.nonzero(r["counts"] == 0)[0]
    assert len(empty) == w.E - 2
    assert not got["dW1"][empty].any() and not got["dW2"][empty].any()
    _check_against_oracle(w, dc, got, r, l64, seed=1)


def test_mx_backward_zero_tokens():
    from grouped_gemm_expert_amd import ops
    w = _wl("mid_softmax", T=0)
    hz.say("mx backward T=0")
    cfg = ops.config_from_workload(w)
    saved = ops.alloc_saved(cfg)
    w1 = torch.zeros((w.E, 2 * w.I, w.H), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((w.E, w.H, w.I), dtype=torch.bfloat16, device="cuda")
    cache = ops.MxWeightCache(backward=True)
    cache.get(w1, w2)
    x = torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda")
    Wr = torch.zeros((w.E, w.H), device="cuda")
    dx = torch.empty((0, w.H), device="cuda")
    dl = torch.empty((0, w.E), device="cuda")
    dWr = torch.full((w.E, w.H), 5.0, device="cuda")
    dW1 = torch.full((w.E, 2 * w.I, w.H), 5.0, device="cuda")
    dW2 = torch.full((w.E, w.H, w.I), 5.0, device="cuda")
    da = torch.ones((1,), device="cuda")
    aux = torch.empty((1,), device="cuda")
    ops.moe_forward_mx(cfg, x, Wr, None, cache.w1_mx, cache.w2_mx, torch.empty((0, w.H), device="cuda"),
                       aux, saved, ops.workspace(cfg, "fwd"))
    ws = ops.workspace(cfg, "bwd")
    ops.moe_backward_mx(cfg, saved, x, Wr, cache.w1t_mx, cache.w2t_mx, dy, da, dx, dl, dWr, dW1,
                        dW2, ws)
    torch.cuda.synchronize()
    assert not dW1.any() and not dW2.any() and not dWr.any()


def test_mx_graph_capture_replays_to_eager():
    """The MXFP8 forward + backward captured into one HIP graph (stages, on
    the cached MX weights) replays to the eager one-call results, replay
    after replay, with eager work in between.  (Unlike the pages' fp8 op,
    which holds a cross-rank handshake, nothing here keeps the path out of a
    graph.)"""
    from grouped_gemm_expert_amd import ops
    w = inputs.WORKLOADS["mid_sigmoid"]
    hz.say(f"mx graph {inputs.describe(w)}")
    d = hz.to_device(inputs.make_inputs(w, seed=7))
    cfg = ops.config_from_workload(w)
    cache = ops.MxWeightCache(backward=True)
    cache.get(d["w1"], d["w2"])
    outs = ["y", "aux", "dx", "dl", "dWr", "dW1", "dW2"]

    def alloc():
        return dict(saved=ops.alloc_saved(cfg), y=torch.empty((w.T, w.H), device="cuda"),
                    aux=torch.empty((1,), device="cuda"), dx=torch.empty((w.T, w.H), device="cuda"),
                    dl=torch.empty((w.T, w.E), device="cuda"), dWr=torch.empty((w.E, w.H), device="cuda"),
                    dW1=torch.empty((w.E, 2 * w.I, w.H), device="cuda"),
                    dW2=torch.empty((w.E, w.H, w.I), device="cuda"), da=torch.ones((1,), device="cuda"),
                    wsf=ops.workspace(cfg, "fwd"), wsb=ops.workspace(cfg, "bwd"))

    def one_call(t):
        ops.moe_forward_mx(cfg, d["x"], d["Wr"], d["bias"], cache.w1_mx, cache.w2_mx, t["y"], t["aux"],
                           t["saved"], t["wsf"])
        ops.moe_backward_mx(cfg, t["saved"], d["x"], d["Wr"], cache.w1t_mx, cache.w2t_mx, d["dy"],
                            t["da"], t["dx"], t["dl"], t["dWr"], t["dW1"], t["dW2"], t["wsb"])

    def staged(t):
        ops.moe_stage1_forward_mx(cfg, d["x"], d["Wr"], d["bias"], cache.w1_mx, t["aux"], t["saved"],
                                  t["wsf"])
        ops.moe_stage2_forward_mx(cfg, cache.w2_mx, t["saved"], t["y"], t["wsf"])
        ops.moe_stage2_backward_mx(cfg, t["saved"], cache.w2t_mx, d["dy"], t["dW2"], t["wsb"])
        ops.moe_stage1_backward_mx(cfg, t["saved"], d["x"], d["Wr"], cache.w1t_mx, t["da"], t["dx"],
                                   t["dl"], t["dWr"], t["dW1"], t["wsb"])

    ref = alloc()
    one_call(ref)
    torch.cuda.synchronize()
    t = alloc()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the default stream before capture
        staged(t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        staged(t)
    torch.cuda.synchronize()
    other = alloc()
    for rep in range(3):
        for k in outs:                       # poison every output before the replay
            t[k].fill_(float("nan"))
        g.replay()
        one_call(other)                      # eager work of the program between replays
        torch.cuda.synchronize()
        hz.say(f"mx graph replay {rep}")
        for k in outs:
            assert torch.equal(t[k], ref[k]), f"replay {rep} {k}"
            assert torch.equal(other[k], ref[k]), f"eager {rep} {k}"
