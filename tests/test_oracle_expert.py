"""Pins for the oracle's expert half (GEMM1 -> SwiGLU -> GEMM2 -> combine) and
its hand-derived backward.  CPU only."""
import dataclasses

import numpy as np
import pytest
import torch

from grouped_gemm_expert_amd import inputs
from tests.dense_reference import dense_loss

SCORE = {"softmax": 0, "sigmoid": 1}


def _bits(t):
    return inputs.bf16_bits(t)


def _small(score, renorm, G=1, kg=1, E=8, k=3, T=40, H=32, I=24, bias=None, logits=None, seed=0):
    w = inputs.Workload("t", T=T, H=H, I=I, E=E, k=k, n_groups=G, topk_groups=kg, score=score,
                        renorm=renorm, scale=2.5 if score == "sigmoid" else 1.0,
                        x_std=1.0, w_std=0.2, wr_std=0.3, bias_std=bias, logits=logits)
    return inputs.make_inputs(w, seed=seed), w


def _route(oracle_lib, d, w):
    x = _bits(d["x"])
    if d["Wr"] is not None:
        l64 = oracle_lib.logits(x, d["Wr"].numpy())
    else:
        l64 = d["logits"].double().numpy()
    bias = None if d["bias"] is None else d["bias"].numpy()
    r = oracle_lib.route(l64, score=SCORE[w.score], k=w.k, n_groups=w.n_groups,
                         topk_groups=w.topk_groups, bias=bias, renorm=w.renorm,
                         scale=w.scale, coeff=w.aux_coeff)
    return l64, r


# -------------------------------------------------------------- forward ----

@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_forward_single_expert_is_dense_swiglu_mlp(oracle_lib, score):
    d, w = _small(score, False, E=1, k=1, T=17, H=48, I=40)
    l64, r = _route(oracle_lib, d, w)
    assert (r["idx"] == 0).all()
    assert abs(r["aux"] - w.aux_coeff) < 1e-15
    y = oracle_lib.forward(_bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), r["idx"], r["w"])
    x = d["x"].double().numpy()
    w1 = d["w1"][0].double().numpy()
    w2 = d["w2"][0].double().numpy()
    gate, up = x @ w1[:40].T, x @ w1[40:].T          # gate rows first, then up rows
    ref = (gate * scipy_expit(gate) * up) @ w2.T
    if score == "sigmoid":
        ref = ref * w.scale
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def scipy_expit(z):
    import scipy.special
    return scipy.special.expit(z)


def test_forward_token_permutation(oracle_lib):
    d, w = _small("sigmoid", False, G=4, kg=2, bias=0.1)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2 = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"])
    y = oracle_lib.forward(X, W1, W2, r["idx"], r["w"])
    perm = np.random.default_rng(0).permutation(w.T)
    r2 = oracle_lib.route(l64[perm], score=1, k=w.k, n_groups=4, topk_groups=2,
                          bias=d["bias"].numpy(), scale=w.scale, coeff=w.aux_coeff)
    y2 = oracle_lib.forward(X[perm], W1, W2, r2["idx"], r2["w"])
    assert np.array_equal(r2["idx"], r["idx"][perm])
    assert np.array_equal(y2, y[perm])
    assert np.array_equal(r2["counts"], r["counts"])


def test_forward_linear_in_w2_and_token_subset(oracle_lib):
    d, w = _small("softmax", True)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2 = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"])
    y = oracle_lib.forward(X, W1, W2, r["idx"], r["w"])
    W2x2 = _bits((d["w2"].float() * 2).to(torch.bfloat16))
    assert np.array_equal(oracle_lib.forward(X, W1, W2x2, r["idx"], r["w"]), 2 * y)
    toks = np.array([5, 0, 39, 5])
    assert np.array_equal(oracle_lib.forward(X, W1, W2, r["idx"], r["w"], toks=toks), y[toks])


def test_forward_matches_dense_formulation(oracle_lib):
    d, w = _small("softmax", True, E=8, k=3)
    l64, r = _route(oracle_lib, d, w)
    y = oracle_lib.forward(_bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), r["idx"], r["w"])
    _, yd, auxd, _ = dense_loss(d["x"].double(), d["w1"].double(), d["w2"].double(),
                                torch.from_numpy(r["idx"]).long(), d["dy"].double(),
                                score="softmax", renorm=True, scale=1.0, coeff=w.aux_coeff,
                                d_aux=1.0, counts=torch.from_numpy(r["counts"]),
                                Wr=d["Wr"].double())
    assert np.allclose(y, yd.numpy(), rtol=1e-12, atol=1e-13)
    assert abs(float(auxd) - r["aux"]) < 1e-14


def test_forward_empty_batch(oracle_lib):
    X = np.zeros((0, 8), np.uint16)
    W1 = np.zeros((2, 8, 8), np.uint16)
    W2 = np.zeros((2, 8, 4), np.uint16)
    y = oracle_lib.forward(X, W1, W2, np.zeros((0, 1), np.int32), np.zeros((0, 1)))
    assert y.shape == (0, 8)


# ------------------------------------------------------------- backward ----

CASES = [
    dict(score="softmax", renorm=True),
    dict(score="softmax", renorm=False),
    dict(score="sigmoid", renorm=False, G=4, kg=2, bias=0.1),
    dict(score="sigmoid", renorm=False),
    dict(score="sigmoid", renorm=False, G=4, kg=2, logits="zipf"),
    dict(score="softmax", renorm=True, logits="normal", k=8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_backward_matches_autograd_of_dense_formulation(oracle_lib, case):
    d, w = _small(**case)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2, DY = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), _bits(d["dy"])
    Wr = None if d["Wr"] is None else d["Wr"].numpy()
    d_aux = 3.0
    dx, dl = oracle_lib.backward_tokens(X, Wr, l64, W1, W2, r["idx"], r["counts"], DY,
                                        score=SCORE[w.score], renorm=w.renorm, scale=w.scale,
                                        coeff=w.aux_coeff, d_aux=d_aux)
    dW1, dW2 = oracle_lib.weight_grads(X, W1, W2, r["idx"], r["w"], DY)

    x = d["x"].double().requires_grad_()
    w1 = d["w1"].double().requires_grad_()
    w2 = d["w2"].double().requires_grad_()
    kw = dict(score=w.score, renorm=w.renorm, scale=w.scale, coeff=w.aux_coeff, d_aux=d_aux,
              counts=torch.from_numpy(r["counts"]))
    if d["Wr"] is not None:
        Wr_t = d["Wr"].double().requires_grad_()
        loss, _, _, logits = dense_loss(x, w1, w2, torch.from_numpy(r["idx"]).long(),
                                        d["dy"].double(), Wr=Wr_t, **kw)
        logits.retain_grad()
        loss.backward()
        dWr = oracle_lib.router_weight_grad(X, dl)
        assert np.allclose(dWr, Wr_t.grad.numpy(), rtol=1e-9, atol=1e-12)
        gl = logits.grad.numpy()
    else:
        lt = torch.from_numpy(l64).clone().requires_grad_()
        loss, _, _, _ = dense_loss(x, w1, w2, torch.from_numpy(r["idx"]).long(),
                                   d["dy"].double(), logits=lt, **kw)
        loss.backward()
        gl = lt.grad.numpy()
    scale = lambda a: max(1e-30, float(np.abs(a).max()))
    assert np.abs(dl - gl).max() <= 1e-10 * scale(gl)
    assert np.abs(dx - x.grad.numpy()).max() <= 1e-10 * scale(x.grad.numpy())
    assert np.abs(dW1 - w1.grad.numpy()).max() <= 1e-10 * scale(w1.grad.numpy())
    assert np.abs(dW2 - w2.grad.numpy()).max() <= 1e-10 * scale(w2.grad.numpy())


@pytest.mark.parametrize("case", CASES[:4], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_router_backward_central_differences(oracle_lib, case):
    """d loss / d logits by central differences of the oracle's own forward
    (weights + expert forward + aux), routing and counts held fixed."""
    d, w = _small(**case, T=12)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2, DY = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), _bits(d["dy"])
    dyd = d["dy"].double().numpy()
    d_aux = 2.0
    score = SCORE[w.score]

    def loss(l):
        wts = oracle_lib.weights(l, r["idx"], score, w.renorm, w.scale)
        y = oracle_lib.forward(X, W1, W2, r["idx"], wts)
        return float((y * dyd).sum()) + d_aux * oracle_lib.aux(l, r["counts"], w.k, score, w.aux_coeff)

    _, dl = oracle_lib.backward_tokens(X, None, l64, W1, W2, r["idx"], r["counts"], DY,
                                       score=score, renorm=w.renorm, scale=w.scale,
                                       coeff=w.aux_coeff, d_aux=d_aux)
    eps = 1e-5
    rng = np.random.default_rng(1)
    for _ in range(25):
        t, e = rng.integers(w.T), rng.integers(w.E)
        lp, lm = l64.copy(), l64.copy()
        lp[t, e] += eps
        lm[t, e] -= eps
        fd = (loss(lp) - loss(lm)) / (2 * eps)
        assert abs(fd - dl[t, e]) <= 1e-6 * max(1.0, abs(dl[t, e])), (t, e, fd, dl[t, e])


def test_weight_grad_elements_agree_with_full(oracle_lib):
    d, w = _small("sigmoid", False, G=4, kg=2, bias=0.1)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2, DY = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), _bits(d["dy"])
    dW1, dW2 = oracle_lib.weight_grads(X, W1, W2, r["idx"], r["w"], DY)
    rng = np.random.default_rng(2)
    n = 40
    which = rng.integers(1, 3, n)
    ee = rng.integers(0, w.E, n)
    rr = np.where(which == 1, rng.integers(0, 2 * w.I, n), rng.integers(0, w.H, n))
    cc = np.where(which == 1, rng.integers(0, w.H, n), rng.integers(0, w.I, n))
    got = oracle_lib.weight_grad_elements(X, W1, W2, r["idx"], r["w"], DY, which, ee, rr, cc)
    ref = np.where(which == 1, dW1[ee, rr % (2 * w.I), cc % w.H], dW2[ee, rr % w.H, cc % w.I])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)
    # an expert subset and a token subset give the same partial sums
    sub1, sub2 = oracle_lib.weight_grads(X, W1, W2, r["idx"], r["w"], DY, experts=[3, 0])
    assert np.array_equal(sub1[0], dW1[3]) and np.array_equal(sub2[1], dW2[0])


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_weight_grad_lines_match_autograd_of_dense_formulation(oracle_lib, case):
    """Rows of dW1 and columns of dW2 (whole lines, the form the full-size
    parity tests use) against torch.autograd of the dense formulation."""
    d, w = _small(**case)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2, DY = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), _bits(d["dy"])
    x = d["x"].double()
    w1 = d["w1"].double().requires_grad_()
    w2 = d["w2"].double().requires_grad_()
    kw = dict(score=w.score, renorm=w.renorm, scale=w.scale, coeff=0.0, d_aux=0.0,
              counts=torch.from_numpy(r["counts"]))
    # routing weights are inputs of the lines: take the oracle's, as the
    # dense formulation derives the same ones from the same logits
    loss, _, _, _ = dense_loss(x, w1, w2, torch.from_numpy(r["idx"]).long(), d["dy"].double(),
                               logits=torch.from_numpy(l64), **kw)
    loss.backward()
    g1, g2 = w1.grad.numpy(), w2.grad.numpy()
    ee = np.repeat(np.arange(w.E), 4)
    rows = np.tile([0, w.I - 1, w.I, 2 * w.I - 1], w.E)        # gate and up halves, both ends
    cols = np.tile([0, 5, w.I // 2, w.I - 1], w.E)
    lines1 = oracle_lib.weight_grad_lines(X, W1, W2, r["idx"], r["w"], DY, np.ones_like(ee), ee,
                                          rows)
    lines2 = oracle_lib.weight_grad_lines(X, W1, W2, r["idx"], r["w"], DY, np.full_like(ee, 2),
                                          ee, cols)
    tol = lambda a: 1e-10 * max(1e-30, float(np.abs(a).max()))
    assert np.abs(lines1 - g1[ee, rows, :]).max() <= tol(g1)
    assert np.abs(lines2 - g2[ee, :, cols]).max() <= tol(g2)
    assert np.abs(lines1).max() > 0 and np.abs(lines2).max() > 0


def test_weight_grads_linear_in_dy_and_token_permutation(oracle_lib):
    d, w = _small("softmax", True)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2, DY = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), _bits(d["dy"])
    dW1, dW2 = oracle_lib.weight_grads(X, W1, W2, r["idx"], r["w"], DY)
    DY2 = _bits((d["dy"].float() * 2).to(torch.bfloat16))
    a1, a2 = oracle_lib.weight_grads(X, W1, W2, r["idx"], r["w"], DY2)
    assert np.array_equal(a1, 2 * dW1) and np.array_equal(a2, 2 * dW2)
    perm = np.random.default_rng(3).permutation(w.T)
    p1, p2 = oracle_lib.weight_grads(X[perm], W1, W2, r["idx"][perm], r["w"][perm], DY[perm])
    assert np.allclose(p1, dW1, rtol=1e-12, atol=1e-15)
    assert np.allclose(p2, dW2, rtol=1e-12, atol=1e-15)


def test_empty_expert_gets_zero_weight_grad(oracle_lib):
    d, w = _small("softmax", True, E=8, k=2)
    X, W1, W2, DY = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"]), _bits(d["dy"])
    idx = np.tile(np.array([[1, 4]], np.int32), (w.T, 1))
    wt = np.full((w.T, 2), 0.5)
    dW1, dW2 = oracle_lib.weight_grads(X, W1, W2, idx, wt, DY)
    for e in (0, 2, 3, 5, 6, 7):
        assert not dW1[e].any() and not dW2[e].any()
    assert dW1[1].any() and dW2[4].any()


def test_expert_rows_recombine_to_forward(oracle_lib):
    d, w = _small("softmax", True)
    l64, r = _route(oracle_lib, d, w)
    X, W1, W2 = _bits(d["x"]), _bits(d["w1"]), _bits(d["w2"])
    y = oracle_lib.forward(X, W1, W2, r["idx"], r["w"])
    slots = np.arange(w.T * w.k)
    g, u, a, o = oracle_lib.expert_rows(X, W1, W2, r["idx"], slots)
    yy = (o.reshape(w.T, w.k, w.H) * r["w"][:, :, None]).sum(1)
    assert np.allclose(yy, y, rtol=1e-13, atol=1e-15)
    # gate / up halves: single expert reduces to the dense products
    x = d["x"].double().numpy()
    for f in (0, 7, 100):
        t, e = f // w.k, r["idx"].ravel()[f]
        w1e = d["w1"][e].double().numpy()
        assert np.allclose(g[f], x[t] @ w1e[:w.I].T, rtol=1e-13, atol=1e-15)
        assert np.allclose(u[f], x[t] @ w1e[w.I:].T, rtol=1e-13, atol=1e-15)
