"""GPU parity of the router and the dispatch bookkeeping: bit-exact integer
results given the same fp32 logits, routing weights and aux within fp32
rounding, and the router projection within its fp32 error bound."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_expert_amd import inputs
from tests import harness as hz

pytestmark = pytest.mark.gpu

ROUTER_CASES = ["tiny", "mid_softmax", "mid_sigmoid", "mid_skewed", "deepseek_v3", "skewed",
                "uniform", "fine_grained", "mid_even", "even_softmax", "ep8_share"]


def _logits_for(w, seed=0):
    """fp32 logits the test hands to both sides: generated ones, or the
    oracle's projection of the generated x and router weight."""
    if w.logits is not None:
        dc = inputs.make_inputs(w, seed=seed, with_dy=False)
        return dc, dc["logits"].numpy()
    dc = inputs.make_inputs(w, seed=seed, with_dy=False)
    l64 = oracle.logits(hz.bits(dc["x"]), dc["Wr"].numpy())
    return dc, l64.astype(np.float32)


# Router shapes outside the workloads: the selection runs on 16 lanes a token
# up to E = 256, G = 16 and k = 16 and on a whole wave a token beyond; these
# cover the wide kernel and the narrow one at its limits.
WIDE_ROUTER = {
    "wide_E384": dict(base="mid_sigmoid", E=384, n_groups=24, topk_groups=6, k=18),
    "wide_k20": dict(base="mid_sigmoid", E=64, n_groups=4, topk_groups=3, k=20),
    "wide_softmax_E512": dict(base="mid_softmax", E=512, n_groups=1, topk_groups=1, k=8),
    "narrow_limits": dict(base="mid_sigmoid", E=256, n_groups=16, topk_groups=5, k=16),
}


def _router_workload(name):
    if name in WIDE_ROUTER:
        kw = dict(WIDE_ROUTER[name])
        return dataclasses.replace(inputs.WORKLOADS[kw.pop("base")], name=name, **kw)
    return inputs.WORKLOADS[name]


@pytest.mark.parametrize("name", ROUTER_CASES + sorted(WIDE_ROUTER))
def test_router_bit_exact_given_logits(name):
    from grouped_gemm_expert_amd import ops
    w = _router_workload(name)
    hz.say(f"router {inputs.describe(w)}")
    dc, l32 = _logits_for(w)
    bias = None if dc["bias"] is None else dc["bias"].numpy()
    cfg = ops.config_from_workload(w)
    dev = "cuda"
    logits = torch.from_numpy(l32).to(dev)
    bias_d = None if dc["bias"] is None else dc["bias"].to(dev)
    sel = torch.empty_like(logits)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = ops.workspace(cfg, "fwd", dev)
    ops.moe_router(cfg, None, None, bias_d, logits, sel, idx, wts, counts, aux, ws)
    torch.cuda.synchronize()

    # The integer decision is taken on the fp32 selection scores S the router
    # exports: the oracle's top-k runs on the GPU's S and must give the GPU's
    # experts bit for bit.  S itself is l (softmax: no arithmetic, so equal
    # bit for bit) or fp32(sigmoid(l)) + bias, held to 4 ulp of the oracle's.
    S_ref = oracle.selection_scores(l32, hz.SCORE[w.score], bias)
    sel_g = sel.cpu().numpy()
    if w.score == "softmax":
        assert np.array_equal(sel_g.view(np.uint32), S_ref.view(np.uint32))
    else:
        ulp = np.spacing(np.abs(S_ref).astype(np.float32)).astype(np.float64)
        err = np.abs(sel_g.astype(np.float64) - S_ref.astype(np.float64))
        hz.say(f"router S: {int((err > 0).sum())} of {err.size} scores differ, "
               f"largest {float((err / ulp).max()):.1f} ulp")
        assert (err <= 4 * ulp).all()
    if w.route == "even":
        idx_ref = oracle.even_topk(w.T, w.E, w.k)
    else:
        idx_ref = oracle.topk(sel_g, w.k, w.n_groups, w.topk_groups)
    idx_g = idx.cpu().numpy()
    assert np.array_equal(idx_g, idx_ref)
    if w.route != "even" and not np.array_equal(sel_g, S_ref):
        same = (idx_ref == oracle.topk(S_ref, w.k, w.n_groups, w.topk_groups)).all(1)
        hz.say(f"router: oracle's own S routes {int(same.sum())} of {w.T} tokens the same")
    l64 = l32.astype(np.float64)
    w_ref = oracle.weights(l64, idx_ref, hz.SCORE[w.score], w.renorm, w.scale)
    counts_ref, *_ = oracle.permute(idx_ref, w.E)
    aux_ref = oracle.aux(l64, counts_ref, w.k, hz.SCORE[w.score], w.aux_coeff)
    assert np.array_equal(counts.cpu().numpy(), counts_ref)
    wg = wts.cpu().numpy().astype(np.float64)
    assert np.abs(wg - w_ref).max() <= 4e-6 * max(1.0, w.scale)
    assert abs(float(aux.cpu()) - aux_ref) <= 1e-4 * abs(aux_ref) + 1e-9
    hz.say(f"router ok: counts min={counts_ref.min()} max={counts_ref.max()} "
           f"empty={(counts_ref == 0).sum()} aux={aux_ref:.6g}")


@pytest.mark.parametrize("name", ["mid_sigmoid", "mid_softmax", "mid_skewed", "wide_E384"])
def test_router_nan_scores_give_valid_experts(name):
    """Regression: NaN logits (from a NaN input) made the arg-max lanes
    disagree, which could leave a slot without an expert.  A NaN selection
    score now ranks as -inf on both sides: every slot gets a valid, distinct
    expert, the oracle's top-k on the exported scores gives the same experts,
    and a NaN logit exports as -inf.  Only the router runs here; its output
    is checked on the host before anything would use it."""
    from grouped_gemm_expert_amd import ops
    w = _router_workload(name)
    hz.say(f"router with NaN logits {inputs.describe(w)}")
    dc, l32 = _logits_for(w)
    l32 = l32.copy()
    rng = np.random.default_rng(3)
    l32[rng.random(l32.shape) < 0.1] = np.nan
    l32[0, :] = np.nan                 # a token with no number at all
    l32[1, : w.E - 1] = np.nan         # one finite expert
    bias = None if dc["bias"] is None else dc["bias"].numpy()
    cfg = ops.config_from_workload(w)
    dev = "cuda"
    logits = torch.from_numpy(l32).to(dev)
    bias_d = None if dc["bias"] is None else dc["bias"].to(dev)
    sel = torch.empty_like(logits)
    idx = torch.full((w.T, w.k), -7, dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    ops.moe_router(cfg, None, None, bias_d, logits, sel, idx, wts, counts, aux,
                   ops.workspace(cfg, "fwd", dev))
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy()
    assert ((idx_g >= 0) & (idx_g < w.E)).all()
    assert all(len(set(r.tolist())) == w.k for r in idx_g)
    sel_g = sel.cpu().numpy()
    S_ref = oracle.selection_scores(l32, hz.SCORE[w.score], bias)
    nan_ref = np.isnan(S_ref)
    assert np.array_equal(np.isneginf(sel_g), nan_ref | np.isneginf(S_ref))
    fin = ~nan_ref
    ulp = np.spacing(np.abs(S_ref[fin]).astype(np.float32)).astype(np.float64)
    assert (np.abs(sel_g[fin].astype(np.float64) - S_ref[fin].astype(np.float64)) <= 4 * ulp).all()
    assert np.array_equal(idx_g, oracle.topk(sel_g, w.k, w.n_groups, w.topk_groups))
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx_g.ravel(), minlength=w.E))


@pytest.mark.parametrize("name", ["tiny", "mid_softmax", "mid_sigmoid", "fine_grained"])
def test_router_projection_and_routing_with_router_weight(name):
    """The GPU computes its own fp32 logits; they must sit within the fp32
    accumulation bound of the oracle's, and every routing difference must be
    explained by a perturbation within that bound."""
    from grouped_gemm_expert_amd import ops
    w = inputs.WORKLOADS[name]
    if name == "fine_grained":
        w = dataclasses.replace(w, T=2048)
    hz.say(f"router+projection {inputs.describe(w)}")
    dc = inputs.make_inputs(w, with_dy=False)
    d = hz.to_device(dc)
    cfg = ops.config_from_workload(w)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    counts = torch.empty((w.E,), dtype=torch.int32, device="cuda")
    aux = torch.empty((1,), dtype=torch.float32, device="cuda")
    ws = ops.workspace(cfg, "fwd")
    ops.moe_router(cfg, d["x"], d["Wr"], d["bias"], logits, None, idx, wts, counts, aux, ws)
    torch.cuda.synchronize()
    l64 = oracle.logits(hz.bits(dc["x"]), dc["Wr"].numpy())
    eps = hz.projection_error_bound(dc["x"], dc["Wr"])
    lg = logits.cpu().numpy().astype(np.float64)
    assert (np.abs(lg - l64) <= eps + np.spacing(np.abs(l64).astype(np.float32))).all()
    bias = None if dc["bias"] is None else dc["bias"].numpy()
    S = oracle.selection_scores(l64.astype(np.float32), hz.SCORE[w.score], bias)
    idx_ref = oracle.topk(S, w.k, w.n_groups, w.topk_groups)
    ig = idx.cpu().numpy()
    diff = (ig != idx_ref).any(1)
    hz.say(f"tokens routed differently: {int(diff.sum())} of {w.T}")
    ok = hz.routing_valid_under_perturbation(w, l64, bias, ig, eps)
    assert ok[diff].all()
    assert diff.sum() <= max(1, w.T // 200)


PERMUTE_CASES = [
    ("uniform", 1000, 8, 2), ("uniform", 4097, 64, 6), ("uniform", 8192, 256, 8),
    ("one_expert", 3000, 16, 1), ("one_hot_expert", 2500, 32, 4), ("even", 512, 8, 2),
    ("zipf", 16384, 128, 8), ("single_token", 1, 8, 8), ("empty_most", 777, 1024, 2),
]


@pytest.mark.parametrize("pattern,T,E,k", PERMUTE_CASES)
def test_permute_bit_exact(pattern, T, E, k):
    from grouped_gemm_expert_amd import ops
    hz.say(f"permute {pattern} T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E + k)
    if pattern == "uniform":
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    elif pattern == "one_expert":
        idx = np.full((T, k), 3 % E)
    elif pattern == "one_hot_expert":
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        idx[:, 0] = 5
        idx[:, 1:] = np.where(idx[:, 1:] == 5, 6, idx[:, 1:])
    elif pattern == "even":
        idx = (np.arange(T * k) % E).reshape(T, k)
    elif pattern == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        idx = rng.choice(E, size=(T, k), p=p / p.sum())
    elif pattern == "single_token":
        idx = rng.permutation(E)[:k][None, :]
    else:
        idx = rng.choice([1, 1000], size=(T, k))
    idx = idx.astype(np.int32)
    cfg = ops.config(T=T, H=64, I=64, E=E, k=k)
    dev = "cuda"
    M = T * k
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    row_map = torch.empty((M,), dtype=torch.int32, device=dev)
    pos = torch.empty((M,), dtype=torch.int32, device=dev)
    ws = ops.workspace(cfg, "fwd", dev)
    ops.moe_permute(cfg, torch.from_numpy(idx).to(dev), counts, offsets, row_map, pos, ws)
    torch.cuda.synchronize()
    c, o, rm, ps = oracle.permute(idx, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(row_map.cpu().numpy(), rm)
    assert np.array_equal(pos.cpu().numpy(), ps)


CHECKED_CASES = [("valid", 3000, 16, 4, 0.0), ("valid_zipf", 16384, 128, 8, 0.0),
                 ("some_bad", 2500, 32, 4, 0.05), ("many_bad", 777, 1024, 2, 0.5),
                 ("all_bad", 300, 8, 2, 1.0), ("empty", 0, 8, 2, 0.0)]


@pytest.mark.parametrize("pattern,T,E,k,frac", CHECKED_CASES)
def test_permute_checked(pattern, T, E, k, frac):
    """moe_permute_checked reads every id as data: valid ids give moe_permute's
    results bit for bit; ids outside [0, E) (negative, E, far past E) are
    skipped and counted, as tests/harness.checked_permute_reference states."""
    from grouped_gemm_expert_amd import ops
    hz.say(f"permute_checked {pattern} T={T} E={E} k={k} bad fraction {frac}")
    rng = np.random.default_rng(T * 7 + E + k)
    if pattern == "valid_zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        idx = rng.choice(E, size=(T, k), p=p / p.sum())
    else:
        idx = rng.integers(0, E, (T, k))
    bad = rng.random((T, k)) < frac
    junk = rng.choice(np.array([-1, -1000, E, E + 1, 1 << 30, -(1 << 31)], np.int64), size=(T, k))
    idx = np.where(bad, junk, idx).astype(np.int32)
    cfg = ops.config(T=T, H=64, I=64, E=E, k=k)
    dev = "cuda"
    M = T * k
    out = dict(counts=torch.empty((E,), dtype=torch.int32, device=dev),
               offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
               row_map=torch.empty((max(M, 1),), dtype=torch.int32, device=dev),
               pos=torch.empty((max(M, 1),), dtype=torch.int32, device=dev))
    n_bad = torch.full((1,), -5, dtype=torch.int32, device=dev)
    ws = ops.workspace(cfg, "fwd", dev)
    idx_d = torch.from_numpy(idx).to(dev) if M else torch.empty((1, k), dtype=torch.int32,
                                                                device=dev)
    ops.moe_permute_checked(cfg, idx_d, out["counts"], out["offsets"], out["row_map"], out["pos"],
                            n_bad, ws)
    torch.cuda.synchronize()
    c, o, rm, ps, nb = hz.checked_permute_reference(idx, E)
    assert int(n_bad.cpu()) == nb
    assert np.array_equal(out["counts"].cpu().numpy(), c)
    assert np.array_equal(out["offsets"].cpu().numpy(), o)
    if M:
        assert np.array_equal(out["row_map"].cpu().numpy(), rm)
        assert np.array_equal(out["pos"].cpu().numpy(), ps)
    if nb == 0 and M:
        plain = {kk: torch.empty_like(v) for kk, v in out.items()}
        ops.moe_permute(cfg, idx_d, plain["counts"], plain["offsets"], plain["row_map"],
                        plain["pos"], ws)
        torch.cuda.synchronize()
        for kk in out:
            assert torch.equal(out[kk], plain[kk]), kk
