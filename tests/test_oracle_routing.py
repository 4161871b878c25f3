"""Pins for the oracle's router half: selection scores, group-limited top-k,
weights, dispatch bookkeeping and the aux loss.  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- top-k ----

def _brute_topk(s, k, G, kg):
    """Top-k by enumerating every subset: the chosen set is the subset whose
    sorted (value desc, index asc) key list is lexicographically smallest."""
    E = len(s)
    s = [np.float32(v) for v in s]
    if G > 1:
        gsz = E // G
        gs = []
        for g in range(G):
            vals = sorted((s[e] for e in range(g * gsz, (g + 1) * gsz)), reverse=True)
            gs.append(np.float32(vals[0] + vals[1]) if gsz > 1 else vals[0])
        best = None
        for comb in itertools.combinations(range(G), kg):
            key = sorted((-float(gs[g]), g) for g in comb)
            if best is None or key < best[0]:
                best = (key, comb)
        eligible = [e for g in best[1] for e in range(g * gsz, (g + 1) * gsz)]
    else:
        eligible = list(range(E))
    best = None
    for comb in itertools.combinations(eligible, k):
        key = sorted((-float(s[e]), e) for e in comb)
        if best is None or key < best[0]:
            best = (key, comb)
    return [e for _, e in best[0]]


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_subset_enumeration(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    cases = [(8, 2, 1, 1), (8, 3, 4, 2), (12, 4, 3, 2), (12, 3, 6, 3), (10, 4, 5, 2),
             (9, 2, 3, 1), (6, 6, 1, 1), (8, 1, 2, 1)]
    for E, k, G, kg in cases:
        T = 20
        if seed % 3 == 0:      # heavy ties: few distinct values
            S = rng.integers(-2, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)
        elif seed % 3 == 1:
            S = rng.standard_normal((T, E)).astype(np.float32)
        else:                   # ties only inside some groups
            S = np.repeat(rng.standard_normal((T, E // 2)), 2, axis=1)[:, :E].astype(np.float32)
        got = oracle_lib.topk(S, k, G, kg)
        for t in range(T):
            assert list(got[t]) == _brute_topk(S[t], k, G, kg), (E, k, G, kg, S[t])


def test_topk_all_equal_scores_closed_form(oracle_lib):
    # all scores equal: ties everywhere go to the lower index
    for E, k, G, kg in [(8, 2, 1, 1), (256, 8, 8, 4), (64, 4, 8, 4), (16, 5, 4, 2)]:
        S = np.zeros((5, E), np.float32)
        idx = oracle_lib.topk(S, k, G, kg)
        assert (idx == np.arange(k, dtype=np.int32)[None, :]).all()


def test_topk_signed_zero_is_a_tie(oracle_lib):
    S = np.array([[-0.0, 0.0, -1.0, -0.0]], np.float32)
    assert list(oracle_lib.topk(S, 3)[0]) == [0, 1, 3]
    S = np.array([[0.0, -0.0, -1.0, 0.0]], np.float32)
    assert list(oracle_lib.topk(S, 2)[0]) == [0, 1]


def test_topk_nan_scores_rank_below_every_number(oracle_lib):
    """Reading: a NaN selection score ranks as -inf (below every number; equal
    keys by lower index), so the order stays total and k valid experts come
    out.  Hand example, then subset enumeration with NaN taken as -inf, a
    whole NaN group, and an all-NaN row."""
    import oracle
    nan = np.float32("nan")
    S = np.array([[nan, 0.5, nan, 0.2]], np.float32)
    assert oracle.topk(S, 3, 1, 1).tolist() == [[1, 3, 0]]
    assert oracle.topk(np.full((1, 4), nan, np.float32), 2, 1, 1).tolist() == [[0, 1]]
    # group 1 (experts 2, 3) all NaN: its score is -inf and it is not kept
    S = np.array([[0.1, 0.2, nan, nan, 0.3, 0.05, 0.4, 0.0]], np.float32)
    assert oracle.topk(S, 3, 4, 2).tolist() == [[6, 4, 5]]   # kept: groups 3 and 2
    rng = np.random.default_rng(7)
    for _ in range(40):
        E, G = 8, int(rng.choice([1, 2, 4]))
        kg = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, kg * (E // G) + 1))
        S = rng.standard_normal((1, E)).astype(np.float32)
        S[rng.random((1, E)) < 0.3] = nan
        keyed = np.where(np.isnan(S), -np.inf, S).astype(np.float32)
        assert oracle.topk(S, k, G, kg)[0].tolist() == _brute_topk(keyed[0], k, G, kg)


def test_topk_group_limit_excludes_higher_experts(oracle_lib):
    # group 1 holds the single best expert but a weak second; groups 0 and 2 win
    E, G, kg, k = 6, 3, 2, 2
    S = np.array([[0.5, 0.5, 0.9, -5.0, 0.4, 0.4]], np.float32)
    # group scores: g0 = 1.0, g1 = -4.1, g2 = 0.8 -> keep g0, g2
    assert list(oracle_lib.topk(S, k, G, kg)[0]) == [0, 1]


# ----------------------------------------------------- selection scores ----

def test_selection_scores_softmax_is_logits(oracle_lib):
    l = np.random.default_rng(1).standard_normal((7, 9)).astype(np.float32)
    S = oracle_lib.selection_scores(l, oracle_lib.SOFTMAX)
    assert np.array_equal(S.view(np.uint32), l.view(np.uint32))


def test_selection_scores_sigmoid_special_values(oracle_lib):
    l = np.array([[0.0, 40.0, -200.0, 2.0, -2.0]], np.float32)
    b = np.array([0.25, -0.5, 0.0, 0.0, 0.0], np.float32)
    S = oracle_lib.selection_scores(l, oracle_lib.SIGMOID, b)
    assert S[0, 0] == np.float32(0.75)          # sigmoid(0) = 1/2 exactly
    assert S[0, 1] == np.float32(0.5)           # sigmoid(40) rounds to 1 in fp32
    assert S[0, 2] == np.float32(0.0) or S[0, 2] < np.float32(1e-80)
    # sigmoid(2) + sigmoid(-2) = 1 (to fp32 rounding)
    assert abs(float(S[0, 3]) + float(S[0, 4]) - 1.0) < 1e-7
    # strictly increasing in the logit
    ll = np.linspace(-8, 8, 1001, dtype=np.float32)[None, :]
    s = oracle_lib.selection_scores(ll, oracle_lib.SIGMOID)[0]
    assert (np.diff(s) >= 0).all() and s[-1] > s[0]


# --------------------------------------------------------------- weights ----

def test_weights_renorm_sum_to_one_and_sigmoid_to_scale(oracle_lib):
    rng = np.random.default_rng(2)
    l = rng.standard_normal((50, 16))
    idx = oracle_lib.topk(l.astype(np.float32), 4)
    w = oracle_lib.weights(l, idx, oracle_lib.SOFTMAX, True, 1.0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=4e-16)
    w = oracle_lib.weights(l, idx, oracle_lib.SIGMOID, False, 2.5)
    assert np.allclose(w.sum(1), 2.5, rtol=0, atol=1e-15)
    # no renorm: the weights are the softmax probabilities themselves
    w = oracle_lib.weights(l, idx, oracle_lib.SOFTMAX, False, 1.0)
    p = scipy.special.softmax(l, axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=1e-14, atol=0)
    # sigmoid: proportional to sigmoid(l) of the selected experts
    w = oracle_lib.weights(l, idx, oracle_lib.SIGMOID, False, 1.0)
    s = np.take_along_axis(scipy.special.expit(l), idx.astype(np.int64), 1)
    assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=1e-14, atol=0)


def test_weights_single_expert(oracle_lib):
    l = np.random.default_rng(3).standard_normal((9, 1))
    idx = np.zeros((9, 1), np.int32)
    assert np.array_equal(oracle_lib.weights(l, idx, oracle_lib.SOFTMAX, False, 1.0), np.ones((9, 1)))
    assert np.allclose(oracle_lib.weights(l, idx, oracle_lib.SIGMOID, False, 2.5), 2.5, rtol=0, atol=1e-15)


# --------------------------------------------------------------- permute ----

def _read_even_cases():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "even_routing.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in vals}
            cases.append(cur)
        else:
            cur[key] = np.array([int(v) for v in vals], np.int32)
    return cases


def test_permute_even_routing_golden(oracle_lib):
    for c in _read_even_cases():
        T, k, E = c["T"], c["k"], c["E"]
        f = np.arange(T * k)
        idx = (f % E).astype(np.int32).reshape(T, k)   # the `even` formula
        assert np.array_equal(idx.ravel(), c["idx"])
        counts, offsets, row_map, pos = oracle_lib.permute(idx, E)
        assert np.array_equal(counts, c["counts"])
        assert np.array_equal(offsets, c["offsets"])
        assert np.array_equal(row_map, c["row_map"])
        assert np.array_equal(pos, c["pos"])


@pytest.mark.parametrize("T,k,E", [(256, 2, 8), (8192, 8, 256), (1000, 4, 16)])
def test_permute_even_routing_closed_form(oracle_lib, T, k, E):
    assert (T * k) % E == 0
    idx = (np.arange(T * k) % E).astype(np.int32).reshape(T, k)
    counts, offsets, row_map, pos = oracle_lib.permute(idx, E)
    n = T * k // E
    assert (counts == n).all()
    assert np.array_equal(offsets, np.arange(E + 1) * n)
    for e in range(E):
        assert np.array_equal(row_map[offsets[e]:offsets[e + 1]], e + np.arange(n) * E)


def test_even_route_golden(oracle_lib):
    """The oracle's `even` forced routing against the hand-worked cases."""
    for c in _read_even_cases():
        T, k, E = c["T"], c["k"], c["E"]
        l64 = np.random.default_rng(T * 100 + E).normal(size=(T, E))
        r = oracle_lib.route(l64, score=oracle_lib.SOFTMAX, k=k, renorm=True, coeff=0.01,
                             route_mode="even")
        assert np.array_equal(r["idx"].ravel(), c["idx"])
        assert np.array_equal(r["counts"], c["counts"])
        assert np.array_equal(r["offsets"], c["offsets"])
        assert np.array_equal(r["row_map"], c["row_map"])
        assert np.array_equal(r["pos"], c["pos"])


@pytest.mark.parametrize("score,renorm", [(0, False), (0, True), (1, True)])
def test_even_route_weights(oracle_lib, score, renorm):
    """Forced indices, learned weight rule: softmax p at the forced experts
    (renormalised or not), or scale * s / sum(s) for the sigmoid router;
    groups play no part."""
    T, E, k = 37, 16, 4
    rng = np.random.default_rng(11)
    l64 = rng.normal(size=(T, E))
    r = oracle_lib.route(l64, score=score, k=k, n_groups=4, topk_groups=1, renorm=renorm,
                         scale=2.5, coeff=0.01, route_mode="even")
    idx = r["idx"]
    # the forced experts, whatever the scores of their groups
    assert idx[1].tolist() == [4, 5, 6, 7] and idx[4].tolist() == [0, 1, 2, 3]
    if score == oracle_lib.SOFTMAX:
        p = np.exp(l64 - l64.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ref = np.take_along_axis(p, idx, 1)
        if renorm:
            ref = ref / ref.sum(1, keepdims=True)
    else:
        s = 1.0 / (1.0 + np.exp(-l64))
        ref = np.take_along_axis(s, idx, 1)
        ref = 2.5 * ref / ref.sum(1, keepdims=True)
    assert np.allclose(r["w"], ref, rtol=1e-12, atol=1e-15)


def test_even_route_counts_equal(oracle_lib):
    T, E, k = 96, 24, 8
    r = oracle_lib.route(np.zeros((T, E)), score=oracle_lib.SOFTMAX, k=k, route_mode="even")
    assert (r["counts"] == T * k // E).all()


def test_permute_matches_stable_argsort(oracle_lib):
    rng = np.random.default_rng(4)
    for E, T, k in [(8, 300, 2), (64, 257, 6), (5, 1, 5)]:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
        idx[:, 0] = 0 if E > 3 else idx[:, 0]             # a hot expert
        counts, offsets, row_map, pos = oracle_lib.permute(idx, E)
        order = np.argsort(idx.ravel(), kind="stable")
        assert np.array_equal(row_map, order)
        assert np.array_equal(pos[row_map], np.arange(T * k))
        assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))


def test_permute_empty(oracle_lib):
    idx = np.zeros((0, 4), np.int32)
    counts, offsets, row_map, pos = oracle_lib.permute(idx, 8)
    assert (counts == 0).all() and (offsets == 0).all() and row_map.size == 0


# ------------------------------------------------------------------- aux ----

def test_aux_hand_example_golden(oracle_lib):
    d = {}
    for line in open(os.path.join(GOLDEN, "aux_hand_example.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            d[key] = [float(v) for v in vals]
    T, E, k = int(d["T"][0]), int(d["E"][0]), int(d["k"][0])
    l = np.array(d["logits"], np.float64).reshape(T, E)
    r = oracle_lib.route(l, score=oracle_lib.SOFTMAX, k=k, coeff=d["coeff"][0])
    assert list(r["idx"].ravel()) == [int(v) for v in d["idx"]]
    assert list(r["counts"]) == [int(v) for v in d["counts"]]
    assert math.isclose(r["aux"], d["aux"][0], rel_tol=1e-14)


@pytest.mark.parametrize("score", [0, 1])
def test_aux_uniform_probabilities_equals_coeff(oracle_lib, score):
    # equal logits -> p = 1/E for every token -> aux = coeff for ANY routing
    rng = np.random.default_rng(5)
    T, E, k = 37, 12, 3
    l = np.full((T, E), 0.3)
    for _ in range(3):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, *_ = oracle_lib.permute(idx, E)
        assert math.isclose(oracle_lib.aux(l, counts, k, score, 0.01), 0.01, rel_tol=1e-13)


def test_aux_single_expert_equals_coeff(oracle_lib):
    l = np.random.default_rng(6).standard_normal((11, 1))
    counts = np.array([11], np.int32)
    for score in (0, 1):
        assert math.isclose(oracle_lib.aux(l, counts, 1, score, 0.01), 0.01, rel_tol=1e-13)


def test_aux_empty_batch(oracle_lib):
    assert oracle_lib.aux(np.zeros((0, 4)), np.zeros(4, np.int32), 2, 0, 0.01) == 0.0


def test_aux_token_permutation_invariant(oracle_lib):
    rng = np.random.default_rng(7)
    l = rng.standard_normal((64, 16))
    r = oracle_lib.route(l, score=oracle_lib.SOFTMAX, k=4, renorm=True, coeff=0.01)
    perm = rng.permutation(64)
    r2 = oracle_lib.route(l[perm], score=oracle_lib.SOFTMAX, k=4, renorm=True, coeff=0.01)
    assert np.array_equal(r["counts"], r2["counts"])
    assert np.array_equal(r["offsets"], r2["offsets"])
    assert np.array_equal(r2["idx"], r["idx"][perm])
    assert math.isclose(r["aux"], r2["aux"], rel_tol=1e-12)


def test_logits_match_library_matmul(oracle_lib):
    import torch
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((37, 96)).astype(np.float32)).to(torch.bfloat16)
    Wr = rng.standard_normal((11, 96)).astype(np.float32) * 0.02
    bits = x.view(torch.int16).numpy().view(np.uint16)
    l = oracle_lib.logits(bits, Wr)
    ref = x.double().numpy() @ Wr.astype(np.float64).T
    assert np.allclose(l, ref, rtol=1e-13, atol=1e-15)
