"""Pins, on the CPU, the expected results of moe_permute_checked that the GPU
test compares the kernel with: with valid ids they are the oracle's
permutation; with ids outside [0, E) they are the oracle's permutation of a
layer with one extra expert E that collects those slots, cut at that expert."""
import numpy as np
import pytest

import oracle
from tests import harness as hz


@pytest.mark.parametrize("T,k,E,frac", [(300, 4, 16, 0.0), (257, 3, 8, 0.1), (1000, 8, 64, 0.5),
                                        (50, 2, 4, 1.0)])
def test_checked_permute_reference_against_the_oracle(T, k, E, frac):
    rng = np.random.default_rng(T + k + E)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    bad = rng.random((T, k)) < frac
    junk = rng.choice(np.array([-1, -7, E, E + 5, 2 ** 31 - 1, -2 ** 31], np.int64), size=(T, k))
    idx = np.where(bad, junk, idx).astype(np.int32)
    counts, offsets, row_map, pos, n_bad = hz.checked_permute_reference(idx, E)
    assert n_bad == int(bad.sum())
    sent = np.where(bad, E, idx).astype(np.int32)          # the extra expert E
    c, o, rm, ps = oracle.permute(sent, E + 1)
    assert np.array_equal(counts, c[:E])
    assert np.array_equal(offsets, o[:E + 1])
    placed = int(o[E])
    assert np.array_equal(row_map[:placed], rm[:placed]) and (row_map[placed:] == -1).all()
    flat_bad = bad.ravel()
    assert np.array_equal(pos[~flat_bad], ps[~flat_bad]) and (pos[flat_bad] == -1).all()
