"""Pins of the oracle's per-row top-k (CPU only).

Brute force with sorted() on tiny rows, heapq.nlargest (a library routine) on
larger ones, exact ties built by duplicating values, and -1 padding for rows
with fewer than k candidates.
"""
import heapq

import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("seed", range(5))
def test_topk_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    rows = [rng.integers(-3, 4, size=rng.integers(0, 9)).astype(np.float64) for _ in range(20)]
    for k in (1, 3, 8, 12):
        got = oracle.topk_per_row(rows, k)
        for r, v in enumerate(rows):
            ranked = sorted(range(len(v)), key=lambda i: (-v[i], i))
            want = ranked[:k] + [-1] * max(0, k - len(v))
            assert got[r].tolist() == want


def test_topk_matches_nlargest_on_long_rows():
    lens = [0, 5, 2047, 2048, 2049, 10000, 40000]
    dense = synth.make_logit_rows(len(lens), max(lens), lens, seed=3)
    rows = [dense[r, :n].astype(np.float64) for r, n in enumerate(lens)]
    got = oracle.topk_per_row(rows, 2048)
    for r, v in enumerate(rows):
        want = [i for _, i in heapq.nlargest(2048, ((x, -i) for i, x in enumerate(v)))]
        want = [-i for i in want]
        m = min(2048, len(v))
        assert sorted(got[r, :m].tolist()) == sorted(want)
        assert np.all(got[r, m:] == -1)


def test_topk_ties_take_lowest_indices():
    v = np.array([1.0, 5.0, 3.0, 5.0, 3.0, 3.0, 0.0])
    got = oracle.topk_per_row([v], 4)[0].tolist()
    assert got == [1, 3, 2, 4]
