"""Pins of the oracle's selection producer (qso_select): top-K causal cells by
score, equal scores to the smaller cell, ascending ids, -1 padding.

The rule is a reading of the pages (they never print one); these tests tie the
oracle to hand-worked rows, to the defining property checked directly, and to
closed forms, so that a reversed order, a wrong tie-break or an off-by-one in
the causal range fails here.
"""
import numpy as np
import pytest

import oracle


def test_hand_worked_row():
    # p = 7, cells 0..7: scores 0.5, 2, -1, 2, +0, -0, 7, 1
    s = np.array([[0.5, 2.0, -1.0, 2.0, 0.0, -0.0, 7.0, 1.0]], np.float32)
    assert oracle.select(s, 7, 4, 8)[0].tolist() == [1, 3, 6, 7, -1, -1, -1, -1]   # 7, 2, 2, 1
    assert oracle.select(s, 7, 5, 8)[0].tolist() == [0, 1, 3, 6, 7, -1, -1, -1]    # + 0.5
    # +0 (cell 4) and -0 (cell 5) are equal: the smaller cell wins
    assert oracle.select(s, 7, 6, 8)[0].tolist() == [0, 1, 3, 4, 6, 7, -1, -1]
    assert oracle.select(s, 7, 7, 8)[0].tolist() == [0, 1, 3, 4, 5, 6, 7, -1]
    assert oracle.select(s, 7, 20, 64)[0].tolist() == list(range(8)) + [-1] * 56   # fewer cells than K


def test_only_causal_cells_are_read():
    # row t sees cells 0 .. pos0 + t; later cells (a large value there) never count
    T, pos0, K = 4, 10, 5
    s = np.zeros((T, 20), np.float32)
    s[:, :] = np.arange(20, dtype=np.float32)[None, :]          # increasing: the last causal cells win
    ids = oracle.select(s, pos0, K, 64)
    for t in range(T):
        p = pos0 + t
        assert ids[t, :K].tolist() == list(range(p - K + 1, p + 1))
        assert np.all(ids[t, K:] == -1)


@pytest.mark.parametrize("kind", ["decreasing", "increasing", "constant"])
def test_closed_forms(kind):
    n, K = 300, 64
    base = {"decreasing": -np.arange(n), "increasing": np.arange(n), "constant": np.zeros(n)}[kind]
    s = base.astype(np.float32)[None, :]
    ids = oracle.select(s, n - 1, K, 128)[0]
    want = {"decreasing": range(K), "increasing": range(n - K, n), "constant": range(K)}[kind]
    assert ids[:K].tolist() == list(want) and np.all(ids[K:] == -1)


@pytest.mark.parametrize("K", [1, 63, 64, 65, 299, 300, 301])
def test_count_at_the_boundary(K):
    # a row of n = 300 cells gives min(K, 300) ids
    s = np.random.default_rng(K).standard_normal((1, 300)).astype(np.float32)
    ids = oracle.select(s, 299, K, 384)[0]
    take = min(K, 300)
    assert np.all(ids[:take] >= 0) and np.all(ids[take:] == -1)


def check_defining_property(scores, pos0, K, ids):
    T = scores.shape[0]
    for t in range(T):
        n = pos0 + t + 1
        row = scores[t, :n].astype(np.float64)
        take = min(K, n)
        sel = ids[t, :take]
        assert np.all(ids[t, take:] == -1)
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < n          # ascending, unique, causal
        chosen = np.zeros(n, bool)
        chosen[sel] = True
        m = row[chosen].min()
        assert not np.any(row[~chosen] > m)                                        # nothing left out above
        eq = np.flatnonzero(row == m)
        k_eq = chosen[eq].sum()
        assert np.all(chosen[eq[:k_eq]]) and not np.any(chosen[eq[k_eq:]])         # ties: the smaller cells


def test_defining_property_with_many_ties():
    rng = np.random.default_rng(7)
    T, pos0, K = 24, 500, 200
    # values on a coarse grid (many equal scores), signed zeros among them
    s = (rng.integers(-20, 21, (T, pos0 + T)) / 4.0).astype(np.float32)
    s[rng.random(s.shape) < 0.05] = -0.0
    ids = oracle.select(s, pos0, K, 256, threads=4)
    check_defining_property(s, pos0, K, ids)


def test_defining_property_random_rows():
    rng = np.random.default_rng(8)
    T, pos0, K = 16, 3000, 321
    s = rng.standard_normal((T, pos0 + T)).astype(np.float32)
    s[:, 5] = np.inf
    s[:, 9] = -np.inf
    ids = oracle.select(s, pos0, K, 384, threads=4)
    check_defining_property(s, pos0, K, ids)
    assert np.all(np.any(ids == 5, axis=1))                                        # +inf always chosen
