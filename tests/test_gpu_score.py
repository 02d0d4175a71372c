"""GPU parity of qsa_score against the CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest

from sparse_selection_attention_amd import synth

from gpu_util import check_score_case, run_score

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Hs", [1, 12])
def test_prompt_start_scores(Hs):
    sc = synth.score_case(T=1984, pos0=0, Hs=Hs)
    print("score prompt Hs=%d worst err/A %g" % (Hs, check_score_case(sc)), flush=True)


@pytest.mark.parametrize("pos0", [2051, 8192, 30000])
def test_long_position_scores(pos0):
    sc = synth.score_case(T=1984, pos0=pos0, Hs=12)
    print("score pos0=%d worst err/A %g" % (pos0, check_score_case(sc, n_sample=8)), flush=True)


@pytest.mark.parametrize("T,pos0,Hs,extra,dead", [
    (1, 0, 1, 0, -math.inf), (1, 63, 2, 5, -1e30), (65, 0, 3, 1, -math.inf), (64, 64, 1, 64, 0.0),
    (100, 37, 16, 3, -7.25), (130, 1, 5, 200, math.nan)])
def test_edge_shapes_and_tails(T, pos0, Hs, extra, dead):
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, row_stride=pos0 + T + extra, dead=dead, seed=T + pos0,
                          scale=0.7)
    check_score_case(sc, n_sample=64)


def test_integer_scores_are_exact():
    T, pos0, Hs = 100, 30, 4
    rng = np.random.default_rng(1)
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, scale=0.25)
    sc.q[:] = rng.integers(-3, 4, sc.q.shape)
    sc.k[:] = rng.integers(-3, 4, sc.k.shape)
    g = run_score(sc)
    ref = 0.25 * (sc.q.astype(np.int64).sum(1) @ sc.k.astype(np.int64).T)
    for t in range(T):
        assert np.array_equal(g[t, : pos0 + t + 1], ref[t, : pos0 + t + 1].astype(np.float32))


def test_score_determinism():
    sc = synth.score_case(T=200, pos0=100, Hs=12)
    a = run_score(sc)
    b = run_score(sc)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
