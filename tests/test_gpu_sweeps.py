"""Sweeps over the pages' shape grids, against the oracle.

* query tokens x cache position: T in {96, 512, 1024, 1984} and pos0 in
  {0, 1984, 2050, 2052, 30000}, the grid the pages time their attention and
  score kernels on ("round 11 track b: qsa attention and score", sections
  "implementation and evaluator" and "score: valid negative result"), with the
  evenly spaced selection of up to 2051 cells;
* decode widths 1, 31, 64, 65, 128, 319, 320, 321, 383 and 384 ("round 5
  track b: cached residual norms and fused mtp attention", sections "mtp
  attention" and "actual verification"): two tokens (one at width 384), with
  the most recent cells and with scattered cells.

Each case checks sampled tokens of both attention paths (chunk records + merge,
and the fused dispatch) and, for the score, every row's extents and sampled
rows' values.
"""
import numpy as np
import pytest

from sparse_selection_attention_amd import synth

from gpu_util import check_attn_case, check_fused_case, check_score_case

pytestmark = pytest.mark.gpu

GRID_T = (96, 512, 1024, 1984)
GRID_POS0 = (0, 1984, 2050, 2052, 30000)


@pytest.mark.parametrize("pos0", GRID_POS0)
@pytest.mark.parametrize("T", GRID_T)
def test_attention_grid(T, pos0):
    case = synth.make_case("grid_T%d_p%d" % (T, pos0), T, pos0, 12, synth.evenly_spaced_ids(pos0, T, 2051))
    print("attention grid T=%d pos0=%d" % (T, pos0), flush=True)
    check_attn_case(case, n_sample=6, seed=T + pos0)
    check_fused_case(case, n_sample=6, seed=T + pos0 + 1)


@pytest.mark.parametrize("pos0", GRID_POS0)
@pytest.mark.parametrize("T", (96, 1984))
def test_score_grid(T, pos0):
    print("score grid T=%d pos0=%d" % (T, pos0), flush=True)
    check_score_case(synth.score_case(T=T, pos0=pos0, Hs=12), n_sample=4, seed=T + pos0)


def decode_ids(pos0, ntok, width, scattered):
    """Row t (p = pos0 + t): `width` causal cells, the most recent ones or spread
    over 0..p, padded with -1 to a multiple of 64."""
    stride = 64 * ((width + 63) // 64)
    ids = np.full((ntok, stride), -1, dtype=np.int32)
    for t in range(ntok):
        p = pos0 + t
        if scattered:
            ids[t, :width] = synth.evenly_spaced_ids(p, 1, width)[0, :width]
        else:
            ids[t, :width] = np.arange(p - width + 1, p + 1, dtype=np.int32)
    return ids


@pytest.mark.parametrize("scattered", [False, True])
@pytest.mark.parametrize("width", [1, 31, 64, 65, 128, 319, 320, 321, 383, 384])
def test_decode_widths(width, scattered):
    ntok = 1 if width == 384 else 2
    pos0 = 3000
    case = synth.make_case("decode_w%d" % width, ntok, pos0, 12, decode_ids(pos0, ntok, width, scattered),
                           seed=width)
    print("decode width %d scattered=%s" % (width, scattered), flush=True)
    check_attn_case(case, n_sample=ntok)
    check_fused_case(case, n_sample=ntok)
