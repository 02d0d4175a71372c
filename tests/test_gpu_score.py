"""GPU parity of qsa_score against the CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest

import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

import oracle
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



@pytest.mark.parametrize("T,pos0,Hs,extra", [(1000, 0, 3, 7), (777, 13, 12, 0), (1999, 77, 5, 65), (900, 4000, 2, 1)])
def test_ragged_row_tiles_in_both_workgroup_orders(T, pos0, Hs, extra):
    """Row counts off the 64-row grid with eight or more row tiles. The first
    three take the order in which XCDs own every eighth row tile (their causal
    rows differ a lot in length), the last the run-major order; every row's
    extents are checked, and the values of 24 rows against the oracle."""
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, row_stride=pos0 + T + extra, seed=T + 7 * pos0, scale=0.6)
    print("score ragged T=%d pos0=%d worst err/A %g" % (T, pos0, check_score_case(sc, n_sample=24, seed=T)),
          flush=True)


# (T, pos0, Hs, whether the first pass runs): it runs where q is 4 MB or more
# and every XCD reads all of q (the run-major order of long contexts); near the
# start of a sequence (row-major order), with small q or one head it does not,
# and the workspace keeps its contents
WS_SHAPES = [(1984, 30000, 12, True), (1984, 8192, 12, True), (700, 30000, 16, True), (2100, 5000, 4, True),
             (600, 30000, 14, True), (1984, 0, 12, False), (777, 13, 16, False), (1000, 0, 3, False),
             (96, 30000, 12, False), (1984, 30000, 1, False), (17, 5, 2, False), (1, 0, 1, False)]


@pytest.mark.parametrize("T,pos0,Hs,prepared", WS_SHAPES)
def test_workspace_path_gives_the_same_bits(T, pos0, Hs, prepared):
    """qsa_score_ws: scores, tails and untouched cells are qsa_score's bit for
    bit, and the workspace is written exactly where the first pass runs."""
    import torch
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, row_stride=pos0 + T + 5, seed=11 * T + pos0, scale=0.8, dead=-3.5)
    ws = torch.full((qsa.qsa_score_ws_bytes(T),), 0xA5, dtype=torch.uint8, device="cuda")
    a = run_score(sc)
    b = run_score(sc, workspace=ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert bool((ws != 0xA5).any()) == prepared


def test_workspace_path_against_the_oracle():
    sc = synth.score_case(T=1984, pos0=30000, Hs=12)
    print("score_ws pos0=30000 worst err/A %g" % check_score_case(sc, n_sample=8, workspace=True), flush=True)


def test_workspace_reused_across_calls():
    """One workspace for two calls in a row that both take the first pass, the
    second with fewer rows (a ragged last row tile): each call's scores are
    those of qsa_score."""
    import torch
    ws = torch.full((qsa.qsa_score_ws_bytes(1984),), 0x5A, dtype=torch.uint8, device="cuda")
    for T, pos0, Hs in [(1984, 30000, 12), (700, 30000, 16)]:
        sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, seed=T + 1)
        assert np.array_equal(run_score(sc, workspace=ws).view(np.uint32), run_score(sc).view(np.uint32)), T


@pytest.mark.parametrize("offset", [1, 8, 16])
def test_scores_buffer_off_the_64_byte_grid(offset):
    """A scores pointer 4, 32 or 64 bytes past an aligned base, with an even row
    stride: rows that do not start 64-byte aligned take cached stores (the
    first two offsets), aligned ones nontemporal stores. The scores, tails and
    untouched cells are those of the aligned call, bit for bit."""
    import torch
    sc = synth.score_case(T=700, pos0=3000, Hs=12, row_stride=3000 + 700 + 12, seed=offset, scale=0.5, dead=-2.0)
    want = run_score(sc)
    q, k = torch.from_numpy(sc.q).cuda(), torch.from_numpy(sc.k).cuda()
    n = sc.T * sc.row_stride
    buf = torch.full((n + offset,), float("nan"), dtype=torch.float32, device="cuda")
    scores = buf[offset: offset + n].view(sc.T, sc.row_stride)
    qsa.qsa_score(q, k, sc.pos0, float(sc.scale), float(sc.dead), scores)
    torch.cuda.synchronize()
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), want.view(np.uint32))

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


def _compare_causal(sc, g, rows):
    """Oracle comparison on whole causal rows, non-finite values included:
    finite oracle scores within 1e-4 of the error scale, infinities with the
    same sign, NaN where the oracle has NaN."""
    A_q = np.abs(sc.q.astype(np.float64)).sum(axis=1)
    for t in rows:
        p = sc.pos0 + t
        r = oracle.score(sc.q[t: t + 1], sc.k, p, sc.scale, sc.dead, sc.row_stride)[0, : p + 1]
        x = g[t, : p + 1].astype(np.float64)
        nan = np.isnan(r)
        assert np.array_equal(np.isnan(x), nan), "row %d: NaN pattern" % t
        inf = np.isinf(r)
        assert np.array_equal(x[inf], r[inf]), "row %d: infinities" % t
        fin = ~(nan | inf)
        with np.errstate(invalid="ignore", over="ignore"):
            A = abs(float(sc.scale)) * (np.abs(sc.k[: p + 1].astype(np.float64)) @ A_q[t])
        err = np.abs(x[fin] - r[fin])
        assert np.all(np.isfinite(x[fin])), "row %d: a finite oracle score came out non-finite" % t
        assert np.all(err <= 1e-4 * np.maximum(np.abs(r[fin]), A[fin])), "row %d: err/A %g" % (t, (err / A[fin]).max())


def test_scores_beyond_the_bf16_range():
    """Operands above the largest finite bf16 (3.3895e38, below fp32's 3.4028e38)
    still give finite scores within the bound: the kernel's high part is taken
    from the clamped value and the remainder is finite."""
    T, pos0, Hs = 70, 100, 1
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, scale=1.0)
    rng = np.random.default_rng(3)
    n = sc.n_cells
    sc.q[:, 0, 0] = np.float32(3.40e38) * rng.choice([-1.0, 1.0], T).astype(np.float32)
    sc.k[:, 0] = (rng.uniform(1e-3, 1e-2, n) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    sc.k[:, 1] = np.float32(3.395e38) * rng.choice([-1.0, 1.0], n).astype(np.float32)
    sc.q[:, 0, 1] = (rng.uniform(1e-4, 1e-3, T)).astype(np.float32)
    sc.k[:, 2:] = 0.0                                  # keep every score within fp32 range
    g = run_score(sc)
    _compare_causal(sc, g, range(T))


def test_infinite_and_nan_operands():
    """An infinite q or K component gives an infinity of the same sign (the
    other operand's matching component is a normal number), and NaN stays NaN."""
    T, pos0, Hs = 66, 30, 2
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, scale=0.5)
    rng = np.random.default_rng(4)
    n = sc.n_cells
    sc.k[:, 5] = (rng.uniform(0.5, 1.0, n) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    sc.q[3, 1, 5] = np.inf                             # row 3: +inf times K's column 5
    sc.q[40, 0, 5] = -np.inf                           # row 40: -inf
    sc.q[50, 0, 7] = np.nan                            # row 50: NaN
    sc.q[:, :, 9] = np.abs(sc.q[:, :, 9]) + 0.5       # column 9 of q: normal, positive
    sc.k[17, 9] = np.inf                               # cell 17: +inf for every row ...
    sc.k[17, 5] = 0.75                                 # ... also row 3's (+inf from both sides)
    g = run_score(sc)
    assert np.isinf(g[3, : pos0 + 4]).all() and g[3, 17] == np.inf
    row40 = g[40, : pos0 + 41]
    assert np.isnan(row40[17])                         # -inf from column 5 meets +inf from column 9
    assert np.isinf(np.delete(row40, 17)).all()
    assert np.isnan(g[50, : pos0 + 51]).all()
    assert (g[[0, 20, 65], 17] == np.inf).all()
    _compare_causal(sc, g, [0, 3, 17, 20, 40, 50, 65])


@pytest.mark.parametrize("T,pos0,Hs", [(1, 30000, 12), (8, 30000, 12), (16, 4000, 3), (17, 4000, 1)])
def test_decode_sized_score_calls(T, pos0, Hs):
    """Calls of a few rows (a decode step) spread one column tile per
    workgroup; every row against the oracle, tail and untouched cells included."""
    print("score decode-sized", check_score_case(synth.score_case(T=T, pos0=pos0, Hs=Hs), n_sample=T), flush=True)
