"""GPU parity of qsa_select (the selection producer) against the oracle.

Ids are integers chosen by comparing the same fp32 scores on both sides, so
the bar is bit-exact: every id and every -1 pad, on every row checked.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

pytestmark = pytest.mark.gpu


def run(scores, pos0, K, ids_stride):
    s = torch.from_numpy(scores).cuda()
    ids = torch.full((scores.shape[0], ids_stride), -7, dtype=torch.int32, device="cuda")
    print("qsa_select T=%d pos0=%d K=%d stride=%d" % (scores.shape[0], pos0, K, ids_stride), flush=True)
    qsa.qsa_select(s, pos0, K, ids)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def stride_for(K, pos0, T):
    return 64 * ((min(K, pos0 + T) + 63) // 64)


@pytest.mark.parametrize("kind", synth.SCORE_KINDS)
@pytest.mark.parametrize("T,pos0,K", [(64, 3000, 321), (40, 100, 64), (300, 100, 256), (16, 4000, 4000),
                                      (8, 9000, 2048), (6, 12000, 1000), (6, 20000, 3000)])
def test_matches_oracle_bitwise(kind, T, pos0, K):
    # row lengths across every keys-per-thread size, rows shorter and longer than K
    scores = synth.select_scores(T, pos0, seed=T + K, kind=kind)
    stride = stride_for(K, pos0, T)
    got = run(scores, pos0, K, stride)
    want = oracle.select(scores, pos0, K, stride, threads=8)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first differences (row, slot): %s" % bad[:5].tolist()


def test_longest_rows_supported():
    # pos0 + T = 32768: 32 keys per thread of 1024
    T, pos0, K = 4, 32764, 2051
    scores = synth.select_scores(T, pos0, seed=3, kind="ties")
    stride = stride_for(K, pos0, T)
    assert np.array_equal(run(scores, pos0, K, stride), oracle.select(scores, pos0, K, stride, threads=4))


def test_long_context_workload_rows():
    # the long-context shape: 1984 rows at pos0 = 30000, K = 2051 evenly sized with
    # the attention workload; every row checked for the defining property, 48
    # rows against the oracle bit for bit
    T, pos0, K = 1984, 30000, 2051
    scores = synth.select_scores(T, pos0, seed=5, kind="normal")
    stride = stride_for(K, pos0, T)
    got = run(scores, pos0, K, stride)
    assert np.all(got[:, K:] == -1)
    sel = got[:, :K]
    assert np.all(np.diff(sel, axis=1) > 0) and np.all(sel[:, 0] >= 0)
    assert np.all(sel[:, -1] <= pos0 + np.arange(T))
    rows = np.unique(np.r_[0, 1, T - 1, np.linspace(0, T - 1, 45).astype(int)])
    for t in rows:
        # the oracle on the row alone: row t of the workload is row 0 at pos0 + t
        w = oracle.select(scores[t: t + 1], pos0 + t, K, stride)
        assert np.array_equal(got[t], w[0]), "row %d" % t
    # defining property on every row: nothing left out above the smallest chosen score
    for t in range(T):
        p = pos0 + t
        row = scores[t, :p + 1]
        chosen = np.zeros(p + 1, bool)
        chosen[sel[t]] = True
        m = row[chosen].min()
        assert not np.any(row[~chosen] > m), t


def test_zero_rows_and_host_checks():
    ids = torch.full((0, 64), -7, dtype=torch.int32, device="cuda")
    s = torch.zeros(0, 10, dtype=torch.float32, device="cuda")
    qsa.qsa_select(s, 5, 3, ids)
    ids = torch.zeros(2, 64, dtype=torch.int32, device="cuda")
    with pytest.raises(qsa.QsaError):
        qsa.qsa_select(torch.zeros(2, 10, dtype=torch.float32, device="cuda"), 9, 3, ids)   # row_stride < pos0 + T
    with pytest.raises(qsa.QsaError):
        qsa.qsa_select(torch.zeros(2, 40000, dtype=torch.float32, device="cuda"), 2 ** 25 - 1, 3, ids)   # too long


def test_score_select_attend_pipeline():
    # scores (qsa_score) -> ids (qsa_select) -> attention (qsa_attn_merge), all
    # on the device: the ids chosen from the device scores satisfy the rule, and
    # the attention over them is finite and deterministic
    T, pos0, H, K = 96, 3000, 12, 321
    sc = synth.score_case(T=T, pos0=pos0, Hs=H)
    layer = synth.make_layer(5, 0, T, H, pos0 + T)
    dev = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    scores = torch.empty(T, sc.row_stride, dtype=torch.float32, device=dev)
    qsa.qsa_score(up(sc.q), up(sc.k), pos0, 1.0, float("-inf"), scores)
    stride = stride_for(K, pos0, T)
    ids = torch.empty(T, stride, dtype=torch.int32, device=dev)
    qsa.qsa_select(scores, pos0, K, ids)
    out = torch.empty(T, H, 128, dtype=torch.float16, device=dev)
    args = (up(layer.q), up(layer.kq), up(layer.vq), up(layer.ksc), up(layer.vsc), ids, pos0, 0.0883883476)
    qsa.qsa_attn_merge(*args, out)
    out2 = torch.empty_like(out)
    qsa.qsa_attn_merge(*args, out2)
    torch.cuda.synchronize()
    s_h, ids_h = scores.cpu().numpy(), ids.cpu().numpy()
    for t in range(T):
        p = pos0 + t
        sel = ids_h[t, :K]
        assert np.all(np.diff(sel) > 0) and sel[-1] <= p and np.all(ids_h[t, K:] == -1)
        chosen = np.zeros(p + 1, bool)
        chosen[sel] = True
        assert not np.any(s_h[t, :p + 1][~chosen] > s_h[t, :p + 1][chosen].min())
    assert torch.isfinite(out.float()).all() and torch.equal(out, out2)


@pytest.mark.parametrize("n_in_bin", [0, 1, 4000, 8192, 8193, 20000])
def test_rows_crowded_into_one_top_byte_bin(n_in_bin):
    """Rows with 1, 4000, 8192, 8193 and 20000 keys in [1, 2) (one top-byte
    bin, the rest below it), with repeated values among them, and
    (n_in_bin = 0) rows whose every key shares one top byte: the threshold is
    decided by the lower bytes, against the oracle bit for bit."""
    T, pos0 = 4, 20000
    rng = np.random.default_rng(n_in_bin + 7)
    scores = rng.uniform(0.25, 0.5, (T, pos0 + T)).astype(np.float32)
    pos = rng.choice(pos0, size=n_in_bin, replace=False)
    vals = rng.uniform(1.0, 2.0, n_in_bin).astype(np.float32)
    if n_in_bin:
        vals[::7] = vals[0]                          # runs of one equal value
    scores[:, pos] = vals
    for K in (1, 100, 2051, max(1, n_in_bin - 1)):
        stride = stride_for(K, pos0, T)
        got = run(scores, pos0, K, stride)
        want = oracle.select(scores, pos0, K, stride, threads=8)
        bad = np.argwhere(got != want)
        assert bad.size == 0, "K=%d first differences (row, slot): %s" % (K, bad[:5].tolist())


@pytest.mark.parametrize("kind", synth.SCORE_KINDS)
@pytest.mark.parametrize("T,pos0,K", [(20, 32760, 2051), (3, 70000, 4000), (2, 131000, 2051), (2, 40000, 45000)])
def test_rows_past_the_register_limit(kind, T, pos0, K):
    """Rows of more than 32768 cells stream their scores on every pass; a call
    whose rows straddle 32768 cells runs both kernels. Every id and pad against
    the oracle, bit for bit (the last case has K above some rows' length)."""
    scores = synth.select_scores(T, pos0, seed=T + K + pos0 % 97, kind=kind)
    stride = stride_for(K, pos0, T)
    got = run(scores, pos0, K, stride)
    want = oracle.select(scores, pos0, K, stride, threads=8)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first differences (row, slot): %s" % bad[:5].tolist()
