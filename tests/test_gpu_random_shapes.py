"""Seeded random shapes for every entry point, against the oracle.

Each case draws its shape from a fixed seed, so a failure names a
reproducible case: token counts, head counts, cache positions, selection
widths, poisoned slots, row strides and cache offsets off the workloads'
grid. Every token (attention), every row (selection, cache writer) or the
sampled rows (score) are compared, to the same bars as the workload tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

from gpu_util import check_out, check_records, check_score_case, chunk_magnitude, oracle_token, run_attn, run_fused

pytestmark = pytest.mark.gpu


def _attn_shape(seed):
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.integers(1, 121))
    H = int(rng.integers(1, 17))
    pos0 = int(rng.integers(0, 5001))
    n_cells = pos0 + T + int(rng.integers(0, 51))
    implicit = seed % 4 == 3
    ids = None
    if not implicit:
        width = int(rng.integers(1, 601))
        stride = 64 * ((width + 63) // 64)
        ids = np.full((T, stride), -1, np.int32)
        for t in range(T):
            p = pos0 + t
            k = min(width, p + 1)
            ids[t, :k] = np.sort(rng.choice(p + 1, k, replace=False))
            bad = rng.random(stride) < 0.05
            ids[t, bad] = rng.choice(np.array([-1, -5, n_cells, n_cells + 9], np.int32), int(bad.sum()))
    return T, H, pos0, n_cells, ids


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_shapes(seed):
    T, H, pos0, n_cells, ids = _attn_shape(seed)
    print("random attention seed=%d T=%d H=%d pos0=%d n_cells=%d %s" % (
        seed, T, H, pos0, n_cells, "implicit" if ids is None else "width<=%d" % ids.shape[1]), flush=True)
    L = synth.make_layer(2000 + seed, 0, T, H, n_cells)
    scale = synth.SCALE_1_SQRT_128
    out, o, m, l, C = run_attn(L, ids, pos0, scale, implicit=ids is None)
    fout = run_fused(L, ids, pos0, scale, implicit=ids is None)
    for t in range(T):
        r = oracle_token(L, ids, pos0, scale, t)
        check_out(out[t], r["out64"], "random seed=%d t=%d" % (seed, t))
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, ids, pos0, scale, t, C), t, "random seed=%d" % seed)
        check_out(fout[t], r["out64"], "random fused seed=%d t=%d" % (seed, t))


@pytest.mark.parametrize("seed", range(10))
def test_score_random_shapes(seed):
    rng = np.random.default_rng(3000 + seed)
    T = int(rng.integers(1, 400))
    pos0 = int(rng.integers(0, 6001))
    Hs = int(rng.integers(1, 17))
    extra = int(rng.integers(0, 130))
    dead = [-math.inf, -1e30, 0.0, math.nan][seed % 4]
    scale = float(rng.choice([1.0, 0.5, synth.SCALE_1_SQRT_128]))
    print("random score seed=%d T=%d pos0=%d Hs=%d extra=%d" % (seed, T, pos0, Hs, extra), flush=True)
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, seed=3000 + seed, row_stride=pos0 + T + extra, scale=scale,
                          dead=dead)
    check_score_case(sc, n_sample=8, seed=seed)


@pytest.mark.parametrize("seed", range(10))
def test_select_random_shapes(seed):
    rng = np.random.default_rng(4000 + seed)
    T = int(rng.integers(1, 50))
    pos0 = int(rng.integers(0, 20001))
    K = int(rng.integers(1, 3001))
    kind = synth.SCORE_KINDS[seed % len(synth.SCORE_KINDS)]
    scores = synth.select_scores(T, pos0, seed=4000 + seed, kind=kind)
    stride = 64 * ((min(K, pos0 + T) + 63) // 64)
    print("random select seed=%d T=%d pos0=%d K=%d kind=%s" % (seed, T, pos0, K, kind), flush=True)
    ids = torch.full((T, stride), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_select(torch.from_numpy(scores).cuda(), pos0, K, ids)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    want = oracle.select(scores, pos0, K, stride, threads=8)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first differences (row, slot): %s" % bad[:5].tolist()


@pytest.mark.parametrize("seed", range(8))
def test_quant_random_shapes(seed):
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(1, 500))
    cell0 = int(rng.integers(0, 300))
    cap = cell0 + n + int(rng.integers(0, 40))
    kinds = synth.ROW_KINDS
    xk = synth.cache_rows(n, seed=5000 + seed, kind=kinds[seed % len(kinds)], which=0)
    xv = synth.cache_rows(n, seed=5000 + seed, kind=kinds[(seed + 2) % len(kinds)], which=1)
    print("random quant seed=%d n=%d cell0=%d cap=%d" % (seed, n, cell0, cap), flush=True)
    kq = torch.full((cap, 128), 0x5A, dtype=torch.int8, device="cuda")
    vq = torch.full((cap, 128), 0x5A, dtype=torch.int8, device="cuda")
    ksc = torch.full((cap, 4), 0x7E00, dtype=torch.int16, device="cuda").view(torch.float16)
    vsc = torch.full((cap, 4), 0x7E00, dtype=torch.int16, device="cuda").view(torch.float16)
    qsa.qsa_quant_append(torch.from_numpy(xk).cuda(), torch.from_numpy(xv).cuda(), kq, vq, ksc, vsc, cell0)
    torch.cuda.synchronize()
    for x, codes, scales in ((xk, kq, ksc), (xv, vq, vsc)):
        codes = codes.cpu().numpy()
        scales = scales.cpu().view(torch.int16).numpy().view(np.uint16)
        rc, rs = oracle.quant_rows(x)
        assert np.array_equal(codes[cell0:cell0 + n], rc)
        assert np.array_equal(scales[cell0:cell0 + n], rs)
        outside = np.r_[0:cell0, cell0 + n:cap]
        assert np.all(codes[outside] == 0x5A) and np.all(scales[outside] == 0x7E00)
