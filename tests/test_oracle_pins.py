"""Pins of the CPU oracle against things other than itself.

Each test ties one part of the oracle to a library routine, a closed form, an
invariant of the method or a figure the pages print, so that a dropped term, a
wrong index or sign, or a transposed operand in the oracle fails here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from sparse_selection_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# binary16 codec, against numpy's conversions


def test_half_decode_all_patterns(oracle_lib):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.qso_half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # signed zeros too


def test_half_encode_matches_numpy_rne(oracle_lib):
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        # exact ties between neighbouring fp16 values, normal and subnormal
        (np.arange(-3000, 3000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -10,
        [0.0, -0.0, 65504.0, 65519.999, 65520.0, -65520.0, 1e30, -1e-30, 2.0 ** -25, 3 * 2.0 ** -25,
         math.inf, -math.inf],
    ])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle_lib.qso_double_to_half(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert oracle_lib.qso_double_to_half(math.nan) & 0x7C00 == 0x7C00


# ---------------------------------------------------------------------------
# helpers


def deq_rows(xq, sc, cells):
    """Dequantised rows in fp64, by numpy broadcasting (int8 row times its group scale)."""
    D = xq.shape[1]
    s = np.repeat(sc[cells].astype(np.float64), synth.GROUP, axis=1)
    assert s.shape[1] == D
    return xq[cells].astype(np.float64) * s


def sdpa_reference(L, ids, pos0, scale, n_cells):
    """Plain softmax attention over each row's valid ids, by torch's SDPA in fp64."""
    T, H, D = L.q.shape
    out = np.zeros((T, H, D))
    for t in range(T):
        row = ids[t] if ids is not None else np.where(np.arange(64 * ((pos0 + T + 63) // 64)) <= pos0 + t,
                                                      np.arange(64 * ((pos0 + T + 63) // 64)), -1)
        cells = np.array([c for c in row if 0 <= c < n_cells], dtype=np.int64)
        if len(cells) == 0:
            continue
        K = torch.from_numpy(deq_rows(L.kq, L.ksc, cells))[None, None].expand(1, H, -1, -1)
        V = torch.from_numpy(deq_rows(L.vq, L.vsc, cells))[None, None].expand(1, H, -1, -1)
        Q = torch.from_numpy(L.q[t].astype(np.float64))[None, :, None, :]
        o = F.scaled_dot_product_attention(Q, K, V, scale=float(np.float32(scale)))
        out[t] = o[0, :, 0, :].numpy()
    return out


def random_case(rng, T, H, n_cells, C, p_poison, pos0=None, dup=False, D=128):
    if pos0 is None:
        pos0 = n_cells - T
    L = synth.make_layer(int(rng.integers(1 << 30)), 0, T, H, n_cells, D)
    ids = np.full((T, 64 * C), -1, dtype=np.int32)
    for t in range(T):
        p = pos0 + t
        cand = rng.integers(0, p + 1, 64 * C)
        if not dup:
            cand = rng.permutation(p + 1)[: 64 * C] if p + 1 >= 64 * C else np.concatenate(
                [rng.permutation(p + 1), rng.integers(0, p + 1, 64 * C - p - 1)])
        keep = rng.random(64 * C) >= p_poison
        row = np.where(keep, cand, -1)
        # poison of other kinds: ids past the cache and other negatives
        bad = rng.random(64 * C) < 0.05
        row = np.where(bad, rng.choice([n_cells, n_cells + 7, -5, -(1 << 31)], 64 * C), row)
        ids[t] = row
    return L, ids, pos0


# ---------------------------------------------------------------------------
# attention: chunked softmax + max-first merge == plain softmax attention


@pytest.mark.parametrize("seed", range(6))
def test_attn_matches_library_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 6))
    H = int(rng.integers(1, 4))
    C = int(rng.integers(1, 7))
    n_cells = int(rng.integers(T + 1, 300))
    L, ids, pos0 = random_case(rng, T, H, n_cells, C, p_poison=float(rng.random() * 0.8),
                               dup=bool(seed % 2))
    scale = np.float32(rng.choice([1 / math.sqrt(128), 0.0625, 0.5]))
    out64, out16, _ = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, pos0, scale)
    ref = sdpa_reference(L, ids, pos0, scale, n_cells)
    assert np.allclose(out64, ref, rtol=1e-11, atol=1e-14)
    # the fp16 output is the ties-to-even rounding of the fp64 value
    assert np.array_equal(out16.view(np.uint16), out64.astype(np.float16).view(np.uint16))


def test_attn_implicit_rows_match_sdpa_causal():
    L = synth.make_layer(7, 0, 5, 2, 140)
    pos0 = 135
    out64, _, _ = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, None, pos0, synth.SCALE_1_SQRT_128)
    ref = sdpa_reference(L, None, pos0, synth.SCALE_1_SQRT_128, 140)
    assert np.allclose(out64, ref, rtol=1e-11, atol=1e-14)


def test_large_logits_do_not_overflow():
    rng = np.random.default_rng(3)
    L, ids, pos0 = random_case(rng, 3, 2, 200, 3, 0.3)
    L.q[:] = (L.q.astype(np.float32) * 300).astype(np.float16)   # |S| reaches ~1e4
    scale = np.float32(1.0)
    out64, _, (m, _, _) = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, pos0, scale)
    assert np.nanmax(np.abs(m[np.isfinite(m)])) > 1e3
    assert np.all(np.isfinite(out64))
    ref = sdpa_reference(L, ids, pos0, scale, 200)
    assert np.allclose(out64, ref, rtol=1e-10, atol=1e-13)


def test_chunk_partition_invariance():
    """The same multiset of valid ids, laid out in different chunks, gives the same output."""
    rng = np.random.default_rng(11)
    T, H, n_cells = 3, 2, 400
    L = synth.make_layer(9, 0, T, H, n_cells)
    pos0 = n_cells - T
    outs = []
    base = [rng.integers(0, pos0 + t + 1, 150) for t in range(T)]
    for C in (3, 4, 6):
        ids = np.full((T, 64 * C), -1, dtype=np.int32)
        for t in range(T):
            slots = rng.permutation(64 * C)[:150]
            ids[t, slots] = rng.permutation(base[t])
        outs.append(oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, pos0, synth.SCALE_1_SQRT_128)[0])
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# closed forms


def test_one_cell_selection_returns_dequantised_v_exactly():
    T, H, n_cells = 4, 3, 90
    L = synth.make_layer(13, 0, T, H, n_cells)
    ids = np.full((T, 128), -1, dtype=np.int32)
    cells = [0, 17, 63, 89]
    for t, c in enumerate(cells):
        ids[t, 70 + t] = c                      # lone valid slot, in the second chunk
    out64, out16, (m, l, o) = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, n_cells - T,
                                          synth.SCALE_1_SQRT_128)
    for t, c in enumerate(cells):
        v = L.vq[c].astype(np.float64) * np.repeat(L.vsc[c].astype(np.float64), 32)
        assert np.array_equal(out64[t], np.broadcast_to(v, (H, 128)))
        assert np.array_equal(out16[t].view(np.uint16),
                              np.broadcast_to(v.astype(np.float16).view(np.uint16), (H, 128)))
        assert np.all(l[t, 1] == 1.0) and np.all(m[t, 0] == -np.inf) and np.all(l[t, 0] == 0.0)


def test_uniform_probe_gives_exact_integer_records():
    """q = 1, K = 0 makes every score 0, so l counts valid slots and o sums V rows."""
    rng = np.random.default_rng(5)
    L, ids, pos0 = random_case(rng, 4, 2, 250, 4, 0.4, dup=True)
    L.q[:] = 1.0
    L.kq[:] = 0
    L.vsc[:] = 1.0
    _, _, (m, l, o) = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, pos0, np.float32(0.37))
    for t in range(4):
        for k in range(4):
            row = ids[t, 64 * k: 64 * k + 64]
            cells = row[(row >= 0) & (row < 250)]
            if len(cells) == 0:
                assert np.all(m[t, k] == -np.inf) and np.all(l[t, k] == 0)
                continue
            assert np.all(m[t, k] == 0.0) and np.all(l[t, k] == len(cells))
            s = L.vq[cells].astype(np.int64).sum(axis=0)
            assert np.array_equal(o[t, k], np.broadcast_to(s.astype(np.float64), (2, 128)))


def test_k_address_probe_max_is_exact():
    """One-hot q at d0 and unit scales make each score the cell's own K byte at d0."""
    T, H, n_cells = 3, 1, 500
    L = synth.make_layer(21, 0, T, H, n_cells)
    d0 = 77
    L.q[:] = 0.0
    L.q[:, :, d0] = 1.0
    L.ksc[:] = 1.0
    L.kq[:, d0] = ((np.arange(n_cells) * 2654435761) % 255 - 127).astype(np.int8)
    rng = np.random.default_rng(2)
    ids = rng.integers(-1, n_cells - T, (T, 256)).astype(np.int32)
    _, _, (m, _, _) = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, n_cells - T, np.float32(1.0))
    for t in range(T):
        for k in range(4):
            row = ids[t, 64 * k: 64 * k + 64]
            assert m[t, k, 0] == L.kq[row[row >= 0], d0].astype(np.float64).max()


def test_poison_independence_and_empty_records():
    rng = np.random.default_rng(8)
    L, ids, pos0 = random_case(rng, 3, 2, 300, 3, 0.5)
    ids[1, 64:128] = -1                        # an empty chunk
    ids[2, :] = -1                             # an empty row
    sentinel = 12345.0
    T, H, D = L.q.shape
    C = 3
    m0 = np.full((T, C, H), np.nan)
    l0 = np.full((T, C, H), np.nan)
    o0 = np.full((T, C, H, D), sentinel)
    m, l, o = oracle.attn_chunks(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, pos0, synth.SCALE_1_SQRT_128,
                                 m=m0, l=l0, o=o0)
    assert np.all(m[1, 1] == -np.inf) and np.all(l[1, 1] == 0.0) and np.all(o[1, 1] == sentinel)
    assert np.all(np.signbit(l[1, 1]) == False)  # noqa: E712  (+0, not -0)
    out64, out16 = oracle.merge(m, l, o)
    assert np.array_equal(out16[2].view(np.uint16), np.zeros((H, D), np.uint16))  # +0
    # change everything no valid slot points at, including row 0 when unused
    used = set(int(c) for c in ids.ravel() if 0 <= c < 300)
    L2 = synth.Layer(L.q.copy(), L.kq.copy(), L.vq.copy(), L.ksc.copy(), L.vsc.copy())
    for c in range(300):
        if c not in used:
            L2.kq[c] = 99
            L2.vq[c] = -99
            L2.ksc[c] = 7.0
            L2.vsc[c] = 3.0
    # every kind of invalid id is the same as -1
    ids2 = ids.copy()
    ids2[ids2 < 0] = -1
    ids2[ids2 >= 300] = -1
    out64b, _, _ = oracle.attn(L2.q, L2.kq, L2.vq, L2.ksc, L2.vsc, ids2, pos0, synth.SCALE_1_SQRT_128)
    assert np.array_equal(out64.view(np.uint64), out64b.view(np.uint64))


@pytest.mark.parametrize("variant", ["signed_zero", "cancel"])
def test_edge_variants_reduce_to_mean_of_selected_v(variant):
    case = synth.long_ctx(layers=1, T=8, variant=variant)
    L = case.layers[0]
    toks = [0, 4] if variant == "signed_zero" else [1, 5]
    heads = [0, 6] if variant == "signed_zero" else list(range(12))
    for t in toks:
        out64, out16, (m, l, o) = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, case.ids, case.pos0,
                                              case.scale, t_range=(t, t + 1))
        row = case.ids[t]
        cells = row[row >= 0]
        mean = deq_rows(L.vq, L.vsc, cells).mean(axis=0)
        for h in heads:
            assert np.all(m[t, :, h] == 0.0)              # every score is +-0
            assert not np.any(np.isnan(out64[t, h]))
            ulp = np.spacing(np.abs(mean).astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(out16[t, h].astype(np.float64) - mean) <= ulp)


# ---------------------------------------------------------------------------
# causal scores


@pytest.mark.parametrize("T,pos0,Hs,row_stride", [(5, 0, 1, 5), (70, 3, 12, 80), (9, 130, 2, 139),
                                                  (33, 64, 3, 200)])
def test_score_matches_matmul_and_tail_extents(T, pos0, Hs, row_stride):
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, D=128, row_stride=row_stride, seed=T + pos0,
                          scale=0.3, dead=-7.5)
    got = oracle.score(sc.q, sc.k, pos0, sc.scale, sc.dead, row_stride)
    q64 = sc.q.astype(np.float64)
    k64 = sc.k.astype(np.float64)
    ref = np.float64(np.float32(0.3)) * np.einsum("thd,cd->tc", q64, k64)
    for t in range(T):
        p = pos0 + t
        assert np.allclose(got[t, : p + 1], ref[t, : p + 1], rtol=1e-12, atol=1e-12)
        tail_end = min(64 * ((p + 1 + 63) // 64), row_stride)
        assert np.all(got[t, p + 1: tail_end] == -7.5)
        assert np.all(np.isnan(got[t, tail_end:]))


def test_score_integer_probe_exact():
    T, pos0, Hs = 6, 60, 3
    rng = np.random.default_rng(4)
    q = rng.integers(-3, 4, (T, Hs, 128)).astype(np.float32)
    k = rng.integers(-3, 4, (pos0 + T, 128)).astype(np.float32)
    got = oracle.score(q, k, pos0, np.float32(0.25), -math.inf, pos0 + T)
    ref = 0.25 * (q.astype(np.int64).sum(axis=1) @ k.astype(np.int64).T)
    for t in range(T):
        assert np.array_equal(got[t, : pos0 + t + 1], ref[t, : pos0 + t + 1].astype(np.float64))


# ---------------------------------------------------------------------------
# selections and the pages' own figures


def test_evenly_spaced_selection_closed_form():
    for pos0, K, T in [(30000, 2051, 40), (8192, 2048, 40), (0, 2048, 70), (2040, 2051, 30)]:
        ids = synth.evenly_spaced_ids(pos0, T, K)
        assert ids.shape[1] == 64 * ((K + 63) // 64)
        for t in range(T):
            p = pos0 + t
            row = ids[t][ids[t] >= 0]
            assert len(row) == min(p + 1, K)
            assert row[0] == 0 and row[-1] == p
            assert np.all(np.diff(row) >= 1)
            assert np.all(ids[t][len(row):] == -1)


def test_mtp_window_composition():
    ids = synth.mtp_window_ids(3000, 8)
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["mtp_partial_bytes"]["window"]
    assert ids.shape[1] == g["max_width"] and ids.shape[1] * 4 == g["staged_ids_bytes"]
    for t in range(8):
        p = 3000 + t
        row = ids[t][ids[t] >= 0]
        assert len(row) == g["width"] == g["sink"] + g["local"] + g["current"]
        assert list(row[:64]) == list(range(64))
        assert list(row[64:320]) == list(range(p - 256, p)) and row[320] == p
        assert (ids[t][320:384] >= 0).sum() == 1        # the sixth chunk holds one cell


def test_pages_partial_record_figures():
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    mtp = g["mtp_partial_bytes"]
    # a record is {chunk max, denominator, partial output[D]}: 2 + D fp32 values per head
    width = mtp["window"]["width"]
    chunks = (width + 63) // 64
    assert chunks == mtp["chunks"]
    assert chunks * mtp["heads"] * mtp["floats_per_record"] * 4 == mtp["bytes"]
    assert 2 * mtp["bytes"] / 1024 == mtp["roundtrip_kib"]
    lg = g["long_partial_buffers"]
    ids = synth.evenly_spaced_ids(lg["pos0"], 4, 2051)
    C = ids.shape[1] // 64
    total = lg["buffers"] * lg["T"] * C * lg["heads"] * (2 + lg["head_dim"]) * 4
    assert abs(total - lg["approx_bytes"]) <= lg["rel_tol"] * lg["approx_bytes"]
    fc = g["long_final_chunk"]
    last = synth.evenly_spaced_ids(fc["pos0"], fc["T"], fc["selected"])
    for t in (0, fc["T"] // 2, fc["T"] - 1):
        assert (last[t, -64:] >= 0).sum() == fc["final_chunk_valid"]
