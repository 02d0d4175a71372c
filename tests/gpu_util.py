"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded inputs.

Tolerances, from the acceptance bar and the arithmetic of the two paths:
  * fp16 attention output: |g - r| <= 2e-3 and |g - r| <= 1e-2 * max(|r|, 1e-2)
    against the oracle's fp64 value (no NaN or Inf allowed);
  * chunk max m: |dm| <= 1e-5 * A, where A = max over the chunk's valid cells of
    |scale| * sum_d |q_d k_d| (the dot products' own magnitude: fp16 x int8
    products are exact and the fp32 sums carry < 40 roundings);
  * denominator l: |dl| <= (2^-11 + 2e-5 * A) * l + 1e-7 (p is rounded to fp16
    once; score errors shift p by at most exp(|dS - dm|));
  * partial output o: |do| <= (2 * 2^-11 + 2e-5 * A) * oabs + 1e-6, where oabs is
    the oracle's sum_j p_j |v_jd| (p and v are each rounded to fp16 once);
  * fp32 scores: |g - r| <= 1e-4 * max(|r|, A) with A = |scale| sum_h sum_d |q k|.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
U16 = 2.0 ** -11

OUT_ATOL = 2e-3
OUT_RTOL = 1e-2
OUT_RFLOOR = 1e-2


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda:0")


def to_dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def sample_tokens(T, n=20, seed=0):
    if T <= n:
        return list(range(T))
    e = min(4, n // 4)
    ends = list(range(e)) + list(range(T - e, T))
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(e, T - e), n - len(ends), replace=False)
    return sorted(set(ends + [int(x) for x in mid]))


def run_attn(layer: synth.Layer, ids, pos0, scale, part_fill=0xFF, ids_dev=None, implicit=False):
    """Run qsa_attn + qsa_merge on the GPU; returns numpy (out, o, m, l) and C."""
    T, H, D = layer.q.shape
    q, kq, vq = to_dev(layer.q), to_dev(layer.kq), to_dev(layer.vq)
    ksc, vsc = to_dev(layer.ksc), to_dev(layer.vsc)
    ids_t = None if implicit else (ids_dev if ids_dev is not None else to_dev(ids))
    C = qsa.chunk_count(ids_t, pos0, T)
    part = qsa.alloc_part(T, H, D, C)
    part.fill_(part_fill)
    qsa.qsa_attn(q, kq, vq, ksc, vsc, ids_t, pos0, float(scale), part)
    out = torch.full((T, H, D), float("nan"), dtype=torch.float16, device=dev())
    qsa.qsa_merge(part, C, out)
    torch.cuda.synchronize()
    o, m, l = qsa.part_views(part, T, H, D, C)
    return out.cpu().numpy(), o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy(), C


def oracle_token(layer, ids, pos0, scale, t):
    """Oracle records and output for one token, computed on that token's row alone."""
    q = layer.q[t: t + 1]
    row = None if ids is None else ids[t: t + 1]
    m, l, o, oabs = oracle.attn_chunks(q, layer.kq, layer.vq, layer.ksc, layer.vsc, row, pos0 + t, scale,
                                       want_abs=True)
    out64, out16 = oracle.merge(m, l, o)
    return dict(m=m[0], l=l[0], o=o[0], oabs=oabs[0], out64=out64[0], out16=out16[0])


def oracle_tokens(layer, ids, pos0, scale, toks):
    with cf.ThreadPoolExecutor(THREADS) as ex:
        res = list(ex.map(lambda t: oracle_token(layer, ids, pos0, scale, t), toks))
    return dict(zip(toks, res))


def chunk_magnitude(layer, ids, pos0, scale, t, C):
    """A per (chunk, head): max over valid cells of |scale| * sum_d |q_d| |k_d|."""
    H = layer.q.shape[1]
    p = pos0 + t
    if ids is None:
        row = np.arange(64 * C)
        row = np.where(row <= p, row, -1)
    else:
        row = ids[t]
    n_cells = layer.kq.shape[0]
    A = np.zeros((C, H))
    qa = np.abs(layer.q[t].astype(np.float64))
    for k in range(C):
        r = row[64 * k: 64 * k + 64]
        cells = r[(r >= 0) & (r < n_cells)]
        if len(cells) == 0:
            continue
        kabs = np.abs(layer.kq[cells].astype(np.float64) * np.repeat(layer.ksc[cells].astype(np.float64), 32, axis=1))
        A[k] = (qa @ kabs.T).max(axis=1) * abs(float(scale))
    return A


def check_out(g16, r64, what=""):
    g = g16.astype(np.float64)
    assert not np.any(np.isnan(g)) and not np.any(np.isinf(g)), "NaN/Inf in output " + what
    err = np.abs(g - r64)
    assert err.max() <= OUT_ATOL, "%s abs err %g" % (what, err.max())
    rel = err / np.maximum(np.abs(r64), OUT_RFLOOR)
    assert rel.max() <= OUT_RTOL, "%s rel err %g" % (what, rel.max())
    return err.max(), rel.max()


def check_records(o, m, l, ref, A, t, what=""):
    """GPU records of one token against the oracle's, chunk by chunk."""
    C_ref = ref["m"].shape[0]
    for k in range(o.shape[0]):
        if k >= C_ref:                       # implicit rows: chunks past the token's own row are empty
            assert np.all(m[k] == -np.inf) and np.all(l[k] == 0), "%s t=%d k=%d" % (what, t, k)
            continue
        rm, rl = ref["m"][k], ref["l"][k]
        if np.all(rm == -np.inf):
            assert np.all(m[k] == -np.inf), "%s t=%d k=%d empty m" % (what, t, k)
            assert np.all(l[k].view(np.uint32) == 0), "%s t=%d k=%d empty l" % (what, t, k)
            continue
        a = A[k]
        assert np.all(np.abs(m[k] - rm) <= 1e-5 * a + 1e-30), "%s t=%d k=%d m" % (what, t, k)
        assert np.all(np.abs(l[k] - rl) <= (U16 + 2e-5 * a) * rl + 1e-7), "%s t=%d k=%d l" % (what, t, k)
        tol = (2 * U16 + 2e-5 * a)[:, None] * ref["oabs"][k] + 1e-6
        assert np.all(np.abs(o[k] - ref["o"][k]) <= tol), "%s t=%d k=%d o err %g" % (
            what, t, k, np.abs(o[k] - ref["o"][k]).max())


def check_attn_case(case: synth.AttnCase, n_sample=20, records=True, implicit=False, seed=0):
    """GPU vs oracle on sampled tokens of every layer of a case."""
    toks = sample_tokens(case.T, n_sample, seed)
    worst = (0.0, 0.0)
    for li, L in enumerate(case.layers):
        out, o, m, l, C = run_attn(L, case.ids, case.pos0, case.scale, implicit=implicit)
        assert not np.any(np.isnan(out)), "NaN output %s layer %d" % (case.name, li)
        refs = oracle_tokens(L, None if implicit else case.ids, case.pos0, case.scale, toks)
        for t in toks:
            r = refs[t]
            e = check_out(out[t], r["out64"], "%s layer %d t=%d" % (case.name, li, t))
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
            if records:
                A = chunk_magnitude(L, None if implicit else case.ids, case.pos0, case.scale, t, C)
                check_records(o[t], m[t], l[t], r, A, t, "%s layer %d" % (case.name, li))
    return worst


def run_score(sc: synth.ScoreCase, fill=np.nan, workspace=None):
    """qsa_score, or qsa_score_ws through `workspace` (a device byte tensor, or
    True for a fresh one filled with a byte pattern rather than zeros)."""
    q, k = to_dev(sc.q), to_dev(sc.k)
    scores = torch.full((sc.T, sc.row_stride), float(fill), dtype=torch.float32, device=dev())
    if workspace is None:
        qsa.qsa_score(q, k, sc.pos0, float(sc.scale), float(sc.dead), scores)
    else:
        if workspace is True:
            workspace = torch.full((max(qsa.qsa_score_ws_bytes(sc.T), 1),), 0xA5, dtype=torch.uint8, device=dev())
        qsa.qsa_score_ws(q, k, sc.pos0, float(sc.scale), float(sc.dead), scores, workspace)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def check_score_case(sc: synth.ScoreCase, n_sample=16, seed=0, workspace=None):
    g = run_score(sc, workspace=workspace)
    T = sc.T
    # extents for every row: causal cells finite, the tail holds `dead`, the rest untouched
    for t in range(T):
        p = sc.pos0 + t
        tail_end = min(64 * ((p + 1 + 63) // 64), sc.row_stride)
        assert np.all(np.isfinite(g[t, : p + 1])), "row %d causal" % t
        if np.isnan(sc.dead):
            assert np.all(np.isnan(g[t, p + 1: tail_end]))
        else:
            assert np.array_equal(g[t, p + 1: tail_end], np.full(tail_end - p - 1, sc.dead, np.float32)), \
                "row %d tail" % t
        assert np.all(np.isnan(g[t, tail_end:])), "row %d untouched" % t
    toks = sample_tokens(T, n_sample, seed)
    qs_abs = np.abs(sc.q.astype(np.float64)).sum(axis=1)          # [T][D]
    kabs = np.abs(sc.k.astype(np.float64))

    def one(t):
        return oracle.score(sc.q[t: t + 1], sc.k, sc.pos0 + t, sc.scale, sc.dead, sc.row_stride)[0]

    with cf.ThreadPoolExecutor(THREADS) as ex:
        refs = list(ex.map(one, toks))
    worst = 0.0
    for t, r in zip(toks, refs):
        p = sc.pos0 + t
        A = abs(float(sc.scale)) * (kabs[: p + 1] @ qs_abs[t])
        err = np.abs(g[t, : p + 1].astype(np.float64) - r[: p + 1])
        lim = 1e-4 * np.maximum(np.abs(r[: p + 1]), A)
        assert np.all(err <= lim), "score row %d: max err/lim %g" % (t, (err / lim).max())
        worst = max(worst, float((err / np.maximum(A, 1e-30)).max()))
    return worst


def run_fused(layer: synth.Layer, ids, pos0, scale, implicit=False):
    """Run qsa_attn_merge on the GPU; returns the fp16 output as numpy."""
    T, H, D = layer.q.shape
    q, kq, vq = to_dev(layer.q), to_dev(layer.kq), to_dev(layer.vq)
    ksc, vsc = to_dev(layer.ksc), to_dev(layer.vsc)
    ids_t = None if implicit else to_dev(ids)
    out = torch.full((T, H, D), float("nan"), dtype=torch.float16, device=dev())
    qsa.qsa_attn_merge(q, kq, vq, ksc, vsc, ids_t, pos0, float(scale), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_fused_case(case: synth.AttnCase, n_sample=20, implicit=False, seed=0):
    """qsa_attn_merge vs the oracle on sampled tokens of every layer of a case."""
    toks = sample_tokens(case.T, n_sample, seed)
    worst = (0.0, 0.0)
    for li, L in enumerate(case.layers):
        out = run_fused(L, case.ids, case.pos0, case.scale, implicit=implicit)
        assert not np.any(np.isnan(out)), "NaN output %s layer %d" % (case.name, li)
        refs = oracle_tokens(L, None if implicit else case.ids, case.pos0, case.scale, toks)
        for t in toks:
            e = check_out(out[t], refs[t]["out64"], "fused %s layer %d t=%d" % (case.name, li, t))
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    return worst
