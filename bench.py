#!/usr/bin/env python3
"""Benchmark of the explicit-selection attention path on one MI355X.

Workload: long-context prompt attention -- T=1984 query tokens at pos0=30000,
12 fp16 query heads over one int8 K/V head (head dim 128, per-32 fp16 scales),
up to 2051 evenly spaced causal cells per token in 33 chunks, 3 independent
layers, seed 5. One step is qsa_attn + qsa_merge for each of the 3 layers on
one stream, with every input resident in HBM before the timed region.

Prints one JSON line: query-token*heads per second (whole timed region, and
the median step), per-step median / min / max from HIP events, a cold-cache
sample (the caches scrubbed before each step), the HBM roofline of the
dominant kernel (qsa_attn) with its counted traffic, the single-dispatch
attention + merge, the gated output, the companion causal-score kernel, the
selection producer on its output, the int8 cache writer, the shared-tile
prompt path, the decode window, and the CPU oracle timed on bounded samples
on this host's cores.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA (the score kernel's split products)
FP16_MFMA_PEAK_TFLOPS = 2500.0


def attn_bytes(ids, n_cells, T, H, D, C):
    """Algorithmic bytes of one qsa_attn launch, summed over tokens.

    Per token: K+V rows and their scales once per valid cell (not per head),
    every id slot, the token's q, and one (m, l) pair per chunk plus o[D] per
    non-empty chunk for every head.
    """
    import numpy as np
    v = (ids >= 0) & (ids < n_cells)
    n = v.sum(axis=1)
    c = v.reshape(T, C, 64).any(axis=2).sum(axis=1)
    per = n * (2 * D + 2 * 2 * (D // 32)) + 4 * 64 * C + 2 * H * D + H * (8 * C + 4 * D * c)
    return int(per.sum()), c


def attn_min_bytes(ids, n_cells, T, H, D, C):
    """Fewest HBM bytes one qsa_attn launch can move: every selected cell's K
    and V rows and scales once (however many tokens select it), every id slot,
    q, and the chunk records written. This is the per-token count with the
    K/V term taken per distinct cell of the launch."""
    import numpy as np
    v = (ids >= 0) & (ids < n_cells)
    uniq = int(np.unique(ids[v]).size)
    c = v.reshape(T, C, 64).any(axis=2).sum(axis=1)
    return uniq * (2 * D + 2 * 2 * (D // 32)) + 4 * 64 * C * T + 2 * H * D * T + int((H * (8 * C + 4 * D * c)).sum())


# Address-unit cost of one vector-memory instruction of a 64-lane wave, in CU
# cycles, by access shape (a microbenchmark of random L2-resident rows on gfx950;
# the cost follows the distinct rows each group of four lanes touches)
GATHER_CYCLES = {"16B_lane_8_rows": 21, "8B_lane_4_rows": 21, "8B_lane_16_rows": 66, "8B_lane_64_rows": 85}
CLOCK_GHZ = 2.4


def attn_gather_model(T, c_nonempty, n_cu=256):
    """Lower bound on qsa_attn's time from its load instructions alone: per
    non-empty (token, chunk) wave, 8 K-row copies (16 B per lane, 8 full rows),
    16 V-row loads (8 B per lane, 4 full rows), 2 scale loads (8 B per lane, 64
    rows), 4 q loads (16 rows per instruction, costed as the 16-row shape) and 1
    id load (64 consecutive ids, costed as a full-row shape), spread evenly over
    the CUs. The record stores are not modelled."""
    g = GATHER_CYCLES
    per_wave = (8 * g["16B_lane_8_rows"] + 16 * g["8B_lane_4_rows"] + 2 * g["8B_lane_64_rows"]
                + 4 * g["8B_lane_16_rows"] + 1 * g["16B_lane_8_rows"])
    waves = int(c_nonempty.sum())
    return {"cycles_per_wave": per_wave, "waves": waves, "cus": n_cu, "clock_ghz": CLOCK_GHZ,
            "us": waves / n_cu * per_wave / (CLOCK_GHZ * 1e3)}


def merge_bytes(T, H, D, C, c):
    # reads (m, l) of every chunk and o of non-empty chunks, writes fp16 out
    return int((H * 8 * C + H * 4 * D * c + 2 * H * D).sum()) if hasattr(c, "sum") else None


def src_hash(*paths):
    """sha256 over the concatenated sources a kernel is built from."""
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def attn_sources():
    csrc = os.path.join(ROOT, "sparse_selection_attention_amd", "csrc")
    return [os.path.join(csrc, f) for f in ("qsa_attn.hip", "qsa_device.h", "qsa_internal.h")]


def read_traffic(profile_md, kernel_srcs):
    """HBM bytes per launch from a committed counter summary, if it matches the source."""
    try:
        text = open(profile_md).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel source sha256[^:]*:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm bytes per launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash(*kernel_srcs):
        return None
    return int(m_bytes.group(1))


def host_cpu():
    """(worker threads for the oracle, logical CPUs this process may run on, CPU model).

    The oracle's worker pool takes the CPU share the host gives this process:
    OMP_NUM_THREADS when it is set (the share of one GPU on a shared GPU host),
    else every CPU in the affinity mask."""
    visible = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    threads = max(1, min(visible, share)) if share > 0 else visible
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return threads, visible, model


def _oracle_tokens(case, L, toks, threads):
    """Oracle output of the given tokens, one token per task, on `threads` host threads."""
    import oracle

    def one(t):
        ids = None if case.ids is None else case.ids[t: t + 1]
        m, l, o = oracle.attn_chunks(L.q[t: t + 1], L.kq, L.vq, L.ksc, L.vsc, ids, case.pos0 + t, case.scale)
        return oracle.merge(m, l, o)[0][0]

    t0 = time.perf_counter()
    if threads == 1:
        res = [one(t) for t in toks]
    else:
        with cf.ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(one, toks))
    return res, time.perf_counter() - t0


def cpu_baseline(case, out_gpu, n_tokens, single_tokens):
    """The oracle, as it stands, on bounded samples of the benchmark's workload
    (and single-thread on the tiny and decode-window workloads), on this host."""
    import numpy as np
    from sparse_selection_attention_amd import synth

    threads, visible, model = host_cpu()
    L = case.layers[0]
    toks = np.linspace(0, case.T - 1, n_tokens).astype(int).tolist()
    res, dt = _oracle_tokens(case, L, toks, threads)
    err = max(float(np.abs(out_gpu[t].astype(np.float64) - r).max()) for t, r in zip(toks, res))
    # one thread: a smaller sample of the same layer, and two whole small workloads
    stoks = np.linspace(0, case.T - 1, single_tokens).astype(int).tolist()
    _, dt1 = _oracle_tokens(case, L, stoks, 1)
    single = {"long_context_layer_sample": {
        "tokens": single_tokens, "seconds": dt1, "query-token*heads/s": single_tokens * case.H / dt1,
        "projected_seconds_per_layer": dt1 * case.T / single_tokens}}
    for name, small in (("tiny", synth.tiny()), ("decode_window_8_tokens", synth.mtp(8))):
        _, dts = _oracle_tokens(small, small.layers[0], list(range(small.T)), 1)
        single[name] = {"tokens": small.T, "heads": small.H, "seconds": dts,
                        "query-token*heads/s": small.T * small.H / dts}
    return {
        "value": n_tokens * case.H / dt,
        "unit": "query-token*heads/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d evenly spaced tokens of layer 0 of the same workload (fp64 C oracle, %d threads, %.1f s wall)"
                  % (n_tokens, threads, dt),
        "host": {"cpu_model": model, "logical_cpus_host": os.cpu_count(), "logical_cpus_visible": visible,
                 "threads_used": threads,
                 "why": "the oracle's pool takes this process's CPU share (OMP_NUM_THREADS when set, else the "
                        "affinity mask)"},
        "single_thread": single,
        "max_abs_diff_vs_gpu": err,
    }


def score_errors(sc, scores_gpu, n_rows, threads):
    """Largest score error on sampled rows, against the oracle, as err / A (A the
    dot product's error scale |scale| sum_d |sum_h q_d| |k_d|) and as err / |r|
    over cells with r != 0."""
    import numpy as np
    import oracle

    rows = np.linspace(0, sc.T - 1, n_rows).astype(int).tolist()
    qs = np.abs(sc.q.astype(np.float64).sum(axis=1))
    kabs = np.abs(sc.k.astype(np.float64))

    def one(t):
        r = oracle.score(sc.q[t: t + 1], sc.k, sc.pos0 + t, sc.scale, sc.dead, sc.row_stride)[0]
        p = sc.pos0 + t
        g = scores_gpu[t, : p + 1].astype(np.float64)
        err = np.abs(g - r[: p + 1])
        A = abs(float(sc.scale)) * (kabs[: p + 1] @ qs[t])
        nz = r[: p + 1] != 0
        return float((err / A).max()), float((err[nz] / np.abs(r[: p + 1][nz])).max()), \
            float(np.mean(err[nz] > 1e-4 * np.abs(r[: p + 1][nz])))

    with cf.ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, rows))
    return {"rows_sampled": n_rows, "max_err_over_A": max(r[0] for r in res),
            "max_err_over_abs_r": max(r[1] for r in res),
            "fraction_of_cells_above_1e-4_of_abs_r": float(np.mean([r[2] for r in res])),
            "note": "A = |scale| sum_d |sum_h q[t][h][d]| |k[c][d]|; the bar is err <= 1e-4 max(|r|, A)"}


def stats(xs):
    import numpy as np
    xs = np.asarray(xs, dtype=np.float64)
    return {"n": int(xs.size), "median": float(np.median(xs)), "min": float(xs.min()), "max": float(xs.max()),
            "mean": float(xs.mean())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=3)
    ap.add_argument("--cold-samples", type=int, default=9,
                    help="steps timed after scrubbing L2 and the Infinity Cache (0 to skip)")
    ap.add_argument("--cpu-tokens", type=int, default=384)
    ap.add_argument("--cpu-single-tokens", type=int, default=96)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-score", action="store_true", help="skip the companion score kernel")
    ap.add_argument("--no-fused", action="store_true", help="skip the single-dispatch attention + merge line")
    ap.add_argument("--no-quant", action="store_true", help="skip the int8 cache writer line")
    ap.add_argument("--no-prompt", action="store_true", help="skip the prompt-start (shared tile) line")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-window latency line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU; --gpus %d is not supported (the path would shard by "
              "query token, with no exchange between GPUs)" % args.gpus, file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: run one process on one GPU", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sparse_selection_attention_amd as qsa
    from sparse_selection_attention_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating inputs", file=sys.stderr, flush=True)
    case = synth.long_ctx(layers=args.layers)
    T, H, D, C = case.T, case.H, case.D, case.n_chunks
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    layers = [tuple(up(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc)) for L in case.layers]
    ids = up(case.ids)
    part = qsa.alloc_part(T, H, D, C, device=dev)
    outs = [torch.empty(T, H, D, dtype=torch.float16, device=dev) for _ in range(args.layers)]
    stream = torch.cuda.current_stream()
    scale = float(case.scale)

    a_bytes, c_nonempty = attn_bytes(case.ids, case.n_cells, T, H, D, C)
    a_min = attn_min_bytes(case.ids, case.n_cells, T, H, D, C)
    m_bytes = merge_bytes(T, H, D, C, c_nonempty)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(e=None):
        # e: per layer [start, after attn, after merge] events on the launch stream
        for li, (q, kq, vq, ksc, vsc) in enumerate(layers):
            if e is not None:
                e[li][0].record(stream)
            qsa.qsa_attn(q, kq, vq, ksc, vsc, ids, case.pos0, scale, part, stream=stream)
            if e is not None:
                e[li][1].record(stream)
            qsa.qsa_merge(part, C, outs[li], stream=stream)
            if e is not None:
                e[li][2].record(stream)

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    evs = [[[ev() for _ in range(3)] for _ in range(args.layers)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_us = [1e3 * evs[s_][li][0].elapsed_time(evs[s_][li][1]) for s_ in range(args.steps) for li in range(args.layers)]
    merge_us = [1e3 * evs[s_][li][1].elapsed_time(evs[s_][li][2]) for s_ in range(args.steps) for li in range(args.layers)]
    step_ms = [evs[s_][0][0].elapsed_time(evs[s_][-1][2]) for s_ in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps
    work = T * H * args.layers

    attn_avg_s = float(np.mean(attn_us)) * 1e-6
    merge_avg_s = float(np.mean(merge_us)) * 1e-6
    step_bytes = args.layers * (a_bytes + m_bytes)
    traffic = read_traffic(os.path.join(ROOT, "profiles", "qsa_kernels_hbm_counters_bench_workloads.md"),
                           attn_sources())
    achieved = a_min / attn_avg_s / 1e9

    result = {
        "metric": "query-token*heads/sec + achieved HBM GB/s, T=1984 pos0=30000 attention",
        "value": work / (ms_per_step * 1e-3),
        "unit": "query-token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded SplitMix64: fp16 N(0,1) queries, int8 uniform [-127,127] K/V, "
                "fp16 U[1e-3,2e-2] scales)",
        "config": {
            "workload": "long-context prompt attention: T=1984, pos0=30000, 12 heads, head dim 128, one int8 K/V "
                        "head with per-32 fp16 scales, 2051 evenly spaced causal cells in 33 chunks, %d layers"
                        % args.layers,
            "T": T, "pos0": case.pos0, "heads": H, "head_dim": D, "chunks": C, "selected": 2051,
            "layers": args.layers, "n_cells": case.n_cells,
        },
        # every step of the timed region from HIP events on the launch stream
        "step_ms": stats(step_ms),
        "value_at_median_step": work / (float(np.median(step_ms)) * 1e-3),
        "achieved_gbs": achieved,
        "effective_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "per_token_bytes_per_step": step_bytes,
        "kernels": {
            "qsa_attn": {"us": stats(attn_us), "min_bytes_per_launch": a_min, "per_token_bytes_per_launch": a_bytes,
                         "effective_gbs": a_bytes / attn_avg_s / 1e9},
            "qsa_merge": {"us": stats(merge_us), "bytes_per_launch": m_bytes,
                          "gbs": m_bytes / merge_avg_s / 1e9, "frac": m_bytes / merge_avg_s / 1e9 / HBM_PEAK_GBS},
        },
        # achieved: the fewest HBM bytes one launch can move (each selected cell
        # once, ids, q, chunk records) over the launch's average time; traffic:
        # the counted L2-to-memory bytes (FETCH_SIZE + WRITE_SIZE, calibrated)
        # of the same kernel source, or null when the counters predate it
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": a_min,
            "kernel": "qsa_attn",
            "avg_us": attn_avg_s * 1e6,
            "counted_gbs": None if traffic is None else traffic / attn_avg_s / 1e9,
            "counted_frac": None if traffic is None else traffic / attn_avg_s / 1e9 / HBM_PEAK_GBS,
            "per_token_gbs": a_bytes / attn_avg_s / 1e9,
            # the load instructions' address-unit time, spread evenly over the CUs
            "gather_model": attn_gather_model(T, c_nonempty),
        },
    }

    if args.cold_samples > 0:
        # the caches are scrubbed before each sample by reading a 1 GiB buffer
        # (four times the Infinity Cache), outside the sample's events
        print("bench: %d cold-cache samples" % args.cold_samples, file=sys.stderr, flush=True)
        scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        cold = []
        for _ in range(args.cold_samples):
            float(scrub.sum())
            e = [[ev() for _ in range(3)] for _ in range(args.layers)]
            step(e)
            torch.cuda.synchronize()
            cold.append(e[0][0].elapsed_time(e[-1][2]))
        del scrub
        result["cold_cache"] = {"step_ms": stats(cold),
                                "value_at_median_step": work / (float(np.median(cold)) * 1e-3),
                                "note": "each sample follows a read of 1 GiB that evicts L2 and the Infinity Cache"}

    # the same step with each layer run as two calls of half the tokens: a half's
    # chunk records (204 MB at the long workload) fit in the 256 MB Infinity
    # Cache, so its merge reads them from there
    Th = T // 2
    hpart = qsa.alloc_part(T - Th, H, D, C, device=dev)
    houts = [torch.empty_like(o) for o in outs]

    def half_step():
        for li, (q, kq, vq, ksc, vsc) in enumerate(layers):
            for t0, t1 in ((0, Th), (Th, T)):
                qsa.qsa_attn(q[t0:t1], kq, vq, ksc, vsc, ids[t0:t1], case.pos0 + t0, scale, hpart, stream=stream)
                qsa.qsa_merge(hpart, C, houts[li][t0:t1], stream=stream)

    for _ in range(2):
        half_step()
    torch.cuda.synchronize()
    hev = [[ev(), ev()] for _ in range(args.steps)]
    for s_ in range(args.steps):
        hev[s_][0].record(stream)
        half_step()
        hev[s_][1].record(stream)
    torch.cuda.synchronize()
    h_ms = [e[0].elapsed_time(e[1]) for e in hev]
    result["two_token_halves"] = {
        "step_ms": stats(h_ms),
        "value_at_median_step": work / (float(np.median(h_ms)) * 1e-3),
        "outputs_bitwise_equal": all(bool(torch.equal(a_, b_)) for a_, b_ in zip(outs, houts)),
        "note": "the same three layers, each as qsa_attn + qsa_merge on tokens 0..991 and then 992..1983",
    }
    del hpart, houts

    if not args.no_fused:
        # attention and merge in one dispatch (no chunk records in memory)
        fout = [torch.empty(T, H, D, dtype=torch.float16, device=dev) for _ in range(args.layers)]

        def fstep():
            for li, (q, kq, vq, ksc, vsc) in enumerate(layers):
                qsa.qsa_attn_merge(q, kq, vq, ksc, vsc, ids, case.pos0, scale, fout[li], stream=stream)

        for _ in range(2):
            fstep()
        torch.cuda.synchronize()
        fev = [[ev(), ev()] for _ in range(args.steps)]
        for s_ in range(args.steps):
            fev[s_][0].record(stream)
            fstep()
            fev[s_][1].record(stream)
        torch.cuda.synchronize()
        f_ms = [e[0].elapsed_time(e[1]) for e in fev]
        fdiff = float((fout[0].float() - outs[0].float()).abs().max())
        result["fused_path"] = {
            "entry": "qsa_attn_merge",
            "value": work / (float(np.median(f_ms)) * 1e-3),
            "unit": "query-token*heads/s",
            "step_ms": stats(f_ms),
            "avg_us_per_launch": float(np.mean(f_ms)) * 1e3 / args.layers,
            "max_abs_diff_vs_two_kernel_path": fdiff,
        }
        # the same with the sigmoid gate and the per-16 sums
        gate = up(synth.gates(T, H, seed=5))
        gsum = torch.empty(T, H, D // 16, dtype=torch.float32, device=dev)
        q0, kq0, vq0, ks0, vs0 = layers[0]
        for _ in range(2):
            qsa.qsa_attn_merge_gated(q0, kq0, vq0, ks0, vs0, ids, case.pos0, scale, gate, fout[0], gsum,
                                     stream=stream)
        # gated and plain launches alternate on layer 0, so both see the same
        # cache state and clocks
        gev = [[ev(), ev(), ev()] for _ in range(args.steps)]
        for s_ in range(args.steps):
            gev[s_][0].record(stream)
            qsa.qsa_attn_merge(q0, kq0, vq0, ks0, vs0, ids, case.pos0, scale, fout[1], stream=stream)
            gev[s_][1].record(stream)
            qsa.qsa_attn_merge_gated(q0, kq0, vq0, ks0, vs0, ids, case.pos0, scale, gate, fout[0], gsum,
                                     stream=stream)
            gev[s_][2].record(stream)
        torch.cuda.synchronize()
        g_us = [1e3 * e[1].elapsed_time(e[2]) for e in gev]
        p_us = [1e3 * e[0].elapsed_time(e[1]) for e in gev]
        result["gated_fused_path"] = {"entry": "qsa_attn_merge_gated (fp32 gates, per-16 sums), layer 0",
                                      "us_per_launch": stats(g_us),
                                      "plain_us_per_launch_alternating": stats(p_us),
                                      "gated_over_plain_median": float(np.median(g_us) / np.median(p_us))}
        del fout, gate, gsum

    if not args.no_score:
        sc = synth.score_case(T=T, pos0=case.pos0, Hs=12)
        sq, sk = up(sc.q), up(sc.k)
        scores = torch.empty(T, sc.row_stride, dtype=torch.float32, device=dev)
        # qsa_score, alternating launch by launch with qsa_score_ws (the same
        # scores, q's heads summed once into a workspace by a first pass; both
        # of its kernels inside its timed region)
        ws = torch.empty(qsa.qsa_score_ws_bytes(T), dtype=torch.uint8, device=dev)
        for _ in range(2):
            qsa.qsa_score(sq, sk, sc.pos0, 1.0, float("-inf"), scores, stream=stream)
            qsa.qsa_score_ws(sq, sk, sc.pos0, 1.0, float("-inf"), scores, ws, stream=stream)
        reps = 10
        sev = [[ev(), ev()] for _ in range(reps)]
        wev = [[ev(), ev()] for _ in range(reps)]
        for e, f in zip(sev, wev):
            e[0].record(stream)
            qsa.qsa_score(sq, sk, sc.pos0, 1.0, float("-inf"), scores, stream=stream)
            e[1].record(stream)
            f[0].record(stream)
            qsa.qsa_score_ws(sq, sk, sc.pos0, 1.0, float("-inf"), scores, ws, stream=stream)
            f[1].record(stream)
        torch.cuda.synchronize()
        s_us = [1e3 * e[0].elapsed_time(e[1]) for e in sev]
        w_us = [1e3 * e[0].elapsed_time(e[1]) for e in wev]
        us = float(np.mean(s_us))
        e0, e1 = ev(), ev()
        flops = 2.0 * 128 * sum(case.pos0 + t + 1 for t in range(T))   # heads summed before the contraction
        # the kernel runs each fp32 product as three bf16 products (hi*hi + hi*lo + lo*hi)
        # on the bf16 matrix cores: the roofline is theirs, for the products executed
        executed = 3.0 * flops
        score_bytes = (4.0 * sum(case.pos0 + t + 1 for t in range(T))      # causal scores written
                       + 4.0 * sc.n_cells * 128 + 4.0 * T * 12 * 128)      # K and q read once
        mfma_roof = {"bound": "mfma", "achieved": executed / (us * 1e-6) / 1e12, "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": executed / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
        hbm_roof = {"bound": "hbm", "achieved": score_bytes / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": score_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        # the binding roofline is the one whose lower bound on the time is larger:
        # the scores' write at 8 TB/s outlasts the split products at 2.5 PFLOP/s
        t_mfma = executed / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        t_hbm = score_bytes / (HBM_PEAK_GBS * 1e9)
        result["companion_score"] = {
            "workload": "qsa_score T=1984 pos0=30000 Hs=12",
            "dtype": "fp32 in/out, bf16x3 products (each fp32 product split into bf16 parts, hi*hi + hi*lo + lo*hi, "
                     "fp32 accumulation)",
            "avg_us": us,
            "us": stats(s_us),
            "hbm_gbs": score_bytes / (us * 1e-6) / 1e9,
            "roofline": hbm_roof if t_hbm >= t_mfma else mfma_roof,
            "other_roofline": mfma_roof if t_hbm >= t_mfma else hbm_roof,
            "lower_bound_us": {"hbm": t_hbm * 1e6, "bf16_mfma": t_mfma * 1e6},
        }
        wavg = float(np.mean(w_us))
        ref = torch.full_like(scores, float("nan"))
        alt = torch.full_like(scores, float("nan"))
        qsa.qsa_score(sq, sk, sc.pos0, 1.0, float("-inf"), ref, stream=stream)
        qsa.qsa_score_ws(sq, sk, sc.pos0, 1.0, float("-inf"), alt, ws, stream=stream)
        torch.cuda.synchronize()
        result["companion_score"]["with_workspace"] = {
            "entry": "qsa_score_ws", "workspace_bytes": int(ws.numel()), "avg_us": wavg, "us": stats(w_us),
            "roofline": {"bound": "hbm", "achieved": score_bytes / (wavg * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": score_bytes / (wavg * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "bitwise_equal_to_qsa_score": bool(torch.equal(ref.view(torch.int32), alt.view(torch.int32))),
            "over_qsa_score_median": float(np.median(w_us) / np.median(s_us)),
            "note": "timed alternating launch by launch with qsa_score",
        }
        del ref, alt, ws
        if not args.no_cpu:
            print("bench: score errors against the oracle", file=sys.stderr, flush=True)
            result["companion_score"]["errors"] = score_errors(sc, scores.cpu().numpy(), 24, host_cpu()[0])
        # selection producer on those scores: K = 2051 ids per row (the long-context selection size)
        K_sel = 2051
        sel_stride = 64 * ((K_sel + 63) // 64)
        sel_ids = torch.empty(T, sel_stride, dtype=torch.int32, device=dev)
        for _ in range(2):
            qsa.qsa_select(scores, sc.pos0, K_sel, sel_ids, stream=stream)
        e0.record(stream)
        for _ in range(reps):
            qsa.qsa_select(scores, sc.pos0, K_sel, sel_ids, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us_sel = e0.elapsed_time(e1) * 1e3 / reps
        sel_bytes = 4.0 * sum(sc.pos0 + t + 1 for t in range(T)) + 4.0 * T * sel_stride
        result["selection_producer"] = {
            "entry": "qsa_select",
            "workload": "top-2051 of the causal scores of 1984 rows at pos0=30000 (qsa_score's output)",
            "avg_us": us_sel,
            "roofline": {"bound": "hbm", "achieved": sel_bytes / (us_sel * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": sel_bytes / (us_sel * 1e-6) / 1e9 / HBM_PEAK_GBS},
        }
        del scores, sel_ids

    if not args.no_quant:
        # int8 cache writer: fp32 K and V rows -> int8 rows + per-32 fp16 scales.
        # Algorithmic bytes per row pair: 2 x 512 read + 2 x (128 + 8) written.
        def time_quant(rows, reps):
            xk = up(synth.cache_rows(rows, which=0))
            xv = up(synth.cache_rows(rows, which=1))
            ckq = torch.empty(rows, D, dtype=torch.int8, device=dev)
            cvq = torch.empty_like(ckq)
            cks = torch.empty(rows, D // 32, dtype=torch.float16, device=dev)
            cvs = torch.empty_like(cks)
            for _ in range(2):
                qsa.qsa_quant_append(xk, xv, ckq, cvq, cks, cvs, 0, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                qsa.qsa_quant_append(xk, xv, ckq, cvq, cks, cvs, 0, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            return us, rows * 2 * (4 * D + D + 2 * (D // 32))

        big_rows = 1 << 18
        us_big, b_big = time_quant(big_rows, 20)
        us_layer, b_layer = time_quant(case.n_cells, 50)
        us_prompt, _ = time_quant(T, 50)
        gbs = b_big / (us_big * 1e-6) / 1e9
        result["cache_producer"] = {
            "entry": "qsa_quant_append",
            "workload": "262144 K and V rows (a 256k-cell cache, 340 MB moved, more than the Infinity Cache holds)",
            "avg_us": us_big,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS},
            "long_context_layer_31984_rows_us": us_layer,
            "long_context_layer_gbs": b_layer / (us_layer * 1e-6) / 1e9,
            "prompt_1984_rows_us": us_prompt,
        }

    if not args.no_prompt:
        # prompt start: T=1984 at pos0=0, every causal cell (implicit rows). Blocks of
        # (token, head) rows share each chunk's cells: QK and PV run as MFMA tiles.
        pc = synth.prompt_start(implicit=True)
        pe = synth.prompt_start(implicit=False)
        PL = pc.layers[0]
        pq, pkq, pvq, pks, pvs = up(PL.q), up(PL.kq), up(PL.vq), up(PL.ksc), up(PL.vsc)
        pids = up(pe.ids)
        pC = pc.n_chunks
        ppart = qsa.alloc_part(pc.T, pc.H, D, pC, device=dev)
        pout = torch.empty(pc.T, pc.H, D, dtype=torch.float16, device=dev)

        def time_it(fn, reps=20):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        def two_kernel():
            qsa.qsa_attn(pq, pkq, pvq, pks, pvs, None, 0, float(pc.scale), ppart, stream=stream)
            qsa.qsa_merge(ppart, pC, pout, stream=stream)

        us_fused = time_it(lambda: qsa.qsa_attn_merge(pq, pkq, pvq, pks, pvs, None, 0, float(pc.scale), pout,
                                                      stream=stream))
        us_two = time_it(two_kernel)
        us_expl = time_it(lambda: qsa.qsa_attn_merge(pq, pkq, pvq, pks, pvs, pids, 0, float(pc.scale), pout,
                                                     stream=stream))
        # causal QK and PV: 2 x 2 x D flops per (token, head, selected cell)
        pflops = 4.0 * D * pc.H * sum(pc.pos0 + t + 1 for t in range(pc.T))
        tf = pflops / (us_fused * 1e-6) / 1e12
        result["prompt_tiles"] = {
            "workload": "prompt start: T=1984, pos0=0, 12 heads, every causal cell (implicit rows), one layer",
            "entry": "qsa_attn_merge (ids NULL)",
            "avg_us": us_fused,
            "value": pc.T * pc.H / (us_fused * 1e-6),
            "unit": "query-token*heads/s",
            "roofline": {"bound": "mfma", "achieved": tf, "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / FP16_MFMA_PEAK_TFLOPS},
            "two_kernel_us": us_two,
            "explicit_rows_per_token_kernel_us": us_expl,
        }
        del ppart

    if not args.no_decode:
        # decode: ntok tokens at pos0=3000 over the 321-cell window (64 sink + 256
        # local + current), 12 heads: latency of one call, fused and two-kernel
        lat = {}
        for ntok in (1, 2, 4, 8):
            mc = synth.mtp(ntok)
            ML = mc.layers[0]
            mq, mkq, mvq, mks, mvs = up(ML.q), up(ML.kq), up(ML.vq), up(ML.ksc), up(ML.vsc)
            mids = up(mc.ids)
            mout = torch.empty(ntok, mc.H, D, dtype=torch.float16, device=dev)
            mpart = qsa.alloc_part(ntok, mc.H, D, mc.n_chunks, device=dev)

            def fused():
                qsa.qsa_attn_merge(mq, mkq, mvq, mks, mvs, mids, mc.pos0, float(mc.scale), mout, stream=stream)

            def two():
                qsa.qsa_attn(mq, mkq, mvq, mks, mvs, mids, mc.pos0, float(mc.scale), mpart, stream=stream)
                qsa.qsa_merge(mpart, mc.n_chunks, mout, stream=stream)

            row = {}
            for name, fn in (("fused_us", fused), ("two_kernel_us", two)):
                for _ in range(5):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(100):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                row[name] = e0.elapsed_time(e1) * 1e3 / 100

            # the same 100 calls captured in one HIP graph and replayed: the
            # per-call time without the host's launch cost
            def fused_cur():
                qsa.qsa_attn_merge(mq, mkq, mvq, mks, mvs, mids, mc.pos0, float(mc.scale), mout)

            def two_cur():
                qsa.qsa_attn(mq, mkq, mvq, mks, mvs, mids, mc.pos0, float(mc.scale), mpart)
                qsa.qsa_merge(mpart, mc.n_chunks, mout)

            for name, fn in (("fused_graph_us", fused_cur), ("two_kernel_graph_us", two_cur)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(100):
                        fn()
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                row[name] = e0.elapsed_time(e1) * 1e3 / 100
                del g
            lat["ntok_%d" % ntok] = row
        result["decode_latency"] = {
            "workload": "decode window: ntok tokens at pos0=3000, 321 cells (64 sink + 256 local + current), 12 heads, "
                        "back-to-back calls on one stream; *_graph_us: the same calls captured in one HIP graph "
                        "of 100 and replayed",
            **lat,
        }

    if args.copy_calibration:
        # one elementwise kernel that reads n bytes and writes n bytes
        # (its input is first pushed out of L2 and the Infinity Cache by reading a
        # larger buffer, so no dirty lines are written back while the copy runs)
        n = args.copy_calibration << 20
        flush = torch.full((3 * n // 4,), 2.0, dtype=torch.float32, device=dev)
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        flush.sum()
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del flush
        result["copy_calibration_bytes"] = n

    if not args.no_cpu:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, outs[0].cpu().numpy(), args.cpu_tokens, args.cpu_single_tokens)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
