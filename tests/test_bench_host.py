"""Host logic of bench.py: the one-GPU guard, the algorithmic byte counts the
roofline is computed from, and the rule that a counted traffic figure is used
only for the kernel source it was taken on."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_selection_attention_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_long_context_algorithmic_bytes():
    """Per token: 272 B per valid cell (K and V rows, 8 B of scales each), 256 B
    per chunk of ids, 3072 B of q, and 520 B per (non-empty chunk, head) of
    records; the merge reads the records and writes 3072 B of output. At the
    long-context workload (2051 cells in 33 chunks, all non-empty) that is
    1,538,219,008 B for qsa_attn and 414,640,128 B for qsa_merge."""
    case = synth.long_ctx(layers=1)
    a, c = bench.attn_bytes(case.ids, case.n_cells, case.T, case.H, case.D, case.n_chunks)
    m = bench.merge_bytes(case.T, case.H, case.D, case.n_chunks, c)
    assert np.all(c == 33)
    per_token_attn = 2051 * 272 + 256 * 33 + 2 * 12 * 128 + 12 * (8 * 33 + 4 * 128 * 33)
    per_token_merge = 12 * (8 * 33 + 4 * 128 * 33) + 2 * 12 * 128
    assert a == 1984 * per_token_attn == 1538219008
    assert m == 1984 * per_token_merge == 414640128


def test_bytes_count_only_valid_cells_and_non_empty_chunks():
    T, H, D, C, n_cells = 3, 2, 128, 2, 100
    ids = np.full((T, 64 * C), -1, dtype=np.int32)
    ids[0, :10] = np.arange(10)                      # 10 cells, one chunk
    ids[1, 70] = 5                                   # 1 cell in the second chunk
    ids[1, 71] = n_cells                             # out of range: not a cell
    a, c = bench.attn_bytes(ids, n_cells, T, H, D, C)
    assert list(c) == [1, 1, 0]
    rec = lambda k: H * (8 * C + 4 * D * k)
    assert a == (10 + 1) * 272 + 3 * (256 * C + 2 * H * D) + rec(1) + rec(1) + rec(0)
    assert bench.merge_bytes(T, H, D, C, c) == rec(1) + rec(1) + rec(0) + 3 * 2 * H * D


def test_traffic_is_read_only_for_the_source_it_was_taken_on(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    prof = tmp_path / "p.md"
    prof.write_text("hbm bytes per launch: 12345\nkernel source sha256: %s\n" % bench.src_hash(str(src)))
    assert bench.read_traffic(str(prof), [str(src)]) == 12345
    src.write_text("kernel v2\n")
    assert bench.read_traffic(str(prof), [str(src)]) is None
    assert bench.read_traffic(str(tmp_path / "missing.md"), [str(src)]) is None


def test_minimum_bytes_take_each_selected_cell_once():
    """The roofline's bytes per launch: every distinct selected cell's K and V
    rows and scales once, every id slot, q, and the records; at the long-context
    workload the evenly spaced selections of neighbouring tokens overlap, so the
    distinct cells are far fewer than 1984 x 2051."""
    T, H, D, C, n_cells = 3, 2, 128, 2, 100
    ids = np.full((T, 64 * C), -1, dtype=np.int32)
    ids[0, :10] = np.arange(10)
    ids[1, :10] = np.arange(10)                      # the same cells again
    ids[1, 70] = 50
    ids[2, 3] = n_cells + 7                          # not a cell
    rec = lambda k: H * (8 * C + 4 * D * k)
    assert bench.attn_min_bytes(ids, n_cells, T, H, D, C) == 11 * 272 + T * (256 * C + 2 * H * D) + rec(1) + rec(2) + rec(0)
    case = synth.long_ctx(layers=1)
    a_min = bench.attn_min_bytes(case.ids, case.n_cells, case.T, case.H, case.D, case.n_chunks)
    a, _ = bench.attn_bytes(case.ids, case.n_cells, case.T, case.H, case.D, case.n_chunks)
    uniq = np.unique(case.ids[case.ids >= 0]).size
    assert uniq < case.n_cells and a_min == a - (1984 * 2051 - uniq) * 272
    # 8.5 MB of distinct K/V rows: the chunk records (408 MB) dominate
    assert 430e6 < a_min < 450e6


def test_host_cpu_share(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    threads, visible, model = bench.host_cpu()
    assert threads == min(3, visible) and visible == len(os.sched_getaffinity(0)) and model
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_cpu()[0] == len(os.sched_getaffinity(0))


def test_stats():
    s = bench.stats([3.0, 1.0, 2.0, 10.0])
    assert s == {"n": 4, "median": 2.5, "min": 1.0, "max": 10.0, "mean": 4.0}


def test_gather_model_counts_every_non_empty_wave():
    """The load-instruction model: 8 x 21 + 16 x 21 + 2 x 85 + 4 x 66 + 21 = 959
    address-unit cycles per (token, chunk) wave; at the long-context workload
    (1984 x 33 non-empty waves over 256 CUs at 2.4 GHz) about 102 us."""
    case = synth.long_ctx(layers=1)
    _, c = bench.attn_bytes(case.ids, case.n_cells, case.T, case.H, case.D, case.n_chunks)
    g = bench.attn_gather_model(case.T, c)
    assert g["cycles_per_wave"] == 959
    assert g["waves"] == 1984 * 33
    assert abs(g["us"] - 1984 * 33 / 256 * 959 / 2400.0) < 1e-9
    # an empty chunk issues no gathers, so it costs no modelled cycles
    c2 = c.copy()
    c2[:10] -= 1
    assert bench.attn_gather_model(case.T, c2)["waves"] == g["waves"] - 10
