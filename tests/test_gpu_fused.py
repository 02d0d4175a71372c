"""GPU parity of qsa_attn_merge (attention and merge in one dispatch) against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest

from sparse_selection_attention_amd import synth

from gpu_util import (check_fused_case, check_out, oracle_token, oracle_tokens, run_attn, run_fused)
from test_gpu_attn import probe_case

pytestmark = pytest.mark.gpu


def test_fused_tiny_all_tokens():
    case = synth.tiny()
    out = run_fused(case.layers[0], case.ids, case.pos0, case.scale)
    for t in range(case.T):
        r = oracle_token(case.layers[0], case.ids, case.pos0, case.scale, t)
        check_out(out[t], r["out64"], "fused tiny t=%d" % t)


@pytest.mark.parametrize("ntok", range(1, 9))
def test_fused_mtp_decode_window(ntok):
    print("fused mtp", ntok, check_fused_case(synth.mtp(ntok)), flush=True)


def test_fused_prompt_start_explicit_and_implicit():
    case = synth.prompt_start()
    print("fused prompt", check_fused_case(case, n_sample=12), flush=True)
    print("fused prompt implicit", check_fused_case(case, n_sample=12, implicit=True), flush=True)


def test_fused_mid_context_three_layers():
    print("fused mid", check_fused_case(synth.mid(layers=3), n_sample=10), flush=True)


def test_fused_long_context_three_layers():
    print("fused long", check_fused_case(synth.long_ctx(layers=3), n_sample=10), flush=True)


@pytest.mark.parametrize("variant", ["signed_zero", "cancel"])
def test_fused_long_context_edge_variants(variant):
    case = synth.long_ctx(layers=1, variant=variant)
    L = case.layers[0]
    out = run_fused(L, case.ids, case.pos0, case.scale)
    toks = [0, 4] if variant == "signed_zero" else [1, 5]
    heads = [0, 6] if variant == "signed_zero" else list(range(12))
    for t in toks:
        row = case.ids[t]
        cells = row[row >= 0]
        mean = (L.vq[cells].astype(np.float64) * np.repeat(L.vsc[cells].astype(np.float64), 32, axis=1)).mean(0)
        for h in heads:
            check_out(out[t, h], mean, "fused %s t=%d h=%d" % (variant, t, h))


def test_fused_matches_two_kernel_path():
    """Both paths approximate the same values; they agree far inside the output tolerance."""
    case = synth.long_ctx(layers=1, T=256)
    L = case.layers[0]
    a = run_attn(L, case.ids, case.pos0, case.scale)[0].astype(np.float64)
    b = run_fused(L, case.ids, case.pos0, case.scale).astype(np.float64)
    assert np.abs(a - b).max() <= 2e-4


def test_fused_probe_case_all_tokens():
    L, ids, pos0 = probe_case(seed=11)
    out = run_fused(L, ids, pos0, synth.SCALE_1_SQRT_128)
    refs = oracle_tokens(L, ids, pos0, synth.SCALE_1_SQRT_128, list(range(ids.shape[0])))
    for t, r in refs.items():
        check_out(out[t], r["out64"], "fused probe t=%d" % t)
    assert np.all(out[7].view(np.uint16) == 0)    # the row with no valid slot is +0


@pytest.mark.parametrize("T", [150, 40])          # 4 waves (5 chunks each) and 8 waves (2 or 3 each)
def test_fused_walk_over_empty_chunks(T):
    """Rows of 20 chunks, so each wave walks several and issues the next
    chunk's reads during the current one. Whole chunks are empty at the start
    of a wave's walk, in the middle, several in a row, and at the end; one row
    has no valid slot and another a single one. Every token against the oracle."""
    L, ids, pos0 = probe_case(T=T, C=20, n_cells=2000, seed=17, p_poison=0.2)
    for c in (0, 5, 6, 7, 13, 19):               # empty chunks in every row
        ids[:, 64 * c: 64 * c + 64] = -1
    ids[11, :] = -1                              # a row with no valid slot
    ids[12, :] = -1
    ids[12, 64 * 9 + 3] = 77                     # a row with one cell
    out = run_fused(L, ids, pos0, synth.SCALE_1_SQRT_128)
    refs = oracle_tokens(L, ids, pos0, synth.SCALE_1_SQRT_128, list(range(T)))
    for t, r in refs.items():
        check_out(out[t], r["out64"], "fused empty-chunk walk T=%d t=%d" % (T, t))
    assert np.all(out[11].view(np.uint16) == 0)
    rec = run_attn(L, ids, pos0, synth.SCALE_1_SQRT_128)[0]
    assert np.abs(rec.astype(np.float64) - out.astype(np.float64)).max() <= 2e-4


def test_fused_one_cell_selection_is_bitwise():
    T, H, n_cells = 64, 12, 300
    L = synth.make_layer(4, 0, T, H, n_cells)
    rng = np.random.default_rng(1)
    ids = np.full((T, 320), -1, dtype=np.int32)
    cells = rng.integers(0, n_cells - T, T)
    ids[np.arange(T), rng.integers(0, 320, T)] = cells
    out = run_fused(L, ids, n_cells - T, synth.SCALE_1_SQRT_128)
    v = L.vq[cells].astype(np.float64) * np.repeat(L.vsc[cells].astype(np.float64), 32, axis=1)
    assert np.array_equal(out.view(np.uint16), np.repeat(v.astype(np.float16)[:, None, :], H, axis=1).view(np.uint16))


@pytest.mark.parametrize("T", [150, 40])          # a prompt-sized and a decode-sized token count
def test_fused_poison_and_unselected_data_do_not_matter(T):
    L, ids, pos0 = probe_case(T=T, seed=12)
    n_cells = L.kq.shape[0]
    a = run_fused(L, ids, pos0, synth.SCALE_1_SQRT_128)
    used = np.zeros(n_cells, bool)
    used[ids[(ids >= 0) & (ids < n_cells)]] = True
    L2 = synth.Layer(L.q.copy(), L.kq.copy(), L.vq.copy(), L.ksc.copy(), L.vsc.copy())
    L2.kq[~used] = -127
    L2.vq[~used] = 127
    L2.ksc[~used] = 30000.0
    L2.vsc[~used] = 500.0
    ids2 = ids.copy()
    ids2[(ids2 < 0) | (ids2 >= n_cells)] = -1
    b = run_fused(L2, ids2, pos0, synth.SCALE_1_SQRT_128)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("T", [150, 40])
def test_fused_determinism(T):
    L, ids, pos0 = probe_case(T=T, seed=13)
    a = run_fused(L, ids, pos0, synth.SCALE_1_SQRT_128)
    b = run_fused(L, ids, pos0, synth.SCALE_1_SQRT_128)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("T,H,n_cells,pos0", [(1, 1, 1, 0), (1, 16, 65, 64), (5, 7, 130, 125), (70, 16, 200, 130),
                                             (33, 2, 64, 31), (3, 12, 250, 247)])
def test_fused_edge_shapes_implicit_rows(T, H, n_cells, pos0):
    L = synth.make_layer(T + H + 1, 0, T, H, n_cells)
    out = run_fused(L, None, pos0, synth.SCALE_1_SQRT_128, implicit=True)
    for t in range(T):
        r = oracle_token(L, None, pos0, synth.SCALE_1_SQRT_128, t)
        check_out(out[t], r["out64"], "fused edge t=%d" % t)


def test_fused_large_and_tiny_scales():
    L, ids, pos0 = probe_case(T=40, seed=14)
    base = L.vsc.astype(np.float32)
    L.vsc[:] = (base * 10000).astype(np.float16)
    L.vsc[::3] = (base[::3] * 1e-3).astype(np.float16)
    L.ksc[:5] = np.float16(2.0 ** -24)
    L.q[:] = (L.q.astype(np.float32) * 40).astype(np.float16)
    out = run_fused(L, ids, pos0, np.float32(1.0))
    refs = oracle_tokens(L, ids, pos0, np.float32(1.0), list(range(40)))
    for t, r in refs.items():
        scale_out = max(1.0, float(np.abs(r["out64"]).max()))
        g = out[t].astype(np.float64)
        assert np.all(np.isfinite(g))
        assert np.abs(g - r["out64"]).max() <= 2e-3 * scale_out


@pytest.mark.parametrize("C,H,T", [(c, 12, 12) for c in range(1, 11)] + [(8, 16, 12), (8, 1, 12), (9, 16, 12)]
                         + [(9, 12, 65), (11, 16, 65), (17, 3, 64), (17, 3, 65)])
def test_fused_chunk_counts_and_wave_counts(C, H, T):
    """Rows of 1 to 8 chunks run one wave per chunk (8 waves and 16 heads is
    the largest LDS footprint, about 80 KB); longer rows run eight waves that
    each walk several chunks in calls of at most 64 tokens, four waves in
    larger calls: sampled tokens against the oracle, and three runs bitwise
    equal."""
    L, ids, pos0 = probe_case(T=T, H=H, C=C, seed=40 + C + H + T)
    outs = [run_fused(L, ids, pos0, synth.SCALE_1_SQRT_128) for _ in range(3)]
    assert all(np.array_equal(outs[0].view(np.uint16), o.view(np.uint16)) for o in outs[1:])
    toks = list(range(12)) + [T - 2, T - 1] if T > 12 else list(range(T))
    refs = oracle_tokens(L, ids, pos0, synth.SCALE_1_SQRT_128, toks)
    for t, r in refs.items():
        check_out(outs[0][t], r["out64"], "fused C=%d H=%d T=%d t=%d" % (C, H, T, t))


@pytest.mark.parametrize("T", [1, 8, 64, 65])
def test_fused_long_selection_small_calls(T):
    """Decode-sized calls over 2051 selected cells (33 chunks) at pos0 = 30000:
    eight waves walk the chunks up to 64 tokens, four from 65; against the
    oracle, and two runs bitwise equal."""
    case = synth.long_ctx(layers=1, T=T)
    L = case.layers[0]
    a = run_fused(L, case.ids, case.pos0, case.scale)
    b = run_fused(L, case.ids, case.pos0, case.scale)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    toks = sorted({0, T // 2, T - 1})
    refs = oracle_tokens(L, case.ids, case.pos0, case.scale, toks)
    for t, r in refs.items():
        check_out(a[t], r["out64"], "fused long T=%d t=%d" % (T, t))
