"""Chunks whose V scales reach 2^9 and above next to scales of 1e-3 and 1e-4.

In such a chunk vq * vsc could leave the fp16 range, so the kernels convert the
V codes times 2^-k and take 2^k back out. The small scales must keep their
precision: rows whose weight sits on small-scale cells are checked at the
plain 2e-3 / 1e-2 bar, on the records kernel, the fused per-token kernel and
both shared-tile kernels. Rows where large-scale cells carry weight are
checked against the fp16 output step plus a bound relative to the magnitude
of the terms (their values also cancel to near zero in some dims)."""
import numpy as np
import pytest

from sparse_selection_attention_amd import synth

from gpu_util import check_out, check_records, chunk_magnitude, oracle_tokens, run_attn, run_fused

pytestmark = pytest.mark.gpu

# large V scales: all at or above 2^9, so every chunk with such a cell takes the
# renormalised path. Where those cells carry weight, their values must stay
# inside the fp16 output range, hence the smaller set.
BIG_HIDDEN = (1000.0, 2.0 ** 14, 600.0, 513.0)
BIG_SHOWN = (512.0, 512.5, 513.0, 515.0)     # 127 * 515 < 65504
SMALL = (1e-3, 1e-4, 2.5e-4, 7e-4)


def mixed_layer(T, H, pos0, seed, hide_big):
    """Every cell c = 5 mod 16 gets large V scales (from BIG_*, in turn, one
    scale group of four per cell), the others small ones (from SMALL). With
    hide_big, q is positive and the large cells' K rows are -127 with scale
    0.5, so their scores are around -570 and their weights underflow: the
    output rests on the small-scale cells."""
    n_cells = pos0 + T
    L = synth.make_layer(seed, 0, T, H, n_cells)
    rng = np.random.default_rng(seed)
    vsc = rng.choice(np.array(SMALL), size=(n_cells, 4)).astype(np.float16)
    big = np.arange(n_cells) % 16 == 5
    bigs = np.array(BIG_HIDDEN if hide_big else BIG_SHOWN, np.float16)
    vsc[big] = bigs[(np.arange(big.sum())[:, None] + np.arange(4)) % 4]
    L.vsc[:] = vsc
    if hide_big:
        L.q[:] = np.abs(L.q)
        L.kq[big] = -127
        L.ksc[big] = np.float16(0.5)
    return L


def merged_magnitude(ref):
    """sum_j p_j |v_j| / L per (head, dim), from the oracle's chunk records: the
    scale of the sum the kernels form, against which fp32 products and sums
    carry their error."""
    m, l, oabs = ref["m"], ref["l"], ref["oabs"]
    live = ~np.isinf(m)
    M = np.where(live, m, -np.inf).max(axis=0)
    w = np.where(live, np.exp(np.where(live, m, 0.0) - M), 0.0)
    L = (w * np.where(live, l, 0.0)).sum(axis=0)
    return (w[..., None] * np.where(live[..., None], oabs, 0.0)).sum(axis=0) / L[:, None]


def _check(out, refs, toks, hide_big, what):
    worst = 0.0
    for t in toks:
        r = refs[t]["out64"]
        if hide_big:
            check_out(out[t], r, "%s t=%d" % (what, t))
        else:
            # values in the thousands that also cancel to near zero in some
            # dims: the fp16 output step (2^-11 of the value), plus fp32
            # product and sum errors against the magnitude of the terms (about
            # 2^-21 of it; the bar allows 2^-17)
            g = out[t].astype(np.float64)
            assert np.all(np.isfinite(g)), "%s t=%d" % (what, t)
            err = np.abs(g - r)
            mag = merged_magnitude(refs[t])
            lim = 2.0 ** -10 * np.abs(r) + 2.0 ** -17 * mag
            assert np.all(err <= lim), "%s t=%d err/lim %g" % (what, t, (err / lim).max())
            worst = max(worst, float(((err - 2.0 ** -10 * np.abs(r)).clip(0) / mag).max()))
    print("%s: worst (err - output rounding) / magnitude %.3g" % (what, worst), flush=True)


@pytest.mark.parametrize("hide_big", [True, False])
@pytest.mark.parametrize("nc,pos0", [(5, 900), (20, 2000)])   # one chunk per wave; several (pipelined fused walk)
def test_explicit_ids_records_and_fused(hide_big, nc, pos0):
    T, H = 24, 12
    L = mixed_layer(T, H, pos0, 41, hide_big)
    rng = np.random.default_rng(2)
    ids = np.full((T, nc * 64), -1, np.int32)
    for t in range(T):
        p = pos0 + t
        width = int(rng.integers(40, nc * 64))
        ids[t, :width] = np.sort(rng.choice(p + 1, width, replace=False))
    scale = synth.SCALE_1_SQRT_128
    out, o, m, l, C = run_attn(L, ids, pos0, scale)
    fout = run_fused(L, ids, pos0, scale)
    toks = list(range(T))
    refs = oracle_tokens(L, ids, pos0, scale, toks)
    _check(out, refs, toks, hide_big, "records+merge")
    _check(fout, refs, toks, hide_big, "fused")
    if hide_big:
        for t in toks:
            check_records(o[t], m[t], l[t], refs[t], chunk_magnitude(L, ids, pos0, scale, t, C), t, "renorm")


@pytest.mark.parametrize("hide_big", [True, False])
def test_implicit_rows_shared_tiles(hide_big):
    T, H, pos0 = 150, 12, 40
    L = mixed_layer(T, H, pos0, 43, hide_big)
    scale = synth.SCALE_1_SQRT_128
    out, o, m, l, C = run_attn(L, None, pos0, scale, implicit=True)
    fout = run_fused(L, None, pos0, scale, implicit=True)
    toks = list(range(T))
    refs = oracle_tokens(L, None, pos0, scale, toks)
    _check(out, refs, toks, hide_big, "tile records+merge")
    _check(fout, refs, toks, hide_big, "tile fused")
