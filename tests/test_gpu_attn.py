"""GPU parity of qsa_attn + qsa_merge against the CPU oracle, through the C ABI.

Covers the five workloads at their full sizes (tokens sampled for the oracle),
and the bit-exact probes of id and selection handling."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

from gpu_util import (check_attn_case, check_out, check_records, chunk_magnitude, dev, oracle_token,
                      oracle_tokens, run_attn, run_fused, to_dev)

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# the five workloads


def test_tiny_all_tokens():
    case = synth.tiny()
    L = case.layers[0]
    out, o, m, l, C = run_attn(L, case.ids, case.pos0, case.scale)
    for t in range(case.T):
        r = oracle_token(L, case.ids, case.pos0, case.scale, t)
        check_out(out[t], r["out64"], "tiny t=%d" % t)
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, case.ids, case.pos0, case.scale, t, C), t, "tiny")


@pytest.mark.parametrize("ntok", range(1, 9))
def test_mtp_decode_window(ntok):
    case = synth.mtp(ntok)
    _print("mtp ntok", ntok, check_attn_case(case))


def test_prompt_start_explicit():
    _print("prompt", check_attn_case(synth.prompt_start(), n_sample=16))


def test_prompt_start_implicit_rows_match_explicit():
    """Implicit rows run on the shared-tile kernel, explicit ones on the per-token
    kernel: the same selection (empty records bit for bit), the same outputs and
    records within tolerance, on every token."""
    case = synth.prompt_start()
    L = case.layers[0]
    a = run_attn(L, case.ids, case.pos0, case.scale)
    b = run_attn(L, None, case.pos0, case.scale, implicit=True)
    assert a[4] == b[4]
    empty_a, empty_b = np.isinf(a[2]), np.isinf(b[2])
    assert np.array_equal(empty_a, empty_b)
    assert np.all(b[2][empty_b] == -np.inf) and np.all(b[3][empty_b].view(np.uint32) == 0)
    for t in range(case.T):
        check_out(b[0][t], a[0][t].astype(np.float64), "implicit vs explicit t=%d" % t)
    ne = ~empty_a
    assert np.all(np.abs(a[2][ne] - b[2][ne]) <= 1e-4 * np.maximum(1.0, np.abs(a[2][ne])))
    assert np.all(np.abs(a[3][ne] - b[3][ne]) <= 2e-3 * a[3][ne])


def test_prompt_start_implicit_vs_oracle():
    _print("prompt implicit", check_attn_case(synth.prompt_start(), n_sample=12, implicit=True))


def test_mid_context_three_layers():
    _print("mid", check_attn_case(synth.mid(layers=3), n_sample=12))


def test_long_context_three_layers():
    _print("long", check_attn_case(synth.long_ctx(layers=3), n_sample=12))


@pytest.mark.parametrize("name", ["mid", "long"])
def test_every_token_of_layer0(name):
    """Every one of the 1984 tokens of layer 0, on the records path (records
    and merged output) and on the fused path, against the oracle; the
    three-layer tests above sample layers 1 and 2."""
    import concurrent.futures as cf
    from gpu_util import THREADS
    case = synth.mid(layers=1) if name == "mid" else synth.long_ctx(layers=1)
    L = case.layers[0]
    out, o, m, l, C = run_attn(L, case.ids, case.pos0, case.scale)
    fout = run_fused(L, case.ids, case.pos0, case.scale)
    toks = list(range(case.T))
    refs = oracle_tokens(L, case.ids, case.pos0, case.scale, toks)

    def one(t):
        r = refs[t]
        e1 = check_out(out[t], r["out64"], "%s records path t=%d" % (name, t))
        e2 = check_out(fout[t], r["out64"], "%s fused t=%d" % (name, t))
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, case.ids, case.pos0, case.scale, t, C), t, name)
        return max(e1[0], e2[0]), max(e1[1], e2[1])

    with cf.ThreadPoolExecutor(THREADS) as ex:
        errs = list(ex.map(one, toks))
    _print("%s layer 0, all %d tokens: worst abs %.3g rel %.3g" % (name, case.T, max(e[0] for e in errs),
                                                                  max(e[1] for e in errs)))


@pytest.mark.parametrize("variant", ["signed_zero", "cancel"])
def test_long_context_edge_variants(variant):
    case = synth.long_ctx(layers=1, variant=variant)
    L = case.layers[0]
    out, o, m, l, C = run_attn(L, case.ids, case.pos0, case.scale)
    toks = [0, 4, 1980] if variant == "signed_zero" else [1, 5, 1981]
    heads = [0, 6] if variant == "signed_zero" else list(range(12))
    refs = oracle_tokens(L, case.ids, case.pos0, case.scale, toks + [2, 3])
    for t in toks:
        row = case.ids[t]
        cells = row[row >= 0]
        mean = (L.vq[cells].astype(np.float64) * np.repeat(L.vsc[cells].astype(np.float64), 32, axis=1)).mean(0)
        for h in heads:
            assert np.all(m[t, :, h] == 0.0), "scores must be exactly +-0"
            assert np.all(l[t, :32, h] == 64.0) and l[t, 32, h] == 3.0
            check_out(out[t, h], mean, "%s t=%d h=%d" % (variant, t, h))
        check_out(out[t], refs[t]["out64"], "%s t=%d" % (variant, t))
    for t in (2, 3):                             # untouched tokens keep plain parity
        check_out(out[t], refs[t]["out64"], "%s t=%d" % (variant, t))


# ---------------------------------------------------------------------------
# bit-exact probes of ids and selection


def probe_case(T=150, H=12, n_cells=700, C=5, seed=1, p_poison=0.3):
    rng = np.random.default_rng(seed)
    L = synth.make_layer(seed, 0, T, H, n_cells)
    pos0 = n_cells - T
    ids = np.full((T, 64 * C), -1, dtype=np.int32)
    for t in range(T):
        p = pos0 + t
        row = rng.integers(0, p + 1, 64 * C)
        row[rng.random(64 * C) < p_poison] = -1
        bad = rng.random(64 * C) < 0.03
        row[bad] = rng.choice([n_cells, n_cells + 999, -2, -(2 ** 31)], bad.sum())
        ids[t] = row
    ids[3, 64:128] = -1                          # an empty chunk
    ids[7, :] = -1                               # an empty row
    ids[9, -64:] = -1
    ids[9, -64 + 17] = 5                         # a lone cell in the ragged last chunk
    return L, ids, pos0


def valid_counts(ids, n_cells):
    T, S = ids.shape
    v = (ids >= 0) & (ids < n_cells)
    return v.reshape(T, S // 64, 64).sum(axis=2)


def test_uniform_probe_records_are_exact():
    """q = 1, K = 0, unit V scales: l counts the valid slots, o sums the selected V rows."""
    L, ids, pos0 = probe_case()
    L.q[:] = 1.0
    L.kq[:] = 0
    L.vsc[:] = 1.0
    n_cells = L.kq.shape[0]
    out, o, m, l, C = run_attn(L, ids, pos0, np.float32(0.3))
    cnt = valid_counts(ids, n_cells)
    H = L.q.shape[1]
    assert np.array_equal(l, np.repeat(cnt[:, :, None], H, axis=2).astype(np.float32))
    ne = cnt > 0
    assert np.all(m[ne] == 0.0) and np.all(m[~ne] == -np.inf)
    for t in range(ids.shape[0]):
        for k in range(C):
            r = ids[t, 64 * k: 64 * k + 64]
            cells = r[(r >= 0) & (r < n_cells)]
            if len(cells):
                s = L.vq[cells].astype(np.int64).sum(0).astype(np.float32)
                assert np.array_equal(o[t, k], np.broadcast_to(s, (H, 128))), (t, k)


def test_uniform_probe_full_long_selection():
    """The same probe over the full long-context selection: every chunk's count is exact."""
    case = synth.long_ctx(layers=1)
    L = case.layers[0]
    L.q[:] = 1.0
    L.kq[:] = 0
    L.vsc[:] = 1.0
    out, o, m, l, C = run_attn(L, case.ids, case.pos0, case.scale)
    cnt = valid_counts(case.ids, case.n_cells)
    assert np.array_equal(l, np.repeat(cnt[:, :, None], 12, axis=2).astype(np.float32))
    assert np.all(m == 0.0)
    for t in (0, 777, 1983):
        for k in (0, 17, 32):
            r = case.ids[t, 64 * k: 64 * k + 64]
            s = L.vq[r[r >= 0]].astype(np.int64).sum(0).astype(np.float32)
            assert np.array_equal(o[t, k], np.broadcast_to(s, (12, 128)))


def test_k_address_probe_max_is_exact():
    L, ids, pos0 = probe_case(H=3, seed=2)
    d0 = 93
    n_cells = L.kq.shape[0]
    L.q[:] = 0.0
    L.q[:, :, d0] = 1.0
    L.ksc[:] = 1.0
    L.kq[:, d0] = ((np.arange(n_cells) * 2654435761) % 255 - 127).astype(np.int8)
    out, o, m, l, C = run_attn(L, ids, pos0, np.float32(1.0))
    for t in range(ids.shape[0]):
        for k in range(C):
            r = ids[t, 64 * k: 64 * k + 64]
            cells = r[(r >= 0) & (r < n_cells)]
            want = L.kq[cells, d0].astype(np.float32).max() if len(cells) else -np.inf
            assert np.all(m[t, k] == want), (t, k)


def test_one_cell_selection_is_bitwise_dequantised_v():
    T, H, n_cells = 64, 12, 300
    L = synth.make_layer(4, 0, T, H, n_cells)
    rng = np.random.default_rng(0)
    ids = np.full((T, 192), -1, dtype=np.int32)
    cells = rng.integers(0, n_cells - T, T)
    slots = rng.integers(0, 192, T)
    ids[np.arange(T), slots] = cells
    out, o, m, l, C = run_attn(L, ids, n_cells - T, synth.SCALE_1_SQRT_128)
    v = (L.vq[cells].astype(np.float64) * np.repeat(L.vsc[cells].astype(np.float64), 32, axis=1))
    want = v.astype(np.float16)
    assert np.array_equal(out.view(np.uint16), np.repeat(want[:, None, :], H, axis=1).view(np.uint16))


def test_poison_and_unselected_data_do_not_matter():
    L, ids, pos0 = probe_case(seed=3)
    n_cells = L.kq.shape[0]
    a = run_attn(L, ids, pos0, synth.SCALE_1_SQRT_128)
    used = np.zeros(n_cells, bool)
    v = ids[(ids >= 0) & (ids < n_cells)]
    used[v] = True
    L2 = synth.Layer(L.q.copy(), L.kq.copy(), L.vq.copy(), L.ksc.copy(), L.vsc.copy())
    L2.kq[~used] = 127
    L2.vq[~used] = -127
    L2.ksc[~used] = 60000.0
    L2.vsc[~used] = 1000.0
    ids2 = ids.copy()
    ids2[(ids2 < 0) | (ids2 >= n_cells)] = -1
    b = run_attn(L2, ids2, pos0, synth.SCALE_1_SQRT_128)
    assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
    assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))


def test_empty_chunk_and_row():
    L, ids, pos0 = probe_case(seed=4)
    out, o, m, l, C = run_attn(L, ids, pos0, synth.SCALE_1_SQRT_128, part_fill=0x7F)
    sentinel = np.array([0x7F7F7F7F], np.uint32).view(np.float32)[0]
    assert np.all(m[3, 1] == -np.inf) and np.all(l[3, 1].view(np.uint32) == 0)
    assert np.all(o[3, 1] == sentinel)            # o of an empty chunk is not written
    assert np.all(m[7] == -np.inf)
    assert np.all(out[7].view(np.uint16) == 0)    # a row with no valid slot is +0
    r = oracle_token(L, ids, pos0, synth.SCALE_1_SQRT_128, 9)
    check_out(out[9], r["out64"], "ragged lone cell")


def test_run_to_run_determinism():
    L, ids, pos0 = probe_case(seed=5)
    a = run_attn(L, ids, pos0, synth.SCALE_1_SQRT_128)
    b = run_attn(L, ids, pos0, synth.SCALE_1_SQRT_128)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("H,T", [(12, 700), (5, 1700)])
def test_large_call_records_match_small_calls(H, T):
    """A call whose records exceed 128 MB stores them nontemporal; a small call
    stores them cached. Both write each record in whole 1 KB runs. The records
    and outputs of the tokens a small call covers must be bitwise equal to the
    large call's (a token's records depend on its own row only). H = 5 leaves
    half of each record's last run unused."""
    pos0, K, D = 30000, 2051, 128
    L = synth.make_layer(7, 0, T, H, pos0 + T)
    ids = synth.evenly_spaced_ids(pos0, T, K)
    C = ids.shape[1] // 64
    assert T * C * H * D * 4 > (128 << 20)
    q, kq, vq, ksc, vsc = (to_dev(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc))
    ids_d = to_dev(ids)
    scale = float(synth.SCALE_1_SQRT_128)
    big = qsa.alloc_part(T, H, D, C)
    big.fill_(0xFF)
    out_big = torch.empty(T, H, D, dtype=torch.float16, device=dev())
    qsa.qsa_attn(q, kq, vq, ksc, vsc, ids_d, pos0, scale, big)
    qsa.qsa_merge(big, C, out_big)
    ob, mb, lb = qsa.part_views(big, T, H, D, C)
    for t0 in (0, T // 2 - 37, T - 64):
        n = 64
        small = qsa.alloc_part(n, H, D, C)
        small.fill_(0xFF)
        out_s = torch.empty(n, H, D, dtype=torch.float16, device=dev())
        qsa.qsa_attn(q[t0:t0 + n], kq, vq, ksc, vsc, ids_d[t0:t0 + n], pos0 + t0, scale, small)
        qsa.qsa_merge(small, C, out_s)
        os_, ms, ls = qsa.part_views(small, n, H, D, C)
        torch.cuda.synchronize()
        _print("large vs small call: H=%d T=%d tokens %d..%d" % (H, T, t0, t0 + n - 1))
        assert torch.equal(ms.view(torch.int32), mb[t0:t0 + n].view(torch.int32))
        assert torch.equal(ls.view(torch.int32), lb[t0:t0 + n].view(torch.int32))
        written = torch.isfinite(ms)
        assert torch.equal(os_[written].view(torch.int32), ob[t0:t0 + n][written].view(torch.int32))
        assert torch.equal(out_s.view(torch.int16), out_big[t0:t0 + n].view(torch.int16))
    # and the large call against the oracle on a few tokens
    for t in (0, T // 3, T - 1):
        r = oracle_token(L, ids, pos0, synth.SCALE_1_SQRT_128, t)
        check_out(out_big[t].cpu().numpy(), r["out64"], "large call H=%d t=%d" % (H, t))


def test_probe_case_vs_oracle_all_tokens():
    L, ids, pos0 = probe_case(seed=6)
    out, o, m, l, C = run_attn(L, ids, pos0, synth.SCALE_1_SQRT_128)
    refs = oracle_tokens(L, ids, pos0, synth.SCALE_1_SQRT_128, list(range(ids.shape[0])))
    for t, r in refs.items():
        check_out(out[t], r["out64"], "probe t=%d" % t)
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, ids, pos0, synth.SCALE_1_SQRT_128, t, C), t, "probe")


@pytest.mark.parametrize("T,H,n_cells,pos0", [(1, 1, 1, 0), (1, 16, 65, 64), (5, 7, 130, 125), (70, 16, 200, 130),
                                             (33, 2, 64, 31)])
def test_edge_shapes_implicit_rows(T, H, n_cells, pos0):
    L = synth.make_layer(T + H, 0, T, H, n_cells)
    out, o, m, l, C = run_attn(L, None, pos0, synth.SCALE_1_SQRT_128, implicit=True)
    for t in range(T):
        r = oracle_token(L, None, pos0, synth.SCALE_1_SQRT_128, t)
        check_out(out[t], r["out64"], "edge t=%d" % t)
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, None, pos0, synth.SCALE_1_SQRT_128, t, C), t, "edge")


@pytest.mark.parametrize("T,H,n_cells,pos0,width", [(3, 1, 100, 90, 70), (9, 5, 300, 250, 128), (40, 16, 700, 600, 321),
                                                   (2, 16, 64, 62, 1), (6, 3, 520, 500, 450)])
def test_edge_shapes_explicit_ids(T, H, n_cells, pos0, width):
    """Explicit ids at head counts 1 .. 16 (so 15 .. 0 padding heads on the MFMA
    tile), ragged widths, and about a tenth of the slots poisoned with -1, a
    negative id or an id at or past n_cells: records, two-kernel output and
    fused output against the oracle on every token."""
    rng = np.random.default_rng(T + 17 * H)
    stride = 64 * ((width + 63) // 64)
    ids = np.full((T, stride), -1, np.int32)
    for t in range(T):
        p = pos0 + t
        k = min(width, p + 1)
        ids[t, :k] = np.sort(rng.choice(p + 1, k, replace=False))
        bad = rng.random(stride) < 0.1
        ids[t, bad] = rng.choice(np.array([-1, -7, n_cells, n_cells + 5], np.int32), int(bad.sum()))
    L = synth.make_layer(T + H + 1, 0, T, H, n_cells)
    scale = synth.SCALE_1_SQRT_128
    print("explicit edge T=%d H=%d n_cells=%d pos0=%d width=%d" % (T, H, n_cells, pos0, width), flush=True)
    out, o, m, l, C = run_attn(L, ids, pos0, scale)
    fout = run_fused(L, ids, pos0, scale)
    for t in range(T):
        r = oracle_token(L, ids, pos0, scale, t)
        check_out(out[t], r["out64"], "explicit edge t=%d" % t)
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, ids, pos0, scale, t, C), t, "explicit edge")
        check_out(fout[t], r["out64"], "explicit edge fused t=%d" % t)


def test_largest_cache_rows():
    """A cache of 2^25 rows, the most the library takes: ids reaching its last row
    exercise the 32-bit byte offsets of the gathers (id * 128 < 2^32). Only the
    selected rows hold data (8.6 GB of zeros otherwise); the oracle runs on a
    compact copy of those rows with the ids renumbered."""
    n_cells = 1 << 25
    T, H, width = 4, 12, 130
    pos0 = n_cells - T
    rng = np.random.default_rng(25)
    pool = np.unique(np.concatenate([np.arange(n_cells - 70, n_cells),                 # the last rows
                                     np.arange((1 << 24) - 8, (1 << 24) + 8),          # around 2^24
                                     rng.choice(pos0, 200, replace=False)]))           # anywhere below
    compact = synth.make_layer(26, 0, T, H, len(pool))
    stride = 64 * ((width + 63) // 64)
    ids = np.full((T, stride), -1, np.int32)
    ids_c = np.full((T, stride), -1, np.int32)
    for t in range(T):
        causal = np.nonzero(pool <= pos0 + t)[0]
        pick = np.sort(np.concatenate([causal[-20:], rng.choice(causal[:-20], width - 20, replace=False)]))
        ids[t, :width] = pool[pick]
        ids_c[t, :width] = pick
    assert ids.max() == n_cells - T + (T - 1)          # the cache's last row is selected
    d = dev()
    idx = torch.from_numpy(pool.astype(np.int64)).to(d)
    big = {}
    for name, arr, dt in (("kq", compact.kq, torch.int8), ("vq", compact.vq, torch.int8),
                          ("ksc", compact.ksc, torch.float16), ("vsc", compact.vsc, torch.float16)):
        full = torch.zeros((n_cells,) + arr.shape[1:], dtype=dt, device=d)
        full[idx] = torch.from_numpy(arr).to(d)
        big[name] = full
    q = torch.from_numpy(compact.q).to(d)
    ids_t = torch.from_numpy(ids).to(d)
    scale = synth.SCALE_1_SQRT_128
    print("largest cache: n_cells=%d pos0=%d, %d pooled rows" % (n_cells, pos0, len(pool)), flush=True)
    C = qsa.chunk_count(ids_t, pos0, T)
    part = qsa.alloc_part(T, H, 128, C)
    qsa.qsa_attn(q, big["kq"], big["vq"], big["ksc"], big["vsc"], ids_t, pos0, float(scale), part)
    out = torch.empty((T, H, 128), dtype=torch.float16, device=d)
    qsa.qsa_merge(part, C, out)
    fout = torch.empty_like(out)
    qsa.qsa_attn_merge(q, big["kq"], big["vq"], big["ksc"], big["vsc"], ids_t, pos0, float(scale), fout)
    torch.cuda.synchronize()
    o, m, l = [x.cpu().numpy() for x in qsa.part_views(part, T, H, 128, C)]
    out, fout = out.cpu().numpy(), fout.cpu().numpy()
    del big, part
    for t in range(T):
        r = oracle_token(compact, ids_c, pos0, scale, t)
        check_out(out[t], r["out64"], "largest cache t=%d" % t)
        check_records(o[t], m[t], l[t], r, chunk_magnitude(compact, ids_c, pos0, scale, t, C), t, "largest cache")
        check_out(fout[t], r["out64"], "largest cache fused t=%d" % t)


def test_large_and_tiny_scales():
    """V scales far from the configs' range, and large logits: no overflow, parity holds."""
    L, ids, pos0 = probe_case(T=40, seed=7)
    base = L.vsc.astype(np.float32)
    L.vsc[:] = (base * 10000).astype(np.float16)                       # up to 200
    L.vsc[::3] = (base[::3] * 1e-3).astype(np.float16)                 # fp16 subnormals
    L.ksc[:5] = np.float16(2.0 ** -24)                                 # subnormal scales
    L.q[:] = (L.q.astype(np.float32) * 40).astype(np.float16)           # logits of several hundred
    out, o, m, l, C = run_attn(L, ids, pos0, np.float32(1.0))
    refs = oracle_tokens(L, ids, pos0, np.float32(1.0), list(range(40)))
    for t, r in refs.items():
        scale_out = max(1.0, float(np.abs(r["out64"]).max()))
        g = out[t].astype(np.float64)
        assert np.all(np.isfinite(g[np.isfinite(r["out64"])]))
        assert np.abs(g - r["out64"]).max() <= 2e-3 * scale_out


def test_stream_argument_is_honoured():
    case = synth.tiny()
    L = case.layers[0]
    s = torch.cuda.Stream()
    q, kq, vq, ksc, vsc = (to_dev(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc))
    ids = to_dev(case.ids)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        part = qsa.alloc_part(16, 2, 128, 1)
        out = torch.empty(16, 2, 128, dtype=torch.float16, device=dev())
        qsa.qsa_attn(q, kq, vq, ksc, vsc, ids, 0, float(case.scale), part, stream=s)
        qsa.qsa_merge(part, 1, out, stream=s)
    s.synchronize()
    ref, _, _ = oracle.attn(L.q, L.kq, L.vq, L.ksc, L.vsc, case.ids, 0, case.scale)
    check_out(out.cpu().numpy(), ref, "stream")


@pytest.mark.parametrize("C", [0, 3])
def test_merge_rows_without_records_give_plus_zero(C):
    """A row with no finite chunk maximum -- no chunks at all, or only empty-chunk
    records (m = -inf, l = +0, o holding NaN bytes) -- merges to +0 in every
    dim, whatever the output held before."""
    T, H, D = 5, 12, 128
    part = qsa.alloc_part(T, H, D, C)
    part.fill_(0xFF)                         # every o float a NaN
    if C:
        o, m, l = qsa.part_views(part, T, H, D, C)
        m.fill_(float("-inf"))
        l.zero_()
    out = torch.full((T, H, D), float("nan"), dtype=torch.float16, device="cuda")
    qsa.qsa_merge(part, C, out)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy().view(np.uint16) == 0)


@pytest.mark.parametrize("implicit", [False, True])
def test_token_pieces_match_one_call(implicit):
    """A layer run as several calls on consecutive token ranges (pos0 moved by
    each range's first token) gives the one-call output bit for bit: the way a
    caller keeps one call's chunk records inside the Infinity Cache."""
    import torch
    import sparse_selection_attention_amd as qsa
    from gpu_util import to_dev
    case = synth.mid(layers=1) if not implicit else synth.prompt_start(implicit=True)
    L = case.layers[0]
    T, H, D = L.q.shape
    q, kq, vq, ksc, vsc = (to_dev(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc))
    ids = None if implicit else to_dev(case.ids)
    C = qsa.chunk_count(ids, case.pos0, T)
    part = qsa.alloc_part(T, H, D, C)
    full = torch.empty(T, H, D, dtype=torch.float16, device=q.device)
    qsa.qsa_attn(q, kq, vq, ksc, vsc, ids, case.pos0, float(case.scale), part)
    qsa.qsa_merge(part, C, full)
    pieces = torch.full((T, H, D), float("nan"), dtype=torch.float16, device=q.device)
    for t0, t1 in ((0, 700), (700, 701), (701, 1300), (1300, T)):
        if implicit:
            # implicit rows: a piece's rows are cells 0 .. pos0 + t of the same cache
            n = t1 - t0
            Cp = qsa.chunk_count(None, case.pos0 + t0, n)
            pp = qsa.alloc_part(n, H, D, Cp)
            qsa.qsa_attn(q[t0:t1], kq, vq, ksc, vsc, None, case.pos0 + t0, float(case.scale), pp)
            qsa.qsa_merge(pp, Cp, pieces[t0:t1])
        else:
            pp = qsa.alloc_part(t1 - t0, H, D, C)
            qsa.qsa_attn(q[t0:t1], kq, vq, ksc, vsc, ids[t0:t1], case.pos0 + t0, float(case.scale), pp)
            qsa.qsa_merge(pp, C, pieces[t0:t1])
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), pieces.view(torch.int16))
