"""GPU parity of the shared-tile path: implicit rows (no id rows), where blocks
of (token, head) rows share every chunk's cells and QK / PV run as MFMA tile
contractions. Both entry points (chunk records and the fused output) take this
path for implicit rows."""
import numpy as np
import pytest
import torch

import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

from gpu_util import (check_out, check_records, chunk_magnitude, oracle_tokens, run_attn, run_fused)

pytestmark = pytest.mark.gpu


def _case(T, pos0, H, n_cells=None, seed=3):
    n_cells = pos0 + T if n_cells is None else n_cells
    return synth.make_layer(seed, 0, T, H, n_cells)


@pytest.mark.parametrize("T,pos0,H", [(300, 100, 12), (97, 0, 12), (64, 2000, 12), (129, 64, 5), (40, 30, 16)])
def test_every_token_against_the_oracle(T, pos0, H):
    # several row blocks, a ragged last block, chunks cut by the causal edge
    L = _case(T, pos0, H)
    scale = synth.SCALE_1_SQRT_128
    out, o, m, l, C = run_attn(L, None, pos0, scale, implicit=True)
    fout = run_fused(L, None, pos0, scale, implicit=True)
    refs = oracle_tokens(L, None, pos0, scale, list(range(T)))
    for t, r in refs.items():
        check_out(out[t], r["out64"], "tile records t=%d" % t)
        check_out(fout[t], r["out64"], "tile fused t=%d" % t)
        check_records(o[t], m[t], l[t], r, chunk_magnitude(L, None, pos0, scale, t, C), t, "tile")


def test_uniform_probe_is_exact():
    """q = 1, K = 0, unit V scales: each row's chunk k holds min(64, p + 1 - 64k)
    cells, all with p = 1, so l counts them and o sums the V rows exactly."""
    T, pos0, H = 200, 37, 12
    L = _case(T, pos0, H, seed=5)
    L.q[:] = 1.0
    L.kq[:] = 0
    L.vsc[:] = 1.0
    out, o, m, l, C = run_attn(L, None, pos0, np.float32(0.7), implicit=True)
    csum = np.cumsum(L.vq.astype(np.int64), axis=0)
    for t in range(T):
        p = pos0 + t
        for k in range(C):
            n = min(64, p + 1 - 64 * k)
            if n <= 0:
                assert np.all(m[t, k] == -np.inf) and np.all(l[t, k].view(np.uint32) == 0)
                continue
            assert np.all(m[t, k] == 0.0) and np.all(l[t, k] == n), (t, k)
            lo = csum[64 * k - 1] if k else 0
            want = (csum[64 * k + n - 1] - lo).astype(np.float32)
            assert np.array_equal(o[t, k], np.broadcast_to(want, (H, 128))), (t, k)
    # the fused output is the mean of the V rows 0 .. p (integers up to 127 in
    # size), rounded to fp16: within an fp16 rounding of the exact mean, plus
    # the fp32 sum and quotient before it
    fout = run_fused(L, None, pos0, np.float32(0.7), implicit=True)
    for t in range(T):
        mean = csum[pos0 + t] / (pos0 + t + 1.0)
        g = fout[t].astype(np.float64)
        assert np.all(np.abs(g - mean) <= np.abs(mean) * (2.0 ** -11 + 2.0 ** -20) + 2.0 ** -25), t


def test_cache_shorter_than_the_causal_range_is_refused():
    """n_cells below pos0 + T is QSA_ERR_ARG for implicit rows, on both paths,
    and nothing is written."""
    T, pos0, H, n_cells = 90, 60, 12, 100
    L = _case(T, pos0, H, n_cells=n_cells, seed=8)
    d = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(d)
    q, kq, vq, ksc, vsc = up(L.q), up(L.kq), up(L.vq), up(L.ksc), up(L.vsc)
    C = qsa.chunk_count(None, pos0, T)
    part = torch.full((qsa.qsa_part_bytes(T, H, 128, C),), 0x5A, dtype=torch.uint8, device=d)
    out = torch.full((T, H, 128), float("nan"), dtype=torch.float16, device=d)
    for call in (lambda: qsa.qsa_attn(q, kq, vq, ksc, vsc, None, pos0, 0.1, part),
                 lambda: qsa.qsa_attn_merge(q, kq, vq, ksc, vsc, None, pos0, 0.1, out)):
        with pytest.raises(qsa.QsaError) as e:
            call()
        assert e.value.status == qsa.QSA_ERR_ARG and "n_cells" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(part == 0x5A) and torch.all(torch.isnan(out))


def test_one_cell_cache_and_first_tokens():
    # the smallest cache a call can take (n_cells = pos0 + T = 1), and the
    # first tokens of a prompt, whose rows hold one and two cells
    L = _case(1, 0, 12, seed=4)
    out, o, m, l, C = run_attn(L, None, 0, 0.1, implicit=True)
    fout = run_fused(L, None, 0, 0.1, implicit=True)
    v = L.vq[0].astype(np.float64) * np.repeat(L.vsc[0].astype(np.float64), 32)
    ref = v.astype(np.float16)                   # one cell: the output is its V row, rounded once
    for h in range(12):
        assert np.array_equal(out[0, h].view(np.uint16), ref.view(np.uint16))
        assert np.array_equal(fout[0, h].view(np.uint16), ref.view(np.uint16))
    assert np.all(l[0, 0] == 1.0)


def test_large_and_tiny_scales():
    # V scales up to ~200 (power-of-two renormalisation), fp16-subnormal V and K
    # scales, logits of several hundred
    T, pos0, H = 120, 200, 12
    L = _case(T, pos0, H, seed=9)
    base = L.vsc.astype(np.float32)
    L.vsc[:] = (base * 10000).astype(np.float16)
    L.vsc[::3] = (base[::3] * 1e-3).astype(np.float16)
    L.ksc[:5] = np.float16(2.0 ** -24)
    L.q[:] = (L.q.astype(np.float32) * 40).astype(np.float16)
    out, o, m, l, C = run_attn(L, None, pos0, np.float32(1.0), implicit=True)
    fout = run_fused(L, None, pos0, np.float32(1.0), implicit=True)
    refs = oracle_tokens(L, None, pos0, np.float32(1.0), list(range(T)))
    for t, r in refs.items():
        scale_out = max(1.0, float(np.abs(r["out64"]).max()))
        for g16 in (out[t], fout[t]):
            g = g16.astype(np.float64)
            assert np.all(np.isfinite(g))
            assert np.abs(g - r["out64"]).max() <= 2e-3 * scale_out


def test_fused_tile_is_deterministic():
    case = synth.prompt_start(implicit=True)
    L = case.layers[0]
    a = run_fused(L, None, case.pos0, case.scale, implicit=True)
    b = run_fused(L, None, case.pos0, case.scale, implicit=True)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
