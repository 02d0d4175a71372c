"""Pins of the oracle's sigmoid gate and per-16 sums.

Each pin ties qso_gate or qso_sums16 to something other than the oracle: the
sigmoid's closed forms and symmetry, torch's own sigmoid on a whole attention
chain, and Python's exactly rounded sum (math.fsum), so that a sign error in
the exponent, a dropped gate, a wrong block size or a sequential float sum fails
here.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from sparse_selection_attention_amd import synth


def test_sigmoid_closed_forms():
    # sigmoid(ln k) = k / (k + 1); the gate is an fp32 value, so the exact
    # sigmoid of that value is within |dg| / 4 of k / (k + 1)
    ks = np.array([1.0, 2.0, 3.0, 9.0, 0.5, 0.25, 1e-3, 1e3])
    g = np.log(ks).astype(np.float32)
    dg = np.abs(g.astype(np.float64) - np.log(ks))
    out64, _ = oracle.gate(np.ones_like(ks), g)
    assert np.all(np.abs(out64 - ks / (ks + 1.0)) <= dg / 4 + 4e-16)


def test_sigmoid_symmetry_and_range():
    g = (synth.gates(40, 3, kind="normal") * 4.0).ravel()
    a, _ = oracle.gate(np.ones(g.size), g)
    b, _ = oracle.gate(np.ones(g.size), -g)
    assert np.all(np.abs(a + b - 1.0) <= 4 * 2.0 ** -53)
    assert np.all((a >= 0) & (a <= 1))
    # monotone in the gate
    o = np.argsort(g, kind="stable")
    assert np.all(np.diff(a[o]) >= 0)


def test_gate_edges_are_exact():
    rng = np.random.default_rng(3)
    y = rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 4, 2000)
    y16 = np.array([oracle.double_to_half(v) for v in y], dtype=np.uint16).view(np.float16)
    zero = np.zeros(y.size, np.float32)
    # sigmoid(0) = 1/2 exactly: the value is halved, and so is its binary16
    # rounding wherever halving stays clear of the subnormal range
    h64, h16 = oracle.gate(y, zero)
    assert np.array_equal(h64, y * 0.5)
    big = np.abs(y16.astype(np.float64)) >= 2.0 ** -13
    assert np.array_equal(h16[big].astype(np.float64), y16[big].astype(np.float64) * 0.5)
    # sigmoid(+inf) = 1: the ungated value and rounding, bit for bit
    p64, p16 = oracle.gate(y, np.full(y.size, np.inf, np.float32))
    assert np.array_equal(p64, y) and np.array_equal(p16.view(np.uint16), y16.view(np.uint16))
    # sigmoid(-inf) = 0: zeros with the value's sign
    n64, n16 = oracle.gate(y, np.full(y.size, -np.inf, np.float32))
    assert np.all(n64 == 0) and np.array_equal(np.signbit(n64), np.signbit(y))
    assert np.array_equal(n16.view(np.uint16), np.where(np.signbit(y), 0x8000, 0).astype(np.uint16))


def test_gated_attention_chain_against_torch():
    """Merged attention by torch's SDPA and torch.sigmoid (fp64), against the
    oracle's records -> merge -> gate chain, on ragged poisoned rows."""
    T, H, n_cells, C = 6, 3, 200, 3
    rng = np.random.default_rng(11)
    L = synth.make_layer(7, 0, T, H, n_cells)
    pos0 = n_cells - T
    ids = np.full((T, 64 * C), -1, np.int32)
    for t in range(T):
        row = rng.integers(0, pos0 + t + 1, 64 * C)
        row[rng.random(64 * C) < 0.4] = -1
        ids[t] = row
    g = synth.gates(T, H, seed=9, kind="special")
    scale = synth.SCALE_1_SQRT_128
    out64, out16, sums = oracle.attn_gated(L.q, L.kq, L.vq, L.ksc, L.vsc, ids, pos0, scale, g)
    for t in range(T):
        cells = ids[t][ids[t] >= 0].astype(np.int64)
        K = torch.from_numpy(L.kq[cells].astype(np.float64) * np.repeat(L.ksc[cells].astype(np.float64), 32, 1))
        V = torch.from_numpy(L.vq[cells].astype(np.float64) * np.repeat(L.vsc[cells].astype(np.float64), 32, 1))
        Q = torch.from_numpy(L.q[t].astype(np.float64))[:, None, :]
        y = F.scaled_dot_product_attention(Q[None], K[None, None].expand(1, H, -1, -1),
                                           V[None, None].expand(1, H, -1, -1), scale=float(scale))[0, :, 0]
        ref = torch.sigmoid(torch.from_numpy(g[t].astype(np.float64))) * y
        assert np.allclose(out64[t], ref.numpy(), rtol=1e-12, atol=1e-15)
        assert np.array_equal(out16[t], ref.numpy().astype(np.float16))
    assert sums.shape == (T, H, 8)


def _fsum_rows(x16):
    xs = x16.astype(np.float64).reshape(-1, 16)
    return np.array([np.float32(math.fsum(r)) for r in xs], dtype=np.float32)


def test_sums16_are_exact_sums_rounded_once():
    rng = np.random.default_rng(5)
    # magnitudes spread over many binades, so that a float32 running sum (in
    # any fixed order) often differs from the correctly rounded exact sum
    x = (rng.standard_normal(16 * 4000) * 2.0 ** rng.integers(-20, 14, 16 * 4000)).astype(np.float16)
    x = x.reshape(-1, 128)
    got = oracle.sums16(x).ravel()
    ref = _fsum_rows(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    seq = np.zeros(ref.size, np.float32)
    xs = x.astype(np.float32).reshape(-1, 16)
    for i in range(16):
        seq = seq + xs[:, i]
    assert np.any(seq != ref), "the data must separate an fp32 running sum from the exact rounding"


def test_sums16_blocks_and_specials():
    x = np.zeros((2, 128), np.float16)
    x[0, :16] = 1.0                 # block 0 of row 0
    x[0, 16:32] = np.float16(2.0 ** -24)
    x[1, 112:] = -0.5               # last block of row 1
    x[1, 0] = np.inf
    s = oracle.sums16(x)
    assert s[0, 0] == 16.0 and s[0, 1] == np.float32(16 * 2.0 ** -24) and np.all(s[0, 2:] == 0)
    assert s[1, 7] == -8.0 and s[1, 0] == np.inf and np.all(s[1, 1:7] == 0)
