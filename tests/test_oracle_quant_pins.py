"""Pins of the oracle's int8 cache quantisation (qso_quant_rows).

The rule (symmetric absmax per 32-element group, fp16 scale, round half to
even) is a reading of the pages, which do not print it; these tests tie the
oracle's arithmetic to hand-worked values, closed forms and invariants that
any correct implementation of that rule must satisfy.
"""
import numpy as np
import pytest

import oracle


def f16(bits):
    return float(np.uint16(bits).view(np.float16))


def group_row(values, D=128):
    x = np.zeros((1, D), dtype=np.float32)
    x[0, :len(values)] = values
    return x


def test_hand_worked_row():
    # a = 1: a / 127 = 0.0078740157..., whose nearest fp16 is
    # 2^-7 * (1 + 8/1024) = 0.00787353515625 (bits 0x2008). 1 / s = 127.0078 -> 127;
    # 0.5 / s = 63.5039 -> 64: the scale's rounding moves this code across .5
    c, s = oracle.quant_rows(group_row([1.0, 0.5]))
    assert s[0, 0] == 0x2008
    assert list(c[0, :3]) == [127, 64, 0]
    assert np.all(s[0, 1:] == 0) and np.all(c[0, 32:] == 0)


def test_exact_grid_codes():
    # a = 63.5 gives s = 0.5 exactly (63.5 / 127), so x = j / 2 has code j
    j = np.array([127, -127, 0, 1, -1, 2, -2, 3, 50, -77, 126, -126, 64, -64, 100, 5] * 2, dtype=np.int64)
    c, s = oracle.quant_rows(group_row(j / 2.0))
    assert f16(s[0, 0]) == 0.5
    assert np.array_equal(c[0, :32].astype(np.int64), j)


def test_ties_round_half_to_even():
    # s = 0.5; x / s = 0.5, 1.5, 2.5, -0.5, -1.5, -2.5 -> 0, 2, 2, 0, -2, -2
    c, s = oracle.quant_rows(group_row([63.5, 0.25, 0.75, 1.25, -0.25, -0.75, -1.25]))
    assert f16(s[0, 0]) == 0.5
    assert list(c[0, :7]) == [127, 0, 2, 2, 0, -2, -2]


def test_zero_groups():
    x = np.zeros((2, 128), dtype=np.float32)
    x[1] = -0.0
    x[1, 40] = 3.0                     # only group 1 of row 1 is non-zero
    c, s = oracle.quant_rows(x)
    assert np.all(s[0] == 0) and np.all(c[0] == 0)
    assert s[1, 0] == 0 and s[1, 2] == 0 and s[1, 3] == 0     # -0 groups give +0 scales
    assert s[1, 1] != 0 and c[1, 40] == 127


def random_rows(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128))
    # per-group magnitudes from 1e-1 to 1e4: every scale, also after a factor
    # 2^-3 or 2^5, is a normal fp16 number
    mag = 10.0 ** rng.uniform(-1, 4, (n, 4))
    return (x * np.repeat(mag, 32, axis=1)).astype(np.float32)


def test_normal_scale_bounds_and_round_trip():
    x = random_rows(400, 3)
    c, s = oracle.quant_rows(x)
    sc = np.repeat(s.view(np.float16).astype(np.float64), 32, axis=1)
    a = np.repeat(np.abs(x.astype(np.float64)).reshape(400, 4, 32).max(axis=2), 32, axis=1)
    assert np.all(sc >= 2.0 ** -14)                               # normal fp16 scales here
    # the fp16 scale is within half an fp16 ulp (2^-11 relative) of a / 127
    assert np.all(np.abs(sc - a / 127.0) <= 2.0 ** -11 * a / 127.0 * (1 + 1e-6))
    # |x / s| <= 127 (1 + 2^-11) < 127.5, so no code is clamped and the round trip
    # is within half a scale step, plus the binary32 quotient's own rounding
    err = np.abs(x.astype(np.float64) - c.astype(np.float64) * sc)
    assert np.all(err <= sc * (0.5 + 2.0 ** -16))
    # the element of largest magnitude in each group maps to +-127
    g = np.abs(x).reshape(400, 4, 32).argmax(axis=2)
    top = np.take_along_axis(c.reshape(400, 4, 32).astype(np.int64), g[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.abs(c.astype(np.int64)) <= 127)


def test_sign_and_power_of_two_invariance():
    x = random_rows(200, 4)
    c, s = oracle.quant_rows(x)
    cn, sn = oracle.quant_rows(-x)
    assert np.array_equal(sn, s) and np.array_equal(cn.astype(np.int64), -c.astype(np.int64))
    for k in (-3, 5):
        ck, sk = oracle.quant_rows(x * np.float32(2.0 ** k))
        assert np.array_equal(ck, c)
        assert np.array_equal(sk.view(np.float16).astype(np.float64), s.view(np.float16).astype(np.float64) * 2.0 ** k)


def test_subnormal_scale_clamps_at_127():
    # a = 1.4 * 127 * 2^-24: a / 127 = 1.4 * 2^-24 rounds to the fp16 subnormal
    # 2^-24, so a / s = 177.8 and the code clamps to 127; -a clamps to -127
    a = np.float32(1.4 * 127 * 2.0 ** -24)
    c, s = oracle.quant_rows(group_row([a, -a, a / 2]))
    assert s[0, 0] == 0x0001
    assert list(c[0, :3]) == [127, -127, 89]          # 88.9 -> 89


@pytest.mark.parametrize("bits", [0x3C00, 0x2008, 0x0400, 0x7BFF])
def test_codes_of_multiples_of_a_scale(bits):
    # x = j * s for an fp16 s and |j| <= 127 with max |j| = 127: the scale
    # recovers s (127 s / 127 = s) and the codes recover j
    s = np.float64(f16(bits))
    rng = np.random.default_rng(bits)
    j = rng.integers(-127, 128, 32)
    j[5] = -127
    x = group_row((j * s).astype(np.float32))
    assert np.array_equal(x[0, :32].astype(np.float64), j * s)        # exact in fp32
    c, sc = oracle.quant_rows(x)
    assert sc[0, 0] == bits
    assert np.array_equal(c[0, :32].astype(np.int64), j)
