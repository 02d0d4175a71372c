"""Seeded synthetic inputs for the explicit-selection attention path.

This module only draws inputs. It holds none of the attention arithmetic and is
shared by the tests, the benchmark and the smoke check, so that the CPU oracle
and the HIP kernels are fed the same bytes.

Workloads follow the pages' descriptions of their test data:
  * "round 11 track b: qsa attention and score", section "boundaries and
    provenance": seed 5; signed int8 K/V caches drawn at random; positive,
    finite fp16 scales; fp16 queries; selected ids spread evenly over the
    causal cells without repeats; random fp32 inputs for the score kernel;
  * "round 5 track b: cached residual norms and fused mtp attention", section
    "mtp attention": the decode window is 64 sink cells, the 256 cells before
    the current one, and the current cell (321 cells, six 64-cell chunks).

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) in its counter form: the i-th
draw of a stream with key K is mix(K + (i + 1) * GAMMA). One stream per
(seed, layer, tensor) keeps every tensor independent of how many values other
tensors drew.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

# tensor ids used to key the streams
TID_Q, TID_KQ, TID_VQ, TID_KSC, TID_VSC, TID_SCORE_Q, TID_SCORE_K, TID_EDGE = range(8)
TID_ROWS, TID_ROWS_MAG, TID_ROWS_INT = range(8, 11)
TID_SEL, TID_SEL_INT = range(11, 13)
TID_GATE = 13

HEAD_DIM = 128
GROUP = 32          # one fp16 scale per 32 consecutive dims of a cached row
CHUNK = 64          # selected slots are processed in 64-cell chunks
SCALE_1_SQRT_128 = np.float32(1.0 / math.sqrt(128.0))


def _mix_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def _mix_arr(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, layer: int, tensor: int) -> int:
    return _mix_int(seed) ^ _mix_int(1000 * layer + tensor)


def raw_u64(key: int, n: int) -> np.ndarray:
    """First n outputs of the SplitMix64 stream with the given key."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        state = np.uint64(key) + i * np.uint64(GAMMA)
        return _mix_arr(state)


def uniform01(key: int, n: int) -> np.ndarray:
    """Doubles in [0, 1) from the top 53 bits of each draw."""
    return (raw_u64(key, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(key: int, n: int) -> np.ndarray:
    """Standard normals by the Box-Muller transform on consecutive draw pairs."""
    m = (n + 1) // 2
    u = uniform01(key, 2 * m)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))       # 1 - u1 lies in (0, 1]
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * math.pi * u2)
    z[1::2] = r * np.sin(2.0 * math.pi * u2)
    return z[:n]


def int8_sym(key: int, n: int) -> np.ndarray:
    """Integers uniform in [-127, 127] (-128 is never drawn)."""
    return ((raw_u64(key, n) % np.uint64(255)).astype(np.int64) - 127).astype(np.int8)


def f16_uniform(key: int, n: int, lo: float, hi: float) -> np.ndarray:
    """fp16 values (round-to-nearest-even from fp64) of U[lo, hi]."""
    return (lo + (hi - lo) * uniform01(key, n)).astype(np.float16)


# ---------------------------------------------------------------------------
# selections


def causal_all_ids(pos0: int, T: int, stride: int) -> np.ndarray:
    """Row t lists cells 0..pos0+t in order, then -1 up to `stride` slots."""
    ids = np.full((T, stride), -1, dtype=np.int32)
    for t in range(T):
        p = pos0 + t
        ids[t, : p + 1] = np.arange(p + 1, dtype=np.int32)
    return ids


def evenly_spaced_ids(pos0: int, T: int, K: int) -> np.ndarray:
    """Up to K causal cells per row, evenly spaced and without repeats, padded with -1.

    Row t (p = pos0 + t) holds every cell 0..p when p + 1 <= K, otherwise
    floor(j * p / (K - 1)) for j = 0..K-1: ascending, unique (the step p/(K-1)
    is at least 1), and containing the sink cell 0 and the current cell p
    (K = 1 holds the current cell alone). The row is padded with -1 to a whole
    number of 64-cell chunks.
    """
    stride = CHUNK * ((K + CHUNK - 1) // CHUNK)
    ids = np.full((T, stride), -1, dtype=np.int32)
    j = np.arange(K, dtype=np.int64)
    for t in range(T):
        p = pos0 + t
        if p + 1 <= K:
            ids[t, : p + 1] = np.arange(p + 1, dtype=np.int32)
        elif K == 1:
            ids[t, 0] = p
        else:
            ids[t, :K] = (j * p) // (K - 1)
    return ids


def mtp_window_ids(pos0: int, ntok: int, sink: int = 64, local: int = 256) -> np.ndarray:
    """Decode window: sink cells, the previous `local` cells, then the current cell."""
    width = sink + local + 1
    stride = CHUNK * ((width + CHUNK - 1) // CHUNK)
    ids = np.full((ntok, stride), -1, dtype=np.int32)
    for t in range(ntok):
        p = pos0 + t
        if p - local < sink:
            raise ValueError("window overlaps the sink cells: p=%d" % p)
        row = np.concatenate([np.arange(sink), np.arange(p - local, p), [p]])
        ids[t, :width] = row
    return ids


# ---------------------------------------------------------------------------
# attention cases


@dataclasses.dataclass
class Layer:
    q: np.ndarray      # fp16 [T][H][D]
    kq: np.ndarray     # int8 [n_cells][D]
    vq: np.ndarray     # int8 [n_cells][D]
    ksc: np.ndarray    # fp16 [n_cells][D/32]
    vsc: np.ndarray    # fp16 [n_cells][D/32]


@dataclasses.dataclass
class AttnCase:
    name: str
    T: int
    pos0: int
    H: int
    D: int
    n_cells: int
    ids: Optional[np.ndarray]   # int32 [T][ids_stride], or None for implicit all-causal rows
    ids_stride: int
    scale: np.float32
    layers: List[Layer]

    @property
    def n_chunks(self) -> int:
        if self.ids is None:
            return (self.pos0 + self.T + CHUNK - 1) // CHUNK
        return self.ids_stride // CHUNK


def make_layer(seed: int, layer: int, T: int, H: int, n_cells: int, D: int = HEAD_DIM,
               scale_lo: float = 1e-3, scale_hi: float = 2e-2) -> Layer:
    G = D // GROUP
    q = normal(stream_key(seed, layer, TID_Q), T * H * D).astype(np.float16).reshape(T, H, D)
    kq = int8_sym(stream_key(seed, layer, TID_KQ), n_cells * D).reshape(n_cells, D)
    vq = int8_sym(stream_key(seed, layer, TID_VQ), n_cells * D).reshape(n_cells, D)
    ksc = f16_uniform(stream_key(seed, layer, TID_KSC), n_cells * G, scale_lo, scale_hi).reshape(n_cells, G)
    vsc = f16_uniform(stream_key(seed, layer, TID_VSC), n_cells * G, scale_lo, scale_hi).reshape(n_cells, G)
    return Layer(q, kq, vq, ksc, vsc)


def make_case(name: str, T: int, pos0: int, H: int, ids: Optional[np.ndarray], layers: int = 1,
              seed: int = 5, n_cells: Optional[int] = None, D: int = HEAD_DIM,
              scale: np.float32 = SCALE_1_SQRT_128) -> AttnCase:
    if n_cells is None:
        n_cells = pos0 + T
    stride = 0 if ids is None else int(ids.shape[1])
    ls = [make_layer(seed, li, T, H, n_cells, D) for li in range(layers)]
    return AttnCase(name, T, pos0, H, D, n_cells, ids, stride, np.float32(scale), ls)


def tiny() -> AttnCase:
    """T=16 at pos0=0, 2 heads, 16 cells, every causal cell selected, one chunk."""
    return make_case("tiny", 16, 0, 2, causal_all_ids(0, 16, CHUNK))


def mtp(ntok: int, layers: int = 1) -> AttnCase:
    """Decode window at pos0=3000: 64 sink + 256 local + 1 current cells, 12 heads."""
    return make_case("mtp%d" % ntok, ntok, 3000, 12, mtp_window_ids(3000, ntok), layers=layers)


def prompt_start(implicit: bool = False, layers: int = 1, T: int = 1984) -> AttnCase:
    """T=1984 at pos0=0, every causal cell selected (explicit ids, or implicit rows)."""
    stride = CHUNK * ((T + CHUNK - 1) // CHUNK)
    ids = None if implicit else causal_all_ids(0, T, stride)
    return make_case("prompt" + ("_implicit" if implicit else ""), T, 0, 12, ids, layers=layers)


def mid(layers: int = 3, T: int = 1984) -> AttnCase:
    """T=1984 at pos0=8192, up to 2048 evenly spaced causal cells per row."""
    return make_case("mid", T, 8192, 12, evenly_spaced_ids(8192, T, 2048), layers=layers)


def long_ctx(layers: int = 3, T: int = 1984, variant: Optional[str] = None) -> AttnCase:
    """T=1984 at pos0=30000, up to 2051 evenly spaced causal cells per row.

    variant "signed_zero": for tokens t = 0 mod 4, heads 0 and 6 get q = -0.0 in
    every dim, and cached K rows of cells c = 0 mod 3 are made non-negative, so
    those scores are exactly -0 or +0.
    variant "cancel": for tokens t = 1 mod 4, in each 32-dim group the first 16
    dims of q are +-2^-24 (random signs) and the last 16 are their negatives, and
    every cached K row repeats its first 16 dims of each group in the last 16, so
    each group's dot product cancels to zero exactly.
    """
    name = "long" if variant is None else "long_" + variant
    case = make_case(name, T, 30000, 12, evenly_spaced_ids(30000, T, 2051), layers=layers)
    if variant is None:
        return case
    for li, L in enumerate(case.layers):
        if variant == "signed_zero":
            qb = L.q.view(np.uint16)
            qb[0::4, [0, 6], :] = 0x8000
            L.kq[0::3] = np.abs(L.kq[0::3])
        elif variant == "cancel":
            sign = raw_u64(stream_key(5, li, TID_EDGE), T * L.q.shape[1] * 4 * 16) & np.uint64(1)
            sign = sign.reshape(T, L.q.shape[1], 4, 16)
            qb = L.q.view(np.uint16).reshape(T, L.q.shape[1], 4, 32)
            pos = np.where(sign == 0, 0x0001, 0x8001).astype(np.uint16)
            neg = pos ^ np.uint16(0x8000)
            qb[1::4, :, :, :16] = pos[1::4]
            qb[1::4, :, :, 16:] = neg[1::4]
            kq = L.kq.reshape(-1, 4, 32)
            kq[:, :, 16:] = kq[:, :, :16]
        else:
            raise ValueError(variant)
    return case


# ---------------------------------------------------------------------------
# score inputs


@dataclasses.dataclass
class ScoreCase:
    name: str
    T: int
    pos0: int
    Hs: int
    D: int
    n_cells: int
    q: np.ndarray       # fp32 [T][Hs][D]
    k: np.ndarray       # fp32 [n_cells][D]
    scale: np.float32
    dead: np.float32
    row_stride: int


def score_case(T: int = 1984, pos0: int = 0, Hs: int = 1, seed: int = 5, D: int = HEAD_DIM,
               row_stride: Optional[int] = None, scale: float = 1.0,
               dead: float = -math.inf, n_cells: Optional[int] = None) -> ScoreCase:
    if n_cells is None:
        n_cells = pos0 + T
    if row_stride is None:
        row_stride = pos0 + T
    q = normal(stream_key(seed, 0, TID_SCORE_Q), T * Hs * D).astype(np.float32).reshape(T, Hs, D)
    k = normal(stream_key(seed, 0, TID_SCORE_K), n_cells * D).astype(np.float32).reshape(n_cells, D)
    return ScoreCase("score_T%d_p%d_h%d" % (T, pos0, Hs), T, pos0, Hs, D, n_cells, q, k,
                     np.float32(scale), np.float32(dead), row_stride)


# ---------------------------------------------------------------------------
# fp32 rows for the int8 cache writer


ROW_KINDS = ("normal", "spread", "ties", "near", "special")


def cache_rows(n: int, seed: int = 5, kind: str = "normal", which: int = 0, D: int = HEAD_DIM) -> np.ndarray:
    """fp32 rows [n][D] to be quantised into the cache; `which` (0 for K, 1 for V)
    picks an independent stream.

    normal   N(0, 1) values, the scale of normalised K and V rows;
    spread   N(0, 1) times a per-group magnitude 10^U(-8, 6): fp16 scales from
             zero (underflow) and subnormal up to ~3e4;
    ties     per group an fp16 step s, one element 127 s and the others
             (j + 1/2) s for integers |j| <= 126, so that x / s falls exactly
             halfway between two codes;
    near     like ties, but each element moved off the half-integer by a few
             binary32 ulps or by 2^-15 .. 2^-12 of the step, either side;
    special  zero and negative-zero groups, groups with one non-zero element,
             subnormal-step groups and groups at the top of the fp16 range,
             mixed with normal ones.
    """
    G = D // GROUP
    layer = 100 + 10 * which + ROW_KINDS.index(kind)
    z = normal(stream_key(seed, layer, TID_ROWS), n * D).reshape(n, G, GROUP)
    u = uniform01(stream_key(seed, layer, TID_ROWS_MAG), n * G).reshape(n, G, 1)
    if kind == "normal":
        x = z
    elif kind == "spread":
        x = z * 10.0 ** (-8.0 + 14.0 * u)
    elif kind == "ties":
        step = (10.0 ** (-3.0 + 5.0 * u)).astype(np.float16).astype(np.float64)       # an fp16 step
        j = (raw_u64(stream_key(seed, layer, TID_ROWS_INT), n * D) % np.uint64(253)).astype(np.int64) - 126
        x = (j.reshape(n, G, GROUP) + 0.5) * step
        x[:, :, 0] = 127.0 * step[:, :, 0]
        x = x * np.where(z > 0, 1.0, -1.0)
    elif kind == "near":
        step = (10.0 ** (-3.0 + 5.0 * u)).astype(np.float16).astype(np.float64)
        j = (raw_u64(stream_key(seed, layer, TID_ROWS_INT), n * D) % np.uint64(253)).astype(np.int64) - 126
        pick = (raw_u64(stream_key(seed, layer, TID_ROWS_INT + 100), n * D) % np.uint64(12)).astype(np.int64)
        sign = np.where(pick % 2 == 0, 1.0, -1.0)
        frac = np.array([0, 0, 0, 0, 0, 0, 2.0 ** -15, 2.0 ** -15, 2.0 ** -14, 2.0 ** -14, 2.0 ** -12, 2.0 ** -12])[pick]
        ulps = np.array([1, 1, 2, 2, 5, 5, 0, 0, 0, 0, 0, 0])[pick]
        t = ((j + 0.5) + sign * frac).reshape(n, G, GROUP) * step
        x = t.astype(np.float32)
        # ulp steps away from the half-integer in binary32
        x = np.where(ulps.reshape(n, G, GROUP) > 0,
                     x + sign.reshape(n, G, GROUP) * ulps.reshape(n, G, GROUP) * np.spacing(x), x)
        x[:, :, 0] = 127.0 * step[:, :, 0]
        x = x * np.where(z > 0, 1.0, -1.0)
    elif kind == "special":
        x = z.copy()
        sel = (raw_u64(stream_key(seed, layer, TID_ROWS_INT), n * G) % np.uint64(6)).reshape(n, G)
        x[sel == 0] = 0.0
        x[sel == 1] = -0.0
        one = x[sel == 2]
        one[:, 1:] = 0.0
        x[sel == 2] = one
        x[sel == 3] *= 1e-6
        x[sel == 4] *= 127.0 * 65504.0 / 5.0
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(x.reshape(n, D).astype(np.float32))


# ---------------------------------------------------------------------------
# score rows for the selection producer


SCORE_KINDS = ("normal", "ties", "special")


def select_scores(T: int, pos0: int, seed: int = 5, kind: str = "normal", row_stride: Optional[int] = None) -> np.ndarray:
    """fp32 score rows [T][row_stride] (row_stride >= pos0 + T) to select from.

    normal   N(0, 1) values;
    ties     values on a grid of quarters in [-5, 5] (many equal scores), with
             signed zeros;
    special  N(0, 1) with +-inf, +-0 and large runs of one repeated value.
    Cells past each row's causal edge hold 3e38, larger than every causal
    score, so a selection that read past the edge would pick them.
    """
    if row_stride is None:
        row_stride = pos0 + T
    n = T * row_stride
    z = normal(stream_key(seed, 200 + SCORE_KINDS.index(kind), TID_SEL), n).reshape(T, row_stride)
    if kind == "normal":
        x = z
    elif kind == "ties":
        r = raw_u64(stream_key(seed, 200 + SCORE_KINDS.index(kind), TID_SEL_INT), n).reshape(T, row_stride)
        x = ((r % np.uint64(41)).astype(np.int64) - 20) / 4.0
        x = np.where((r >> np.uint64(40)) % np.uint64(16) == 0, np.where(z > 0, 0.0, -0.0), x)
    elif kind == "special":
        r = raw_u64(stream_key(seed, 200 + SCORE_KINDS.index(kind), TID_SEL_INT), n).reshape(T, row_stride)
        sel = (r % np.uint64(50)).astype(np.int64)
        x = z.copy()
        x[sel == 0] = np.inf
        x[sel == 1] = -np.inf
        x[sel == 2] = 0.0
        x[sel == 3] = -0.0
        x[(sel >= 4) & (sel < 12)] = 1.25
    else:
        raise ValueError(kind)
    x = x.astype(np.float32)
    # beyond the causal edge: a huge value, so reading it would change the selection
    cols = np.arange(row_stride)[None, :]
    p = pos0 + np.arange(T)[:, None]
    x[cols > p] = np.float32(3e38)
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------------------
# output gates


GATE_KINDS = ("normal", "special")


def gates(T: int, H: int, seed: int = 5, layer: int = 0, kind: str = "normal", D: int = HEAD_DIM) -> np.ndarray:
    """fp32 gate inputs [T][H][D], one per output element.

    "normal": N(0, 2^2), so the sigmoid runs from about 0.002 to 0.998;
    "special": the same draws with every 7th element replaced, in turn, by 0,
    +inf, -inf, +100, -100, -0.0, 1e-30 and -1e-30.
    """
    if kind not in GATE_KINDS:
        raise ValueError(kind)
    g = (2.0 * normal(stream_key(seed, layer, TID_GATE), T * H * D)).astype(np.float32)
    if kind == "special":
        picks = np.array([0.0, math.inf, -math.inf, 100.0, -100.0, -0.0, 1e-30, -1e-30], dtype=np.float32)
        idx = np.arange(0, g.size, 7)
        g[idx] = picks[np.arange(idx.size) % picks.size]
    return g.reshape(T, H, D)
