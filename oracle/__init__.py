"""ctypes wrapper of the C oracle (qsa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product package. It computes in
fp64 with plain sequential loops; see the header of qsa_oracle.c for what each
function follows on the pages.
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes as _ct
import os as _os
import subprocess as _sp

import numpy as _np

_HERE = _os.path.dirname(_os.path.abspath(__file__))
_SRC = _os.path.join(_HERE, "qsa_oracle.c")
LIB_PATH = _os.path.join(_HERE, "libqsa_oracle.so")
CHUNK = 64

_lib = None


def build() -> str:
    """Compile the oracle with gcc: -O2, no contraction, no fast-math."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Werror", _SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    _sp.run(cmd, check=True)
    _os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not _os.path.exists(LIB_PATH):
            build()
        L = _ct.CDLL(LIB_PATH)
        P = _ct.c_void_p
        i32 = _ct.c_int32
        L.qso_half_to_double.argtypes = [_ct.c_uint16]
        L.qso_half_to_double.restype = _ct.c_double
        L.qso_double_to_half.argtypes = [_ct.c_double]
        L.qso_double_to_half.restype = _ct.c_uint16
        L.qso_attn_chunks.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32,
                                      _ct.c_double, i32, i32, P, P, P, P]
        L.qso_attn_chunks.restype = _ct.c_int
        L.qso_merge.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P]
        L.qso_merge.restype = _ct.c_int
        L.qso_score.argtypes = [P, P, i32, i32, i32, i32, i32, _ct.c_double, _ct.c_double,
                                P, _ct.c_int64, i32, i32]
        L.qso_score.restype = _ct.c_int
        L.qso_quant_rows.argtypes = [P, i32, i32, P, P]
        L.qso_quant_rows.restype = _ct.c_int
        L.qso_select.argtypes = [P, _ct.c_int64, i32, i32, i32, P, i32, i32, i32]
        L.qso_select.restype = _ct.c_int
        L.qso_gate.argtypes = [P, P, _ct.c_int64, P, P]
        L.qso_gate.restype = _ct.c_int
        L.qso_sums16.argtypes = [P, _ct.c_int64, i32, P]
        L.qso_sums16.restype = _ct.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_ct.c_void_p)


def _ranges(t_lo, t_hi, threads):
    n = t_hi - t_lo
    threads = max(1, min(threads, n))
    step = (n + threads - 1) // threads
    return [(a, min(a + step, t_hi)) for a in range(t_lo, t_hi, step)]


def half_to_double(h: int) -> float:
    return lib().qso_half_to_double(int(h))


def double_to_half(x: float) -> int:
    return lib().qso_double_to_half(float(x))


def n_chunks(ids, ids_stride, pos0, T):
    return ids_stride // CHUNK if ids is not None else (pos0 + T + CHUNK - 1) // CHUNK


def attn_chunks(q, kq, vq, ksc, vsc, ids, pos0, scale, t_range=None, want_abs=False,
                threads=1, m=None, l=None, o=None):
    """Chunk records (m, l, o[, oabs]) as fp64 arrays [T][C][H](,[D]).

    q fp16 [T][H][D]; kq, vq int8 [n_cells][D]; ksc, vsc fp16 [n_cells][D/32];
    ids int32 [T][stride] or None (implicit all-causal rows); scale fp32.
    Only tokens in t_range = (t_begin, t_end) are computed; other rows keep the
    contents of the arrays passed in (NaN when the arrays are created here).
    Empty chunks leave o unchanged, as the method does.
    """
    T, H, D = q.shape
    n_cells = kq.shape[0]
    q = _np.ascontiguousarray(q)
    stride = 0 if ids is None else ids.shape[1]
    C = n_chunks(ids, stride, pos0, T)
    if m is None:
        m = _np.full((T, C, H), _np.nan)
        l = _np.full((T, C, H), _np.nan)
        o = _np.full((T, C, H, D), _np.nan)
    oabs = _np.full((T, C, H, D), _np.nan) if want_abs else None
    t0, t1 = (0, T) if t_range is None else t_range
    args = [_ptr(q.view(_np.uint16)), _ptr(kq), _ptr(vq), _ptr(ksc.view(_np.uint16)),
            _ptr(vsc.view(_np.uint16)), n_cells, _ptr(ids), stride, pos0, T, H, D,
            float(_np.float32(scale))]

    def run(r):
        rc = lib().qso_attn_chunks(*args, r[0], r[1], _ptr(m), _ptr(l), _ptr(o), _ptr(oabs))
        if rc != 0:
            raise ValueError("oracle rejected the shape")

    _run_ranges(run, _ranges(t0, t1, threads))
    return (m, l, o, oabs) if want_abs else (m, l, o)


def merge(m, l, o, t_range=None, threads=1):
    """Max-first merge: returns (out64 [T][H][D] fp64, out16 [T][H][D] fp16)."""
    T, C, H, D = o.shape
    out64 = _np.full((T, H, D), _np.nan)
    out16 = _np.full((T, H, D), 0x7E00, dtype=_np.uint16)
    t0, t1 = (0, T) if t_range is None else t_range

    def run(r):
        rc = lib().qso_merge(_ptr(m), _ptr(l), _ptr(o), C, T, H, D, r[0], r[1],
                             _ptr(out64), _ptr(out16))
        if rc != 0:
            raise ValueError("oracle rejected the shape")

    _run_ranges(run, _ranges(t0, t1, threads))
    return out64, out16.view(_np.float16)


def attn(q, kq, vq, ksc, vsc, ids, pos0, scale, t_range=None, threads=1):
    """Whole path: chunk records then merge. Returns (out64, out16, (m, l, o))."""
    m, l, o = attn_chunks(q, kq, vq, ksc, vsc, ids, pos0, scale, t_range=t_range, threads=threads)
    out64, out16 = merge(m, l, o, t_range=t_range, threads=threads)
    return out64, out16, (m, l, o)


def score(q, k, pos0, scale, dead, row_stride, t_range=None, threads=1, fill=_np.nan):
    """Causal scores as fp64 [T][row_stride]; untouched cells hold `fill`."""
    T, Hs, D = q.shape
    n_cells = k.shape[0]
    q = _np.ascontiguousarray(q, dtype=_np.float32)
    k = _np.ascontiguousarray(k, dtype=_np.float32)
    out = _np.full((T, row_stride), fill, dtype=_np.float64)
    t0, t1 = (0, T) if t_range is None else t_range

    def run(r):
        rc = lib().qso_score(_ptr(q), _ptr(k), n_cells, pos0, T, Hs, D, float(_np.float32(scale)),
                             float(dead), _ptr(out), row_stride, r[0], r[1])
        if rc != 0:
            raise ValueError("oracle rejected the shape")

    _run_ranges(run, _ranges(t0, t1, threads))
    return out


def _run_ranges(fn, ranges):
    if len(ranges) == 1:
        fn(ranges[0])
        return
    # ctypes releases the GIL for the duration of each foreign call
    with _cf.ThreadPoolExecutor(len(ranges)) as ex:
        for f in [ex.submit(fn, r) for r in ranges]:
            f.result()


def quant_rows(x):
    """Int8 codes and fp16 scale bits (uint16) of fp32 rows x[n][D], one scale
    per 32-element group (qso_quant_rows)."""
    x = _np.ascontiguousarray(x, dtype=_np.float32)
    n, D = x.shape
    codes = _np.zeros((n, D), dtype=_np.int8)
    scales = _np.zeros((n, D // 32), dtype=_np.uint16)
    if lib().qso_quant_rows(_ptr(x), n, D, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("qso_quant_rows: bad arguments")
    return codes, scales


def select(scores, pos0, K, ids_stride, t_range=None, threads=1):
    """Top-K causal cell ids per row (qso_select): int32 [T][ids_stride], -1 padded."""
    scores = _np.ascontiguousarray(scores, dtype=_np.float32)
    T, row_stride = scores.shape
    ids = _np.full((T, ids_stride), -2, dtype=_np.int32)
    t0, t1 = (0, T) if t_range is None else t_range

    def run(r):
        if lib().qso_select(_ptr(scores), row_stride, pos0, T, K, _ptr(ids), ids_stride, r[0], r[1]) != 0:
            raise ValueError("qso_select rejected the arguments")

    _run_ranges(run, _ranges(t0, t1, threads))
    return ids


def gate(y64, g):
    """Sigmoid-gated output (qso_gate): y64 fp64 merged values, g fp32 gates of
    the same shape. Returns (out64 fp64, out16 fp16)."""
    y64 = _np.ascontiguousarray(y64, dtype=_np.float64)
    g = _np.ascontiguousarray(g, dtype=_np.float32)
    if y64.shape != g.shape:
        raise ValueError("gates must have the output's shape")
    out64 = _np.empty_like(y64)
    out16 = _np.empty(y64.shape, dtype=_np.uint16)
    if lib().qso_gate(_ptr(y64), _ptr(g), y64.size, _ptr(out64), _ptr(out16)) != 0:
        raise ValueError("qso_gate: bad arguments")
    return out64, out16.view(_np.float16)


def sums16(x16):
    """Per-16 sums (qso_sums16) of fp16 values [..., D]: float32 [..., D/16]."""
    x16 = _np.ascontiguousarray(x16, dtype=_np.float16)
    D = x16.shape[-1]
    rows = x16.size // D
    out = _np.empty(x16.shape[:-1] + (D // 16,), dtype=_np.float32)
    if lib().qso_sums16(_ptr(x16.view(_np.uint16)), rows, D, _ptr(out)) != 0:
        raise ValueError("qso_sums16: bad arguments")
    return out


def attn_gated(q, kq, vq, ksc, vsc, ids, pos0, scale, g, t_range=None, threads=1):
    """Whole gated path: chunk records, merge, sigmoid gate, per-16 sums.
    Returns (out64, out16, sums) for the tokens in t_range (other rows NaN)."""
    y64, _, _ = attn(q, kq, vq, ksc, vsc, ids, pos0, scale, t_range=t_range, threads=threads)
    t0, t1 = (0, q.shape[0]) if t_range is None else t_range
    out64 = _np.full(y64.shape, _np.nan)
    out16 = _np.full(y64.shape, _np.nan, dtype=_np.float16)
    sums = _np.full(y64.shape[:-1] + (y64.shape[-1] // 16,), _np.nan, dtype=_np.float32)
    a, b = gate(y64[t0:t1], g[t0:t1])
    out64[t0:t1], out16[t0:t1] = a, b
    sums[t0:t1] = sums16(b)
    return out64, out16, sums
