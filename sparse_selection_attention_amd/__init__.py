"""Python binding of libqsa.so: explicit-selection attention on MI355X.

The functions carry the C ABI's names (include/qsa.h) and only marshal
arguments: they check dtypes, shapes, devices and contiguity of torch tensors,
then pass raw device pointers and the current HIP stream to the library. Every
step of the computation runs in the library's HIP kernels; there is no CPU
fallback, and a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "QsaError", "CHUNK", "GROUP", "HEAD_DIM",
    "qsa_attn", "qsa_attn_merge", "qsa_attn_merge_gated", "qsa_merge", "qsa_merge_gated", "qsa_split_merge_static", "qsa_score", "qsa_score_ws", "qsa_score_ws_bytes", "qsa_quant_append", "qsa_select", "qsa_part_bytes",
    "qsa_part_offsets",
    "qsa_last_error",
    "alloc_part", "part_views", "chunk_count", "lib", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa.so")

QSA_OK, QSA_ERR_ARG, QSA_ERR_UNSUPPORTED, QSA_ERR_DEVICE = 0, 1, 2, 3
_STATUS = {1: "QSA_ERR_ARG", 2: "QSA_ERR_UNSUPPORTED", 3: "QSA_ERR_DEVICE"}
CHUNK = 64
GROUP = 32
HEAD_DIM = 128

_lib = None


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libqsa.so (built in-tree by sparse_selection_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqsa.so is not built (%s); run `python -m sparse_selection_attention_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.qsa_attn.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, P, P]
        L.qsa_attn.restype = ctypes.c_int
        L.qsa_attn_merge.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, P, P]
        L.qsa_attn_merge.restype = ctypes.c_int
        L.qsa_merge.argtypes = [P, i32, i32, i32, i32, P, P]
        L.qsa_merge.restype = ctypes.c_int
        L.qsa_merge_gated.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
        L.qsa_merge_gated.restype = ctypes.c_int
        L.qsa_attn_merge_gated.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, P, P, P, P]
        L.qsa_attn_merge_gated.restype = ctypes.c_int
        L.qsa_split_merge_static.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, P, P]
        L.qsa_split_merge_static.restype = ctypes.c_int
        L.qsa_score.argtypes = [P, P, i32, i32, i32, i32, i32, f32, f32, P, i64, P]
        L.qsa_score.restype = ctypes.c_int
        L.qsa_score_ws.argtypes = [P, P, i32, i32, i32, i32, i32, f32, f32, P, i64, P, i64, P]
        L.qsa_score_ws.restype = ctypes.c_int
        L.qsa_score_ws_bytes.argtypes = [i32]
        L.qsa_score_ws_bytes.restype = i64
        L.qsa_quant_append.argtypes = [P, P, i32, i32, P, P, P, P, i32, i32, P]
        L.qsa_quant_append.restype = ctypes.c_int
        L.qsa_select.argtypes = [P, i64, i32, i32, i32, P, i32, P]
        L.qsa_select.restype = ctypes.c_int
        L.qsa_part_bytes.argtypes = [i32, i32, i32, i32]
        L.qsa_part_bytes.restype = ctypes.c_size_t
        L.qsa_part_offsets.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t),
                                       ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.qsa_part_offsets.restype = None
        L.qsa_last_error.argtypes = []
        L.qsa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def qsa_last_error() -> str:
    return lib().qsa_last_error().decode()


def _raise_on(status: int):
    if status != QSA_OK:
        raise QsaError(status, qsa_last_error())


def qsa_part_bytes(T: int, H: int, D: int, n_chunks: int) -> int:
    return int(lib().qsa_part_bytes(T, H, D, n_chunks))


def qsa_part_offsets(T: int, H: int, D: int, n_chunks: int) -> Tuple[int, int, int]:
    o, m, l = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    lib().qsa_part_offsets(T, H, D, n_chunks, ctypes.byref(o), ctypes.byref(m), ctypes.byref(l))
    return o.value, m.value, l.value


def chunk_count(ids: Optional[torch.Tensor], pos0: int, T: int) -> int:
    """Chunks per token row: ids_stride / 64, or ceil((pos0 + T) / 64) for implicit rows."""
    if ids is None:
        return (pos0 + T + CHUNK - 1) // CHUNK
    return ids.shape[1] // CHUNK


def alloc_part(T: int, H: int, D: int, C: int, device="cuda") -> torch.Tensor:
    """A byte tensor large enough for the chunk records (torch's allocator aligns to 512 B)."""
    return torch.empty(max(qsa_part_bytes(T, H, D, C), 1), dtype=torch.uint8, device=device)


def part_views(part: torch.Tensor, T: int, H: int, D: int, C: int):
    """(o [T][C][H][D], m [T][C][H], l [T][C][H]) fp32 views into a part buffer."""
    o_off, m_off, l_off = qsa_part_offsets(T, H, D, C)
    f = part.view(torch.uint8)
    o = f[o_off: o_off + 4 * T * C * H * D].view(torch.float32).view(T, C, H, D)
    m = f[m_off: m_off + 4 * T * C * H].view(torch.float32).view(T, C, H)
    l = f[l_off: l_off + 4 * T * C * H].view(torch.float32).view(T, C, H)
    return o, m, l


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims (got shape %s)" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_attn_inputs(q, kq, vq, ksc, vsc, ids):
    _need(q, "q", torch.float16, 3)
    T, H, D = q.shape
    _need(kq, "kq", torch.int8, 2)
    _need(vq, "vq", torch.int8, 2)
    _need(ksc, "ksc", torch.float16, 2)
    _need(vsc, "vsc", torch.float16, 2)
    n_cells = kq.shape[0]
    if kq.shape != (n_cells, D) or vq.shape != (n_cells, D):
        raise ValueError("kq and vq must be [n_cells][%d]" % D)
    if ksc.shape != (n_cells, D // GROUP) or vsc.shape != (n_cells, D // GROUP):
        raise ValueError("ksc and vsc must be [n_cells][%d]" % (D // GROUP))
    stride = 0
    if ids is not None:
        _need(ids, "ids", torch.int32, 2)
        if ids.shape[0] != T:
            raise ValueError("ids must have T rows")
        stride = ids.shape[1]
    return T, H, D, n_cells, stride


def qsa_attn_merge(q: torch.Tensor, kq: torch.Tensor, vq: torch.Tensor, ksc: torch.Tensor, vsc: torch.Tensor,
                   ids: Optional[torch.Tensor], pos0: int, scale: float, out: torch.Tensor, stream=None) -> None:
    """Attention and the merge in one dispatch: fp16 out [T][H][D], no chunk records."""
    T, H, D, n_cells, stride = _check_attn_inputs(q, kq, vq, ksc, vsc, ids)
    _need(out, "out", torch.float16, 3)
    if tuple(out.shape) != (T, H, D):
        raise ValueError("out must be [T][H][D]")
    _raise_on(lib().qsa_attn_merge(_ptr(q), _ptr(kq), _ptr(vq), _ptr(ksc), _ptr(vsc), n_cells, _ptr(ids), stride,
                                   pos0, T, H, D, float(scale), _ptr(out), _stream(stream)))


STATIC_PART_BYTES = 16 << 20


def qsa_split_merge_static(q: torch.Tensor, kq: torch.Tensor, vq: torch.Tensor, ksc: torch.Tensor,
                           vsc: torch.Tensor, ids: Optional[torch.Tensor], pos0: int, scale: float,
                           out: torch.Tensor, stream=None) -> None:
    """qsa_attn then qsa_merge with the chunk records in the library's static
    workspace (no allocation; at most STATIC_PART_BYTES of records)."""
    T, H, D, n_cells, stride = _check_attn_inputs(q, kq, vq, ksc, vsc, ids)
    _need(out, "out", torch.float16, 3)
    if tuple(out.shape) != (T, H, D):
        raise ValueError("out must be [T][H][D]")
    _raise_on(lib().qsa_split_merge_static(_ptr(q), _ptr(kq), _ptr(vq), _ptr(ksc), _ptr(vsc), n_cells, _ptr(ids),
                                           stride, pos0, T, H, D, float(scale), _ptr(out), _stream(stream)))


def qsa_attn(q: torch.Tensor, kq: torch.Tensor, vq: torch.Tensor, ksc: torch.Tensor, vsc: torch.Tensor,
             ids: Optional[torch.Tensor], pos0: int, scale: float, part: torch.Tensor,
             stream=None) -> int:
    """Chunk records of explicit-selection attention; returns the chunk count C.

    q fp16 [T][H][D]; kq, vq int8 [n_cells][D]; ksc, vsc fp16 [n_cells][D/32];
    ids int32 [T][64*C] with -1 poison, or None for implicit all-causal rows;
    part: a byte tensor of at least qsa_part_bytes(T, H, D, C) bytes.
    """
    T, H, D, n_cells, stride = _check_attn_inputs(q, kq, vq, ksc, vsc, ids)
    C = chunk_count(ids, pos0, T)
    if part.device.type != "cuda" or not part.is_contiguous():
        raise ValueError("part must be a contiguous device tensor")
    if part.numel() * part.element_size() < qsa_part_bytes(T, H, D, C):
        raise ValueError("part is smaller than qsa_part_bytes(T, H, D, C)")
    _raise_on(lib().qsa_attn(_ptr(q), _ptr(kq), _ptr(vq), _ptr(ksc), _ptr(vsc), n_cells, _ptr(ids), stride,
                             pos0, T, H, D, float(scale), _ptr(part), _stream(stream)))
    return C


def qsa_merge(part: torch.Tensor, n_chunks: int, out: torch.Tensor, stream=None) -> None:
    """Max-first merge of chunk records into out (fp16 [T][H][D])."""
    _need(out, "out", torch.float16, 3)
    T, H, D = out.shape
    if part.device.type != "cuda" or not part.is_contiguous():
        raise ValueError("part must be a contiguous device tensor")
    if part.numel() * part.element_size() < qsa_part_bytes(T, H, D, n_chunks):
        raise ValueError("part is smaller than qsa_part_bytes(T, H, D, C)")
    _raise_on(lib().qsa_merge(_ptr(part), n_chunks, T, H, D, _ptr(out), _stream(stream)))


def _check_gate(gate: torch.Tensor, sums16: Optional[torch.Tensor], T: int, H: int, D: int):
    _need(gate, "gate", torch.float32, 3)
    if tuple(gate.shape) != (T, H, D):
        raise ValueError("gate must be [T][H][D]")
    if sums16 is not None:
        _need(sums16, "sums16", torch.float32, 3)
        if tuple(sums16.shape) != (T, H, D // 16):
            raise ValueError("sums16 must be [T][H][D/16]")


def qsa_merge_gated(part: torch.Tensor, n_chunks: int, gate: torch.Tensor, out: torch.Tensor,
                    sums16: Optional[torch.Tensor] = None, stream=None) -> None:
    """Max-first merge with the sigmoid gate: out = fp16(sigmoid(gate) * merged),
    gate fp32 [T][H][D]; optional per-16 sums of out into sums16 (fp32 [T][H][D/16])."""
    _need(out, "out", torch.float16, 3)
    T, H, D = out.shape
    _check_gate(gate, sums16, T, H, D)
    if part.device.type != "cuda" or not part.is_contiguous():
        raise ValueError("part must be a contiguous device tensor")
    if part.numel() * part.element_size() < qsa_part_bytes(T, H, D, n_chunks):
        raise ValueError("part is smaller than qsa_part_bytes(T, H, D, C)")
    _raise_on(lib().qsa_merge_gated(_ptr(part), n_chunks, T, H, D, _ptr(gate), _ptr(out), _ptr(sums16),
                                    _stream(stream)))


def qsa_attn_merge_gated(q: torch.Tensor, kq: torch.Tensor, vq: torch.Tensor, ksc: torch.Tensor,
                         vsc: torch.Tensor, ids: Optional[torch.Tensor], pos0: int, scale: float,
                         gate: torch.Tensor, out: torch.Tensor, sums16: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """Attention, merge and sigmoid gate in one dispatch (see qsa_merge_gated)."""
    T, H, D, n_cells, stride = _check_attn_inputs(q, kq, vq, ksc, vsc, ids)
    _need(out, "out", torch.float16, 3)
    if tuple(out.shape) != (T, H, D):
        raise ValueError("out must be [T][H][D]")
    _check_gate(gate, sums16, T, H, D)
    _raise_on(lib().qsa_attn_merge_gated(_ptr(q), _ptr(kq), _ptr(vq), _ptr(ksc), _ptr(vsc), n_cells, _ptr(ids),
                                         stride, pos0, T, H, D, float(scale), _ptr(gate), _ptr(out), _ptr(sums16),
                                         _stream(stream)))


def qsa_score(q: torch.Tensor, k: torch.Tensor, pos0: int, scale: float, dead: float,
              scores: torch.Tensor, stream=None) -> None:
    """fp32 causal scores with a dead-key tail into scores (fp32 [T][row_stride])."""
    _need(q, "q", torch.float32, 3)
    _need(k, "k", torch.float32, 2)
    _need(scores, "scores", torch.float32, 2)
    T, Hs, D = q.shape
    if k.shape[1] != D:
        raise ValueError("k must be [n_cells][%d]" % D)
    if scores.shape[0] != T:
        raise ValueError("scores must have T rows")
    _raise_on(lib().qsa_score(_ptr(q), _ptr(k), k.shape[0], pos0, T, Hs, D, float(scale), float(dead),
                              _ptr(scores), scores.shape[1], _stream(stream)))


def qsa_score_ws_bytes(T: int) -> int:
    return int(lib().qsa_score_ws_bytes(T))


def qsa_score_ws(q: torch.Tensor, k: torch.Tensor, pos0: int, scale: float, dead: float,
                 scores: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """qsa_score with the head sum of q taken once, through workspace (a contiguous
    byte tensor on the same device, at least qsa_score_ws_bytes(T) bytes)."""
    _need(q, "q", torch.float32, 3)
    _need(k, "k", torch.float32, 2)
    _need(scores, "scores", torch.float32, 2)
    _need(workspace, "workspace", torch.uint8, 1)
    T, Hs, D = q.shape
    if k.shape[1] != D:
        raise ValueError("k must be [n_cells][%d]" % D)
    if scores.shape[0] != T:
        raise ValueError("scores must have T rows")
    _raise_on(lib().qsa_score_ws(_ptr(q), _ptr(k), k.shape[0], pos0, T, Hs, D, float(scale), float(dead),
                                 _ptr(scores), scores.shape[1], _ptr(workspace), workspace.numel(),
                                 _stream(stream)))


def qsa_quant_append(k: torch.Tensor, v: torch.Tensor, kq: torch.Tensor, vq: torch.Tensor, ksc: torch.Tensor,
                     vsc: torch.Tensor, cell0: int, stream=None) -> None:
    """Quantise fp32 rows k, v [n][D] into the int8 cache at cells cell0 .. cell0 + n - 1
    (kq, vq int8 [cap][D]; ksc, vsc fp16 [cap][D/32]), one fp16 scale per 32 elements."""
    _need(k, "k", torch.float32, 2)
    _need(v, "v", torch.float32, 2)
    _need(kq, "kq", torch.int8, 2)
    _need(vq, "vq", torch.int8, 2)
    _need(ksc, "ksc", torch.float16, 2)
    _need(vsc, "vsc", torch.float16, 2)
    n, D = k.shape
    cap = kq.shape[0]
    if tuple(v.shape) != (n, D):
        raise ValueError("k and v must have the same shape")
    if tuple(kq.shape) != (cap, D) or tuple(vq.shape) != (cap, D):
        raise ValueError("kq and vq must be [cap][%d]" % D)
    if tuple(ksc.shape) != (cap, D // GROUP) or tuple(vsc.shape) != (cap, D // GROUP):
        raise ValueError("ksc and vsc must be [cap][%d]" % (D // GROUP))
    _raise_on(lib().qsa_quant_append(_ptr(k), _ptr(v), n, D, _ptr(kq), _ptr(vq), _ptr(ksc), _ptr(vsc), cell0, cap,
                                     _stream(stream)))


def qsa_select(scores: torch.Tensor, pos0: int, K: int, ids: torch.Tensor, stream=None) -> None:
    """Top-K causal cell ids per row of scores (fp32 [T][row_stride]) into ids
    (int32 [T][ids_stride]), ascending, -1 padded."""
    _need(scores, "scores", torch.float32, 2)
    _need(ids, "ids", torch.int32, 2)
    T, row_stride = scores.shape
    if ids.shape[0] != T:
        raise ValueError("ids must have T rows")
    _raise_on(lib().qsa_select(_ptr(scores), row_stride, pos0, T, K, _ptr(ids), ids.shape[1], _stream(stream)))
