"""C-ABI checks that need no GPU: the library loads, exports what include/*.h
declares, sizes the part workspace, and rejects bad arguments on the host
before anything reaches a device."""
import ctypes
import glob
import os
import re

import pytest

import sparse_selection_attention_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names |= set(re.findall(r"QSA_API\s+[^;(]*?\b(qsa_\w+)\s*\(", text))
    return names


def test_library_loads_and_exports_every_declared_symbol():
    L = qsa.lib()
    names = declared_symbols()
    assert {"qsa_attn", "qsa_attn_merge", "qsa_merge", "qsa_score", "qsa_score_ws", "qsa_score_ws_bytes",
            "qsa_quant_append", "qsa_select",
            "qsa_merge_gated", "qsa_attn_merge_gated",
            "qsa_part_bytes", "qsa_part_offsets", "qsa_last_error"} <= names
    for n in names:
        assert hasattr(L, n), n


def test_no_unexpected_exports():
    out = os.popen("nm -D --defined-only %s" % qsa.LIB_PATH).read()
    exported = set(re.findall(r"\bT (qsa_\w+)", out))
    assert exported == declared_symbols()


def test_part_layout():
    T, H, D, C = 1984, 12, 128, 33
    o, m, l = qsa.qsa_part_offsets(T, H, D, C)
    assert o == 0
    assert m == 4 * T * C * H * D                      # already a multiple of 256
    assert l == m + ((4 * T * C * H + 255) // 256) * 256
    assert qsa.qsa_part_bytes(T, H, D, C) == l + ((4 * T * C * H + 255) // 256) * 256
    # same bytes per record as the pages' {max, denominator, output[D]} records
    assert 4 * T * C * H * (2 + D) <= qsa.qsa_part_bytes(T, H, D, C) < 4 * T * C * H * (2 + D) + 512
    for T_, H_, C_ in [(1, 1, 1), (3, 5, 7), (17, 16, 2)]:
        o, m, l = qsa.qsa_part_offsets(T_, H_, 128, C_)
        assert o % 256 == 0 and m % 256 == 0 and l % 256 == 0
        assert m >= 4 * T_ * C_ * H_ * 128 and l >= m + 4 * T_ * C_ * H_
    assert qsa.qsa_part_bytes(-1, 1, 128, 1) == 0


FAKE = 0x10000        # a 256-byte aligned host address that is never dereferenced


def attn(**kw):
    a = dict(q=FAKE, kq=FAKE, vq=FAKE, ksc=FAKE, vsc=FAKE, n_cells=100, ids=FAKE, ids_stride=64,
             pos0=10, T=4, H=12, D=128, scale=0.1, part=FAKE, stream=None)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_attn(P(a["q"]), P(a["kq"]), P(a["vq"]), P(a["ksc"]), P(a["vsc"]), a["n_cells"],
                              P(a["ids"]), a["ids_stride"], a["pos0"], a["T"], a["H"], a["D"], a["scale"],
                              P(a["part"]), P(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), qsa.QSA_ERR_ARG),
    (dict(pos0=-3), qsa.QSA_ERR_ARG),
    (dict(n_cells=-1), qsa.QSA_ERR_ARG),
    (dict(H=0), qsa.QSA_ERR_ARG),
    (dict(H=17), qsa.QSA_ERR_UNSUPPORTED),
    (dict(D=64), qsa.QSA_ERR_UNSUPPORTED),
    (dict(D=256), qsa.QSA_ERR_UNSUPPORTED),
    (dict(ids_stride=0), qsa.QSA_ERR_ARG),
    (dict(ids_stride=100), qsa.QSA_ERR_ARG),
    (dict(ids_stride=-64), qsa.QSA_ERR_ARG),
    (dict(q=None), qsa.QSA_ERR_ARG),
    (dict(kq=None), qsa.QSA_ERR_ARG),
    (dict(vq=None), qsa.QSA_ERR_ARG),
    (dict(ksc=None), qsa.QSA_ERR_ARG),
    (dict(vsc=None), qsa.QSA_ERR_ARG),
    (dict(part=None), qsa.QSA_ERR_ARG),
    (dict(q=FAKE + 8), qsa.QSA_ERR_ARG),
    (dict(kq=FAKE + 4), qsa.QSA_ERR_ARG),
    (dict(vq=FAKE + 1), qsa.QSA_ERR_ARG),
    (dict(ksc=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(vsc=FAKE + 4), qsa.QSA_ERR_ARG),
    (dict(part=FAKE + 128), qsa.QSA_ERR_ARG),
    (dict(ids=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(pos0=2**31 - 2, T=4), qsa.QSA_ERR_ARG),
])
def test_attn_rejects_bad_arguments_on_host(kw, status):
    assert attn(**kw) == status
    assert qsa.qsa_last_error() != ""


def test_zero_tokens_is_a_no_op():
    # T == 0 returns OK before touching any pointer or device
    assert attn(T=0, q=None, kq=None, part=None) == qsa.QSA_OK
    assert qsa.qsa_last_error() == ""
    P = ctypes.c_void_p
    assert qsa.lib().qsa_merge(P(None), 5, 0, 12, 128, P(None), P(None)) == qsa.QSA_OK
    assert qsa.lib().qsa_score(P(None), P(None), 10, 10, 0, 1, 128, 1.0, 0.0, P(None), 10, P(None)) == qsa.QSA_OK
    assert qsa.lib().qsa_score_ws(P(None), P(None), 10, 10, 0, 1, 128, 1.0, 0.0, P(None), 10, P(None), 0,
                                  P(None)) == qsa.QSA_OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, 3, -1, 12, 128, FAKE), qsa.QSA_ERR_ARG),
    ((FAKE, -1, 2, 12, 128, FAKE), qsa.QSA_ERR_ARG),
    ((FAKE, 3, 2, 0, 128, FAKE), qsa.QSA_ERR_ARG),
    ((FAKE, 3, 2, 17, 128, FAKE), qsa.QSA_ERR_UNSUPPORTED),
    ((FAKE, 3, 2, 12, 96, FAKE), qsa.QSA_ERR_UNSUPPORTED),
    ((None, 3, 2, 12, 128, FAKE), qsa.QSA_ERR_ARG),
    ((FAKE, 3, 2, 12, 128, None), qsa.QSA_ERR_ARG),
    ((FAKE + 64, 3, 2, 12, 128, FAKE), qsa.QSA_ERR_ARG),
    ((FAKE, 3, 2, 12, 128, FAKE + 2), qsa.QSA_ERR_ARG),
])
def test_merge_rejects_bad_arguments_on_host(args, status):
    P = ctypes.c_void_p
    part, C, T, H, D, out = args
    assert qsa.lib().qsa_merge(P(part), C, T, H, D, P(out), P(None)) == status
    assert qsa.qsa_last_error().startswith("qsa_merge")


def score(**kw):
    a = dict(q=FAKE, k=FAKE, n_cells=100, pos0=10, T=4, Hs=1, D=128, scale=1.0, dead=-1.0, scores=FAKE,
             row_stride=14)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_score(P(a["q"]), P(a["k"]), a["n_cells"], a["pos0"], a["T"], a["Hs"], a["D"],
                               a["scale"], a["dead"], P(a["scores"]), a["row_stride"], P(None))


@pytest.mark.parametrize("kw,status", [
    (dict(T=-2), qsa.QSA_ERR_ARG),
    (dict(pos0=-2), qsa.QSA_ERR_ARG),
    (dict(Hs=0), qsa.QSA_ERR_ARG),
    (dict(Hs=17), qsa.QSA_ERR_UNSUPPORTED),
    (dict(D=64), qsa.QSA_ERR_UNSUPPORTED),
    (dict(n_cells=13), qsa.QSA_ERR_ARG),
    (dict(row_stride=13), qsa.QSA_ERR_ARG),
    (dict(q=None), qsa.QSA_ERR_ARG),
    (dict(k=None), qsa.QSA_ERR_ARG),
    (dict(scores=None), qsa.QSA_ERR_ARG),
    (dict(q=FAKE + 4), qsa.QSA_ERR_ARG),
    (dict(k=FAKE + 8), qsa.QSA_ERR_ARG),
    (dict(scores=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(T=64 * 65536, pos0=0, n_cells=64 * 65536, row_stride=64 * 65536), qsa.QSA_ERR_ARG),
])
def test_score_rejects_bad_arguments_on_host(kw, status):
    assert score(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_score")
    assert score_ws(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_score_ws")


def score_ws(**kw):
    a = dict(q=FAKE, k=FAKE, n_cells=100, pos0=10, T=4, Hs=1, D=128, scale=1.0, dead=-1.0, scores=FAKE,
             row_stride=14, ws=FAKE, ws_bytes=64 * 512)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_score_ws(P(a["q"]), P(a["k"]), a["n_cells"], a["pos0"], a["T"], a["Hs"], a["D"],
                                  a["scale"], a["dead"], P(a["scores"]), a["row_stride"], P(a["ws"]),
                                  a["ws_bytes"], P(None))


def test_score_workspace_size():
    # 512 bytes per row, rows rounded up to a multiple of 64
    for T, want in [(-3, 0), (0, 0), (1, 32768), (64, 32768), (65, 65536), (1984, 1015808)]:
        assert qsa.qsa_score_ws_bytes(T) == want, T


@pytest.mark.parametrize("kw", [dict(ws=None), dict(ws_bytes=64 * 512 - 1), dict(ws_bytes=0),
                                dict(ws=FAKE + 8), dict(T=65, n_cells=100, row_stride=75)])
def test_score_ws_rejects_bad_workspaces_on_host(kw):
    assert score_ws(**kw) == qsa.QSA_ERR_ARG
    assert qsa.qsa_last_error().startswith("qsa_score_ws")


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(2, 1, 128, dtype=torch.float16)
    kq = torch.zeros(4, 128, dtype=torch.int8)
    sc = torch.ones(4, 4, dtype=torch.float16)
    with pytest.raises(ValueError):
        qsa.qsa_attn(q, kq, kq, sc, sc, None, 2, 0.1, torch.zeros(1 << 16, dtype=torch.uint8))


def attn_merge(**kw):
    a = dict(q=FAKE, kq=FAKE, vq=FAKE, ksc=FAKE, vsc=FAKE, n_cells=100, ids=FAKE, ids_stride=64,
             pos0=10, T=4, H=12, D=128, scale=0.1, out=FAKE)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_attn_merge(P(a["q"]), P(a["kq"]), P(a["vq"]), P(a["ksc"]), P(a["vsc"]), a["n_cells"],
                                    P(a["ids"]), a["ids_stride"], a["pos0"], a["T"], a["H"], a["D"], a["scale"],
                                    P(a["out"]), P(None))


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), qsa.QSA_ERR_ARG),
    (dict(H=0), qsa.QSA_ERR_ARG),
    (dict(H=17), qsa.QSA_ERR_UNSUPPORTED),
    (dict(D=64), qsa.QSA_ERR_UNSUPPORTED),
    (dict(ids_stride=32), qsa.QSA_ERR_ARG),
    (dict(n_cells=(1 << 25) + 1), qsa.QSA_ERR_UNSUPPORTED),
    (dict(out=None), qsa.QSA_ERR_ARG),
    (dict(out=FAKE + 8), qsa.QSA_ERR_ARG),
    (dict(q=None), qsa.QSA_ERR_ARG),
    (dict(ksc=FAKE + 4), qsa.QSA_ERR_ARG),
])
def test_attn_merge_rejects_bad_arguments_on_host(kw, status):
    assert attn_merge(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_attn_merge")


def test_attn_merge_zero_tokens_is_a_no_op():
    assert attn_merge(T=0, q=None, out=None) == qsa.QSA_OK


def test_build_rejects_spilling_kernels():
    from sparse_selection_attention_amd import build
    text = "\n".join([
        "a.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 120 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     Occupancy [waves/SIMD]: 4 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 60 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:17:1: remark: Function Name: kern_c [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:17:1: remark:     VGPRs: 57 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:17:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:17:1: remark:     SGPRs Spill: 70 [-Rpass-analysis=kernel-resource-usage]",
    ])
    res = build.kernel_resources(text)
    assert res == {"kern_a": {"VGPRs": 120, "ScratchSize": 0, "Occupancy": 4},
                   "kern_b": {"VGPRs": 128, "ScratchSize": 60},
                   "kern_c": {"VGPRs": 57, "ScratchSize": 0, "SGPRSpill": 70}}


def quant(**kw):
    a = dict(k=FAKE, v=FAKE, n_rows=10, D=128, kq=FAKE, vq=FAKE, ksc=FAKE, vsc=FAKE, cell0=5, cap=100)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_quant_append(P(a["k"]), P(a["v"]), a["n_rows"], a["D"], P(a["kq"]), P(a["vq"]),
                                      P(a["ksc"]), P(a["vsc"]), a["cell0"], a["cap"], P(None))


@pytest.mark.parametrize("kw,status", [
    (dict(n_rows=-1), qsa.QSA_ERR_ARG),
    (dict(cell0=-1), qsa.QSA_ERR_ARG),
    (dict(cap=-1), qsa.QSA_ERR_ARG),
    (dict(D=64), qsa.QSA_ERR_UNSUPPORTED),
    (dict(cell0=91), qsa.QSA_ERR_ARG),             # 91 + 10 > 100
    (dict(cell0=2**31 - 5, cap=2**31 - 1), qsa.QSA_ERR_ARG),
    (dict(k=None), qsa.QSA_ERR_ARG),
    (dict(v=None), qsa.QSA_ERR_ARG),
    (dict(kq=None), qsa.QSA_ERR_ARG),
    (dict(vsc=None), qsa.QSA_ERR_ARG),
    (dict(k=FAKE + 8), qsa.QSA_ERR_ARG),
    (dict(v=FAKE + 4), qsa.QSA_ERR_ARG),
    (dict(kq=FAKE + 4), qsa.QSA_ERR_ARG),
    (dict(vq=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(ksc=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(vsc=FAKE + 4), qsa.QSA_ERR_ARG),
])
def test_quant_append_rejects_bad_arguments_on_host(kw, status):
    assert quant(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_quant_append")


def test_quant_append_zero_rows_is_a_no_op():
    assert quant(n_rows=0, k=None, kq=None, cell0=100) == qsa.QSA_OK
    assert qsa.qsa_last_error() == ""


def select(**kw):
    a = dict(scores=FAKE, row_stride=100, pos0=50, T=10, K=20, ids=FAKE, ids_stride=64)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_select(P(a["scores"]), a["row_stride"], a["pos0"], a["T"], a["K"], P(a["ids"]),
                                a["ids_stride"], P(None))


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), qsa.QSA_ERR_ARG),
    (dict(pos0=-1), qsa.QSA_ERR_ARG),
    (dict(K=0), qsa.QSA_ERR_ARG),
    (dict(row_stride=59), qsa.QSA_ERR_ARG),          # < pos0 + T
    (dict(ids_stride=0), qsa.QSA_ERR_ARG),
    (dict(ids_stride=32), qsa.QSA_ERR_ARG),          # not a multiple of 64
    (dict(K=100, pos0=100, row_stride=200, ids_stride=64), qsa.QSA_ERR_ARG),   # min(K, pos0 + T) = 100 > 64
    (dict(pos0=2**25 - 5, T=10, row_stride=2**25 + 5), qsa.QSA_ERR_UNSUPPORTED),
    (dict(scores=None), qsa.QSA_ERR_ARG),
    (dict(ids=None), qsa.QSA_ERR_ARG),
    (dict(scores=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(ids=FAKE + 1), qsa.QSA_ERR_ARG),
])
def test_select_rejects_bad_arguments_on_host(kw, status):
    assert select(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_select")


def test_select_zero_rows_is_a_no_op():
    assert select(T=0, scores=None, ids=None) == qsa.QSA_OK


# ---------------------------------------------------------------------------
# the cache must hold every causal cell of the call: n_cells >= pos0 + T


@pytest.mark.parametrize("fn", ["attn", "attn_merge", "attn_merge_gated"])
def test_attention_rejects_a_cache_shorter_than_the_causal_range(fn):
    call = {"attn": attn, "attn_merge": attn_merge, "attn_merge_gated": attn_merge_gated}[fn]
    assert call(n_cells=13, pos0=10, T=4) == qsa.QSA_ERR_ARG
    assert "n_cells" in qsa.qsa_last_error()
    assert call(n_cells=13, pos0=10, T=4, ids=None) == qsa.QSA_ERR_ARG      # implicit rows too
    assert call(n_cells=0, pos0=0, T=1) == qsa.QSA_ERR_ARG
    # exactly pos0 + T cells passes the host checks (the next check needs a device)
    assert call(n_cells=14, pos0=10, T=4) != qsa.QSA_ERR_ARG


# ---------------------------------------------------------------------------
# gated entry points


def attn_merge_gated(**kw):
    a = dict(q=FAKE, kq=FAKE, vq=FAKE, ksc=FAKE, vsc=FAKE, n_cells=100, ids=FAKE, ids_stride=64,
             pos0=10, T=4, H=12, D=128, scale=0.1, gate=FAKE, out=FAKE, sums=None)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_attn_merge_gated(P(a["q"]), P(a["kq"]), P(a["vq"]), P(a["ksc"]), P(a["vsc"]),
                                          a["n_cells"], P(a["ids"]), a["ids_stride"], a["pos0"], a["T"], a["H"],
                                          a["D"], a["scale"], P(a["gate"]), P(a["out"]), P(a["sums"]), P(None))


def merge_gated(**kw):
    a = dict(part=FAKE, C=3, T=2, H=12, D=128, gate=FAKE, out=FAKE, sums=FAKE)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_merge_gated(P(a["part"]), a["C"], a["T"], a["H"], a["D"], P(a["gate"]), P(a["out"]),
                                     P(a["sums"]), P(None))


@pytest.mark.parametrize("kw,status", [
    (dict(gate=None), qsa.QSA_ERR_ARG),
    (dict(gate=FAKE + 8), qsa.QSA_ERR_ARG),
    (dict(sums=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(out=None), qsa.QSA_ERR_ARG),
    (dict(out=FAKE + 8), qsa.QSA_ERR_ARG),
    (dict(H=17), qsa.QSA_ERR_UNSUPPORTED),
    (dict(D=64), qsa.QSA_ERR_UNSUPPORTED),
    (dict(T=-1), qsa.QSA_ERR_ARG),
    (dict(ids_stride=32), qsa.QSA_ERR_ARG),
])
def test_attn_merge_gated_rejects_bad_arguments_on_host(kw, status):
    assert attn_merge_gated(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_attn_merge_gated")


@pytest.mark.parametrize("kw,status", [
    (dict(gate=None), qsa.QSA_ERR_ARG),
    (dict(gate=FAKE + 4), qsa.QSA_ERR_ARG),
    (dict(sums=FAKE + 1), qsa.QSA_ERR_ARG),
    (dict(part=None), qsa.QSA_ERR_ARG),
    (dict(part=FAKE + 64), qsa.QSA_ERR_ARG),
    (dict(out=FAKE + 2), qsa.QSA_ERR_ARG),
    (dict(C=-1), qsa.QSA_ERR_ARG),
    (dict(H=0), qsa.QSA_ERR_ARG),
    (dict(H=17), qsa.QSA_ERR_UNSUPPORTED),
    (dict(D=96), qsa.QSA_ERR_UNSUPPORTED),
])
def test_merge_gated_rejects_bad_arguments_on_host(kw, status):
    assert merge_gated(**kw) == status
    assert qsa.qsa_last_error().startswith("qsa_merge_gated")


def test_gated_zero_tokens_is_a_no_op():
    assert merge_gated(T=0, part=None, gate=None, out=None, sums=None) == qsa.QSA_OK
    assert attn_merge_gated(T=0, q=None, gate=None, out=None) == qsa.QSA_OK
    # sums16 is optional: a NULL one passes the host checks
    assert merge_gated(sums=None) != qsa.QSA_ERR_ARG
    assert attn_merge_gated(sums=None) != qsa.QSA_ERR_ARG


# ---------------------------------------------------------------------------
# the split path through the library's static workspace


def split_static(**kw):
    a = dict(q=FAKE, kq=FAKE, vq=FAKE, ksc=FAKE, vsc=FAKE, n_cells=40000, ids=FAKE, ids_stride=2112,
             pos0=30000, T=64, H=12, D=128, scale=0.1, out=FAKE)
    a.update(kw)
    P = ctypes.c_void_p
    return qsa.lib().qsa_split_merge_static(P(a["q"]), P(a["kq"]), P(a["vq"]), P(a["ksc"]), P(a["vsc"]),
                                            a["n_cells"], P(a["ids"]), a["ids_stride"], a["pos0"], a["T"], a["H"],
                                            a["D"], a["scale"], P(a["out"]), P(None))


def test_split_static_limit_and_host_checks():
    # 64 tokens of 33 chunks at 12 heads fit the 16 MiB workspace; 90 do not
    assert qsa.qsa_part_bytes(64, 12, 128, 33) <= qsa.STATIC_PART_BYTES < qsa.qsa_part_bytes(90, 12, 128, 33)
    assert split_static(T=90) == qsa.QSA_ERR_ARG
    assert "static workspace" in qsa.qsa_last_error()
    assert split_static(T=64) != qsa.QSA_ERR_ARG           # fits: the next check needs a device
    assert split_static(T=0, q=None, out=None) == qsa.QSA_OK
    assert split_static(out=None) == qsa.QSA_ERR_ARG
    assert split_static(out=FAKE + 8) == qsa.QSA_ERR_ARG
    assert split_static(n_cells=100) == qsa.QSA_ERR_ARG    # n_cells < pos0 + T
    assert split_static(H=17) == qsa.QSA_ERR_UNSUPPORTED
    assert split_static(ids=None, pos0=0, n_cells=6000, T=6000, H=12) == qsa.QSA_ERR_ARG   # implicit rows too large


def test_static_workspace_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "qsa.h")).read()
    m = re.search(r"#define QSA_STATIC_PART_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == qsa.STATIC_PART_BYTES
