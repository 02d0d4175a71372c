"""GPU parity of the sigmoid-gated output and its per-16 sums, through the C ABI.

qsa_merge_gated (after qsa_attn), and qsa_attn_merge_gated on both of its
kernels (explicit ids: the per-token kernel; implicit rows: the shared-tile
kernel), against the oracle's records -> merge -> gate chain. The per-16 sums
are checked bit for bit against the exact sums of the GPU's own fp16 outputs
rounded once (numpy's fp64 sum is exact for 16 binary16 values, in any order),
and within the output tolerance of the oracle's sums."""
import numpy as np
import pytest
import torch

import oracle
import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

from gpu_util import OUT_ATOL, check_out, dev, oracle_tokens, sample_tokens, to_dev

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def run_gated(L, ids, pos0, scale, g, path, sums=True):
    """path: "two" (qsa_attn + qsa_merge_gated) or "fused" (qsa_attn_merge_gated).
    Returns numpy (out fp16, sums fp32 or None)."""
    T, H, D = L.q.shape
    q, kq, vq, ksc, vsc = (to_dev(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc))
    ids_t = to_dev(ids) if ids is not None else None
    gt = to_dev(g)
    out = torch.full((T, H, D), float("nan"), dtype=torch.float16, device=dev())
    s = torch.full((T, H, D // 16), float("nan"), dtype=torch.float32, device=dev()) if sums else None
    if path == "two":
        C = qsa.chunk_count(ids_t, pos0, T)
        part = qsa.alloc_part(T, H, D, C)
        qsa.qsa_attn(q, kq, vq, ksc, vsc, ids_t, pos0, float(scale), part)
        qsa.qsa_merge_gated(part, C, gt, out, s)
    else:
        qsa.qsa_attn_merge_gated(q, kq, vq, ksc, vsc, ids_t, pos0, float(scale), gt, out, s)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (s.cpu().numpy() if sums else None)


def exact_sums(out16):
    x = out16.astype(np.float64)
    return x.reshape(x.shape[:-1] + (x.shape[-1] // 16, 16)).sum(-1).astype(np.float32)


def check_gated(out, sums, L, ids, pos0, scale, g, toks, what):
    refs = oracle_tokens(L, ids, pos0, scale, toks)
    worst = 0.0
    for t in toks:
        r64, r16 = oracle.gate(refs[t]["out64"], g[t])
        e, _ = check_out(out[t], r64, "%s t=%d" % (what, t))
        worst = max(worst, e)
        if sums is not None:
            assert np.array_equal(sums[t].view(np.uint32), exact_sums(out[t]).view(np.uint32)), \
                "%s t=%d: sums are not the exact sums of the written values" % (what, t)
            rs = oracle.sums16(r16).astype(np.float64)
            assert np.all(np.abs(sums[t] - rs) <= 16 * OUT_ATOL), "%s t=%d sums" % (what, t)
    return worst


@pytest.mark.parametrize("ntok", [1, 2, 3, 8])
@pytest.mark.parametrize("path", ["two", "fused"])
@pytest.mark.parametrize("kind", ["normal", "special"])
def test_decode_window(ntok, path, kind):
    case = synth.mtp(ntok)
    L = case.layers[0]
    g = synth.gates(ntok, case.H, seed=ntok, kind=kind)
    out, sums = run_gated(L, case.ids, case.pos0, case.scale, g, path)
    _print("gated decode ntok=%d %s %s" % (ntok, path, kind),
           check_gated(out, sums, L, case.ids, case.pos0, case.scale, g, list(range(ntok)), "decode"))


@pytest.mark.parametrize("path", ["two", "fused"])
def test_long_context(path):
    case = synth.long_ctx(layers=1)
    L = case.layers[0]
    g = synth.gates(case.T, case.H, seed=11, kind="special")
    out, sums = run_gated(L, case.ids, case.pos0, case.scale, g, path)
    toks = sample_tokens(case.T, 40, seed=3)
    _print("gated long", path, check_gated(out, sums, L, case.ids, case.pos0, case.scale, g, toks, "long"))


@pytest.mark.parametrize("path", ["two", "fused"])
def test_prompt_start_implicit_rows(path):
    # the fused entry point takes the shared-tile kernel for implicit rows
    case = synth.prompt_start(implicit=True, T=300)
    L = case.layers[0]
    g = synth.gates(case.T, case.H, seed=12, kind="special")
    out, sums = run_gated(L, None, case.pos0, case.scale, g, path)
    _print("gated prompt", path,
           check_gated(out, sums, L, None, case.pos0, case.scale, g, list(range(case.T)), "prompt"))


@pytest.mark.parametrize("implicit", [False, True])
@pytest.mark.parametrize("path", ["two", "fused"])
def test_gate_edges_are_exact(path, implicit):
    """g = +inf reproduces the ungated output bit for bit; g = 0 halves it
    exactly (outputs clear of the fp16 subnormals); g = -inf gives zeros with
    the ungated value's sign."""
    case = synth.prompt_start(implicit=implicit, T=130)
    L = case.layers[0]
    ids = None if implicit else case.ids
    T, H, D = L.q.shape
    q, kq, vq, ksc, vsc = (to_dev(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc))
    ids_t = to_dev(ids) if ids is not None else None
    C = qsa.chunk_count(ids_t, case.pos0, T)
    part = qsa.alloc_part(T, H, D, C)
    y = torch.empty((T, H, D), dtype=torch.float16, device=dev())
    if path == "two":
        qsa.qsa_attn(q, kq, vq, ksc, vsc, ids_t, case.pos0, float(case.scale), part)
        qsa.qsa_merge(part, C, y)
    else:
        qsa.qsa_attn_merge(q, kq, vq, ksc, vsc, ids_t, case.pos0, float(case.scale), y)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for gv in (np.inf, 0.0, -np.inf):
        g = np.full((T, H, D), gv, np.float32)
        out, sums = run_gated(L, ids, case.pos0, case.scale, g, path)
        if gv == np.inf:
            assert np.array_equal(out.view(np.uint16), y.view(np.uint16))
        elif gv == 0.0:
            big = np.abs(y.astype(np.float64)) >= 2.0 ** -13
            assert np.array_equal(out[big].astype(np.float64), y[big].astype(np.float64) * 0.5)
        else:
            assert np.all(out == 0) and np.array_equal(np.signbit(out), np.signbit(y))
        assert np.array_equal(sums.view(np.uint32), exact_sums(out).view(np.uint32))


def test_sums_are_optional_and_do_not_change_the_output():
    case = synth.mtp(4)
    L = case.layers[0]
    g = synth.gates(4, case.H, seed=2)
    for path in ("two", "fused"):
        a, _ = run_gated(L, case.ids, case.pos0, case.scale, g, path, sums=False)
        b, _ = run_gated(L, case.ids, case.pos0, case.scale, g, path, sums=True)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_rows_without_a_valid_slot_give_plus_zero():
    T, H, n_cells = 6, 12, 400
    L = synth.make_layer(31, 0, T, H, n_cells)
    ids = np.full((T, 128), -1, np.int32)
    ids[0, :5] = [1, 2, 3, 4, 5]
    ids[3, 70] = 17
    g = synth.gates(T, H, seed=4, kind="normal")
    for path in ("two", "fused"):
        out, sums = run_gated(L, ids, n_cells - T, synth.SCALE_1_SQRT_128, g, path)
        for t in (1, 2, 4, 5):
            assert np.all(out[t].view(np.uint16) == 0) and np.all(sums[t].view(np.uint32) == 0)
        check_gated(out, sums, L, ids, n_cells - T, synth.SCALE_1_SQRT_128, g, [0, 3], "sparse rows " + path)
