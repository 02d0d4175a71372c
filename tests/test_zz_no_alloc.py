"""qsa_split_merge_static, the entry point that allocates nothing: its chunk
records live in the library's static per-device workspace. Its output must
match qsa_attn + qsa_merge with a caller workspace (the same kernels: bit for
bit) and the oracle (the workload bar), on two calls in a row, the second with
a smaller input, and on implicit rows; a call whose records do not fit is
refused before anything is launched."""
import numpy as np
import pytest
import torch

import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

from gpu_util import check_out, dev, oracle_tokens, sample_tokens, to_dev

pytestmark = pytest.mark.gpu


def _inputs(L, ids):
    return [to_dev(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc)] + [to_dev(ids) if ids is not None else None]


def _split_with_workspace(t, pos0, scale):
    q, kq, vq, ksc, vsc, ids = t
    T, H, D = q.shape
    C = qsa.chunk_count(ids, pos0, T)
    part = qsa.alloc_part(T, H, D, C)
    out = torch.empty((T, H, D), dtype=torch.float16, device=dev())
    qsa.qsa_attn(q, kq, vq, ksc, vsc, ids, pos0, float(scale), part)
    qsa.qsa_merge(part, C, out)
    return out


def _static(t, pos0, scale):
    q, kq, vq, ksc, vsc, ids = t
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device=dev())
    qsa.qsa_split_merge_static(q, kq, vq, ksc, vsc, ids, pos0, float(scale), out)
    return out


def test_two_calls_in_a_row_the_second_smaller():
    # 64 long-context tokens (33 chunks x 12 heads: 13.2 MB of records), then
    # a 3-token decode window (6 chunks) that reuses the start of the workspace
    big = synth.long_ctx(layers=1, T=64)
    small = synth.mtp(3)
    cases = [(big, 64), (small, 3)]
    for case, T in cases:
        L = case.layers[0]
        t = _inputs(L, case.ids)
        C = case.n_chunks
        assert qsa.qsa_part_bytes(T, case.H, 128, C) <= qsa.STATIC_PART_BYTES
        ref = _split_with_workspace(t, case.pos0, case.scale)
        got = _static(t, case.pos0, case.scale)
        torch.cuda.synchronize()
        print("static workspace: %s T=%d C=%d" % (case.name, T, C), flush=True)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), case.name
        toks = sample_tokens(T, 12)
        refs = oracle_tokens(L, case.ids, case.pos0, case.scale, toks)
        g = got.cpu().numpy()
        for tk in toks:
            check_out(g[tk], refs[tk]["out64"], "%s t=%d" % (case.name, tk))


def test_implicit_rows():
    case = synth.prompt_start(implicit=True, T=100)
    L = case.layers[0]
    t = _inputs(L, None)
    ref = _split_with_workspace(t, case.pos0, case.scale)
    got = _static(t, case.pos0, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    refs = oracle_tokens(L, None, case.pos0, case.scale, [0, 1, 50, 99])
    g = got.cpu().numpy()
    for tk, r in refs.items():
        check_out(g[tk], r["out64"], "implicit t=%d" % tk)


def test_records_that_do_not_fit_are_refused():
    case = synth.long_ctx(layers=1, T=90)          # 90 x 33 x 12 records: 18.5 MB
    L = case.layers[0]
    t = _inputs(L, case.ids)
    assert qsa.qsa_part_bytes(90, 12, 128, case.n_chunks) > qsa.STATIC_PART_BYTES
    out = torch.full((90, 12, 128), float("nan"), dtype=torch.float16, device=dev())
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_split_merge_static(*t[:5], t[5], case.pos0, float(case.scale), out)
    assert e.value.status == qsa.QSA_ERR_ARG and "static workspace" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(out))
