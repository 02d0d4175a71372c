"""GPU parity of qsa_quant_append (the int8 cache writer) against the oracle.

Codes and scales are integers decided in binary32 on both sides, so the bar is
bit-exact: every int8 code and every fp16 scale pattern, and every cell outside
the written range left as it was.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

from gpu_util import check_out

pytestmark = pytest.mark.gpu

SENTINEL_CODE = 0x5A
SENTINEL_SCALE = 0x7E00       # an fp16 NaN pattern never produced by the writer


def empty_cache(cap):
    dev = "cuda"
    kq = torch.full((cap, 128), SENTINEL_CODE, dtype=torch.int8, device=dev)
    vq = torch.full((cap, 128), SENTINEL_CODE, dtype=torch.int8, device=dev)
    ksc = torch.full((cap, 4), SENTINEL_SCALE, dtype=torch.int16, device=dev).view(torch.float16)
    vsc = torch.full((cap, 4), SENTINEL_SCALE, dtype=torch.int16, device=dev).view(torch.float16)
    return kq, vq, ksc, vsc


def run(xk, xv, cap, cell0, stream=None):
    kq, vq, ksc, vsc = empty_cache(cap)
    k = torch.from_numpy(xk).cuda()
    v = torch.from_numpy(xv).cuda()
    print("qsa_quant_append n=%d cap=%d cell0=%d" % (xk.shape[0], cap, cell0), flush=True)
    qsa.qsa_quant_append(k, v, kq, vq, ksc, vsc, cell0, stream=stream)
    torch.cuda.synchronize()
    return (kq.cpu().numpy(), vq.cpu().numpy(), ksc.cpu().view(torch.int16).numpy().view(np.uint16),
            vsc.cpu().view(torch.int16).numpy().view(np.uint16))


def check(xk, xv, cap, cell0, stream=None):
    n = xk.shape[0]
    kq, vq, ksc, vsc = run(xk, xv, cap, cell0, stream)
    for x, codes, scales in ((xk, kq, ksc), (xv, vq, vsc)):
        rc, rs = oracle.quant_rows(x)
        assert np.array_equal(codes[cell0:cell0 + n], rc), "codes differ at %s" % (
            np.argwhere(codes[cell0:cell0 + n] != rc)[:5].tolist(),)
        assert np.array_equal(scales[cell0:cell0 + n], rs), "scales differ at %s" % (
            np.argwhere(scales[cell0:cell0 + n] != rs)[:5].tolist(),)
        outside = np.r_[0:cell0, cell0 + n:cap]
        assert np.all(codes[outside] == SENTINEL_CODE)
        assert np.all(scales[outside] == SENTINEL_SCALE)


@pytest.mark.parametrize("kind", synth.ROW_KINDS)
def test_prompt_rows_bitwise(kind):
    # a prompt's worth of rows (1984) appended after 3000 cached cells
    xk = synth.cache_rows(1984, kind=kind, which=0)
    xv = synth.cache_rows(1984, kind=kind, which=1)
    check(xk, xv, cap=5100, cell0=3000)


def test_whole_long_context_layer_bitwise():
    # the long-context cache of one layer, 31984 rows, written from cell 0
    xk = synth.cache_rows(31984, kind="normal", which=0)
    xv = synth.cache_rows(31984, kind="spread", which=1)
    check(xk, xv, cap=31984, cell0=0)


@pytest.mark.parametrize("n,cell0,cap", [(1, 0, 1), (1, 3000, 3001), (2, 7, 20), (3, 17, 20), (17, 1, 18),
                                         (15, 0, 64), (33, 31, 64)])
def test_ragged_counts_and_positions(n, cell0, cap):
    xk = synth.cache_rows(n, seed=11, kind="special", which=0)
    xv = synth.cache_rows(n, seed=11, kind="ties", which=1)
    check(xk, xv, cap=cap, cell0=cell0)


def test_zero_rows_touch_nothing():
    kq, vq, ksc, vsc = empty_cache(8)
    z = torch.zeros(0, 128, dtype=torch.float32, device="cuda")
    qsa.qsa_quant_append(z, z, kq, vq, ksc, vsc, 8)
    torch.cuda.synchronize()
    assert torch.all(kq == SENTINEL_CODE) and torch.all(vq == SENTINEL_CODE)


def test_on_a_side_stream():
    xk = synth.cache_rows(500, seed=3, kind="normal", which=0)
    xv = synth.cache_rows(500, seed=3, kind="normal", which=1)
    s = torch.cuda.Stream()
    check(xk, xv, cap=600, cell0=50, stream=s)


def test_capacity_is_checked_on_host():
    kq, vq, ksc, vsc = empty_cache(10)
    k = torch.zeros(4, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(qsa.QsaError):
        qsa.qsa_quant_append(k, k, kq, vq, ksc, vsc, 7)
    torch.cuda.synchronize()
    assert torch.all(kq == SENTINEL_CODE)


def test_decode_step_append_then_attend():
    # decode: the new token's K/V row is appended at cell p, then the token
    # attends over its window (sink, local, itself), which now holds that row
    pos0, ntok = 3000, 2
    case = synth.mtp(ntok)
    L = case.layers[0]
    dev = "cuda"
    kq = torch.from_numpy(L.kq).to(dev)
    vq = torch.from_numpy(L.vq).to(dev)
    ksc = torch.from_numpy(L.ksc).to(dev)
    vsc = torch.from_numpy(L.vsc).to(dev)
    xk = synth.cache_rows(ntok, seed=21, kind="normal", which=0)
    xv = synth.cache_rows(ntok, seed=21, kind="normal", which=1)
    qsa.qsa_quant_append(torch.from_numpy(xk).to(dev), torch.from_numpy(xv).to(dev), kq, vq, ksc, vsc, pos0)
    q = torch.from_numpy(L.q).to(dev)
    ids = torch.from_numpy(case.ids).to(dev)
    out = torch.empty(ntok, L.q.shape[1], 128, dtype=torch.float16, device=dev)
    qsa.qsa_attn_merge(q, kq, vq, ksc, vsc, ids, pos0, float(case.scale), out)
    torch.cuda.synchronize()

    # oracle: its own quantisation of the same rows, then its own attention
    rk, rks = oracle.quant_rows(xk)
    rv, rvs = oracle.quant_rows(xv)
    okq, ovq, oks, ovs = L.kq.copy(), L.vq.copy(), L.ksc.copy(), L.vsc.copy()
    okq[pos0:pos0 + ntok], ovq[pos0:pos0 + ntok] = rk, rv
    oks[pos0:pos0 + ntok], ovs[pos0:pos0 + ntok] = rks.view(np.float16), rvs.view(np.float16)
    assert np.array_equal(kq.cpu().numpy(), okq) and np.array_equal(vq.cpu().numpy(), ovq)
    ref64, _, _ = oracle.attn(L.q, okq, ovq, oks, ovs, case.ids, pos0, float(case.scale))
    check_out(out.cpu().numpy(), ref64, "after append")
