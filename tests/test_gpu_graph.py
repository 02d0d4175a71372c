"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph around the C ABI
calls). The entry points launch kernels only (no allocation, no memset), so a
captured step replays them. Every replay, with eager work and synchronisation
between replays, must give the eager output bit for bit."""
import numpy as np
import pytest
import torch

import sparse_selection_attention_amd as qsa
from sparse_selection_attention_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(ntok):
    mc = synth.mtp(ntok)
    L = mc.layers[0]
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return mc, [up(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc)], up(mc.ids)


@pytest.mark.parametrize("ntok", [1, 8])
@pytest.mark.parametrize("path", ["fused", "two_kernel"])
def test_graph_replays_match_eager(ntok, path):
    mc, (q, kq, vq, ks, vs), ids = _inputs(ntok)
    out = torch.full((ntok, mc.H, 128), float("nan"), dtype=torch.float16, device="cuda")
    part = qsa.alloc_part(ntok, mc.H, 128, mc.n_chunks)

    def step():
        if path == "fused":
            qsa.qsa_attn_merge(q, kq, vq, ks, vs, ids, mc.pos0, float(mc.scale), out)
        else:
            qsa.qsa_attn(q, kq, vq, ks, vs, ids, mc.pos0, float(mc.scale), part)
            qsa.qsa_merge(part, mc.n_chunks, out)

    step()
    torch.cuda.synchronize()
    want = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(3):
        out.fill_(float("nan"))
        scratch.add_(1.0)                    # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (path, ntok, r)
