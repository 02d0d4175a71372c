"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph around the C ABI
calls): fused, two-kernel, and through the static record array. The entry
points launch kernels only (no allocation, no memset), so a captured step
replays them. Every replay, with eager work and synchronisation
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
@pytest.mark.parametrize("path", ["fused", "two_kernel", "static"])
def test_graph_replays_match_eager(ntok, path):
    mc, (q, kq, vq, ks, vs), ids = _inputs(ntok)
    out = torch.full((ntok, mc.H, 128), float("nan"), dtype=torch.float16, device="cuda")
    part = qsa.alloc_part(ntok, mc.H, 128, mc.n_chunks)

    def step():
        if path == "fused":
            qsa.qsa_attn_merge(q, kq, vq, ks, vs, ids, mc.pos0, float(mc.scale), out)
        elif path == "static":           # records in the library's static array, for callers that cannot allocate
            qsa.qsa_split_merge_static(q, kq, vq, ks, vs, ids, mc.pos0, float(mc.scale), out)
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


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.float16 else t.view(torch.int32) if t.element_size() == 4 else t


@pytest.mark.parametrize("T,pos0,Hs,K,attn", [
    (4, 5000, 12, 321, "fused"),            # decode: score, select and fused gated attention
    (4, 5000, 12, 321, "two_kernel"),
    (1024, 30000, 8, 2051, "fused"),        # large enough that the workspace score takes its first pass
])
def test_graph_replays_whole_step(T, pos0, Hs, K, attn):
    """One serving step in one graph: the new rows' K and V appended to the
    cache, scores (plain and through a workspace), top-K ids, then gated
    attention over them. Every output of every entry point must match eager."""
    H = 12
    n_cells = pos0 + T
    dev = "cuda"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    L = synth.make_layer(7, 0, T, H, n_cells)
    q, kq, vq, ks, vs = (up(x) for x in (L.q, L.kq, L.vq, L.ksc, L.vsc))
    xk = up(synth.cache_rows(T, seed=23, kind="normal", which=0))
    xv = up(synth.cache_rows(T, seed=23, kind="normal", which=1))
    sc = synth.score_case(T=T, pos0=pos0, Hs=Hs, seed=9)
    sq, sk = up(sc.q), up(sc.k)
    gate = up(synth.gates(T, H, seed=9))
    scale = float(synth.SCALE_1_SQRT_128)
    row_stride = pos0 + T + 3
    scores = torch.empty(T, row_stride, dtype=torch.float32, device=dev)
    scores_ws = torch.empty_like(scores)
    workspace = torch.empty(qsa.qsa_score_ws_bytes(T), dtype=torch.uint8, device=dev)
    stride = 64 * ((min(K, n_cells) + 63) // 64)
    ids = torch.empty(T, stride, dtype=torch.int32, device=dev)
    out = torch.empty(T, H, 128, dtype=torch.float16, device=dev)
    sums = torch.empty(T, H, 8, dtype=torch.float32, device=dev)
    C = stride // 64
    part = qsa.alloc_part(T, H, 128, C)
    outputs = (kq, vq, ks, vs, scores, scores_ws, ids, out, sums)

    def step():
        qsa.qsa_quant_append(xk, xv, kq, vq, ks, vs, pos0)
        qsa.qsa_score(sq, sk, pos0, 1.0, float("-inf"), scores)
        qsa.qsa_score_ws(sq, sk, pos0, 1.0, float("-inf"), scores_ws, workspace)
        qsa.qsa_select(scores, pos0, K, ids)
        if attn == "fused":
            qsa.qsa_attn_merge_gated(q, kq, vq, ks, vs, ids, pos0, scale, gate, out, sums)
        else:
            qsa.qsa_attn(q, kq, vq, ks, vs, ids, pos0, scale, part)
            qsa.qsa_merge_gated(part, C, gate, out, sums)

    def reset():
        # the scores' last columns (past n_cells) are never written: the same
        # fill before the eager step and before every replay
        for o in (scores, scores_ws, out, sums):
            o.fill_(float("nan"))
        ids.fill_(-7)
        workspace.fill_(0xA5)

    print("graph step T=%d pos0=%d Hs=%d K=%d %s" % (T, pos0, Hs, K, attn), flush=True)
    reset()
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    assert torch.equal(_bits(scores), _bits(scores_ws))

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
        reset()
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the first pass of the workspace score runs only where q's head rows
        # reach 4 MB; the walk reads what it wrote in this same replay
        assert bool((workspace != 0xA5).any()) == (T * Hs * 128 * 4 >= 4 << 20), r
        for name, o, w in zip(("kq", "vq", "ksc", "vsc", "scores", "scores_ws", "ids", "out", "sums16"),
                              outputs, want):
            assert torch.equal(_bits(o), _bits(w)), (name, r)
