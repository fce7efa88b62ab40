"""The whole layer (reblock, select, sparse attention) captured in a HIP graph through torch's
graph capture: the library enqueues only kernels on the caller's stream (no allocation, no
memset, no host synchronisation), so every replay must reproduce the eager results bit for bit,
also with new inputs copied into the captured input buffers and with eager work between the
replays."""
import numpy as np
import pytest
import torch

from block_sparse_video_reblock_amd import _lib as ops
from block_sparse_video_reblock_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(seed):
    wl = synth.WORKLOADS["mid_bf16"]
    q, k, v = synth.make_qkv(wl, heads=[seed, seed + 1])
    return wl, [torch.from_numpy(x).to(DEV).to(torch.bfloat16) for x in (q, k, v)]


def test_layer_replays_in_a_graph():
    wl, (q, k, v) = _inputs(0)
    H, N, D = q.shape
    nb = N // 64
    topk = ops.topk_count(nb, wl.topk_ratio)
    d = ops.desc_for(q)
    ws = ops.workspace(d, q.device)
    pq = torch.empty(H, N, dtype=torch.int32, device=DEV)
    pk = torch.empty_like(pq)
    lists = torch.empty(H, nb, topk, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    L, P, st = ops.lib(), ops._dev_ptr, ops._stream

    def layer():
        ops.check(L.bsa_reblock(d, P(q), P(k), P(pq), P(pk), None, P(ws), ws.numel(), st()))
        ops.check(L.bsa_select(d, P(q), P(k), P(pq), P(pk), 0.0, topk, P(lists), None, P(ws),
                               ws.numel(), st()))
        ops.check(L.bsa_sparse_attn(d, P(q), P(k), P(v), P(pq), P(pk), P(lists), topk, 0, 0.0,
                                    P(out), None, P(ws), ws.numel(), st()))

    def eager(qx, kx, vx):
        q.copy_(qx), k.copy_(kx), v.copy_(vx)
        layer()
        torch.cuda.synchronize()
        return pq.clone(), pk.clone(), lists.clone(), out.clone()

    ref0 = eager(q.clone(), k.clone(), v.clone())
    _, (q1, k1, v1) = _inputs(2)
    ref1 = eager(q1, k1, v1)
    assert not torch.equal(ref0[3], ref1[3])
    _, (q0, k0, v0) = _inputs(0)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()

    for rep, (inp, ref) in enumerate((((q0, k0, v0), ref0), ((q1, k1, v1), ref1),
                                      ((q0, k0, v0), ref0))):
        for dst, src in zip((q, k, v), inp):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (pq, pk, lists, out)
        for name, a, b in zip(("perm_q", "perm_k", "lists", "out"), got, ref):
            assert torch.equal(a, b), (rep, name)
        # eager work between replays, on other buffers
        scratch = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch).item()
