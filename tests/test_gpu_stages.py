"""GPU parity of the select, summaries and attention stages against the CPU oracle, each fed
the same inputs (the oracle's permutations and lists where a stage consumes them).  The bars:
bit-exact for lists and permutations, max-abs 1e-4 for fp32 outputs, rel-L2 1e-2 and max-abs
3e-2 for bf16 outputs."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_video_reblock_amd import _lib as ops
from block_sparse_video_reblock_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.fixture(scope="module")
def mid():
    """Two heads of the 16,384-token bf16 workload with the oracle's layouts and lists."""
    wl = synth.WORKLOADS["mid_bf16"]
    q, k, v = synth.make_qkv(wl, heads=[0, 1])
    H = q.shape[0]
    perms = [O.reblock_head(q[h].astype(np.float64), k[h].astype(np.float64))[:2]
             for h in range(H)]
    pq = np.stack([p[0] for p in perms]).astype(np.int32)
    pk = np.stack([p[1] for p in perms]).astype(np.int32)
    K = O.topk_count(wl.n_blocks, wl.topk_ratio)
    lists = np.stack([O.topk_lists(O.block_scores(q[h].astype(np.float64),
                                                  k[h].astype(np.float64), pq[h], pk[h])
                                   .astype(np.float32), K) for h in range(H)]).astype(np.int32)
    return wl, q, k, v, pq, pk, lists


@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny_f32"]
    q, k, v = synth.make_qkv(wl)
    pq, pk, _, _ = O.reblock_head(q[0].astype(np.float64), k[0].astype(np.float64))
    K = O.topk_count(wl.n_blocks, wl.topk_ratio)
    lists = O.topk_lists(O.block_scores(q[0].astype(np.float64), k[0].astype(np.float64),
                                        pq, pk).astype(np.float32), K)
    return wl, q, k, v, pq[None].astype(np.int32), pk[None].astype(np.int32), \
        lists[None].astype(np.int32)


# ----------------------------------------------------------------------- top-K hook

# rows of up to 2,048 blocks are selected from registers, longer ones re-read memory per pass
@pytest.mark.parametrize("rows,nb,k", [(37, 64, 16), (300, 256, 51), (50, 1134, 113),
                                       (9, 70, 70), (5, 1, 1), (64, 1620, 162), (6, 2048, 205),
                                       (7, 2049, 300), (3, 4100, 410)])
def test_topk_hook_bitexact(rows, nb, k):
    rng = np.random.default_rng(rows * 7 + nb)
    S = rng.standard_normal((rows, nb)).astype(np.float32)
    S[: rows // 2] = np.round(S[: rows // 2] * 2) / 2          # many exact ties
    S[0, : min(nb, 5)] = -0.0
    S[1, : min(nb, 5)] = 0.0
    got = ops.topk_from_scores(torch.from_numpy(S).to(DEV), k).cpu().numpy()
    assert np.array_equal(got, O.topk_lists(S, k))


# ------------------------------------------------------------------- partition hook

def test_partition_hook_bitexact_oracle_projections(tiny, mid):
    for wl, q, k in ((tiny[0], tiny[1], tiny[2]), (mid[0], mid[1], mid[2])):
        projs, perms = [], []
        for h in range(q.shape[0]):
            pq, pk, prq, prk = O.reblock_head(q[h].astype(np.float64), k[h].astype(np.float64))
            projs += [prq, prk]
            perms += [pq, pk]
        got = ops.reblock_from_projections(torch.from_numpy(np.stack(projs)).to(DEV))
        assert np.array_equal(got.cpu().numpy(), np.stack(perms))


@pytest.mark.parametrize("n_blocks", [1, 2, 3, 37, 70, 129])
def test_partition_hook_bitexact_random_ties(n_blocks):
    rng = np.random.default_rng(n_blocks)
    N = 64 * n_blocks
    L = O.tree_levels(n_blocks)
    proj = rng.integers(-3, 4, size=(3, max(L, 1), N)).astype(np.float32)[:, :L]
    proj[0] *= 0.0                                              # all ties, including -0.0
    proj[1] = rng.standard_normal((L, N)).astype(np.float32)
    got = ops.reblock_from_projections(torch.from_numpy(np.ascontiguousarray(proj)).to(DEV))
    ref = np.stack([O.partition_from_projections(proj[p], N) for p in range(3)])
    assert np.array_equal(got.cpu().numpy(), ref)


# ------------------------------------------------------------------------ summaries

@pytest.mark.parametrize("mode", ["reweight", "meanpool"])
def test_summaries_parity(mid, tiny, mode):
    flags = ops.BSA_MEANPOOL if mode == "meanpool" else 0
    for wl, q, k, v, pq, pk, lists in (mid, tiny):
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        kt, vt, b = ops.summaries(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                                  torch.from_numpy(pk).to(DEV), flags=flags)
        for h in range(q.shape[0]):
            rkt, rvt, rb = O.summaries(q[h], k[h], v[h], pk[h], mode=mode)
            assert np.max(np.abs(kt[h].cpu().numpy() - rkt)) < 2e-5 * max(1, np.abs(rkt).max())
            assert np.max(np.abs(vt[h].cpu().numpy() - rvt)) < 2e-5 * max(1, np.abs(rvt).max())
            assert np.max(np.abs(b[h].cpu().numpy() - rb)) < 2e-5


# ------------------------------------------------------------------------ attention

def _oracle_attn(q, k, v, pq, pk, lists, mode="reweight", branches=False, tail="token"):
    outs = [O.sparse_attention_head(q[h], k[h], v[h], pq[h], pk[h], lists[h], mode=mode,
                                    return_branches=branches, tail=tail)
            for h in range(q.shape[0])]
    return [np.stack([o[i] for o in outs]) for i in range(len(outs[0]))]


def test_attention_parity_f32_tiny(tiny):
    wl, q, k, v, pq, pk, lists = tiny
    dt = torch.float32
    o, lse = ops.sparse_attn(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                             torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
                             torch.from_numpy(lists).to(DEV), with_lse=True)
    ro, rl = _oracle_attn(q, k, v, pq, pk, lists)
    assert np.max(np.abs(o.cpu().numpy() - ro)) < 1e-4
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-4


@pytest.mark.parametrize("mode", ["reweight", "meanpool"])
def test_attention_parity_bf16_mid(mid, mode):
    wl, q, k, v, pq, pk, lists = mid
    flags = ops.BSA_MEANPOOL if mode == "meanpool" else 0
    dt = torch.bfloat16
    o, lse = ops.sparse_attn(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                             torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
                             torch.from_numpy(lists).to(DEV), flags=flags, with_lse=True)
    ro, rl = _oracle_attn(q, k, v, pq, pk, lists, mode=mode)
    got = o.float().cpu().numpy()
    assert rel_l2(got, ro) < 1e-2
    assert np.max(np.abs(got - ro)) < 3e-2
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 3e-2


def test_attention_branches_bf16(mid):
    wl, q, k, v, pq, pk, lists = mid
    dt = torch.bfloat16
    args = (to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), torch.from_numpy(pq).to(DEV),
            torch.from_numpy(pk).to(DEV), torch.from_numpy(lists).to(DEV))
    oe, le = ops.sparse_attn(*args, flags=ops.BSA_EXACT_ONLY, with_lse=True)
    oc, lc = ops.sparse_attn(*args, flags=ops.BSA_COMPRESSED_ONLY, with_lse=True)
    _, _, ro_e, rl_e, ro_c, rl_c = _oracle_attn(q, k, v, pq, pk, lists, branches=True)
    for got, ref in ((oe, ro_e), (oc, ro_c)):
        g = got.float().cpu().numpy()
        assert rel_l2(g, ref) < 1e-2 and np.max(np.abs(g - ref)) < 3e-2
    assert np.max(np.abs(le.cpu().numpy() - rl_e)) < 3e-2
    assert np.max(np.abs(lc.cpu().numpy() - rl_c)) < 3e-2


def test_density_one_is_dense_bf16(mid):
    wl, q, k, v, pq, pk, lists = mid
    H, N, D = q.shape
    nb = N // 64
    allb = np.tile(np.arange(nb, dtype=np.int32), (H, nb, 1))
    ident = synth.identity_perm(H, N)
    dt = torch.bfloat16
    o = ops.sparse_attn(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                        torch.from_numpy(ident).to(DEV), torch.from_numpy(ident).to(DEV),
                        torch.from_numpy(allb).to(DEV))
    rows = np.arange(0, N, 37)
    ref = np.stack([O.dense_attention_head(q[h], k[h], v[h], rows=rows)[0] for h in range(H)])
    got = o.float().cpu().numpy()[:, rows]
    assert rel_l2(got, ref) < 1e-2 and np.max(np.abs(got - ref)) < 3e-2


@pytest.mark.parametrize("n_blocks,topk,H", [(70, 9, 2), (1, 1, 2), (2, 1, 2), (65, 65, 2),
                                             (37, 5, 4), (1, 1, 4), (70, 9, 8), (2, 1, 12)])
def test_attention_ragged_shapes_bf16(n_blocks, topk, H):
    """Summary tiles with a ragged tail, a single block, density 1 with a partial tile.  With H
    a multiple of 4 the launch deals each head's query blocks to a pair of XCDs in two halves
    (an odd block count leaves the second half one block short): every row is still written
    once."""
    rng = np.random.default_rng(n_blocks + 1000 * H)
    N, D = 64 * n_blocks, 128
    q, k, v = (synth.bf16_round(rng.standard_normal((H, N, D)).astype(np.float32) * s)
               for s in (0.3, 1.0, 1.0))
    pq = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    pk = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    lists = np.sort(np.stack([[rng.choice(n_blocks, topk, replace=False) for _ in range(n_blocks)]
                              for _ in range(H)]), axis=-1).astype(np.int32)
    dt = torch.bfloat16
    o, lse = ops.sparse_attn(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                             torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
                             torch.from_numpy(lists).to(DEV), with_lse=True)
    ro, rl = _oracle_attn(q, k, v, pq, pk, lists)
    g = o.float().cpu().numpy()
    assert rel_l2(g, ro) < 1e-2 and np.max(np.abs(g - ro)) < 3e-2
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 3e-2


# ------------------------------------------- block-level compressed branch (tail granularity)

@pytest.mark.parametrize("mode", ["reweight", "meanpool"])
def test_attention_tail_block_bf16_mid(mid, mode):
    """BSA_TAIL_BLOCK: the compressed branch of every query of a block uses the block's mean
    query; the merged output, and the compressed branch alone, against the oracle's
    tail="block"."""
    wl, q, k, v, pq, pk, lists = mid
    base = ops.BSA_TAIL_BLOCK | (ops.BSA_MEANPOOL if mode == "meanpool" else 0)
    dt = torch.bfloat16
    args = (to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), torch.from_numpy(pq).to(DEV),
            torch.from_numpy(pk).to(DEV), torch.from_numpy(lists).to(DEV))
    o, lse = ops.sparse_attn(*args, flags=base, with_lse=True)
    oc, lc = ops.sparse_attn(*args, flags=base | ops.BSA_COMPRESSED_ONLY, with_lse=True)
    ro, rl, _, _, ro_c, rl_c = _oracle_attn(q, k, v, pq, pk, lists, mode=mode, branches=True,
                                            tail="block")
    for got, ref in ((o, ro), (oc, ro_c)):
        g = got.float().cpu().numpy()
        assert rel_l2(g, ref) < 1e-2 and np.max(np.abs(g - ref)) < 3e-2
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 3e-2
    assert np.max(np.abs(lc.cpu().numpy() - rl_c)) < 3e-2
    # one state per block: every row of a block holds the same compressed branch
    H, N, D = q.shape
    rows = torch.from_numpy(pq.astype(np.int64)).to(DEV)
    blk = oc.float().gather(1, rows[..., None].expand(H, N, D)).view(H, N // 64, 64, D)
    assert torch.equal(blk, blk[:, :, :1].expand_as(blk))
    # differs from the per-query branch
    o_tok = ops.sparse_attn(*args, flags=base & ~ops.BSA_TAIL_BLOCK)
    assert (o.float() - o_tok.float()).abs().max().item() > 1e-2


def test_attention_tail_block_f32_tiny(tiny):
    wl, q, k, v, pq, pk, lists = tiny
    dt = torch.float32
    o, lse = ops.sparse_attn(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                             torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
                             torch.from_numpy(lists).to(DEV), flags=ops.BSA_TAIL_BLOCK,
                             with_lse=True)
    ro, rl = _oracle_attn(q, k, v, pq, pk, lists, tail="block")
    assert np.max(np.abs(o.cpu().numpy() - ro)) < 1e-4
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-4


@pytest.mark.parametrize("n_blocks,topk", [(70, 9), (1, 1), (2, 1), (65, 65), (130, 3)])
def test_attention_tail_block_ragged_bf16(n_blocks, topk):
    """Block groups with a ragged last group of pooled queries, a single block, every block
    selected (an empty compressed branch), three groups."""
    rng = np.random.default_rng(100 + n_blocks)
    H, N, D = 2, 64 * n_blocks, 128
    q, k, v = (synth.bf16_round(rng.standard_normal((H, N, D)).astype(np.float32) * s)
               for s in (0.3, 1.0, 1.0))
    pq = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    pk = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    lists = np.sort(np.stack([[rng.choice(n_blocks, topk, replace=False) for _ in range(n_blocks)]
                              for _ in range(H)]), axis=-1).astype(np.int32)
    dt = torch.bfloat16
    o, lse = ops.sparse_attn(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt),
                             torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
                             torch.from_numpy(lists).to(DEV), flags=ops.BSA_TAIL_BLOCK,
                             with_lse=True)
    ro, rl = _oracle_attn(q, k, v, pq, pk, lists, tail="block")
    g = o.float().cpu().numpy()
    assert rel_l2(g, ro) < 1e-2 and np.max(np.abs(g - ro)) < 3e-2
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 3e-2


# ------------------------------------------------- mixed sequences (exact context tokens)

def _oracle_mixed(q, k, v, qc, kc, vc, pq, pk, lists, **kw):
    outs = [O.mixed_attention_head(q[h], k[h], v[h], qc[h], kc[h], vc[h], pq[h], pk[h],
                                   lists[h], **kw) for h in range(q.shape[0])]
    return [np.stack([o[i] for o in outs]) for i in range(4)]


def _check_bf16(got, ref):
    g = got.float().cpu().numpy()
    assert rel_l2(g, ref) < 1e-2 and np.max(np.abs(g - ref)) < 3e-2


@pytest.mark.parametrize("tail", ["token", "block"])
def test_mixed_sequence_bf16_mid(mid, tail):
    """1,000 context tokens beside the 16,384-token grid: video queries add every context key
    to their exact branch, context queries attend densely to all keys."""
    wl, q, k, v, pq, pk, lists = mid
    qc, kc, vc = synth.make_ctx(wl, synth.CTX_TOKENS, (q, k, v), heads=[0, 1])
    dt = torch.bfloat16
    flags = ops.BSA_TAIL_BLOCK if tail == "block" else 0
    o, oc, lse, lc = ops.sparse_attn_ctx(
        *(to_dev(x, dt) for x in (q, k, v, qc, kc, vc)), torch.from_numpy(pq).to(DEV),
        torch.from_numpy(pk).to(DEV), torch.from_numpy(lists).to(DEV), flags=flags,
        with_lse=True)
    ro, rl, roc, rlc = _oracle_mixed(q, k, v, qc, kc, vc, pq, pk, lists, tail=tail)
    _check_bf16(o, ro)
    _check_bf16(oc, roc)
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 3e-2
    assert np.max(np.abs(lc.cpu().numpy() - rlc)) < 3e-2


@pytest.mark.parametrize("n_ctx", [1, 63, 64, 65, 200])
def test_mixed_sequence_ragged_bf16(n_ctx):
    """Context lengths around the 64-row tile, on a 70-block grid (ragged summary tiles), with
    the branch flags: context keys belong to the exact branch."""
    rng = np.random.default_rng(500 + n_ctx)
    H, nbk, topk, D = 2, 70, 9, 128
    N = 64 * nbk
    q, k, v, qc, kc, vc = (synth.bf16_round(rng.standard_normal((H, n, D)).astype(np.float32) * s)
                           for n, s in ((N, 0.3), (N, 1.0), (N, 1.0), (n_ctx, 0.3),
                                        (n_ctx, 1.0), (n_ctx, 1.0)))
    pq = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    pk = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    lists = np.sort(np.stack([[rng.choice(nbk, topk, replace=False) for _ in range(nbk)]
                              for _ in range(H)]), axis=-1).astype(np.int32)
    dt = torch.bfloat16
    args = (*(to_dev(x, dt) for x in (q, k, v, qc, kc, vc)), torch.from_numpy(pq).to(DEV),
            torch.from_numpy(pk).to(DEV), torch.from_numpy(lists).to(DEV))
    o, oc, lse, lc = ops.sparse_attn_ctx(*args, with_lse=True)
    ro, rl, roc, rlc = _oracle_mixed(q, k, v, qc, kc, vc, pq, pk, lists)
    _check_bf16(o, ro)
    _check_bf16(oc, roc)
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 3e-2
    assert np.max(np.abs(lc.cpu().numpy() - rlc)) < 3e-2
    # branches: the exact branch holds the context keys; context queries have no compressed
    # branch
    ctx = [(kc[h], vc[h]) for h in range(H)]
    br = [O.sparse_attention_head(q[h], k[h], v[h], pq[h], pk[h], lists[h], ctx=ctx[h],
                                  return_branches=True) for h in range(H)]
    oe, _, le, _ = ops.sparse_attn_ctx(*args, flags=ops.BSA_EXACT_ONLY, with_lse=True)
    _check_bf16(oe, np.stack([b[2] for b in br]))
    assert np.max(np.abs(le.cpu().numpy() - np.stack([b[3] for b in br]))) < 3e-2
    ocmp, occ, lcmp, lcc = ops.sparse_attn_ctx(*args, flags=ops.BSA_COMPRESSED_ONLY,
                                               with_lse=True)
    _check_bf16(ocmp, np.stack([b[4] for b in br]))
    assert torch.all(occ.float() == 0).item() and torch.all(torch.isinf(lcc)).item()


def test_mixed_sequence_f32_tiny(tiny):
    wl, q, k, v, pq, pk, lists = tiny
    qc, kc, vc = synth.make_ctx(wl, 77, (q, k, v))
    dt = torch.float32
    for flags, tail in ((0, "token"), (ops.BSA_TAIL_BLOCK, "block")):
        o, oc, lse, lc = ops.sparse_attn_ctx(
            *(to_dev(x, dt) for x in (q, k, v, qc, kc, vc)), torch.from_numpy(pq).to(DEV),
            torch.from_numpy(pk).to(DEV), torch.from_numpy(lists).to(DEV), flags=flags,
            with_lse=True)
        ro, rl, roc, rlc = _oracle_mixed(q, k, v, qc, kc, vc, pq, pk, lists, tail=tail)
        for got, ref in ((o, ro), (oc, roc), (lse, rl), (lc, rlc)):
            assert np.max(np.abs(got.cpu().numpy() - ref)) < 1e-4


def test_mixed_sequence_two_phase_equals_one_call(mid):
    wl, q, k, v, pq, pk, lists = mid
    qc, kc, vc = synth.make_ctx(wl, 300, (q, k, v), heads=[0, 1])
    dt = torch.bfloat16
    t = [to_dev(x, dt) for x in (q, k, v, qc, kc, vc)]
    perms = [torch.from_numpy(x).to(DEV) for x in (pq, pk, lists)]
    o1, oc1 = ops.sparse_attn_ctx(*t, *perms)
    d = ops.desc_for(t[0])
    ws = ops.workspace_ctx(d, 300, DEV)
    o2, oc2 = torch.empty_like(t[0]), torch.empty_like(t[3])
    L, P = ops.lib(), ops._dev_ptr
    ops.check(L.bsa_prepare_kv_ctx(d, 300, P(t[0]), P(t[1]), P(t[2]), P(t[4]), P(t[5]),
                                   P(perms[1]), 0, 0.0, P(ws), ws.numel(), ops._stream()))
    ops.check(L.bsa_attend_ctx(d, 300, *(P(x) for x in t), *(P(x) for x in perms),
                               int(lists.shape[-1]), 0, 0.0, P(o2), P(oc2), None, None, P(ws),
                               ws.numel(), ops._stream()))
    assert torch.equal(o1, o2) and torch.equal(oc1, oc2)


def test_mixed_sequence_without_context_is_the_plain_layer(mid):
    wl, q, k, v, pq, pk, lists = mid
    dt = torch.bfloat16
    args = (to_dev(q, dt), to_dev(k, dt), to_dev(v, dt))
    empty = torch.empty(q.shape[0], 0, q.shape[2], dtype=dt, device=DEV)
    perms = (torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
             torch.from_numpy(lists).to(DEV))
    o, oc = ops.sparse_attn_ctx(*args, empty, empty, empty, *perms)
    assert oc.numel() == 0
    assert torch.equal(o, ops.sparse_attn(*args, *perms))


def test_option_paths_are_deterministic(mid):
    """Two runs of each option path give bitwise-identical results: the Lite tree, the
    block-level tail, and a mixed sequence (both outputs)."""
    wl, q, k, v, pq, pk, lists = mid
    dt = torch.bfloat16
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    perms = (torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
             torch.from_numpy(lists).to(DEV))
    for run in (lambda: ops.reblock(qd, kd, power_iters=ops.BSA_POWER_ITERS_LITE,
                                    shared_deep=True, subtree_blocks=ops.BSA_LITE_SUBTREE_BLOCKS),
                lambda: (ops.sparse_attn(qd, kd, vd, *perms, flags=ops.BSA_TAIL_BLOCK),)):
        a, b = run(), run()
        assert all(torch.equal(x, y) for x, y in zip(a, b))
    qc, kc, vc = (to_dev(x, dt) for x in synth.make_ctx(wl, 300, (q, k, v), heads=[0, 1]))
    a = ops.sparse_attn_ctx(qd, kd, vd, qc, kc, vc, *perms)
    b = ops.sparse_attn_ctx(qd, kd, vd, qc, kc, vc, *perms)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_attention_is_deterministic(mid):
    wl, q, k, v, pq, pk, lists = mid
    dt = torch.bfloat16
    args = (to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), torch.from_numpy(pq).to(DEV),
            torch.from_numpy(pk).to(DEV), torch.from_numpy(lists).to(DEV))
    a = ops.sparse_attn(*args)
    b = ops.sparse_attn(*args)
    assert torch.equal(a, b)


# --------------------------------------------------------------------------- select

def test_select_parity(mid, tiny):
    for wl, q, k, v, pq, pk, lists in (mid, tiny):
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        got_l, got_s = ops.select(to_dev(q, dt), to_dev(k, dt), torch.from_numpy(pq).to(DEV),
                                  torch.from_numpy(pk).to(DEV), topk_ratio=wl.topk_ratio,
                                  with_scores=True)
        got_l, got_s = got_l.cpu().numpy(), got_s.cpu().numpy()
        K = O.topk_count(wl.n_blocks, wl.topk_ratio)
        for h in range(q.shape[0]):
            S = O.block_scores(q[h], k[h], pq[h], pk[h])
            assert np.max(np.abs(got_s[h] - S)) < 1e-5 * max(1.0, np.abs(S).max())
            # selection is exact on the GPU's own fp32 scores
            assert np.array_equal(got_l[h], O.topk_lists(got_s[h], K))
            # and agrees with the oracle's lists except where scores tie within 1e-5
            for i in range(S.shape[0]):
                a, b = set(got_l[h, i]), set(lists[h, i])
                if a != b:
                    kth = np.sort(S[i])[::-1][K - 1]
                    for j in a ^ b:
                        assert abs(S[i, j] - kth) <= 1e-5


# ------------------------------------------------------------------- strict list checks

def test_check_lists_finds_malformed_rows(mid):
    """bsa_check_lists on valid lists reports none; planted defects (an entry equal to nb, a
    negative entry, a repeated entry, two entries out of order) are each counted once, and
    the smallest defective row is reported.  Malformed lists go to the checker only."""
    wl, q, k, v, pq, pk, lists = mid
    nb = wl.n_blocks
    good = torch.from_numpy(lists).to(DEV)
    assert ops.check_lists(good, nb) == (0, -1)
    H, R, K = lists.shape
    for row, fix in ((5, lambda r: r.__setitem__(-1, nb)),
                     (R + 17, lambda r: r.__setitem__(0, -1)),
                     (3, lambda r: r.__setitem__(2, r[1])),
                     (R - 1, lambda r: r.__setitem__(slice(0, 2), r[1::-1].copy()))):
        bad = lists.copy().reshape(H * R, K)
        fix(bad[row])
        assert ops.check_lists(torch.from_numpy(bad).to(DEV), nb) == (1, row)
    bad = lists.copy().reshape(H * R, K)
    for row in (40, 7, R + 3):
        bad[row, -1] = nb + row
    assert ops.check_lists(torch.from_numpy(bad).to(DEV), nb) == (3, 7)


def test_attention_with_list_check_on_valid_lists(mid):
    """With BSA_CHECK_LISTS and valid lists the output is bit-identical to the unchecked call
    and the workspace's list status reports no malformed row (bf16 and the block-level tail)."""
    wl, q, k, v, pq, pk, lists = mid
    dt = torch.bfloat16
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    perms = (torch.from_numpy(pq).to(DEV), torch.from_numpy(pk).to(DEV),
             torch.from_numpy(lists).to(DEV))
    ws = ops.workspace(ops.desc_for(qd), qd.device)
    for flags in (0, ops.BSA_TAIL_BLOCK):
        ref = ops.sparse_attn(qd, kd, vd, *perms, flags=flags, ws=ws)
        got = ops.sparse_attn(qd, kd, vd, *perms, flags=flags | ops.BSA_CHECK_LISTS, ws=ws)
        assert ops.list_status(ws) == (0, -1)
        assert torch.equal(ref, got)
