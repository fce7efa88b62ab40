"""GPU checks of the workload variants and of the full-size configurations.

* Fixed-tile baseline (positional 4x4x4 cubes, mean-pooled summaries): layout bit-exact with the
  oracle's, lists equal to the oracle's top-K except for ties within 1e-5, outputs against the
  oracle run on the GPU's lists (bf16: rel-L2 1e-2, max-abs 3e-2).
* Recall measured the way the benchmark measures it -- exp(lse over the selected blocks - dense
  lse), both from the attention kernel -- against the oracle's fp64 dense-softmax recall.
* Full-size layers (72,576 tokens, and all four 103,680-token layers, 24 heads), run as the
  benchmark runs them: structural checks on every head; on the first and last head the block
  scores and lists against the oracle; whole heads' outputs (every query block) against the
  oracle run on the GPU's layouts and lists, for both compressed-branch granularities; every
  split of both trees of head 0 at 72,576 tokens replayed on the oracle.
* The largest accepted sequence (524,288 tokens): sampled blocks, the first levels replayed."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_video_reblock_amd import _lib as ops
from block_sparse_video_reblock_amd import synth
from replay import replay_partition

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def lists_agree(got, S, K, tol=1e-5):
    """got: int [nb][K] lists; S: oracle scores [nb][nb].  Equal to the oracle's top-K except
    for blocks whose scores tie with the K-th within tol."""
    ref = O.topk_lists(S.astype(np.float32), K)
    for i in range(S.shape[0]):
        a, b = set(got[i].tolist()), set(ref[i].tolist())
        if a != b:
            kth = np.sort(S[i])[::-1][K - 1]
            for j in a ^ b:
                assert abs(S[i, j] - kth) <= tol, (i, j, S[i, j], kth)


@pytest.mark.parametrize("grid,tile", [((16, 32, 32), (4, 4, 4)), ((21, 48, 72), (1, 8, 8)),
                                       ((30, 48, 72), (1, 8, 8)), ((4, 32, 32), (4, 4, 4))])
def test_tile_layout_bitexact(grid, tile):
    got = ops.tile_layout(3, grid, tile, device=DEV).cpu().numpy()
    ref = O.fixed_tile_perm(grid, tile)
    for h in range(3):
        assert np.array_equal(got[h], ref)


@pytest.fixture(scope="module")
def mid2():
    wl = synth.WORKLOADS["mid_bf16"]
    q, k, v = synth.make_qkv(wl, heads=[0, 1])
    return wl, q, k, v


def test_fixed_tile_layer_meanpool(mid2):
    wl, q, k, v = mid2
    H = q.shape[0]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    perm = ops.tile_layout(H, wl.grid, device=DEV)
    lists = ops.select(qd, kd, perm, perm, topk_ratio=wl.topk_ratio)
    o = ops.sparse_attn(qd, kd, vd, perm, perm, lists, flags=ops.BSA_MEANPOOL)
    perm, lists, o = perm.cpu().numpy(), lists.cpu().numpy(), o.float().cpu().numpy()
    K = O.topk_count(wl.n_blocks, wl.topk_ratio)
    for h in range(H):
        lists_agree(lists[h], O.block_scores(q[h], k[h], perm[h], perm[h]), K)
        ro, _ = O.sparse_attention_head(q[h], k[h], v[h], perm[h], perm[h], lists[h],
                                        mode="meanpool")
        assert rel_l2(o[h], ro) < 1e-2
        assert np.max(np.abs(o[h] - ro)) < 3e-2


def gpu_recall(qd, kd, vd, pq, pk, lists):
    """Recall as the benchmark measures it: mean over queries of exp(lse_sel - lse_dense)."""
    H, N = qd.shape[0], qd.shape[1]
    nb = N // 64
    _, lse_sel = ops.sparse_attn(qd, kd, vd, pq, pk, lists, flags=ops.BSA_EXACT_ONLY,
                                 with_lse=True)
    ident = torch.arange(N, dtype=torch.int32, device=qd.device).repeat(H, 1).contiguous()
    every = torch.arange(nb, dtype=torch.int32, device=qd.device).repeat(H, nb, 1).contiguous()
    _, lse_all = ops.sparse_attn(qd, kd, vd, ident, ident, every, flags=ops.BSA_EXACT_ONLY,
                                 with_lse=True)
    return torch.exp(lse_sel - lse_all).mean(dim=1).cpu().numpy()


@pytest.mark.parametrize("ratio", [0.1, 1.0])
def test_recall_from_lse_matches_oracle(mid2, ratio):
    wl, q, k, v = mid2
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pq, pk = ops.reblock(qd, kd)
    lists = ops.select(qd, kd, pq, pk, topk_ratio=ratio)
    rec = gpu_recall(qd, kd, vd, pq, pk, lists)
    pq, pk, ln = pq.cpu().numpy(), pk.cpu().numpy(), lists.cpu().numpy()
    for h in range(q.shape[0]):
        ref = O.recall_head(q[h], k[h], pq[h], pk[h], ln[h])
        assert abs(rec[h] - ref) < 2e-3, (h, rec[h], ref)
    if ratio == 1.0:
        assert np.all(np.abs(rec - 1.0) < 1e-3)


def test_log_mass_error_measurement_matches_oracle(mid2):
    """The benchmark's log-mass error (torch on the device, from the library's summaries)
    against the oracle's fp64 log_mass_error_head, for Reweight and mean pooling on the GPU's
    layouts and lists."""
    import bench
    wl, q, k, v = mid2
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pq, pk = ops.reblock(qd, kd)
    lists = ops.select(qd, kd, pq, pk, topk_ratio=wl.topk_ratio)
    got = {m: bench.log_mass_error(torch, ops, qd, kd, vd, pq, pk, lists,
                                   meanpool=(m == "meanpool")) for m in ("reweight", "meanpool")}
    pq, pk, ln = pq.cpu().numpy(), pk.cpu().numpy(), lists.cpu().numpy()
    for m in ("reweight", "meanpool"):
        ref = np.mean([O.log_mass_error_head(q[h], k[h], v[h], pq[h], pk[h], ln[h], mode=m)
                       for h in range(q.shape[0])])
        print(m, got[m], ref, flush=True)
        assert abs(got[m] - ref) < 1e-4 * max(1.0, ref), (m, got[m], ref)
    assert got["reweight"] < got["meanpool"]


# ----------------------------------------------------------------- full-size layers

_LAYERS = {}


def _full_layer(wl, layer, with_proj=False):
    """One layer of a workload run as the benchmark runs it (one workspace; reblock, select,
    prepare, attend), with the block-level tail as a second attend; cached per (workload,
    layer) so the tests of one layer share a single GPU run."""
    key = (wl.name, layer)
    if key in _LAYERS:
        return _LAYERS[key]
    _LAYERS.clear()                     # keep one full-size layer resident at a time
    q, k, v = synth.make_qkv(wl, layer=layer)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    d = ops.desc_for(qd)
    ws = ops.workspace(d, qd.device)
    if with_proj:
        pq, pk, proj = ops.reblock(qd, kd, ws=ws, with_proj=True)
        proj = proj.cpu().numpy()
    else:
        pq, pk = ops.reblock(qd, kd, ws=ws)
        proj = None
    lists, scores = ops.select(qd, kd, pq, pk, topk_ratio=wl.topk_ratio, ws=ws, with_scores=True)
    out = torch.empty_like(qd)
    out_tb = torch.empty_like(qd)
    ops.prepare_kv(qd, kd, vd, pk, ws=ws)
    ops.attend(qd, kd, vd, pq, pk, lists, ws=ws, out=out)
    ops.attend(qd, kd, vd, pq, pk, lists, ws=ws, out=out_tb, flags=ops.BSA_TAIL_BLOCK)
    torch.cuda.synchronize()
    del ws
    res = (q, k, v, pq.cpu().numpy(), pk.cpu().numpy(), lists.cpu().numpy(), scores, out, out_tb,
           proj)
    _LAYERS[key] = res
    return res


def _structure_and_select(wl, layer):
    """Every head: layouts are bijections with ascending 64-token leaves, lists ascending and in
    range, outputs finite.  First and last head: fp32 block scores against the oracle's, lists
    bit-exact on the GPU's own scores and equal to the oracle's top-K up to 1e-5 ties."""
    H, N, nb = wl.heads, wl.tokens, wl.n_blocks
    K = O.topk_count(nb, wl.topk_ratio)
    q, k, v, pq, pk, lists, scores, out, out_tb, _ = _full_layer(wl, layer, with_proj=True)
    ident = np.arange(N)
    for h in range(H):
        for perm in (pq[h], pk[h]):
            assert np.array_equal(np.sort(perm), ident)
            assert np.all(np.diff(perm.reshape(nb, 64), axis=1) > 0)
    assert lists.shape == (H, nb, K)
    assert np.all(np.diff(lists, axis=2) > 0) and lists.min() >= 0 and lists.max() < nb
    assert torch.isfinite(out.float()).all().item()
    assert torch.isfinite(out_tb.float()).all().item()
    for h in (0, H - 1):
        Qh, Kh = q[h].astype(np.float64), k[h].astype(np.float64)
        S = O.block_scores(Qh, Kh, pq[h], pk[h])
        got_s = scores[h].cpu().numpy()
        assert np.max(np.abs(got_s - S)) < 1e-5 * max(1.0, np.abs(S).max())
        assert np.array_equal(lists[h], O.topk_lists(got_s, K))
        lists_agree(lists[h], S, K)


def _head_output(wl, layer, h, tail):
    """Every query block of one head (the benchmark's launch, all heads in one call) against
    the oracle run on the GPU's layouts and lists: rel-L2 <= 1e-2, max-abs <= 3e-2."""
    q, k, v, pq, pk, lists, scores, out, out_tb, _ = _full_layer(wl, layer, with_proj=True)
    Qh, Kh, Vh = (x[h].astype(np.float64) for x in (q, k, v))
    ro, _ = O.sparse_attention_head(Qh, Kh, Vh, pq[h], pk[h], lists[h], tail=tail)
    got = (out if tail == "token" else out_tb)[h].float().cpu().numpy()
    rel, err = rel_l2(got, ro), float(np.max(np.abs(got - ro)))
    print(f"  rel-L2 {rel:.2e} max-abs {err:.2e}", flush=True)
    assert rel < 1e-2 and err < 3e-2, (rel, err)


def _tree_replay(wl, layer, side):
    """Every split of every level of head 0's query (side 0) or key (side 1) tree in the
    benchmark's 24-head launch, replayed on the oracle with the 1e-5 tie rule; the GPU's own
    fp32 projections against the oracle's."""
    q, k, v, pq, pk, lists, scores, out, out_tb, proj = _full_layer(wl, layer, with_proj=True)
    X, Y = (q[0], k[0]) if side == 0 else (k[0], q[0])
    U = O.metric_embed(X.astype(np.float64), O.second_moment(Y.astype(np.float64)))
    st = replay_partition(U, (pq if side == 0 else pk)[0], proj[0, side])
    print("  replay", st, flush=True)
    assert st["splits"] == wl.n_blocks - 1
    assert st["mismatched_splits"] <= 0.02 * st["splits"], st
    assert st["max_proj_err"] < 3e-5, st


# Cases grouped by layer, so that each full-size layer runs once on the GPU: the 72,576-token
# layer (structure, first and last head with both compressed-branch granularities, both trees
# of head 0 replayed) and every 103,680-token layer (structure and one whole head each).
FULL_CASES = [
    ("clip10s_bf16", 0, "structure", None, None),
    ("clip10s_bf16", 0, "head", 0, "token"), ("clip10s_bf16", 0, "head", 23, "token"),
    ("clip10s_bf16", 0, "head", 0, "block"), ("clip10s_bf16", 0, "head", 23, "block"),
    ("clip10s_bf16", 0, "replay", 0, None), ("clip10s_bf16", 0, "replay", 1, None),
    ("clip14s_bf16", 0, "structure", None, None), ("clip14s_bf16", 0, "head", 0, "token"),
    ("clip14s_bf16", 1, "structure", None, None), ("clip14s_bf16", 1, "head", 23, "token"),
    ("clip14s_bf16", 2, "structure", None, None), ("clip14s_bf16", 2, "head", 0, "token"),
    ("clip14s_bf16", 3, "structure", None, None), ("clip14s_bf16", 3, "head", 23, "token"),
    ("clip14s_bf16", 3, "head", 0, "block"),
]


@pytest.mark.parametrize("name,layer,kind,arg,tail", FULL_CASES)
def test_full_size_layer(name, layer, kind, arg, tail):
    wl = synth.WORKLOADS[name]
    print(f"{name} layer {layer}: {kind} {arg} {tail}", flush=True)
    if kind == "structure":
        _structure_and_select(wl, layer)
    elif kind == "head":
        _head_output(wl, layer, arg, tail)
    else:
        _tree_replay(wl, layer, arg)


def test_full_size_mixed_sequence_sampled():
    """The 72,576-token grid with 1,000 exact context tokens, in the launch configuration the
    benchmark times with --ctx: sampled video blocks and context rows against the oracle."""
    wl = synth.WORKLOADS["clip10s_bf16"]
    H, N, nb = wl.heads, wl.tokens, wl.n_blocks
    q, k, v = synth.make_qkv(wl)
    qc, kc, vc = synth.make_ctx(wl, synth.CTX_TOKENS, (q, k, v))
    print(f"mixed: H={H} N={N} n_ctx={qc.shape[1]}", flush=True)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    pq, pk = ops.reblock(qd, kd)
    lists = ops.select(qd, kd, pq, pk, topk_ratio=wl.topk_ratio)
    o, oc = ops.sparse_attn_ctx(qd, kd, vd, to_dev(qc), to_dev(kc), to_dev(vc), pq, pk, lists)
    torch.cuda.synchronize()
    pq, pk, lists = pq.cpu().numpy(), pk.cpu().numpy(), lists.cpu().numpy()
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(oc.float()).all().item()
    rng = np.random.default_rng(21)
    for h in (0, H - 1):
        Qh, Kh, Vh = (x[h].astype(np.float64) for x in (q, k, v))
        blocks = np.sort(rng.choice(nb, size=4, replace=False))
        ro, _ = O.sparse_attention_head(Qh, Kh, Vh, pq[h], pk[h], lists[h], blocks=blocks,
                                        ctx=(kc[h], vc[h]))
        rows = np.concatenate([pq[h][64 * i:64 * i + 64] for i in blocks])
        got = o[h, torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
        assert rel_l2(got, ro[rows]) < 1e-2 and np.max(np.abs(got - ro[rows])) < 3e-2
        crow = np.sort(rng.choice(qc.shape[1], size=64, replace=False))
        rc, _ = O.dense_attention_head(qc[h], np.concatenate([kc[h], Kh]),
                                       np.concatenate([vc[h], Vh]), rows=crow)
        gotc = oc[h, torch.from_numpy(crow).to(DEV)].float().cpu().numpy()
        assert rel_l2(gotc, rc) < 1e-2 and np.max(np.abs(gotc - rc)) < 3e-2


def test_max_tokens_layer_sampled():
    """The largest sequence the boundary accepts (524,288 tokens = 8,192 blocks, a 13-level
    tree, 819 selected blocks per row, 128 summary tiles), two heads: layouts, scores, lists and
    sampled outputs against the oracle."""
    wl = synth.WORKLOADS["max_bf16"]
    H, N, nb = wl.heads, wl.tokens, wl.n_blocks
    assert N == 1 << 19
    K = O.topk_count(nb, wl.topk_ratio)
    props = torch.cuda.get_device_properties(0)
    print(f"max: H={H} N={N} nb={nb} K={K}; device LDS per block "
          f"{getattr(props, 'shared_memory_per_block', '?')}", flush=True)
    q, k, v, pq, pk, lists, scores, out, out_tb, _ = _full_layer(wl, 0)
    print("max: layer done", flush=True)
    ident = np.arange(N)
    for h in range(H):
        for perm in (pq[h], pk[h]):
            assert np.array_equal(np.sort(perm), ident)
            assert np.all(np.diff(perm.reshape(nb, 64), axis=1) > 0)
    assert lists.shape == (H, nb, K)
    assert np.all(np.diff(lists, axis=2) > 0) and lists.min() >= 0 and lists.max() < nb
    assert torch.isfinite(out.float()).all().item() and torch.isfinite(out_tb.float()).all().item()
    rng = np.random.default_rng(11)
    for h in range(H):
        Qh, Kh, Vh = (x[h].astype(np.float64) for x in (q, k, v))
        rows_s = np.sort(rng.choice(nb, size=4, replace=False))
        S = O.block_means(Qh, pq[h])[rows_s] @ O.block_means(Kh, pk[h]).T / np.sqrt(Qh.shape[1])
        got_s = scores[h].cpu().numpy()[rows_s]
        assert np.max(np.abs(got_s - S)) < 1e-5 * max(1.0, np.abs(S).max())
        assert np.array_equal(lists[h][rows_s], O.topk_lists(got_s, K))
        blocks = np.sort(rng.choice(nb, size=3, replace=False))
        rows = np.concatenate([pq[h][64 * i:64 * i + 64] for i in blocks])
        summ = O.summaries(Qh, Kh, Vh, pk[h])
        for o_dev, tail in ((out, "token"), (out_tb, "block")):
            ro, _ = O.sparse_attention_head(Qh, Kh, Vh, pq[h], pk[h], lists[h], blocks=blocks,
                                            tail=tail, summ=summ)
            got = o_dev[h, torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
            assert rel_l2(got, ro[rows]) < 1e-2 and np.max(np.abs(got - ro[rows])) < 3e-2
    # the first two tree levels of head 0's key side, replayed on the oracle
    U = O.metric_embed(k[0].astype(np.float64), O.second_moment(q[0].astype(np.float64)))
    st = replay_partition(U, pk[0], None, max_level=2)
    print("replay", st, flush=True)
    assert st["splits"] == 3 and st["mismatched_splits"] == 0, st
