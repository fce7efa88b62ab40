"""GPU reblock and end-to-end layer parity against the oracle.

Permutations: every GPU split is replayed on the oracle (tests/replay.py) and must agree with
it except for tokens whose oracle projections tie within 1e-5 at the cut.  The GPU's own fp32
projections must agree with the oracle's within 3e-5: fp32 rounding of the group covariance
and metric (about 6e-8 relative) is amplified by groups whose two leading eigenvalues are close,
because 8 power steps do not separate them.  Outputs: compared with
the oracle run on the GPU's own layouts and lists (bf16: rel-L2 1e-2, max-abs 3e-2; fp32: 1e-4)."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_video_reblock_amd import _lib as ops
from block_sparse_video_reblock_amd import synth
from replay import replay_partition

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def _check_layouts(q, k, perm_q, perm_k, proj, tol_proj, iters=O.POWER_ITERS, shared=False,
                   subtree=0):
    """Replay both sides of every head; returns the summed statistics."""
    total = {"splits": 0, "mismatched_splits": 0, "max_proj_err": 0.0}
    for h in range(q.shape[0]):
        Qh, Kh = q[h].astype(np.float64), k[h].astype(np.float64)
        for side, (X, Mo, perm) in enumerate(((Qh, O.second_moment(Kh), perm_q[h]),
                                              (Kh, O.second_moment(Qh), perm_k[h]))):
            assert np.array_equal(np.sort(perm), np.arange(X.shape[0]))
            assert np.all(np.diff(perm.reshape(-1, 64), axis=1) > 0)
            st = replay_partition(O.metric_embed(X, Mo), perm,
                                  None if proj is None else proj[h, side], iters=iters,
                                  shared_deep=shared, subtree_blocks=subtree or 8)
            for key in ("splits", "mismatched_splits"):
                total[key] += st[key]
            total["max_proj_err"] = max(total["max_proj_err"], st["max_proj_err"])
    assert total["max_proj_err"] < tol_proj, total
    return total


@pytest.fixture(scope="module")
def tiny():
    wl = synth.WORKLOADS["tiny_f32"]
    return (wl,) + synth.make_qkv(wl)


@pytest.fixture(scope="module")
def mid():
    wl = synth.WORKLOADS["mid_bf16"]
    return (wl,) + synth.make_qkv(wl, heads=[0, 1])


# (power steps per split, one direction per shared subtree, subtree size in blocks; 0 = the
# default 8): the default tree, fewer power steps, shared subtrees of several sizes (deeper and
# higher than the on-chip subtree level), and the Lite preset
TREES = [(O.POWER_ITERS, False, 0), (ops.BSA_POWER_ITERS_LITE, False, 0),
         (ops.BSA_POWER_ITERS_LITE, True, 0), (O.POWER_ITERS, True, 2),
         (ops.BSA_POWER_ITERS_LITE, True, 4), (O.POWER_ITERS, True, 16),
         (ops.BSA_POWER_ITERS_LITE, True, 32),
         (ops.BSA_POWER_ITERS_LITE, True, ops.BSA_LITE_SUBTREE_BLOCKS)]


@pytest.mark.parametrize("iters,shared,subtree", TREES)
def test_reblock_f32_tiny(tiny, iters, shared, subtree):
    wl, q, k, v = tiny
    dt = torch.float32
    pq, pk, proj = ops.reblock(to_dev(q, dt), to_dev(k, dt), with_proj=True, power_iters=iters,
                               shared_deep=shared, subtree_blocks=subtree)
    pq, pk, proj = pq.cpu().numpy(), pk.cpu().numpy(), proj.cpu().numpy()
    st = _check_layouts(q, k, pq, pk, proj, tol_proj=3e-5, iters=iters, shared=shared,
                        subtree=subtree)
    print("tiny replay", iters, shared, subtree, st)
    rq, rk, _, _ = O.reblock_head(q[0].astype(np.float64), k[0].astype(np.float64), iters=iters,
                                  shared_deep=shared, subtree_blocks=subtree or 8)
    if st["mismatched_splits"] == 0:
        assert np.array_equal(pq[0], rq) and np.array_equal(pk[0], rk)


@pytest.mark.parametrize("iters,shared,subtree", TREES)
def test_reblock_bf16_mid(mid, iters, shared, subtree):
    wl, q, k, v = mid
    dt = torch.bfloat16
    pq, pk, proj = ops.reblock(to_dev(q, dt), to_dev(k, dt), with_proj=True, power_iters=iters,
                               shared_deep=shared, subtree_blocks=subtree)
    pq, pk, proj = pq.cpu().numpy(), pk.cpu().numpy(), proj.cpu().numpy()
    st = _check_layouts(q, k, pq, pk, proj, tol_proj=3e-5, iters=iters, shared=shared,
                        subtree=subtree)
    print("mid replay", iters, shared, subtree, st)
    assert st["mismatched_splits"] <= 0.02 * st["splits"]


@pytest.mark.parametrize("n_blocks,iters,shared,subtree", [
    (600, 8, False, 0), (1134, 8, False, 0), (1134, 2, True, 0),
    (1134, 2, True, 32), (1134, 2, True, ops.BSA_LITE_SUBTREE_BLOCKS), (2200, 8, False, 0)])
def test_reblock_bf16_narrow_levels(n_blocks, iters, shared, subtree):
    """Enough blocks for the one-workgroup-per-parent levels (left-only statistics, right
    child from the parent's covariance) between the wide levels and the subtree kernel: every
    split of both sides replayed on the oracle.  At 2,200 blocks the first of those levels has
    groups of more than 2,048 keys, which the kernel selects and partitions from global memory
    (smaller groups from LDS).  There (140,800 tokens) the GPU's projections sit up to 6.4e-5
    from the oracle's, measured, against under 3e-5 up to 72,576 tokens: the wide levels' groups
    are twice as large and accumulate more fp32 rounding.  The bar for that case is 1e-4, and
    every split must still agree with the oracle's as in the other cases."""
    rng = np.random.default_rng(n_blocks)
    wl = synth.WORKLOADS["clip10s_bf16" if 64 * n_blocks <= 72576 else "max_bf16"]
    q, k, _ = synth.make_qkv(wl, heads=[5 if wl.name == "clip10s_bf16" else 0])
    sel = np.sort(rng.choice(wl.tokens, size=64 * n_blocks, replace=False))
    q, k = q[:, sel], k[:, sel]
    pq, pk, proj = ops.reblock(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                               with_proj=True, power_iters=iters, shared_deep=shared,
                               subtree_blocks=subtree)
    st = _check_layouts(q, k, pq.cpu().numpy(), pk.cpu().numpy(), proj.cpu().numpy(),
                        tol_proj=3e-5 if 64 * n_blocks <= 72576 else 1e-4, iters=iters,
                        shared=shared, subtree=subtree)
    print("narrow replay", iters, shared, subtree, st)
    assert st["mismatched_splits"] <= 0.02 * st["splits"]


def test_reblock_deterministic(mid):
    wl, q, k, v = mid
    dt = torch.bfloat16
    a = ops.reblock(to_dev(q, dt), to_dev(k, dt))
    b = ops.reblock(to_dev(q, dt), to_dev(k, dt))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("n_blocks", [1, 2, 3, 5, 37])
def test_reblock_small_and_odd_shapes(n_blocks):
    rng = np.random.default_rng(100 + n_blocks)
    H, N, D = 2, 64 * n_blocks, 128
    q = synth.bf16_round(rng.standard_normal((H, N, D)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((H, N, D)).astype(np.float32))
    pq, pk = ops.reblock(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16))
    pq, pk = pq.cpu().numpy(), pk.cpu().numpy()
    if n_blocks == 1:
        assert np.array_equal(pq, synth.identity_perm(H, N))
        return
    _check_layouts(q, k, pq, pk, None, tol_proj=1.0)


def test_reblock_duplicate_tokens_split_by_id():
    """Identical tokens tie in every projection: the split falls back to token order."""
    H, N, D = 1, 64 * 4, 128
    rng = np.random.default_rng(9)
    base = synth.bf16_round(rng.standard_normal((1, 1, D)).astype(np.float32))
    q = np.repeat(base, N, axis=1)
    k = synth.bf16_round(rng.standard_normal((H, N, D)).astype(np.float32))
    pq, _ = ops.reblock(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16))
    assert np.array_equal(pq.cpu().numpy()[0], np.arange(N))


def _full_layer(q, k, v, dt, ratio):
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    pq, pk = ops.reblock(qd, kd)
    lists = ops.select(qd, kd, pq, pk, topk_ratio=ratio)
    o, lse = ops.sparse_attn(qd, kd, vd, pq, pk, lists, with_lse=True)
    return (pq.cpu().numpy(), pk.cpu().numpy(), lists.cpu().numpy(), o.float().cpu().numpy(),
            lse.cpu().numpy())


def test_full_layer_f32_tiny(tiny):
    wl, q, k, v = tiny
    pq, pk, lists, o, lse = _full_layer(q, k, v, torch.float32, wl.topk_ratio)
    ro, rl = O.sparse_attention_head(q[0], k[0], v[0], pq[0], pk[0], lists[0])
    assert np.max(np.abs(o[0] - ro)) < 1e-4
    assert np.max(np.abs(lse[0] - rl)) < 1e-4


def test_full_layer_bf16_mid(mid):
    wl, q, k, v = mid
    pq, pk, lists, o, lse = _full_layer(q, k, v, torch.bfloat16, wl.topk_ratio)
    for h in range(q.shape[0]):
        ro, rl = O.sparse_attention_head(q[h], k[h], v[h], pq[h], pk[h], lists[h])
        assert np.linalg.norm(o[h] - ro) / np.linalg.norm(ro) < 1e-2
        assert np.max(np.abs(o[h] - ro)) < 3e-2
        assert np.max(np.abs(lse[h] - rl)) < 3e-2


# --------------------------------------------------------------- queries reuse the key layout

@pytest.mark.parametrize("which", ["tiny", "mid"])
def test_reblock_q_reuse_k_equals_key_layout(which, tiny, mid):
    """Key-reuse layout: perm_q is a copy of perm_k, and perm_k is bit-identical to the key
    layout of the separate reblock (the key trees are the same computation)."""
    wl, q, k, v = tiny if which == "tiny" else mid
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    qd, kd = to_dev(q, dt), to_dev(k, dt)
    sq, sk = ops.reblock(qd, kd)
    rq, rk, proj = ops.reblock(qd, kd, layout="q_reuse_k", with_proj=True)
    assert torch.equal(rk, sk)
    assert torch.equal(rq, rk)
    proj = proj.cpu().numpy()
    assert not proj[:, 0].any()                      # the query side is not partitioned
    # the key side against the oracle, split by split
    for h in range(q.shape[0]):
        st = replay_partition(O.metric_embed(k[h].astype(np.float64),
                                             O.second_moment(q[h].astype(np.float64))),
                              rk[h].cpu().numpy(), proj[h, 1])
        assert st["max_proj_err"] < 3e-5, st
        assert st["mismatched_splits"] <= 0.02 * st["splits"]


def test_full_layer_q_reuse_k_bf16_mid(mid):
    wl, q, k, v = mid
    dt = torch.bfloat16
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    pq, pk = ops.reblock(qd, kd, layout="q_reuse_k")
    lists = ops.select(qd, kd, pq, pk, topk_ratio=wl.topk_ratio)
    o, lse = ops.sparse_attn(qd, kd, vd, pq, pk, lists, with_lse=True)
    pq, pk, lists = pq.cpu().numpy(), pk.cpu().numpy(), lists.cpu().numpy()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(pq, pk)
    for h in range(q.shape[0]):
        ro, rl = O.sparse_attention_head(q[h], k[h], v[h], pq[h], pk[h], lists[h])
        assert np.linalg.norm(o[h] - ro) / np.linalg.norm(ro) < 1e-2
        assert np.max(np.abs(o[h] - ro)) < 3e-2
        assert np.max(np.abs(lse[h] - rl)) < 3e-2


@pytest.mark.parametrize("which", ["tiny", "mid"])
def test_reblock_one_side_equals_both(which, tiny, mid):
    """bsa_reblock_side builds each side alone, bit-identical to the two-sided call (the Lite
    step count too), with this side's projections and the other side's left 0."""
    wl, q, k, v = tiny if which == "tiny" else mid
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    qd, kd = to_dev(q, dt), to_dev(k, dt)
    for iters, shared, subtree in TREES:
        pq, pk, proj = ops.reblock(qd, kd, with_proj=True, power_iters=iters, shared_deep=shared,
                                   subtree_blocks=subtree)
        for side, ref in ((0, pq), (1, pk)):
            perm, pr = ops.reblock_side(qd, kd, side, power_iters=iters, with_proj=True,
                                        shared_deep=shared, subtree_blocks=subtree)
            assert torch.equal(perm, ref), (side, iters)
            assert torch.equal(pr[:, side], proj[:, side])
            assert torch.all(pr[:, 1 - side] == 0).item()
