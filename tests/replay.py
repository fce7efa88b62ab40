"""Tie-aware replay of a GPU tree partition against the oracle (test helper).

Every level's groups are contiguous position ranges of the final permutation, so the GPU's
groups can be read back from its output alone.  For each split the oracle recomputes the
projections on the GPU's own group; the GPU split is accepted when every token it sent left
projects no higher than every token it sent right, up to a tolerance (ties within `tol` may go
either way).  Optionally the GPU's own fp32 projections are compared with the oracle's."""
import numpy as np

import oracle as O


def replay_partition(U, perm, proj=None, tol=1e-5, leaf=64, max_level=None,
                     iters=O.POWER_ITERS, shared_deep=False,
                     subtree_blocks=O.LITE_SUBTREE_BLOCKS):
    """U: oracle unit vectors [N][D]; perm: GPU permutation; proj: GPU projections [L][N] by
    token id or None; max_level: replay only the first levels.  Returns a dict of statistics;
    raises AssertionError on a bad split."""
    N = U.shape[0]
    nb = N // leaf
    L = O.tree_levels(nb)
    stats = {"splits": 0, "mismatched_splits": 0, "max_proj_err": 0.0, "min_gap": np.inf}
    # Lite tree: below the root level every subtree keeps its root's projections
    root = O.shared_root_level(nb, subtree_blocks) if shared_deep else L
    key = np.zeros(N)
    groups = [(0, nb)]
    for lvl in range(L if max_level is None else min(L, max_level)):
        nxt = []
        for b0, m in groups:
            if m < 2:
                nxt.append((b0, m))
                continue
            ids = np.sort(perm[b0 * leaf:(b0 + m) * leaf])
            if lvl <= root:
                v = O.split_direction(U[ids], iters=iters)
                key[ids] = U[ids] @ v
            p = key[ids]
            cut = (m // 2) * leaf
            left = set(perm[b0 * leaf:b0 * leaf + cut].tolist())
            is_left = np.array([i in left for i in ids])
            hi_left = p[is_left].max()
            lo_right = p[~is_left].min()
            assert hi_left <= lo_right + tol, (lvl, b0, m, hi_left, lo_right)
            order = np.lexsort((ids, p.astype(np.float32)))
            ref_left = set(ids[order[:cut]].tolist())
            stats["splits"] += 1
            stats["mismatched_splits"] += int(ref_left != left)
            ps = np.sort(p)
            stats["min_gap"] = min(stats["min_gap"], ps[cut] - ps[cut - 1])
            if proj is not None:
                err = np.abs(proj[lvl][ids].astype(np.float64) - p).max()
                stats["max_proj_err"] = max(stats["max_proj_err"], float(err))
            nxt += [(b0, m // 2), (b0 + m // 2, m - m // 2)]
        groups = nxt
    return stats
