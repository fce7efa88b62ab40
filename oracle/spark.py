"""fp64 CPU oracle of the Spark-Attn layer (test infrastructure; see the package docstring).

All functions take float arrays holding the exact input values (for bf16 inputs: the
bf16-rounded values) and compute in float64.  Shapes: one head at a time, X is [N][D];
permutations are int arrays "token id at position p"; query block i is positions
[64 i, 64 i + 64) of perm_q, key block j is positions [64 j, 64 j + 64) of perm_k.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "LEAF", "POWER_ITERS", "LITE_SUBTREE_BLOCKS", "shared_root_level", "second_moment",
    "metric_factor", "metric_embed", "tree_levels",
    "split_direction", "partition", "partition_from_projections", "reblock_head",
    "topk_count", "block_means", "block_scores", "topk_lists", "summaries",
    "sparse_attention_head", "mixed_attention_head", "dense_attention_head", "recall_head",
    "log_mass_error_head",
    "logsumexp", "fixed_tile_perm",
]

LEAF = 64
POWER_ITERS = 8


def logsumexp(x: np.ndarray, axis=-1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


# ----------------------------------------------------------------------------- (1) Reblock

def second_moment(X: np.ndarray) -> np.ndarray:
    """Uncentred per-head second moment E[x x^T] = (1/N) sum_i x_i x_i^T.

    [P2] "What it's doing under the hood": M_K = E[k k^T] serves the queries, M_Q the keys.
    Reading: uncentred, normalised by N (the partition is invariant to the normalisation)."""
    X = np.asarray(X, dtype=np.float64)
    return X.T @ X / X.shape[0]


def metric_factor(M: np.ndarray, kind: str = "eigh") -> np.ndarray:
    """A factor F with F^T F = M, so that x^T M y = (F x).(F y).

    kind="eigh": F = diag(sqrt(lambda)) V^T (any positive semi-definite M);
    kind="cholesky": F = L^T with M = L L^T (positive-definite M).
    The partition depends on M only through inner products, hence not on this choice."""
    M = np.asarray(M, dtype=np.float64)
    if kind == "cholesky":
        return np.linalg.cholesky(M).T
    lam, V = np.linalg.eigh(M)
    return (V * np.sqrt(np.clip(lam, 0.0, None))).T


def metric_embed(X: np.ndarray, M_opp: np.ndarray, kind: str = "eigh") -> np.ndarray:
    """Unit vectors u_i = F x_i / |F x_i| whose dot products are the Mahalanobis cosines
    cos_M(x_i, x_j) = x_i^T M x_j / sqrt(x_i^T M x_i  x_j^T M x_j).

    [P1] "What Spark-Attn changes" (two queries are alike when their score patterns over the
    keys are alike) and [P2] (distance from the opposite side's second moment).  Reading: the
    score-pattern inner product sum_j (q1.k_j)(q2.k_j) = N q1^T M_K q2, so the metric tensor is
    M_opp itself, not its inverse.  A token with x^T M x = 0 gets u = 0."""
    F = metric_factor(M_opp, kind)
    Y = np.asarray(X, dtype=np.float64) @ F.T
    n = np.sqrt(np.einsum("ij,ij->i", Y, Y))
    U = np.zeros_like(Y)
    nz = n > 0
    U[nz] = Y[nz] / n[nz, None]
    return U


def tree_levels(n_blocks: int) -> int:
    """Number of split levels: ceil(log2(n_blocks)) (0 for a single block)."""
    return 0 if n_blocks <= 1 else int(math.ceil(math.log2(n_blocks)))


def split_direction(Ug: np.ndarray, iters: int = POWER_ITERS) -> np.ndarray:
    """Principal direction of one group by power iteration (rows of Ug in ascending token id).

    Reading of [P1]/[P2]'s hierarchical partitioner (the pages name no split rule): a
    principal-direction split.  c = group mean, C = (1/|G|) sum (u - c)(u - c)^T; start from
    u_{i0} - c for the smallest token id i0 whose centred vector is non-zero; T power steps
    v <- C v / |C v|; orient so that (u_{i0} - c).v >= 0.  A group with no spread gets v = 0
    (every projection ties and the split falls back to token id)."""
    c = Ug.mean(axis=0)
    d = Ug - c
    C = d.T @ d / Ug.shape[0]
    nz = np.flatnonzero(np.any(d != 0.0, axis=1))
    if nz.size == 0:
        return np.zeros(Ug.shape[1])
    d0 = d[nz[0]]
    v = d0.copy()
    for _ in range(iters):
        w = C @ v
        nw = np.sqrt(w @ w)
        if nw == 0.0:
            return np.zeros(Ug.shape[1])
        v = w / nw
    if d0 @ v < 0:
        v = -v
    return v


def _split_by_rank(ids: np.ndarray, p32: np.ndarray, n_left: int):
    """The n_left smallest (p, token id) pairs go left (capacity cut); both halves are
    returned in ascending token id."""
    order = np.lexsort((ids, p32))
    return np.sort(ids[order[:n_left]]), np.sort(ids[order[n_left:]])


# Subtree size of the Lite preset (in blocks).  The pages give no number for it: 8 is a chosen
# value of this reading, a parameter of the tree, not a fact of the method.
LITE_SUBTREE_BLOCKS = 8


def shared_root_level(n_blocks: int, subtree_blocks: int = LITE_SUBTREE_BLOCKS) -> int:
    """The first tree level whose groups all hold at most `subtree_blocks` blocks (the largest
    group of level l holds ceil(nb / 2^l) blocks)."""
    if subtree_blocks < 1:
        raise ValueError("subtree_blocks must be >= 1")
    lvl = 0
    while -(-n_blocks // (1 << lvl)) > subtree_blocks:
        lvl += 1
    return lvl


def partition(U: np.ndarray, leaf: int = LEAF, iters: int = POWER_ITERS,
              shared_deep: bool = False, subtree_blocks: int = LITE_SUBTREE_BLOCKS):
    """Capacity-constrained hierarchical tree partition into exactly-`leaf`-token leaves.

    [P2] "What it's doing under the hood": a tree partition under a capacity limit whose
    leaves hold 64 tokens each; [P1]: groups are split until every leaf has the block size, in
    O(N log N).  Reading: a group of m blocks (m >= 2) splits into floor(m/2) blocks (the
    floor(m/2)*leaf tokens of smallest (p, token id), p = u.v rounded to fp32) and the rest;
    recursion left first; leaves in that depth-first order; ascending token id inside a leaf.

    shared_deep (the Lite tree; [P1] "Benchmarks" names a lighter Spark-H3-Lite without its
    mechanism): from the first level whose groups hold at most `subtree_blocks` blocks, each
    group takes one direction and its descendants split along the same projections (no new
    direction), so that subtree is its tokens in (p, token id) order cut into leaves.

    Returns (perm, proj): perm[p] = token id at position p; proj[l][i] = the fp32 projection
    token i received at level l (0 where its group was already a leaf)."""
    N = U.shape[0]
    if N % leaf:
        raise ValueError("token count must be a multiple of the leaf size")
    nb = N // leaf
    L = tree_levels(nb)
    root = shared_root_level(nb, subtree_blocks) if shared_deep else L
    proj = np.zeros((L, N), dtype=np.float32)
    key = np.zeros(N, dtype=np.float32)   # the projections a shared subtree keeps using
    groups = [np.arange(N)]
    for lvl in range(L):
        nxt = []
        for ids in groups:
            m = ids.size // leaf
            if m < 2:
                nxt.append(ids)
                continue
            if lvl <= root:
                v = split_direction(U[ids], iters)
                key[ids] = (U[ids] @ v).astype(np.float32)
            p32 = key[ids]
            proj[lvl, ids] = p32
            left, right = _split_by_rank(ids, p32, (m // 2) * leaf)
            nxt += [left, right]
        groups = nxt
    perm = np.concatenate(groups).astype(np.int64)
    return perm, proj


def partition_from_projections(proj: np.ndarray, n_tokens: int, leaf: int = LEAF) -> np.ndarray:
    """The same tree, with each level's projections given (fp32, by token id)."""
    nb = n_tokens // leaf
    groups = [np.arange(n_tokens)]
    for lvl in range(tree_levels(nb)):
        nxt = []
        for ids in groups:
            m = ids.size // leaf
            if m < 2:
                nxt.append(ids)
                continue
            nxt += list(_split_by_rank(ids, np.asarray(proj[lvl][ids], np.float32),
                                       (m // 2) * leaf))
        groups = nxt
    return np.concatenate(groups).astype(np.int64)


def reblock_head(Q: np.ndarray, K: np.ndarray, leaf: int = LEAF, iters: int = POWER_ITERS,
                 kind: str = "eigh", layout: str = "separate", shared_deep: bool = False,
                 subtree_blocks: int = LITE_SUBTREE_BLOCKS):
    """Query layout from M_K, key layout from M_Q, each partitioned on its own ([P2]).
    Returns (perm_q, perm_k, proj_q, proj_k).  Q/K/V values are untouched.

    layout "q_reuse_k" ([P1] "Workflows": every shipped workflow pins reblock_layout =
    q_reuse_k; the pages do not define it, and the reading taken is its name): only the key
    layout is partitioned and the queries reuse it, perm_q = perm_k; proj_q is then None."""
    if layout not in ("separate", "q_reuse_k"):
        raise ValueError(f"unknown layout {layout!r}")
    M_q = second_moment(Q)
    perm_k, proj_k = partition(metric_embed(K, M_q, kind), leaf, iters, shared_deep,
                               subtree_blocks)
    if layout == "q_reuse_k":
        return perm_k.copy(), perm_k, None, proj_k
    M_k = second_moment(K)
    perm_q, proj_q = partition(metric_embed(Q, M_k, kind), leaf, iters, shared_deep,
                               subtree_blocks)
    return perm_q, perm_k, proj_q, proj_k


# ------------------------------------------------------------------ (2) scoring and top-K

def topk_count(n_blocks: int, ratio: float) -> int:
    """Selected blocks per query block for a topk_ratio budget ([P2] "Inputs you'll actually
    set").  Reading: the ratio is a float32; K = clamp(floor(ratio * nb + 1e-6), 1, nb)."""
    r = float(np.float32(ratio))
    return int(min(max(math.floor(r * n_blocks + 1e-6), 1), n_blocks))


def block_means(X: np.ndarray, perm: np.ndarray, leaf: int = LEAF) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    nb = X.shape[0] // leaf
    return X[np.asarray(perm)].reshape(nb, leaf, X.shape[1]).mean(axis=1)


def block_scores(Q, K, perm_q, perm_k, scale=None, leaf: int = LEAF) -> np.ndarray:
    """S_ij = s * mean(query block i) . mean(key block j), s = 1/sqrt(D) by default.
    Reading: mean-pooled block logits (the pages do not print the scoring rule)."""
    s = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    return s * block_means(Q, perm_q, leaf) @ block_means(K, perm_k, leaf).T


def topk_lists(S: np.ndarray, k: int) -> np.ndarray:
    """Per row the k largest scores, ties to the lower block index; each list ascending."""
    S = np.asarray(S)
    nb = S.shape[1]
    out = np.empty((S.shape[0], k), dtype=np.int64)
    j = np.arange(nb)
    for i in range(S.shape[0]):
        order = np.lexsort((j, -S[i].astype(np.float64)))
        out[i] = np.sort(order[:k])
    return out


# -------------------------------------------------------- (4) compressed-branch summaries

def summaries(Q, K, V, perm_k, scale=None, mode: str = "reweight", leaf: int = LEAF):
    """Per key block j a summary key kt_j, value vt_j and log-mass bias b_j.

    reweight ([P1] "What Spark-Attn changes", Spark-Reweight; [P2]): the anchor is the head's
    mean query qa; with x_t = s qa.k_t over the block's keys and w = softmax(x):
    kt = sum w_t k_t, vt = sum w_t v_t, b = logsumexp(x) - s qa.kt, so that for the anchor
    exp(s qa.kt + b) equals the block's exact exp-mass sum_t exp(x_t) ([P1] figure).
    meanpool (the fixed-block baseline): kt, vt are plain means, b = ln(leaf) (the block-count
    term only; the Jensen correction is what is dropped).
    Reading: every synthetic token is a video token, so the anchor is the mean of all N."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    nb = K.shape[0] // leaf
    Kb = K[np.asarray(perm_k)].reshape(nb, leaf, -1)
    Vb = V[np.asarray(perm_k)].reshape(nb, leaf, -1)
    if mode == "meanpool":
        return Kb.mean(axis=1), Vb.mean(axis=1), np.full(nb, math.log(leaf))
    if mode != "reweight":
        raise ValueError(mode)
    qa = Q.mean(axis=0)
    x = s * np.einsum("jtd,d->jt", Kb, qa)
    lse = logsumexp(x, axis=1)
    w = np.exp(x - lse[:, None])
    kt = np.einsum("jt,jtd->jd", w, Kb)
    vt = np.einsum("jt,jtd->jd", w, Vb)
    b = lse - s * kt @ qa
    return kt, vt, b


# ------------------------------------------ (3)(4)(5) branches, merge and inverse permutation

def _softmax_branch(logits: np.ndarray, values: np.ndarray):
    if logits.shape[1] == 0:
        return np.zeros((logits.shape[0], values.shape[1])), np.full(logits.shape[0], -np.inf)
    lse = logsumexp(logits, axis=1)
    return np.exp(logits - lse[:, None]) @ values, lse


def sparse_attention_head(Q, K, V, perm_q, perm_k, lists, scale=None, mode="reweight",
                          leaf: int = LEAF, summ=None, return_branches=False, blocks=None,
                          tail: str = "token", ctx=None):
    """One head of the two-branch layer, output in token order.

    [P1] "What Spark-Attn changes": an exact branch fully computes the top-ranked K/V blocks
    and a compressed branch covers the rest; [P2]: in the compressed branch each query uses its
    own vector and only keys and values are pooled.  For query block i and each of its
    queries q:
      exact:      softmax over s q.k for the keys of the selected blocks -> (O_e, lse_e)
      compressed: softmax over s q.kt_j + b_j for the unselected blocks j, values vt_j
                  -> (O_c, lse_c); no unselected block gives lse_c = -inf
      merge:      lse = logaddexp(lse_e, lse_c), O = e^(lse_e-lse) O_e + e^(lse_c-lse) O_c
      inverse permutation: row p of the block goes to token perm_q[p].
    tail = "block" is the tail_granularity option of [P2] "What it's doing under the hood"
    (ComfyUI's block-level behaviour): the compressed branch of every query of block i uses
    one pooled query, the mean of the block's queries, in place of the query's own; the exact
    branch and the merge are unchanged.  Reading: "pooled" is the plain mean.
    ctx = (K_ctx, V_ctx), context keys and values (text, audio, conditioning) that every
    query attends exactly ([P3] "Warmup and step counts need explicit definitions": exact
    handling of that context while the video grid is sparsified): they join the exact branch.
    Returns (O, lse) or, with return_branches, (O, lse, O_e, lse_e, O_c, lse_c).  With
    blocks (query block indices) only those blocks' rows are computed; the others hold NaN."""
    if tail not in ("token", "block"):
        raise ValueError(f"unknown tail granularity {tail!r}")
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, D = Q.shape
    s = 1.0 / math.sqrt(D) if scale is None else scale
    nb = N // leaf
    perm_q = np.asarray(perm_q)
    perm_k = np.asarray(perm_k)
    kt, vt, b = summaries(Q, K, V, perm_k, s, mode, leaf) if summ is None else summ
    key_rows = perm_k.reshape(nb, leaf)
    O = np.full((N, D), np.nan)
    lse = np.full(N, np.nan)
    parts = [np.full((N, D), np.nan), np.full(N, np.nan), np.full((N, D), np.nan),
             np.full(N, np.nan)]
    for i in (range(nb) if blocks is None else blocks):
        rows = perm_q[i * leaf:(i + 1) * leaf]
        q = Q[rows]
        sel = np.asarray(lists[i])
        keys = key_rows[sel].ravel()
        Ke, Ve = K[keys], V[keys]
        if ctx is not None:
            Ke = np.concatenate([Ke, np.asarray(ctx[0], np.float64)])
            Ve = np.concatenate([Ve, np.asarray(ctx[1], np.float64)])
        Oe, le = _softmax_branch(s * q @ Ke.T, Ve)
        mask = np.ones(nb, dtype=bool)
        mask[sel] = False
        qc = q if tail == "token" else np.repeat(q.mean(axis=0, keepdims=True), leaf, axis=0)
        Oc, lc = _softmax_branch(s * qc @ kt[mask].T + b[mask][None, :], vt[mask])
        lt = np.logaddexp(le, lc)
        O[rows] = np.exp(le - lt)[:, None] * Oe + np.exp(lc - lt)[:, None] * Oc
        lse[rows] = lt
        parts[0][rows], parts[1][rows], parts[2][rows], parts[3][rows] = Oe, le, Oc, lc
    if return_branches:
        return (O, lse, *parts)
    return O, lse


def dense_attention_head(Q, K, V, scale=None, rows=None, chunk: int = 1024):
    """Plain softmax(s Q K^T) V (and its row log-sum-exp), optionally for selected rows."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    idx = np.arange(Q.shape[0]) if rows is None else np.asarray(rows)
    O = np.empty((idx.size, V.shape[1]))
    lse = np.empty(idx.size)
    for a in range(0, idx.size, chunk):
        sl = slice(a, a + chunk)
        lg = s * Q[idx[sl]] @ K.T
        lse[sl] = logsumexp(lg, axis=1)
        O[sl] = np.exp(lg - lse[sl, None]) @ V
    return O, lse


def mixed_attention_head(Qv, Kv, Vv, Qc, Kc, Vc, perm_q, perm_k, lists, scale=None,
                         mode="reweight", tail: str = "token", leaf: int = LEAF):
    """One head of a mixed sequence: a video grid (Qv, Kv, Vv, [N][D], laid out by perm_q /
    perm_k with block lists) and context tokens (Qc, Kc, Vc, [n_ctx][D]: text, audio,
    conditioning).  [P3] "Warmup and step counts need explicit definitions": the context is
    handled exactly while only the video grid is sparsified; [P1] "What Spark-Attn changes":
    the Reweight anchor is the mean of the video queries.  Reading:
      video queries:   the sparse layer over the video grid, with every context key added to
                       the exact branch (summaries from the video tokens only);
      context queries: dense softmax attention over all keys, context and video.
    Returns (O_video, lse_video, O_ctx, lse_ctx), each in token order."""
    Ov, lv = sparse_attention_head(Qv, Kv, Vv, perm_q, perm_k, lists, scale, mode, leaf,
                                   tail=tail, ctx=(Kc, Vc))
    Kall = np.concatenate([np.asarray(Kc, np.float64), np.asarray(Kv, np.float64)])
    Vall = np.concatenate([np.asarray(Vc, np.float64), np.asarray(Vv, np.float64)])
    Oc, lc = dense_attention_head(Qc, Kall, Vall, scale)
    return Ov, lv, Oc, lc


# ------------------------------------------------------------ fixed-tile baseline layout

def fixed_tile_perm(grid, tile=(4, 4, 4)) -> np.ndarray:
    """Positional layout that Reblock replaces ([P1] "What Spark-Attn changes": fixed
    spatiotemporal tiles; [P2] "What it's doing under the hood": recall against fixed blocks).
    The latent grid (T, H, W), token id (t H + y) W + x, is cut into a x b x c cubes of 64
    tokens; blocks are the cubes in raster order of their corner, tokens in raster order inside
    a cube.  Returns token ids by position."""
    T, H, W = grid
    a, b, c = tile
    if a * b * c != LEAF or T % a or H % b or W % c:
        raise ValueError(f"tile {tile} does not cut grid {grid} into {LEAF}-token cubes")
    out = []
    for ct in range(T // a):
        for cy in range(H // b):
            for cx in range(W // c):
                for t in range(ct * a, ct * a + a):
                    for y in range(cy * b, cy * b + b):
                        for x in range(cx * c, cx * c + c):
                            out.append((t * H + y) * W + x)
    return np.asarray(out, dtype=np.int32)


# ------------------------------------------------------------------ measurements ([P2])

def recall_head(Q, K, perm_q, perm_k, lists, scale=None, leaf: int = LEAF) -> float:
    """Attention-mass recall: mean over queries of the dense softmax mass that falls on the
    keys of the query's selected blocks ([P2] reports it for Reblock vs fixed blocks)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    s = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    nb = Q.shape[0] // leaf
    key_rows = np.asarray(perm_k).reshape(nb, leaf)
    total = 0.0
    for i in range(nb):
        q = Q[np.asarray(perm_q)[i * leaf:(i + 1) * leaf]]
        lg = s * q @ K.T
        P = np.exp(lg - logsumexp(lg, axis=1)[:, None])
        total += P[:, key_rows[np.asarray(lists[i])].ravel()].sum()
    return total / Q.shape[0]


def log_mass_error_head(Q, K, V, perm_q, perm_k, lists, scale=None, mode="reweight",
                        leaf: int = LEAF) -> float:
    """Mean absolute log-mass error over (query, unselected block) pairs: the block's true
    log-mass logsumexp_t(s q.k_t) against the compressed estimate s q.kt_j + b_j ([P2]
    reports it for Reweight vs mean pooling)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    s = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    nb = Q.shape[0] // leaf
    kt, _, b = summaries(Q, K, V, perm_k, s, mode, leaf)
    Kb = K[np.asarray(perm_k)].reshape(nb, leaf, -1)
    err, cnt = 0.0, 0
    for i in range(nb):
        q = Q[np.asarray(perm_q)[i * leaf:(i + 1) * leaf]]
        mask = np.ones(nb, dtype=bool)
        mask[np.asarray(lists[i])] = False
        if not mask.any():
            continue
        true = logsumexp(s * np.einsum("qd,jtd->qjt", q, Kb[mask]), axis=2)
        est = s * q @ kt[mask].T + b[mask][None, :]
        err += np.abs(true - est).sum()
        cnt += true.size
    return err / max(cnt, 1)
