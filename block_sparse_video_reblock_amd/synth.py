"""Seeded synthetic video-shaped Q/K/V: the one module both the kernels' tests and the oracle's
tests draw inputs from.

It holds none of the attention method's arithmetic.  It only builds inputs whose shape and
structure follow the workloads the pages describe: a 10-second 768p clip is 72,576 video tokens,
i.e. 1,134 blocks of 64 (comfy.icu "MiniMax H3 Spark Attention (SM89)", section "What it's doing
under the hood"); the budgets are the node's topk_ratio values 0.1 / 0.2 / 0.3 (same page,
section "Inputs you'll actually set").  The real activations (MiniMax-H3 weights on VBench
prompts) are not available; these tensors stand in for them.

Recipe (per configuration, per layer):
  * token id n = (t*H + y)*W + x on a latent grid (T, H, W); normalised position
    p = ((t+1/2)/T, (y+1/2)/H, (x+1/2)/W).
  * R = 32 random Fourier features phi_r = sqrt(2/R) cos(2 pi w_r . p + b_r),
    w_r ~ N(0, 3^2 I), b_r ~ U[0, 2 pi).
  * C spatial clusters: seeds s_m ~ U[0,1]^2 in (y, x), drift d_m ~ N(0, 0.3^2 I); centre at
    frame t is s_m + d_m (t+1/2)/T; a token belongs to its nearest centre (ties to lower m).
    Layer l (the long-clip workload) shifts every seed by l * D_m, D_m ~ N(0, 0.05^2 I).
  * per layer, shared by the heads: G_X (32 x D) and mu_X (C x D), both N(0, 1), X in {Q,K,V}.
  * per head: X = phi G_X + mu_X[region] + eps, eps ~ N(0, 0.5^2).
  * optional per-head Haar rotation of Q (so that head layouts differ).
  * per head, Q is scaled so that q.k/sqrt(D) over 65,536 random (query, key) pairs has std 2.
  * bf16 workloads are rounded to bf16 (round to nearest even); fp32 workloads stay fp32.
Seeds: numpy PCG64 from SeedSequence([workload, layer, stream]); stream 0 is shared, 1 + h is
head h.  The scene (Fourier features, cluster seeds, drifts, shifts) uses layer 0's stream 0.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int          # first SeedSequence word
    dtype: str            # "f32" or "bf16"
    heads: int
    head_dim: int
    grid: tuple           # (T, H, W)
    clusters: int
    topk_ratio: float
    rotate_q: bool
    layers: int = 1

    @property
    def tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_blocks(self) -> int:
        return self.tokens // BLOCK


WORKLOADS = {
    # tiny fp32 check: 1 head, 4,096 tokens on 4x32x32, head_dim 64, 25 % budget
    "tiny_f32": Workload("tiny_f32", 1, "f32", 1, 64, (4, 32, 32), 8, 0.25, False),
    # 8 heads, 16,384 tokens on 16x32x32, head_dim 128, 20 % budget
    "mid_bf16": Workload("mid_bf16", 2, "bf16", 8, 128, (16, 32, 32), 16, 0.2, False),
    # 24 heads, 72,576 tokens on 21x48x72 (1,134 blocks), 10 % budget, per-head rotation
    "clip10s_bf16": Workload("clip10s_bf16", 3, "bf16", 24, 128, (21, 48, 72), 32, 0.1, True),
    # 24 heads, 103,680 tokens on 30x48x72 (1,620 blocks), 10 % budget, four layers
    "clip14s_bf16": Workload("clip14s_bf16", 5, "bf16", 24, 128, (30, 48, 72), 32, 0.1, True, 4),
    # the largest sequence the library accepts: 2 heads, 524,288 tokens on 32x128x128
    # (8,192 blocks, 13 tree levels), 10 % budget
    "max_bf16": Workload("max_bf16", 6, "bf16", 2, 128, (32, 128, 128), 32, 0.1, True),
}
# the density sweep reuses the mid-size tensors at these budgets
SWEEP_RATIOS = (0.1, 0.2, 0.3, 1.0)
# context tokens of the mixed-sequence workloads (text, audio, conditioning): a count that is
# not a multiple of 64, so the last context tile is ragged
CTX_TOKENS = 1000


def _rng(*words) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words))))


def bf16_round_(x: np.ndarray) -> np.ndarray:
    """In place: round finite float32 values to the nearest bfloat16 (ties to even)."""
    bits = x.view(np.uint32)
    lsb = (bits >> 16) & np.uint32(1)
    bits += np.uint32(0x7FFF)
    bits += lsb
    bits &= np.uint32(0xFFFF0000)
    return x


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); returns float32."""
    return bf16_round_(np.array(x, dtype=np.float32, copy=True))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def token_coords(grid):
    t, h, w = grid
    tt, yy, xx = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    return tt.ravel(), yy.ravel(), xx.ravel()


def _scene(wl: Workload, layer: int):
    g = _rng(wl.seed_id, 0, 0)
    R = 32
    omega = g.normal(0.0, 3.0, size=(R, 3))
    beta = g.uniform(0.0, 2 * math.pi, size=R)
    seeds = g.uniform(0.0, 1.0, size=(wl.clusters, 2))
    drift = g.normal(0.0, 0.3, size=(wl.clusters, 2))
    shift = g.normal(0.0, 0.05, size=(wl.clusters, 2))
    T, H, W = wl.grid
    tt, yy, xx = token_coords(wl.grid)
    pos = np.stack([(tt + 0.5) / T, (yy + 0.5) / H, (xx + 0.5) / W], axis=1)
    phi = math.sqrt(2.0 / R) * np.cos(2 * math.pi * pos @ omega.T + beta)
    s = seeds + layer * shift
    frac = (tt + 0.5) / T
    best = np.full(tt.shape, np.inf)
    region = np.zeros(tt.shape, dtype=np.int64)
    for m in range(wl.clusters):
        cy = s[m, 0] + drift[m, 0] * frac
        cx = s[m, 1] + drift[m, 1] * frac
        d2 = (pos[:, 1] - cy) ** 2 + (pos[:, 2] - cx) ** 2
        closer = d2 < best
        best = np.where(closer, d2, best)
        region = np.where(closer, m, region)
    return phi.astype(np.float32), region


def _haar(g: np.random.Generator, d: int) -> np.ndarray:
    a = g.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def make_qkv(wl: Workload, layer: int = 0, heads=None):
    """Return (q, k, v) float32 arrays of shape [len(heads)][N][D] for the given heads (all by
    default).  bf16 workloads hold bf16-representable values."""
    if heads is None:
        heads = range(wl.heads)
    heads = list(heads)
    D = wl.head_dim
    phi, region = _scene(wl, layer)
    gl = _rng(wl.seed_id, layer, 0)
    base = []
    for _ in range(3):
        G = gl.standard_normal((32, D))
        mu = gl.standard_normal((wl.clusters, D))
        base.append((phi @ G.astype(np.float32)) + mu.astype(np.float32)[region])
    N = wl.tokens
    out = np.empty((3, len(heads), N, D), dtype=np.float32)

    def one_head(slot):
        h = heads[slot]
        gh = _rng(wl.seed_id, layer, 1 + h)
        for x in range(3):
            eps = out[x, slot]
            gh.standard_normal(dtype=np.float32, out=eps)
            eps *= np.float32(0.5)
            eps += base[x]
        if wl.rotate_q:
            rot = _haar(gh, D).astype(np.float32)
            out[0, slot] = out[0, slot] @ rot
        qi = gh.integers(0, N, size=65536)
        ki = gh.integers(0, N, size=65536)
        qk = np.einsum("ij,ij->i", out[0, slot][qi].astype(np.float64),
                       out[1, slot][ki].astype(np.float64)) / math.sqrt(D)
        out[0, slot] *= np.float32(2.0 / qk.std())
        if wl.dtype == "bf16":
            for x in range(3):
                bf16_round_(out[x, slot])

    # heads are independent streams; numpy releases the GIL in the bulk operations
    workers = max(1, min(len(heads), 16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one_head, range(len(heads))))
    return out[0], out[1], out[2]


def make_ctx(wl: Workload, n_ctx: int, like, layer: int = 0, heads=None):
    """Context tokens for a mixed sequence: (q, k, v) float32 [len(heads)][n_ctx][D].

    Two token types, a prefix of round(0.3 n_ctx) "text" tokens and the rest "audio /
    conditioning", with type means N(0, I) shared by the heads (SeedSequence([workload, layer,
    1000])), plus per-head noise N(0, 0.5^2) (SeedSequence([workload, layer, 1001 + h])); each
    tensor is then scaled to the RMS of the same head's video tensor in `like` = (q, k, v)
    (arrays over the same heads), and bf16 workloads are rounded to bf16."""
    if heads is None:
        heads = range(wl.heads)
    heads = list(heads)
    D = wl.head_dim
    gl = _rng(wl.seed_id, layer, 1000)
    means = [gl.standard_normal((2, D)).astype(np.float32) for _ in range(3)]
    kind = (np.arange(n_ctx) >= round(0.3 * n_ctx)).astype(np.int64)
    out = np.empty((3, len(heads), n_ctx, D), dtype=np.float32)
    for slot, h in enumerate(heads):
        gh = _rng(wl.seed_id, layer, 1001 + h)
        for x in range(3):
            y = means[x][kind] + np.float32(0.5) * gh.standard_normal((n_ctx, D), dtype=np.float32)
            ref = np.sqrt(np.mean(np.square(like[x][slot], dtype=np.float64)))
            y *= np.float32(ref / np.sqrt(np.mean(np.square(y, dtype=np.float64))))
            out[x, slot] = bf16_round(y) if wl.dtype == "bf16" else y
    return out[0], out[1], out[2]


def identity_perm(heads: int, tokens: int) -> np.ndarray:
    return np.tile(np.arange(tokens, dtype=np.int32), (heads, 1))
