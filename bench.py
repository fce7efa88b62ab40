#!/usr/bin/env python3
"""Benchmark of the Spark-Attn block-sparse attention layer on one MI355X.

One step is the whole layer on one batch of synthetic video-shaped Q/K/V already resident in
HBM: reblock (both layouts of every head), block scoring + top-K, summaries, and the two-branch
attention with merge and inverse permutation.  Timed with HIP events on the stream the library
launches on.  Prints one JSON line (the last line of stdout).

Default (the headline): 24 heads x 72,576 tokens x 128, bf16, 10 % density.
  value      dense-equivalent effective TFLOP/s = 4 N^2 D H / layer time
  roofline   the attention kernel (the dominant one): algorithmic flops of the exact and
             compressed branches per launch / its mean launch time, against the bf16 MFMA peak
  dense      the same attention kernel with every block selected and identity layouts (dense
             softmax attention), timed on the same GPU
  cpu_baseline  the CPU oracle (fp64 numpy) on one head of the same workload, extrapolated to
             all heads
  machine    practical ceilings measured beside it: a vendor bf16 GEMM and a device copy
Options on the headline (same JSON line, recorded in config): --layout q_reuse_k (queries reuse
the key layout), --tail block (block-level compressed branch), --ctx N (N exact context tokens
beside the video grid), --lite (the Lite reblock).
Other modes (each prints its own JSON line):
  --workload clip14s_bf16   four independently generated 103,680-token layers back to back,
                            reblock recomputed per layer; value per layer
  --sweep                   the 16,384-token shape at densities 0.1 / 0.2 / 0.3 / 1.0, with
                            Reblock layouts (default, 2 power steps, Lite, key layout reused)
                            and with the fixed-tile baseline (positional 4x4x4 cubes,
                            mean-pooled summaries); layer time and attention-mass recall
                            against dense softmax, both measured on the GPU
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "sparse attn layer ms + effective TFLOP/s at 72,576 tok, 10% density, vs dense"
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
# Bytes one attention launch moves between L2 and memory: rocprofv3 FETCH_SIZE x 2 +
# WRITE_SIZE x 1 (the factors a plain 1 GiB copy gives those counters), per configuration
# (workload, tail granularity, context tokens, reblock layout), from the counter runs kept in
# profiles/.  They hold only for the attention source they were taken on: the benchmark
# reports traffic null when the hash of that source differs.
ATTN_SOURCES = ("block_sparse_video_reblock_amd/csrc/attn.hip",
                "block_sparse_video_reblock_amd/csrc/common.h",
                "block_sparse_video_reblock_amd/csrc/internal.h")
ATTN_TRAFFIC = {"source_sha16": "d50ffa2e1cf7a196", "bytes": {
    # key: workload / tail granularity / context tokens / reblock layout / tree
    "clip10s_bf16/token/0/separate/full": 4.4294e10,
    "clip10s_bf16/block/0/separate/full": 3.7701e10,
    "clip10s_bf16/token/1000/separate/full": 6.0276e10,
    "clip10s_bf16/token/0/q_reuse_k/full": 5.3572e10,
    "clip10s_bf16/token/0/separate/lite": 2.0720e10,
}}
# The pages' own figures for the method, quoted as context (other hardware, other workloads,
# end-to-end or attention-op times not always stated): they are not targets for this run.
PAGE_FIGURES = [
    {"figure": "2.37x faster than dense attention, fidelity mode (first 20% of evaluations "
               "dense)", "hardware": "RTX 4090 (SM89), BF16",
     "workload": "LightX2V 768p 8-step workflow, 1344x768, 345 frames",
     "source": "comfy.icu 'MiniMax H3 Spark Attention (SM89)', opening paragraph"},
    {"figure": "4.35x faster than dense attention, speed mode (sparse from the first "
               "evaluation)", "hardware": "RTX 4090 (SM89), BF16",
     "workload": "LightX2V 768p 8-step workflow, 1344x768, 345 frames",
     "source": "comfy.icu 'MiniMax H3 Spark Attention (SM89)', opening paragraph"},
    {"figure": "+2.94 dB PSNR over Sol-H3 at 10% density, slightly faster",
     "hardware": "RTX PRO 6000 Blackwell (SM120)",
     "workload": "VBench prompts, 1344x768, 240 frames, 19-step MiniMax-H3, PSNR against "
                 "the dense render",
     "source": "comfyui-wiki.com 'Spark-H3 ...', section 'Benchmarks'"},
]


def source_sha16(paths):
    """First 16 hex digits of the SHA-256 of the given repository files, concatenated."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in paths:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attn_traffic(workload, tail, ctx, layout, lite):
    """Measured L2<->memory bytes of one attention launch in this configuration, or None when
    no counter run covers it or the attention source has changed since."""
    if source_sha16(ATTN_SOURCES) != ATTN_TRAFFIC["source_sha16"]:
        return None
    tree = "lite" if lite else "full"
    return ATTN_TRAFFIC["bytes"].get(f"{workload}/{tail}/{ctx}/{layout}/{tree}")


# The reblock kernels hold a subtree in LDS from the first level whose groups have at most this
# many blocks; the levels below it cost one pass over the tensors together.
ON_CHIP_SUBTREE_BLOCKS = 8


def on_chip_root_level(nb, blocks=ON_CHIP_SUBTREE_BLOCKS):
    lvl = 0
    while -(-nb // (1 << lvl)) > blocks:
        lvl += 1
    return lvl


def reblock_bytes(nb, x_bytes, sides, subtree_root):
    """Algorithmic HBM bytes of the reblock: per side, one pass over the tensor for the moments,
    one for the norms, a statistics and a projection pass for every tree level above the first
    level whose groups are held on chip, and one pass for that on-chip tail of the tree.
    Also the plain algorithm's count, with the two passes for every level."""
    levels = max(0, (nb - 1).bit_length())
    hbm_levels = min(levels, subtree_root)
    tail = 1 if hbm_levels < levels else 0
    return (sides * x_bytes * (2 + 2 * hbm_levels + tail),
            sides * x_bytes * (2 + 2 * levels))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(H, N, D, topk, tail="token"):
    """Algorithmic flops of one attend: 4 D per (query, key) pair for the exact branch and per
    (query, summary) pair for the compressed one (one pooled query per block with tail "block")."""
    nb = N // 64
    exact = 4.0 * N * (topk * 64) * D * H
    rows = N if tail == "token" else nb
    compressed = 4.0 * rows * (nb - topk) * D * H
    return exact, compressed


def cpu_baseline(wl, q, k, v):
    """Oracle on head 0; returns (seconds for one head, threads used)."""
    import numpy as np
    import oracle as O
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()),
                      default=1)
    except Exception:  # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    Q, K, V = (x[0].astype(np.float64) for x in (q, k, v))
    t0 = time.perf_counter()
    pq, pk, _, _ = O.reblock_head(Q, K)
    kk = O.topk_count(wl.n_blocks, wl.topk_ratio)
    lists = O.topk_lists(O.block_scores(Q, K, pq, pk).astype(np.float32), kk)
    O.sparse_attention_head(Q, K, V, pq, pk, lists)
    return time.perf_counter() - t0, threads


class Layer:
    """Device buffers and the four stage calls of one layer (Reblock or fixed-tile layouts)."""

    def __init__(self, ops, torch, wl, q, k, v, topk, fixed_tiles=False, ws=None,
                 layout="separate", tail="token", ctx=None, power_iters=8, lite_tree=False,
                 subtree_blocks=0):
        self.ops, self.torch = ops, torch
        dev = torch.device("cuda:0")
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.wl = wl
        self.H, self.N = wl.heads, wl.tokens
        self.nb = self.N // 64
        self.topk = topk
        self.qd, self.kd, self.vd = (torch.from_numpy(x).to(dev).to(dt) for x in (q, k, v))
        self.d = ops.desc_for(self.qd)
        # context tokens of a mixed sequence (exact), or none
        self.n_ctx = 0 if ctx is None else ctx[0].shape[1]
        if self.n_ctx:
            self.qcd, self.kcd, self.vcd = (torch.from_numpy(x).to(dev).to(dt) for x in ctx)
            self.out_ctx = torch.empty_like(self.qcd)
            self.ws = ops.workspace_ctx(self.d, self.n_ctx, dev)
        else:
            self.ws = ops.workspace(self.d, dev) if ws is None else ws
        self.perm_q = torch.empty(self.H, self.N, dtype=torch.int32, device=dev)
        self.perm_k = torch.empty_like(self.perm_q)
        self.lists = torch.empty(self.H, self.nb, topk, dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.qd)
        self.fixed = fixed_tiles
        self.reblock_layout = ops._LAYOUTS[layout]
        self.power_iters = power_iters
        self.tree_flags = ops.tree_flags(lite_tree, subtree_blocks if lite_tree else 0)
        self.subtree_blocks = (subtree_blocks or ops.BSA_DEFAULT_SUBTREE_BLOCKS) if lite_tree \
            else 0
        self.flags = ((ops.BSA_MEANPOOL if fixed_tiles else 0) |
                      (ops.BSA_TAIL_BLOCK if tail == "block" else 0))
        self.L = ops.lib()
        self.stream = ops._stream()

    @staticmethod
    def p(t):
        return ctypes.c_void_p(t.data_ptr())

    def layout(self):
        p, ops = self.p, self.ops
        if self.fixed:
            T, Hh, W = self.wl.grid
            ops.check(self.L.bsa_tile_layout(self.H, T, Hh, W, 4, 4, 4, p(self.perm_q),
                                             self.stream))
            ops.check(self.L.bsa_tile_layout(self.H, T, Hh, W, 4, 4, 4, p(self.perm_k),
                                             self.stream))
        else:
            ops.check(self.L.bsa_reblock_ex(ctypes.byref(self.d), p(self.qd), p(self.kd),
                                            self.reblock_layout, self.power_iters,
                                            self.tree_flags, p(self.perm_q), p(self.perm_k),
                                            None, p(self.ws), self.ws.numel(), self.stream))

    def select(self):
        p = self.p
        self.ops.check(self.L.bsa_select(ctypes.byref(self.d), p(self.qd), p(self.kd),
                                         p(self.perm_q), p(self.perm_k), 0.0, self.topk,
                                         p(self.lists), None, p(self.ws), self.ws.numel(),
                                         self.stream))

    def prepare(self, pk=None, flags=None):
        p = self.p
        if self.n_ctx:
            self.ops.check(self.L.bsa_prepare_kv_ctx(
                ctypes.byref(self.d), self.n_ctx, p(self.qd), p(self.kd), p(self.vd),
                p(self.kcd), p(self.vcd), p(self.perm_k if pk is None else pk),
                self.flags if flags is None else flags, 0.0, p(self.ws), self.ws.numel(),
                self.stream))
            return
        self.ops.check(self.L.bsa_prepare_kv(ctypes.byref(self.d), p(self.qd), p(self.kd),
                                             p(self.vd), p(self.perm_k if pk is None else pk),
                                             self.flags if flags is None else flags, 0.0,
                                             p(self.ws), self.ws.numel(), self.stream))

    def attend(self, pq=None, pk=None, ls=None, flags=None, lse=None):
        p = self.p
        ls = self.lists if ls is None else ls
        if self.n_ctx:
            self.ops.check(self.L.bsa_attend_ctx(
                ctypes.byref(self.d), self.n_ctx, p(self.qd), p(self.kd), p(self.vd),
                p(self.qcd), p(self.kcd), p(self.vcd), p(self.perm_q if pq is None else pq),
                p(self.perm_k if pk is None else pk), p(ls), int(ls.shape[-1]),
                self.flags if flags is None else flags, 0.0, p(self.out), p(self.out_ctx),
                None if lse is None else p(lse), None, p(self.ws), self.ws.numel(),
                self.stream))
            return
        self.ops.check(self.L.bsa_attend(ctypes.byref(self.d), p(self.qd), p(self.kd),
                                         p(self.vd), p(self.perm_q if pq is None else pq),
                                         p(self.perm_k if pk is None else pk), p(ls),
                                         int(ls.shape[-1]), self.flags if flags is None else flags,
                                         0.0, p(self.out), None if lse is None else p(lse),
                                         p(self.ws), self.ws.numel(), self.stream))

    def stages(self):
        return (("layout" if self.fixed else "reblock", self.layout), ("select", self.select),
                ("prepare", self.prepare), ("attend", self.attend))

    def dense_inputs(self):
        torch, dev = self.torch, self.qd.device
        ident = torch.arange(self.N, dtype=torch.int32, device=dev).repeat(self.H, 1).contiguous()
        every = torch.arange(self.nb, dtype=torch.int32,
                             device=dev).repeat(self.H, self.nb, 1).contiguous()
        return ident, every

    def recall(self, lse_dense):
        """Mean over heads and queries of exp(lse over the selected blocks - dense lse): the
        dense softmax mass that the selected blocks capture."""
        torch = self.torch
        lse = torch.empty(self.H, self.N, dtype=torch.float32, device=self.qd.device)
        self.prepare()
        self.attend(flags=self.ops.BSA_EXACT_ONLY | (self.flags & self.ops.BSA_MEANPOOL), lse=lse)
        return float(torch.exp(lse - lse_dense).mean().item())

    def dense_lse(self):
        torch = self.torch
        ident, every = self.dense_inputs()
        lse = torch.empty(self.H, self.N, dtype=torch.float32, device=self.qd.device)
        self.prepare(pk=ident, flags=self.ops.BSA_EXACT_ONLY)
        self.attend(pq=ident, pk=ident, ls=every, flags=self.ops.BSA_EXACT_ONLY, lse=lse)
        return lse


def log_mass_error(torch, ops, qd, kd, vd, perm_q, perm_k, lists, meanpool=False, chunk=16):
    """Mean absolute log-mass error of the compressed branch over (query, unselected block)
    pairs, measured on the GPU from the library's block summaries (comfy.icu 'MiniMax H3 Spark
    Attention (SM89)', 'What it's doing under the hood', reports it for Reweight against mean
    pooling): for query q and key block j the true log-mass is logsumexp_t(s q.k_t) over the
    block's keys and the estimate s q.kt_j + b_j.  Plain torch in fp32 on the device tensors;
    a measurement beside the layer, not a step of it."""
    H, N, D = qd.shape
    nb = N // 64
    s = 1.0 / (D ** 0.5)
    kt, _, b = ops.summaries(qd, kd, vd, perm_k, flags=ops.BSA_MEANPOOL if meanpool else 0)
    total, count = 0.0, 0
    for h in range(H):
        kp = kd[h].float()[perm_k[h].long()]                 # keys in key-block order
        sel = torch.zeros(nb, nb, dtype=torch.bool, device=qd.device)
        sel.scatter_(1, lists[h].long(), True)
        for i0 in range(0, nb, chunk):
            i1 = min(nb, i0 + chunk)
            rows = perm_q[h, 64 * i0:64 * i1].long()
            q = qd[h].float()[rows]
            true = torch.logsumexp((s * q @ kp.T).view(-1, nb, 64), dim=2)
            est = s * q @ kt[h].T + b[h][None, :]
            unsel = (~sel[i0:i1]).repeat_interleave(64, dim=0)
            total += float((true - est).abs()[unsel].double().sum().item())
            count += int(unsel.sum().item())
    return total / max(count, 1)


def time_steps(torch, fns_per_step, steps, warmup):
    """Time `steps` steps, each the list of (name, fn) calls; returns (ms per step, {name: mean
    ms}, {name: [ms per step]})."""
    import numpy as np
    for _ in range(warmup):
        for _, f in fns_per_step:
            f()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    n = len(fns_per_step)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur)
    for s in range(steps):
        ev[s][0].record(cur)
        for i, (_, f) in enumerate(fns_per_step):
            f()
            ev[s][i + 1].record(cur)
    stop.record(cur)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    per = {}
    for i, (name, _) in enumerate(fns_per_step):
        per.setdefault(name, []).append([ev[s][i].elapsed_time(ev[s][i + 1])
                                         for s in range(steps)])
    means = {k: float(np.mean(np.sum(v, axis=0))) for k, v in per.items()}
    series = {k: list(np.sum(v, axis=0)) for k, v in per.items()}
    return ms_step, means, series


def measure_machine(torch, np):
    """Practical ceilings measured on this GPU in the same run: a large bf16 GEMM (the vendor
    library's MFMA kernel) and a device-to-device copy, each the best of five."""
    dev = torch.device("cuda:0")
    n, kk = 8192, 16384
    a = torch.randn(n, kk, device=dev).to(torch.bfloat16)
    b = torch.randn(kk, n, device=dev).to(torch.bfloat16)
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cur = torch.cuda.current_stream()

    def best(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            fn()
            e1.record(cur)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(min(ts))
    gemm_ms = best(lambda: a @ b)
    copy_ms = best(lambda: dst.copy_(src))
    out = {"gemm_bf16_tflops": 2.0 * n * n * kk / (gemm_ms * 1e-3) / 1e12,
           "gemm": f"torch.matmul bf16 {n}x{kk} @ {kk}x{n}",
           "copy_gbs": 2.0 * src.numel() / (copy_ms * 1e-3) / 1e9,
           "copy": "2 GiB device-to-device copy, read + write bytes"}
    del a, b, src, dst
    torch.cuda.empty_cache()
    return out


def main_headline(args, ops, synth, torch, np):
    wl = synth.WORKLOADS[args.workload]
    H, N, D = wl.heads, wl.tokens, wl.head_dim
    nb = N // 64
    topk = ops.topk_count(nb, wl.topk_ratio)
    log(f"[bench] workload {wl.name}: H={H} N={N} D={D} nb={nb} topk={topk} dtype={wl.dtype}")
    t0 = time.perf_counter()
    q, k, v = synth.make_qkv(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    ctx = synth.make_ctx(wl, args.ctx, (q, k, v)) if args.ctx else None
    lay = Layer(ops, torch, wl, q, k, v, topk, layout=args.layout, tail=args.tail, ctx=ctx,
                power_iters=ops.BSA_POWER_ITERS_LITE if args.lite else ops.BSA_POWER_ITERS,
                lite_tree=args.lite, subtree_blocks=args.lite_subtree)
    ms_step, stage_ms, series = time_steps(torch, lay.stages(), args.steps, args.warmup)
    steps_ms = [sum(x) for x in zip(*series.values())]
    assert torch.isfinite(lay.out.float()).all().item(), "non-finite output"
    log(f"[bench] layer {ms_step:.3f} ms/step; stages " +
        ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))

    exact_f, comp_f = attention_flops(H, N, D, topk, args.tail)
    # context tokens: video queries x context keys, context queries x every key
    exact_f += 4.0 * (N * args.ctx + args.ctx * (N + args.ctx)) * D * H
    attn_ms = stage_ms["attend"]
    achieved = (exact_f + comp_f) / (attn_ms * 1e-3) / 1e12
    dense_flops = 4.0 * (N + args.ctx) ** 2 * D * H
    eff = dense_flops / (ms_step * 1e-3) / 1e12

    # HBM-bound stages: algorithmic bytes (inputs read once per pass the algorithm needs)
    elt = 2 if wl.dtype == "bf16" else 4
    x_bytes = H * N * D * elt
    sides = 1 if args.layout == "q_reuse_k" else 2
    if args.lite:
        # the Lite tree stops at the shared root level, whose groups each take a statistics and
        # a projection pass and are then sorted on chip
        lr = on_chip_root_level(nb, lay.subtree_blocks)
        rb_bytes = sides * x_bytes * (2 + 2 * lr + 2)
        rb_plain = reblock_bytes(nb, x_bytes, sides, on_chip_root_level(nb))[1]
    else:
        rb_bytes, rb_plain = reblock_bytes(nb, x_bytes, sides, on_chip_root_level(nb))
    hbm = {
        "reblock": {"bytes": rb_bytes, "plain_passes_bytes": rb_plain,
                    "passes": ("moments, norms, a statistics and a projection pass per tree "
                               "level above the shared root, and a statistics and a "
                               "projection pass for the shared subtrees" if args.lite else
                               "moments, norms, a statistics and a projection pass per tree "
                               "level until the groups fit on chip, and one pass for the "
                               "subtrees held on chip") + ", over " +
                              ("K" if sides == 1 else "Q and K") +
                              " (plain_passes_bytes: two passes for every level)"},
        "select": {"bytes": 2 * x_bytes + H * nb * nb * 4, "passes": "Q, K once; scores"},
        # the permutation: K and V written once more in block-contiguous (operand) order
        "prepare": {"bytes": 5 * x_bytes + 4 * H * args.ctx * D * elt,
                    "read_only_bytes": 3 * x_bytes + 2 * H * args.ctx * D * elt,
                    "passes": "Q (anchor), K, V read once; K, V written once in key-block "
                              "order (the permutation)" +
                              (", context K, V read and written once" if args.ctx else "")},
    }
    for name, h in hbm.items():
        gbs = h["bytes"] / (stage_ms[name] * 1e-3) / 1e9
        h.update({"ms": stage_ms[name], "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS})

    machine = roof = None
    if not args.no_machine:
        machine = measure_machine(torch, np)
        log(f"[bench] machine: bf16 GEMM {machine['gemm_bf16_tflops']:.0f} TFLOP/s, copy "
            f"{machine['copy_gbs']:.0f} GB/s")
        roof = achieved / machine["gemm_bf16_tflops"]
        for h in hbm.values():
            h["frac_of_copy"] = h["GB/s"] / machine["copy_gbs"]

    dense = None
    if not args.no_dense and not args.ctx:
        ident, every = lay.dense_inputs()
        lay.prepare(pk=ident, flags=ops.BSA_EXACT_ONLY)
        cur = torch.cuda.current_stream()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            lay.attend(pq=ident, pk=ident, ls=every, flags=ops.BSA_EXACT_ONLY)
            e1.record(cur)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        dense_ms = float(min(times[1:]))
        dense = {"ms": dense_ms, "tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
                 "speedup_of_sparse_layer": dense_ms / ms_step,
                 "kernel": "same attention kernel, every block selected, identity layouts"}
        log(f"[bench] dense attention {dense_ms:.2f} ms ({dense['tflops']:.0f} TFLOP/s); "
            f"sparse layer speed-up {dense_ms / ms_step:.2f}x")
        del every

    recall = None
    if args.recall and not args.ctx:
        # attention-mass recall of this run's layouts at the pages' three budgets, measured on
        # the GPU against dense softmax (the exact branch alone, then every block)
        lse_dense = lay.dense_lse()
        recall = {}
        for r in (0.1, 0.2, 0.3):
            kr = ops.topk_count(nb, r)
            lists_r = torch.empty(H, nb, kr, dtype=torch.int32, device=lay.qd.device)
            ops.check(lay.L.bsa_select(ctypes.byref(lay.d), lay.p(lay.qd), lay.p(lay.kd),
                                       lay.p(lay.perm_q), lay.p(lay.perm_k), 0.0, kr,
                                       lay.p(lists_r), None, lay.p(lay.ws), lay.ws.numel(),
                                       lay.stream))
            lse = torch.empty(H, N, dtype=torch.float32, device=lay.qd.device)
            lay.prepare()
            lay.attend(ls=lists_r, flags=ops.BSA_EXACT_ONLY, lse=lse)
            recall[str(r)] = float(torch.exp(lse - lse_dense).mean().item())
            del lists_r
        log("[bench] recall " + ", ".join(f"{k}: {v:.4f}" for k, v in recall.items()))

    cpu = None
    if not args.no_cpu_baseline and not args.ctx:
        log("[bench] timing the CPU oracle on head 0 ...")
        t_head, threads = cpu_baseline(wl, q, k, v)
        layer_s = t_head * H
        cpu = {"value": dense_flops / layer_s / 1e12, "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "ms_per_layer": layer_s * 1e3,
               "sample": f"fp64 numpy oracle, full layer (reblock both sides, scores, top-K, "
                         f"summaries, exact + compressed attention) on head 0 of {H}: "
                         f"{t_head:.1f} s, extrapolated x{H}"}
        log(f"[bench] oracle head 0: {t_head:.1f} s -> {layer_s * 1e3:.0f} ms per layer")

    return {
        "metric": METRIC,
        "value": eff,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "heads": H, "tokens": N, "head_dim": D,
                   "topk_ratio": wl.topk_ratio, "topk_blocks": topk, "grid": list(wl.grid),
                   "reblock_layout": args.layout, "tail_granularity": args.tail,
                   "context_tokens": args.ctx,
                   "reblock_power_iters": lay.power_iters,
                   "reblock_lite_tree": bool(lay.tree_flags),
                   "reblock_lite_subtree_blocks": lay.subtree_blocks,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": attn_traffic(wl.name, args.tail, args.ctx, args.layout,
                                             args.lite),
                     "traffic_source_sha16": source_sha16(ATTN_SOURCES),
                     "kernel": "k_attn_bf16",
                     "launch_ms": attn_ms, "launch_ms_min": float(min(series["attend"])),
                     "frac_of_gemm": roof,
                     "flops_per_launch": exact_f + comp_f},
        "stages_ms": stage_ms,
        "step_ms_median": float(np.median(steps_ms)),
        "step_ms_min": float(min(steps_ms)),
        "step_ms_max": float(max(steps_ms)),
        "machine": machine,
        "hbm": hbm,
        "dense": dense,
        "recall": recall,
        "cpu_baseline": cpu,
        "page_figures": PAGE_FIGURES,
    }


def main_layers(args, ops, synth, torch, np):
    """Several independently generated layers back to back (the long-clip workload)."""
    wl = synth.WORKLOADS[args.workload]
    H, N, D = wl.heads, wl.tokens, wl.head_dim
    nb = N // 64
    topk = ops.topk_count(nb, wl.topk_ratio)
    log(f"[bench] workload {wl.name}: {wl.layers} layers, H={H} N={N} D={D} nb={nb} "
        f"topk={topk}")
    layers = []
    ws = None
    for layer in range(wl.layers):
        t0 = time.perf_counter()
        q, k, v = synth.make_qkv(wl, layer=layer)
        lay = Layer(ops, torch, wl, q, k, v, topk, ws=ws)
        ws = lay.ws  # layers run one after another: one workspace serves them all
        layers.append(lay)
        log(f"[bench] layer {layer} inputs generated in {time.perf_counter() - t0:.1f} s")
    fns = [(f"L{i}.{name}", f) for i, lay in enumerate(layers) for name, f in lay.stages()]
    ms_step, stage_ms, _ = time_steps(torch, fns, args.steps, args.warmup)
    for lay in layers:
        assert torch.isfinite(lay.out.float()).all().item(), "non-finite output"
    per_layer = ms_step / wl.layers
    by_stage = {s: float(np.mean([stage_ms[f"L{i}.{s}"] for i in range(wl.layers)]))
                for s in ("reblock", "select", "prepare", "attend")}
    exact_f, comp_f = attention_flops(H, N, D, topk)
    dense_flops = 4.0 * N * N * D * H
    log(f"[bench] {wl.layers} layers {ms_step:.3f} ms/step, {per_layer:.3f} ms per layer; "
        "per-layer stages " + ", ".join(f"{k} {v:.3f}" for k, v in by_stage.items()))
    achieved = (exact_f + comp_f) / (by_stage["attend"] * 1e-3) / 1e12
    return {
        "metric": f"sparse attn layer ms + effective TFLOP/s at {N:,} tok, "
                  f"{int(round(100 * wl.topk_ratio))}% density, {wl.layers} layers back to back",
        "value": dense_flops / (per_layer * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "ms_per_layer": per_layer,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "heads": H, "tokens": N,
                   "head_dim": D, "topk_ratio": wl.topk_ratio, "topk_blocks": topk,
                   "grid": list(wl.grid), "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None, "kernel": "k_attn_bf16", "launch_ms": by_stage["attend"],
                     "flops_per_launch": exact_f + comp_f},
        "stages_ms_per_layer": by_stage,
    }


def main_sweep(args, ops, synth, torch, np):
    """Density sweep with Reblock layouts and with the fixed-tile baseline."""
    wl = synth.WORKLOADS["mid_bf16"]
    H, N, D = wl.heads, wl.tokens, wl.head_dim
    nb = N // 64
    q, k, v = synth.make_qkv(wl)
    log(f"[bench] sweep on {wl.name}: H={H} N={N} D={D} nb={nb}")
    base = Layer(ops, torch, wl, q, k, v, nb)
    lse_dense = base.dense_lse()
    ident, every = base.dense_inputs()
    base.prepare(pk=ident, flags=ops.BSA_EXACT_ONLY)
    dense_ms, _, _ = time_steps(
        torch, [("dense", lambda: base.attend(pq=ident, pk=ident, ls=every,
                                              flags=ops.BSA_EXACT_ONLY))], 3, 1)
    rows = []
    for ratio in synth.SWEEP_RATIOS:
        topk = ops.topk_count(nb, ratio)
        for fixed, layout, iters, shared, name in (
                (False, "separate", 8, False, "reblock, reweighted summaries"),
                (False, "separate", 2, False, "reblock with 2 power steps per split, "
                                              "reweighted summaries"),
                (False, "separate", 2, True, f"Lite reblock (2 power steps, one direction per "
                                             f"subtree of at most {args.lite_subtree} blocks), "
                                             "reweighted summaries"),
                (False, "q_reuse_k", 8, False, "reblock of the keys reused for the queries, "
                                               "reweighted summaries"),
                (True, "separate", 8, False, "fixed 4x4x4 tiles, mean-pooled summaries")):
            lay = Layer(ops, torch, wl, q, k, v, topk, fixed_tiles=fixed, ws=base.ws,
                        layout=layout, power_iters=iters, lite_tree=shared,
                        subtree_blocks=args.lite_subtree)
            ms_step, stage_ms, _ = time_steps(torch, lay.stages(), args.steps, args.warmup)
            rec = lay.recall(lse_dense)
            row = {"topk_ratio": ratio, "topk_blocks": topk, "layout": name,
                   "layer_ms": ms_step, "stages_ms": stage_ms, "recall": rec,
                   "speedup_vs_dense_attention": dense_ms / ms_step}
            if ratio < 1.0 and (fixed or (layout == "separate" and iters == 8)):
                # log-mass error of the compressed branch: Reweight against mean pooling on
                # the same layouts and lists (the fixed-tile baseline uses mean pooling)
                lm = {m: log_mass_error(torch, ops, lay.qd, lay.kd, lay.vd, lay.perm_q,
                                        lay.perm_k, lay.lists, meanpool=(m == "meanpool"))
                      for m in (("meanpool",) if fixed else ("reweight", "meanpool"))}
                row["log_mass_error"] = lm
                if "reweight" in lm:
                    row["log_mass_error_reweight_vs_meanpool"] = \
                        lm["reweight"] / lm["meanpool"] - 1.0
                log(f"[bench]   log-mass error " +
                    ", ".join(f"{m} {e:.4f}" for m, e in lm.items()))
            rows.append(row)
            tag = "fixed    " if fixed else ("q_reuse_k" if layout == "q_reuse_k" else
                                              "reblock  " if iters == 8 else
                                              "lite     " if shared else "2 steps  ")
            log(f"[bench] ratio {ratio:.1f} {tag}: layer {ms_step:.3f} ms, recall {rec:.4f}")
            del lay
    return {
        "metric": "density sweep at 16,384 tok: layer ms and attention-mass recall vs dense "
                  "softmax, reblock (separate or key layout reused) vs fixed tiles",
        "value": rows[0]["recall"], "unit": "recall at 10% density (reblock)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "heads": H, "tokens": N, "head_dim": D,
                   "grid": list(wl.grid), "ratios": list(synth.SWEEP_RATIOS),
                   "parallelism": "single GPU"},
        "dense_attention_ms": dense_ms,
        "sweep": rows,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="clip10s_bf16")
    ap.add_argument("--sweep", action="store_true",
                    help="density sweep with Reblock and fixed-tile layouts on 16,384 tokens")
    ap.add_argument("--layout", choices=("separate", "q_reuse_k"), default="separate",
                    help="reblock layouts: one tree per side (default), or the key tree "
                         "reused for the queries")
    ap.add_argument("--tail", choices=("token", "block"), default="token",
                    help="compressed branch per query (default) or per query block "
                         "(the block's mean query)")
    ap.add_argument("--ctx", type=int, default=0, metavar="N",
                    help="mixed sequence: N exact context tokens (text, audio, conditioning) "
                         "beside the video grid")
    ap.add_argument("--lite", action="store_true",
                    help="Lite reblock: 2 power steps per split and one direction per subtree "
                         "(of at most --lite-subtree blocks)")
    ap.add_argument("--lite-subtree", type=int, default=64, metavar="S",
                    help="blocks of the Lite tree's shared subtrees (2 .. 64; default 64)")
    ap.add_argument("--recall", action="store_true",
                    help="also measure the attention-mass recall of the run's layouts at "
                         "densities 0.1 / 0.2 / 0.3 against dense softmax")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-machine", action="store_true",
                    help="skip the GEMM and copy ceilings measured beside the headline")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run three device-to-device copies of MIB MiB (a plain copy kernel "
                         "of known traffic, for scaling the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer shards by head with no communication, so "
              "only --gpus 1 is run here", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.calibrate_copy} MiB three times")
        return

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from block_sparse_video_reblock_amd import _lib as ops
    from block_sparse_video_reblock_amd import synth

    if args.sweep:
        res = main_sweep(args, ops, synth, torch, np)
    elif synth.WORKLOADS[args.workload].layers > 1:
        res = main_layers(args, ops, synth, torch, np)
    else:
        res = main_headline(args, ops, synth, torch, np)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
