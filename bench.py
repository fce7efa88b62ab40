#!/usr/bin/env python3
"""Benchmark of the Spark-Attn block-sparse attention layer on one MI355X.

One step is the whole layer on one batch of synthetic video-shaped Q/K/V already resident in
HBM: reblock (both layouts of every head), block scoring + top-K, summaries, and the two-branch
attention with merge and inverse permutation.  Timed with HIP events on the stream the library
launches on.  Prints one JSON line (the last line of stdout).

  value      dense-equivalent effective TFLOP/s = 4 N^2 D H / layer time
  roofline   the attention kernel (the dominant one): algorithmic flops of the exact and
             compressed branches per launch / its mean launch time, against the bf16 MFMA peak
  dense      the same attention kernel with every block selected and identity layouts (dense
             softmax attention), timed on the same GPU
  cpu_baseline  the CPU oracle (fp64 numpy) on one head of the same workload, extrapolated to
             all heads
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "sparse attn layer ms + effective TFLOP/s at 72,576 tok, 10% density, vs dense"
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(H, N, D, topk):
    nb = N // 64
    exact = 4.0 * N * (topk * 64) * D * H
    compressed = 4.0 * N * (nb - topk) * D * H
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="clip10s_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    wl = synth.WORKLOADS[args.workload]
    H, N, D = wl.heads, wl.tokens, wl.head_dim
    nb = N // 64
    topk = ops.topk_count(nb, wl.topk_ratio)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    log(f"[bench] workload {wl.name}: H={H} N={N} D={D} nb={nb} topk={topk} dtype={wl.dtype}")

    t0 = time.perf_counter()
    q, k, v = synth.make_qkv(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(dev).to(dt) for x in (q, k, v))
    d = ops.desc_for(qd)
    ws = ops.workspace(d, dev)
    perm_q = torch.empty(H, N, dtype=torch.int32, device=dev)
    perm_k = torch.empty_like(perm_q)
    lists = torch.empty(H, nb, topk, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    L = ops.lib()
    stream = ops._stream()
    import ctypes

    def p(t):
        return ctypes.c_void_p(t.data_ptr())

    def reblock():
        ops.check(L.bsa_reblock(ctypes.byref(d), p(qd), p(kd), p(perm_q), p(perm_k), None, p(ws),
                                ws.numel(), stream))

    def select():
        ops.check(L.bsa_select(ctypes.byref(d), p(qd), p(kd), p(perm_q), p(perm_k),
                               float(wl.topk_ratio), 0, p(lists), None, p(ws), ws.numel(),
                               stream))

    def prepare(pk=None, flags=0):
        ops.check(L.bsa_prepare_kv(ctypes.byref(d), p(qd), p(kd), p(vd),
                                   p(perm_k if pk is None else pk), flags, 0.0, p(ws), ws.numel(),
                                   stream))

    def attend(pq=None, pk=None, ls=None, flags=0):
        ls = lists if ls is None else ls
        ops.check(L.bsa_attend(ctypes.byref(d), p(qd), p(kd), p(vd),
                               p(perm_q if pq is None else pq), p(perm_k if pk is None else pk),
                               p(ls), int(ls.shape[-1]), flags, 0.0, p(out), None, p(ws),
                               ws.numel(), stream))

    stages = ("reblock", "select", "prepare", "attend")
    fns = (reblock, select, prepare, attend)
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur)
    for s in range(args.steps):
        ev[s][0].record(cur)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(cur)
    stop.record(cur)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    stage_ms = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1])
                                     for s in range(args.steps)]))
                for i, name in enumerate(stages)}
    attn_ms_all = [ev[s][3].elapsed_time(ev[s][4]) for s in range(args.steps)]
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    log(f"[bench] layer {ms_step:.3f} ms/step; stages " +
        ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))

    exact_f, comp_f = attention_flops(H, N, D, topk)
    attn_ms = float(np.mean(attn_ms_all))
    achieved = (exact_f + comp_f) / (attn_ms * 1e-3) / 1e12
    dense_flops = 4.0 * N * N * D * H
    eff = dense_flops / (ms_step * 1e-3) / 1e12

    # HBM-bound stages: algorithmic bytes (inputs read once per pass the algorithm needs)
    elt = 2 if wl.dtype == "bf16" else 4
    x_bytes = H * N * D * elt
    levels = max(0, (nb - 1).bit_length())
    hbm = {
        "reblock": {"bytes": (2 + 2 * levels) * 2 * x_bytes,
                    "passes": "moments, norms, and per tree level a statistics and a "
                              "projection pass over Q and K"},
        "select": {"bytes": 2 * x_bytes + H * nb * nb * 4, "passes": "Q, K once; scores"},
        "prepare": {"bytes": 3 * x_bytes, "passes": "Q (anchor), K, V once"},
    }
    for name, h in hbm.items():
        gbs = h["bytes"] / (stage_ms[name] * 1e-3) / 1e9
        h.update({"ms": stage_ms[name], "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS})

    dense = None
    if not args.no_dense:
        ident = torch.arange(N, dtype=torch.int32, device=dev).repeat(H, 1).contiguous()
        all_lists = torch.arange(nb, dtype=torch.int32, device=dev).repeat(H, nb, 1).contiguous()
        prepare(pk=ident)
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            attend(pq=ident, pk=ident, ls=all_lists, flags=ops.BSA_EXACT_ONLY)
            e1.record(cur)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        dense_ms = float(min(times[1:]))
        dense = {"ms": dense_ms, "tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
                 "speedup_of_sparse_layer": dense_ms / ms_step,
                 "kernel": "same attention kernel, every block selected, identity layouts"}
        log(f"[bench] dense attention {dense_ms:.2f} ms ({dense['tflops']:.0f} TFLOP/s); "
            f"sparse layer speed-up {dense_ms / ms_step:.2f}x")
        del all_lists

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on head 0 ...")
        t_head, threads = cpu_baseline(wl, q, k, v)
        layer_s = t_head * H
        cpu = {"value": dense_flops / layer_s / 1e12, "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "ms_per_layer": layer_s * 1e3,
               "sample": f"fp64 numpy oracle, full layer (reblock both sides, scores, top-K, "
                         f"summaries, exact + compressed attention) on head 0 of {H}: "
                         f"{t_head:.1f} s, extrapolated x{H}"}
        log(f"[bench] oracle head 0: {t_head:.1f} s -> {layer_s * 1e3:.0f} ms per layer")

    res = {
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
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None, "kernel": "k_attn_bf16", "launch_ms": attn_ms,
                     "flops_per_launch": exact_f + comp_f},
        "stages_ms": stage_ms,
        "hbm": hbm,
        "dense": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
