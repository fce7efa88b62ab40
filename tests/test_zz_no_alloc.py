"""GPU check of the allocation-free summaries call (bsa_summaries_noalloc, the library's static
device scratch) against bsa_summaries with a caller workspace: bit-identical outputs, on two
calls in a row, the second with a smaller input, for both summary modes."""
import numpy as np
import pytest
import torch

from block_sparse_video_reblock_amd import _lib as ops
from block_sparse_video_reblock_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(name, heads):
    wl = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(wl, heads=heads)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(DEV).to(dt) for x in (q, k, v))
    rng = np.random.default_rng(17)
    perm = np.stack([rng.permutation(wl.tokens) for _ in heads]).astype(np.int32)
    return qd, kd, vd, torch.from_numpy(perm).to(DEV)


@pytest.mark.parametrize("flags", [0, ops.BSA_MEANPOOL])
def test_summaries_noalloc_matches_workspace_call(flags):
    big = _inputs("clip10s_bf16", range(3))          # 3 heads x 72,576 tokens
    small = _inputs("mid_bf16", [0, 5])              # 2 heads x 16,384 tokens
    for case, (qd, kd, vd, pk) in (("big", big), ("small", small)):
        print(f"noalloc {case}: heads {qd.shape[0]} tokens {qd.shape[1]} flags {flags}",
              flush=True)
        ref = ops.summaries(qd, kd, vd, pk, flags=flags)
        got = ops.summaries_noalloc(qd, kd, vd, pk, flags=flags)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.isfinite(g).all().item()
            assert torch.equal(r, g), case
