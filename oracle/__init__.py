"""CPU oracle for the Spark-Attn block-sparse attention layer.  TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, fp64 numpy statement of what the layer computes.  It exists to
check the HIP path; it is not part of it.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  It imports nothing from the HIP package and shares no code
with it.

Sources (cited by page title and section):
  [P1] comfyui-wiki.com news "Spark-H3: block-sparse attention speeds up MiniMax-H3 in
       ComfyUI", section "What Spark-Attn changes" (two-branch split; Reblock; Reweight) and
       the figure on exp(E[x]) vs E[exp(x)].
  [P2] comfy.icu node page "MiniMax H3 Spark Attention (SM89)", section "What it's doing under
       the hood" (M_K = E[k k^T] for queries, M_Q for keys; leaves of 64 tokens; the output of
       the reblock is a permutation only; each query keeps its own vector in the compressed
       branch) and section
       "Inputs you'll actually set" (topk_ratio / topk_blocks budgets).
  [P3] h3vid.app guide, section "Warmup and step counts need explicit definitions" (exact
       handling of text, audio and conditioning context while the video grid is sparsified).
Where the pages leave a step open the oracle takes one plain reading; each is listed in the
functions' docstrings.  Parity-unpinned readings (fixed only by this reading, no page value):
the power-iteration count T = 8 and its start vector, the budget rounding, the block-score
formula.
"""
from .spark import *  # noqa: F401,F403
