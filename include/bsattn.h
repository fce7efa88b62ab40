/* bsattn.h -- C ABI of the MI355X (gfx950) Spark-Attn block-sparse attention layer.
 *
 * The layer, as the pages describe it (page titles below), runs in five stages:
 *   (1) reblock:  per-head second moments M_K = E[k k^T] (used to compare queries) and
 *                 M_Q = E[q q^T] (used to compare keys) define a Mahalanobis cosine; a
 *                 capacity-constrained hierarchical tree partition puts queries, and
 *                 separately keys, into leaves of exactly 64 tokens.  Only a permutation is
 *                 produced; the tensors themselves are left as they are.
 *                 [comfy.icu "MiniMax H3 Spark Attention (SM89)", "What it's doing under the
 *                 hood"; comfyui-wiki.com "Spark-H3 ...", "What Spark-Attn changes"]
 *   (2) select:   block scores and a per-query-block top-K at a topk_ratio (or fixed
 *                 topk_blocks) budget.  [comfy.icu page, "Inputs you'll actually set"]
 *   (3) exact branch over the selected key blocks, flash-style.
 *   (4) compressed branch over the unselected blocks: anchor-weighted key/value summaries
 *                 plus a log-mass bias (Spark-Reweight); every query keeps its own Q.
 *                 [comfyui-wiki.com page, "What Spark-Attn changes" and its figure]
 *   (5) log-sum-exp merge of the two branches and the inverse permutation to token order.
 * Options on the same path: the key layout reused for the queries (bsa_reblock_layout), the
 * Lite tree (bsa_reblock_ex: power steps per split, one direction per small subtree), either
 * side's tree alone (bsa_reblock_side), the block-level compressed branch (BSA_TAIL_BLOCK),
 * and exact context tokens beside the video grid (bsa_sparse_attn_ctx).
 *
 * Conventions shared by every call
 *   - Tensors are dense, row-major [heads][tokens][head_dim] device buffers, batch 1.
 *   - Supported (dtype, head_dim): (BSA_BF16, 128) and (BSA_F32, 64).  tokens must be a
 *     positive multiple of 64, at most BSA_MAX_TOKENS.
 *   - A permutation perm[h][p] holds the token id placed at position p.  Query block i is
 *     positions [64 i, 64 i + 64) of perm_q; key block j is positions [64 j, 64 j + 64) of
 *     perm_k; V follows K.  nb = tokens / 64.
 *   - Every pointer is a device pointer owned by the caller; the library allocates nothing and
 *     keeps no state beyond a per-device architecture check.  `ws` is caller-provided
 *     scratch of at least bsa_workspace_bytes(desc) bytes (bsa_workspace_bytes_ctx for the
 *     mixed-sequence calls; contents need not be initialised and are clobbered).
 *   - Calls are asynchronous on `stream`.  The return value reports argument validation and
 *     launch errors; argument checks run on the host before any HIP call.  There is no silent
 *     fallback: an unsupported input is an error (BSA_E_ARG / BSA_E_UNSUPPORTED), never a
 *     different code path.  bsa_last_error() gives a message for the calling thread.
 *   - Results are deterministic: identical inputs give bitwise-identical outputs.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_E_ARG = -1,          /* bad argument: null pointer, shape, budget, flags, scale */
  BSA_E_UNSUPPORTED = -2,  /* (dtype, head_dim) not supported, or the device is not gfx950 */
  BSA_E_WORKSPACE = -3,    /* ws too small */
  BSA_E_HIP = -4           /* a HIP runtime call or kernel launch failed */
} bsa_status;

typedef enum { BSA_F32 = 0, BSA_BF16 = 1 } bsa_dtype;

#define BSA_BLOCK 64
#define BSA_MAX_TOKENS (1 << 19)

typedef struct {
  int32_t heads;     /* >= 1 */
  int32_t tokens;    /* N, multiple of 64 */
  int32_t head_dim;  /* D */
  int32_t dtype;     /* bsa_dtype */
} bsa_desc;

/* sparse_attn flags */
#define BSA_MEANPOOL 1u        /* fixed-block baseline: mean-pooled summaries, bias ln 64 */
#define BSA_EXACT_ONLY 2u      /* debug: output only the exact branch (O_e, lse_e) */
#define BSA_COMPRESSED_ONLY 4u /* debug: output only the compressed branch (O_c, lse_c) */
/* tail_granularity = block (comfy.icu page, "What it's doing under the hood": the node option
 * that switches to ComfyUI's block-level compressed branch).  Every query of query block i uses
 * the block's pooled query, the mean of its 64 queries (in fp32), in place of its own in the
 * compressed branch: logit s qbar_i.kt_j + b_j.  The exact branch and the merge are unchanged.
 * bsa_prepare_kv ignores this flag. */
#define BSA_TAIL_BLOCK 8u
/* strict lists: before the attention kernels, every list is checked on the device (entries in
 * [0, nb), strictly ascending) and the result kept in ws; with a malformed list the attention
 * kernels return before reading any list entry, o and lse_opt are left unwritten, and
 * bsa_list_status reports the first malformed row.  Without this flag the lists are trusted:
 * a malformed list is outside the contract of the call. */
#define BSA_CHECK_LISTS 16u

const char* bsa_status_str(int32_t status);
/* Message describing the last failed call on this thread ("" if none). */
const char* bsa_last_error(void);

/* Blocks selected per query block for a budget ratio (comfy.icu page, "Inputs you'll actually
 * set": topk_ratio).  K = clamp(floor(ratio * nb + 1e-6), 1, nb), computed in double from the
 * float ratio.  Returns -1 if nb < 1 or ratio is not in (0, 1]. */
int32_t bsa_topk_count(int32_t n_blocks, float ratio);

/* Scratch bytes that bsa_reblock, bsa_select, bsa_summaries and bsa_sparse_attn need for this
 * descriptor (one buffer serves all of them).  0 for an invalid descriptor. */
size_t bsa_workspace_bytes(const bsa_desc* desc);

/* (1) Reblock.  perm_q[h][.] (query layout, from M_K) and perm_k[h][.] (key layout, from
 * M_Q), each int32 [heads][tokens].  Leaves are in depth-first (left first) order, tokens in
 * ascending id inside a leaf.  If proj_opt is non-null it receives the fp32 projection every
 * token got at every split level, by token id: float [heads][2][levels][tokens] with side 0 =
 * queries, 1 = keys, levels = ceil(log2 nb) (0 where the token's group was already a leaf). */
bsa_status bsa_reblock(const bsa_desc* desc, const void* q, const void* k,
                       int32_t* perm_q, int32_t* perm_k, float* proj_opt,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* (1a) Reblock with a layout choice.  [comfyui-wiki.com "Spark-H3 ...", "Workflows" ("工作流")]:
 * every shipped workflow pins reblock_layout = q_reuse_k; the pages do not define it, and the
 * reading taken here is its name: the queries reuse the key layout.
 *   BSA_LAYOUT_SEPARATE  exactly bsa_reblock (perm_q and perm_k must be distinct buffers).
 *   BSA_LAYOUT_Q_REUSE_K only the key trees are built (keys under M_Q, as in bsa_reblock, with
 *                        the identical result for perm_k); perm_q receives a copy of perm_k,
 *                        and perm_q may be the same buffer as perm_k.  proj_opt then holds
 *                        the key side only (the query side is left 0).
 * Same workspace, leaf order and errors as bsa_reblock; an unknown layout is BSA_E_ARG. */
typedef enum { BSA_LAYOUT_SEPARATE = 0, BSA_LAYOUT_Q_REUSE_K = 1 } bsa_layout;
bsa_status bsa_reblock_layout(const bsa_desc* desc, const void* q, const void* k, int32_t layout,
                              int32_t* perm_q, int32_t* perm_k, float* proj_opt,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* (1b) Reblock with a layout choice, a power-step count per split and tree flags.
 * bsa_reblock_layout is power_iters = BSA_POWER_ITERS (8), tree_flags = 0.
 * BSA_TREE_SHARED_DEEP: from the first level whose groups hold at most S blocks, each group
 * takes one direction and its descendants keep cutting along the same projections, so the
 * subtree is the group's tokens in (projection, token id) order cut into 64-token leaves (each
 * in ascending token id); proj_opt then repeats those projections at the deeper levels.  S is
 * given as BSA_TREE_SUBTREE_BLOCKS(S) in the same flags, 2 <= S <= BSA_MAX_SUBTREE_BLOCKS;
 * without it S = BSA_DEFAULT_SUBTREE_BLOCKS.
 * Lite: [comfyui-wiki.com "Spark-H3 ...", "Benchmarks" ("基准测试")] names a lighter
 * Spark-H3-Lite that halves the reblock latency for a small fidelity loss at 20 % and 30 %
 * density and does not say how; the reading taken here is the lighter tree
 * BSA_TREE_SHARED_DEEP | BSA_TREE_SUBTREE_BLOCKS(BSA_LITE_SUBTREE_BLOCKS) with
 * BSA_POWER_ITERS_LITE (2) power steps per split, the start vector, capacity cut and leaf
 * order unchanged (S and the step count are this reading's choices, not page values).
 * power_iters outside [1, BSA_MAX_POWER_ITERS], an unknown tree flag, a subtree size outside
 * [2, BSA_MAX_SUBTREE_BLOCKS] or a subtree size without BSA_TREE_SHARED_DEEP is BSA_E_ARG. */
#define BSA_POWER_ITERS 8
#define BSA_POWER_ITERS_LITE 2
#define BSA_MAX_POWER_ITERS 64
#define BSA_TREE_SHARED_DEEP 1u
#define BSA_TREE_SUBTREE_BLOCKS(s) ((uint32_t)(s) << 8)
#define BSA_DEFAULT_SUBTREE_BLOCKS 8
#define BSA_MAX_SUBTREE_BLOCKS 64
#define BSA_LITE_SUBTREE_BLOCKS 64
bsa_status bsa_reblock_ex(const bsa_desc* desc, const void* q, const void* k, int32_t layout,
                          int32_t power_iters, uint32_t tree_flags, int32_t* perm_q,
                          int32_t* perm_k, float* proj_opt, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* (1c) One side of the reblock: side 0 builds the query layouts (queries under M_K) into
 * perm, side 1 the key layouts (keys under M_Q); each equals the corresponding output of
 * bsa_reblock_ex with the same power_iters and tree_flags.  The two sides are independent, so a caller may
 * run them on two streams (each with its own ws) and start bsa_prepare_kv once the key side is
 * done.  proj_opt, if non-null, receives this side's projections in the same
 * [heads][2][levels][tokens] layout (the other side's rows are left 0).  Errors as
 * bsa_reblock_ex; a side other than 0 or 1 is BSA_E_ARG. */
bsa_status bsa_reblock_side(const bsa_desc* desc, const void* q, const void* k, int32_t side,
                            int32_t power_iters, uint32_t tree_flags, int32_t* perm,
                            float* proj_opt, void* ws, size_t ws_bytes, hipStream_t stream);

/* (2) Select.  Block scores S[h][i][j] = s * mean(query block i) . mean(key block j) with
 * s = 1/sqrt(D); per row the K largest (ties to the lower j), written ascending to
 * lists[h][i][0..K).  K = topk_blocks if topk_blocks > 0 (must be <= nb), else
 * bsa_topk_count(nb, topk_ratio).  scores_opt, if non-null, receives S (float [heads][nb][nb]).
 */
bsa_status bsa_select(const bsa_desc* desc, const void* q, const void* k,
                      const int32_t* perm_q, const int32_t* perm_k,
                      float topk_ratio, int32_t topk_blocks,
                      int32_t* lists, float* scores_opt,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* (3)+(4)+(5) Sparse attention.  For query block i of head h and each of its queries q:
 * the exact branch attends over the keys of blocks lists[h][i][0..topk) (each list
 * strictly ascending, entries in [0, nb)); the compressed branch attends over every other
 * block j with logit s q.kt_j + b_j and value vt_j, where (kt, vt, b) are the block summaries of
 * bsa_summaries; the branches merge by log-sum-exp and row p of block i is written to output
 * row perm_q[h][p].  o has the input dtype, [heads][tokens][head_dim]; lse_opt (float
 * [heads][tokens], natural log) receives the merged log-sum-exp of the scaled logits.
 * scale = 0 means 1/sqrt(D).  flags: BSA_MEANPOOL, BSA_TAIL_BLOCK, and at most one of
 * BSA_EXACT_ONLY / BSA_COMPRESSED_ONLY (an empty branch gives lse = -inf and a zero row).  With
 * topk = nb (every block selected) this is dense softmax attention. */
bsa_status bsa_sparse_attn(const bsa_desc* desc, const void* q, const void* k, const void* v,
                           const int32_t* perm_q, const int32_t* perm_k,
                           const int32_t* lists, int32_t topk, uint32_t flags, float scale,
                           void* o, float* lse_opt,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Two-phase form of bsa_sparse_attn, for callers that time the phases separately or reuse the
 * prepared key side.  bsa_prepare_kv computes the anchor and the block summaries (and, for
 * bf16, block-contiguous copies of K and V in the MFMA operand order) into ws;
 * bsa_attend then runs the attention kernel alone.  bsa_attend must receive the same desc, k, v,
 * perm_k, flags (BSA_TAIL_BLOCK aside) and scale as the bsa_prepare_kv call that filled ws, with
 * nothing else written to ws in between; with that, prepare followed by attend equals
 * bsa_sparse_attn.  With BSA_TAIL_BLOCK bsa_attend launches three more kernels (block means,
 * selection bitmaps, the per-block compressed branch) before the attention kernel. */
bsa_status bsa_prepare_kv(const bsa_desc* desc, const void* q, const void* k, const void* v,
                          const int32_t* perm_k, uint32_t flags, float scale,
                          void* ws, size_t ws_bytes, hipStream_t stream);
bsa_status bsa_attend(const bsa_desc* desc, const void* q, const void* k, const void* v,
                      const int32_t* perm_q, const int32_t* perm_k,
                      const int32_t* lists, int32_t topk, uint32_t flags, float scale,
                      void* o, float* lse_opt, void* ws, size_t ws_bytes, hipStream_t stream);

/* (3')+(4)+(5) Mixed sequences: a video grid plus context tokens (text, audio, conditioning).
 * [h3vid.app guide, "Warmup and step counts need explicit definitions"]: the context is handled
 * exactly while only the video grid is sparsified; [comfyui-wiki.com "Spark-H3 ...", "What
 * Spark-Attn changes"]: the Reweight anchor is the mean of the video queries.
 * q, k, v, perm_q, perm_k, lists, topk, o, lse_opt: the video grid exactly as in bsa_sparse_attn
 * (reblock and select it with bsa_reblock / bsa_select on the video tensors alone).
 * q_ctx, k_ctx, v_ctx: [heads][n_ctx][head_dim], desc's dtype, n_ctx >= 0 (any count; 0 = none,
 * then the context pointers may be null and this is bsa_sparse_attn).
 * Each video query attends every context key in its exact branch; each context query attends
 * every key (context and video) densely, output o_ctx [heads][n_ctx][head_dim] and
 * lse_ctx_opt [heads][n_ctx].  Flags as in bsa_sparse_attn; the context keys belong to the
 * exact branch (BSA_COMPRESSED_ONLY drops them and leaves the context rows zero with
 * lse -inf).  ws must hold bsa_workspace_bytes_ctx(desc, n_ctx) bytes. */
size_t bsa_workspace_bytes_ctx(const bsa_desc* desc, int32_t n_ctx);
bsa_status bsa_sparse_attn_ctx(const bsa_desc* desc, int32_t n_ctx, const void* q, const void* k,
                               const void* v, const void* q_ctx, const void* k_ctx,
                               const void* v_ctx, const int32_t* perm_q, const int32_t* perm_k,
                               const int32_t* lists, int32_t topk, uint32_t flags, float scale,
                               void* o, void* o_ctx, float* lse_opt, float* lse_ctx_opt,
                               void* ws, size_t ws_bytes, hipStream_t stream);
/* Two-phase form of bsa_sparse_attn_ctx, with the same contract as bsa_prepare_kv /
 * bsa_attend: the prepare phase also lays out the context keys and values (k_ctx, v_ctx) in
 * ws, and bsa_attend_ctx must receive the same desc, n_ctx, k, v, k_ctx, v_ctx, perm_k, flags
 * (BSA_TAIL_BLOCK aside) and scale, with nothing else written to ws in between. */
bsa_status bsa_prepare_kv_ctx(const bsa_desc* desc, int32_t n_ctx, const void* q, const void* k,
                              const void* v, const void* k_ctx, const void* v_ctx,
                              const int32_t* perm_k, uint32_t flags, float scale, void* ws,
                              size_t ws_bytes, hipStream_t stream);
bsa_status bsa_attend_ctx(const bsa_desc* desc, int32_t n_ctx, const void* q, const void* k,
                          const void* v, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                          const int32_t* perm_q, const int32_t* perm_k, const int32_t* lists,
                          int32_t topk, uint32_t flags, float scale, void* o, void* o_ctx,
                          float* lse_opt, float* lse_ctx_opt, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* (4) Block summaries alone (the compressed branch's keys, values and biases), fp32:
 * kt[h][j][D], vt[h][j][D], bias[h][j].  Reweight (default): anchor qa = mean of the head's
 * queries, x_t = s qa.k_t over block j's keys, w = softmax(x), kt = sum w_t k_t,
 * vt = sum w_t v_t, b = logsumexp(x) - s qa.kt.  BSA_MEANPOOL: plain means and b = ln 64. */
bsa_status bsa_summaries(const bsa_desc* desc, const void* q, const void* k, const void* v,
                         const int32_t* perm_k, uint32_t flags, float scale,
                         float* kt, float* vt, float* bias,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture that must not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation): bsa_summaries without a
 * workspace argument.  Its scratch (the anchor's partial column sums) is a device-resident
 * array inside the library, BSA_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first call
 * on a device until the process ends; the call allocates nothing.  Arguments, outputs and
 * results are those of bsa_summaries (bit-identical: the same kernels).
 * Limits: the descriptor must need at most BSA_NOALLOC_SCRATCH_BYTES bytes of scratch
 * (bsa_summaries_noalloc_bytes; 24 heads of up to 524,288 tokens at head_dim 128 fit), else
 * BSA_E_ARG before any HIP call.  All calls on one GPU share its one array: calls that
 * overlap in time on one GPU (two streams, two threads) race and must be serialised by the
 * caller; consecutive calls on one stream are safe. */
#define BSA_NOALLOC_SCRATCH_BYTES (16u << 20)
size_t bsa_summaries_noalloc_bytes(const bsa_desc* desc);
bsa_status bsa_summaries_noalloc(const bsa_desc* desc, const void* q, const void* k,
                                 const void* v, const int32_t* perm_k, uint32_t flags,
                                 float scale, float* kt, float* vt, float* bias,
                                 hipStream_t stream);

/* Fixed-tile layout: the positional baseline that (1) replaces.  [comfyui-wiki.com
 * "Spark-H3 ...", "What Spark-Attn changes": Reblock takes the place of fixed spatiotemporal
 * tiles; comfy.icu page, "What it's doing under the hood": recall against fixed blocks]
 * The latent grid (grid_t, grid_h, grid_w), token id (t grid_h + y) grid_w + x, is cut into
 * tile_t x tile_h x tile_w cubes of 64 tokens: position p holds cube p / 64 (cubes in raster
 * order of their corner), token p % 64 of it (raster order inside the cube).
 * perm: int32 [heads][grid_t grid_h grid_w], the same layout for every head; use it as both
 * perm_q and perm_k.  BSA_E_ARG unless tile_t tile_h tile_w = 64, each tile side divides its
 * grid side and the grid holds at most BSA_MAX_TOKENS tokens. */
bsa_status bsa_tile_layout(int32_t heads, int32_t grid_t, int32_t grid_h, int32_t grid_w,
                           int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t* perm,
                           hipStream_t stream);

/* Parity hook for (1): the tree partition with every level's projections supplied.
 * proj: float [problems][levels][tokens] by token id (levels = ceil(log2(tokens/64)));
 * perm: int32 [problems][tokens].  Each split sends the floor(m/2)*64 tokens of smallest
 * (projection, token id) of an m-block group to the left child; -0.0 equals +0.0; NaN is
 * an error of the caller (the order of NaN projections is unspecified).  Needs
 * bsa_partition_workspace_bytes(problems, tokens) bytes of ws. */
size_t bsa_partition_workspace_bytes(int32_t problems, int32_t tokens);
bsa_status bsa_reblock_from_projections(int32_t problems, int32_t tokens, const float* proj,
                                        int32_t* perm, void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/* Strict check of block lists (the lists argument of bsa_sparse_attn and the calls like it):
 * lists int32 [rows][topk] on the device, read only.  result (device, 2 int32) receives the
 * number of rows whose list has an entry outside [0, n_blocks) or an entry not above its
 * predecessor, and the smallest such row (-1 if none).  Asynchronous on stream; BSA_E_ARG for
 * rows or n_blocks < 1, topk outside [1, n_blocks], or a null pointer. */
bsa_status bsa_check_lists(int32_t rows, int32_t n_blocks, int32_t topk, const int32_t* lists,
                           int32_t* result, hipStream_t stream);
/* The result of the list check of the last attention call on this ws that was given
 * BSA_CHECK_LISTS (the same two values as bsa_check_lists), copied to the host array result[2].
 * Synchronous: waits for stream.  The value is undefined if no such call wrote ws. */
bsa_status bsa_list_status(const void* ws, size_t ws_bytes, int32_t* result,
                           hipStream_t stream);

/* Parity hook for (2): top-K of given scores.  scores: float [rows][n_blocks];
 * lists: int32 [rows][topk], each ascending; ties go to the lower block index; -0.0 equals
 * +0.0. */
bsa_status bsa_topk_from_scores(int32_t rows, int32_t n_blocks, int32_t topk,
                                const float* scores, int32_t* lists, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BSATTN_H */
