// Host-side launchers of the gfx950 kernels.  Shapes are validated by the C-ABI layer before
// any of these is called; each launcher only enqueues kernels on `stream` and returns the
// launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsa {

constexpr int kBlk = 64;
constexpr int kColChunk = 512;     // tokens per partial of the anchor / column-sum reduction

__host__ __device__ inline int ceil_div(long a, long b) { return int((a + b - 1) / b); }
__host__ __device__ inline int summary_tiles(int nb) { return ceil_div(nb, 64); }

// ---------------------------------------------------------------- summaries (stage 4)
// anchor[h][d] = mean over tokens of x[h][.][d]; partial: float [H][ceil(N/kColChunk)][D]
hipError_t launch_anchor(bool bf16, const void* x, int H, int N, int D, float* partial,
                         float* anchor, hipStream_t s);
// per key block j: fp32 summaries kt/vt [H][nb][D], bias [H][ldb]; optionally (bf16 only)
// the block-swizzled copies of K and V used by the attention kernel.
hipError_t launch_summaries(bool bf16, const void* k, const void* v, const int32_t* perm_k,
                            const float* anchor, int H, int N, int D, float scale, bool meanpool,
                            float* kt, float* vt, float* bias, int ldb, void* ksw, void* vsw,
                            hipStream_t s);
// swizzled bf16 summary tiles for the attention kernel; pads bias rows >= nb with -inf
hipError_t launch_summary_tiles(const float* kt, const float* vt, float* bias, int H, int nb,
                                void* ktsw, void* vtsw, hipStream_t s);
// swizzled bf16 context tiles [H][ceil(n_ctx/64)][1024] from bf16 k_ctx, v_ctx [H][n_ctx][128];
// rows past n_ctx are zero
hipError_t launch_ctx_tiles(const void* k_ctx, const void* v_ctx, int H, int n_ctx, void* ctsw,
                            void* cvsw, hipStream_t s);

// ------------------------------------------------------------ attention (stages 3, 4, 5)
struct AttnLaunch {
  // video queries: exact tiles n_exact (= topk or 0), biased tiles tau0 .. tau0 + n_comp - 1
  // (summary tiles 0 .. tiles - 1, then context tiles)
  int H, N, nb, topk, n_exact, n_comp, tau0;
  float scale;
  const void* q;
  const int32_t* perm_q;
  const int32_t* lists;
  const float* bias;                        // [H][tiles*64], -inf on pads
  void* o;
  float* lse;
  // bf16 path: swizzled tiles
  const void *ksw, *vsw, *ktsw, *vtsw;
  // f32 path: plain tensors and fp32 summaries
  const void *k, *v;
  const int32_t* perm_k;
  const float *kt, *vt;
  // block-level compressed branch (null: per-query).  bf16: the compressed state of every query
  // block, tail_o [H][nb][D] (normalised) and tail_lse [H][nb] (log2 units), merged in place of
  // the summary tiles; f32: the pooled queries qbar [H][nb][D], used for the summary tiles in
  // place of each query's own.
  const float *tail_o, *tail_lse, *qbar;
  // context tokens (n_ctx = 0: none): [H][n_ctx][D] each; context queries attend ctx_n_exact
  // video blocks (nb or 0) and ctx_n_comp context tiles (all or 0)
  int n_ctx, ctx_n_exact, ctx_n_comp;
  const void *q_ctx, *k_ctx, *v_ctx;
  const void *ctsw, *cvsw;                  // bf16 path: swizzled context tiles
  void* o_ctx;
  float* lse_ctx;
  // result of a list check run before the launch (see launch_check_lists), or null: with a
  // malformed list the attention kernels return at once, before any list entry is read
  const int32_t* list_status;
  // the lists in exact-tile walk order (launch_list_walk), or null to walk `lists` as given
  const int32_t* walk;
};
hipError_t launch_attn_bf16(const AttnLaunch& a, hipStream_t s);
// walk[h][i][.] = lists[h][i][.] ordered by (selection count of the key block among the head's
// lists, highest first; index); pop [H][nb] is scratch.  Only where list_walk_applies.
hipError_t launch_list_walk(const int32_t* lists, int H, int nb, int topk, int32_t* pop,
                            int32_t* walk, hipStream_t s);
bool list_walk_applies(int nb, int topk);
hipError_t launch_attn_f32(const AttnLaunch& a, hipStream_t s);
// Block-level compressed branch (bf16): from the pooled queries qbar [H][nb][D] (fp32), the
// lists and the summary tiles of the launch `a` (n_comp ignored), the per-block state
// tail_o / tail_lse; bits [H][nb][2 * tiles] is scratch for the selection bitmaps.
hipError_t launch_tail_block_bf16(const AttnLaunch& a, const float* qbar, uint32_t* bits,
                                  float* tail_o, float* tail_lse, hipStream_t s);

// ------------------------------------------------------------------- select (stage 2)
hipError_t launch_block_means(bool bf16, const void* x, const int32_t* perm, int H, int N, int D,
                              float* means, hipStream_t s);
hipError_t launch_block_scores(const float* qm, const float* km, int H, int nb, int D,
                               float scale, float* scores, hipStream_t s);
hipError_t launch_tile_layout(int heads, int T, int H, int W, int tt, int th, int tw,
                              int32_t* perm, hipStream_t s);
hipError_t launch_topk(const float* scores, int rows, int nb, int k, int32_t* lists,
                       hipStream_t s);
// result (device, 2 ints): malformed rows of lists [rows][k] (entries outside [0, nb) or not
// strictly ascending) and the smallest such row (-1 if none)
hipError_t launch_check_lists(const int32_t* lists, int rows, int nb, int k, int32_t* result,
                              hipStream_t s);

// ------------------------------------------------------------- allocation-free scratch
// Size of the device-resident scratch array behind bsa_summaries_noalloc (one per device).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
// The calling thread's current device's copy of that array (its address looked up once per
// device with hipGetSymbolAddress).
hipError_t noalloc_scratch(void** out);

// ------------------------------------------------------------------ reblock (stage 1)
size_t reblock_ws_bytes(int H, int N, int D);
// sides: which trees to build (queries under M_K into perm_q, keys under M_Q into perm_k);
// copy_q: perm_q becomes a copy of perm_k afterwards; iters: power steps per split;
// shared_blocks: 0 for the full tree, else the Lite tree with one direction per subtree from
// the first level whose groups hold at most that many blocks (2 .. 64)
constexpr int kSideQueries = 1, kSideKeys = 2, kSideBoth = 3;
hipError_t launch_reblock(bool bf16, const void* q, const void* k, int H, int N, int D,
                          int32_t* perm_q, int32_t* perm_k, float* proj_opt, int sides,
                          bool copy_q, int iters, int shared_blocks, void* ws, hipStream_t s);
size_t partition_ws_bytes(int P, int N);
hipError_t launch_partition_from_proj(int P, int N, const float* proj, int32_t* perm, void* ws,
                                      hipStream_t s);

}  // namespace bsa
