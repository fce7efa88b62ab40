// C ABI of the Spark-Attn layer: argument validation (on the host, before any HIP call),
// workspace carving and launch sequencing.  The operations themselves are documented in
// include/bsattn.h; every step runs in the HIP kernels of this directory.
#include "bsattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.h"
#include "tree.h"

static_assert(bsa::kNoallocScratchBytes == BSA_NOALLOC_SCRATCH_BYTES,
              "the header and the library disagree on the static scratch size");

namespace {

thread_local char g_err[320] = "";

bsa_status fail(bsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bsa_status ok() {
  g_err[0] = '\0';
  return BSA_OK;
}

bsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Architecture check, cached per device.  BSATTN_ARCH_OVERRIDE replaces the queried name (used
// by the host tests to exercise the rejection path without a GPU).
bsa_status check_device() {
  const char* ovr = std::getenv("BSATTN_ARCH_OVERRIDE");
  if (ovr != nullptr) {
    if (std::strncmp(ovr, "gfx950", 6) != 0)
      return fail(BSA_E_UNSUPPORTED, "device architecture %s is not gfx950", ovr);
    return ok();
  }
  static std::atomic<int> cache[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(BSA_E_UNSUPPORTED, "device index %d out of range", dev);
  int c = cache[dev].load();
  if (c == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    c = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    cache[dev].store(c);
  }
  if (c != 1) return fail(BSA_E_UNSUPPORTED, "device %d is not gfx950", dev);
  return ok();
}

bool is_bf16(const bsa_desc* d) { return d->dtype == BSA_BF16; }

bsa_status check_desc(const bsa_desc* d) {
  if (d == nullptr) return fail(BSA_E_ARG, "desc is null");
  if (d->heads < 1) return fail(BSA_E_ARG, "heads = %d must be >= 1", d->heads);
  if (d->tokens < BSA_BLOCK || d->tokens % BSA_BLOCK != 0)
    return fail(BSA_E_ARG, "tokens = %d must be a positive multiple of 64", d->tokens);
  if (d->tokens > BSA_MAX_TOKENS)
    return fail(BSA_E_ARG, "tokens = %d exceeds %d", d->tokens, BSA_MAX_TOKENS);
  if (d->dtype != BSA_F32 && d->dtype != BSA_BF16)
    return fail(BSA_E_UNSUPPORTED, "dtype %d is not supported", d->dtype);
  if (!((d->dtype == BSA_BF16 && d->head_dim == 128) || (d->dtype == BSA_F32 && d->head_dim == 64)))
    return fail(BSA_E_UNSUPPORTED, "(dtype %s, head_dim %d) is not supported; use (bf16, 128) "
                "or (f32, 64)", d->dtype == BSA_BF16 ? "bf16" : "f32", d->head_dim);
  if ((int64_t)d->heads * d->tokens > (int64_t)1 << 30)
    return fail(BSA_E_ARG, "heads * tokens = %lld is too large",
                (long long)d->heads * d->tokens);
  return ok();
}

float resolve_scale(const bsa_desc* d, float scale) {
  return scale == 0.f ? 1.f / std::sqrt(float(d->head_dim)) : scale;
}

// ----------------------------------------------------------------- workspace layouts
struct AttnWs {
  size_t status, anchor_partial, anchor, kt, vt, bias, ktsw, vtsw, ksw, vsw, qbar, tbits, tail_o,
      tail_lse, ctsw, cvsw, pop, walk, total;
};

AttnWs attn_layout(const bsa_desc* d, int n_ctx = 0) {
  const size_t H = d->heads, N = d->tokens, D = d->head_dim, nb = N / 64;
  const size_t nt = bsa::summary_tiles(int(nb));
  AttnWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  // first, at the same offset for every descriptor: the result of the last list check
  w.status = take(2 * sizeof(int32_t));
  w.anchor_partial = take(H * bsa::ceil_div(long(N), bsa::kColChunk) * D * 4);
  w.anchor = take(H * D * 4);
  w.kt = take(H * nb * D * 4);
  w.vt = take(H * nb * D * 4);
  w.bias = take(H * nt * 64 * 4);
  if (is_bf16(d)) {
    w.ktsw = take(H * nt * 64 * D * 2);
    w.vtsw = take(H * nt * 64 * D * 2);
    w.ksw = take(H * N * D * 2);
    w.vsw = take(H * N * D * 2);
  }
  // block-level compressed branch: pooled queries; for bf16 also the selection bitmaps and
  // the per-block compressed state
  w.qbar = take(H * nb * D * 4);
  if (is_bf16(d)) {
    w.tbits = take(H * nb * 2 * nt * 4);
    w.tail_o = take(H * nb * D * 4);
    w.tail_lse = take(H * nb * 4);
  }
  // context tokens (bf16 path): swizzled 64-row tiles of their keys and values
  if (is_bf16(d) && n_ctx > 0) {
    const size_t nc = bsa::ceil_div(n_ctx, 64);
    w.ctsw = take(H * nc * 64 * D * 2);
    w.cvsw = take(H * nc * 64 * D * 2);
  }
  // bf16 path: the exact-tile walk order of sparse lists (selection counts and reordered
  // lists, for the longest list that gets one)
  if (is_bf16(d)) {
    w.pop = take(H * nb * 4);
    w.walk = take(H * nb * std::min<size_t>(nb, 256) * 4);
  }
  w.total = off;
  return w;
}

// context tokens of a mixed sequence (n = 0: none)
struct Ctx {
  int n;
  const void *q, *k, *v;
  void* o;
  float* lse;
};

struct SelWs {
  size_t qm, km, scores, total;
};

SelWs select_layout(const bsa_desc* d) {
  const size_t H = d->heads, N = d->tokens, D = d->head_dim, nb = N / 64;
  SelWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  w.qm = take(H * nb * D * 4);
  w.km = take(H * nb * D * 4);
  w.scores = take(H * nb * nb * 4);
  w.total = off;
  return w;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// The Lite tree's subtree size from the reblock tree flags: 0 for the full tree.
bsa_status tree_shared_blocks(uint32_t flags, int* blocks) {
  *blocks = 0;
  if (flags & ~uint32_t(BSA_TREE_SHARED_DEEP | BSA_TREE_SUBTREE_BLOCKS(0xFF)))
    return fail(BSA_E_ARG, "unknown tree flags 0x%x", flags);
  const int b = int((flags >> 8) & 0xFF);
  if (!(flags & BSA_TREE_SHARED_DEEP)) {
    if (b != 0) return fail(BSA_E_ARG, "a subtree size needs BSA_TREE_SHARED_DEEP");
    return ok();
  }
  if (b != 0 && (b < 2 || b > BSA_MAX_SUBTREE_BLOCKS))
    return fail(BSA_E_ARG, "subtree size %d is not in [2, %d]", b, BSA_MAX_SUBTREE_BLOCKS);
  *blocks = b == 0 ? BSA_DEFAULT_SUBTREE_BLOCKS : b;
  return ok();
}

bsa_status check_ws(const void* ws, size_t have, size_t need) {
  if (have < need)
    return fail(BSA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", have,
                need);
  if (need > 0 && ws == nullptr) return fail(BSA_E_ARG, "workspace pointer is null");
  return ok();
}

// anchor + summaries into the attention workspace (shared by bsa_summaries / bsa_sparse_attn)
hipError_t run_summaries(const bsa_desc* d, const AttnWs& L, void* ws, const void* q,
                         const void* k, const void* v, const int32_t* perm_k, bool meanpool,
                         float scale, float* kt, float* vt, float* bias, int ldb, bool swizzle,
                         hipStream_t s) {
  const bool bf = is_bf16(d);
  float* anchor = reinterpret_cast<float*>(at(ws, L.anchor));
  hipError_t e = hipSuccess;
  if (!meanpool) {
    e = bsa::launch_anchor(bf, q, d->heads, d->tokens, d->head_dim,
                           reinterpret_cast<float*>(at(ws, L.anchor_partial)), anchor, s);
    if (e != hipSuccess) return e;
  }
  return bsa::launch_summaries(bf, k, v, perm_k, anchor, d->heads, d->tokens, d->head_dim, scale,
                               meanpool, kt, vt, bias, ldb, swizzle ? at(ws, L.ksw) : nullptr,
                               swizzle ? at(ws, L.vsw) : nullptr, s);
}

}  // namespace

extern "C" {

const char* bsa_status_str(int32_t st) {
  switch (st) {
    case BSA_OK: return "ok";
    case BSA_E_ARG: return "invalid argument";
    case BSA_E_UNSUPPORTED: return "unsupported";
    case BSA_E_WORKSPACE: return "workspace too small";
    case BSA_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* bsa_last_error(void) { return g_err; }

int32_t bsa_topk_count(int32_t n_blocks, float ratio) {
  if (n_blocks < 1 || !(ratio > 0.f && ratio <= 1.f)) return -1;
  long k = (long)std::floor(double(ratio) * double(n_blocks) + 1e-6);
  if (k < 1) k = 1;
  if (k > n_blocks) k = n_blocks;
  return int32_t(k);
}

size_t bsa_workspace_bytes(const bsa_desc* d) {
  if (check_desc(d) != BSA_OK) return 0;
  size_t a = attn_layout(d).total, s = select_layout(d).total;
  size_t r = bsa::reblock_ws_bytes(d->heads, d->tokens, d->head_dim);
  size_t m = a > s ? a : s;
  return m > r ? m : r;
}

bsa_status bsa_reblock_layout(const bsa_desc* d, const void* q, const void* k, int32_t layout,
                              int32_t* perm_q, int32_t* perm_k, float* proj_opt, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  return bsa_reblock_ex(d, q, k, layout, BSA_POWER_ITERS, 0, perm_q, perm_k, proj_opt, ws,
                        ws_bytes, stream);
}

bsa_status bsa_reblock_ex(const bsa_desc* d, const void* q, const void* k, int32_t layout,
                          int32_t power_iters, uint32_t tree_flags, int32_t* perm_q,
                          int32_t* perm_k, float* proj_opt, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  bsa_status st = check_desc(d);
  if (st != BSA_OK) return st;
  if (layout != BSA_LAYOUT_SEPARATE && layout != BSA_LAYOUT_Q_REUSE_K)
    return fail(BSA_E_ARG, "unknown layout %d", (int)layout);
  if (power_iters < 1 || power_iters > BSA_MAX_POWER_ITERS)
    return fail(BSA_E_ARG, "power_iters = %d is not in [1, %d]", (int)power_iters,
                BSA_MAX_POWER_ITERS);
  int shared_blocks = 0;
  st = tree_shared_blocks(tree_flags, &shared_blocks);
  if (st != BSA_OK) return st;
  if (!q || !k || !perm_q || !perm_k) return fail(BSA_E_ARG, "null tensor pointer");
  if (layout == BSA_LAYOUT_SEPARATE && perm_q == perm_k)
    return fail(BSA_E_ARG, "separate layouts need two permutation buffers");
  st = check_ws(ws, ws_bytes, bsa::reblock_ws_bytes(d->heads, d->tokens, d->head_dim));
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(bsa::launch_reblock(is_bf16(d), q, k, d->heads, d->tokens, d->head_dim,
                                        perm_q, perm_k, proj_opt,
                                        layout == BSA_LAYOUT_Q_REUSE_K ? bsa::kSideKeys
                                                                       : bsa::kSideBoth,
                                        layout == BSA_LAYOUT_Q_REUSE_K, power_iters,
                                        shared_blocks, ws, stream),
                    "reblock launch");
}

bsa_status bsa_reblock_side(const bsa_desc* d, const void* q, const void* k, int32_t side,
                            int32_t power_iters, uint32_t tree_flags, int32_t* perm,
                            float* proj_opt, void* ws, size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_desc(d);
  if (st != BSA_OK) return st;
  if (side != 0 && side != 1) return fail(BSA_E_ARG, "side = %d is not 0 or 1", (int)side);
  if (power_iters < 1 || power_iters > BSA_MAX_POWER_ITERS)
    return fail(BSA_E_ARG, "power_iters = %d is not in [1, %d]", (int)power_iters,
                BSA_MAX_POWER_ITERS);
  int shared_blocks = 0;
  st = tree_shared_blocks(tree_flags, &shared_blocks);
  if (st != BSA_OK) return st;
  if (!q || !k || !perm) return fail(BSA_E_ARG, "null tensor pointer");
  st = check_ws(ws, ws_bytes, bsa::reblock_ws_bytes(d->heads, d->tokens, d->head_dim));
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(bsa::launch_reblock(is_bf16(d), q, k, d->heads, d->tokens, d->head_dim,
                                        perm, perm, proj_opt,
                                        side ? bsa::kSideKeys : bsa::kSideQueries, false,
                                        power_iters, shared_blocks, ws, stream),
                    "reblock launch");
}

bsa_status bsa_reblock(const bsa_desc* d, const void* q, const void* k, int32_t* perm_q,
                       int32_t* perm_k, float* proj_opt, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return bsa_reblock_layout(d, q, k, BSA_LAYOUT_SEPARATE, perm_q, perm_k, proj_opt, ws,
                            ws_bytes, stream);
}

bsa_status bsa_select(const bsa_desc* d, const void* q, const void* k, const int32_t* perm_q,
                      const int32_t* perm_k, float topk_ratio, int32_t topk_blocks,
                      int32_t* lists, float* scores_opt, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  bsa_status st = check_desc(d);
  if (st != BSA_OK) return st;
  if (!q || !k || !perm_q || !perm_k || !lists) return fail(BSA_E_ARG, "null tensor pointer");
  const int nb = d->tokens / BSA_BLOCK;
  int K;
  if (topk_blocks > 0) {
    if (topk_blocks > nb) return fail(BSA_E_ARG, "topk_blocks = %d exceeds %d blocks",
                                      topk_blocks, nb);
    K = topk_blocks;
  } else {
    if (topk_blocks < 0) return fail(BSA_E_ARG, "topk_blocks = %d is negative", topk_blocks);
    K = bsa_topk_count(nb, topk_ratio);
    if (K < 1) return fail(BSA_E_ARG, "topk_ratio = %g is not in (0, 1]", double(topk_ratio));
  }
  const SelWs L = select_layout(d);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  const bool bf = is_bf16(d);
  float* qm = reinterpret_cast<float*>(at(ws, L.qm));
  float* km = reinterpret_cast<float*>(at(ws, L.km));
  float* S = scores_opt ? scores_opt : reinterpret_cast<float*>(at(ws, L.scores));
  hipError_t e = bsa::launch_block_means(bf, q, perm_q, d->heads, d->tokens, d->head_dim, qm,
                                         stream);
  if (e == hipSuccess)
    e = bsa::launch_block_means(bf, k, perm_k, d->heads, d->tokens, d->head_dim, km, stream);
  if (e == hipSuccess)
    e = bsa::launch_block_scores(qm, km, d->heads, nb, d->head_dim,
                                 1.f / std::sqrt(float(d->head_dim)), S, stream);
  if (e == hipSuccess) e = bsa::launch_topk(S, d->heads * nb, nb, K, lists, stream);
  return hip_status(e, "select launch");
}

bsa_status bsa_summaries(const bsa_desc* d, const void* q, const void* k, const void* v,
                         const int32_t* perm_k, uint32_t flags, float scale, float* kt,
                         float* vt, float* bias, void* ws, size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_desc(d);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !perm_k || !kt || !vt || !bias)
    return fail(BSA_E_ARG, "null tensor pointer");
  if (flags & ~uint32_t(BSA_MEANPOOL)) return fail(BSA_E_ARG, "unknown flags 0x%x", flags);
  if (!(std::isfinite(scale) && scale >= 0.f)) return fail(BSA_E_ARG, "bad scale %g", scale);
  const AttnWs L = attn_layout(d);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(run_summaries(d, L, ws, q, k, v, perm_k, (flags & BSA_MEANPOOL) != 0,
                                  resolve_scale(d, scale), kt, vt, bias, d->tokens / BSA_BLOCK,
                                  false, stream),
                    "summaries launch");
}

size_t bsa_summaries_noalloc_bytes(const bsa_desc* d) {
  if (check_desc(d) != BSA_OK) return 0;
  const AttnWs L = attn_layout(d);
  return L.anchor + align_up(size_t(d->heads) * d->head_dim * 4);
}

bsa_status bsa_summaries_noalloc(const bsa_desc* d, const void* q, const void* k, const void* v,
                                 const int32_t* perm_k, uint32_t flags, float scale, float* kt,
                                 float* vt, float* bias, hipStream_t stream) {
  bsa_status st = check_desc(d);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !perm_k || !kt || !vt || !bias)
    return fail(BSA_E_ARG, "null tensor pointer");
  if (flags & ~uint32_t(BSA_MEANPOOL)) return fail(BSA_E_ARG, "unknown flags 0x%x", flags);
  if (!(std::isfinite(scale) && scale >= 0.f)) return fail(BSA_E_ARG, "bad scale %g", scale);
  // the summaries read only the anchor's partial sums and the anchor from the workspace, which
  // attn_layout places first; that prefix has to fit in the static scratch
  const size_t need = bsa_summaries_noalloc_bytes(d);
  if (need > BSA_NOALLOC_SCRATCH_BYTES)
    return fail(BSA_E_ARG, "heads %d x tokens %d need %zu bytes of scratch, more than the %zu "
                "of the static scratch", d->heads, d->tokens, need,
                size_t(BSA_NOALLOC_SCRATCH_BYTES));
  st = check_device();
  if (st != BSA_OK) return st;
  void* ws = nullptr;
  hipError_t e = bsa::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "static scratch lookup");
  return hip_status(run_summaries(d, attn_layout(d), ws, q, k, v, perm_k,
                                  (flags & BSA_MEANPOOL) != 0, resolve_scale(d, scale), kt, vt,
                                  bias, d->tokens / BSA_BLOCK, false, stream),
                    "summaries launch");
}

namespace {

bsa_status check_attn_args(const bsa_desc* d, const void* q, const void* k, const void* v,
                           const int32_t* perm_k, uint32_t flags, float scale) {
  bsa_status st = check_desc(d);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !perm_k) return fail(BSA_E_ARG, "null tensor pointer");
  const uint32_t known =
      BSA_MEANPOOL | BSA_EXACT_ONLY | BSA_COMPRESSED_ONLY | BSA_TAIL_BLOCK | BSA_CHECK_LISTS;
  if (flags & ~known) return fail(BSA_E_ARG, "unknown flags 0x%x", flags);
  if ((flags & BSA_EXACT_ONLY) && (flags & BSA_COMPRESSED_ONLY))
    return fail(BSA_E_ARG, "BSA_EXACT_ONLY and BSA_COMPRESSED_ONLY are exclusive");
  if (!(std::isfinite(scale) && scale >= 0.f)) return fail(BSA_E_ARG, "bad scale %g", scale);
  return ok();
}

bsa_status check_attend_args(const bsa_desc* d, const int32_t* perm_q, const int32_t* lists,
                             int32_t topk, void* o) {
  if (!perm_q || !lists || !o) return fail(BSA_E_ARG, "null tensor pointer");
  const int nb = d->tokens / BSA_BLOCK;
  if (topk < 1 || topk > nb) return fail(BSA_E_ARG, "topk = %d is not in [1, %d]", topk, nb);
  return ok();
}

hipError_t do_prepare(const bsa_desc* d, const AttnWs& L, void* ws, const void* q,
                      const void* k, const void* v, const int32_t* perm_k, uint32_t flags,
                      float sc, hipStream_t stream, const Ctx& ctx = Ctx{}) {
  const bool bf = is_bf16(d);
  const int nb = d->tokens / BSA_BLOCK, nt = bsa::summary_tiles(nb);
  float* kt = reinterpret_cast<float*>(at(ws, L.kt));
  float* vt = reinterpret_cast<float*>(at(ws, L.vt));
  float* bias = reinterpret_cast<float*>(at(ws, L.bias));
  hipError_t e = run_summaries(d, L, ws, q, k, v, perm_k, (flags & BSA_MEANPOOL) != 0, sc, kt,
                               vt, bias, nt * 64, bf, stream);
  if (e == hipSuccess && bf)
    e = bsa::launch_summary_tiles(kt, vt, bias, d->heads, nb, at(ws, L.ktsw), at(ws, L.vtsw),
                                  stream);
  if (e == hipSuccess && bf && ctx.n > 0)
    e = bsa::launch_ctx_tiles(ctx.k, ctx.v, d->heads, ctx.n, at(ws, L.ctsw), at(ws, L.cvsw),
                              stream);
  return e;
}

hipError_t do_attend(const bsa_desc* d, const AttnWs& L, void* ws, const void* q,
                     const void* k, const void* v, const int32_t* perm_q,
                     const int32_t* perm_k, const int32_t* lists, int32_t topk, uint32_t flags,
                     float sc, void* o, float* lse, hipStream_t stream,
                     const Ctx& ctx = Ctx{}) {
  const int nb = d->tokens / BSA_BLOCK, nt = bsa::summary_tiles(nb);
  const int nt_c = ctx.n > 0 ? bsa::ceil_div(ctx.n, 64) : 0;
  const bool exact_on = !(flags & BSA_COMPRESSED_ONLY), comp_on = !(flags & BSA_EXACT_ONLY);
  // block-level compressed branch: pooled query of every query block (the block means the
  // select stage scores with)
  const bool tail_block = (flags & BSA_TAIL_BLOCK) && comp_on;
  bsa::AttnLaunch a{};
  a.H = d->heads;
  a.N = d->tokens;
  a.nb = nb;
  a.topk = topk;
  // video queries: exact tiles, then the biased tiles (summary tiles unless the compressed
  // branch is off or computed per block on the bf16 path, then context tiles, which belong to
  // the exact branch)
  a.n_exact = exact_on ? topk : 0;
  const bool summ_tiles = comp_on && !(tail_block && is_bf16(d));
  a.tau0 = summ_tiles ? 0 : nt;
  a.n_comp = (summ_tiles ? nt : 0) + (exact_on ? nt_c : 0);
  // context queries: every video block and every context tile, all exact
  a.n_ctx = ctx.n;
  a.ctx_n_exact = exact_on ? nb : 0;
  a.ctx_n_comp = exact_on ? nt_c : 0;
  a.q_ctx = ctx.q;
  a.k_ctx = ctx.k;
  a.v_ctx = ctx.v;
  a.o_ctx = ctx.o;
  a.lse_ctx = ctx.lse;
  a.scale = sc;
  a.q = q;
  a.perm_q = perm_q;
  a.lists = lists;
  a.bias = reinterpret_cast<const float*>(at(ws, L.bias));
  a.o = o;
  a.lse = lse;
  if (flags & BSA_CHECK_LISTS) {
    int32_t* status = reinterpret_cast<int32_t*>(at(ws, L.status));
    hipError_t e = bsa::launch_check_lists(lists, d->heads * nb, nb, topk, status, stream);
    if (e != hipSuccess) return e;
    a.list_status = status;
  }
  float* qbar = reinterpret_cast<float*>(at(ws, L.qbar));
  if (tail_block) {
    hipError_t e = bsa::launch_block_means(is_bf16(d), q, perm_q, d->heads, d->tokens,
                                           d->head_dim, qbar, stream);
    if (e != hipSuccess) return e;
  }
  if (is_bf16(d)) {
    if (exact_on && bsa::list_walk_applies(nb, topk)) {
      int32_t* walk = reinterpret_cast<int32_t*>(at(ws, L.walk));
      hipError_t e = bsa::launch_list_walk(lists, d->heads, nb, topk,
                                           reinterpret_cast<int32_t*>(at(ws, L.pop)), walk,
                                           stream);
      if (e != hipSuccess) return e;
      a.walk = walk;
    }
    a.ksw = at(ws, L.ksw);
    a.vsw = at(ws, L.vsw);
    a.ktsw = at(ws, L.ktsw);
    a.vtsw = at(ws, L.vtsw);
    if (ctx.n > 0) {
      a.ctsw = at(ws, L.ctsw);
      a.cvsw = at(ws, L.cvsw);
    }
    if (tail_block) {
      float* tail_o = reinterpret_cast<float*>(at(ws, L.tail_o));
      float* tail_lse = reinterpret_cast<float*>(at(ws, L.tail_lse));
      hipError_t e = bsa::launch_tail_block_bf16(
          a, qbar, reinterpret_cast<uint32_t*>(at(ws, L.tbits)), tail_o, tail_lse, stream);
      if (e != hipSuccess) return e;
      a.tail_o = tail_o;
      a.tail_lse = tail_lse;
    }
    return bsa::launch_attn_bf16(a, stream);
  }
  a.k = k;
  a.v = v;
  a.perm_k = perm_k;
  a.kt = reinterpret_cast<const float*>(at(ws, L.kt));
  a.vt = reinterpret_cast<const float*>(at(ws, L.vt));
  a.qbar = tail_block ? qbar : nullptr;
  return bsa::launch_attn_f32(a, stream);
}

}  // namespace

bsa_status bsa_prepare_kv(const bsa_desc* d, const void* q, const void* k, const void* v,
                          const int32_t* perm_k, uint32_t flags, float scale, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_attn_args(d, q, k, v, perm_k, flags, scale);
  if (st != BSA_OK) return st;
  const AttnWs L = attn_layout(d);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(do_prepare(d, L, ws, q, k, v, perm_k, flags, resolve_scale(d, scale), stream),
                    "prepare launch");
}

bsa_status bsa_attend(const bsa_desc* d, const void* q, const void* k, const void* v,
                      const int32_t* perm_q, const int32_t* perm_k, const int32_t* lists,
                      int32_t topk, uint32_t flags, float scale, void* o, float* lse_opt,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_attn_args(d, q, k, v, perm_k, flags, scale);
  if (st != BSA_OK) return st;
  st = check_attend_args(d, perm_q, lists, topk, o);
  if (st != BSA_OK) return st;
  const AttnWs L = attn_layout(d);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(do_attend(d, L, ws, q, k, v, perm_q, perm_k, lists, topk, flags,
                              resolve_scale(d, scale), o, lse_opt, stream),
                    "attention launch");
}

bsa_status bsa_sparse_attn(const bsa_desc* d, const void* q, const void* k, const void* v,
                           const int32_t* perm_q, const int32_t* perm_k, const int32_t* lists,
                           int32_t topk, uint32_t flags, float scale, void* o, float* lse_opt,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_attn_args(d, q, k, v, perm_k, flags, scale);
  if (st != BSA_OK) return st;
  st = check_attend_args(d, perm_q, lists, topk, o);
  if (st != BSA_OK) return st;
  const AttnWs L = attn_layout(d);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  const float sc = resolve_scale(d, scale);
  hipError_t e = do_prepare(d, L, ws, q, k, v, perm_k, flags, sc, stream);
  if (e != hipSuccess) return hip_status(e, "prepare launch");
  return hip_status(do_attend(d, L, ws, q, k, v, perm_q, perm_k, lists, topk, flags, sc, o,
                              lse_opt, stream),
                    "attention launch");
}

size_t bsa_workspace_bytes_ctx(const bsa_desc* d, int32_t n_ctx) {
  const size_t base = bsa_workspace_bytes(d);
  if (base == 0 || n_ctx < 0 || n_ctx > BSA_MAX_TOKENS ||
      (int64_t)d->heads * n_ctx > (int64_t)1 << 30)
    return 0;
  const size_t a = attn_layout(d, n_ctx).total;
  return a > base ? a : base;
}

namespace {

// the checks shared by the mixed-sequence calls (phase: 0 both, 1 prepare, 2 attend)
bsa_status check_ctx_call(const bsa_desc* d, int32_t n_ctx, const void* q, const void* k,
                          const void* v, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                          const int32_t* perm_q, const int32_t* perm_k, const int32_t* lists,
                          int32_t topk, uint32_t flags, float scale, const void* o,
                          const void* o_ctx, const void* ws, size_t ws_bytes, int phase) {
  bsa_status st = check_attn_args(d, q, k, v, perm_k, flags, scale);
  if (st != BSA_OK) return st;
  if (phase != 1) {
    st = check_attend_args(d, perm_q, lists, topk, const_cast<void*>(o));
    if (st != BSA_OK) return st;
  }
  if (n_ctx < 0 || n_ctx > BSA_MAX_TOKENS || (int64_t)d->heads * n_ctx > (int64_t)1 << 30)
    return fail(BSA_E_ARG, "n_ctx = %d is out of range", n_ctx);
  if (n_ctx > 0 && (!k_ctx || !v_ctx || (phase != 1 && (!q_ctx || !o_ctx))))
    return fail(BSA_E_ARG, "null context tensor pointer");
  st = check_ws(ws, ws_bytes, attn_layout(d, n_ctx).total);
  if (st != BSA_OK) return st;
  return check_device();
}

}  // namespace

bsa_status bsa_sparse_attn_ctx(const bsa_desc* d, int32_t n_ctx, const void* q, const void* k,
                               const void* v, const void* q_ctx, const void* k_ctx,
                               const void* v_ctx, const int32_t* perm_q, const int32_t* perm_k,
                               const int32_t* lists, int32_t topk, uint32_t flags, float scale,
                               void* o, void* o_ctx, float* lse_opt, float* lse_ctx_opt,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_ctx_call(d, n_ctx, q, k, v, q_ctx, k_ctx, v_ctx, perm_q, perm_k, lists,
                                 topk, flags, scale, o, o_ctx, ws, ws_bytes, 0);
  if (st != BSA_OK) return st;
  const AttnWs L = attn_layout(d, n_ctx);
  const float sc = resolve_scale(d, scale);
  const Ctx ctx{n_ctx, q_ctx, k_ctx, v_ctx, o_ctx, lse_ctx_opt};
  hipError_t e = do_prepare(d, L, ws, q, k, v, perm_k, flags, sc, stream, ctx);
  if (e != hipSuccess) return hip_status(e, "prepare launch");
  return hip_status(do_attend(d, L, ws, q, k, v, perm_q, perm_k, lists, topk, flags, sc, o,
                              lse_opt, stream, ctx),
                    "attention launch");
}

bsa_status bsa_prepare_kv_ctx(const bsa_desc* d, int32_t n_ctx, const void* q, const void* k,
                              const void* v, const void* k_ctx, const void* v_ctx,
                              const int32_t* perm_k, uint32_t flags, float scale, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  bsa_status st = check_ctx_call(d, n_ctx, q, k, v, nullptr, k_ctx, v_ctx, nullptr, perm_k,
                                 nullptr, 0, flags, scale, nullptr, nullptr, ws, ws_bytes, 1);
  if (st != BSA_OK) return st;
  const Ctx ctx{n_ctx, nullptr, k_ctx, v_ctx, nullptr, nullptr};
  return hip_status(do_prepare(d, attn_layout(d, n_ctx), ws, q, k, v, perm_k, flags,
                               resolve_scale(d, scale), stream, ctx),
                    "prepare launch");
}

bsa_status bsa_attend_ctx(const bsa_desc* d, int32_t n_ctx, const void* q, const void* k,
                          const void* v, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                          const int32_t* perm_q, const int32_t* perm_k, const int32_t* lists,
                          int32_t topk, uint32_t flags, float scale, void* o, void* o_ctx,
                          float* lse_opt, float* lse_ctx_opt, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  bsa_status st = check_ctx_call(d, n_ctx, q, k, v, q_ctx, k_ctx, v_ctx, perm_q, perm_k, lists,
                                 topk, flags, scale, o, o_ctx, ws, ws_bytes, 2);
  if (st != BSA_OK) return st;
  const Ctx ctx{n_ctx, q_ctx, k_ctx, v_ctx, o_ctx, lse_ctx_opt};
  return hip_status(do_attend(d, attn_layout(d, n_ctx), ws, q, k, v, perm_q, perm_k, lists,
                              topk, flags, resolve_scale(d, scale), o, lse_opt, stream, ctx),
                    "attention launch");
}

bsa_status bsa_check_lists(int32_t rows, int32_t n_blocks, int32_t topk, const int32_t* lists,
                           int32_t* result, hipStream_t stream) {
  if (rows < 1 || n_blocks < 1) return fail(BSA_E_ARG, "rows and n_blocks must be >= 1");
  if (topk < 1 || topk > n_blocks)
    return fail(BSA_E_ARG, "topk = %d is not in [1, %d]", topk, n_blocks);
  if ((int64_t)rows * topk > (int64_t)1 << 31) return fail(BSA_E_ARG, "too many list entries");
  if (!lists || !result) return fail(BSA_E_ARG, "null tensor pointer");
  bsa_status st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(bsa::launch_check_lists(lists, rows, n_blocks, topk, result, stream),
                    "list check launch");
}

bsa_status bsa_list_status(const void* ws, size_t ws_bytes, int32_t* result, hipStream_t stream) {
  if (!ws || !result) return fail(BSA_E_ARG, "null pointer");
  if (ws_bytes < 2 * sizeof(int32_t))
    return fail(BSA_E_WORKSPACE, "workspace of %zu bytes holds no list status", ws_bytes);
  bsa_status st = check_device();
  if (st != BSA_OK) return st;
  // the status is the first item of every attention workspace layout
  hipError_t e = hipMemcpyAsync(result, ws, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_status(e, "list status read");
}

size_t bsa_partition_workspace_bytes(int32_t problems, int32_t tokens) {
  if (problems < 1 || tokens < BSA_BLOCK || tokens % BSA_BLOCK || tokens > BSA_MAX_TOKENS)
    return 0;
  return bsa::partition_ws_bytes(problems, tokens);
}

bsa_status bsa_reblock_from_projections(int32_t problems, int32_t tokens, const float* proj,
                                        int32_t* perm, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (problems < 1) return fail(BSA_E_ARG, "problems = %d must be >= 1", problems);
  if (tokens < BSA_BLOCK || tokens % BSA_BLOCK || tokens > BSA_MAX_TOKENS)
    return fail(BSA_E_ARG, "tokens = %d must be a positive multiple of 64 up to %d", tokens,
                BSA_MAX_TOKENS);
  if ((int64_t)problems * tokens > (int64_t)1 << 30)
    return fail(BSA_E_ARG, "problems * tokens is too large");
  if (!perm || (!proj && bsa::tree_levels(tokens / BSA_BLOCK) > 0))
    return fail(BSA_E_ARG, "null tensor pointer");
  bsa_status st = check_ws(ws, ws_bytes, bsa::partition_ws_bytes(problems, tokens));
  if (st != BSA_OK) return st;
  st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(bsa::launch_partition_from_proj(problems, tokens, proj, perm, ws, stream),
                    "partition launch");
}

bsa_status bsa_topk_from_scores(int32_t rows, int32_t n_blocks, int32_t topk,
                                const float* scores, int32_t* lists, hipStream_t stream) {
  if (rows < 1 || n_blocks < 1) return fail(BSA_E_ARG, "rows and n_blocks must be >= 1");
  if (topk < 1 || topk > n_blocks)
    return fail(BSA_E_ARG, "topk = %d is not in [1, %d]", topk, n_blocks);
  if ((int64_t)rows * n_blocks > (int64_t)1 << 31) return fail(BSA_E_ARG, "too many scores");
  if (!scores || !lists) return fail(BSA_E_ARG, "null tensor pointer");
  bsa_status st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(bsa::launch_topk(scores, rows, n_blocks, topk, lists, stream),
                    "top-K launch");
}

bsa_status bsa_tile_layout(int32_t heads, int32_t grid_t, int32_t grid_h, int32_t grid_w,
                           int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t* perm,
                           hipStream_t stream) {
  if (heads < 1) return fail(BSA_E_ARG, "heads must be >= 1");
  if (grid_t < 1 || grid_h < 1 || grid_w < 1 || tile_t < 1 || tile_h < 1 || tile_w < 1)
    return fail(BSA_E_ARG, "grid and tile sides must be >= 1");
  if ((int64_t)tile_t * tile_h * tile_w != BSA_BLOCK)
    return fail(BSA_E_ARG, "tile %dx%dx%d does not hold %d tokens", tile_t, tile_h, tile_w,
                BSA_BLOCK);
  if (grid_t % tile_t || grid_h % tile_h || grid_w % tile_w)
    return fail(BSA_E_ARG, "tile %dx%dx%d does not divide grid %dx%dx%d", tile_t, tile_h, tile_w,
                grid_t, grid_h, grid_w);
  const int64_t n = (int64_t)grid_t * grid_h * grid_w;
  if (n > BSA_MAX_TOKENS) return fail(BSA_E_ARG, "grid has %lld tokens (max %d)", (long long)n,
                                      BSA_MAX_TOKENS);
  if (!perm) return fail(BSA_E_ARG, "null tensor pointer");
  bsa_status st = check_device();
  if (st != BSA_OK) return st;
  return hip_status(bsa::launch_tile_layout(heads, grid_t, grid_h, grid_w, tile_t, tile_h, tile_w,
                                            perm, stream),
                    "tile layout launch");
}

}  // extern "C"
