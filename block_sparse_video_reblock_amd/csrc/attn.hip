// Two-branch block-sparse attention for gfx950: exact branch over the selected key blocks,
// compressed branch over the anchor-weighted block summaries, log-sum-exp merge and the
// inverse query permutation, in one kernel.
//
// [comfyui-wiki.com "Spark-H3 ...", "What Spark-Attn changes"]: an exact branch fully computes
// the top-ranked key/value blocks while a compressed branch covers the rest; Spark-Reweight
// replaces mean-pooled summaries by weighted summaries plus a log-mass bias.
// [comfy.icu "MiniMax H3 Spark Attention (SM89)", "What it's doing under the hood"]: in the
// compressed branch each query still uses its own query vector; only the key/value side is
// pooled per block.
//
// Both branches are softmax attentions of the same 64 queries, so a single online softmax over
// the exact key tiles followed by the summary tiles (selected blocks masked to -inf) is the
// log-sum-exp merge of the two branch results.
//
// bf16 kernel layout (D = 128): one workgroup of 4 waves per (head, query block).  Every wave
// keeps all 64 queries of the block in registers and takes every 4th tile of the work list
// (exact tiles first, then summary tiles and context tiles), so the waves run independent
// online softmaxes that are merged at the end.  Options: context query blocks (mixed
// sequences) in the same launch, and a block-level compressed state computed beforehand
// (k_tail_block_bf16) merged in place of the summary tiles.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: the accumulator layout of S^T is then directly the B operand of
// O^T = V^T P^T.  K/V tiles arrive pre-swizzled (see summaries.hip) so that every wave load
// is 1 KiB contiguous and no LDS transpose is needed.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSelWords = (1 << 19) / 64 / 32;   // bitmap words for the largest nb

BSA_DEV bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// A wave-uniform read of memory that no kernel writes while it runs, through the constant
// address space: a scalar load (counted by lgkmcnt, so waiting for it never waits for the
// vector loads in flight).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
BSA_DEV int load_uniform(const int32_t* p) { return *(const_i32_ptr)p; }

// word 3 of a raw buffer resource: 32-bit data format (untyped loads need a nonzero format)
constexpr int kBufferDword3 = 0x00020000;

template <bool B>
struct KindTag {
  static constexpr bool value = B;
};

// acc + the sum of the eight bf16 values of an MFMA operand, in fp32 (v_dot2_f32_bf16 with
// ones)
BSA_DEV float row_sum_bf16(const bf16x8_t& p, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  const uint4 u = __builtin_bit_cast(uint4, p);
  const bf2 one = __builtin_bit_cast(bf2, 0x3F803F80u);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), one, acc, false);
}

// Running-max slack: the online softmax keeps a stale maximum until a row's new maximum exceeds
// it by more than this (log2 units), so probabilities stay below 2^8 and the accumulator is
// rescaled only when the maximum really moves.  The result is the same softmax.
constexpr float kMaxSlack = 8.f;

BSA_DEV bf16x8_t pack8(const f32x16_t& s, int base) {
  uint4 u;
  u.x = cvt_pk_bf16(s[base + 0], s[base + 1]);
  u.y = cvt_pk_bf16(s[base + 2], s[base + 3]);
  u.z = cvt_pk_bf16(s[base + 4], s[base + 5]);
  u.w = cvt_pk_bf16(s[base + 6], s[base + 7]);
  return as_bf16x8(u);
}

// Map workgroup ids so that each XCD (ids are dealt round-robin over 8 XCDs) processes a
// contiguous range of (head, query block) pairs: neighbouring query blocks of one head (tree
// neighbours, which select overlapping key blocks) then share that XCD's L2.
BSA_DEV int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + min(x, r) + k;
}

// The video launch with H a multiple of 4: XCDs 2c and 2c + 1 take heads c, c + 4, c + 8, ...
// in turn, each a contiguous half of the head's query blocks (half = ceil(nbq / 2) per XCD and
// head, grid 2 H half).  Each XCD still walks neighbouring query blocks, and only four heads'
// key and value tiles are in use at a time instead of eight.  False for an id past the last
// block of its half.
constexpr int kHeadsPerRound = 4;
BSA_DEV bool xcd_pair_remap(int bid, int nbq, int& h, int& i) {
  const int x = bid & 7, k = bid >> 3, half = (nbq + 1) >> 1;
  const int round = k / half;
  h = (x >> 1) + kHeadsPerRound * round;
  i = (x & 1) * half + (k - round * half);
  return i < nbq;
}

// One set of query blocks of an attention launch and the work list of each block.
struct QSide {
  const uint16_t* q;     // [H][rows][D]
  const int32_t* perm;   // [H][rows] layout (block i = rows perm[64 i ..]), or null: block i
                         // holds rows 64 i .. 64 i + 63; rows past `rows` are padding, not written
  bool listed;           // exact key blocks from the kernel's lists [H][nbq][topk]; else
                         // blocks 0 .. n_exact - 1
  const float* tail_o;   // block-level compressed state [H][nbq][D], [H][nbq] (log2), or null
  const float* tail_lse;
  uint16_t* o;           // [H][rows][D]
  float* lse;            // [H][rows] (natural log) or null
  int rows, nbq, topk;
  int n_exact;           // exact key tiles per block
  int n_comp, tau0;      // biased tiles tau0 .. tau0 + n_comp - 1: summary tiles 0 .. nt_s - 1,
                         // then context tiles nt_s .. nt_s + nt_c - 1
};
// The key side: key / value blocks, summary tiles and context tiles, all in MFMA operand order.
struct KSide {
  const uint4 *ksw, *vsw;    // [H][nb][1024]
  const uint4 *ktsw, *vtsw;  // [H][nt_s][1024]
  const float* bias;         // [H][nt_s * 64] summary bias, -inf on padding rows
  const uint4 *ctsw, *cvsw;  // [H][nt_c][1024], rows past n_ctx zero
  int nb, nt_s, nt_c, n_ctx;
  const int32_t* list_status;  // nonzero: a list is malformed and nothing is computed (or null)
};

// Workgroups 0 .. wg_c - 1 take the query blocks of side `cs` (context queries: few, long
// blocks, dispatched first and spread over every XCD), the rest those of side `vs`.  The lists
// are a separate read-only argument so that the work loop reads them with scalar loads.  CTX
// false compiles the launch without context tokens (no context side, every block listed, no
// context tiles), whose work loops carry none of the context branches.
template <bool CTX>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(QSide cs, QSide vs, int wg_c, KSide ks,
                                                       const int32_t* __restrict__ lists, int H,
                                                       float scale_log2) {
  constexpr int D = 128;
  __shared__ uint32_t sel_bits[kMaxSelWords];
  __shared__ float sm_m[4][64];
  __shared__ float sm_l[4][64];
  __shared__ float sm_o[64 * 129];
  __shared__ float sm_tail[D];  // block-level compressed output of this query block
  __shared__ float sm_wc[64];   // and its weight in each row's merge
  __shared__ uint4 sq[2][8][64];  // the queries in B-operand order (see below)
  // [nt_s * 64] summary-row bias * log2 e (-inf if selected), then with context tiles two
  // 64-row masks: 0 for a full context tile, 0 / -inf for the valid / padding rows of the last
  extern __shared__ float sbias[];

  if (ks.list_status != nullptr && load_uniform(ks.list_status) != 0) return;
  const bool is_ctx = CTX && blockIdx.x < wg_c;
  const QSide S = is_ctx ? cs : vs;
  int h, i;
  if (!CTX && H % kHeadsPerRound == 0) {
    if (!xcd_pair_remap(blockIdx.x, S.nbq, h, i)) return;
  } else {
    const int local = is_ctx ? blockIdx.x : xcd_remap(blockIdx.x - wg_c, H * vs.nbq);
    h = local / S.nbq;
    i = local - h * S.nbq;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ntiles = ks.nt_s, nb = ks.nb;
  const int n_exact = S.n_exact, n_comp = S.n_comp, tau0 = S.tau0, topk = S.topk;
  const bool listed = !CTX || S.listed;
  // Sparse lists (at most half of the key blocks) are walked from a rotated start: the 64
  // workgroups that run together on an XCD begin at 64 evenly spaced points of their lists.
  // (With every block selected the lists coincide and an unrotated walk shares each tile in L2
  // across those workgroups, so full lists are not rotated.)  The order changes only the
  // rounding of the sums.
  const int rot = (!is_ctx && 2 * n_exact <= nb)
                      ? (((blockIdx.x - wg_c) >> 3) & 63) * n_exact / 64
                      : 0;
  const int32_t* list = listed ? lists + ((size_t)h * S.nbq + i) * topk : nullptr;

  // bitmap of this query block's selected key blocks (masks them in the compressed branch);
  // cleared over every summary row, padding included
  const bool permuted = !CTX || S.perm != nullptr;
  const int32_t* pq = permuted ? S.perm + (size_t)h * S.rows + (size_t)i * kBlk : nullptr;
  const float* bias_h = ks.bias + (size_t)h * ntiles * 64;
  if (n_comp > 0 && tau0 < ntiles) {
    const int words = (ntiles * 64 + 31) >> 5;
    for (int w = tid; w < words; w += 256) sel_bits[w] = 0u;
    __syncthreads();
    for (int t = tid; t < topk; t += 256) {
      const int j = list[t];
      atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();  // bitmap complete
    for (int key = tid; key < ntiles * 64; key += 256) {
      const bool sel = (sel_bits[key >> 5] >> (key & 31)) & 1u;
      sbias[key] = sel ? -INFINITY : bias_h[key] * kLog2e;  // padding rows hold -inf already
    }
  }
  if (CTX && n_comp > 0 && ks.nt_c > 0 && tid < 128) {
    const int last_rows = ks.n_ctx - (ks.nt_c - 1) * 64;
    sbias[ntiles * 64 + tid] = (tid < 64 || tid - 64 < last_rows) ? 0.f : -INFINITY;
  }
  // queries of the block, as the B operand of S^T = K Q^T: lane holds query 32n + l32,
  // head-dim elements 16c + 8g .. +8
  // (sq[n][c][lane] = the 8 elements 16c + 8g .. +8 of query 32n + l32), loaded once
  for (int u = tid; u < 2 * 8 * 64; u += 256) {
    const int n = u >> 9, c = (u >> 6) & 7, ln = u & 63;
    const int r = 32 * n + (ln & 31);
    const int tok = permuted ? pq[r] : min(i * kBlk + r, S.rows - 1);
    sq[n][c][ln] =
        reinterpret_cast<const uint4*>(S.q + ((size_t)h * S.rows + tok) * D)[2 * c + (ln >> 5)];
  }
  const bool tail = S.tail_o != nullptr;
  if (tail && tid < D) sm_tail[tid] = S.tail_o[((size_t)h * S.nbq + i) * D + tid];
  __syncthreads();

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][n][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  // this lane's part of the row sums (its half of every key chunk); the two halves of a row
  // are added at the end
  float l_run[2] = {0.f, 0.f};

  // work items of this wave: it = wave, wave + 4, ... over the exact tiles and then the
  // summary tiles; each is processed as two 32-key halves, and the keys of the next half are
  // loaded while the current one finishes.  The two kinds run in separate loops (compiled
  // separately), so neither carries the other's arithmetic or register copies.
  const int n_items = n_exact + n_comp;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto run = [&](auto kind, int it, int it_end) {
    constexpr bool EXACT = decltype(kind)::value;
    if (it >= it_end) return;
    auto tile_ptrs = [&](int t, const uint4*& kp, const uint4*& vp, int& k0) {
      if (EXACT) {
        const int tr = t + rot < n_exact ? t + rot : t + rot - n_exact;
        const size_t blk = (size_t)h * nb + (listed ? load_uniform(list + tr) : tr);
        kp = ks.ksw + blk * 1024;
        vp = ks.vsw + blk * 1024;
        k0 = 0;
      } else {
        const int tau = t - n_exact + tau0;
        if (!CTX || tau < ntiles) {
          const size_t blk = (size_t)h * ntiles + tau;
          kp = ks.ktsw + blk * 1024;
          vp = ks.vtsw + blk * 1024;
          k0 = tau * 64;
        } else {
          const int ct = tau - ntiles;
          const size_t blk = (size_t)h * ks.nt_c + ct;
          kp = ks.ctsw + blk * 1024;
          vp = ks.cvsw + blk * 1024;
          k0 = (ntiles + (ct == ks.nt_c - 1 ? 1 : 0)) * 64;
        }
      }
    };
    const uint4 *kb, *vb;
    int key0;
    tile_ptrs(it, kb, vb, key0);
    uint4 kr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kr[c] = kb[c * 64 + lane];
    int hh = 0;
#pragma unroll 1
    while (it < it_end) {
      // the next half of this wave (scalar work, ahead of the vector code); past the last
      // item it points at a valid tile, and the keys loaded from there go unused
      int it_n = it, hh_n = hh + 1;
      const uint4 *kb_n = kb, *vb_n = vb;
      int key0_n = key0;
      if (hh_n == 2) {
        it_n += 4;
        hh_n = 0;
        if (it_n < it_end) tile_ptrs(it_n, kb_n, vb_n, key0_n);
      }
      // keep the query operands in LDS: re-read them per use instead of pinning 64 registers
      asm volatile("" ::: "memory");
      // S^T[n]: lane holds query 32n + l32 and keys 32hh + 8(r/4) + 4g + (r%4), r = 0..15
      auto scores = [&](int n) {
        f32x16_t t;
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[c]),
                                                      as_bf16x8(sq[n][c][lane]), t, 0, 0, 0);
        return t;
      };
      // logits in log2 units (s * scale_log2, plus bias * log2 e for summary rows, -inf if the
      // block is selected or past the end); returns the max the exponentials subtract
      auto row_max = [&](int n, f32x16_t& t) {
        float mx = -INFINITY;
        if (EXACT) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, t[r]);
          mx *= scale_log2;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 b4 =
                *reinterpret_cast<const float4*>(&sbias[key0 + 32 * hh + 8 * j + 4 * g]);
            const float bj[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              t[4 * j + u] = fmaf(t[4 * j + u], scale_log2, bj[u]);
              mx = fmaxf(mx, t[4 * j + u]);
            }
          }
        }
        mx = xor32_max(mx);
        // lazy rescale: move the running max only when it grows by more than kMaxSlack
        const bool grow = mx > m_run[n] + kMaxSlack;
        if (__any(grow)) {
          const float m_new = grow ? mx : m_run[n];
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[n] - m_new) : 1.f;
          m_run[n] = m_new;
          l_run[n] *= alpha;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][n][r] *= alpha;
        }
        return (m_run[n] == -INFINITY) ? 0.f : m_run[n];
      };
      // P^T in bf16: the B operand of key chunk c = 2hh + cc is registers 8cc..8cc+8 of S^T[n]
      bf16x8_t pb[2][2];
      auto probs = [&](int n, f32x16_t& t, float m_use) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          t[r] = __builtin_amdgcn_exp2f(EXACT ? fmaf(t[r], scale_log2, -m_use) : t[r] - m_use);
        pb[0][n] = pack8(t, 0);
        pb[1][n] = pack8(t, 8);
        // row sum of the bf16 probabilities the value products use (bf16 dot products with
        // ones, fp32 accumulation)
        l_run[n] = row_sum_bf16(pb[1][n], row_sum_bf16(pb[0][n], l_run[n]));
      };
      uint4 vr[8];
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, 1024 * 16, kBufferDword3);
      // O^T[d chunk a][n] += V^T[a][key chunk c] P^T[c][n]
      auto values = [&](int n) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            acc[a][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr[a * 2 + cc]),
                                                                pb[cc][n], acc[a][n], 0, 0, 0);
      };
      // order: the score products of rows 32..63 run while the vector unit exponentiates rows
      // 0..31, and the value products of rows 0..31 while it exponentiates rows 32..63
      f32x16_t s0 = scores(0);
      const float m0 = row_max(0, s0);
      f32x16_t s1 = scores(1);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          vr[a * 2 + cc] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16,
                                                           (a * 4 + 2 * hh + cc) * 1024, 0));
      probs(0, s0, m0);
      // (an empty use keeps the exponentials of rows 0..31 ahead of the branch below, in the
      // block of the score products they overlap)
      asm volatile("" ::"v"(pb[0][0]), "v"(pb[1][0]));
      const float m1 = row_max(1, s1);
      values(0);
      probs(1, s1, m1);
      // the next half's keys load during the value products of this one (buffer loads:
      // plain loads here would be merged with the ones before the loop into one load at the
      // loop head, after the wait)
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)kb_n, 0, 1024 * 16, kBufferDword3);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        kr[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rk, lane * 16, (hh_n * 8 + c) * 1024, 0));
      values(1);
      it = it_n;
      hh = hh_n;
      kb = kb_n;
      vb = vb_n;
      key0 = key0_n;
    }
  };
  run(KindTag<true>{}, wv, n_exact);
  // the first summary item of this wave in the same round-robin sequence
  run(KindTag<false>{}, wv + 4 * ((max(n_exact - wv, 0) + 3) / 4), n_items);

  // merge the four waves' online-softmax states
#pragma unroll
  for (int n = 0; n < 2; ++n) l_run[n] = xor32_sum(l_run[n]);
  if (g == 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      sm_m[wave][32 * n + l32] = m_run[n];
      sm_l[wave][32 * n + l32] = l_run[n];
    }
  }
  __syncthreads();
  // (with a block-level compressed state, that state is a fifth softmax part: max lc, sum 1,
  // output sm_tail)
  const float lc = tail ? S.tail_lse[(size_t)h * S.nbq + i] : -INFINITY;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int qq = 32 * n + l32;
    float M = lc;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][qq]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float lt = __builtin_amdgcn_exp2f(lc - Mu);
    float L = lt;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += sm_l[w][qq] * __builtin_amdgcn_exp2f(sm_m[w][qq] - Mu);
    const float f = (L > 0.f) ? __builtin_amdgcn_exp2f(m_run[n] - Mu) / L : 0.f;
    if (tail && wave == 0 && g == 0) sm_wc[qq] = (L > 0.f) ? lt / L : 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][n][r] *= f;
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int idx = (32 * n + l32) * 129 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
            sm_o[idx] = (w == 0) ? acc[a][n][r] : sm_o[idx] + acc[a][n][r];
          }
    }
    __syncthreads();
  }

  // inverse permutation: row qq of the block is token perm_q[64 i + qq]
  const int qq = tid >> 2, part = tid & 3;
  const int tok = permuted ? pq[qq] : i * kBlk + qq;
  if (permuted || tok < S.rows) {
    uint4* dst = reinterpret_cast<uint4*>(S.o + ((size_t)h * S.rows + tok) * D + part * 32);
    float* src = sm_o + qq * 129 + part * 32;
    if (tail) {  // the block-level compressed output, weighted per row
      const float wq = sm_wc[qq];
#pragma unroll
      for (int e = 0; e < 32; ++e) src[e] = fmaf(wq, sm_tail[part * 32 + e], src[e]);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint4 u;
      u.x = pack_bf16x2(src[8 * v + 0], src[8 * v + 1]);
      u.y = pack_bf16x2(src[8 * v + 2], src[8 * v + 3]);
      u.z = pack_bf16x2(src[8 * v + 4], src[8 * v + 5]);
      u.w = pack_bf16x2(src[8 * v + 6], src[8 * v + 7]);
      dst[v] = u;
    }
    if (S.lse != nullptr && part == 0) {
      float M = lc;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][qq]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float L = __builtin_amdgcn_exp2f(lc - Mu);
      for (int w = 0; w < 4; ++w) L += sm_l[w][qq] * __builtin_amdgcn_exp2f(sm_m[w][qq] - Mu);
      S.lse[(size_t)h * S.rows + tok] = (L > 0.f) ? (Mu + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// fp32 path (D = 64): one wave per (head, query block), one query per lane, K/V tiles staged
// in LDS.  Plain fp32 FMA arithmetic.  Query and key sides as in the bf16 kernel, with plain
// row-major tensors in place of the swizzled tiles.
struct QSide32 {
  const float* q;        // [H][rows][D]
  const int32_t* perm;   // [H][rows] or null (identity blocks, padding rows not written)
  const int32_t* lists;  // [H][nbq][topk] or null (blocks 0 .. n_exact - 1)
  const float* qbar;     // pooled query per block [H][nbq][D] for the summary tiles, or null
  float* o;              // [H][rows][D]
  float* lse;            // [H][rows] or null
  int rows, nbq, topk, n_exact, n_comp, tau0;
};
struct KSide32 {
  const float *k, *v;       // video keys / values [H][N][D]
  const int32_t* perm_k;    // [H][N]
  const float *kt, *vt;     // summaries [H][nb][D]
  const float* bias;        // [H][nt_s * 64]
  const float *kc, *vc;     // context keys / values [H][n_ctx][D]
  int N, nb, nt_s, nt_c, n_ctx;
  const int32_t* list_status;  // nonzero: a list is malformed and nothing is computed (or null)
};

__global__ __launch_bounds__(64) void k_attn_f32(QSide32 cs, QSide32 vs, int wg_c, KSide32 ks,
                                                 int H, float scale_log2) {
  constexpr int D = 64;
  __shared__ float sk[64][D + 1];
  __shared__ float sv[64][D + 1];
  __shared__ float sb[64];
  __shared__ uint32_t sel_bits[kMaxSelWords];
  if (ks.list_status != nullptr && load_uniform(ks.list_status) != 0) return;
  const bool is_ctx = blockIdx.x < wg_c;
  const QSide32 S = is_ctx ? cs : vs;
  const int local = is_ctx ? blockIdx.x : xcd_remap(blockIdx.x - wg_c, H * vs.nbq);
  const int h = local / S.nbq, i = local - h * S.nbq;
  const int t = threadIdx.x;
  const int nb = ks.nb, ntiles = ks.nt_s, N = ks.N;
  const int n_exact = S.n_exact, n_comp = S.n_comp, tau0 = S.tau0, topk = S.topk;
  const int32_t* list = S.lists ? S.lists + ((size_t)h * S.nbq + i) * topk : nullptr;
  const int words = (nb + 31) >> 5;
  for (int w = t; w < words; w += 64) sel_bits[w] = 0u;
  __syncthreads();
  if (list != nullptr)
    for (int x = t; x < topk; x += 64) atomicOr(&sel_bits[list[x] >> 5], 1u << (list[x] & 31));

  const int row = i * kBlk + t;
  const int tok = S.perm ? S.perm[(size_t)h * S.rows + row] : min(row, S.rows - 1);
  const float* qrow = S.q + ((size_t)h * S.rows + tok) * D;
  float qv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = qrow[d];
    acc[d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float* bias_h = ks.bias + (size_t)h * ntiles * 64;
  for (int it = 0; it < n_exact + n_comp; ++it) {
    const bool exact = it < n_exact;
    const int tau = it - n_exact + tau0;
    // block-level compressed branch: the summary tiles see the block's pooled query, the
    // context tiles (exact) the query's own
    if (S.qbar != nullptr && !exact && (tau == 0 || tau == ntiles)) {
      const float* src = tau == 0 ? S.qbar + ((size_t)h * S.nbq + i) * D : qrow;
#pragma unroll
      for (int d = 0; d < D; ++d) qv[d] = src[d];
    }
    __syncthreads();
    if (exact) {
      const int j = list ? list[it] : it;
      const int ktok = ks.perm_k[(size_t)h * N + (size_t)j * kBlk + t];
      for (int d = 0; d < D; ++d) {
        sk[t][d] = ks.k[((size_t)h * N + ktok) * D + d];
        sv[t][d] = ks.v[((size_t)h * N + ktok) * D + d];
      }
      sb[t] = 0.f;
    } else if (tau < ntiles) {
      const int key = tau * 64 + t;
      const bool masked = key >= nb || ((sel_bits[key >> 5] >> (key & 31)) & 1u);
      for (int d = 0; d < D; ++d) {
        sk[t][d] = key < nb ? ks.kt[((size_t)h * nb + key) * D + d] : 0.f;
        sv[t][d] = key < nb ? ks.vt[((size_t)h * nb + key) * D + d] : 0.f;
      }
      sb[t] = masked ? -INFINITY : bias_h[key] * kLog2e;
    } else {
      const int r = (tau - ntiles) * 64 + t;
      const bool ok = r < ks.n_ctx;
      for (int d = 0; d < D; ++d) {
        sk[t][d] = ok ? ks.kc[((size_t)h * ks.n_ctx + r) * D + d] : 0.f;
        sv[t][d] = ok ? ks.vc[((size_t)h * ks.n_ctx + r) * D + d] : 0.f;
      }
      sb[t] = ok ? 0.f : -INFINITY;
    }
    __syncthreads();
    float x[64];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qv[d], sk[r][d], dot);
      x[r] = dot * scale_log2 + sb[r];
      mx = fmaxf(mx, x[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      const float p = exp2f(x[r] - m_use);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sv[r][d], acc[d]);
    }
    m_run = m_new;
  }
  if (S.perm == nullptr && row >= S.rows) return;  // padding row of a context block
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int d = 0; d < D; ++d) S.o[((size_t)h * S.rows + tok) * D + d] = acc[d] * inv;
  if (S.lse != nullptr)
    S.lse[(size_t)h * S.rows + tok] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// ------------------------------------------------ block-level compressed branch (bf16 path)
//
// [comfy.icu "MiniMax H3 Spark Attention (SM89)", "What it's doing under the hood"]: the node's
// tail_granularity option switches the compressed branch to one pooled query per query block.
// Every query of block i then sees the same compressed state, so it is computed once per block:
// a small masked attention of the nb pooled queries of a head over its summary tiles, whose
// result the attention kernel merges in place of its summary tiles.

// bits[h][i][w]: bit b set iff key block 32 w + b is in lists[h][i] (lists ascending)
__global__ __launch_bounds__(256) void k_tail_bits(const int32_t* __restrict__ lists, size_t rows,
                                                  int topk, int W, uint32_t* __restrict__ bits) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * W) return;
  const size_t row = idx / W;
  const int w = int(idx - row * W), lo_key = 32 * w;
  const int32_t* l = lists + row * topk;
  int lo = 0, hi = topk;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (l[mid] < lo_key) lo = mid + 1; else hi = mid;
  }
  uint32_t word = 0u;
  for (int t = lo; t < topk && l[t] < lo_key + 32; ++t) word |= 1u << (l[t] - lo_key);
  bits[idx] = word;
}

// One workgroup per (64 pooled queries, head): rows i0 .. i0+63 of the head's query blocks.
// The 4 waves take every 4th summary tile, each over all 64 rows, with the score / value MFMA
// layout of k_attn_bf16; the pooled queries enter as bf16 hi + lo pairs (fp32 accuracy in the
// logits, whose keys are the bf16 summary tiles).  Row r masks the blocks of its own list.
// Output per row: the normalised compressed output and its log2-sum-exp (-inf if every block
// is selected).
__global__ __launch_bounds__(256, 1) void k_tail_block_bf16(
    const float* __restrict__ qbar, const uint32_t* __restrict__ bits,
    const uint4* __restrict__ ktsw, const uint4* __restrict__ vtsw,
    const float* __restrict__ bias, int nb, int ntiles, float scale_log2,
    float* __restrict__ tail_o, float* __restrict__ tail_lse) {
  constexpr int D = 128;
  // the query operands (32 KiB) and, after the tile loop, the merged outputs share one buffer
  __shared__ __align__(16) float sm_o[64 * 129];
  __shared__ float sm_m[4][64];
  __shared__ float sm_l[4][64];
  uint4 (*sqh)[8][64] = reinterpret_cast<uint4 (*)[8][64]>(sm_o);
  uint4 (*sql)[8][64] = sqh + 2;
  const int h = blockIdx.y, i0 = blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int W = 2 * ntiles;

  // sqh/sql[n][c][lane]: elements 16c + 8g .. +8 of pooled row 32n + l32, split x = hi + lo
  for (int u = tid; u < 2 * 8 * 64; u += 256) {
    const int n = u >> 9, c = (u >> 6) & 7, ln = u & 63;
    const int row = i0 + 32 * n + (ln & 31);
    float x[8];
    if (row < nb) {
      const float4* src =
          reinterpret_cast<const float4*>(qbar + ((size_t)h * nb + row) * D + 16 * c + 8 * (ln >> 5));
      const float4 a = src[0], b = src[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hw[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      const float r0 = x[2 * e] - bf16_to_f32(uint16_t(hw[e] & 0xFFFFu));
      const float r1 = x[2 * e + 1] - bf16_to_f32(uint16_t(hw[e] >> 16));
      lw[e] = pack_bf16x2(r0, r1);
    }
    sqh[n][c][ln] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    sql[n][c][ln] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  __syncthreads();

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][n][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  // selection words of this lane's rows (clamped: rows past nb compute unused values)
  const uint32_t* bits_row[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
    bits_row[n] = bits + ((size_t)h * nb + min(i0 + 32 * n + l32, nb - 1)) * W;
  const float* bias_h = bias + (size_t)h * ntiles * 64;

#pragma unroll 1
  for (int tau = wave; tau < ntiles; tau += 4) {
    const uint4* kb = ktsw + ((size_t)h * ntiles + tau) * 1024;
    const uint4* vb = vtsw + ((size_t)h * ntiles + tau) * 1024;
#pragma unroll 1
    for (int hh = 0; hh < 2; ++hh) {
      uint4 kr[8], vr[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) kr[c] = kb[(hh * 8 + c) * 64 + lane];
      // S^T: lane holds row 32n + l32 and keys 32hh + 8(r/4) + 4g + (r%4) of the tile
      f32x16_t st[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x16_t t;
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[c]), as_bf16x8(sqh[n][c][lane]),
                                                      t, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 8; ++c)
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[c]), as_bf16x8(sql[n][c][lane]),
                                                      t, 0, 0, 0);
        st[n] = t;
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) vr[a * 2 + cc] = vb[(a * 4 + 2 * hh + cc) * 64 + lane];
      const int key0 = tau * 64 + 32 * hh;
      float bj[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 b4 = *reinterpret_cast<const float4*>(bias_h + key0 + 8 * j + 4 * g);
        bj[4 * j + 0] = b4.x * kLog2e;
        bj[4 * j + 1] = b4.y * kLog2e;
        bj[4 * j + 2] = b4.z * kLog2e;
        bj[4 * j + 3] = b4.w * kLog2e;
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x16_t& t = st[n];
        const uint32_t word = bits_row[n][2 * tau + hh];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * j + u;
            const bool sel = (word >> (8 * j + 4 * g + u)) & 1u;
            t[r] = sel ? -INFINITY : fmaf(t[r], scale_log2, bj[r]);
            mx = fmaxf(mx, t[r]);
          }
        mx = xor32_max(mx);
        const float m_new = fmaxf(m_run[n], mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[n] - m_use);
        m_run[n] = m_new;
        l_run[n] *= alpha;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[a][n][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = __builtin_amdgcn_exp2f(t[r] - m_use);
        const bf16x8_t p0 = pack8(t, 0), p1 = pack8(t, 8);
        l_run[n] = row_sum_bf16(p1, row_sum_bf16(p0, l_run[n]));
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          acc[a][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr[a * 2]), p0, acc[a][n],
                                                              0, 0, 0);
          acc[a][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr[a * 2 + 1]), p1,
                                                              acc[a][n], 0, 0, 0);
        }
      }
    }
  }

  // merge the four waves and write the rows of this group (the barrier also ends every
  // wave's use of the query operands, whose memory the outputs reuse)
#pragma unroll
  for (int n = 0; n < 2; ++n) l_run[n] = xor32_sum(l_run[n]);
  if (g == 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      sm_m[wave][32 * n + l32] = m_run[n];
      sm_l[wave][32 * n + l32] = l_run[n];
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int qq = 32 * n + l32;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][qq]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += sm_l[w][qq] * __builtin_amdgcn_exp2f(sm_m[w][qq] - Mu);
    const float f = (L > 0.f) ? __builtin_amdgcn_exp2f(m_run[n] - Mu) / L : 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][n][r] *= f;
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int idx = (32 * n + l32) * 129 + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
            sm_o[idx] = (w == 0) ? acc[a][n][r] : sm_o[idx] + acc[a][n][r];
          }
    }
    __syncthreads();
  }
  {
    const int qq = tid >> 2, part = tid & 3, row = i0 + qq;
    if (row < nb) {
      float4* dst = reinterpret_cast<float4*>(tail_o + ((size_t)h * nb + row) * D + part * 32);
      const float* src = sm_o + qq * 129 + part * 32;
#pragma unroll
      for (int v = 0; v < 8; ++v)
        dst[v] = make_float4(src[4 * v], src[4 * v + 1], src[4 * v + 2], src[4 * v + 3]);
      if (part == 0) {
        float M = -INFINITY;
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][qq]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float L = 0.f;
        for (int w = 0; w < 4; ++w) L += sm_l[w][qq] * __builtin_amdgcn_exp2f(sm_m[w][qq] - Mu);
        tail_lse[(size_t)h * nb + row] = (L > 0.f) ? Mu + __log2f(L) : -INFINITY;
      }
    }
  }
}

// ------------------------------------------------------------- exact-tile walk order
// The order in which a query block walks its selected key blocks changes only the rounding of
// its softmax sums.  Walking the blocks that many query blocks of the head selected first makes
// the workgroups that run together on an XCD request those shared tiles close in time, so more
// of them come from L2: each list is reordered by (selection count of the key block, highest
// first; key block index).

__global__ void k_zero_i32(size_t n, int32_t* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    out[i] = 0;
}

// pop[h][j] = number of lists of head h that contain key block j.  Grid (chunks, H): each
// workgroup counts its chunk of the head's entries in LDS, then adds its nonzero counts.
constexpr int kPopMaxBlocks = 8192;  // nb of the largest sequence (LDS histogram)
__global__ __launch_bounds__(256) void k_list_popularity(const int32_t* __restrict__ lists,
                                                         int nb, int topk,
                                                         int32_t* __restrict__ pop) {
  __shared__ int hist[kPopMaxBlocks];
  const int h = blockIdx.y;
  for (int j = threadIdx.x; j < nb; j += 256) hist[j] = 0;
  __syncthreads();
  const size_t n = (size_t)nb * topk;
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t e0 = blockIdx.x * per, e1 = min(n, e0 + per);
  const int32_t* l = lists + (size_t)h * n;
  for (size_t e = e0 + threadIdx.x; e < e1; e += 256) {
    const int j = l[e];
    if (j >= 0 && j < nb) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += 256)
    if (hist[j] != 0) atomicAdd(&pop[(size_t)h * nb + j], hist[j]);
}

// one 64-thread workgroup per list: sort its entries by (nb - pop, index) in LDS
constexpr int kWalkMax = 256;  // longest list that gets the popularity order
__global__ __launch_bounds__(64) void k_list_walk(const int32_t* __restrict__ lists,
                                                  const int32_t* __restrict__ pop, int nb,
                                                  int topk, int32_t* __restrict__ walk) {
  __shared__ uint32_t v[kWalkMax];
  const size_t row = blockIdx.x;
  const int h = int(row / (size_t)nb);
  const int32_t* l = lists + row * topk;
  int n2 = 1;
  while (n2 < topk) n2 <<= 1;
  for (int t = threadIdx.x; t < n2; t += 64) {
    uint32_t key = 0xFFFFFFFFu;
    if (t < topk) {
      const int j = l[t];
      const int c = (j >= 0 && j < nb) ? pop[(size_t)h * nb + j] : 0;
      key = (uint32_t(nb - c) << 13) | uint32_t(j & 8191);
    }
    v[t] = key;
  }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < (n2 >> 1); t += 64) {
        const int i = 2 * t - (t & (j - 1)), ip = i + j;
        const uint32_t x = v[i], y = v[ip];
        if ((x > y) == ((i & k) == 0)) {
          v[i] = y;
          v[ip] = x;
        }
      }
      __syncthreads();
    }
  for (int t = threadIdx.x; t < topk; t += 64) walk[row * topk + t] = int32_t(v[t] & 8191u);
}

}  // namespace

hipError_t launch_list_walk(const int32_t* lists, int H, int nb, int topk, int32_t* pop,
                            int32_t* walk, hipStream_t s) {
  const size_t np = (size_t)H * nb;
  k_zero_i32<<<(unsigned)std::min<size_t>((np + 255) / 256, 1024), 256, 0, s>>>(np, pop);
  const size_t n = (size_t)nb * topk;
  k_list_popularity<<<dim3((unsigned)std::min<size_t>((n + 4095) / 4096, 32), H), 256, 0, s>>>(
      lists, nb, topk, pop);
  k_list_walk<<<(unsigned)np, 64, 0, s>>>(lists, pop, nb, topk, walk);
  return hipGetLastError();
}

bool list_walk_applies(int nb, int topk) { return topk <= kWalkMax && 2 * topk <= nb; }

hipError_t launch_tail_block_bf16(const AttnLaunch& a, const float* qbar, uint32_t* bits,
                                  float* tail_o, float* tail_lse, hipStream_t s) {
  const int nt = summary_tiles(a.nb);
  const size_t rows = (size_t)a.H * a.nb;
  const size_t words = rows * 2 * nt;
  k_tail_bits<<<ceil_div(long(words), 256), 256, 0, s>>>(a.lists, rows, a.topk, 2 * nt, bits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_tail_block_bf16<<<dim3(ceil_div(a.nb, 64), a.H), 256, 0, s>>>(
      qbar, bits, static_cast<const uint4*>(a.ktsw), static_cast<const uint4*>(a.vtsw), a.bias,
      a.nb, nt, a.scale * kLog2e, tail_o, tail_lse);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnLaunch& a, hipStream_t s) {
  const int nt_s = summary_tiles(a.nb), nt_c = a.n_ctx > 0 ? ceil_div(a.n_ctx, 64) : 0;
  KSide ks{};
  ks.ksw = static_cast<const uint4*>(a.ksw);
  ks.vsw = static_cast<const uint4*>(a.vsw);
  ks.ktsw = static_cast<const uint4*>(a.ktsw);
  ks.vtsw = static_cast<const uint4*>(a.vtsw);
  ks.bias = a.bias;
  ks.ctsw = static_cast<const uint4*>(a.ctsw);
  ks.cvsw = static_cast<const uint4*>(a.cvsw);
  ks.nb = a.nb;
  ks.nt_s = nt_s;
  ks.nt_c = nt_c;
  ks.n_ctx = a.n_ctx;
  ks.list_status = a.list_status;
  QSide vs{static_cast<const uint16_t*>(a.q), a.perm_q, true, a.tail_o, a.tail_lse,
           static_cast<uint16_t*>(a.o), a.lse, a.N, a.nb, a.topk, a.n_exact, a.n_comp, a.tau0};
  QSide cs{static_cast<const uint16_t*>(a.q_ctx), nullptr, false, nullptr, nullptr,
           static_cast<uint16_t*>(a.o_ctx), a.lse_ctx, a.n_ctx, nt_c, 0, a.ctx_n_exact,
           a.ctx_n_comp, nt_s};
  const int wg_c = a.H * nt_c;
  const bool biased = a.n_comp > 0 || (nt_c > 0 && a.ctx_n_comp > 0);
  const size_t dyn = biased ? (size_t)(nt_s + (nt_c > 0 ? 2 : 0)) * 64 * sizeof(float) : 0;
  const int32_t* lists = a.walk != nullptr ? a.walk : a.lists;
  if (wg_c > 0)
    k_attn_bf16<true><<<wg_c + a.H * a.nb, 256, dyn, s>>>(cs, vs, wg_c, ks, lists, a.H,
                                                          a.scale * kLog2e);
  else
    k_attn_bf16<false><<<a.H % kHeadsPerRound == 0 ? 2 * a.H * ((a.nb + 1) / 2) : a.H * a.nb, 256,
                         dyn, s>>>(cs, vs, 0, ks, lists, a.H, a.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnLaunch& a, hipStream_t s) {
  const int nt_s = summary_tiles(a.nb), nt_c = a.n_ctx > 0 ? ceil_div(a.n_ctx, 64) : 0;
  KSide32 ks{};
  ks.k = static_cast<const float*>(a.k);
  ks.v = static_cast<const float*>(a.v);
  ks.perm_k = a.perm_k;
  ks.kt = a.kt;
  ks.vt = a.vt;
  ks.bias = a.bias;
  ks.kc = static_cast<const float*>(a.k_ctx);
  ks.vc = static_cast<const float*>(a.v_ctx);
  ks.N = a.N;
  ks.nb = a.nb;
  ks.nt_s = nt_s;
  ks.nt_c = nt_c;
  ks.n_ctx = a.n_ctx;
  ks.list_status = a.list_status;
  QSide32 vs{static_cast<const float*>(a.q), a.perm_q, a.lists, a.qbar, static_cast<float*>(a.o),
             a.lse, a.N, a.nb, a.topk, a.n_exact, a.n_comp, a.tau0};
  QSide32 cs{static_cast<const float*>(a.q_ctx), nullptr, nullptr, nullptr,
             static_cast<float*>(a.o_ctx), a.lse_ctx, a.n_ctx, nt_c, 0, a.ctx_n_exact,
             a.ctx_n_comp, nt_s};
  const int wg_c = a.H * nt_c;
  k_attn_f32<<<wg_c + a.H * a.nb, 64, 0, s>>>(cs, vs, wg_c, ks, a.H, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace bsa
