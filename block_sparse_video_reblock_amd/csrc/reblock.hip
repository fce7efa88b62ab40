// Reblock (stage 1) for gfx950: per-head second moments, Mahalanobis-cosine normalisation and
// the capacity-constrained hierarchical tree partition into 64-token leaves.
//
// [comfy.icu "MiniMax H3 Spark Attention (SM89)", "What it's doing under the hood"]: queries are
// compared through M_K = E[k k^T] and keys through M_Q = E[q q^T] (a Mahalanobis cosine); a
// tree partition under a capacity limit cuts them into leaves of 64 tokens each, rebuilt for
// every layer, step and head; the result is a permutation, and the tensors keep their values.
// [comfyui-wiki.com "Spark-H3 ...", "What Spark-Attn changes"]: two queries are alike when their
// attention score patterns over the keys are alike; the partitioner splits until every leaf has
// the block size, in O(N log N).
//
// Split rule (plain reading, see tree.h): principal direction of the group in the metric, found
// by 8 power steps from the group's smallest token id, and a capacity cut at floor(m/2) blocks.
//
// Formulation on the GPU.  With y_i = x_i / sqrt(x_i^T M x_i) and any F with F^T F = M, the unit
// vectors of the metric are u_i = F y_i.  Writing the power step v <- C_u v / |C_u v| in terms of
// w = F^T v gives   z = C_y w,  t = M z,  w <- t / sqrt(z . t),   start w0 = M (y_i0 - mu),
// and the projection u_i . v = y_i . w.  So no factorisation of M is needed: the kernels keep
// the group covariance of y (C_y) and M, both 128 x 128 fp32.
//
// Per level and group: C_y is accumulated by MFMA from 16-bit splits of the centred values
// d = y - shift (shift = the parent group's mean, so cancellation stays small): s d = hi + mid
// with two fp16 terms under a power-of-two scale s per problem, and the three products down to
// 2^-22 relative size accumulated in fp32 (a two-term bf16 split, 16 bits, leaves errors near
// 1e-4 in the projections of ill-conditioned groups; 22 bits match an exact covariance to fp32
// rounding of the projections).  Wide levels
// (few large groups) split each group over several workgroups and reduce the partials in a fixed
// order; narrow levels run one fused workgroup per group.  All reductions have a fixed order,
// so results are deterministic.
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "tree.h"

namespace bsa {
namespace {

constexpr int kMomChunk = 2048;   // tokens per partial of the second-moment reduction
constexpr int kSlots = 32;        // workgroups per problem at the widest levels
#ifndef BSA_LAST_WIDE
#define BSA_LAST_WIDE 5
#endif
// Levels 0..kLastWide are wide (each group's statistics split over several workgroups, then
// a direction, a projection and a split kernel); deeper levels run one workgroup per parent
// or per subtree.
constexpr int kLastWide = BSA_LAST_WIDE;
// partial covariances per problem: every left group of the deepest wide level, 2 slices each
constexpr int kPartialSlots = kLastWide > 4 ? (1 << kLastWide) : kSlots;

// workgroups per group at a wide level (1: the level is not wide)
inline int wide_slices(int level, int nb) {
  if (level > kLastWide) return 1;
  return std::min(kSlots >> std::min(level, 4), nb >> level);
}
constexpr int kIters = 8;         // power steps per split (the default; Lite takes fewer)
// Elements per LDS row of the staged (transposed) chunk.  Measured on gfx950: the 32 x 32 x 16
// operand reads of the raw moments (stats_mfma) meet no bank conflicts with 144-byte rows, the
// 16 x 16 x 32 operand reads of the symmetric statistics (sym_mfma) none with 160-byte rows
// (four conflict cycles per read with 144-byte rows, and no swizzle of the 16-byte chunks by
// row removed them).
constexpr int kMomStride = 72, kSymStride = 80;

BSA_DEV bf16x8_t lds_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Register-resident D x D accumulator: 4 waves, each holding TILES 32 x 32 MFMA tiles.  For
// D = 128 wave w holds the column block w of every row block (FULL_COLS): each lane then holds
// a whole column of the symmetric matrix over its two half-waves, so a product C v needs no
// exchange between waves.  For D = 64 wave w holds the single tile (w / 2, w % 2).
template <int D>
struct Cov {
  static constexpr int AC = D / 32;
  static constexpr int TILES = AC * AC / 4;
  static constexpr bool FULL_COLS = (D == 128);
  BSA_DEV static int ac(int w, int t) { return D == 128 ? t : (w >> 1); }
  BSA_DEV static int bc(int w, int t) { return D == 128 ? w : (w & 1); }
};

// How the centred values d of a chunk are split into 16-bit MFMA operands:
//  kExact:   one bf16 term; d is exact in bf16 (raw bf16 inputs, no scale, no shift).
//  kBf16x3:  d = hi + mid + lo, bf16 each (24 significant bits); the products hi hi, hi mid,
//            mid hi, hi lo, lo hi, mid mid are accumulated, the dropped ones lie below fp32
//            rounding of the sum.
//  kF16x2:   s d = hi + mid, fp16 each, with s a power of two per problem chosen so that
//            |s d| <= 2^14 for every token (no overflow).  hi and mid carry 11 significant bits
//            each, so hi + mid represents s d to about 2^-22 relative (or 2^-25 absolute where
//            mid is subnormal); the products hi hi, hi mid, mid hi are accumulated (mid mid is
//            below 2^-22 relative) and the sum is multiplied by 1 / s^2 (exact).  Half the
//            MFMA work of kBf16x3 for a covariance accurate to a few parts in 10^7.
constexpr int kExact = 1, kF16x2 = 2, kBf16x3 = 3;
template <int MODE>
constexpr int split_terms() { return MODE == kExact ? 1 : (MODE == kF16x2 ? 2 : 3); }

template <int D, int NT, int S = kMomStride>
struct __align__(16) StageLds {
  uint16_t t[NT][D][S];
};
// the staging of the symmetric statistics: two fp16 terms, 160-byte rows
template <int D>
using SymStage = StageLds<D, 2, kSymStride>;

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
BSA_DEV f16x8_t lds_f16x8(const uint16_t* p) {
  return __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(p));
}
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
// round-to-nearest-even pack of two floats to fp16 (v_cvt_pk_f16_f32)
BSA_DEV uint32_t cvt_pk_f16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
BSA_DEV f32x2_t unpack_f16x2(uint32_t u) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, u), f32x2_t);
}

// One 64-position chunk of the covariance accumulation.  Thread t stages the token pair
// (2 (t%32), 2 (t%32) + 1) for the DPT = D/8 elements of element group t/32 (see stat_dim):
// d = x * scale - shift, split into 16-bit terms written as packed pairs of tokens; the
// transposed staging rows of the two groups of a wave sit 8 rows apart (32 banks with 144-byte
// rows; with 160-byte rows the two halves meet, about 0.8 conflict cycles per write).
// tokmap == nullptr means position = token id; inv_n == nullptr means scale 1.
template <int D>
BSA_DEV int stat_dim(int dg, int j) {
  return D == 128 ? ((j < 8) ? dg * 8 + j : 64 + dg * 8 + (j - 8)) : dg * 8 + j;
}

// The DPT elements of element group dg of one row, as two 16-byte pieces (raw input bits).
template <typename T, int D>
BSA_DEV void load_dims(const T* row, int dg, uint4* raw);
template <>
BSA_DEV void load_dims<uint16_t, 128>(const uint16_t* row, int dg, uint4* raw) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) raw[h2] = *reinterpret_cast<const uint4*>(row + h2 * 64 + dg * 8);
}
template <>
BSA_DEV void load_dims<float, 64>(const float* row, int dg, uint4* raw) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) raw[h2] = *reinterpret_cast<const uint4*>(row + dg * 8 + 4 * h2);
}
template <typename T, int D>
BSA_DEV void unpack_dims(const uint4* raw, float* out);
template <>
BSA_DEV void unpack_dims<uint16_t, 128>(const uint4* raw, float* out) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const uint32_t w[4] = {raw[h2].x, raw[h2].y, raw[h2].z, raw[h2].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[h2 * 8 + 2 * i] = __uint_as_float(w[i] << 16);
      out[h2 * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}
template <>
BSA_DEV void unpack_dims<float, 64>(const uint4* raw, float* out) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    out[4 * h2] = __uint_as_float(raw[h2].x);
    out[4 * h2 + 1] = __uint_as_float(raw[h2].y);
    out[4 * h2 + 2] = __uint_as_float(raw[h2].z);
    out[4 * h2 + 3] = __uint_as_float(raw[h2].w);
  }
}

// Raw inputs of one chunk for one thread: its two tokens' DPT elements (input bits, 16
// registers) and scales.
template <typename T, int D>
struct ChunkRegs {
  uint4 raw[2][2];
  float sc[2];
};

template <typename T, int D>
BSA_DEV void stats_load(const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                        const float* __restrict__ inv_n, int c0, ChunkRegs<T, D>& r) {
  const int tp = threadIdx.x & 31, dg = threadIdx.x >> 5;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pos = c0 + 2 * tp + u;
    const int tok = tokmap ? tokmap[pos] : pos;
    r.sc[u] = inv_n ? inv_n[tok] : 1.f;
    load_dims<T, D>(X + (size_t)tok * D, dg, r.raw[u]);
  }
}
// The two token ids this thread loads for the chunk at position c0 (see stats_load).
BSA_DEV void chunk_tokens(const int32_t* __restrict__ tokmap, int c0, int (&tok)[2]) {
  const int tp = threadIdx.x & 31;
#pragma unroll
  for (int u = 0; u < 2; ++u) tok[u] = tokmap ? tokmap[c0 + 2 * tp + u] : c0 + 2 * tp + u;
}
// stats_load with the token ids already read
template <typename T, int D>
BSA_DEV void stats_load_tok(const T* __restrict__ X, const float* __restrict__ inv_n,
                            const int (&tok)[2], ChunkRegs<T, D>& r) {
  const int dg = threadIdx.x >> 5;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    r.sc[u] = inv_n ? inv_n[tok[u]] : 1.f;
    load_dims<T, D>(X + (size_t)tok[u] * D, dg, r.raw[u]);
  }
}

// Stage one chunk (centred, split) into LDS and accumulate d; no barrier.  ysc: the kF16x2
// scale s.
template <typename T, int D, int MODE, int S>
BSA_DEV void stats_stage(const ChunkRegs<T, D>& r, const float* sh_shift, float ysc,
                         StageLds<D, split_terms<MODE>(), S>& st, float* dpart) {
  constexpr int DPT = D / 8;
  const int tp = threadIdx.x & 31, dg = threadIdx.x >> 5;
  float xv[2][DPT];
  unpack_dims<T, D>(r.raw[0], xv[0]);
  unpack_dims<T, D>(r.raw[1], xv[1]);
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int e = stat_dim<D>(dg, j);
    const float sh = sh_shift[e];
    const float d0 = xv[0][j] * r.sc[0] - sh, d1 = xv[1][j] * r.sc[1] - sh;
    dpart[j] += d0 + d1;
    // round-to-nearest-even packs (one instruction per token pair and term)
    if (MODE == kF16x2) {
      const float s0 = d0 * ysc, s1 = d1 * ysc;  // exact: ysc is a power of two
      const uint32_t hp = cvt_pk_f16(s0, s1);
      const f32x2_t hv = unpack_f16x2(hp);
      reinterpret_cast<uint32_t*>(&st.t[0][e][0])[tp] = hp;
      reinterpret_cast<uint32_t*>(&st.t[1][e][0])[tp] = cvt_pk_f16(s0 - hv.x, s1 - hv.y);
    } else {
      const uint32_t hp = cvt_pk_bf16(d0, d1);
      reinterpret_cast<uint32_t*>(&st.t[0][e][0])[tp] = hp;
      if (MODE == kBf16x3) {
        const float r0 = d0 - __uint_as_float(hp << 16);
        const float r1 = d1 - __uint_as_float(hp & 0xFFFF0000u);
        const uint32_t mp = cvt_pk_bf16(r0, r1);
        reinterpret_cast<uint32_t*>(&st.t[1][e][0])[tp] = mp;
        reinterpret_cast<uint32_t*>(&st.t[2][e][0])[tp] =
            cvt_pk_bf16(r0 - __uint_as_float(mp << 16), r1 - __uint_as_float(mp & 0xFFFF0000u));
      }
    }
  }
}

template <int D, int MODE>
BSA_DEV void stats_mfma(const StageLds<D, split_terms<MODE>()>& st, f32x16_t* acc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int t = 0; t < Cov<D>::TILES; ++t) {
      const int ra = 32 * Cov<D>::ac(w, t) + l32, rb = 32 * Cov<D>::bc(w, t) + l32;
      const int col = 16 * ks + 8 * g;
      if (MODE == kF16x2) {
        const f16x8_t aH = lds_f16x8(&st.t[0][ra][col]);
        const f16x8_t bH = lds_f16x8(&st.t[0][rb][col]);
        const f16x8_t aM = lds_f16x8(&st.t[1][ra][col]);
        const f16x8_t bM = lds_f16x8(&st.t[1][rb][col]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aH, bH, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aH, bM, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aM, bH, acc[t], 0, 0, 0);
        continue;
      }
      const bf16x8_t aH = lds_bf16x8(&st.t[0][ra][col]);
      const bf16x8_t bH = lds_bf16x8(&st.t[0][rb][col]);
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aH, bH, acc[t], 0, 0, 0);
      if (MODE == kBf16x3) {
        const bf16x8_t aM = lds_bf16x8(&st.t[1][ra][col]);
        const bf16x8_t bM = lds_bf16x8(&st.t[1][rb][col]);
        const bf16x8_t aL = lds_bf16x8(&st.t[2][ra][col]);
        const bf16x8_t bL = lds_bf16x8(&st.t[2][rb][col]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aH, bM, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aM, bH, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aH, bL, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL, bH, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aM, bM, acc[t], 0, 0, 0);
      }
    }
  }
}

// Accumulate the chunks [blk0, blk1) (64-position blocks).  With PREFETCH the next chunk's
// inputs are loaded into registers while the current chunk's MFMAs run (for kernels with
// registers to spare); without it each chunk's loads complete before it is staged.
template <typename T, int D, int MODE, bool PREFETCH>
BSA_DEV void stats_range(const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                         const float* __restrict__ inv_n, int blk0, int blk1,
                         const float* sh_shift, float ysc, StageLds<D, split_terms<MODE>()>& st,
                         f32x16_t* acc, float* dpart) {
  if (blk0 >= blk1) return;
  ChunkRegs<T, D> cur;
  if (PREFETCH) stats_load<T, D>(X, tokmap, inv_n, blk0 * kBlk, cur);
  for (int b = blk0; b < blk1; ++b) {
    if (!PREFETCH) stats_load<T, D>(X, tokmap, inv_n, b * kBlk, cur);
    stats_stage<T, D, MODE, kMomStride>(cur, sh_shift, ysc, st, dpart);
    __syncthreads();
    if (PREFETCH && b + 1 < blk1) stats_load<T, D>(X, tokmap, inv_n, (b + 1) * kBlk, cur);
    stats_mfma<D, MODE>(st, acc);
    __syncthreads();
  }
}

template <int D>
BSA_DEV void zero_acc(f32x16_t* acc) {
#pragma unroll
  for (int t = 0; t < Cov<D>::TILES; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
}

// Sum the per-thread d partials over the 32 token pairs: result in out[D] (LDS).  Each
// element group lives in one half-wave, so a 32-lane reduction suffices.  red is unused.
template <int D>
BSA_DEV void reduce_dpart(const float* dpart, float* red, float* out) {
  constexpr int DPT = D / 8;
  const int tid = threadIdx.x, tp = tid & 31, dg = tid >> 5;
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    float x = row16_sum(dpart[j]);
    x += __shfl_xor(x, 16, 64);
    if (tp == 0) out[stat_dim<D>(dg, j)] = x;
  }
  __syncthreads();
}

// Register dump order of an accumulator: element ((w*TILES + t)*16 + r)*64 + lane.
template <int D>
BSA_DEV void store_acc(float* dst, const f32x16_t* acc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < Cov<D>::TILES; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[((w * Cov<D>::TILES + t) * 16 + r) * 64 + lane] = acc[t][r];
}
template <int D>
BSA_DEV void add_acc(const float* src, f32x16_t* acc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < Cov<D>::TILES; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] += src[((w * Cov<D>::TILES + t) * 16 + r) * 64 + lane];
}

// (a, b) coordinates of accumulator element (t, r) of this lane
template <int D>
BSA_DEV int acc_row(int t, int r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return 32 * Cov<D>::ac(w, t) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <int D>
BSA_DEV int acc_col(int t) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return 32 * Cov<D>::bc(w, t) + (lane & 31);
}

// ------------------------------------------------- symmetric covariance statistics
// The group statistics D D^T (D: centred values, d x tokens) are symmetric, so only the upper
// triangle of its (d/16) x (d/16) grid of 16 x 16 tiles is accumulated, with
// v_mfma_f32_16x16x32_f16: lane l of an operand holds row (or column) l % 16 and the 8 tokens
// 8 (l / 16) .. + 8 of a 32-token step, so the operand of block x serves as A for tile row x
// and as B for tile column x.  The tiles are dealt to the 4 waves so that each wave touches
// few blocks: for d = 128 waves 0 and 1 take the triangles of blocks 0-3 and 4-7 (10 tiles
// each), waves 2 and 3 the rectangles {0,1} x {4..7} and {2,3} x {4..7} (8 tiles each).
// The result lane l of a tile holds column l % 16 and rows 4 (l / 16) .. + 4.
template <int D> struct SymPlan;
template <> struct SymPlan<128> {
  static constexpr int NB = 8, MAXT = 10;
  static constexpr int nt[4] = {10, 10, 8, 8};
  static constexpr int a[4][10] = {{0, 0, 0, 0, 1, 1, 1, 2, 2, 3}, {4, 4, 4, 4, 5, 5, 5, 6, 6, 7},
                                   {0, 0, 0, 0, 1, 1, 1, 1, 0, 0}, {2, 2, 2, 2, 3, 3, 3, 3, 0, 0}};
  static constexpr int b[4][10] = {{0, 1, 2, 3, 1, 2, 3, 2, 3, 3}, {4, 5, 6, 7, 5, 6, 7, 6, 7, 7},
                                   {4, 5, 6, 7, 4, 5, 6, 7, 0, 0}, {4, 5, 6, 7, 4, 5, 6, 7, 0, 0}};
};
template <> struct SymPlan<64> {
  static constexpr int NB = 4, MAXT = 3;
  static constexpr int nt[4] = {3, 3, 2, 2};
  static constexpr int a[4][3] = {{0, 0, 1}, {2, 2, 3}, {0, 0, 0}, {1, 1, 0}};
  static constexpr int b[4][3] = {{0, 1, 1}, {2, 3, 3}, {2, 3, 0}, {2, 3, 0}};
};
template <int D, int W>
constexpr bool sym_is_row(int x) {
  for (int t = 0; t < SymPlan<D>::nt[W]; ++t)
    if (SymPlan<D>::a[W][t] == x) return true;
  return false;
}
template <int D, int W>
constexpr bool sym_uses(int x) {
  for (int t = 0; t < SymPlan<D>::nt[W]; ++t)
    if (SymPlan<D>::a[W][t] == x || SymPlan<D>::b[W][t] == x) return true;
  return false;
}

template <int D>
struct SymAcc {
  f32x4_t t[SymPlan<D>::MAXT];
  BSA_DEV void zero() {
#pragma unroll
    for (int i = 0; i < SymPlan<D>::MAXT; ++i) t[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// one 64-token chunk (two 32-token steps) of the staged fp16 split into wave W's tiles
template <int D, int W>
BSA_DEV void sym_mfma_wave(const SymStage<D>& st, SymAcc<D>& acc) {
  using P = SymPlan<D>;
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // operands of the row blocks first; a column block that is not also a row block is read
    // just before its tiles (the tiles are listed by column within each row run)
    f16x8_t oh[P::NB], om[P::NB];
#pragma unroll
    for (int x = 0; x < P::NB; ++x)
      if (sym_is_row<D, W>(x)) {
        oh[x] = lds_f16x8(&st.t[0][16 * x + r16][32 * ks + 8 * kg]);
        om[x] = lds_f16x8(&st.t[1][16 * x + r16][32 * ks + 8 * kg]);
      }
#pragma unroll
    for (int b = 0; b < P::NB; ++b) {
      if (!sym_uses<D, W>(b)) continue;
      f16x8_t bh = oh[b], bm = om[b];
      if (!sym_is_row<D, W>(b)) {
        bh = lds_f16x8(&st.t[0][16 * b + r16][32 * ks + 8 * kg]);
        bm = lds_f16x8(&st.t[1][16 * b + r16][32 * ks + 8 * kg]);
      }
#pragma unroll
      for (int t = 0; t < P::nt[W]; ++t) {
        if (P::b[W][t] != b) continue;
        const int a = P::a[W][t];
        acc.t[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oh[a], bh, acc.t[t], 0, 0, 0);
        acc.t[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oh[a], bm, acc.t[t], 0, 0, 0);
        acc.t[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(om[a], bh, acc.t[t], 0, 0, 0);
      }
    }
  }
}
template <int D>
BSA_DEV void sym_mfma(const SymStage<D>& st, SymAcc<D>& acc) {
  switch (threadIdx.x >> 6) {
    case 0: sym_mfma_wave<D, 0>(st, acc); break;
    case 1: sym_mfma_wave<D, 1>(st, acc); break;
    case 2: sym_mfma_wave<D, 2>(st, acc); break;
    default: sym_mfma_wave<D, 3>(st, acc); break;
  }
}

// Accumulate the chunks [blk0, blk1) with the fp16 two-term split (see stats_range).
// sh_shift (LDS) receives the shift sh_val of the calling thread (threads < D) once the first
// chunk's loads are in flight.
template <typename T, int D, bool PREFETCH>
BSA_DEV void sym_stats_range(const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                             const float* __restrict__ inv_n, int blk0, int blk1,
                             float* sh_shift, float sh_val, float ysc, SymStage<D>& st,
                             SymAcc<D>& acc, float* dpart) {
  ChunkRegs<T, D> cur;
  // with PREFETCH, a block's rows are loaded one block ahead and its token ids two blocks
  // ahead, so the id lookup and the row load do not follow each other on the critical path
  int tnext[2];
  if (PREFETCH && blk0 < blk1) {
    int t0[2];
    chunk_tokens(tokmap, blk0 * kBlk, t0);
    stats_load_tok<T, D>(X, inv_n, t0, cur);
    chunk_tokens(tokmap, min(blk0 + 1, blk1 - 1) * kBlk, tnext);
  }
  if (threadIdx.x < D) sh_shift[threadIdx.x] = sh_val;
  __syncthreads();
  for (int b = blk0; b < blk1; ++b) {
    if (!PREFETCH) stats_load<T, D>(X, tokmap, inv_n, b * kBlk, cur);
    stats_stage<T, D, kF16x2, kSymStride>(cur, sh_shift, ysc, st, dpart);
    __syncthreads();
    if (PREFETCH && b + 1 < blk1) {
      stats_load_tok<T, D>(X, inv_n, tnext, cur);
      chunk_tokens(tokmap, min(b + 2, blk1 - 1) * kBlk, tnext);
    }
    sym_mfma<D>(st, acc);
    __syncthreads();
  }
}

// Write wave W's tiles, times f, as the full symmetric matrix: out(r, c) at
// F[(c - c0) * ld + r] for the columns c in [c0, c0 + ncols) (every element exactly once).
template <int D, int W>
BSA_DEV void sym_store_wave(const SymAcc<D>& acc, float f, float* F, int ld, int c0, int ncols) {
  using P = SymPlan<D>;
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int t = 0; t < P::nt[W]; ++t) {
    const int a = P::a[W][t], b = P::b[W][t];
    const f32x4_t v = acc.t[t] * f;
    // tile element (16 a + 4 kg + i, 16 b + r16): as column 16 b + r16, rows 16 a + 4 kg + i
    const int cb = 16 * b + r16 - c0;
    if (16 * b >= c0 && 16 * b < c0 + ncols)
      *reinterpret_cast<f32x4_t*>(F + (size_t)cb * ld + 16 * a + 4 * kg) = v;
    // its mirror (16 b + r16, 16 a + 4 kg + i): column 16 a + 4 kg + i, row 16 b + r16
    if (a != b && 16 * a >= c0 && 16 * a < c0 + ncols) {
#pragma unroll
      for (int i = 0; i < 4; ++i) F[(size_t)(16 * a + 4 * kg + i - c0) * ld + 16 * b + r16] = v[i];
    }
  }
}
template <int D>
BSA_DEV void sym_store(const SymAcc<D>& acc, float f, float* F, int ld, int c0, int ncols) {
  switch (threadIdx.x >> 6) {
    case 0: sym_store_wave<D, 0>(acc, f, F, ld, c0, ncols); break;
    case 1: sym_store_wave<D, 1>(acc, f, F, ld, c0, ncols); break;
    case 2: sym_store_wave<D, 2>(acc, f, F, ld, c0, ncols); break;
    default: sym_store_wave<D, 3>(acc, f, F, ld, c0, ncols); break;
  }
}

// Position of element (row, col) in the register dump order of Cov<D> (store_acc / add_acc).
template <int D>
BSA_DEV int dump_index(int row, int col) {
  const int w = D == 128 ? (col >> 5) : 2 * (row >> 5) + (col >> 5);
  const int t = D == 128 ? (row >> 5) : 0;
  const int r = 4 * ((row >> 3) & 3) + (row & 3), lane = (col & 31) + 32 * ((row >> 2) & 1);
  return ((w * Cov<D>::TILES + t) * 16 + r) * 64 + lane;
}
// Wave W's tiles (times f) as the full symmetric matrix in that dump order.
template <int D, int W>
BSA_DEV void sym_store_dump_wave(const SymAcc<D>& acc, float f, float* dst) {
  using P = SymPlan<D>;
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int t = 0; t < P::nt[W]; ++t) {
    const int a = P::a[W][t], b = P::b[W][t];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = acc.t[t][i] * f;
      const int row = 16 * a + 4 * kg + i, col = 16 * b + r16;
      dst[dump_index<D>(row, col)] = v;
      if (a != b) dst[dump_index<D>(col, row)] = v;
    }
  }
}
template <int D>
BSA_DEV void sym_store_dump(const SymAcc<D>& acc, float f, float* dst) {
  switch (threadIdx.x >> 6) {
    case 0: sym_store_dump_wave<D, 0>(acc, f, dst); break;
    case 1: sym_store_dump_wave<D, 1>(acc, f, dst); break;
    case 2: sym_store_dump_wave<D, 2>(acc, f, dst); break;
    default: sym_store_dump_wave<D, 3>(acc, f, dst); break;
  }
}

// acc (register layout of Cov<D>) from a symmetric matrix stored by columns: element (r, c) at
// F[(c - c0) * ld + r]; only the registers whose column lies in [c0, c0 + ncols).  ADD sums
// into acc instead.
template <int D, bool ADD>
BSA_DEV void load_cols(f32x16_t* acc, const float* F, int ld, int c0, int ncols) {
#pragma unroll
  for (int t = 0; t < Cov<D>::TILES; ++t) {
    const int c = acc_col<D>(t);
    if (c < c0 || c >= c0 + ncols) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(F + (size_t)(c - c0) * ld + acc_row<D>(t, 4 * j));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][4 * j + i] = ADD ? acc[t][4 * j + i] + v[i] : v[i];
    }
  }
}

// Symmetric tiles (times f) into the register layout of Cov<D>, through the staging LDS in
// passes of 64 columns (stored by columns, D + 4 floats apart: conflict-free 16-byte reads).
template <int D>
BSA_DEV void sym_to_regs(const SymAcc<D>& sacc, float f, SymStage<D>& st, f32x16_t* acc) {
  constexpr int ld = D + 4;
  static_assert(64 * ld * 4 <= sizeof(SymStage<D>), "one pass fits the staging area");
  float* G = reinterpret_cast<float*>(&st);
  for (int c0 = 0; c0 < D; c0 += 64) {
    sym_store<D>(sacc, f, G, ld, c0, 64);
    __syncthreads();
    load_cols<D, false>(acc, G, ld, c0, 64);
    __syncthreads();
  }
}

// s += (lane K of this lane's row of 16 in v) * a: v_fmac_f32 with a DPP row broadcast of its
// first operand (fused, one rounding, as fmaf).  All lanes must be active.
template <int K>
BSA_DEV void fmac_row_bcast_k(float& s, float v, float a) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
      : "+v"(s)
      : "v"(v), "v"(a), "n"(K));
}
// (k is a constant wherever this is called in an unrolled loop; the switch then folds)
BSA_DEV void fmac_row_bcast(int k, float& s, float v, float a) {
  switch (k) {
    case 0: fmac_row_bcast_k<0>(s, v, a); break;
    case 1: fmac_row_bcast_k<1>(s, v, a); break;
    case 2: fmac_row_bcast_k<2>(s, v, a); break;
    case 3: fmac_row_bcast_k<3>(s, v, a); break;
    case 4: fmac_row_bcast_k<4>(s, v, a); break;
    case 5: fmac_row_bcast_k<5>(s, v, a); break;
    case 6: fmac_row_bcast_k<6>(s, v, a); break;
    case 7: fmac_row_bcast_k<7>(s, v, a); break;
    case 8: fmac_row_bcast_k<8>(s, v, a); break;
    case 9: fmac_row_bcast_k<9>(s, v, a); break;
    case 10: fmac_row_bcast_k<10>(s, v, a); break;
    case 11: fmac_row_bcast_k<11>(s, v, a); break;
    case 12: fmac_row_bcast_k<12>(s, v, a); break;
    case 13: fmac_row_bcast_k<13>(s, v, a); break;
    case 14: fmac_row_bcast_k<14>(s, v, a); break;
    default: fmac_row_bcast_k<15>(s, v, a); break;
  }
}

// out = vs * C v for the symmetric register-resident C (column form; v, out 16-byte aligned).
// red: AC*D floats of LDS (used when a wave does not hold whole columns).
template <int D>
BSA_DEV void cov_matvec(const f32x16_t* acc, const float* v, float vs, float* out, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if constexpr (Cov<D>::FULL_COLS) {
    // lane: column 32 w + lane % 32, rows 32 t + 8 j + 4 (lane / 32) + {0..3} of every tile t.
    // The 16 rows of tile t that a half-wave needs sit one per lane in each of its rows of 16
    // lanes (vt[t]); each product takes its factor by a DPP row broadcast.
    const int k = lane & 15;
    float vt[Cov<D>::TILES];
#pragma unroll
    for (int t = 0; t < Cov<D>::TILES; ++t)
      vt[t] = v[32 * t + 8 * (k >> 2) + 4 * (lane >> 5) + (k & 3)];
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < Cov<D>::TILES; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fmac_row_bcast(4 * j, s[j], vt[t], acc[t][4 * j]);
        fmac_row_bcast(4 * j + 1, s[j], vt[t], acc[t][4 * j + 1]);
        fmac_row_bcast(4 * j + 2, s[j], vt[t], acc[t][4 * j + 2]);
        fmac_row_bcast(4 * j + 3, s[j], vt[t], acc[t][4 * j + 3]);
      }
    }
    const float z = xor32_sum((s[0] + s[1]) + (s[2] + s[3]));
    if (lane < 32) out[32 * w + lane] = z * vs;
    __syncthreads();
  } else {
#pragma unroll
    for (int t = 0; t < Cov<D>::TILES; ++t) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s = fmaf(acc[t][r], v[acc_row<D>(t, r)], s);
      s = xor32_sum(s);
      if (lane < 32) red[Cov<D>::ac(w, t) * D + acc_col<D>(t)] = s;
    }
    __syncthreads();
    for (int b = threadIdx.x; b < D; b += 256) {
      float s = 0.f;
#pragma unroll
      for (int a = 0; a < Cov<D>::AC; ++a) s += red[a * D + b];
      out[b] = s * vs;
    }
    __syncthreads();
  }
}

// M held in registers.  D = 128: R = 2 threads per row, each with W = 64 columns; the threads
// of one row of 16 lanes share a column half, so that each product takes its factor of v by a
// DPP row broadcast: lane l of wave w owns row 32 w + 16 (l / 32) + l % 16 and columns
// [64 ((l / 16) % 2), +64).  D = 64: R = 4, thread t owns row t / 4, columns [(t % 4) 16, +16).
template <int D>
struct MRegs {
  static constexpr int R = 256 / D;
  static constexpr int W = D / R;
  float m[W];
  BSA_DEV static int row_of() {
    const int l = threadIdx.x & 63;
    return R == 2 ? 32 * (threadIdx.x >> 6) + 16 * (l >> 5) + (l & 15) : threadIdx.x / R;
  }
  BSA_DEV static int col0() {
    return R == 2 ? W * ((threadIdx.x >> 4) & 1) : (threadIdx.x % R) * W;
  }
  // the thread holding the first column half of a row
  BSA_DEV static bool row_owner() {
    return R == 2 ? ((threadIdx.x >> 4) & 1) == 0 : threadIdx.x % R == 0;
  }
  BSA_DEV void load(const float* M) {
    const int row = row_of(), c0 = col0();
#pragma unroll
    for (int i = 0; i < W; ++i) m[i] = M[row * D + c0 + i];
  }
  // (M v)[row] on every thread of the row's R lanes (v 16-byte aligned LDS)
  BSA_DEV float row_product(const float* v) const {
    const int c0 = col0();
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (R == 2) {
      // the 64 factors of this column half, 16 per register, one per lane of a row of 16
      const int k = threadIdx.x & 15;
      float u[W / 16];
#pragma unroll
      for (int q = 0; q < W / 16; ++q) u[q] = v[c0 + 16 * q + k];
#pragma unroll
      for (int i = 0; i < W; i += 4) {
        float& a = s[(i >> 2) & 3];
        fmac_row_bcast((i & 15), a, u[i >> 4], m[i]);
        fmac_row_bcast((i & 15) + 1, a, u[i >> 4], m[i + 1]);
        fmac_row_bcast((i & 15) + 2, a, u[i >> 4], m[i + 2]);
        fmac_row_bcast((i & 15) + 3, a, u[i >> 4], m[i + 3]);
      }
      // first column half + second, on both (rows of 16 lanes 2c and 2c + 1 exchanged)
      const float r = (s[0] + s[1]) + (s[2] + s[3]);
      const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(r), __float_as_uint(r),
                                                      false, false);
      return __uint_as_float(x[0]) + __uint_as_float(x[1]);
    } else {
#pragma unroll
      for (int i = 0; i < W; i += 4) {
        const float4 vv = *reinterpret_cast<const float4*>(v + c0 + i);
        float& a = s[(i >> 2) & 3];
        a = fmaf(m[i], vv.x, a);
        a = fmaf(m[i + 1], vv.y, a);
        a = fmaf(m[i + 2], vv.z, a);
        a = fmaf(m[i + 3], vv.w, a);
      }
      float r = (s[0] + s[1]) + (s[2] + s[3]);
      r += dpp_mov<0xB1>(r);  // lane ^ 1
      r += dpp_mov<0x4E>(r);  // lane ^ 2
      return r;
    }
  }
  BSA_DEV void matvec(const float* v, float* out) const {
    const float s = row_product(v);
    if (row_owner()) out[row_of()] = s;
    __syncthreads();
  }
  // out = M v, and returns v . out to every thread (sm: 4 floats of LDS).  One barrier.
  BSA_DEV float matvec_dot(const float* v, float* out, float* sm) const {
    const float s = row_product(v);
    float d = 0.f;
    if constexpr (R == 2) {
      // the terms s v[row] summed over the wave in the order of a layout with row 32 w + l / 2
      // on even lane l (and zero on odd lanes)
      const int l = threadIdx.x & 63, row = row_of();
      if (row_owner()) out[row] = s;
      const int r = l >> 1, src = 32 * (r >> 4) + (r & 15);
      const float sr = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(s)));
      if ((l & 1) == 0) d = sr * v[32 * (threadIdx.x >> 6) + r];
    } else {
      if (row_owner()) {
        const int row = row_of();
        out[row] = s;
        d = s * v[row];
      }
    }
    d = wave_total(d);
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = d;
    __syncthreads();
    return (sm[0] + sm[1]) + (sm[2] + sm[3]);
  }
};

// dot product of two LDS vectors, result broadcast to all threads.  sm: 4 floats.
template <int D>
BSA_DEV float block_dot(const float* a, const float* b, float* sm) {
  const int tid = threadIdx.x;
  float s = tid < D ? a[tid] * b[tid] : 0.f;
  s = wave_sum(s);
  if ((tid & 63) == 0) sm[tid >> 6] = s;
  __syncthreads();
  const float r = sm[0] + sm[1] + sm[2] + sm[3];
  __syncthreads();
  return r;
}

struct __align__(16) DirLds {
  float shift[128];
  float mu[128];
  float e0[128];
  float w[128];
  float z[128];
  float t[128];
  float red[4 * 128];
  float sm[8];
  int flag;
};

// Finish a group's statistics and find its split direction.  On entry acc holds
// sum (y - shift)(y - shift)^T over the group's n tokens and L.mu holds sum (y - shift).
// On exit L.w holds the direction w (zero for a group without spread) and L.mu the mean.
// Power step (w form): z = C_y w, t = M z, w <- t / sqrt(z . t); the normalisation is applied
// when the next step reads t.
// Centre the statistics: acc_scale * acc = sum (y - shift)(y - shift)^T and L.mu = sum (y - shift)
// over n tokens become the covariance C = acc_scale * acc / n - delta delta^T and the mean
// shift + delta.
template <int D>
BSA_DEV void finish_stats(f32x16_t* acc, DirLds& L, int n, float acc_scale) {
  const int tid = threadIdx.x;
  const float inv = 1.f / float(n), inv_acc = acc_scale * inv;
  if (tid < D) L.z[tid] = L.mu[tid] * inv;  // delta = mean - shift
  __syncthreads();
#pragma unroll
  for (int t = 0; t < Cov<D>::TILES; ++t) {
    const float zc = L.z[acc_col<D>(t)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 zr = *reinterpret_cast<const float4*>(&L.z[acc_row<D>(t, 4 * j)]);
      acc[t][4 * j] = acc[t][4 * j] * inv_acc - zr.x * zc;
      acc[t][4 * j + 1] = acc[t][4 * j + 1] * inv_acc - zr.y * zc;
      acc[t][4 * j + 2] = acc[t][4 * j + 2] * inv_acc - zr.z * zc;
      acc[t][4 * j + 3] = acc[t][4 * j + 3] * inv_acc - zr.w * zc;
    }
  }
  if (tid < D) L.mu[tid] = L.shift[tid] + L.z[tid];
  __syncthreads();
}

template <typename T, int D>
BSA_DEV void power_direction(f32x16_t* acc, DirLds& L, const MRegs<D>& M, int n,
                             const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                             const float* __restrict__ inv_n, int pos0, float y_first, int iters);

template <typename T, int D>
BSA_DEV void group_direction(f32x16_t* acc, DirLds& L, const MRegs<D>& M, int n, float acc_scale,
                             const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                             const float* __restrict__ inv_n, int pos0, float y_first,
                             int iters) {
  finish_stats<D>(acc, L, n, acc_scale);
  power_direction<T, D>(acc, L, M, n, X, tokmap, inv_n, pos0, y_first, iters);
}

// The scaled input y = x inv_n of token tokmap[pos] at element threadIdx.x (threads < D), for a
// caller that loads the first start candidate ahead of time.
template <typename T, int D>
BSA_DEV float first_candidate(const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                              const float* __restrict__ inv_n, int pos) {
  if (threadIdx.x >= D) return 0.f;
  const int tok = tokmap[pos];
  return load_as_f32(X + (size_t)tok * D + threadIdx.x) * inv_n[tok];
}

// Given the centred covariance in acc and the mean in L.mu, find the split direction L.w after
// `iters` power steps.  y_first: first_candidate(X, tokmap, inv_n, pos0) of the calling thread.
template <typename T, int D>
BSA_DEV void power_direction(f32x16_t* acc, DirLds& L, const MRegs<D>& M, int n,
                             const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                             const float* __restrict__ inv_n, int pos0, float y_first,
                             int iters) {
  const int tid = threadIdx.x;
  // start vector: the first position (smallest token id) whose centred vector is non-zero
  bool found = false;
  for (int p = pos0; p < pos0 + n; ++p) {
    float e = 0.f;
    if (tid < D) {
      const float y = p == pos0 ? y_first : first_candidate<T, D>(X, tokmap, inv_n, p);
      e = y - L.mu[tid];
      L.e0[tid] = e;
    }
    if (__syncthreads_or(e != 0.f)) {  // uniform: a workgroup-wide vote
      found = true;
      break;
    }
  }
  if (!found) {
    if (tid < D) L.w[tid] = 0.f;
    __syncthreads();
    return;
  }
  M.matvec(L.e0, L.t);
  float rn = 1.f;
  for (int it = 0; it < iters; ++it) {
    cov_matvec<D>(acc, L.t, rn, L.z, L.red);
    const float nrm2 = M.matvec_dot(L.z, L.t, L.sm);
    if (!(nrm2 > 0.f)) {
      if (tid < D) L.w[tid] = 0.f;
      __syncthreads();
      return;
    }
    rn = 1.f / sqrtf(nrm2);
  }
  if (tid < D) L.w[tid] = L.t[tid] * rn;
  __syncthreads();
  const float o = block_dot<D>(L.e0, L.w, L.sm);
  if (o < 0.f && tid < D) L.w[tid] = -L.w[tid];
  __syncthreads();
}

// x . w of one position from its four threads' quarter rows (raw: this thread's quarter, NV
// 16-byte pieces); the full sum on every thread of the four.
template <typename T, int D>
BSA_DEV float quarter_dot(const uint4* raw, const float* w) {
  constexpr int E = D / 4;                 // elements per quarter row
  constexpr int NV = E * sizeof(T) / 16;   // 16-byte pieces per quarter row
  const int q = threadIdx.x & 3;
  float xv[E];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t u[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
        xv[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      xv[4 * i] = __uint_as_float(raw[i].x);
      xv[4 * i + 1] = __uint_as_float(raw[i].y);
      xv[4 * i + 2] = __uint_as_float(raw[i].z);
      xv[4 * i + 3] = __uint_as_float(raw[i].w);
    }
  }
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) a = fmaf(xv[e], w[q * E + e], a);
  a += dpp_mov<0xB1>(a);  // lane ^ 1
  a += dpp_mov<0x4E>(a);  // lane ^ 2
  return a;
}

// Projections of the positions of blocks [blk0, blk1): key = inv_n * (x . w), 4 threads per
// position (a quarter row each); the loads of CH blocks are issued together.
template <typename T, int D, int CH = 4>
BSA_DEV void project_range(const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                           const float* __restrict__ inv_n, int blk0, int blk1, const float* w,
                           float* __restrict__ keys, float* __restrict__ proj_out) {
  constexpr int E = D / 4;                 // elements per quarter row
  constexpr int NV = E * sizeof(T) / 16;   // 16-byte pieces per quarter row
  const int tid = threadIdx.x, s = tid >> 2, q = tid & 3;
  for (int b = blk0; b < blk1; b += CH) {
    const int nbk = min(CH, blk1 - b);
    int tok[CH];
    uint4 raw[CH][NV];
    float sc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nbk) tok[c] = tokmap[(b + c) * kBlk + s];
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nbk) {
        const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)tok[c] * D + q * E);
#pragma unroll
        for (int i = 0; i < NV; ++i) raw[c][i] = src[i];
        sc[c] = inv_n[tok[c]];
      }
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (c < nbk) {
        const float a = quarter_dot<T, D>(raw[c], w);
        if (q == 0) {
          const float key = a * sc[c];
          keys[(b + c) * kBlk + s] = key;
          if (proj_out) proj_out[tok[c]] = key;
        }
      }
  }
}

// project_range with the token ids of up to 16 blocks read ahead into registers, so each
// chunk of row loads waits for one memory round trip instead of two (ids, then rows).
template <typename T, int D, int CH = 4>
BSA_DEV void project_range_ids(const T* __restrict__ X, const int32_t* __restrict__ tokmap,
                               const float* __restrict__ inv_n, int blk0, int blk1,
                               const float* w, float* __restrict__ keys,
                               float* __restrict__ proj_out, int key_blk0 = 0) {
  constexpr int E = D / 4;                 // elements per quarter row
  constexpr int NV = E * sizeof(T) / 16;   // 16-byte pieces per quarter row
  constexpr int IDS = 16;                  // blocks whose ids are read at once
  static_assert(IDS % CH == 0, "id groups hold whole chunks");
  const int tid = threadIdx.x, s = tid >> 2, q = tid & 3;
  for (int g0 = blk0; g0 < blk1; g0 += IDS) {
    const int ng = min(IDS, blk1 - g0);
    int ids[IDS];
#pragma unroll
    for (int c = 0; c < IDS; ++c)
      if (c < ng) ids[c] = tokmap[(g0 + c) * kBlk + s];
#pragma unroll
    for (int c0 = 0; c0 < IDS; c0 += CH) {
      if (c0 >= ng) break;
      uint4 raw[CH][NV];
      float sc[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c0 + c < ng) {
          const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)ids[c0 + c] * D + q * E);
#pragma unroll
          for (int i = 0; i < NV; ++i) raw[c][i] = src[i];
          sc[c] = inv_n[ids[c0 + c]];
        }
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (c0 + c < ng) {
          const float a = quarter_dot<T, D>(raw[c], w);
          if (q == 0) {
            const float key = a * sc[c];
            keys[(g0 + c0 + c - key_blk0) * kBlk + s] = key;
            if (proj_out) proj_out[ids[c0 + c]] = key;
          }
        }
    }
  }
}

struct ProblemArgs {
  const void* q;
  const void* k;
  int H, N, nb, L;
  const float* mom;        // [H][2][D][D]: side 0 = M_Q, side 1 = M_K
  const float* inv_n;      // [P][N]
  int32_t* perm_q;         // [H][N] positions of side 0 (query layouts), updated in place
  int32_t* perm_k;         // [H][N] positions of side 1 (key layouts)
  int32_t* tmp;            // [P][N] partition scratch
  float* keys;             // [P][N] projections by position
  float* mu;               // [P][2^L][D] group means, heap order (node (l, g) at 2^l - 1 + g)
  const float* mu_root;    // [P][D] mean of all y (the parent shift of level 0)
  const float* yscale;     // [P][2]: the power-of-two scale s of the fp16 split and 1 / s^2
  float* wdir;             // [P][G][D]
  float* partial;          // [P][kPartialSlots][D*D + D]
  const float* cov_prev;   // [P][Gw][D*D] centred covariances of the previous wide level
  float* cov_cur;          // [P][Gw][D*D] this level's, for the next level's right children
  int gw, left_only;
  const int* lists;        // [L][G] active (m >= 2) nodes per level, ascending
  float* proj;             // optional [H][2][L][N]
  int level, G, slices;
  // problems launched: p = p0 + pstep * (grid index); all 2H (0, 1), the query sides only
  // (0, 2) or the key sides only (1, 2)
  int p0, pstep;
  int iters;               // power steps per split
};

BSA_DEV int problem_of(const ProblemArgs& a, int b) { return a.p0 + a.pstep * b; }

// problem p = 2h + side; side 0 partitions the queries under M_K, side 1 the keys under M_Q
template <typename T, int D>
BSA_DEV const T* problem_x(const ProblemArgs& a, int p) {
  const T* base = static_cast<const T*>((p & 1) ? a.k : a.q);
  return base + (size_t)(p >> 1) * a.N * D;
}
template <int D>
BSA_DEV const float* problem_metric(const ProblemArgs& a, int p) {
  return a.mom + ((size_t)(p >> 1) * 2 + ((p & 1) ? 0 : 1)) * D * D;
}
BSA_DEV int32_t* problem_pos(const ProblemArgs& a, int p) {
  return ((p & 1) ? a.perm_k : a.perm_q) + (size_t)(p >> 1) * a.N;
}
BSA_DEV float* problem_proj(const ProblemArgs& a, int p, int level) {
  return a.proj ? a.proj + ((size_t)p * a.L + level) * a.N : nullptr;
}
template <int D>
BSA_DEV const float* parent_mean(const ProblemArgs& a, int p, int level, int g) {
  if (level == 0) return a.mu_root + (size_t)p * D;
  return a.mu + ((size_t)p * ((size_t)1 << a.L) + (1 << (level - 1)) - 1 + (g >> 1)) * D;
}
template <int D>
BSA_DEV float* group_mean(const ProblemArgs& a, int p, int level, int g) {
  return a.mu + ((size_t)p * ((size_t)1 << a.L) + (1 << level) - 1 + g) * D;
}

// Stable in-place two-way partition of one group's positions around (T, take).
BSA_DEV void partition_in_place(const float* keys, int32_t* pos, int32_t* tmp, int n, int want,
                                uint32_t T, int take, int* sm) {
  block_partition(keys, pos, tmp, n, want, T, take, sm);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256) pos[i] = tmp[i];
  __syncthreads();
}

// ------------------------------------------------------------------- second moments
template <typename T, int D>
__global__ __launch_bounds__(256) void k_moments(const T* __restrict__ q,
                                                 const T* __restrict__ k, int N, int side0,
                                                 float* __restrict__ partial) {
  constexpr int MODE = sizeof(T) == 4 ? kBf16x3 : kExact;
  __shared__ StageLds<D, split_terms<MODE>()> st;
  __shared__ float zero[D];
  // side = side0 + blockIdx.y: 0 = M_Q, 1 = M_K
  const int chunk = blockIdx.x, side = side0 + blockIdx.y, h = blockIdx.z, nch = gridDim.x;
  const T* X = (side ? k : q) + (size_t)h * N * D;
  if (threadIdx.x < D) zero[threadIdx.x] = 0.f;
  __syncthreads();
  f32x16_t acc[Cov<D>::TILES];
  zero_acc<D>(acc);
  float dpart[D / 8];
#pragma unroll
  for (int e = 0; e < D / 8; ++e) dpart[e] = 0.f;
  const int t1 = min(N, (chunk + 1) * kMomChunk);
  stats_range<T, D, MODE, true>(X, nullptr, nullptr, chunk * kMomChunk / kBlk, t1 / kBlk, zero,
                                1.f, st, acc, dpart);
  store_acc<D>(partial + (((size_t)h * 2 + side) * nch + chunk) * D * D, acc);
}

// One thread per matrix element: sum the partials in order, divide by N, write M canonical
// and (bf16 path) its 3-term bf16 split.  grid (D*D/256, 2, H).
template <int D>
__global__ __launch_bounds__(256) void k_moments_finish(const float* __restrict__ partial,
                                                        int nch, int N, int side0,
                                                        float* __restrict__ mom,
                                                        uint16_t* __restrict__ msplit) {
  const int e = blockIdx.x * 256 + threadIdx.x;  // register-dump index
  const int side = side0 + blockIdx.y, h = blockIdx.z;
  const size_t mi = (size_t)h * 2 + side;
  float s = 0.f;
  // (unrolled so that the loads are in flight together; the additions keep their order)
#pragma unroll 8
  for (int c = 0; c < nch; ++c) s += partial[(mi * nch + c) * D * D + e];
  const float m = s / float(N);
  // register-dump index -> (wave, tile, reg, lane) -> (a, b)
  const int lane = e & 63, r = (e >> 6) & 15, wt = e >> 10;
  const int w = wt / Cov<D>::TILES, t = wt % Cov<D>::TILES;
  const int ac = Cov<D>::ac(w, t), bc = Cov<D>::bc(w, t);
  const int a = 32 * ac + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), b = 32 * bc + (lane & 31);
  mom[mi * D * D + a * D + b] = m;
  if (msplit) {
    const uint16_t h1 = f32_to_bf16(m);
    const float r1 = m - bf16_to_f32(h1);
    const uint16_t h2 = f32_to_bf16(r1);
    const uint16_t h3 = f32_to_bf16(r1 - bf16_to_f32(h2));
    msplit[(mi * 3 + 0) * D * D + a * D + b] = h1;
    msplit[(mi * 3 + 1) * D * D + a * D + b] = h2;
    msplit[(mi * 3 + 2) * D * D + a * D + b] = h3;
  }
}

// ---------------------------------------------------------------- metric norms (bf16)
// inv_n[p][t] = 1 / sqrt(x_t^T M x_t) (0 if that is 0), per-workgroup sums of y = x inv_n and
// the per-workgroup max |y| (for the scale of the fp16 covariance split).
// The products by M run on MFMA with M in three bf16 terms held in registers (exact bf16
// inputs, fp32 sums).  The workgroup walks kNormTok tokens in tiles of 64 staged once in LDS
// (16-byte coalesced loads, the next tile's loads in flight while the current one is used).
constexpr int kNormTok = 512;
constexpr int kNormTile = 64;
constexpr int kNormStride = 136;  // bf16 per LDS row: 4-bank skew between rows
// x^T M x by symmetry: with M's 32 x 32 blocks M_ab, it is the sum over a <= b of
// x_a^T M'_ab x_b, M'_aa = M_aa and M'_ab = 2 M_ab for a < b: 10 of the 16 blocks, 20 of the
// 32 column chunks of 16.  The chunks are dealt five to a wave, so that each wave's chunks fall
// in at most two row blocks (NormPlan); a wave accumulates (M' x) for those rows and dots them
// with x.  Against all 16 blocks this is 30 MFMAs per wave and tile instead of 48, and at 168
// registers three workgroups fit per CU.
struct NormPlan {
  // unit u of wave w: row block a, column block b, chunk c (16 columns) within b
  static constexpr int a[4][5] = {{0, 0, 0, 0, 0}, {0, 0, 0, 1, 1}, {1, 1, 1, 1, 2}, {2, 2, 2, 3, 3}};
  static constexpr int b[4][5] = {{0, 0, 1, 1, 2}, {2, 3, 3, 1, 1}, {2, 2, 3, 3, 2}, {2, 3, 3, 3, 3}};
  static constexpr int c[4][5] = {{0, 1, 0, 1, 0}, {1, 0, 1, 0, 1}, {0, 1, 0, 1, 0}, {1, 0, 1, 0, 1}};
  // row block of accumulator slot s of wave w (-1: unused)
  static constexpr int slot_a[4][2] = {{0, -1}, {0, 1}, {1, 2}, {2, 3}};
};

template <int W>
BSA_DEV void norms_sym_body(const ProblemArgs& a, int p, int chunk, int nch,
                            const uint16_t* __restrict__ Ms, float* __restrict__ inv_n_out,
                            float* __restrict__ ysum, float* __restrict__ ymax,
                            uint16_t (*xs)[kNormStride], float (*red)[kNormTile], float* s_inv,
                            float (*s_ys)[128], float* s_max) {
  constexpr int D = 128;
  using P = NormPlan;
  constexpr int NS = P::slot_a[W][1] < 0 ? 1 : 2;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const uint16_t* X = problem_x<uint16_t, D>(a, p);
  // A operands: rows 32 a + l32 of M' (three bf16 terms), columns 32 b + 16 c + 8 g .. + 8
  bf16x8_t mreg[3][5];
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const uint16_t* src =
          Ms + (size_t)s * D * D + (32 * P::a[W][u] + l32) * D + 32 * P::b[W][u] + 16 * P::c[W][u] + 8 * g;
      bf16x8_t v = lds_bf16x8(src);
      if (P::a[W][u] < P::b[W][u]) {
        // times two: exact in bf16 (the exponent moves by one)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] * 2.f);
      }
      mreg[s][u] = v;
    }
  const int t0 = chunk * kNormTok, t_end = min(a.N, t0 + kNormTok);  // N is a multiple of 64
  const uint4* xv = reinterpret_cast<const uint4*>(X) + tid;
  uint4 n0 = xv[(size_t)t0 * 16], n1 = xv[(size_t)t0 * 16 + 256], n2 = xv[(size_t)t0 * 16 + 512],
        n3 = xv[(size_t)t0 * 16 + 768];
  const int d2 = lane;
  float ys0 = 0.f, ys1 = 0.f, ym = 0.f;
  for (int c0 = t0; c0 < t_end; c0 += kNormTile) {
    *reinterpret_cast<uint4*>(&xs[tid >> 4][8 * (tid & 15)]) = n0;
    *reinterpret_cast<uint4*>(&xs[(tid >> 4) + 16][8 * (tid & 15)]) = n1;
    *reinterpret_cast<uint4*>(&xs[(tid >> 4) + 32][8 * (tid & 15)]) = n2;
    *reinterpret_cast<uint4*>(&xs[(tid >> 4) + 48][8 * (tid & 15)]) = n3;
    __syncthreads();
    {
      const size_t cn = (size_t)(c0 + kNormTile < t_end ? c0 + kNormTile : c0) * 16;
      n0 = xv[cn];
      n1 = xv[cn + 256];
      n2 = xv[cn + 512];
      n3 = xv[cn + 768];
    }
    f32x16_t acc[NS][2];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[sl][h][r] = 0.f;
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int sl = (P::a[W][u] == P::slot_a[W][0]) ? 0 : 1;
      const int col = 32 * P::b[W][u] + 16 * P::c[W][u] + 8 * g;
      const bf16x8_t x0 = lds_bf16x8(&xs[l32][col]);
      const bf16x8_t x1 = lds_bf16x8(&xs[32 + l32][col]);
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        acc[sl][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mreg[s][u], x0, acc[sl][0], 0, 0, 0);
        acc[sl][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mreg[s][u], x1, acc[sl][1], 0, 0, 0);
      }
    }
    // lane holds (M' x_tok)[r] for r = 32 a + 8 j + 4 g + i, a the slot's row block
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tok = 32 * h + l32;
      float part = 0.f;
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const int ra = 32 * P::slot_a[W][sl];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 uu = *reinterpret_cast<const uint2*>(&xs[tok][ra + 8 * j + 4 * g]);
          part = fmaf(acc[sl][h][4 * j + 0], __uint_as_float(uu.x << 16), part);
          part = fmaf(acc[sl][h][4 * j + 1], __uint_as_float(uu.x & 0xFFFF0000u), part);
          part = fmaf(acc[sl][h][4 * j + 2], __uint_as_float(uu.y << 16), part);
          part = fmaf(acc[sl][h][4 * j + 3], __uint_as_float(uu.y & 0xFFFF0000u), part);
        }
      }
      part = xor32_sum(part);
      if (g == 0) red[W][tok] = part;
    }
    __syncthreads();
    if (tid < kNormTile) {
      const float n2v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
      const float inv = n2v > 0.f ? 1.f / sqrtf(n2v) : 0.f;
      s_inv[tid] = inv;
      inv_n_out[(size_t)p * a.N + c0 + tid] = inv;
    }
    __syncthreads();
#pragma unroll 4
    for (int t = 16 * W; t < 16 * W + 16; ++t) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(&xs[t][2 * d2]);
      const float sc = s_inv[t];
      const float y0 = __uint_as_float(u << 16) * sc, y1 = __uint_as_float(u & 0xFFFF0000u) * sc;
      ys0 += y0;
      ys1 += y1;
      ym = fmaxf(ym, fmaxf(fabsf(y0), fabsf(y1)));
    }
    __syncthreads();
  }
  s_ys[W][2 * d2] = ys0;
  s_ys[W][2 * d2 + 1] = ys1;
  ym = wave_max(ym);
  if (lane == 0) s_max[W] = ym;
  __syncthreads();
  if (tid < D)
    ysum[((size_t)p * nch + chunk) * D + tid] = (s_ys[0][tid] + s_ys[1][tid]) +
                                                (s_ys[2][tid] + s_ys[3][tid]);
  if (tid == 0)
    ymax[(size_t)p * nch + chunk] = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
}

__global__ __launch_bounds__(256, 3) void k_norms_bf16(ProblemArgs a, const uint16_t* __restrict__ msplit,
                                                    float* __restrict__ inv_n_out,
                                                    float* __restrict__ ysum,
                                                    float* __restrict__ ymax) {
  constexpr int D = 128;
  __shared__ __align__(16) uint16_t xs[kNormTile][kNormStride];
  __shared__ float red[4][kNormTile];
  __shared__ float s_inv[kNormTile];
  __shared__ float s_ys[4][D];
  __shared__ float s_max[4];
  const int chunk = blockIdx.x, p = problem_of(a, blockIdx.y), nch = gridDim.x;
  const int mi = (p >> 1) * 2 + ((p & 1) ? 0 : 1);
  const uint16_t* Ms = msplit + (size_t)mi * 3 * D * D;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: norms_sym_body<0>(a, p, chunk, nch, Ms, inv_n_out, ysum, ymax, xs, red, s_inv, s_ys, s_max); break;
    case 1: norms_sym_body<1>(a, p, chunk, nch, Ms, inv_n_out, ysum, ymax, xs, red, s_inv, s_ys, s_max); break;
    case 2: norms_sym_body<2>(a, p, chunk, nch, Ms, inv_n_out, ysum, ymax, xs, red, s_inv, s_ys, s_max); break;
    default: norms_sym_body<3>(a, p, chunk, nch, Ms, inv_n_out, ysum, ymax, xs, red, s_inv, s_ys, s_max); break;
  }
}
__global__ __launch_bounds__(256) void k_norms_f32(ProblemArgs a, float* __restrict__ inv_n_out,
                                                   float* __restrict__ ysum,
                                                   float* __restrict__ ymax) {
  constexpr int D = 64;
  __shared__ float sm[D][D + 1];
  __shared__ float sx[64][D + 1];
  __shared__ float s_inv[64];
  const int chunk = blockIdx.x, p = problem_of(a, blockIdx.y), nch = gridDim.x;
  const int tid = threadIdx.x, s = tid >> 2, q = tid & 3;
  const float* X = problem_x<float, D>(a, p);
  const float* M = problem_metric<D>(a, p);
  const int c0 = chunk * kBlk;
  for (int e = tid; e < D * D; e += 256) sm[e / D][e % D] = M[e];
  for (int e = tid; e < 64 * D; e += 256) sx[e / D][e % D] = X[(size_t)c0 * D + e];
  __syncthreads();
  float part = 0.f;
  for (int b = 16 * q; b < 16 * q + 16; ++b) {
    float y = 0.f;
    for (int c = 0; c < D; ++c) y = fmaf(sm[b][c], sx[s][c], y);
    part = fmaf(y, sx[s][b], part);
  }
  part += __shfl_xor(part, 1, 64);
  part += __shfl_xor(part, 2, 64);
  if (q == 0) {
    const float inv = part > 0.f ? 1.f / sqrtf(part) : 0.f;
    s_inv[s] = inv;
    inv_n_out[(size_t)p * a.N + c0 + s] = inv;
  }
  __syncthreads();
  float ym = 0.f;
  if (tid < D) {
    float acc = 0.f;
    for (int t = 0; t < 64; ++t) {
      acc = fmaf(sx[t][tid], s_inv[t], acc);
      ym = fmaxf(ym, fabsf(sx[t][tid] * s_inv[t]));
    }
    ysum[((size_t)p * nch + chunk) * D + tid] = acc;
  }
  ym = wave_max(ym);
  if (tid == 0) ymax[(size_t)p * nch + chunk] = ym;  // threads < D = 64 are wave 0
}

// mu_root[p] = (1/N) sum of the chunk sums
template <int D>
__global__ __launch_bounds__(256) void k_root_mean(const float* __restrict__ ysum,
                                                   const float* __restrict__ ymax, int nch, int N,
                                                   int p0, int pstep, float* __restrict__ mu_root,
                                                   float* __restrict__ yscale) {
  constexpr int R = 256 / D;  // chunk strides per element
  __shared__ float part[R][D];
  __shared__ float s_max[4];
  const int p = p0 + pstep * (int)blockIdx.x, d = threadIdx.x % D, r = threadIdx.x / D;
  float s = 0.f;
  // (unrolled so that the loads are in flight together; the additions keep their order)
#pragma unroll 8
  for (int c = r; c < nch; c += R) s += ysum[((size_t)p * nch + c) * D + d];
  part[r][d] = s;
  float m = 0.f;
  for (int c = threadIdx.x; c < nch; c += 256) m = fmaxf(m, ymax[(size_t)p * nch + c]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) t += part[i][threadIdx.x];
    mu_root[(size_t)p * D + threadIdx.x] = t / float(N);
  }
  if (threadIdx.x == 0) {
    // every centred value satisfies |y - shift| <= 2 max|y| <= 2^e; s = 2^(14 - e)
    const float mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    int e = 0;
    frexpf(2.f * mx, &e);
    e = max(-100, min(100, e));
    yscale[2 * p] = ldexpf(1.f, 14 - e);
    yscale[2 * p + 1] = ldexpf(1.f, 2 * (e - 14));
  }
}

// active-node lists: lists[l][0..count) = the nodes g of level l with m >= 2, ascending
__global__ __launch_bounds__(256) void k_group_lists(int nb, int G, int* __restrict__ lists) {
  __shared__ int sm[8];
  const int level = blockIdx.x, n = 1 << level;
  int run = 0;
  for (int base = 0; base < n; base += 256) {
    const int g = base + threadIdx.x;
    int b0, m;
    const int f = (g < n && group_geom(nb, level, g, b0, m) == kGroupSplit) ? 1 : 0;
    int tot;
    const int ex = block_excl_scan(f, sm, &tot);
    if (f) lists[(size_t)level * G + run + ex] = g;
    run += tot;
  }
}

// ---------------------------------------------------------------------- wide levels
// grid (slices, G, P): partial statistics of one slice of one group
template <typename T, int D>
__global__ __launch_bounds__(256, 3) void k_wide_stats(ProblemArgs a) {
  __shared__ SymStage<D> st;
  __shared__ float shift[D];
  __shared__ float red[4 * D];
  __shared__ float dsum[D];
  const int s = blockIdx.x, g = a.left_only ? 2 * blockIdx.y : blockIdx.y,
            p = problem_of(a, blockIdx.z);
  int b0, m;
  if (group_geom(a.nb, a.level, g, b0, m) != kGroupSplit) return;
  const int sb0 = b0 + (int)((long)s * m / a.slices), sb1 = b0 + (int)((long)(s + 1) * m / a.slices);
  const T* X = problem_x<T, D>(a, p);
  const int32_t* tokmap = problem_pos(a, p);
  const float* inv_n = a.inv_n + (size_t)p * a.N;
  const float shv = threadIdx.x < D ? parent_mean<D>(a, p, a.level, g)[threadIdx.x] : 0.f;
  SymAcc<D> acc;
  acc.zero();
  float dpart[D / 8];
#pragma unroll
  for (int e = 0; e < D / 8; ++e) dpart[e] = 0.f;
  sym_stats_range<T, D, true>(X, tokmap, inv_n, sb0, sb1, shift, shv, a.yscale[2 * p], st, acc,
                              dpart);
  reduce_dpart<D>(dpart, red, dsum);
  // the slot holds the full symmetric D x D sum (scaled by s^2) in register dump order, then the
  // D sums of d
  float* slot = a.partial + ((size_t)p * kPartialSlots + blockIdx.y * a.slices + s) * (D * D + D);
  sym_store_dump<D>(acc, 1.f, slot);
  if (threadIdx.x < D) slot[D * D + threadIdx.x] = dsum[threadIdx.x];
}

// grid (G, P) or, for left-only levels, (G/2, P): reduce the slices of a group and find its
// direction.  On left-only levels the statistics were accumulated for the left child only;
// the right child's follow from the parent's centred covariance C_P:
//   sum_R (y - mu_P)(y - mu_P)^T = n_P C_P - sum_L (y - mu_P)(y - mu_P)^T,
//   sum_R (y - mu_P) = -sum_L (y - mu_P).
// Each group's centred covariance is kept for the next level.
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_wide_dir(ProblemArgs a) {
  __shared__ DirLds L;
  const int p = problem_of(a, blockIdx.y);
  // left-only levels: workgroup 2 j + c handles child c of parent j (both children read the
  // left child's partial sums); otherwise workgroup g handles group g
  const int par = a.left_only ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;
  const int child = a.left_only ? (int)(blockIdx.x & 1) : 0;
  MRegs<D> M;
  M.load(problem_metric<D>(a, p));
  const T* X = problem_x<T, D>(a, p);
  const int32_t* pos = problem_pos(a, p);
  const float* inv_n = a.inv_n + (size_t)p * a.N;
  int pb0, pm;
  if (a.left_only) group_geom(a.nb, a.level - 1, par, pb0, pm);
  {
    const int g = a.left_only ? 2 * par + child : par;
    int b0, m;
    if (group_geom(a.nb, a.level, g, b0, m) != kGroupSplit) return;
    const float y_first = first_candidate<T, D>(X, pos, inv_n, b0 * kBlk);
    f32x16_t acc[Cov<D>::TILES];
    zero_acc<D>(acc);
    const float* base = a.partial + ((size_t)p * kPartialSlots + par * a.slices) * (D * D + D);
    float ds = 0.f;
    for (int s = 0; s < a.slices; ++s) {
      add_acc<D>(base + (size_t)s * (D * D + D), acc);
      if (threadIdx.x < D) ds += base[(size_t)s * (D * D + D) + D * D + threadIdx.x];
    }
    const float inv_s2 = a.yscale[2 * p + 1];
#pragma unroll
    for (int t = 0; t < Cov<D>::TILES; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] *= inv_s2;
    if (child == 1) {
      // right child: n_P C_P - S_L, and the negated sum
      const float* cp = a.cov_prev + ((size_t)p * a.gw + par) * D * D;
      const float np = float(pm * kBlk);
      const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
      for (int t = 0; t < Cov<D>::TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[t][r] = np * cp[((w * Cov<D>::TILES + t) * 16 + r) * 64 + lane] - acc[t][r];
      ds = -ds;
    }
    if (threadIdx.x < D) {
      L.mu[threadIdx.x] = ds;
      L.shift[threadIdx.x] = parent_mean<D>(a, p, a.level, g)[threadIdx.x];
    }
    __syncthreads();
    finish_stats<D>(acc, L, m * kBlk, 1.f);
    if (a.cov_cur) store_acc<D>(a.cov_cur + ((size_t)p * a.gw + g) * D * D, acc);
    power_direction<T, D>(acc, L, M, m * kBlk, X, pos, inv_n, b0 * kBlk, y_first,
                          a.iters);
    if (threadIdx.x < D) {
      group_mean<D>(a, p, a.level, g)[threadIdx.x] = L.mu[threadIdx.x];
      a.wdir[((size_t)p * a.G + g) * D + threadIdx.x] = L.w[threadIdx.x];
    }
    __syncthreads();
  }
}

// grid (nb, P): projections of one block's positions onto its group's direction
template <typename T, int D>
__global__ __launch_bounds__(256) void k_wide_proj(ProblemArgs a) {
  __shared__ float w[D];
  constexpr int E = D / 4, NV = E * sizeof(T) / 16;
  const int blk = blockIdx.x, p = problem_of(a, blockIdx.y);
  int b0, m;
  const int g = group_of_block(a.nb, a.level, blk, b0, m);
  if (g < 0 || m < 2) return;
  // as project_range over this one block, with the position's row and norm loads issued
  // before the direction's load and barrier
  const int s = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int tok = problem_pos(a, p)[blk * kBlk + s];
  const uint4* src = reinterpret_cast<const uint4*>(problem_x<T, D>(a, p) + (size_t)tok * D + q * E);
  uint4 raw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) raw[i] = src[i];
  const float sc = a.inv_n[(size_t)p * a.N + tok];
  if (threadIdx.x < D) w[threadIdx.x] = a.wdir[((size_t)p * a.G + g) * D + threadIdx.x];
  __syncthreads();
  const float d = quarter_dot<T, D>(raw, w);
  if (q == 0) {
    const float key = d * sc;
    a.keys[(size_t)p * a.N + blk * kBlk + s] = key;
    float* proj = problem_proj(a, p, a.level);
    if (proj) proj[tok] = key;
  }
}

// grid (G, P), 1024 threads: split threshold and stable in-place partition of one group
__global__ __launch_bounds__(1024) void k_wide_split(ProblemArgs a) {
  __shared__ int hist[16 * 256];
  __shared__ int sm[40];
  const int g = blockIdx.x, p = problem_of(a, blockIdx.y);
  int b0, m;
  if (group_geom(a.nb, a.level, g, b0, m) != kGroupSplit) return;
  const size_t off = (size_t)b0 * kBlk;
  const int n = m * kBlk, want = (m >> 1) * kBlk;
  const float* keys = a.keys + (size_t)p * a.N + off;
  int32_t* pos = problem_pos(a, p) + off;
  int32_t* tmp = a.tmp + (size_t)p * a.N + off;
  int take;
  // large groups: 8 keys (or 64-key steps) per thread in flight, so the passes over the keys in
  // global memory are not a chain of dependent loads
  const uint32_t T = select_smallest_w<1024, 8>(keys, n, want, hist, sm, &take);
  partition_w<1024, 8>(keys, pos, tmp, n, want, T, take, sm);
  for (int i = threadIdx.x; i < n; i += 1024) pos[i] = tmp[i];
}

// ------------------------------------------------------------------ subtree levels
// Split of one group from its raw statistics: acc holds s^2 sum (y - shift)(y - shift)^T times
// acc_scale = 1 / s^2 (or the sum itself with acc_scale 1), L.shift the shift and L.mu the sum
// of y - shift.  Centres the statistics, stores the centred covariance to cov_out (if given,
// for the children's right-child statistics), finds the direction, projects the group's
// positions and partitions them in place (stable, ascending token id within each side).
constexpr int kPairLdsKeys = 2048;  // keys of a pair-kernel group kept in LDS (8 KB)

template <typename T, int D>
BSA_DEV void split_group(const ProblemArgs& a, int p, int level, int g, int b0, int m,
                         f32x16_t* acc, float acc_scale, DirLds& L, float* cov_out, int* hist,
                         int* sm, float y_first, float* skeys) {
  const T* X = problem_x<T, D>(a, p);
  int32_t* pos = problem_pos(a, p);
  int32_t* tmp = a.tmp + (size_t)p * a.N;
  float* keys = a.keys + (size_t)p * a.N;
  const float* inv_n = a.inv_n + (size_t)p * a.N;
  const int n = m * kBlk;
  finish_stats<D>(acc, L, n, acc_scale);
  if (cov_out) store_acc<D>(cov_out, acc);
  {
    // M is read (from L2) for the power steps only, so it holds no registers elsewhere
    MRegs<D> M;
    M.load(problem_metric<D>(a, p));
    power_direction<T, D>(acc, L, M, n, X, pos, inv_n, b0 * kBlk, y_first, a.iters);
  }
  if (threadIdx.x < D) group_mean<D>(a, p, level, g)[threadIdx.x] = L.mu[threadIdx.x];
  const size_t off = (size_t)b0 * kBlk;
  // the group's keys stay in LDS when they fit (the select and the partition then read them
  // from there), else in global memory
  const bool in_lds = n <= kPairLdsKeys;
  float* kk = in_lds ? skeys : keys + off;
  project_range_ids<T, D>(X, pos, inv_n, b0, b0 + m, L.w, in_lds ? skeys : keys,
                          problem_proj(a, p, level), in_lds ? b0 : 0);
  __syncthreads();
  const int want = (m >> 1) * kBlk;
  int take;
  // keys in global memory: 4 per thread (or 64-key steps) in flight per pass
  const uint32_t T_ = select_smallest_w<256, 4>(kk, n, want, hist, sm, &take);
  partition_w<256, 4>(kk, pos + off, tmp + off, n, want, T_, take, sm);
  for (int i = threadIdx.x; i < n; i += 256) pos[off + i] = tmp[off + i];
  __syncthreads();
}

// grid (parents, P): one workgroup per active group gp of level - 1 (lists[level - 1]); it
// splits both children of gp at `level`.  Each child's statistics are accumulated from its own
// tokens: the left child's relative to the parent's mean, the right child's relative to its
// own mean, known from the left child's sum (sum_R (y - mu_P) = -sum_L (y - mu_P)).  (Deriving
// the right child as n_P C_P - S_L instead would carry the parent's fp32 rounding, amplified
// by n_P, into a child whose spread is small next to its distance from mu_P.)
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_subtree_pair(ProblemArgs a, int level) {
  __shared__ SymStage<D> st;
  __shared__ DirLds L;
  __shared__ float dsl[D];
  __shared__ int hist[4 * 256];
  __shared__ int sm[16];
  __shared__ float skeys[kPairLdsKeys];
  const int gp = a.lists[(size_t)(level - 1) * a.G + blockIdx.x], p = problem_of(a, blockIdx.y);
  int pb0, pm;
  group_geom(a.nb, level - 1, gp, pb0, pm);
  if (pm < 3) return;  // both children are leaves
  const int gl = 2 * gp, gr = 2 * gp + 1;
  int lb0, lm, rb0, rm;
  group_geom(a.nb, level, gl, lb0, lm);
  group_geom(a.nb, level, gr, rb0, rm);
  const T* X = problem_x<T, D>(a, p);
  const int32_t* pos = problem_pos(a, p);
  const float* inv_n = a.inv_n + (size_t)p * a.N;
  const float ysc = a.yscale[2 * p], inv_s2 = a.yscale[2 * p + 1];
  const float shv = threadIdx.x < D ? group_mean<D>(a, p, level - 1, gp)[threadIdx.x] : 0.f;
  const float yl = first_candidate<T, D>(X, pos, inv_n, lb0 * kBlk);
  const float yr = first_candidate<T, D>(X, pos, inv_n, rb0 * kBlk);
  f32x16_t acc[Cov<D>::TILES];
  {
    SymAcc<D> sacc;
    sacc.zero();
    float dpart[D / 8];
#pragma unroll
    for (int e = 0; e < D / 8; ++e) dpart[e] = 0.f;
    sym_stats_range<T, D, true>(X, pos, inv_n, lb0, lb0 + lm, L.shift, shv, ysc, st, sacc, dpart);
    reduce_dpart<D>(dpart, L.red, L.mu);
    sym_to_regs<D>(sacc, inv_s2, st, acc);  // S_L, unscaled
  }
  if (threadIdx.x < D) dsl[threadIdx.x] = L.mu[threadIdx.x];
  __syncthreads();
  if (lm >= 2)
    split_group<T, D>(a, p, level, gl, lb0, lm, acc, 1.f, L, nullptr, hist, sm, yl, skeys);
  if (rm >= 2) {
    const float shr =
        threadIdx.x < D ? shv - dsl[threadIdx.x] * (1.f / float(rm * kBlk)) : 0.f;
    SymAcc<D> sacc;
    sacc.zero();
    float dpart[D / 8];
#pragma unroll
    for (int e = 0; e < D / 8; ++e) dpart[e] = 0.f;
    sym_stats_range<T, D, true>(X, pos, inv_n, rb0, rb0 + rm, L.shift, shr, ysc, st, sacc, dpart);
    reduce_dpart<D>(dpart, L.red, L.mu);
    sym_to_regs<D>(sacc, inv_s2, st, acc);
    split_group<T, D>(a, p, level, gr, rb0, rm, acc, 1.f, L, nullptr, hist, sm, yr, skeys);
  }
}

// ------------------------------------------------------- two splits side by side
// The deep levels' groups are small, so a split is a chain of short dependent phases whose
// barriers and latencies, not their arithmetic, set its time.  The subtree kernel therefore
// takes two independent groups at a time: their statistics and directions one after the other
// (one covariance in registers at a time; the staging LDS is shared), then the projections,
// thresholds and partitions of both side by side, each half-workgroup finding its group's
// threshold with the ballot select (no barriers).  Each group's arithmetic is the one-group
// path's, in the same order, so the layouts are unchanged.

// One group of a pair: its positions, keys and partition scratch in LDS.
struct DuoGroup {
  int32_t* pos;
  float* keys;
  int32_t* tmp;
  int g, m;  // node index at the level, blocks
};

// centred-statistics accumulation of one group (positions pos[0 .. 64 m)) relative to shv:
// acc = sum (y - shv)(y - shv)^T (unscaled), L.mu = sum (y - shv), L.shift = shv
template <typename T, int D>
BSA_DEV void group_stats(const T* __restrict__ X, const int32_t* pos,
                         const float* __restrict__ inv_n, int m, DirLds& L, float shv, float ysc,
                         float inv_s2, SymStage<D>& st, f32x16_t* acc) {
  SymAcc<D> sacc;
  sacc.zero();
  float dpart[D / 8];
#pragma unroll
  for (int e = 0; e < D / 8; ++e) dpart[e] = 0.f;
  sym_stats_range<T, D, true>(X, pos, inv_n, 0, m, L.shift, shv, ysc, st, sacc, dpart);
  reduce_dpart<D>(dpart, L.red, L.mu);
  sym_to_regs<D>(sacc, inv_s2, st, acc);
}

// Statistics (relative to shv), centring and direction of one group whose positions are
// pos[0 .. 64 m): L.w, L.mu as in group_direction.
template <typename T, int D>
BSA_DEV void group_direction_small(const ProblemArgs& a, int p, const T* __restrict__ X,
                                   const int32_t* pos, const float* __restrict__ inv_n, int m,
                                   DirLds& L, float shv, float ysc, float inv_s2, float y_first,
                                   SymStage<D>& st) {
  f32x16_t acc[Cov<D>::TILES];
  group_stats<T, D>(X, pos, inv_n, m, L, shv, ysc, inv_s2, st, acc);
  // M is read (from L2) only for the power steps, so it holds no registers during the
  // statistics
  MRegs<D> M;
  M.load(problem_metric<D>(a, p));  // overlaps the centring
  group_direction<T, D>(acc, L, M, m * kBlk, 1.f, X, pos, inv_n, 0, y_first, a.iters);
}

// Split group A (and B if `two`) of `level`: statistics relative to the parent's mean, direction,
// projections (keys in LDS, optional output by token), the capacity cut and the stable
// partition of the positions in place.  Waves 0-1 select and partition A, waves 2-3 B.
template <typename T, int D, int KPL>
BSA_DEV void split_duo(const ProblemArgs& a, int p, int level, const DuoGroup& A,
                       const DuoGroup& B, bool two, SymStage<D>& st, DirLds* L, int* sm) {
  const int tid = threadIdx.x;
  const T* X = problem_x<T, D>(a, p);
  const float* inv_n = a.inv_n + (size_t)p * a.N;
  const float ysc = a.yscale[2 * p], inv_s2 = a.yscale[2 * p + 1];
  const int nA = A.m * kBlk, nB = two ? B.m * kBlk : 0;
  const float shA = tid < D ? parent_mean<D>(a, p, level, A.g)[tid] : 0.f;
  const float shB = two && tid < D ? parent_mean<D>(a, p, level, B.g)[tid] : 0.f;
  const float yA = first_candidate<T, D>(X, A.pos, inv_n, 0);
  const float yB = two ? first_candidate<T, D>(X, B.pos, inv_n, 0) : 0.f;
  // A's statistics and direction, then B's: one covariance in registers at a time
  group_direction_small<T, D>(a, p, X, A.pos, inv_n, A.m, L[0], shA, ysc, inv_s2, yA, st);
  if (two) group_direction_small<T, D>(a, p, X, B.pos, inv_n, B.m, L[1], shB, ysc, inv_s2, yB, st);
  if (tid < D) {
    group_mean<D>(a, p, level, A.g)[tid] = L[0].mu[tid];
    if (two) group_mean<D>(a, p, level, B.g)[tid] = L[1].mu[tid];
  }
  float* proj = problem_proj(a, p, level);
  project_range<T, D>(X, A.pos, inv_n, 0, A.m, L[0].w, A.keys, proj);
  if (two) project_range<T, D>(X, B.pos, inv_n, 0, B.m, L[1].w, B.keys, proj);
  __syncthreads();
  // each half-workgroup takes one group: both of its waves find the threshold (no barrier),
  // then partition together; a half without a group still meets the partition's barriers
  // (read as a wave-uniform value, so that the selects' per-register guards and the inactive
  // half's skips compile to scalar branches rather than per-lane masking)
  const int half = __builtin_amdgcn_readfirstlane(tid >> 7);
  const DuoGroup& S = half ? B : A;
  const bool active = half == 0 || two;
  const int n = active ? S.m * kBlk : 0, want = active ? (S.m >> 1) * kBlk : 0;
  int take = 0;
  const uint32_t cut = active ? wave_select_smallest<KPL>(S.keys, n, want, &take) : 0u;
  partition_waves<2>(S.keys, S.pos, S.tmp, n, want, cut, take, sm + 4 * half, (tid >> 6) & 1);
  for (int i = tid & 127; i < n; i += 128) S.pos[i] = S.tmp[i];
  __syncthreads();
}

// grid (ceil(roots / per), P): `per` (1 or 2) subtrees per workgroup, the active groups
// per x .. per x + per - 1 of level ls (roots of them in all), each of at most kSmallBlocks
// blocks, split down to level `stop` (exclusive) with their positions and keys in LDS.  At
// every level the splitting groups of the workgroup's subtrees are taken two at a time
// (split_duo).
constexpr int kSmallBlocks = 8;
constexpr int kSmallCap = kSmallBlocks * kBlk;
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_subtree_small(ProblemArgs a, int ls, int stop,
                                                          int roots, int per) {
  __shared__ SymStage<D> st;
  __shared__ DirLds L[2];
  __shared__ int32_t spos[2][kSmallCap];
  __shared__ int32_t stmp[2][kSmallCap];
  __shared__ float skeys[2][kSmallCap];
  __shared__ int sm[8];
  const int p = problem_of(a, blockIdx.y);
  const int nsub = min(per, roots - per * (int)blockIdx.x);
  int g0[2] = {0, 0}, rb0[2] = {0, 0}, rm[2] = {0, 0};
  for (int s = 0; s < nsub; ++s) {
    g0[s] = a.lists[(size_t)ls * a.G + per * blockIdx.x + s];
    group_geom(a.nb, ls, g0[s], rb0[s], rm[s]);
  }
  int32_t* pos = problem_pos(a, p);
  for (int s = 0; s < nsub; ++s)
    for (int i = threadIdx.x; i < rm[s] * kBlk; i += 256)
      spos[s][i] = pos[(size_t)rb0[s] * kBlk + i];
  __syncthreads();
  for (int level = ls; level < stop; ++level) {
    const int depth = level - ls;
    // cursor over this level's splitting groups: subtree cs, node cg (uniform)
    int cs = 0, cg = g0[0] << depth;
    auto next = [&](DuoGroup& r) {
      while (cs < nsub) {
        if (cg >= ((g0[cs] + 1) << depth)) {
          if (++cs < nsub) cg = g0[cs] << depth;
          continue;
        }
        const int g = cg++;
        int b0, m;
        if (group_geom(a.nb, level, g, b0, m) != kGroupSplit) continue;
        const int off = (b0 - rb0[cs]) * kBlk;
        r.pos = &spos[cs][off];
        r.keys = &skeys[cs][off];
        r.tmp = &stmp[cs][off];
        r.g = g;
        r.m = m;
        return true;
      }
      return false;
    };
    DuoGroup A{}, B{};  // (B stays empty when a level's count is odd)
    while (next(A)) {
      const bool two = next(B);
      split_duo<T, D, kSmallBlocks>(a, p, level, A, B, two, st, L, sm);
    }
  }
  for (int s = 0; s < nsub; ++s)
    for (int i = threadIdx.x; i < rm[s] * kBlk; i += 256)
      pos[(size_t)rb0[s] * kBlk + i] = spos[s][i];
}

// ------------------------------------------------------------- Lite: shared subtrees
// From the shared root level on, each group takes one direction (its own split) and its
// descendants keep cutting along those projections: the subtree is then its tokens in
// (projection, token id) order cut into 64-token leaves, each leaf in ascending token id.  So
// one workgroup per root group splits it (statistics, direction, projections) and sorts it.
constexpr int kMaxSharedBlocks = 64;  // blocks of the largest shared subtree (LDS capacity)
constexpr int kSharedCap = kMaxSharedBlocks * kBlk;

// the float whose orderable_key is u (-0.0 comes back as +0.0, which sorts equal to it)
BSA_DEV float key_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Bitonic sort in LDS over stages with subsequence lengths k = 2 .. kmax (a power of two): with
// n = kmax it sorts v[0..n) ascending; with n a multiple of kmax it sorts every aligned run of
// kmax entries ascending (the last merge of every run is ascending).
BSA_DEV void lds_bitonic(uint64_t* v, int n, int kmax) {
  for (int k = 2; k <= kmax; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += 256) {
        const int i = 2 * t - (t & (j - 1)), ip = i + j;
        const uint64_t x = v[i], y = v[ip];
        if ((x > y) == (k == kmax || (i & k) == 0)) {
          v[i] = y;
          v[ip] = x;
        }
      }
      __syncthreads();
    }
}

// grid (roots of level lr, P)
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void k_shared_subtree(ProblemArgs a, int lr) {
  constexpr size_t kRaw = sizeof(SymStage<D>) > kSharedCap * sizeof(uint64_t)
                              ? sizeof(SymStage<D>)
                              : kSharedCap * sizeof(uint64_t);
  // staging area of the statistics, afterwards the sort buffer
  __shared__ __align__(16) unsigned char sraw[kRaw];
  __shared__ DirLds L;
  __shared__ int32_t spos[kSharedCap];
  __shared__ float skeys[kSharedCap];
  SymStage<D>& st = *reinterpret_cast<SymStage<D>*>(sraw);
  uint64_t* sbuf = reinterpret_cast<uint64_t*>(sraw);
  const int g = a.lists[(size_t)lr * a.G + blockIdx.x], p = problem_of(a, blockIdx.y);
  int b0, m;
  group_geom(a.nb, lr, g, b0, m);
  const int n = m * kBlk;
  const T* X = problem_x<T, D>(a, p);
  int32_t* pos = problem_pos(a, p) + (size_t)b0 * kBlk;
  const float* inv_n = a.inv_n + (size_t)p * a.N;
  const float ysc = a.yscale[2 * p], inv_s2 = a.yscale[2 * p + 1];
  for (int i = threadIdx.x; i < n; i += 256) spos[i] = pos[i];
  __syncthreads();
  {
    // the root's own split: statistics relative to the parent's mean, direction, projections
    const float shv = threadIdx.x < D ? parent_mean<D>(a, p, lr, g)[threadIdx.x] : 0.f;
    const float y_first = first_candidate<T, D>(X, spos, inv_n, 0);
    f32x16_t acc[Cov<D>::TILES];
    MRegs<D> M;
    {
      SymAcc<D> sacc;
      sacc.zero();
      float dpart[D / 8];
#pragma unroll
      for (int e = 0; e < D / 8; ++e) dpart[e] = 0.f;
      sym_stats_range<T, D, true>(X, spos, inv_n, 0, m, L.shift, shv, ysc, st, sacc, dpart);
      reduce_dpart<D>(dpart, L.red, L.mu);
      sym_to_regs<D>(sacc, inv_s2, st, acc);
    }
    M.load(problem_metric<D>(a, p));
    group_direction<T, D>(acc, L, M, n, 1.f, X, spos, inv_n, 0, y_first, a.iters);
    if (threadIdx.x < D) group_mean<D>(a, p, lr, g)[threadIdx.x] = L.mu[threadIdx.x];
    project_range<T, D>(X, spos, inv_n, 0, m, L.w, skeys, problem_proj(a, p, lr));
    __syncthreads();
  }
  // sort by (projection, token id); positions hold ascending token ids, each below 2^19
  int n2 = kBlk;
  while (n2 < n) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256)
    sbuf[i] = i < n ? (uint64_t(orderable_key(skeys[i])) << 32) | uint32_t(spos[i]) : ~0ull;
  __syncthreads();
  lds_bitonic(sbuf, n2, n2);
  // the deeper levels' projections are the root's (where the token's group still splits)
  if (a.proj != nullptr)
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint64_t e = sbuf[i];
      const int tok = int(uint32_t(e));
      const float key = key_to_float(uint32_t(e >> 32));
      for (int level = lr + 1; level < a.L; ++level) {
        int gb0, gm;
        group_of_block(a.nb, level, b0 + i / kBlk, gb0, gm);
        if (gm >= 2) problem_proj(a, p, level)[tok] = key;
      }
    }
  __syncthreads();
  // leaves: consecutive runs of 64 in that order, each sorted by token id
  for (int i = threadIdx.x; i < n; i += 256) sbuf[i] = uint32_t(sbuf[i]);
  __syncthreads();
  lds_bitonic(sbuf, n, kBlk);
  for (int i = threadIdx.x; i < n; i += 256) pos[i] = int32_t(uint32_t(sbuf[i]));
}

// ------------------------------------------------------------------------- helpers
__global__ void k_fill_identity(int N, int32_t* __restrict__ out) {
  const size_t p = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256) out[p * N + i] = i;
}

// out[p][i] = in[p][i], grid (x, P)
__global__ void k_copy_i32(int N, const int32_t* __restrict__ in, int32_t* __restrict__ out) {
  const size_t p = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256)
    out[p * N + i] = in[p * N + i];
}

__global__ void k_fill_zero(size_t n, float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    out[i] = 0.f;
}

// keys[p][pos] = proj[p][level][in[p][pos]]
__global__ void k_gather_keys(int N, int L, int level, const float* __restrict__ proj,
                              const int32_t* __restrict__ in, float* __restrict__ keys) {
  const size_t p = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256)
    keys[p * N + i] = proj[(p * L + level) * N + in[p * N + i]];
}

struct RebLayout {
  size_t mom, mom_partial, msplit, inv_n, ysum, ymax, yscale, mu_root, tmp, keys, mu, wdir,
      partial, lists, cov0, cov1, total;
  int L, G, nch_mom, nch_n, gw;
};

size_t al(size_t x) { return (x + 255) & ~size_t(255); }

RebLayout reb_layout(int H, int N, int D) {
  RebLayout r{};
  const size_t P = 2 * (size_t)H, nb = N / kBlk;
  r.L = tree_levels((int)nb);
  r.G = r.L > 0 ? (1 << (r.L - 1)) : 1;
  r.nch_mom = ceil_div(N, kMomChunk);
  r.nch_n = D == 128 ? ceil_div(N, kNormTok) : (int)nb;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += al(bytes); return o; };
  r.mom = take((size_t)H * 2 * D * D * 4);
  r.mom_partial = take((size_t)H * 2 * r.nch_mom * D * D * 4);
  r.msplit = take((size_t)H * 2 * 3 * D * D * 2);
  r.inv_n = take(P * N * 4);
  r.ysum = take(P * r.nch_n * D * 4);
  r.ymax = take(P * r.nch_n * 4);
  r.yscale = take(P * 2 * 4);
  r.mu_root = take(P * D * 4);
  r.tmp = take(P * N * 4);
  r.keys = take(P * N * 4);
  r.mu = take(P * ((size_t)1 << r.L) * D * 4);
  r.wdir = take(P * r.G * D * 4);
  r.partial = take(P * kPartialSlots * (size_t)(D * D + D) * 4);
  r.lists = take((size_t)std::max(r.L, 1) * r.G * 4);
  // covariance slots per problem: the groups of the deepest wide level (the wide levels derive
  // each right child's statistics from its parent's centred covariance)
  int last = 0;
  for (int level = 0; level < r.L; ++level) {
    if (wide_slices(level, (int)nb) <= 1 || ceil_div((int)nb, 1 << level) <= kSmallBlocks) break;
    last = level;
  }
  r.gw = 1 << last;
  r.cov0 = take(P * r.gw * (size_t)D * D * 4);
  r.cov1 = take(P * r.gw * (size_t)D * D * 4);
  r.total = off;
  return r;
}

// the first level whose groups all hold at most `blocks` blocks
int shared_root_level(int nb, int blocks) {
  int level = 0;
  while (ceil_div(nb, 1 << level) > blocks) ++level;
  return level;
}

// number of active (m >= 2) nodes of a level
int active_count(int nb, int level) {
  int c = 0, b0, m;
  for (int g = 0; g < (1 << level); ++g) c += group_geom(nb, level, g, b0, m) == kGroupSplit;
  return c;
}

template <typename T, int D>
hipError_t run_reblock(const void* q, const void* k, int H, int N, int32_t* perm_q,
                       int32_t* perm_k, float* proj_opt, int sides, bool copy_q, int iters,
                       int shared_blocks, void* ws, hipStream_t s) {
  const RebLayout R = reb_layout(H, N, D);
  char* w = static_cast<char*>(ws);
  // sides: kSideQueries builds the query trees only (problems 2h, under M_K), kSideKeys the
  // key trees only (problems 2h + 1, under M_Q), kSideBoth all 2H; a one-sided run needs one
  // moment per head (M_K for the queries, M_Q for the keys).  copy_q: the query layouts are
  // copies of the key layouts afterwards.
  const bool both = sides == kSideBoth;
  const int P = both ? 2 * H : H, nb = N / kBlk, msides = both ? 2 : 1;
  const int mside0 = sides == kSideQueries ? 1 : 0;
  float* mom = reinterpret_cast<float*>(w + R.mom);
  uint16_t* msplit = sizeof(T) == 2 ? reinterpret_cast<uint16_t*>(w + R.msplit) : nullptr;
  k_moments<T, D><<<dim3(R.nch_mom, msides, H), 256, 0, s>>>(
      static_cast<const T*>(q), static_cast<const T*>(k), N, mside0,
      reinterpret_cast<float*>(w + R.mom_partial));
  k_moments_finish<D><<<dim3(D * D / 256, msides, H), 256, 0, s>>>(
      reinterpret_cast<float*>(w + R.mom_partial), R.nch_mom, N, mside0, mom, msplit);
  ProblemArgs a{};
  a.iters = iters;
  a.q = q;
  a.k = k;
  a.H = H;
  a.N = N;
  a.nb = nb;
  a.L = R.L;
  a.mom = mom;
  a.inv_n = reinterpret_cast<float*>(w + R.inv_n);
  a.perm_q = perm_q;
  a.perm_k = perm_k;
  a.tmp = reinterpret_cast<int32_t*>(w + R.tmp);
  a.keys = reinterpret_cast<float*>(w + R.keys);
  a.mu = reinterpret_cast<float*>(w + R.mu);
  a.mu_root = reinterpret_cast<float*>(w + R.mu_root);
  a.yscale = reinterpret_cast<float*>(w + R.yscale);
  a.wdir = reinterpret_cast<float*>(w + R.wdir);
  a.partial = reinterpret_cast<float*>(w + R.partial);
  a.lists = reinterpret_cast<int*>(w + R.lists);
  a.proj = proj_opt;
  a.gw = R.gw;
  a.G = R.G;
  a.p0 = sides == kSideKeys ? 1 : 0;
  a.pstep = both ? 1 : 2;
  float* ysum = reinterpret_cast<float*>(w + R.ysum);
  float* ymax = reinterpret_cast<float*>(w + R.ymax);
  if (sizeof(T) == 2)
    k_norms_bf16<<<dim3(R.nch_n, P), 256, 0, s>>>(a, msplit, reinterpret_cast<float*>(w + R.inv_n),
                                                  ysum, ymax);
  else
    k_norms_f32<<<dim3(R.nch_n, P), 256, 0, s>>>(a, reinterpret_cast<float*>(w + R.inv_n), ysum,
                                                 ymax);
  k_root_mean<D><<<P, 256, 0, s>>>(ysum, ymax, R.nch_n, N, a.p0, a.pstep,
                                   reinterpret_cast<float*>(w + R.mu_root),
                                   reinterpret_cast<float*>(w + R.yscale));
  if (proj_opt && R.L > 0) {
    const size_t n = (size_t)2 * H * R.L * N;
    k_fill_zero<<<(unsigned)std::min<size_t>((n + 255) / 256, 4096), 256, 0, s>>>(n, proj_opt);
  }
  const dim3 gridN(std::min(ceil_div(N, 256), 1024), H);
  if (sides & kSideQueries) k_fill_identity<<<gridN, 256, 0, s>>>(N, perm_q);
  if (sides & kSideKeys) k_fill_identity<<<gridN, 256, 0, s>>>(N, perm_k);
  if (R.L > 0) k_group_lists<<<R.L, 256, 0, s>>>(nb, R.G, reinterpret_cast<int*>(w + R.lists));
  // levels whose groups are large are split over several workgroups; below that one
  // workgroup per group, and from the first level whose groups fit in kSmallBlocks blocks,
  // one workgroup per subtree down to the leaves.  The Lite tree stops all of these at the
  // shared root level lr, where one workgroup per group splits it once and sorts it.
  const int lr = shared_blocks > 0 ? shared_root_level(nb, shared_blocks) : R.L;
  int level = 0;
  for (; level < R.L && level < lr; ++level) {
    const int slices = wide_slices(level, nb);
    if (slices <= 1 || ceil_div(nb, 1 << level) <= kSmallBlocks) break;
    a.level = level;
    a.slices = slices;
    const int G = 1 << level;
    a.left_only = level > 0 ? 1 : 0;
    a.cov_prev = reinterpret_cast<float*>(w + ((level & 1) ? R.cov0 : R.cov1));
    a.cov_cur = reinterpret_cast<float*>(w + ((level & 1) ? R.cov1 : R.cov0));
    const int Gs = a.left_only ? G / 2 : G;
    k_wide_stats<T, D><<<dim3(slices, Gs, P), 256, 0, s>>>(a);
    k_wide_dir<T, D><<<dim3(a.left_only ? 2 * Gs : Gs, P), 256, 0, s>>>(a);
    k_wide_proj<T, D><<<dim3(nb, P), 256, 0, s>>>(a);
    k_wide_split<<<dim3(G, P), 1024, 0, s>>>(a);
  }
  // narrow levels: one workgroup per parent, each child's statistics from its own tokens
  for (; level < R.L && level < lr; ++level) {
    const int roots = active_count(nb, level);
    if (roots == 0) continue;
    if (ceil_div(nb, 1 << level) <= kSmallBlocks) {
      // two subtrees per workgroup while that still leaves two rounds of workgroups for the
      // whole GPU (256 CUs x 2), else one (its groups are still taken two at a time)
      const int per = (long)ceil_div(roots, 2) * P >= 1024 ? 2 : 1;
      k_subtree_small<T, D><<<dim3(ceil_div(roots, per), P), 256, 0, s>>>(
          a, level, std::min(lr, R.L), roots, per);
      break;
    }
    k_subtree_pair<T, D><<<dim3(active_count(nb, level - 1), P), 256, 0, s>>>(a, level);
  }
  if (lr < R.L) {
    const int roots = active_count(nb, lr);
    if (roots > 0) k_shared_subtree<T, D><<<dim3(roots, P), 256, 0, s>>>(a, lr);
  }
  if (copy_q && perm_q != perm_k) k_copy_i32<<<gridN, 256, 0, s>>>(N, perm_k, perm_q);
  return hipGetLastError();
}

// ------------------------------------------------------- partition from given projections
// One workgroup per active group of a level, keys already gathered by position; in place.
__global__ __launch_bounds__(256) void k_split_level(int N, int nb, int level, int G,
                                                     const int* __restrict__ lists,
                                                     const float* __restrict__ keys,
                                                     int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ tmp) {
  __shared__ int hist[256];
  __shared__ int sm[8];
  const int g = lists[(size_t)level * G + blockIdx.x];
  const size_t p = blockIdx.y;
  int b0, m;
  group_geom(nb, level, g, b0, m);
  const size_t base = p * N + (size_t)b0 * kBlk;
  const int n = m * kBlk, want = (m >> 1) * kBlk;
  int take;
  const uint32_t T = block_select_smallest(keys + base, n, want, hist, sm, &take);
  partition_in_place(keys + base, pos + base, tmp + base, n, want, T, take, sm);
}

}  // namespace

size_t partition_ws_bytes(int P, int N) {
  const int nb = N / kBlk, L = tree_levels(nb), G = L > 0 ? 1 << (L - 1) : 1;
  return al(size_t(P) * N * 4) * 2 + al((size_t)std::max(L, 1) * G * 4);
}

hipError_t launch_partition_from_proj(int P, int N, const float* proj, int32_t* perm, void* ws,
                                      hipStream_t s) {
  const int nb = N / kBlk, L = tree_levels(nb), G = L > 0 ? 1 << (L - 1) : 1;
  char* w = static_cast<char*>(ws);
  int32_t* tmp = reinterpret_cast<int32_t*>(w);
  float* keys = reinterpret_cast<float*>(w + al(size_t(P) * N * 4));
  int* lists = reinterpret_cast<int*>(w + 2 * al(size_t(P) * N * 4));
  const dim3 grid_n(std::min(ceil_div(N, 256), 1024), P);
  k_fill_identity<<<grid_n, 256, 0, s>>>(N, perm);
  if (L > 0) k_group_lists<<<L, 256, 0, s>>>(nb, G, lists);
  for (int level = 0; level < L; ++level) {
    k_gather_keys<<<grid_n, 256, 0, s>>>(N, L, level, proj, perm, keys);
    const int roots = active_count(nb, level);
    if (roots > 0)
      k_split_level<<<dim3(roots, P), 256, 0, s>>>(N, nb, level, G, lists, keys, perm, tmp);
  }
  return hipGetLastError();
}

size_t reblock_ws_bytes(int H, int N, int D) { return reb_layout(H, N, D).total; }

hipError_t launch_reblock(bool bf16, const void* q, const void* k, int H, int N, int D,
                          int32_t* perm_q, int32_t* perm_k, float* proj_opt, int sides,
                          bool copy_q, int iters, int shared_blocks, void* ws, hipStream_t s) {
  if (bf16)
    return run_reblock<uint16_t, 128>(q, k, H, N, perm_q, perm_k, proj_opt, sides, copy_q,
                                      iters, shared_blocks, ws, s);
  return run_reblock<float, 64>(q, k, H, N, perm_q, perm_k, proj_opt, sides, copy_q, iters,
                                shared_blocks, ws, s);
}

}  // namespace bsa
