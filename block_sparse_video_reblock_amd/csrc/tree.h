// Capacity-constrained tree bookkeeping shared by the reblock kernels: group geometry,
// workgroup scans, the radix select of a split threshold and the stable two-way partition.
//
// [comfy.icu "MiniMax H3 Spark Attention (SM89)", "What it's doing under the hood"]: the tokens
// are split by a tree whose leaves each hold 64 tokens (a capacity limit).  Reading used here: a
// group of m blocks (m >= 2) sends the floor(m/2)*64 tokens of smallest (projection, token id)
// to its left child, the rest to the right; children are laid out left first, so every group
// of every level occupies one contiguous position range and the final leaf order is
// depth-first.  Inside a group positions always hold ascending token ids (the partition is
// stable and starts from the identity), so "lower token id" is "lower position".
#pragma once
#include "common.h"

namespace bsa {

enum GroupKind { kGroupNone = 0, kGroupCopy = 1, kGroupSplit = 2 };

// Node g of level `level` (g's bits, most significant first, are the left/right turns).
// Returns kGroupSplit for a group of m >= 2 blocks, kGroupCopy for a leaf that must be carried
// to the next level's buffer (reported once, by its leftmost descendant index), kGroupNone
// otherwise.
__host__ __device__ inline int group_geom(int nb, int level, int g, int& b0, int& m) {
  b0 = 0;
  m = nb;
  for (int l = level - 1; l >= 0; --l) {
    if (m < 2) return (g & ((2 << l) - 1)) == 0 ? kGroupCopy : kGroupNone;
    const int left = m >> 1;
    if ((g >> l) & 1) {
      b0 += left;
      m -= left;
    } else {
      m = left;
    }
  }
  return m >= 2 ? kGroupSplit : kGroupCopy;
}

// The group (at `level`) that contains block b, and its geometry.
__host__ __device__ inline int group_of_block(int nb, int level, int b, int& b0, int& m) {
  int g = 0;
  b0 = 0;
  m = nb;
  for (int l = 0; l < level; ++l) {
    if (m < 2) return -1;
    const int left = m >> 1;
    if (b >= b0 + left) {
      g = 2 * g + 1;
      b0 += left;
      m -= left;
    } else {
      g = 2 * g;
      m = left;
    }
  }
  return g;
}

__host__ __device__ inline int tree_levels(int nb) {
  int L = 0;
  while ((1 << L) < nb) ++L;
  return L;
}

// Exclusive scan of one int per thread over a 256-thread workgroup; returns the total in
// *total.  `sm` needs 4 ints of LDS.  Contains workgroup barriers.
BSA_DEV int block_excl_scan(int v, int* sm, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) sm[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int s = sm[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// Radix select over n keys (any address space): the threshold T such that the `want`
// smallest keys are all keys < T plus the first *take keys == T in index order.
// Needs 256 ints of LDS in `hist` and 6 in `sm`.  256-thread workgroup, contains barriers.
BSA_DEV uint32_t block_select_smallest(const float* keys, int n, int want, int* hist, int* sm,
                                       int* take) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int remaining = want;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint32_t key = orderable_key(keys[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    const int c = hist[tid];  // thread t owns bin t (ascending)
    int total;
    const int excl = block_excl_scan(c, sm, &total);
    // the digit is the bin where the running count first reaches `remaining`
    if (excl < remaining && excl + c >= remaining) {
      sm[4] = tid;
      sm[5] = excl;
    }
    __syncthreads();
    const int digit = sm[4];
    remaining -= sm[5];
    prefix |= uint32_t(digit) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  *take = remaining;
  return prefix;
}

// Stable two-way partition of the n entries in[0..n) by keys[0..n) around (T, take):
// entries with key < T, and the first `take` entries with key == T, go (in order) to
// out[0..want), the others (in order) to out[want..n).  Each thread handles one contiguous
// run of indices.  Needs 8 ints of LDS in `sm`.  Contains barriers.
BSA_DEV void block_partition(const float* keys, const int32_t* in, int32_t* out, int n,
                             int want, uint32_t T, int take, int* sm) {
  const int tid = threadIdx.x;
  const int run = (n + 255) / 256;
  const int i0 = min(n, tid * run), i1 = min(n, i0 + run);
  int c_lt = 0, c_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = orderable_key(keys[i]);
    c_lt += key < T;
    c_eq += key == T;
  }
  int tot;
  const int eq_before = block_excl_scan(c_eq, sm, &tot);
  const int eq_taken = max(0, min(take - eq_before, c_eq));
  const int left_before = block_excl_scan(c_lt + eq_taken, sm, &tot);
  int li = left_before, ri = want + (i0 - left_before), eq_seen = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = orderable_key(keys[i]);
    bool left = key < T;
    if (key == T) {
      left = eq_seen < take;
      ++eq_seen;
    }
    if (left)
      out[li++] = in[i];
    else
      out[ri++] = in[i];
  }
}

// ---------------------------------------------------------------------------------------
// Wave-parallel variants for any workgroup size NT (a multiple of 64).

// Radix select as above by the NW waves that call it with local wave indices 0 .. NW-1, with
// one private histogram per wave (less atomic contention) and coalesced reads.  hist: NW * 256
// ints of LDS; sm: 2 ints.  Its barriers are workgroup-wide: every thread of the workgroup must
// reach them (waves outside the NW may run another select between them).
// U keys per thread are loaded before any is counted (U loads in flight per thread).
template <int NW, int U = 1>
BSA_DEV uint32_t select_waves(const float* keys, int n, int want, int* hist, int* sm, int* take,
                              int wave) {
  constexpr int NT = NW * 64;
  const int lane = threadIdx.x & 63, ltid = wave * 64 + lane;
  uint32_t prefix = 0, pmask = 0;
  int remaining = want;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = ltid; b < NW * 256; b += NT) hist[b] = 0;
    __syncthreads();
    int* hw = hist + wave * 256;
    for (int i0 = ltid; i0 < n; i0 += U * NT) {
      uint32_t kk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) kk[u] = i0 + u * NT < n ? orderable_key(keys[i0 + u * NT]) : 0u;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * NT < n && (kk[u] & pmask) == prefix)
          atomicAdd(&hw[(kk[u] >> shift) & 255], 1);
    }
    __syncthreads();
    // merged into wave 0's histogram (each bin is read and written by one thread only)
    for (int b = ltid; b < 256; b += NT) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) c += hist[w * 256 + b];
      hist[b] = c;
    }
    __syncthreads();
    if (wave == 0) {
      // wave 0 scans the 256 bins: lane l owns bins 4l .. 4l+3
      int c[4], local = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[u] = hist[4 * lane + u];
        local += c[u];
      }
      int incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const uint64_t hit = __ballot(incl >= remaining);
      const int src = __ffsll((unsigned long long)hit) - 1;
      if (lane == src) {
        int run = incl - local;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (run + c[u] >= remaining) {
            sm[0] = 4 * lane + u;
            sm[1] = run;
            break;
          }
          run += c[u];
        }
      }
    }
    __syncthreads();
    const int digit = sm[0];
    remaining -= sm[1];
    prefix |= uint32_t(digit) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  *take = remaining;
  return prefix;
}

// select_waves by all NT / 64 waves of the workgroup; hist: NT/64 * 256 ints, sm: 2 ints
template <int NT, int U = 1>
BSA_DEV uint32_t select_smallest_w(const float* keys, int n, int want, int* hist, int* sm,
                                   int* take) {
  return select_waves<NT / 64, U>(keys, n, want, hist, sm, take, threadIdx.x >> 6);
}

// Stable two-way partition (same result as block_partition) by the NW waves that call it with
// local wave indices 0 .. NW-1.  Wave w streams one contiguous range of 64-element steps with
// coalesced loads; ballots give in-order ranks.  sm: 2*NW ints.  keys_out, if given, receives
// the keys in the partitioned order.  Two workgroup barriers, which every thread of the
// workgroup must reach (waves outside the NW may run another partition between them).
// U: 64-element steps whose loads are issued before the first of them is processed.
template <int NW, int U = 1>
BSA_DEV void partition_waves(const float* keys, const int32_t* in, int32_t* out, int n, int want,
                             uint32_t T, int take, int* sm, int wave, float* keys_out = nullptr) {
  const int lane = threadIdx.x & 63;
  const int steps = (n + 63) / 64;
  const int per = (steps + NW - 1) / NW;
  const int i0 = min(n, wave * per * 64), i1 = min(n, i0 + per * 64);
  int c_lt = 0, c_eq = 0;
  for (int b0 = i0; b0 < i1; b0 += 64 * U) {
    uint32_t kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = b0 + 64 * u + lane;
      kk[u] = i < i1 ? orderable_key(keys[i]) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = b0 + 64 * u + lane;
      c_lt += __popcll(__ballot(i < i1 && kk[u] < T));
      c_eq += __popcll(__ballot(i < i1 && kk[u] == T));
    }
  }
  if (lane == 0) {
    sm[wave] = c_lt;
    sm[NW + wave] = c_eq;
  }
  __syncthreads();
  int left_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    const int lt = sm[w], eq = sm[NW + w];
    left_before += lt + max(0, min(take - eq_before, eq));
    eq_before += eq;
  }
  int left_run = 0, eq_seen = eq_before;
  for (int b0 = i0; b0 < i1; b0 += 64 * U) {
    float kvs[U];
    int32_t ins[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = b0 + 64 * u + lane;
      kvs[u] = i < i1 ? keys[i] : 0.f;
      ins[u] = i < i1 ? in[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = b0 + 64 * u + lane;
      const bool ok = i < i1;
      const float kv = kvs[u];
      const uint32_t key = ok ? orderable_key(kv) : 0xFFFFFFFFu;
      const bool eq = ok && key == T;
      const uint64_t eqm = __ballot(eq);
      const bool left = ok && (key < T || (eq && eq_seen + lanes_below(eqm) < take));
      const uint64_t lm = __ballot(left);
      if (ok) {
        const int lb = left_before + left_run + lanes_below(lm);  // lefts before i
        const int dst = left ? lb : want + (i - lb);
        out[dst] = ins[u];
        if (keys_out != nullptr) keys_out[dst] = kv;
      }
      left_run += __popcll(lm);
      eq_seen += __popcll(eqm);
    }
  }
  __syncthreads();
}

// partition_waves by all NT / 64 waves of the workgroup
template <int NT, int U = 1>
BSA_DEV void partition_w(const float* keys, const int32_t* in, int32_t* out, int n, int want,
                         uint32_t T, int take, int* sm, float* keys_out = nullptr) {
  partition_waves<NT / 64, U>(keys, in, out, n, want, T, take, sm, threadIdx.x >> 6, keys_out);
}

// The threshold of select_smallest_w found by one wave alone, for n <= 64 * KPL keys held in
// its registers: T (the want-th smallest orderable key) is built bit by bit from the top, each
// bit decided by counting the keys below the candidate with ballots; take = want minus the
// keys below T.  No LDS and no barriers; any number of waves may run it at once.
template <int KPL>
BSA_DEV uint32_t wave_select_smallest(const float* keys, int n, int want, int* take) {
  const int lane = threadIdx.x & 63;
  uint32_t k[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int i = 64 * j + lane;
    // padding never counts: no candidate exceeds 0xFFFFFFFF
    k[j] = i < n ? orderable_key(keys[i]) : 0xFFFFFFFFu;
  }
  // (every register is counted: padding never falls below a candidate, and a count costs
  // less than a branch around it)
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    int below = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) below += __popcll(__ballot(k[j] < c));
    if (below < want) T = c;
  }
  int below = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) below += __popcll(__ballot(k[j] < T));
  *take = want - below;
  return T;
}

}  // namespace bsa
