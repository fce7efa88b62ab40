// Block scoring and per-query-block top-K selection.
//
// [comfy.icu "MiniMax H3 Spark Attention (SM89)", "Inputs you'll actually set"]: topk_ratio sets
// the exact branch's budget (0.2 default, 0.1 fastest, 0.3 most faithful); topk_blocks is the
// fixed-count alternative.  [comfyui-wiki.com "Spark-H3 ...", "What Spark-Attn changes"]: the
// exact branch fully computes the top-ranked key/value blocks.  Block score (plain reading):
// S_ij = s * mean(query block i) . mean(key block j); per row the K largest, ties to the lower
// block index, listed ascending.
#include "common.h"
#include "internal.h"

namespace bsa {
namespace {

// grid (nb, H); thread -> element d.  Means in a fixed summation order.
template <typename T>
__global__ __launch_bounds__(256) void k_block_means(const T* __restrict__ x,
                                                     const int32_t* __restrict__ perm, int N,
                                                     int D, float* __restrict__ means) {
  // 16 threads per row, each summing 16 bytes (E elements) of 4 of the block's 64 rows; then a
  // fixed-order sum over the 16 row phases (D * sizeof(T) = 256 bytes for both shapes)
  constexpr int E = 16 / sizeof(T);
  const int j = blockIdx.x, h = blockIdx.y, nb = gridDim.x;
  const int c16 = threadIdx.x & 15, ph = threadIdx.x >> 4;
  __shared__ int32_t rows[64];
  __shared__ float red[16][129];
  if (threadIdx.x < 64) rows[threadIdx.x] = perm[(size_t)h * N + (size_t)j * kBlk + threadIdx.x];
  __syncthreads();
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = 16 * p + ph;
    const uint4 u = *reinterpret_cast<const uint4*>(x + ((size_t)h * N + rows[r]) * D + c16 * E);
    if constexpr (sizeof(T) == 2) {
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += __uint_as_float(wv[i] << 16);
        acc[2 * i + 1] += __uint_as_float(wv[i] & 0xFFFF0000u);
      }
    } else {
      acc[0] += __uint_as_float(u.x);
      acc[1] += __uint_as_float(u.y);
      acc[2] += __uint_as_float(u.z);
      acc[3] += __uint_as_float(u.w);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[ph][c16 * E + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) t += red[q][threadIdx.x];
    means[((size_t)h * nb + j) * D + threadIdx.x] = t * (1.f / 64.f);
  }
}

// S[h][i][j] = scale * qm[h][i] . km[h][j].
// One 128 x 128 tile of S per workgroup; wave w computes the 64 x 64 quarter (w / 2, w % 2) as
// four 32 x 32 sub-tiles with v_mfma_f32_32x32x2f32 (fp32 products and sums) over pairs of
// dimensions.  The dimensions are staged 64 at a time (two passes for D = 128); every
// element's products are accumulated in the same order as over the whole row.
constexpr int kScoreTile = 128, kScoreChunk = 64;
template <int D>
__global__ __launch_bounds__(256) void k_block_scores(const float* __restrict__ qm,
                                                      const float* __restrict__ km, int nb,
                                                      float scale, float* __restrict__ S) {
  // rows padded to 68 floats: 16-byte aligned for the tile stores, and the MFMA operand reads
  // (lane: row lane % 32, column lane / 32) fall into 2-way bank groups
  __shared__ __align__(16) float sq[kScoreTile][kScoreChunk + 4];
  __shared__ __align__(16) float sk[kScoreTile][kScoreChunk + 4];
  const int ti = blockIdx.x, tj = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi = w >> 1, wj = w & 1;
  constexpr int V = kScoreChunk / 4;  // float4 per staged row
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  for (int d0 = 0; d0 < D; d0 += kScoreChunk) {
    if (d0 > 0) __syncthreads();  // the previous chunk's operands have been read
#pragma unroll
    for (int e = tid; e < kScoreTile * V; e += 256) {
      const int r = e / V, c = e % V;
      // rows past nb read row nb - 1 (valid memory) and are zeroed after the load
      const int i = ti * kScoreTile + r, j = tj * kScoreTile + r;
      float4 a4 = reinterpret_cast<const float4*>(qm + ((size_t)h * nb + min(i, nb - 1)) * D +
                                                  d0)[c];
      float4 b4 = reinterpret_cast<const float4*>(km + ((size_t)h * nb + min(j, nb - 1)) * D +
                                                  d0)[c];
      if (i >= nb) a4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j >= nb) b4 = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&sq[r][4 * c]) = a4;
      *reinterpret_cast<float4*>(&sk[r][4 * c]) = b4;
    }
    __syncthreads();
    // A[i][k] = query mean 64 wi + 32 a + i, dimension d0 + d + k; B[k][j] likewise for keys
#pragma unroll 4
    for (int d = 0; d < kScoreChunk; d += 2) {
      float qa[2], kb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        qa[a] = sq[64 * wi + 32 * a + (lane & 31)][d + (lane >> 5)];
        kb[a] = sk[64 * wj + 32 * a + (lane & 31)][d + (lane >> 5)];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[a], kb[b], acc[a][b], 0, 0, 0);
    }
  }
  // lane holds S[row0 + 8 (r/4) + 4 (lane/32) + r%4][col0 + lane%32] of sub-tile (a, b)
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = tj * kScoreTile + 64 * wj + 32 * b + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = ti * kScoreTile + 64 * wi + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (i < nb && j < nb) S[((size_t)h * nb + i) * nb + j] = acc[a][b][r] * scale;
      }
    }
}

// One wave per row: MSB-first radix select (8-bit digits) of the k-th largest orderable key,
// then an ordered ballot pass that keeps every key above the threshold and the lowest-index
// keys equal to it.  The waves of a workgroup work on separate rows and separate histograms,
// so they never synchronise with each other (LDS operations of one wave complete in order).
// Rows of up to 64 * kTopkRegs keys are read once into registers; longer rows are re-read from
// memory in every pass.
constexpr int kTopkRegs = 32;

template <bool CACHED>
__device__ __forceinline__ void topk_row(const float* __restrict__ srow, int nb, int k,
                                         int* __restrict__ hw, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  uint32_t kc[CACHED ? kTopkRegs : 1];
  if (CACHED) {
#pragma unroll
    for (int u = 0; u < kTopkRegs; ++u) {
      const int j = lane + 64 * u;
      kc[u] = j < nb ? orderable_key(srow[j]) : 0u;
    }
  }
  // key of column lane + 64 u (u < ceil(nb / 64)); only called for columns < nb
  auto key_at = [&](int u) { return CACHED ? kc[u] : orderable_key(srow[lane + 64 * u]); };
  const int nu = (nb + 63) >> 6;
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hw[b] = 0;
    __builtin_amdgcn_wave_barrier();
    if (CACHED) {
#pragma unroll
      for (int u = 0; u < kTopkRegs; ++u) {
        const int j = lane + 64 * u;
        if (j < nb && (kc[u] & pmask) == prefix) atomicAdd(&hw[(kc[u] >> shift) & 255], 1);
      }
    } else {
      for (int u = 0; u < nu; ++u) {
        const int j = lane + 64 * u;
        if (j < nb) {
          const uint32_t key = key_at(u);
          if ((key & pmask) == prefix) atomicAdd(&hw[(key >> shift) & 255], 1);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lane l owns bins 255-4l .. 252-4l (descending); inclusive scan of counts from the top
    int c[4], local = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = hw[255 - 4 * lane - u];
      local += c[u];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const int excl = incl - local;
    // the digit is in the first lane whose inclusive count reaches `remaining`
    const uint64_t hit = __ballot(incl >= remaining);
    const int src = __ffsll((unsigned long long)hit) - 1;
    int digit = 0, above = 0;
    if (lane == src) {
      int run = excl;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (run + c[u] >= remaining) {
          digit = 255 - 4 * lane - u;
          above = run;
          break;
        }
        run += c[u];
      }
    }
    digit = __shfl(digit, src, 64);
    above = __shfl(above, src, 64);
    remaining -= above;
    prefix |= uint32_t(digit) << shift;
    pmask |= 255u << shift;
    __builtin_amdgcn_wave_barrier();  // the histogram reads above precede the next clearing
  }
  // prefix is the threshold key T; take every key > T and the `remaining` lowest-index keys == T
  int taken = 0, eq_before = 0;
  auto emit = [&](int u) {
    const int j = lane + 64 * u;
    const uint32_t key = j < nb ? key_at(u) : 0u;
    const bool eq = j < nb && key == prefix;
    const uint64_t eqm = __ballot(eq);
    const bool sel = j < nb && (key > prefix || (eq && eq_before + lanes_below(eqm) < remaining));
    const uint64_t selm = __ballot(sel);
    if (sel) out[taken + lanes_below(selm)] = j;
    taken += __popcll(selm);
    eq_before += __popcll(eqm);
  };
  if (CACHED) {
#pragma unroll
    for (int u = 0; u < kTopkRegs; ++u)
      if (u < nu) emit(u);
  } else {
    for (int u = 0; u < nu; ++u) emit(u);
  }
}

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ scores, int rows, int nb,
                                              int k, int32_t* __restrict__ lists) {
  __shared__ int hist[4][256];
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const float* srow = scores + (size_t)row * nb;
  int32_t* out = lists + (size_t)row * k;
  if (nb <= 64 * kTopkRegs)
    topk_row<true>(srow, nb, k, hist[wave], out);
  else
    topk_row<false>(srow, nb, k, hist[wave], out);
}

// ------------------------------------------------------------------ list validation
// result[0] = rows whose list is malformed (an entry outside [0, nb) or not strictly above its
// predecessor), result[1] = the smallest such row or -1.  Reads the lists only.
__global__ void k_check_lists_init(int32_t* __restrict__ result) {
  if (threadIdx.x == 0) {
    result[0] = 0;
    result[1] = INT32_MAX;
  }
}

// one wave per row: lane e checks entries e, e + 64, ... against their predecessors
__global__ __launch_bounds__(256) void k_check_lists(const int32_t* __restrict__ lists, int rows,
                                                     int nb, int k, int32_t* __restrict__ result) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int32_t* l = lists + (size_t)row * k;
  bool bad = false;
  for (int e = lane; e < k; e += 64) {
    const int32_t v = l[e];
    bad |= v < 0 || v >= nb || (e > 0 && v <= l[e - 1]);
  }
  if (__any(bad) && lane == 0) {
    atomicAdd(&result[0], 1);
    atomicMin(&result[1], row);
  }
}

__global__ void k_check_lists_finish(int32_t* __restrict__ result) {
  if (threadIdx.x == 0 && result[0] == 0) result[1] = -1;
}

}  // namespace

hipError_t launch_block_means(bool bf16, const void* x, const int32_t* perm, int H, int N, int D,
                              float* means, hipStream_t s) {
  dim3 grid(N / kBlk, H);
  if (bf16)
    k_block_means<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), perm, N, D,
                                                 means);
  else
    k_block_means<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), perm, N, D, means);
  return hipGetLastError();
}

hipError_t launch_block_scores(const float* qm, const float* km, int H, int nb, int D,
                               float scale, float* scores, hipStream_t s) {
  dim3 grid(ceil_div(nb, kScoreTile), ceil_div(nb, kScoreTile), H);
  if (D == 128)
    k_block_scores<128><<<grid, 256, 0, s>>>(qm, km, nb, scale, scores);
  else
    k_block_scores<64><<<grid, 256, 0, s>>>(qm, km, nb, scale, scores);
  return hipGetLastError();
}

hipError_t launch_check_lists(const int32_t* lists, int rows, int nb, int k, int32_t* result,
                              hipStream_t s) {
  k_check_lists_init<<<1, 64, 0, s>>>(result);
  k_check_lists<<<ceil_div(rows, 4), 256, 0, s>>>(lists, rows, nb, k, result);
  k_check_lists_finish<<<1, 64, 0, s>>>(result);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int rows, int nb, int k, int32_t* lists,
                       hipStream_t s) {
  k_topk<<<ceil_div(rows, 4), 256, 0, s>>>(scores, rows, nb, k, lists);
  return hipGetLastError();
}

}  // namespace bsa
