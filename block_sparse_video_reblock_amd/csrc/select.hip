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
__global__ __launch_bounds__(128) void k_block_means(const T* __restrict__ x,
                                                     const int32_t* __restrict__ perm, int N,
                                                     int D, float* __restrict__ means) {
  const int j = blockIdx.x, h = blockIdx.y, nb = gridDim.x, d = threadIdx.x;
  __shared__ int32_t rows[64];
  if (threadIdx.x < 64) rows[threadIdx.x] = perm[(size_t)h * N + (size_t)j * kBlk + threadIdx.x];
  __syncthreads();
  if (d >= D) return;
  float s = 0.f;
  for (int r = 0; r < 64; ++r) s += load_as_f32(x + ((size_t)h * N + rows[r]) * D + d);
  means[((size_t)h * nb + j) * D + d] = s * (1.f / 64.f);
}

// S[h][i][j] = scale * qm[h][i] . km[h][j]; 64 x 64 output tile per workgroup, 4 x 4 per thread,
// fp32 FMA in ascending d.
__global__ __launch_bounds__(256) void k_block_scores(const float* __restrict__ qm,
                                                      const float* __restrict__ km, int nb, int D,
                                                      float scale, float* __restrict__ S) {
  // one 64 x 64 tile of S per workgroup; wave w computes the 32 x 32 sub-tile (w / 2, w % 2)
  // with v_mfma_f32_32x32x2f32 (fp32 products and sums) over pairs of dimensions
  __shared__ float sq[64][129];
  __shared__ float sk[64][129];
  const int ti = blockIdx.x, tj = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < 64 * D; e += 256) {
    const int r = e / D, d = e - r * D;
    const int i = ti * 64 + r, j = tj * 64 + r;
    sq[r][d] = i < nb ? qm[((size_t)h * nb + i) * D + d] : 0.f;
    sk[r][d] = j < nb ? km[((size_t)h * nb + j) * D + d] : 0.f;
  }
  __syncthreads();
  const int wi = w >> 1, wj = w & 1;
  // A[i][k] = query mean 32 wi + i, dimension d + k; B[k][j] = key mean 32 wj + j, same
  const float* qa = &sq[32 * wi + (lane & 31)][lane >> 5];
  const float* kb = &sk[32 * wj + (lane & 31)][lane >> 5];
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int d = 0; d < D; d += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[d], kb[d], acc, 0, 0, 0);
  // lane holds S[32 wi + 8 (r/4) + 4 (lane/32) + r%4][32 wj + lane%32]
  const int j = tj * 64 + 32 * wj + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = ti * 64 + 32 * wi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (i < nb && j < nb) S[((size_t)h * nb + i) * nb + j] = acc[r] * scale;
  }
}

// One wave per row: MSB-first radix select (8-bit digits) of the k-th largest orderable key,
// then an ordered ballot pass that keeps every key above the threshold and the lowest-index
// keys equal to it.
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ scores, int rows, int nb,
                                              int k, int32_t* __restrict__ lists) {
  __shared__ int hist[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  const bool valid = row < rows;   // all waves keep to the same barrier sequence
  const float* srow = scores + (size_t)(valid ? row : 0) * nb;
  int* hw = hist[wave];
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hw[b] = 0;
    __syncthreads();
    for (int j = lane; valid && j < nb; j += 64) {
      const uint32_t key = orderable_key(srow[j]);
      if ((key & pmask) == prefix) atomicAdd(&hw[(key >> shift) & 255], 1);
    }
    __syncthreads();
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
    __syncthreads();
  }
  if (!valid) return;
  // prefix is the threshold key T; take every key > T and the `remaining` lowest-index keys == T
  int32_t* out = lists + (size_t)row * k;
  int taken = 0, eq_before = 0;
  for (int base = 0; base < nb; base += 64) {
    const int j = base + lane;
    const uint32_t key = j < nb ? orderable_key(srow[j]) : 0u;
    const bool eq = j < nb && key == prefix;
    const uint64_t eqm = __ballot(eq);
    const bool sel = j < nb && (key > prefix || (eq && eq_before + lanes_below(eqm) < remaining));
    const uint64_t selm = __ballot(sel);
    if (sel) out[taken + lanes_below(selm)] = j;
    taken += __popcll(selm);
    eq_before += __popcll(eqm);
  }
}

}  // namespace

hipError_t launch_block_means(bool bf16, const void* x, const int32_t* perm, int H, int N, int D,
                              float* means, hipStream_t s) {
  dim3 grid(N / kBlk, H);
  if (bf16)
    k_block_means<uint16_t><<<grid, 128, 0, s>>>(static_cast<const uint16_t*>(x), perm, N, D,
                                                 means);
  else
    k_block_means<float><<<grid, 128, 0, s>>>(static_cast<const float*>(x), perm, N, D, means);
  return hipGetLastError();
}

hipError_t launch_block_scores(const float* qm, const float* km, int H, int nb, int D,
                               float scale, float* scores, hipStream_t s) {
  dim3 grid(ceil_div(nb, 64), ceil_div(nb, 64), H);
  k_block_scores<<<grid, 256, 0, s>>>(qm, km, nb, D, scale, scores);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int rows, int nb, int k, int32_t* lists,
                       hipStream_t s) {
  k_topk<<<ceil_div(rows, 4), 256, 0, s>>>(scores, rows, nb, k, lists);
  return hipGetLastError();
}

}  // namespace bsa
