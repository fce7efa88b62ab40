// Reblock (stage 1): per-head second moments, Mahalanobis-cosine embedding and the
// capacity-constrained hierarchical tree partition into 64-token leaves.  See tree.h for the
// split rule and the layout invariants.
#include "common.h"
#include "internal.h"
#include "tree.h"

namespace bsa {
namespace {

__global__ void k_identity(int N, int32_t* __restrict__ out) {
  const size_t p = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256)
    out[p * N + i] = i;
}

// keys[p][pos] = proj[p][level][in[p][pos]]
__global__ void k_gather_keys(int N, int L, int level, const float* __restrict__ proj,
                              const int32_t* __restrict__ in, float* __restrict__ keys) {
  const size_t p = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256)
    keys[p * N + i] = proj[(p * L + level) * N + in[p * N + i]];
}

// One workgroup per (group, problem) of a level: select the split threshold over the group's
// keys (by position) and write the stable partition of the group's tokens.
__global__ __launch_bounds__(256) void k_split_level(int N, int nb, int level,
                                                     const float* __restrict__ keys,
                                                     const int32_t* __restrict__ in,
                                                     int32_t* __restrict__ out) {
  __shared__ int hist[256];
  __shared__ int sm[8];
  const int g = blockIdx.x;
  const size_t p = blockIdx.y;
  int b0, m;
  const int kind = group_geom(nb, level, g, b0, m);
  if (kind == kGroupNone) return;
  const size_t base = p * N + (size_t)b0 * kBlk;
  const int n = m * kBlk;
  if (kind == kGroupCopy) {
    for (int i = threadIdx.x; i < n; i += 256) out[base + i] = in[base + i];
    return;
  }
  const int want = (m >> 1) * kBlk;
  int take;
  const uint32_t T = block_select_smallest(keys + base, n, want, hist, sm, &take);
  block_partition(keys + base, in + base, out + base, n, want, T, take, sm);
}

}  // namespace

size_t partition_ws_bytes(int P, int N) { return size_t(P) * N * 8 + 512; }

hipError_t launch_partition_from_proj(int P, int N, const float* proj, int32_t* perm, void* ws,
                                      hipStream_t s) {
  const int nb = N / kBlk, L = tree_levels(nb);
  int32_t* tmp = static_cast<int32_t*>(ws);
  float* keys = reinterpret_cast<float*>(static_cast<char*>(ws) + size_t(P) * N * 4 + 256);
  int32_t* buf[2];
  buf[L & 1] = perm;
  buf[(L + 1) & 1] = tmp;
  const dim3 grid_n(ceil_div(N, 256) < 1024 ? ceil_div(N, 256) : 1024, P);
  k_identity<<<grid_n, 256, 0, s>>>(N, buf[0]);
  for (int level = 0; level < L; ++level) {
    k_gather_keys<<<grid_n, 256, 0, s>>>(N, L, level, proj, buf[level & 1], keys);
    k_split_level<<<dim3(1 << level, P), 256, 0, s>>>(N, nb, level, keys, buf[level & 1],
                                                      buf[(level + 1) & 1]);
  }
  return hipGetLastError();
}

size_t reblock_ws_bytes(int H, int N, int D) { return 256; }

hipError_t launch_reblock(bool bf16, const void* q, const void* k, int H, int N, int D,
                          int32_t* perm_q, int32_t* perm_k, float* proj_opt, void* ws,
                          hipStream_t s) {
  return hipErrorNotSupported;
}

}  // namespace bsa
