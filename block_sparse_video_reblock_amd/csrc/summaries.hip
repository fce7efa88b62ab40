// Compressed-branch summaries (Spark-Reweight) and the block-swizzled K/V copies that feed the
// bf16 attention kernel.
//
// [comfyui-wiki.com "Spark-H3 ...", "What Spark-Attn changes" and its figure]: mean pooling
// puts exp(E[x]) where the attention needs E[exp(x)]; weighted summaries plus a log-mass bias
// restore the missing mass, scored against one anchor per head, the mean video query.  For key
// block j with anchor logits x_t = s qa.k_t:  w = softmax(x), kt_j = sum w_t k_t,
// vt_j = sum w_t v_t, b_j = logsumexp(x) - s qa.kt_j, so exp(s qa.kt_j + b_j) = sum_t exp(x_t).
// The fixed-block baseline (mean pooling) uses plain means and b_j = ln 64.
//
// Swizzled tile layouts (64 rows x 128 bf16 = 16 KiB, stored as 16 pieces x 64 lanes x 16 B,
// piece-major) match the MFMA operand registers of the attention kernel:
//   K layout, piece hh*8 + c, lane l: row 32hh + (l%32), elements 16c + 8(l/32) + 0..7
//   V layout, piece a*4 + c, lane l: element 32a + (l%32) of rows
//             16c + 4(l/32) + {0,1,2,3,8,9,10,11}
#include "common.h"
#include "internal.h"

namespace bsa {
namespace {

// V-layout row of slot t (0..7) for key chunk c and lane group g
BSA_DEV int vrow(int c, int g, int t) { return 16 * c + 8 * (t >> 2) + 4 * g + (t & 3); }

// ---------------------------------------------------------------- anchor: column means
template <typename T>
__global__ __launch_bounds__(256) void k_colsum(const T* __restrict__ x, int N, int D,
                                                float* __restrict__ partial) {
  // grid (chunks, H).  16 threads per row, each loading 16 bytes (E elements) of a row, 16 rows
  // per pass (D * sizeof(T) = 256 bytes for both supported shapes); per-thread column sums of
  // the chunk, then a fixed-order sum over the 16 row phases.
  constexpr int E = 16 / sizeof(T);
  const int chunk = blockIdx.x, h = blockIdx.y, nch = gridDim.x;
  const int c16 = threadIdx.x & 15, ph = threadIdx.x >> 4;
  const int t0 = chunk * kColChunk, t1 = min(N, t0 + kColChunk);
  __shared__ float red[16][129];
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int t = t0 + ph; t < t1; t += 16) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + ((size_t)h * N + t) * D + c16 * E);
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
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) s += red[p][threadIdx.x];
    partial[((size_t)h * nch + chunk) * D + threadIdx.x] = s;
  }
}

__global__ __launch_bounds__(256) void k_colsum_finish(const float* __restrict__ partial, int nch,
                                                       int N, int D, float* __restrict__ out) {
  // D columns x (256 / D) interleaved chunk strides, then a fixed-order sum of the strides
  __shared__ float red[256];
  const int h = blockIdx.x, R = 256 / D, d = threadIdx.x % D, r = threadIdx.x / D;
  float s = 0.f;
  for (int c = r; c < nch; c += R) s += partial[((size_t)h * nch + c) * D + d];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
    for (int i = 0; i < R; ++i) t += red[i * D + threadIdx.x];
    out[(size_t)h * D + threadIdx.x] = t / float(N);
  }
}

// ----------------------------------------------------------- per key block summaries
// grid (nb, H), 256 threads.  LDS holds the gathered block as fp32.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_summaries(
    const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ perm_k,
    const float* __restrict__ anchor, int N, float scale, int meanpool, float* __restrict__ kt,
    float* __restrict__ vt, float* __restrict__ bias, int ldb, uint4* __restrict__ ksw,
    uint4* __restrict__ vsw) {
  __shared__ float sk[64][D + 1];
  __shared__ float sv[64][D + 1];
  __shared__ float sw[64];
  __shared__ float sred[2][D];
  __shared__ float s_lse;
  const int j = blockIdx.x, h = blockIdx.y, nb = gridDim.x;
  const int tid = threadIdx.x;
  const int32_t* pk = perm_k + (size_t)h * N + (size_t)j * kBlk;
  for (int e = tid; e < 64 * D; e += 256) {
    const int r = e / D, d = e - r * D;
    const size_t src = ((size_t)h * N + pk[r]) * D + d;
    sk[r][d] = load_as_f32(k + src);
    sv[r][d] = load_as_f32(v + src);
  }
  __syncthreads();
  if (tid < 64) {
    float w;
    if (meanpool) {
      w = 1.f / 64.f;
      if (tid == 0) s_lse = logf(64.f);
    } else {
      const float* qa = anchor + (size_t)h * D;
      float x = 0.f;
      for (int d = 0; d < D; ++d) x = fmaf(qa[d], sk[tid][d], x);
      x *= scale;
      const float mx = wave_max(x);
      const float e = expf(x - mx);
      const float se = wave_sum(e);
      w = e / se;
      if (tid == 0) s_lse = mx + logf(se);
    }
    sw[tid] = w;
  }
  __syncthreads();
  // weighted sums: thread -> element d; rows 0..31 and 32..63 summed separately
  for (int e = tid; e < D; e += 256) {
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
    for (int r = 0; r < 32; ++r) {
      a0 = fmaf(sw[r], sk[r][e], a0);
      b0 = fmaf(sw[r], sv[r][e], b0);
      a1 = fmaf(sw[r + 32], sk[r + 32][e], a1);
      b1 = fmaf(sw[r + 32], sv[r + 32][e], b1);
    }
    const size_t dst = ((size_t)h * nb + j) * D + e;
    kt[dst] = a0 + a1;
    vt[dst] = b0 + b1;
    sred[0][e] = a0 + a1;
  }
  __syncthreads();
  if (tid < 64) {
    float b;
    if (meanpool) {
      b = s_lse;
    } else {
      const float* qa = anchor + (size_t)h * D;
      float x = 0.f;
      for (int d = tid; d < D; d += 64) x = fmaf(qa[d], sred[0][d], x);
      x = wave_sum(x);
      b = s_lse - scale * x;
    }
    if (tid == 0) bias[(size_t)h * ldb + j] = b;
  }
  // block-swizzled bf16 copies (bf16 path only)
  if (ksw != nullptr) {
    uint4* kdst = ksw + ((size_t)h * nb + j) * 1024;
    uint4* vdst = vsw + ((size_t)h * nb + j) * 1024;
    for (int u = tid; u < 1024; u += 256) {
      const int p = u >> 6, l = u & 63, g = l >> 5, l32 = l & 31;
      {  // K layout
        const int hh = p >> 3, c = p & 7;
        const float* src = &sk[32 * hh + l32][16 * c + 8 * g];
        uint4 o;
        o.x = pack_bf16x2(src[0], src[1]);
        o.y = pack_bf16x2(src[2], src[3]);
        o.z = pack_bf16x2(src[4], src[5]);
        o.w = pack_bf16x2(src[6], src[7]);
        kdst[u] = o;
      }
      {  // V layout
        const int a = p >> 2, c = p & 3, d = 32 * a + l32;
        uint4 o;
        o.x = pack_bf16x2(sv[vrow(c, g, 0)][d], sv[vrow(c, g, 1)][d]);
        o.y = pack_bf16x2(sv[vrow(c, g, 2)][d], sv[vrow(c, g, 3)][d]);
        o.z = pack_bf16x2(sv[vrow(c, g, 4)][d], sv[vrow(c, g, 5)][d]);
        o.w = pack_bf16x2(sv[vrow(c, g, 6)][d], sv[vrow(c, g, 7)][d]);
        vdst[u] = o;
      }
    }
  }
}


// bf16, D = 128: 16-byte gathers, bf16 tiles in LDS, K's swizzled copy written straight from the
// gathered registers (a K-layout piece is one 16-byte chunk of one row).  grid (nb, H).
__global__ __launch_bounds__(256) void k_summaries_bf16(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ perm_k, const float* __restrict__ anchor, int N, float scale,
    int meanpool, float* __restrict__ kt, float* __restrict__ vt, float* __restrict__ bias,
    int ldb, uint4* __restrict__ ksw, uint4* __restrict__ vsw) {
  constexpr int D = 128;
  __shared__ uint4 sk[64][17];  // row r: 16 chunks of 8 bf16 (+1 pad)
  __shared__ uint4 sv[64][17];
  __shared__ float sw[64];
  __shared__ float s_lse;
  __shared__ float sred[2][D];
  const int j = blockIdx.x, h = blockIdx.y, nb = gridDim.x;
  const int tid = threadIdx.x;
  const int32_t* pk = perm_k + (size_t)h * N + (size_t)j * kBlk;
  uint4* kdst = ksw ? ksw + ((size_t)h * nb + j) * 1024 : nullptr;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + 256 * u;  // chunk e: row e / 16, 16-byte column e % 16
    const int r = e >> 4, cj = e & 15;
    const size_t src = ((size_t)h * N + pk[r]) * (D / 8) + cj;
    const uint4 kv = reinterpret_cast<const uint4*>(k)[src];
    const uint4 vv = reinterpret_cast<const uint4*>(v)[src];
    sk[r][cj] = kv;
    sv[r][cj] = vv;
    if (kdst) {
      // K layout: piece (r/32)*8 + cj/2, lane (r%32) + 32*(cj%2)
      kdst[((r >> 5) * 8 + (cj >> 1)) * 64 + (r & 31) + 32 * (cj & 1)] = kv;
    }
  }
  __syncthreads();
  auto kel = [&](int r, int d) -> float {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(&sk[r][0]);
    return bf16_to_f32(row[d]);
  };
  auto vel = [&](int r, int d) -> float {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(&sv[r][0]);
    return bf16_to_f32(row[d]);
  };
  if (tid < 64) {
    float w;
    if (meanpool) {
      w = 1.f / 64.f;
      if (tid == 0) s_lse = logf(64.f);
    } else {
      const float* qa = anchor + (size_t)h * D;
      float x = 0.f;
      for (int d = 0; d < D; ++d) x = fmaf(qa[d], kel(tid, d), x);
      x *= scale;
      const float mx = wave_max(x);
      const float ex = expf(x - mx);
      const float se = wave_sum(ex);
      w = ex / se;
      if (tid == 0) s_lse = mx + logf(se);
    }
    sw[tid] = w;
  }
  __syncthreads();
  // weighted sums: thread -> (element d, half of the rows); halves combined in LDS
  {
    const int d = tid & (D - 1), half = tid >> 7;
    float a = 0.f, b = 0.f;
    for (int r = 32 * half; r < 32 * half + 32; ++r) {
      a = fmaf(sw[r], kel(r, d), a);
      b = fmaf(sw[r], vel(r, d), b);
    }
    if (half == 1) {
      sred[0][d] = a;
      sred[1][d] = b;
    }
    __syncthreads();
    if (half == 0) {
      a += sred[0][d];
      b += sred[1][d];
      const size_t dst = ((size_t)h * nb + j) * D + d;
      kt[dst] = a;
      vt[dst] = b;
    }
    __syncthreads();
    if (half == 0) sred[0][d] = a;
    __syncthreads();
  }
  if (tid < 64) {
    float b;
    if (meanpool) {
      b = s_lse;
    } else {
      const float* qa = anchor + (size_t)h * D;
      float x = 0.f;
      for (int d = tid; d < D; d += 64) x = fmaf(qa[d], sred[0][d], x);
      x = wave_sum(x);
      b = s_lse - scale * x;
    }
    if (tid == 0) bias[(size_t)h * ldb + j] = b;
  }
  if (vsw) {
    uint4* vdst = vsw + ((size_t)h * nb + j) * 1024;
    for (int u = tid; u < 1024; u += 256) {
      const int p = u >> 6, l = u & 63, g = l >> 5, l32 = l & 31;
      const int a = p >> 2, c = p & 3, d = 32 * a + l32;
      uint4 o;
      o.x = uint32_t(f32_to_bf16(vel(vrow(c, g, 0), d))) | (uint32_t(f32_to_bf16(vel(vrow(c, g, 1), d))) << 16);
      o.y = uint32_t(f32_to_bf16(vel(vrow(c, g, 2), d))) | (uint32_t(f32_to_bf16(vel(vrow(c, g, 3), d))) << 16);
      o.z = uint32_t(f32_to_bf16(vel(vrow(c, g, 4), d))) | (uint32_t(f32_to_bf16(vel(vrow(c, g, 5), d))) << 16);
      o.w = uint32_t(f32_to_bf16(vel(vrow(c, g, 6), d))) | (uint32_t(f32_to_bf16(vel(vrow(c, g, 7), d))) << 16);
      vdst[u] = o;
    }
  }
}

// --------------------------------- swizzled bf16 summary and context tiles (D = 128)
// Rows [H][nb][D] (fp32 summaries, or bf16 context keys / values) in 64-row tiles, rows past nb
// zero; with bias, padding rows get bias -inf.  grid (tiles, H), 256 threads
template <typename T>
__global__ __launch_bounds__(256) void k_summary_tiles(const T* __restrict__ kt,
                                                       const T* __restrict__ vt,
                                                       float* __restrict__ bias, int nb,
                                                       uint4* __restrict__ ktsw,
                                                       uint4* __restrict__ vtsw) {
  constexpr int D = 128;
  __shared__ float sk[64][D + 1];
  __shared__ float sv[64][D + 1];
  const int tau = blockIdx.x, h = blockIdx.y, ntiles = gridDim.x;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * D; e += 256) {
    const int r = e / D, d = e - r * D;
    const int row = tau * 64 + r;
    const bool ok = row < nb;
    sk[r][d] = ok ? load_as_f32(kt + ((size_t)h * nb + row) * D + d) : 0.f;
    sv[r][d] = ok ? load_as_f32(vt + ((size_t)h * nb + row) * D + d) : 0.f;
  }
  if (bias != nullptr && tid < 64 && tau * 64 + tid >= nb)
    bias[(size_t)h * ntiles * 64 + tau * 64 + tid] = -INFINITY;
  __syncthreads();
  uint4* kdst = ktsw + ((size_t)h * ntiles + tau) * 1024;
  uint4* vdst = vtsw + ((size_t)h * ntiles + tau) * 1024;
  for (int u = tid; u < 1024; u += 256) {
    const int p = u >> 6, l = u & 63, g = l >> 5, l32 = l & 31;
    {
      const int hh = p >> 3, c = p & 7;
      const float* src = &sk[32 * hh + l32][16 * c + 8 * g];
      uint4 o;
      o.x = pack_bf16x2(src[0], src[1]);
      o.y = pack_bf16x2(src[2], src[3]);
      o.z = pack_bf16x2(src[4], src[5]);
      o.w = pack_bf16x2(src[6], src[7]);
      kdst[u] = o;
    }
    {
      const int a = p >> 2, c = p & 3, d = 32 * a + l32;
      uint4 o;
      o.x = pack_bf16x2(sv[vrow(c, g, 0)][d], sv[vrow(c, g, 1)][d]);
      o.y = pack_bf16x2(sv[vrow(c, g, 2)][d], sv[vrow(c, g, 3)][d]);
      o.z = pack_bf16x2(sv[vrow(c, g, 4)][d], sv[vrow(c, g, 5)][d]);
      o.w = pack_bf16x2(sv[vrow(c, g, 6)][d], sv[vrow(c, g, 7)][d]);
      vdst[u] = o;
    }
  }
}

}  // namespace

hipError_t launch_anchor(bool bf16, const void* x, int H, int N, int D, float* partial,
                         float* anchor, hipStream_t s) {
  const int nch = ceil_div(N, kColChunk);
  dim3 grid(nch, H);
  if (bf16)
    k_colsum<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), N, D, partial);
  else
    k_colsum<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), N, D, partial);
  k_colsum_finish<<<H, 256, 0, s>>>(partial, nch, N, D, anchor);
  return hipGetLastError();
}

hipError_t launch_summaries(bool bf16, const void* k, const void* v, const int32_t* perm_k,
                            const float* anchor, int H, int N, int D, float scale, bool meanpool,
                            float* kt, float* vt, float* bias, int ldb, void* ksw, void* vsw,
                            hipStream_t s) {
  dim3 grid(N / kBlk, H);
  if (bf16)
    k_summaries_bf16<<<grid, 256, 0, s>>>(
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), perm_k, anchor, N,
        scale, meanpool ? 1 : 0, kt, vt, bias, ldb, static_cast<uint4*>(ksw),
        static_cast<uint4*>(vsw));
  else
    k_summaries<float, 64><<<grid, 256, 0, s>>>(
        static_cast<const float*>(k), static_cast<const float*>(v), perm_k, anchor, N, scale,
        meanpool ? 1 : 0, kt, vt, bias, ldb, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_summary_tiles(const float* kt, const float* vt, float* bias, int H, int nb,
                                void* ktsw, void* vtsw, hipStream_t s) {
  dim3 grid(summary_tiles(nb), H);
  k_summary_tiles<float><<<grid, 256, 0, s>>>(kt, vt, bias, nb, static_cast<uint4*>(ktsw),
                                              static_cast<uint4*>(vtsw));
  return hipGetLastError();
}

hipError_t launch_ctx_tiles(const void* k_ctx, const void* v_ctx, int H, int n_ctx, void* ctsw,
                            void* cvsw, hipStream_t s) {
  dim3 grid(ceil_div(n_ctx, 64), H);
  k_summary_tiles<uint16_t><<<grid, 256, 0, s>>>(
      static_cast<const uint16_t*>(k_ctx), static_cast<const uint16_t*>(v_ctx), nullptr, n_ctx,
      static_cast<uint4*>(ctsw), static_cast<uint4*>(cvsw));
  return hipGetLastError();
}

}  // namespace bsa
