// Fixed-tile layout for gfx950: the positional baseline that Reblock replaces.
//
// [comfyui-wiki.com "Spark-H3 ...", "What Spark-Attn changes"]: Spark-Reblock takes the place
// of fixed spatiotemporal tiles; [comfy.icu "MiniMax H3 Spark Attention (SM89)", "What it's
// doing under the hood"]: its recall is measured against fixed blocks.
//
// The latent grid (T, H, W), token id (t H + y) W + x, is cut into tt x th x tw cubes of 64
// tokens.  Position p holds: cube p / 64 (cubes in raster order of their corner), token p % 64
// of it (raster order inside the cube).  One thread per position; a pure index map.
#include "common.h"
#include "internal.h"

namespace bsa {
namespace {

__global__ void k_tile_layout(int T, int H, int W, int tt, int th, int tw, int32_t* __restrict__ perm) {
  const int N = T * H * W;
  const size_t head = blockIdx.y;
  const int cubes_y = H / th, cubes_x = W / tw;
  for (int p = blockIdx.x * 256 + threadIdx.x; p < N; p += gridDim.x * 256) {
    const int cube = p / kBlk, r = p - cube * kBlk;
    const int cx = cube % cubes_x, cy = (cube / cubes_x) % cubes_y, ct = cube / (cubes_x * cubes_y);
    const int x = r % tw, y = (r / tw) % th, t = r / (tw * th);
    perm[head * N + p] = ((ct * tt + t) * H + cy * th + y) * W + cx * tw + x;
  }
}

}  // namespace

hipError_t launch_tile_layout(int heads, int T, int H, int W, int tt, int th, int tw,
                              int32_t* perm, hipStream_t s) {
  const int N = T * H * W;
  const dim3 grid(std::min(ceil_div(N, 256), 1024), heads);
  k_tile_layout<<<grid, 256, 0, s>>>(T, H, W, tt, th, tw, perm);
  return hipGetLastError();
}

}  // namespace bsa
