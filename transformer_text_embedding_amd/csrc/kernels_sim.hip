// Cosine-similarity matrix of unit vectors (the -sim example of the tensai
// "テキスト埋め込み" page, introduction).
#include "common.h"
#include "kernels.h"

namespace tte {

namespace {

// Similarity matrix of the page's -sim example (introduction): with unit
// vectors the cosine of two texts is their dot product, sim = E E^T.  One
// wave per 16 x 16 output tile on v_mfma_f32_16x16x4_f32: over each 16-wide
// K chunk a lane reads a float4 of its A row and of its B row and feeds one
// element of each per MFMA (both operands in the same k order).  Rows past
// n are clamped for the loads and never stored.
__global__ __launch_bounds__(64) void k_sim(const float* __restrict__ e, int n, int dim, float* __restrict__ sim) {
  const int lane = threadIdx.x, g = lane >> 4, li = lane & 15;
  const int i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const float* a = e + (size_t)min(i0 + li, n - 1) * dim + 4 * g;
  const float* b = e + (size_t)min(j0 + li, n - 1) * dim + 4 * g;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < dim; k += 16) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(a + k);
    const f32x4 bv = *reinterpret_cast<const f32x4*>(b + k);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
  }
  // lane holds rows 4g + r of column li of the tile
  const int j = j0 + li;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * g + r;
    if (i < n && j < n) sim[(size_t)i * n + j] = acc[r];
  }
}

}  // namespace

void launch_similarity(const float* e, int n, int dim, float* sim, hipStream_t s) {
  if (n <= 0) return;
  const dim3 grid((n + 15) / 16, (n + 15) / 16);
  k_sim<<<grid, 64, 0, s>>>(e, n, dim, sim);
}

}  // namespace tte
