// mb_reduce.hip -- the atomic-free second pass of the gradient reductions, a
// zero fill, and the tiling plan every kernel shares.
//
// The first pass of a backward op leaves R partial rows of fp32 sums; here
// out[c] = sum_{r = 0..R-1} in[r, c] in ascending r, so the result does not
// depend on scheduling (bit-reproducible).
#include <algorithm>

#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ in, int R, int64_t C,
                                                     float* __restrict__ out) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= C) return;
  const float* p = in + c;
  float s = 0.0f;
  int r = 0;
  for (; r + 4 <= R; r += 4) {
    const float v0 = p[static_cast<size_t>(r) * C];
    const float v1 = p[static_cast<size_t>(r + 1) * C];
    const float v2 = p[static_cast<size_t>(r + 2) * C];
    const float v3 = p[static_cast<size_t>(r + 3) * C];
    s = (((s + v0) + v1) + v2) + v3;
  }
  for (; r < R; ++r) s += p[static_cast<size_t>(r) * C];
  out[c] = s;
}

// out[y, c] = sum of in[r, c] for r in [32 y, min(R, 32 y + 32)), ascending
__global__ __launch_bounds__(256) void colsum_chunk_kernel(const float* __restrict__ in, int R, int64_t C,
                                                           float* __restrict__ out) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= C) return;
  const int r0 = static_cast<int>(blockIdx.y) * 32, r1 = r0 + 32 < R ? r0 + 32 : R;
  const float* p = in + c;
  float s = 0.0f;
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    const float v0 = p[static_cast<size_t>(r) * C];
    const float v1 = p[static_cast<size_t>(r + 1) * C];
    const float v2 = p[static_cast<size_t>(r + 2) * C];
    const float v3 = p[static_cast<size_t>(r + 3) * C];
    s = (((s + v0) + v1) + v2) + v3;
  }
  for (; r < r1; ++r) s += p[static_cast<size_t>(r) * C];
  out[static_cast<size_t>(blockIdx.y) * C + c] = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

Tiling plan_tiling(int64_t T, int nvec, int target_blocks) {
  Tiling t;
  t.T = T;
  t.nvec = nvec;
  t.strips = (nvec + kStrip - 1) / kStrip;
  // Round down: a grid slightly larger than the resident capacity would leave a
  // few straggler blocks running alone after the rest finish.
  const int64_t want = std::max<int64_t>(1, target_blocks / t.strips);
  const int64_t most = std::max<int64_t>(1, (T + kWaves - 1) / kWaves);  // every row group owns a row
  t.G = static_cast<int>(std::min<int64_t>(std::min(want, most), 65535));
  return t;
}

hipError_t launch_colsum(const float* in, int R, int64_t C, float* out, hipStream_t s) {
  const int64_t blocks = (C + 255) / 256;
  hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, in, R, C, out);
  return hipGetLastError();
}

int64_t colsum_tall_tmp_floats(int R, int64_t C) { return R <= 32 ? 0 : static_cast<int64_t>((R + 31) / 32) * C; }

hipError_t launch_colsum_tall(const float* in, int R, int64_t C, float* tmp, float* out, hipStream_t s) {
  if (R <= 32) return launch_colsum(in, R, C, out, s);
  const int chunks = (R + 31) / 32;
  const int64_t blocks = (C + 255) / 256;
  hipLaunchKernelGGL(colsum_chunk_kernel, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(chunks)),
                     dim3(256), 0, s, in, R, C, tmp);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_colsum(tmp, chunks, C, out, s);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace mb
