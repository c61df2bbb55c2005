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

// Sum of p[r C] for r in [r0, r1), added in ascending r. The partial rows
// were just written and sit in the caches, so the pass is bound by load
// latency: the loads of 16 rows are issued before their adds (one latency per
// 16 rows instead of one per 4, the same order of adds).
constexpr int kSumBatch = 16;
__device__ __forceinline__ float sum_col(const float* __restrict__ p, int64_t C, int r0, int r1) {
  float s = 0.0f;
  int r = r0;
  for (; r + kSumBatch <= r1; r += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i) v[i] = p[static_cast<size_t>(r + i) * C];
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i) s += v[i];
  }
  if (r < r1) {
    float v[kSumBatch];
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i) v[i] = r + i < r1 ? p[static_cast<size_t>(r + i) * C] : 0.0f;
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i)
      if (r + i < r1) s += v[i];
  }
  return s;
}

// Every kernel below sums one of two independent arrays, chosen by
// blockIdx.z, so that two column sums of one op (dgamma and dbeta; the bias
// and the weights gradients) share their launches; a single sum passes z = 1.
__global__ __launch_bounds__(256) void colsum_kernel(ColSum a, ColSum b) {
  const ColSum& k = blockIdx.z ? b : a;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= k.C) return;
  k.out[c] = sum_col(k.in + c, k.C, 0, k.R);
}

// out[y, c] = sum of in[r, c] for r in [32 y, min(R, 32 y + 32)), ascending
__global__ __launch_bounds__(256) void colsum_chunk_kernel(ColSum a, ColSum b) {
  const ColSum& k = blockIdx.z ? b : a;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int r0 = static_cast<int>(blockIdx.y) * 32;
  if (c >= k.C || r0 >= k.R) return;
  const int r1 = r0 + 32 < k.R ? r0 + 32 : k.R;
  k.out[static_cast<size_t>(blockIdx.y) * k.C + c] = sum_col(k.in + c, k.C, r0, r1);
}

// Up to 16 chunks of 32 partial rows in one launch: wave y of a block sums
// chunk y of 64 columns as colsum_chunk_kernel does, and wave 0 adds the
// chunk sums in ascending order as colsum_kernel does, so the result is bit
// for bit that of the two launches.
constexpr int kFoldChunks = 16;
__global__ __launch_bounds__(64 * kFoldChunks) void colsum_fold_kernel(ColSum a, ColSum b) {
  const ColSum& k = blockIdx.z ? b : a;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  __shared__ float part[kFoldChunks][64];
  const int r0 = w * 32, r1 = r0 + 32 < k.R ? r0 + 32 : k.R;
  float s = 0.0f;
  if (c < k.C && r0 < k.R) s = sum_col(k.in + c, k.C, r0, r1);
  part[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < k.C) {
    const int chunks = (k.R + 31) / 32;
    float t = 0.0f;
    for (int j = 0; j < chunks; ++j) t += part[j][lane];
    k.out[c] = t;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

static unsigned col_blocks(int64_t C) { return static_cast<unsigned>((C + 255) / 256); }

hipError_t launch_colsum2(const ColSum& a, const ColSum& b, hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel, dim3(std::max(col_blocks(a.C), col_blocks(b.C)), 1, 2), dim3(256), 0, s, a, b);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* in, int R, int64_t C, float* out, hipStream_t s) {
  const ColSum a{in, R, C, out};
  hipLaunchKernelGGL(colsum_kernel, dim3(col_blocks(C), 1, 1), dim3(256), 0, s, a, a);
  return hipGetLastError();
}


// a, b: the partial rows; ta, tb: the same with their chunk-sum buffers as `out`
static hipError_t colsum_tall_pair(const ColSum& a, const ColSum& b, float* tmp_a, float* tmp_b, unsigned arrays,
                                   hipStream_t s) {
  if (arrays == 1 && a.R <= 32) return launch_colsum(a.in, a.R, a.C, a.out, s);
  if (arrays == 2 && a.R <= 32 && b.R <= 32) return launch_colsum2(a, b, s);
  const int chunks_a = (a.R + 31) / 32, chunks_b = (b.R + 31) / 32;
  const int chunks = arrays == 2 ? std::max(chunks_a, chunks_b) : chunks_a;
  if (chunks <= kFoldChunks) {
    const int64_t cols = arrays == 2 ? std::max(a.C, b.C) : a.C;
    hipLaunchKernelGGL(colsum_fold_kernel, dim3(static_cast<unsigned>((cols + 63) / 64), 1, arrays),
                       dim3(64 * chunks), 0, s, a, b);
    return hipGetLastError();
  }
  const ColSum ca{a.in, a.R, a.C, tmp_a}, cb{b.in, b.R, b.C, tmp_b};
  hipLaunchKernelGGL(colsum_chunk_kernel,
                     dim3(std::max(col_blocks(a.C), col_blocks(b.C)), static_cast<unsigned>(std::max(chunks_a, chunks_b)),
                          arrays),
                     dim3(256), 0, s, ca, cb);
  if (hipError_t e = hipGetLastError()) return e;
  const ColSum fa{tmp_a, chunks_a, a.C, a.out}, fb{tmp_b, chunks_b, b.C, b.out};
  if (arrays == 1) return launch_colsum(fa.in, fa.R, fa.C, fa.out, s);
  return launch_colsum2(fa, fb, s);
}

hipError_t launch_colsum_tall(const float* in, int R, int64_t C, float* tmp, float* out, hipStream_t s) {
  const ColSum a{in, R, C, out};
  return colsum_tall_pair(a, a, tmp, tmp, 1, s);
}

hipError_t launch_colsum_tall2(const float* in0, const float* in1, int R, int64_t C, float* tmp0, float* tmp1,
                               float* out0, float* out1, hipStream_t s) {
  return colsum_tall_pair(ColSum{in0, R, C, out0}, ColSum{in1, R, C, out1}, tmp0, tmp1, 2, s);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace mb
