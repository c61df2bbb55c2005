// mb_bda.hip -- bias + dropout + residual add (train and inference) and the
// keep-mask export.
//
// Method: Megatron-LM's _bias_dropout_add_func as described by the wmrh.cn
// article on megatron/core/fusions, section 3.2 (one fused branch; the
// residual is cast to x's dtype first; in-place at inference) and section 3.3
// (separate train and inference entry points).
//
// The keep decision of element i = t*H + j comes from Philox4x32-10 with
// counter (i/4, offset) and key seed: the 8 (bf16/fp16) or 4 (fp32) elements
// of a lane's 16-byte vector are exactly 2 or 1 Philox blocks, so no random
// word is wasted and the mask does not depend on the launch shape. The
// residual cast is done in registers (an fp32 residual is read once, never
// materialised in x's dtype).
#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

constexpr int kUnroll = MB_BDA_UNROLL;

template <DT D, DT R, bool TRAIN>
__device__ __forceinline__ u32x4 bda_vec(u32x4 xv, const u32x4* rv, const float* b, uint64_t i0,
                                         const DropoutArgs& d) {
  constexpr int V = Vec<D>::N;
  constexpr int RPER = Vec<R>::N;
  float x[V], r[V];
  unpack<D>(xv, x);
#pragma unroll
  for (int q = 0; q < V / RPER; ++q) unpack<R>(rv[q], r + q * RPER);
  bool keep[V];
  if constexpr (TRAIN) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) keep4((i0 >> 2) + q, d.o0, d.o1, d.k0, d.k1, d.theta, keep + 4 * q);
  }
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const float rp = (R == D) ? r[k] : round_to<D>(r[k]);
    const float z = x[k] + b[k];
    if constexpr (TRAIN)
      x[k] = __builtin_fmaf(keep[k] ? z : 0.0f, d.scale, rp);
    else
      x[k] = rp + z;
  }
  return pack<D>(x);
}

template <DT D, DT R, bool TRAIN, int U>
__global__ __launch_bounds__(kThreads) void bda_kernel(const char* x, const char* bias, const char* res, char* out,
                                                       int64_t T, int nvec, int64_t H, DropoutArgs d) {
  constexpr int V = Vec<D>::N;
  constexpr int RV = V / Vec<R>::N;  // 16-byte residual vectors per group
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  if (cv >= nvec) return;
  float b[V];
  if (bias) {
    unpack<D>(ld_keep(bias + static_cast<size_t>(cv) * 16), b);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) b[k] = 0.0f;
  }
  const size_t px = static_cast<size_t>(nvec) * 16;
  const size_t pr = px * RV;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  const char* xp = x + static_cast<size_t>(cv) * 16;
  const char* rp = res + static_cast<size_t>(cv) * 16 * RV;
  char* op = out + static_cast<size_t>(cv) * 16;
  const uint64_t j0 = static_cast<uint64_t>(cv) * V;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  for (; t + (U - 1) * S < T; t += U * S) {
    u32x4 xv[U], rv[U][RV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xv[u] = ld_stream(xp + (t + u * S) * px);
#pragma unroll
      for (int q = 0; q < RV; ++q) rv[u][q] = ld_stream(rp + (t + u * S) * pr + 16 * q);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t i0 = static_cast<uint64_t>(t + u * S) * static_cast<uint64_t>(H) + j0;
      st_stream(op + (t + u * S) * px, bda_vec<D, R, TRAIN>(xv[u], rv[u], b, i0, d));
    }
  }
  for (; t < T; t += S) {
    u32x4 xv = ld_stream(xp + t * px), rv[RV];
#pragma unroll
    for (int q = 0; q < RV; ++q) rv[q] = ld_stream(rp + t * pr + 16 * q);
    const uint64_t i0 = static_cast<uint64_t>(t) * static_cast<uint64_t>(H) + j0;
    st_stream(op + t * px, bda_vec<D, R, TRAIN>(xv, rv, b, i0, d));
  }
}

// One byte (8 elements) per thread; n is a multiple of 4.
__global__ __launch_bounds__(256) void mask_kernel(uint8_t* bits, int64_t n, DropoutArgs d) {
  const int64_t byte = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbytes = (n + 7) / 8;
  if (byte >= nbytes) return;
  const int64_t i0 = byte * 8;
  bool keep[8] = {false, false, false, false, false, false, false, false};
  keep4(static_cast<uint64_t>(i0) >> 2, d.o0, d.o1, d.k0, d.k1, d.theta, keep);
  if (i0 + 4 < n) keep4((static_cast<uint64_t>(i0) >> 2) + 1, d.o0, d.o1, d.k0, d.k1, d.theta, keep + 4);
  unsigned v = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) v |= (keep[k] ? 1u : 0u) << k;
  bits[byte] = static_cast<uint8_t>(v);
}

template <DT D, DT R>
hipError_t bda_dispatch(bool train, const void* x, const void* bias, const void* res, void* out, int64_t H,
                        const Tiling& t, const DropoutArgs& d, hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  auto xp = static_cast<const char*>(x);
  auto bp = static_cast<const char*>(bias);
  auto rp = static_cast<const char*>(res);
  auto op = static_cast<char*>(out);
  if (train)
    hipLaunchKernelGGL((bda_kernel<D, R, true, kUnroll>), grid, dim3(kThreads), 0, s, xp, bp, rp, op, t.T, t.nvec, H, d);
  else
    hipLaunchKernelGGL((bda_kernel<D, R, false, kUnroll>), grid, dim3(kThreads), 0, s, xp, bp, rp, op, t.T, t.nvec, H, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bda(int dt, int res_dt, bool train, const void* x, const void* bias, const void* residual,
                      void* out, int64_t H, const Tiling& t, const DropoutArgs& d, hipStream_t s) {
  const DT D = static_cast<DT>(dt), R = static_cast<DT>(res_dt);
  if (D == DT::F32 && R == DT::F32) return bda_dispatch<DT::F32, DT::F32>(train, x, bias, residual, out, H, t, d, s);
  if (D == DT::BF16 && R == DT::BF16) return bda_dispatch<DT::BF16, DT::BF16>(train, x, bias, residual, out, H, t, d, s);
  if (D == DT::BF16 && R == DT::F32) return bda_dispatch<DT::BF16, DT::F32>(train, x, bias, residual, out, H, t, d, s);
  if (D == DT::F16 && R == DT::F16) return bda_dispatch<DT::F16, DT::F16>(train, x, bias, residual, out, H, t, d, s);
  if (D == DT::F16 && R == DT::F32) return bda_dispatch<DT::F16, DT::F32>(train, x, bias, residual, out, H, t, d, s);
  return hipErrorInvalidValue;
}

hipError_t launch_dropout_mask(uint8_t* bits, int64_t n, const DropoutArgs& d, hipStream_t s) {
  const int64_t nbytes = (n + 7) / 8;
  const int64_t blocks = (nbytes + 255) / 256;
  hipLaunchKernelGGL(mask_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, bits, n, d);
  return hipGetLastError();
}

}  // namespace mb
