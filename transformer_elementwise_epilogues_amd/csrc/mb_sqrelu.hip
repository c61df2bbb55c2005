// mb_sqrelu.hip -- weighted squared ReLU (MoE experts), forward and backward.
//
// The fusions article names a fused weighted squared ReLU for MoE layers (its
// sections 2 and 8) beside the weighted SwiGLU, without printing a formula.
// Read as that op's pattern (the unweighted activation times the per-token
// weight, section 9) applied to the squared ReLU:
//   out[t, j] = relu(x)^2 * w[t]        dx = g * w[t] * 2 relu(x)
//   dw[t]     = sum_j g * relu(x)^2
// with relu passing NaN through (as torch's does). Without weights it is the
// plain squared ReLU.
//
// Tiling as for the other elementwise kernels: a wave owns a strip of 64
// 16-byte column vectors and walks rows 4y + w + 4Gk; the row's weight is one
// scalar per wave. The weights gradient is a row sum: each wave reduces its
// strip's part of the row with a fixed butterfly, lane 0 writes one partial per
// (strip, row), and a second launch sums the strips in order.
#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

// Cache policy of the streaming stores (st_row: -1 global nt, 2 buffer nt,
// 18 buffer nt sc1), by measurement: buffer nt sc1 stores made the forward
// 1.9 % and the backward 0.5 % faster.
#ifndef MB_SRELU_ST
#define MB_SRELU_ST 18
#endif

constexpr int kUnrollFwd = MB_SRELU_FWD_UNROLL;
constexpr int kUnrollBwd = MB_SRELU_BWD_UNROLL;

template <bool WEIGHTED, DT W>
__device__ __forceinline__ float row_weight(const char* w, int64_t t) {
  if constexpr (!WEIGHTED) return 1.0f;
  if constexpr (W == DT::F32) return reinterpret_cast<const float*>(w)[t];
  if constexpr (W == DT::BF16) {
    const unsigned h = reinterpret_cast<const uint16_t*>(w)[t];
    return as_float(h << 16);
  }
  if constexpr (W == DT::F16) return static_cast<float>(reinterpret_cast<const _Float16*>(w)[t]);
  return 1.0f;
}

__device__ __forceinline__ float relu_nan(float x) {
  const float r = x > 0.0f ? x : 0.0f;
  return x != x ? x : r;
}

template <DT D>
__device__ __forceinline__ u32x4 srelu_vec(u32x4 xv, float w) {
  constexpr int V = Vec<D>::N;
  float f[V];
  unpack<D>(xv, f);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    // (r w) r, not r^2 w: for w = 0 or w < 1 the product stays finite
    // wherever the exact value is, as it does in the oracle's arithmetic
    const float r = relu_nan(f[k]);
    f[k] = (r * w) * r;
  }
  return pack<D>(f);
}

template <DT D, bool WEIGHTED, DT W, int U>
__global__ __launch_bounds__(kThreads) void srelu_fwd_kernel(const char* x, const char* w, char* out, int64_t T,
                                                             int nvec) {
  const int lane = threadIdx.x & 63, wave = wave_index<(MB_SRELU_ST >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  if (cv >= nvec) return;
  const size_t pitch = static_cast<size_t>(nvec) * 16;
  const char* xp = x + static_cast<size_t>(cv) * 16;
  char* op = out + static_cast<size_t>(cv) * 16;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  for (; t + (U - 1) * S < T; t += U * S) {
    u32x4 v[U];
    float wt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = ld_stream(xp + (t + u * S) * pitch);
      wt[u] = row_weight<WEIGHTED, W>(w, t + u * S);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) st_row<MB_SRELU_ST>(op + (t + u * S) * pitch, out + (t + u * S) * pitch, static_cast<uint32_t>(cv) * 16, srelu_vec<D>(v[u], wt[u]));
  }
  for (; t < T; t += S)
    st_row<MB_SRELU_ST>(op + t * pitch, out + t * pitch, static_cast<uint32_t>(cv) * 16, srelu_vec<D>(ld_stream(xp + t * pitch), row_weight<WEIGHTED, W>(w, t)));
}

// dx of one vector; returns the lane's part of the row's weights gradient
template <DT D, bool DW>
__device__ __forceinline__ float srelu_grad_vec(u32x4 gv, u32x4 xv, float w, u32x4* dx) {
  constexpr int V = Vec<D>::N;
  float g[V], f[V];
  unpack<D>(gv, g);
  unpack<D>(xv, f);
  float rowsum = 0.0f;
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const float r = relu_nan(f[k]);
    if constexpr (DW) rowsum = __builtin_fmaf(g[k] * r, r, rowsum);
    f[k] = ((g[k] * w) * 2.0f) * r;
  }
  *dx = pack<D>(f);
  return rowsum;
}

template <DT D, bool WEIGHTED, DT W, int U, bool DW>
__global__ __launch_bounds__(kThreads) void srelu_bwd_kernel(const char* g, const char* x, const char* w, char* dx,
                                                             float* wpart, int64_t T, int nvec) {
  const int lane = threadIdx.x & 63, wave = wave_index<(MB_SRELU_ST >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  const bool active = cv < nvec;
  if constexpr (!DW) {
    if (!active) return;
  }
  const size_t pitch = static_cast<size_t>(nvec) * 16, col = static_cast<size_t>(cv) * 16;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  // the row loop is uniform across the wave (t depends on the wave only), so
  // the weights-gradient butterfly sees every lane
  for (; t + (U - 1) * S < T; t += U * S) {
    u32x4 gv[U], xv[U];
    float wt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t + u * S;
      if (active) {
        gv[u] = ld_stream(g + tt * pitch + col);
        xv[u] = ld_stream(x + tt * pitch + col);
      } else {
        gv[u] = xv[u] = u32x4{0, 0, 0, 0};
      }
      wt[u] = row_weight<WEIGHTED, W>(w, tt);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t + u * S;
      u32x4 d;
      float rs = srelu_grad_vec<D, DW>(gv[u], xv[u], wt[u], &d);
      if (active) st_row<MB_SRELU_ST>(dx + tt * pitch + col, dx + tt * pitch, static_cast<uint32_t>(col), d);
      if constexpr (DW) {
        rs = wave_sum(active ? rs : 0.0f);
        if (lane == 0) wpart[static_cast<size_t>(ti.strip) * T + tt] = rs;
      }
    }
  }
  for (; t < T; t += S) {
    u32x4 gv = {0, 0, 0, 0}, xv = {0, 0, 0, 0};
    if (active) {
      gv = ld_stream(g + t * pitch + col);
      xv = ld_stream(x + t * pitch + col);
    }
    u32x4 d;
    float rs = srelu_grad_vec<D, DW>(gv, xv, row_weight<WEIGHTED, W>(w, t), &d);
    if (active) st_row<MB_SRELU_ST>(dx + t * pitch + col, dx + t * pitch, static_cast<uint32_t>(col), d);
    if constexpr (DW) {
      rs = wave_sum(active ? rs : 0.0f);
      if (lane == 0) wpart[static_cast<size_t>(ti.strip) * T + t] = rs;
    }
  }
}

template <DT D, bool WEIGHTED, DT W>
hipError_t fwd_launch(const void* x, const void* w, void* out, const Tiling& t, hipStream_t s) {
  hipLaunchKernelGGL((srelu_fwd_kernel<D, WEIGHTED, W, kUnrollFwd>), tile_grid(t.strips, t.G), dim3(kThreads), 0, s,
                     static_cast<const char*>(x), static_cast<const char*>(w), static_cast<char*>(out), t.T, t.nvec);
  return hipGetLastError();
}

template <DT D, bool WEIGHTED, DT W>
hipError_t bwd_launch(const void* g, const void* x, const void* w, void* dx, float* wpart, const Tiling& t,
                      hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  auto gp = static_cast<const char*>(g);
  auto xp = static_cast<const char*>(x);
  auto wp = static_cast<const char*>(w);
  auto dp = static_cast<char*>(dx);
  if (wpart)
    hipLaunchKernelGGL((srelu_bwd_kernel<D, WEIGHTED, W, kUnrollBwd, true>), grid, dim3(kThreads), 0, s, gp, xp, wp,
                       dp, wpart, t.T, t.nvec);
  else
    hipLaunchKernelGGL((srelu_bwd_kernel<D, WEIGHTED, W, kUnrollBwd, false>), grid, dim3(kThreads), 0, s, gp, xp, wp,
                       dp, wpart, t.T, t.nvec);
  return hipGetLastError();
}

template <DT D>
hipError_t fwd_by_weight(int wdt, const void* x, const void* w, void* out, const Tiling& t, hipStream_t s) {
  if (!w) return fwd_launch<D, false, DT::F32>(x, w, out, t, s);
  switch (static_cast<DT>(wdt)) {
    case DT::F32: return fwd_launch<D, true, DT::F32>(x, w, out, t, s);
    case DT::F16: return fwd_launch<D, true, DT::F16>(x, w, out, t, s);
    case DT::BF16: return fwd_launch<D, true, DT::BF16>(x, w, out, t, s);
  }
  return hipErrorInvalidValue;
}

template <DT D>
hipError_t bwd_by_weight(int wdt, const void* g, const void* x, const void* w, void* dx, float* wpart, const Tiling& t,
                         hipStream_t s) {
  if (!w) return bwd_launch<D, false, DT::F32>(g, x, w, dx, nullptr, t, s);
  switch (static_cast<DT>(wdt)) {
    case DT::F32: return bwd_launch<D, true, DT::F32>(g, x, w, dx, wpart, t, s);
    case DT::F16: return bwd_launch<D, true, DT::F16>(g, x, w, dx, wpart, t, s);
    case DT::BF16: return bwd_launch<D, true, DT::BF16>(g, x, w, dx, wpart, t, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_srelu_fwd(int dt, int wdt, const void* x, const void* w, void* out, const Tiling& t,
                            hipStream_t s) {
  switch (static_cast<DT>(dt)) {
    case DT::F32: return fwd_by_weight<DT::F32>(wdt, x, w, out, t, s);
    case DT::F16: return fwd_by_weight<DT::F16>(wdt, x, w, out, t, s);
    case DT::BF16: return fwd_by_weight<DT::BF16>(wdt, x, w, out, t, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_srelu_bwd(int dt, int wdt, const void* g, const void* x, const void* w, void* dx, float* wpart,
                            const Tiling& t, hipStream_t s) {
  switch (static_cast<DT>(dt)) {
    case DT::F32: return bwd_by_weight<DT::F32>(wdt, g, x, w, dx, wpart, t, s);
    case DT::F16: return bwd_by_weight<DT::F16>(wdt, g, x, w, dx, wpart, t, s);
    case DT::BF16: return bwd_by_weight<DT::BF16>(wdt, g, x, w, dx, wpart, t, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mb
