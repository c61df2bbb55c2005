// mb_gelu.hip -- bias + GeLU (tanh approximation and the exact erf form),
// forward and backward with the fused bias-gradient column reduction.
//
// Method: Megatron-LM's bias_gelu / bias_gelu_back as described by the
// wmrh.cn article on megatron/core/fusions, section 4.2 (formulas and
// constants) and section 4.3 (the bias gradient is the per-element gradient
// summed over tokens). The kernels evaluate the same functions through the
// logistic identities in mb_device.hpp.
//
// One pass per op: each lane owns one 16-byte column vector (8 bf16/fp16 or
// 4 fp32 values), holds its bias slice in registers for every row it visits,
// and streams rows with U loads in flight. The backward pass accumulates the
// fp32 gradient per lane, combines the 4 waves of a block in LDS in a fixed
// order and writes one partial row per row group; a second launch sums the
// partial rows in order (no atomics, bit-reproducible).
#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

constexpr int kUnrollFwd = MB_GELU_FWD_UNROLL;
// rows in flight per wave in the backward, per form (both 4 at present)
template <int KIND> constexpr int unroll_bwd() { return KIND == 0 ? MB_GELU_BWD_UNROLL : MB_GELU_ERF_BWD_UNROLL; }

template <DT D>
__device__ __forceinline__ void load_bias(const char* bias, int cv, float* b) {
  constexpr int V = Vec<D>::N;
  if (bias) {
    unpack<D>(ld_keep(bias + static_cast<size_t>(cv) * 16), b);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) b[k] = 0.0f;
  }
}

enum Kind { kTanh = 0, kErf = 1 };

// Cache policy of the streaming stores per kind (st_row: -1 global nt,
// 2 buffer nt, 18 buffer nt sc1), by measurement: buffer nt sc1 stores made
// the tanh forward 4-5 % and the exact backward 1.8 % faster; the exact
// forward did not change, and the tanh backward is as fast either way in its
// many-block grid.
#ifndef MB_GELU_FWD_ST
#define MB_GELU_FWD_ST 18
#endif
#ifndef MB_GELU_ERF_FWD_ST
#define MB_GELU_ERF_FWD_ST -1
#endif
#ifndef MB_GELU_BWD_ST
#define MB_GELU_BWD_ST 18
#endif
#ifndef MB_GELU_ERF_BWD_ST
#define MB_GELU_ERF_BWD_ST 18
#endif
template <int KIND> constexpr int st_fwd() { return KIND == kTanh ? MB_GELU_FWD_ST : MB_GELU_ERF_FWD_ST; }
template <int KIND> constexpr int st_bwd() { return KIND == kTanh ? MB_GELU_BWD_ST : MB_GELU_ERF_BWD_ST; }
// Loads likewise (ld_row: -1 global nt, else a buffer load with that cache
// policy): buffer loads made the tanh backward 1.3 % faster (any of nt, nt sc0,
// nt sc1, nt sc0 sc1), changed nothing in the tanh forward and cost the exact
// forms 1-2 %.
#ifndef MB_GELU_FWD_LD
#define MB_GELU_FWD_LD -1
#endif
#ifndef MB_GELU_ERF_FWD_LD
#define MB_GELU_ERF_FWD_LD -1
#endif
#ifndef MB_GELU_BWD_LD
#define MB_GELU_BWD_LD 2
#endif
#ifndef MB_GELU_ERF_BWD_LD
#define MB_GELU_ERF_BWD_LD -1
#endif
template <int KIND> constexpr int ld_fwd() { return KIND == kTanh ? MB_GELU_FWD_LD : MB_GELU_ERF_FWD_LD; }
template <int KIND> constexpr int ld_bwd() { return KIND == kTanh ? MB_GELU_BWD_LD : MB_GELU_ERF_BWD_LD; }

#ifndef MB_GELU_BWD_PIPELINE
#define MB_GELU_BWD_PIPELINE 1
#endif
constexpr bool kPipelineBwd = MB_GELU_BWD_PIPELINE;

template <DT D, int KIND>
__device__ __forceinline__ u32x4 gelu_vec(u32x4 yv, const float* b) {
  constexpr int V = Vec<D>::N;
  float f[V];
  unpack<D>(yv, f);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const ScaledF r = KIND == kTanh ? gelu_tanh_scaled(f[k] + b[k]) : gelu_erf_fwd<(D != DT::F32)>(f[k] + b[k]);
    f[k] = r.v * r.sc;
  }
  return pack<D>(f);
}

template <DT D, int KIND, int U>
__global__ __launch_bounds__(kThreads) void gelu_fwd_kernel(const char* y, const char* bias, char* out,
                                                            int64_t T, int nvec) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(st_fwd<KIND>() >= 0 || ld_fwd<KIND>() >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  if (cv >= nvec) return;
  float b[Vec<D>::N];
  load_bias<D>(bias, cv, b);
  const size_t pitch = static_cast<size_t>(nvec) * 16;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  const char* yp = y + static_cast<size_t>(cv) * 16;
  char* op = out + static_cast<size_t>(cv) * 16;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  for (; t + (U - 1) * S < T; t += U * S) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_row<ld_fwd<KIND>()>(yp + (t + u * S) * pitch, y + (t + u * S) * pitch, static_cast<uint32_t>(cv) * 16);
#pragma unroll
    for (int u = 0; u < U; ++u)
      st_row<st_fwd<KIND>()>(op + (t + u * S) * pitch, out + (t + u * S) * pitch, static_cast<uint32_t>(cv) * 16, gelu_vec<D, KIND>(v[u], b));
  }
  for (; t < T; t += S)
    st_row<st_fwd<KIND>()>(op + t * pitch, out + t * pitch, static_cast<uint32_t>(cv) * 16, gelu_vec<D, KIND>(ld_row<ld_fwd<KIND>()>(yp + t * pitch, y + t * pitch, static_cast<uint32_t>(cv) * 16), b));
}

template <DT D, int KIND>
__device__ __forceinline__ u32x4 gelu_grad_vec(u32x4 gv, u32x4 yv, const float* b, float* acc) {
  constexpr int V = Vec<D>::N;
  float g[V], f[V];
  unpack<D>(gv, g);
  unpack<D>(yv, f);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    float d;
    if constexpr (KIND == kTanh) {
      const GeluB q = gelu_tanh_fwd_bwd(f[k] + b[k]);
      d = __builtin_fmaf(g[k] * q.d, q.sc, q.nan);
    } else {
      const ScaledF r = gelu_erf_grad(f[k] + b[k]);
      d = (g[k] * r.v) * r.sc;
    }
    acc[k] += d;
    f[k] = d;
  }
  return pack<D>(f);
}

template <DT D, int KIND, int U, bool DBIAS>
__global__ __launch_bounds__(kThreads) void gelu_bwd_kernel(const char* g, const char* y, const char* bias,
                                                            char* dgrad, float* partials, int64_t T,
                                                            int nvec) {
  constexpr int V = Vec<D>::N;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(st_bwd<KIND>() >= 0 || ld_bwd<KIND>() >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  const bool active = cv < nvec;
  ColAcc<V> ca;
  ca.init();
  if (active) {
    float b[V];
    load_bias<D>(bias, cv, b);
    const size_t pitch = static_cast<size_t>(nvec) * 16;
    const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
    const size_t col = static_cast<size_t>(cv) * 16;
    int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
    if constexpr (kPipelineBwd) {
      // software pipeline: the next U rows' loads are issued before this U
      // rows' arithmetic, so a wave (often the only one on its SIMD) keeps
      // memory busy while it computes. The steady-state branch always issues
      // them, so the waits before the arithmetic cover only the current rows.
      if (t + (U - 1) * S < T) {
        u32x4 gv[U], yv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const size_t o = (t + u * S) * pitch + col;
          gv[u] = ld_row<ld_bwd<KIND>()>(g + o, g + (o - col), static_cast<uint32_t>(col));
          yv[u] = ld_row<ld_bwd<KIND>()>(y + o, y + (o - col), static_cast<uint32_t>(col));
        }
        for (;;) {
          const int64_t tn = t + U * S;
          if (tn + (U - 1) * S < T) {
            u32x4 gn[U], yn[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const size_t o = (tn + u * S) * pitch + col;
              gn[u] = ld_row<ld_bwd<KIND>()>(g + o, g + (o - col), static_cast<uint32_t>(col));
              yn[u] = ld_row<ld_bwd<KIND>()>(y + o, y + (o - col), static_cast<uint32_t>(col));
            }
            prefetch_fence();
#pragma unroll
            for (int u = 0; u < U; ++u)
              st_row<st_bwd<KIND>()>(dgrad + (t + u * S) * pitch + col, dgrad + (t + u * S) * pitch, static_cast<uint32_t>(col), gelu_grad_vec<D, KIND>(gv[u], yv[u], b, ca.lo));
            if constexpr (DBIAS) ca.tick(U);
#pragma unroll
            for (int u = 0; u < U; ++u) {
              gv[u] = gn[u];
              yv[u] = yn[u];
            }
            t = tn;
          } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
              st_row<st_bwd<KIND>()>(dgrad + (t + u * S) * pitch + col, dgrad + (t + u * S) * pitch, static_cast<uint32_t>(col), gelu_grad_vec<D, KIND>(gv[u], yv[u], b, ca.lo));
            if constexpr (DBIAS) ca.tick(U);
            t = tn;
            break;
          }
        }
      }
    } else {
      for (; t + (U - 1) * S < T; t += U * S) {
        u32x4 gv[U], yv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const size_t o = (t + u * S) * pitch + col;
          gv[u] = ld_row<ld_bwd<KIND>()>(g + o, g + (o - col), static_cast<uint32_t>(col));
          yv[u] = ld_row<ld_bwd<KIND>()>(y + o, y + (o - col), static_cast<uint32_t>(col));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          st_row<st_bwd<KIND>()>(dgrad + (t + u * S) * pitch + col, dgrad + (t + u * S) * pitch, static_cast<uint32_t>(col), gelu_grad_vec<D, KIND>(gv[u], yv[u], b, ca.lo));
        if constexpr (DBIAS) ca.tick(U);
      }
    }
    for (; t < T; t += S) {
      const size_t o = t * pitch + col;
      st_row<st_bwd<KIND>()>(dgrad + o, dgrad + t * pitch, static_cast<uint32_t>(col), gelu_grad_vec<D, KIND>(ld_row<ld_bwd<KIND>()>(g + o, g + t * pitch, static_cast<uint32_t>(col)), ld_row<ld_bwd<KIND>()>(y + o, y + t * pitch, static_cast<uint32_t>(col)), b, ca.lo));
      if constexpr (DBIAS) ca.tick(1);
    }
  }
  float acc[V];
  ca.total(acc);
  if constexpr (DBIAS)
    block_column_partials<V>(acc, wave, lane, active,
                             partials + static_cast<size_t>(ti.rg) * nvec * V + static_cast<size_t>(cv) * V);
}

template <DT D, int KIND>
hipError_t gelu_fwd_dispatch(const void* y, const void* bias, void* out, const Tiling& t, hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  hipLaunchKernelGGL((gelu_fwd_kernel<D, KIND, kUnrollFwd>), grid, dim3(kThreads), 0, s,
                     static_cast<const char*>(y), static_cast<const char*>(bias), static_cast<char*>(out), t.T,
                     t.nvec);
  return hipGetLastError();
}

template <DT D, int KIND>
hipError_t gelu_bwd_dispatch(const void* g, const void* y, const void* bias, void* dgrad, float* partials,
                             const Tiling& t, hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  auto gp = static_cast<const char*>(g);
  auto yp = static_cast<const char*>(y);
  auto bp = static_cast<const char*>(bias);
  auto dp = static_cast<char*>(dgrad);
  if (partials)
    hipLaunchKernelGGL((gelu_bwd_kernel<D, KIND, unroll_bwd<KIND>(), true>), grid, dim3(kThreads), 0, s, gp, yp, bp, dp,
                       partials, t.T, t.nvec);
  else
    hipLaunchKernelGGL((gelu_bwd_kernel<D, KIND, unroll_bwd<KIND>(), false>), grid, dim3(kThreads), 0, s, gp, yp, bp, dp,
                       partials, t.T, t.nvec);
  return hipGetLastError();
}

}  // namespace

template <int KIND>
hipError_t gelu_fwd_any(int dt, const void* y, const void* bias, void* out, const Tiling& t, hipStream_t s) {
  switch (static_cast<DT>(dt)) {
    case DT::F32: return gelu_fwd_dispatch<DT::F32, KIND>(y, bias, out, t, s);
    case DT::F16: return gelu_fwd_dispatch<DT::F16, KIND>(y, bias, out, t, s);
    case DT::BF16: return gelu_fwd_dispatch<DT::BF16, KIND>(y, bias, out, t, s);
  }
  return hipErrorInvalidValue;
}

template <int KIND>
hipError_t gelu_bwd_any(int dt, const void* g, const void* y, const void* bias, void* dgrad, float* partials,
                        const Tiling& t, hipStream_t s) {
  switch (static_cast<DT>(dt)) {
    case DT::F32: return gelu_bwd_dispatch<DT::F32, KIND>(g, y, bias, dgrad, partials, t, s);
    case DT::F16: return gelu_bwd_dispatch<DT::F16, KIND>(g, y, bias, dgrad, partials, t, s);
    case DT::BF16: return gelu_bwd_dispatch<DT::BF16, KIND>(g, y, bias, dgrad, partials, t, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gelu_fwd(int dt, bool exact, const void* y, const void* bias, void* out, const Tiling& t,
                           hipStream_t s) {
  return exact ? gelu_fwd_any<kErf>(dt, y, bias, out, t, s) : gelu_fwd_any<kTanh>(dt, y, bias, out, t, s);
}

hipError_t launch_gelu_bwd(int dt, bool exact, const void* g, const void* y, const void* bias, void* dgrad,
                           float* partials, const Tiling& t, hipStream_t s) {
  return exact ? gelu_bwd_any<kErf>(dt, g, y, bias, dgrad, partials, t, s)
               : gelu_bwd_any<kTanh>(dt, g, y, bias, dgrad, partials, t, s);
}

}  // namespace mb
