// mb_glu.hip -- bias + SwiGLU / GEGLU gated units, forward and backward, with
// the per-token weighted SwiGLU, the fused bias-gradient column reduction and
// the weights-gradient row reduction.
//
// Method: the fused_bias_swiglu / fused_bias_geglu modules named by the
// wmrh.cn article on megatron/core/fusions (section 2), and its section 9:
// weighted SwiGLU equals unweighted SwiGLU times the per-token weights,
// forward and gradients. The input row is split into a = columns [0, H) (the
// activated half) and b = columns [H, 2H).
//
// A lane owns output column vector cv and reads the matching 16-byte vectors
// of both halves, so a and b of the same column meet in registers. The
// backward pass keeps 2 x 8 fp32 bias-gradient sums per lane (combined across
// the block's waves in LDS) and, for weighted SwiGLU, reduces each row's
// g * silu(a) * b across the wave with a fixed butterfly; lane 0 writes one
// partial per (strip, row). Second launches sum both kinds of partials in a
// fixed order.
#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

constexpr int kUnrollFwd = MB_GLU_FWD_UNROLL;
constexpr int kUnrollBwd = MB_GLU_BWD_UNROLL;
#ifndef MB_GLU_BWD_PIPELINE
#define MB_GLU_BWD_PIPELINE 1
#endif

// The bias halves of column vector cv (zero bits, i.e. +0, without a bias).
// The raw vectors are selected before unpacking: selecting unpacked arrays
// made the compiler keep two of their values in scratch memory.
template <DT D>
__device__ __forceinline__ void load_bias_pair(const char* bias, int cv, int nvec, float* ba, float* bb) {
  u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
  if (bias) {
    va = ld_keep(bias + static_cast<size_t>(cv) * 16);
    vb = ld_keep(bias + static_cast<size_t>(nvec + cv) * 16);
  }
  unpack<D>(va, ba);
  unpack<D>(vb, bb);
}

// Per-token weight of row t, or 1 for the unweighted op. The weighted and
// unweighted ops are separate instantiations: a null test inside the row loop
// makes the compiler wait for every outstanding load (vmcnt(0)) at each row.
template <bool WEIGHTED, DT W>
__device__ __forceinline__ float load_weight(const char* w, int64_t t) {
  if constexpr (!WEIGHTED) return 1.0f;
  if constexpr (W == DT::F32) return reinterpret_cast<const float*>(w)[t];
  if constexpr (W == DT::BF16) {
    const unsigned h = reinterpret_cast<const uint16_t*>(w)[t];
    return as_float(h << 16);
  }
  if constexpr (W == DT::F16) return static_cast<float>(reinterpret_cast<const _Float16*>(w)[t]);
  return 1.0f;
}

// Cache policy of the streaming stores (st_row: -1 global nt, 2 buffer nt,
// 18 buffer nt sc1), by measurement: the forward gained 0.7-2 % with buffer
// nt sc1 stores, the SwiGLU backward lost 5 % with them.
#ifndef MB_GLU_FWD_ST
#define MB_GLU_FWD_ST 18
#endif
#ifndef MB_GLU_BWD_ST
#define MB_GLU_BWD_ST -1
#endif

template <DT D, int ACT>
__device__ __forceinline__ u32x4 glu_vec(u32x4 av, u32x4 bv, const float* ba, const float* bb, float w) {
  constexpr int V = Vec<D>::N;
  float a[V], b[V];
  unpack<D>(av, a);
  unpack<D>(bv, b);
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const float x = a[k] + ba[k];
    const float y = b[k] + bb[k];
    if constexpr (ACT == kSwiGLU) {
      const ScaledF r = silu_scaled(x);
      a[k] = ((r.v * y) * w) * r.sc;
    } else {
      const ScaledF r = gelu_tanh_scaled(x);
      a[k] = (r.v * y) * r.sc;
    }
  }
  return pack<D>(a);
}

template <DT D, int ACT, bool WEIGHTED, DT W, int U>
__global__ __launch_bounds__(kThreads) void glu_fwd_kernel(const char* in, const char* bias, const char* w,
                                                           char* out, int64_t T, int nvec) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(MB_GLU_FWD_ST >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  if (cv >= nvec) return;
  constexpr int V = Vec<D>::N;
  float ba[V], bb[V];
  load_bias_pair<D>(bias, cv, nvec, ba, bb);
  const size_t po = static_cast<size_t>(nvec) * 16;
  const size_t pi = 2 * po;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  const char* ap = in + static_cast<size_t>(cv) * 16;
  const char* bp = ap + po;
  char* op = out + static_cast<size_t>(cv) * 16;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  for (; t + (U - 1) * S < T; t += U * S) {
    u32x4 av[U], bv[U];
    float wt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      av[u] = ld_stream(ap + (t + u * S) * pi);
      bv[u] = ld_stream(bp + (t + u * S) * pi);
      wt[u] = load_weight<WEIGHTED, W>(w, t + u * S);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) st_row<MB_GLU_FWD_ST>(op + (t + u * S) * po, out + (t + u * S) * po, static_cast<uint32_t>(cv) * 16, glu_vec<D, ACT>(av[u], bv[u], ba, bb, wt[u]));
  }
  for (; t < T; t += S)
    st_row<MB_GLU_FWD_ST>(op + t * po, out + t * po, static_cast<uint32_t>(cv) * 16,
                           glu_vec<D, ACT>(ld_stream(ap + t * pi), ld_stream(bp + t * pi), ba, bb, load_weight<WEIGHTED, W>(w, t)));
}

// Backward of one column vector of one row. Returns the row's contribution to
// the weights gradient (sum over the lane's columns of g * act(a) * b).
template <DT D, int ACT, bool DW>
__device__ __forceinline__ float glu_grad_vec(u32x4 gv, u32x4 av, u32x4 bv, const float* ba, const float* bb,
                                              float w, float* acc_a, float* acc_b, u32x4* da_out,
                                              u32x4* db_out) {
  constexpr int V = Vec<D>::N;
  float g[V], a[V], b[V];
  unpack<D>(gv, g);
  unpack<D>(av, a);
  unpack<D>(bv, b);
  float rowsum = 0.0f;
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const float x = a[k] + ba[k];
    const float y = b[k] + bb[k];
    float da, db;
    if constexpr (ACT == kSwiGLU) {
      const SiluB s = silu_fwd_bwd(x);
      const float gw = g[k] * w;
      da = ((gw * y) * s.d) * s.sc;
      db = (gw * s.v) * s.sc;
      if constexpr (DW) rowsum += ((g[k] * s.v) * y) * s.sc;
    } else {
      const GeluB r = gelu_tanh_fwd_bwd(x);
      da = __builtin_fmaf((g[k] * y) * r.d, r.sc, r.nan);
      db = (g[k] * r.v) * r.sc;
    }
    acc_a[k] += da;
    acc_b[k] += db;
    a[k] = da;
    b[k] = db;
  }
  *da_out = pack<D>(a);
  *db_out = pack<D>(b);
  return rowsum;
}

template <DT D, int ACT, bool WEIGHTED, DT W, int U, bool DBIAS, bool DW>
__global__ __launch_bounds__(kThreads) void glu_bwd_kernel(const char* g, const char* in, const char* bias,
                                                           const char* w, char* din, float* bpart, float* wpart,
                                                           int64_t T, int nvec) {
  constexpr int V = Vec<D>::N;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(MB_GLU_BWD_ST >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  const bool active = cv < nvec;
  ColAcc<V> ca_a, ca_b;
  ca_a.init();
  ca_b.init();
  float* acc_a = ca_a.lo;
  float* acc_b = ca_b.lo;
  float ba[V], bb[V];
  if (active) {
    load_bias_pair<D>(bias, cv, nvec, ba, bb);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) ba[k] = bb[k] = 0.0f;
  }
  const size_t po = static_cast<size_t>(nvec) * 16;
  const size_t pi = 2 * po;
  const size_t col = static_cast<size_t>(cv) * 16;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  // Row loop is uniform across the wave (t depends on the wave only), so the
  // weights-gradient butterfly below sees every lane. Lanes past the last
  // column vector load a valid vector (clamped) and zero it, so that the
  // loads need no branch and the next rows' loads can be issued before this
  // rows' arithmetic (software pipeline).
  const size_t colc = active ? col : 0;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto fetch = [&](int64_t t0, u32x4* gv, u32x4* av, u32x4* bv, float* wt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t0 + u * S;
      gv[u] = ld_stream(g + tt * po + colc);
      av[u] = ld_stream(in + tt * pi + colc);
      bv[u] = ld_stream(in + tt * pi + po + colc);
      wt[u] = load_weight<WEIGHTED, W>(w, tt);
    }
  };
  auto compute = [&](int64_t t0, u32x4* gv, u32x4* av, u32x4* bv, const float* wt) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t0 + u * S;
      u32x4 dav, dbv;
      float rs = glu_grad_vec<D, ACT, DW>(active ? gv[u] : zero, active ? av[u] : zero, active ? bv[u] : zero, ba, bb,
                                          wt[u], acc_a, acc_b, &dav, &dbv);
      if (active) {
        st_row<MB_GLU_BWD_ST>(din + tt * pi + col, din + tt * pi, static_cast<uint32_t>(col), dav);
        st_row<MB_GLU_BWD_ST>(din + tt * pi + po + col, din + tt * pi, static_cast<uint32_t>(po + col), dbv);
      }
      if constexpr (DW) {
        rs = wave_sum(active ? rs : 0.0f);
        if (lane == 0) wpart[static_cast<size_t>(ti.strip) * T + tt] = rs;
      }
    }
    if constexpr (DBIAS) {
      ca_a.tick(U);
      ca_b.tick(U);
    }
  };
  if (t + (U - 1) * S < T) {
    u32x4 gv[U], av[U], bv[U];
    float wt[U];
    fetch(t, gv, av, bv, wt);
    for (;;) {
      const int64_t tn = t + U * S;
      if (tn + (U - 1) * S < T) {
        u32x4 gn[U], an[U], bn[U];
        float wn[U];
        if constexpr (MB_GLU_BWD_PIPELINE) {
          fetch(tn, gn, an, bn, wn);
          prefetch_fence();
          compute(t, gv, av, bv, wt);
        } else {
          compute(t, gv, av, bv, wt);
          fetch(tn, gn, an, bn, wn);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          gv[u] = gn[u];
          av[u] = an[u];
          bv[u] = bn[u];
          wt[u] = wn[u];
        }
        t = tn;
      } else {
        compute(t, gv, av, bv, wt);
        t = tn;
        break;
      }
    }
  }
  for (; t < T; t += S) {
    u32x4 gv = {0, 0, 0, 0}, av = {0, 0, 0, 0}, bv = {0, 0, 0, 0};
    if (active) {
      gv = ld_stream(g + t * po + col);
      av = ld_stream(in + t * pi + col);
      bv = ld_stream(in + t * pi + po + col);
    }
    u32x4 dav, dbv;
    float rs = glu_grad_vec<D, ACT, DW>(gv, av, bv, ba, bb, load_weight<WEIGHTED, W>(w, t), acc_a, acc_b, &dav, &dbv);
    if (active) {
      st_row<MB_GLU_BWD_ST>(din + t * pi + col, din + t * pi, static_cast<uint32_t>(col), dav);
      st_row<MB_GLU_BWD_ST>(din + t * pi + po + col, din + t * pi, static_cast<uint32_t>(po + col), dbv);
    }
    if constexpr (DW) {
      rs = wave_sum(active ? rs : 0.0f);
      if (lane == 0) wpart[static_cast<size_t>(ti.strip) * T + t] = rs;
    }
    if constexpr (DBIAS) {
      ca_a.tick(1);
      ca_b.tick(1);
    }
  }
  if constexpr (DBIAS) {
    float sa_[V], sb_[V];
    ca_a.total(sa_);
    ca_b.total(sb_);
    __shared__ float red[kWaves][2 * V][64];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      red[wave][k][lane] = sa_[k];
      red[wave][V + k][lane] = sb_[k];
    }
    __syncthreads();
    if (wave == 0 && active) {
      float sa[V], sb[V];
#pragma unroll
      for (int k = 0; k < V; ++k) {
        sa[k] = ((red[0][k][lane] + red[1][k][lane]) + red[2][k][lane]) + red[3][k][lane];
        sb[k] = ((red[0][V + k][lane] + red[1][V + k][lane]) + red[2][V + k][lane]) + red[3][V + k][lane];
      }
      const size_t C = 2 * static_cast<size_t>(nvec) * V;
      float* dst_a = bpart + static_cast<size_t>(ti.rg) * C + static_cast<size_t>(cv) * V;
      float* dst_b = dst_a + static_cast<size_t>(nvec) * V;
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        store_f32x4(dst_a + 4 * q, sa + 4 * q);
        store_f32x4(dst_b + 4 * q, sb + 4 * q);
      }
    }
  }
}

template <DT D, int ACT, DT W>
hipError_t glu_fwd_dispatch(const void* in, const void* bias, const void* w, void* out, const Tiling& t,
                            hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  auto ip = static_cast<const char*>(in);
  auto bp = static_cast<const char*>(bias);
  auto wp = static_cast<const char*>(w);
  auto op = static_cast<char*>(out);
  if (w)
    hipLaunchKernelGGL((glu_fwd_kernel<D, ACT, true, W, kUnrollFwd>), grid, dim3(kThreads), 0, s, ip, bp, wp, op, t.T,
                       t.nvec);
  else
    hipLaunchKernelGGL((glu_fwd_kernel<D, ACT, false, W, kUnrollFwd>), grid, dim3(kThreads), 0, s, ip, bp, wp, op,
                       t.T, t.nvec);
  return hipGetLastError();
}

template <DT D, int ACT, DT W, bool DBIAS, bool DW>
hipError_t glu_bwd_launch(const char* g, const char* in, const char* bias, const char* w, char* din, float* bp,
                          float* wp, const Tiling& t, hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  if (w)
    hipLaunchKernelGGL((glu_bwd_kernel<D, ACT, true, W, kUnrollBwd, DBIAS, DW>), grid, dim3(kThreads), 0, s, g, in,
                       bias, w, din, bp, wp, t.T, t.nvec);
  else
    hipLaunchKernelGGL((glu_bwd_kernel<D, ACT, false, W, kUnrollBwd, DBIAS, false>), grid, dim3(kThreads), 0, s, g,
                       in, bias, w, din, bp, wp, t.T, t.nvec);
  return hipGetLastError();
}

template <DT D, int ACT, DT W>
hipError_t glu_bwd_dispatch(const void* g, const void* in, const void* bias, const void* w, void* din, float* bp,
                            float* wp, const Tiling& t, hipStream_t s) {
  auto gg = static_cast<const char*>(g);
  auto ii = static_cast<const char*>(in);
  auto bb = static_cast<const char*>(bias);
  auto ww = static_cast<const char*>(w);
  auto dd = static_cast<char*>(din);
  if constexpr (ACT == kSwiGLU) {
    if (bp && wp) return glu_bwd_launch<D, ACT, W, true, true>(gg, ii, bb, ww, dd, bp, wp, t, s);
    if (wp) return glu_bwd_launch<D, ACT, W, false, true>(gg, ii, bb, ww, dd, bp, wp, t, s);
  }
  if (bp) return glu_bwd_launch<D, ACT, W, true, false>(gg, ii, bb, ww, dd, bp, wp, t, s);
  return glu_bwd_launch<D, ACT, W, false, false>(gg, ii, bb, ww, dd, bp, wp, t, s);
}

template <DT D, int ACT>
hipError_t glu_fwd_w(int w_dt, const void* in, const void* bias, const void* w, void* out, const Tiling& t,
                     hipStream_t s) {
  if (static_cast<DT>(w_dt) == DT::F32 || D == DT::F32) return glu_fwd_dispatch<D, ACT, DT::F32>(in, bias, w, out, t, s);
  return glu_fwd_dispatch<D, ACT, D>(in, bias, w, out, t, s);
}

template <DT D, int ACT>
hipError_t glu_bwd_w(int w_dt, const void* g, const void* in, const void* bias, const void* w, void* din, float* bp,
                     float* wp, const Tiling& t, hipStream_t s) {
  if (static_cast<DT>(w_dt) == DT::F32 || D == DT::F32)
    return glu_bwd_dispatch<D, ACT, DT::F32>(g, in, bias, w, din, bp, wp, t, s);
  return glu_bwd_dispatch<D, ACT, D>(g, in, bias, w, din, bp, wp, t, s);
}

}  // namespace

hipError_t launch_glu_fwd(int act, int dt, const void* in, const void* bias, const void* w, int w_dt, void* out,
                          int64_t /*H*/, const Tiling& t, hipStream_t s) {
  const DT D = static_cast<DT>(dt);
  if (act == kSwiGLU) {
    if (D == DT::F32) return glu_fwd_w<DT::F32, kSwiGLU>(w_dt, in, bias, w, out, t, s);
    if (D == DT::F16) return glu_fwd_w<DT::F16, kSwiGLU>(w_dt, in, bias, w, out, t, s);
    if (D == DT::BF16) return glu_fwd_w<DT::BF16, kSwiGLU>(w_dt, in, bias, w, out, t, s);
  } else {
    if (D == DT::F32) return glu_fwd_dispatch<DT::F32, kGEGLU, DT::F32>(in, bias, nullptr, out, t, s);
    if (D == DT::F16) return glu_fwd_dispatch<DT::F16, kGEGLU, DT::F16>(in, bias, nullptr, out, t, s);
    if (D == DT::BF16) return glu_fwd_dispatch<DT::BF16, kGEGLU, DT::BF16>(in, bias, nullptr, out, t, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_glu_bwd(int act, int dt, const void* g, const void* in, const void* bias, const void* w, int w_dt,
                          void* din, float* bias_partials, float* w_partials, int64_t /*H*/, const Tiling& t,
                          hipStream_t s) {
  const DT D = static_cast<DT>(dt);
  if (act == kSwiGLU) {
    if (D == DT::F32) return glu_bwd_w<DT::F32, kSwiGLU>(w_dt, g, in, bias, w, din, bias_partials, w_partials, t, s);
    if (D == DT::F16) return glu_bwd_w<DT::F16, kSwiGLU>(w_dt, g, in, bias, w, din, bias_partials, w_partials, t, s);
    if (D == DT::BF16) return glu_bwd_w<DT::BF16, kSwiGLU>(w_dt, g, in, bias, w, din, bias_partials, w_partials, t, s);
  } else {
    if (D == DT::F32) return glu_bwd_dispatch<DT::F32, kGEGLU, DT::F32>(g, in, bias, nullptr, din, bias_partials, nullptr, t, s);
    if (D == DT::F16) return glu_bwd_dispatch<DT::F16, kGEGLU, DT::F16>(g, in, bias, nullptr, din, bias_partials, nullptr, t, s);
    if (D == DT::BF16) return glu_bwd_dispatch<DT::BF16, kGEGLU, DT::BF16>(g, in, bias, nullptr, din, bias_partials, nullptr, t, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mb
