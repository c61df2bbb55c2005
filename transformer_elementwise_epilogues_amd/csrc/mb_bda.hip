// mb_bda.hip -- bias + dropout + residual add (train, inference, backward) and
// the keep-mask export.
//
// Method: Megatron-LM's _bias_dropout_add_func as described by the wmrh.cn
// article on megatron/core/fusions, section 3.2 (one fused branch; the
// residual is cast to x's dtype first; in-place at inference) and section 3.3
// (separate train and inference entry points).
//
// The keep decision of element i = t*H + j comes from Philox4x32-10 with
// counter (i/4, offset) and key seed: a lane's 4 or 8 elements are exactly 1 or
// 2 Philox blocks, so no random word is wasted and the mask does not depend on
// the launch shape. The residual cast is done in registers (an fp32 residual
// is read once, never materialised in x's dtype).
//
// Elements per lane (EPL): 8 for bf16/fp16 (one 16-byte vector), 4 for fp32,
// and 4 when an fp32 residual (or residual gradient) sits beside bf16/fp16
// activations. With 4, the activations move in 8-byte and the residual in
// 16-byte pieces, so every load and store instruction of a wave covers one
// contiguous 512 B / 1 KiB span. (With 8 elements per lane the fp32 tensor
// would be stored 16 B per lane at a 32 B stride: half-line non-temporal
// stores, measured at under 3 TB/s.)
#include <type_traits>

#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

// rows in flight per wave: the fp32-residual layout (4 elements per lane),
// its training pass and the same-dtype layout are tuned apart
template <DT D, DT R, bool TRAIN> constexpr int unroll() {
  return (R == DT::F32 && D != DT::F32) ? (TRAIN ? MB_BDA_MIXED_TRAIN_UNROLL : MB_BDA_MIXED_UNROLL) : MB_BDA_UNROLL;
}

template <DT D, DT R>
constexpr int epl() {
  return (R == DT::F32 && D != DT::F32) ? 4 : Vec<D>::N;
}

// Cache policy of the streaming stores (st_row: -1 global nt, 2 buffer nt,
// 18 buffer nt sc1), by measurement: the forward gained 1-5 % with buffer
// nt sc1 stores, the fp32-residual backward 1.8 %; the same-dtype backward
// was 0.5 % slower with them.
#ifndef MB_BDA_ST
#define MB_BDA_ST 18
#endif
#ifndef MB_BDA_BWD_ST
#define MB_BDA_BWD_ST -1
#endif
#ifndef MB_BDA_BWD_MIXED_ST
#define MB_BDA_BWD_MIXED_ST 18
#endif
template <DT D, DT R> constexpr int st_bwd() { return (R == DT::F32 && D != DT::F32) ? MB_BDA_BWD_MIXED_ST : MB_BDA_BWD_ST; }

#ifndef MB_BDA_BWD_PIPELINE
#define MB_BDA_BWD_PIPELINE 1
#endif

// Non-temporal load of a packed 8- or 16-byte piece, and its unpacking into
// N elements of D (4 bf16/fp16 in 8 bytes, or a full 16-byte vector).
template <typename Raw> __device__ __forceinline__ Raw ld_raw(const char* p) {
  if constexpr (MB_NT_LOAD) return __builtin_nontemporal_load(reinterpret_cast<const Raw*>(p));
  return *reinterpret_cast<const Raw*>(p);
}
__device__ __forceinline__ u32x4 widen(u32x4 v) { return v; }
__device__ __forceinline__ u32x4 widen(u32x2 v) {
  const unsigned a = v.x, b = v.y;
  return u32x4{a, b, 0u, 0u};
}
template <DT D, int N, typename Raw> __device__ __forceinline__ void unpack_raw(Raw v, float* f) {
  float t[Vec<D>::N];
  unpack<D>(widen(v), t);
#pragma unroll
  for (int k = 0; k < N; ++k) f[k] = t[k];
}

// Keep flags of N consecutive elements starting at i0 (a multiple of 4).
template <int N>
__device__ __forceinline__ void keep_n(uint64_t i0, const DropoutArgs& d, bool* keep) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) keep4((i0 >> 2) + q, d.o0, d.o1, d.k0, d.k1, d.theta32, d.drop_all, keep + 4 * q);
}

// Forward. The U rows' loads are issued before any of their stores.
template <DT D, DT R, bool TRAIN, int U>
__global__ __launch_bounds__(kThreads) void bda_kernel(const char* x, const char* bias, const char* res, char* out,
                                                       int64_t T, int lanes, int64_t H, DropoutArgs d) {
  constexpr int N = epl<D, R>();
  constexpr int XB = N * Vec<D>::BYTES, RB = N * Vec<R>::BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(MB_BDA_ST >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  if (cv >= lanes) return;
  float b[N];
  if (bias) {
    ld_elems<D, N>(bias + static_cast<size_t>(cv) * XB, b);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) b[k] = 0.0f;
  }
  const size_t px = static_cast<size_t>(lanes) * XB, pr = static_cast<size_t>(lanes) * RB;
  const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
  const char* xp = x + static_cast<size_t>(cv) * XB;
  const char* rp = res + static_cast<size_t>(cv) * RB;
  char* op = out + static_cast<size_t>(cv) * XB;
  const uint64_t j0 = static_cast<uint64_t>(cv) * N;
  int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
  for (; t < T; t += U * S) {
    // rows t, t+S, ... (at most U of them); the loads of all of them first
    float xv[U][N], rv[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u * S < T) {
        ld_elems<D, N>(xp + (t + u * S) * px, xv[u]);
        ld_elems<R, N>(rp + (t + u * S) * pr, rv[u]);
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tt = t + u * S;
      if (tt >= T) break;
      bool keep[N];
      if constexpr (TRAIN) keep_n<N>(static_cast<uint64_t>(tt) * static_cast<uint64_t>(H) + j0, d, keep);
      float o[N];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        const float r2 = (R == D) ? rv[u][k] : round_to<D>(rv[u][k]);
        const float z = xv[u][k] + b[k];
        if constexpr (TRAIN)
          o[k] = __builtin_fmaf(keep[k] ? z : 0.0f, d.scale, r2);
        else
          o[k] = r2 + z;
      }
      st_row_elems<D, N, MB_BDA_ST>(op + tt * px, out + tt * px, static_cast<uint32_t>(cv) * XB, o);
    }
  }
}

// Backward: dx = keep ? g * s : 0 with the keep decisions regenerated from
// (seed, offset, element index); dresidual = g in the residual's dtype; the
// fp32 dx values are summed per column into one partial row per row group.
// Row order of the backward: strided (a wave's U rows in flight are S apart,
// so the grid sweeps one band of rows) or banded (the U rows come from U
// equal bands of the tensor, so U bands are swept at once). Banded streamed
// 3 % faster for the same-dtype backward at [16384, 8192] and 3 % slower for
// the fp32-residual one at [8192, 4096] (MI355X, two allocation layouts).
#ifndef MB_BDA_BWD_BANDED
#define MB_BDA_BWD_BANDED 1
#endif
template <DT D, DT R> constexpr bool banded_bwd() { return MB_BDA_BWD_BANDED && !(R == DT::F32 && D != DT::F32); }

template <DT D, DT R, int U, bool DBIAS, bool DRES>
__global__ __launch_bounds__(kThreads) void bda_bwd_kernel(const char* g, char* dx, char* dres, float* partials,
                                                           int64_t T, int lanes, int64_t H, DropoutArgs d) {
  // the lane layout depends on the dtypes only, so dx and dbias come out bit
  // for bit the same whether or not the residual gradient is requested
  constexpr int N = epl<D, R>();
  constexpr int XB = N * Vec<D>::BYTES, RB = N * Vec<R>::BYTES;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index<(st_bwd<D, R>() >= 0)>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  const bool active = cv < lanes;
  ColAcc<N> ca;
  ca.init();
  if (active) {
    const size_t px = static_cast<size_t>(lanes) * XB, pr = static_cast<size_t>(lanes) * RB;
    const size_t cx = static_cast<size_t>(cv) * XB, cr = static_cast<size_t>(cv) * RB;
    const int64_t S = static_cast<int64_t>(ti.G) * kWaves;
    const uint64_t j0 = static_cast<uint64_t>(cv) * N;
    int64_t t = static_cast<int64_t>(ti.rg) * kWaves + wave;
    // raw (packed) g of U rows; the next U rows are loaded before this U rows'
    // mask and arithmetic (software pipeline), so memory stays busy while the
    // Philox rounds run
    using Raw = typename std::conditional<N * Vec<D>::BYTES == 16, u32x4, u32x2>::type;
    auto fetch = [&](int64_t t0, Raw* gr) {
#pragma unroll
      for (int u = 0; u < U; ++u) gr[u] = ld_raw<Raw>(g + (t0 + u * S) * px + cx);
    };
    auto row = [&](int64_t tt, Raw graw) {
      float gv[N];
      unpack_raw<D, N>(graw, gv);
      if constexpr (DRES) st_row_elems<R, N, st_bwd<D, R>()>(dres + tt * pr + cr, dres + tt * pr, static_cast<uint32_t>(cr), gv);  // exact: g widened or copied
      bool keep[N];
      keep_n<N>(static_cast<uint64_t>(tt) * static_cast<uint64_t>(H) + j0, d, keep);
      float f[N];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        f[k] = keep[k] ? gv[k] * d.scale : 0.0f;
        ca.lo[k] += f[k];
      }
      st_row_elems<D, N, st_bwd<D, R>()>(dx + tt * px + cx, dx + tt * px, static_cast<uint32_t>(cx), f);
    };
    auto rows = [&](int64_t t0, const Raw* gr) {
      row(t0, gr[0]);
      if constexpr (U > 1) row(t0 + S, gr[1]);
      if constexpr (U > 2) row(t0 + 2 * S, gr[2]);
      if constexpr (U > 3) row(t0 + 3 * S, gr[3]);
      if constexpr (DBIAS) ca.tick(U);
    };
    static_assert(U >= 1 && U <= 4, "1 to 4 rows in flight");
    if constexpr (banded_bwd<D, R>()) {
      // the U rows in flight come from U bands of TB rows: slot u of base j
      // is row u TB + j (the last band may be shorter)
      const int64_t TB = (T + U - 1) / U;
      auto fetch_b = [&](int64_t j, Raw* gr) {
#pragma unroll
        for (int u = 0; u < U; ++u) gr[u] = ld_raw<Raw>(g + (u * TB + j) * px + cx);
      };
      auto rows_b = [&](int64_t j, const Raw* gr) {
#pragma unroll
        for (int u = 0; u < U; ++u) row(u * TB + j, gr[u]);
        if constexpr (DBIAS) ca.tick(U);
      };
      int64_t j = t;
      if (j < TB && (U - 1) * TB + j < T) {
        Raw gr[U];
        fetch_b(j, gr);
        for (;;) {
          const int64_t jn = j + S;
          if (jn < TB && (U - 1) * TB + jn < T) {
            Raw gn[U];
            fetch_b(jn, gn);
            rows_b(j, gr);
#pragma unroll
            for (int u = 0; u < U; ++u) gr[u] = gn[u];
            j = jn;
          } else {
            rows_b(j, gr);
            j = jn;
            break;
          }
        }
      }
      for (; j < TB; j += S) {
        for (int u = 0; u < U; ++u) {
          const int64_t tt = u * TB + j;
          if (tt < T) {
            row(tt, ld_raw<Raw>(g + tt * px + cx));
            if constexpr (DBIAS) ca.tick(1);
          }
        }
      }
    } else {
      if (t + (U - 1) * S < T) {
        Raw gr[U];
        fetch(t, gr);
        for (;;) {
          const int64_t tn = t + U * S;
          if (tn + (U - 1) * S < T) {  // steady state: the next rows' loads always go first
            Raw gn[U];
            if constexpr (MB_BDA_BWD_PIPELINE) {
              fetch(tn, gn);
              rows(t, gr);
            } else {
              rows(t, gr);
              fetch(tn, gn);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) gr[u] = gn[u];
            t = tn;
          } else {
            rows(t, gr);
            t = tn;
            break;
          }
        }
      }
      for (; t < T; t += S) {
        row(t, ld_raw<Raw>(g + t * px + cx));
        if constexpr (DBIAS) ca.tick(1);
      }
    }
  }
  float acc[N];
  ca.total(acc);
  if constexpr (DBIAS)
    block_column_partials<N>(acc, wave, lane, active,
                             partials + static_cast<size_t>(ti.rg) * lanes * N + static_cast<size_t>(cv) * N);
}

// One byte (8 elements) per thread; n is a multiple of 4.
__global__ __launch_bounds__(256) void mask_kernel(uint8_t* bits, int64_t n, DropoutArgs d) {
  const int64_t byte = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbytes = (n + 7) / 8;
  if (byte >= nbytes) return;
  const int64_t i0 = byte * 8;
  bool keep[8] = {false, false, false, false, false, false, false, false};
  keep4(static_cast<uint64_t>(i0) >> 2, d.o0, d.o1, d.k0, d.k1, d.theta32, d.drop_all, keep);
  if (i0 + 4 < n) keep4((static_cast<uint64_t>(i0) >> 2) + 1, d.o0, d.o1, d.k0, d.k1, d.theta32, d.drop_all, keep + 4);
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
    hipLaunchKernelGGL((bda_kernel<D, R, true, unroll<D, R, true>()>), grid, dim3(kThreads), 0, s, xp, bp, rp, op, t.T, t.nvec, H, d);
  else
    hipLaunchKernelGGL((bda_kernel<D, R, false, unroll<D, R, false>()>), grid, dim3(kThreads), 0, s, xp, bp, rp, op, t.T, t.nvec, H, d);
  return hipGetLastError();
}

template <DT D, DT R>
hipError_t bda_bwd_dispatch(const void* g, void* dx, void* dres, float* partials, int64_t H, const Tiling& t,
                            const DropoutArgs& d, hipStream_t s) {
  const dim3 grid = tile_grid(t.strips, t.G);
  auto gp = static_cast<const char*>(g);
  auto xp = static_cast<char*>(dx);
  auto rp = static_cast<char*>(dres);
  constexpr int U = (R == DT::F32 && D != DT::F32) ? MB_BDA_BWD_MIXED_UNROLL : MB_BDA_BWD_UNROLL;
  constexpr int UN = MB_BDA_BWD_NODBIAS_UNROLL;  // rows in flight without the bias gradient
  if (partials && dres)
    hipLaunchKernelGGL((bda_bwd_kernel<D, R, U, true, true>), grid, dim3(kThreads), 0, s, gp, xp, rp, partials, t.T, t.nvec, H, d);
  else if (partials)
    hipLaunchKernelGGL((bda_bwd_kernel<D, R, U, true, false>), grid, dim3(kThreads), 0, s, gp, xp, rp, partials, t.T, t.nvec, H, d);
  else if (dres)
    hipLaunchKernelGGL((bda_bwd_kernel<D, R, UN, false, true>), grid, dim3(kThreads), 0, s, gp, xp, rp, partials, t.T, t.nvec, H, d);
  else
    hipLaunchKernelGGL((bda_bwd_kernel<D, R, UN, false, false>), grid, dim3(kThreads), 0, s, gp, xp, rp, partials, t.T, t.nvec, H, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bda_bwd(int dt, int res_dt, const void* g, void* dx, void* dres, float* partials, int64_t H,
                          const Tiling& t, const DropoutArgs& d, hipStream_t s) {
  const DT D = static_cast<DT>(dt), R = static_cast<DT>(res_dt);
  if (D == DT::F32 && R == DT::F32) return bda_bwd_dispatch<DT::F32, DT::F32>(g, dx, dres, partials, H, t, d, s);
  if (D == DT::BF16 && R == DT::BF16) return bda_bwd_dispatch<DT::BF16, DT::BF16>(g, dx, dres, partials, H, t, d, s);
  if (D == DT::BF16 && R == DT::F32) return bda_bwd_dispatch<DT::BF16, DT::F32>(g, dx, dres, partials, H, t, d, s);
  if (D == DT::F16 && R == DT::F16) return bda_bwd_dispatch<DT::F16, DT::F16>(g, dx, dres, partials, H, t, d, s);
  if (D == DT::F16 && R == DT::F32) return bda_bwd_dispatch<DT::F16, DT::F32>(g, dx, dres, partials, H, t, d, s);
  return hipErrorInvalidValue;
}

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
