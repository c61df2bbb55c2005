// mb_ln.hip -- residual add + LayerNorm, forward and backward, on gfx950.
//
// [fusions §5]: Megatron-LM wraps a fused LayerNorm (a persistent kernel for a
// fixed list of hidden sizes up to 65536, eps in the denominator, optional
// zero-centred gamma used as weight + 1). Here it is fused with the residual
// add in front of it, the step that follows the bias-dropout-add on both
// residual paths of a layer:
//   h = x + residual'   (residual cast to x's dtype first, h rounded to it)
//   y = (h - mean) * rstd * gamma' + beta,   rstd = 1 / sqrt(var + eps)
// with the biased (1/H) variance of the ROUNDED h.
//
// A row is normalised by one group of TPR threads (64, 256 or 1024) that holds
// it in registers: thread l of the group owns the 16-byte vectors l, l + TPR,
// ..., l + (NV-1) TPR of the row (E elements each), so every load and store
// instruction of a wave covers one contiguous span. Row sums are a wave
// butterfly and, across the group's waves, a fixed-order sum through LDS,
// so results do not depend on scheduling. Groups of 64 threads run 4 rows per
// block with no barrier at all. The mean and the variance are two passes over
// the registers (no E[h^2] - E[h]^2 cancellation).
//
// The backward reads the forward's mean and rstd and computes, with
// a = dy * gamma' and xhat = (h - mean) * rstd,
//   dh = rstd * (a - mean_j a - xhat * mean_j (a xhat)) + dh_in
// stored to dx (x's dtype) and optionally to dresidual (the residual's dtype).
// dgamma = sum_t dy xhat and dbeta = sum_t dy accumulate per thread over the
// block's rows (a block owns the same columns on every row it visits), are
// written as one partial row per block, and summed in a fixed order by the
// column-sum passes. Rows of more than 1024 vectors leave no registers for
// those sums beside a register-resident row: their backward is two kernels,
// a row-sum kernel and a column-strip kernel (see "wide rows" below).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "mb_device.hpp"
#include "mb_launch.hpp"

namespace mb {

namespace {

// Elements per vector: 4 when an fp32 residual sits beside 16-bit activations
// (8-byte activation pieces, 16-byte residual pieces), else one 16-byte vector.
template <DT D, DT R> constexpr int ln_epl() { return (R == DT::F32 && D != DT::F32) ? 4 : Vec<D>::N; }

// E elements of D kept packed in registers (8 or 16 bytes): rows live in
// registers in their storage format and are unpacked for each pass, which is
// exact for h (it is rounded to D by definition) and for dy and gamma.
template <DT D, int E> struct Pk {
  static constexpr int BYTES = E * Vec<D>::BYTES;
  static_assert(BYTES == 8 || BYTES == 16, "8- or 16-byte pieces");
  using T = typename std::conditional<BYTES == 16, u32x4, u32x2>::type;
};

template <DT D, int E> __device__ __forceinline__ typename Pk<D, E>::T pk_load(const char* p) {
  using T = typename Pk<D, E>::T;
  if constexpr (MB_NT_LOAD) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  return *reinterpret_cast<const T*>(p);
}
template <DT D, int E> __device__ __forceinline__ typename Pk<D, E>::T pk_load_keep(const char* p) {
  return *reinterpret_cast<const typename Pk<D, E>::T*>(p);
}
template <DT D, int E> __device__ __forceinline__ void pk_store(char* p, typename Pk<D, E>::T v) {
  using T = typename Pk<D, E>::T;
  if constexpr (MB_NT_STORE)
    __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
  else
    *reinterpret_cast<T*>(p) = v;
}
// A packed piece at byte voff + soff of the `bytes`-byte buffer at base, read
// through a buffer descriptor (a read past `bytes` returns zeros): the lane's
// offset is one register and a per-vector step a scalar, where the compiler
// would keep a 64-bit address per vector, hoisted out of a loop, in registers.
template <DT D, int E>
__device__ __forceinline__ typename Pk<D, E>::T pk_load_rsrc(const char* base, uint32_t bytes, uint32_t voff,
                                                             uint32_t soff, bool nt) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, 0x00020000);
  if constexpr (Pk<D, E>::BYTES == 16) {
    return nt ? __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2) : __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  } else {
    return nt ? __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2) : __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  }
}

template <DT D, int E> __device__ __forceinline__ void pk_unpack(typename Pk<D, E>::T v, float* f) {
  if constexpr (Pk<D, E>::BYTES == 16) {
    unpack<D>(v, f);
  } else {
    const unsigned v0 = v.x, v1 = v.y;
    const u32x4 w = {v0, v1, 0u, 0u};
    float t[8];
    unpack<D>(w, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = t[e];
  }
}
template <DT D, int E> __device__ __forceinline__ typename Pk<D, E>::T pk_pack(const float* f) {
  if constexpr (Pk<D, E>::BYTES == 16) {
    return pack<D>(f);
  } else {
    const unsigned w0 = D == DT::BF16 ? pk_bf16(f[0], f[1]) : pk_f16(f[0], f[1]);
    const unsigned w1 = D == DT::BF16 ? pk_bf16(f[2], f[3]) : pk_f16(f[2], f[3]);
    return typename Pk<D, E>::T{w0, w1};
  }
}

// Makes the compiler treat a packed value as changed, so that a later pass
// unpacks it again instead of keeping the unpacked floats of an earlier pass
// alive across the row reduction (twice the registers). Emits no instruction.
template <typename V> __device__ __forceinline__ void opaque(V& v) { asm volatile("" : "+v"(v)); }

// LDS of the in-row reductions: [row in block][slot][wave of the row].
template <int W, int RPB> struct RowLds {
  float v[RPB][4][W];
};

// Sum of `v` over the row group's W waves. W == 1: a wave butterfly, no
// barrier. W > 1: every thread of the block must call it (RPB is 1 then).
template <int W, int RPB>
__device__ __forceinline__ float row_sum(float v, RowLds<W, RPB>& lds, int sub, int wr, int lane, int slot) {
  v = wave_sum(v);
  if constexpr (W == 1) {
    return v;
  } else {
    if (lane == 0) lds.v[sub][slot][wr] = v;
    __syncthreads();
    float t = lds.v[sub][slot][0];
#pragma unroll
    for (int w = 1; w < W; ++w) t += lds.v[sub][slot][w];
    return t;
  }
}

// Two sums with one barrier (slots `slot`, `slot + 1`).
template <int W, int RPB>
__device__ __forceinline__ void row_sum2(float& a, float& b, RowLds<W, RPB>& lds, int sub, int wr, int lane,
                                         int slot) {
  a = wave_sum(a);
  b = wave_sum(b);
  if constexpr (W > 1) {
    if (lane == 0) {
      lds.v[sub][slot][wr] = a;
      lds.v[sub][slot + 1][wr] = b;
    }
    __syncthreads();
    a = lds.v[sub][slot][0];
    b = lds.v[sub][slot + 1][0];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      a += lds.v[sub][slot][w];
      b += lds.v[sub][slot + 1][w];
    }
  }
}

#ifndef MB_LN_PREFETCH
#define MB_LN_PREFETCH 1
#endif
// The next row is prefetched into registers, except for rows of 4096 or more
// vectors (1024 threads of 4 or 8, 512 threads of 8), which have no registers
// to spare.
template <int TPR, int NV> constexpr bool prefetch() { return MB_LN_PREFETCH && TPR * NV < 4096; }

// Parameters (gamma, beta) stay packed in registers unless the row slice is
// the widest one (8 vectors per thread), where they are re-read from cache.
// Re-reading them for every row at 4 vectors per thread as well (130 VGPRs
// against 182, 3 waves per SIMD against 2) was 5-8 % slower on MI355X.
template <int NV> constexpr bool hold_params() { return NV <= 4; }

template <DT D, DT R, int TPR, int NV, int RPB>
__global__ __launch_bounds__(TPR* RPB) void ln_fwd_kernel(const char* __restrict__ x, const char* __restrict__ res,
                                                           const char* __restrict__ gamma,
                                                           const char* __restrict__ beta, char* hout, char* y,
                                                           float* __restrict__ mean_out,
                                                           float* __restrict__ rstd_out, int64_t T, int H,
                                                           float eps, float gshift) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  constexpr bool HOLD = hold_params<NV>();
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ RowLds<W, RPB> lds;
  const int tid = threadIdx.x, sub = tid / TPR, lt = tid % TPR, wr = lt / 64, lane = tid & 63;
  const int nvec = H / E;
  const float fh = static_cast<float>(H);

  int vc[NV];   // clamped vector index (always in bounds)
  bool ok[NV];  // the vector exists in the row
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = lt + k * TPR;
    ok[k] = v < nvec;
    vc[k] = ok[k] ? v : 0;
  }
  PD gp[HOLD ? NV : 1], bp[HOLD ? NV : 1];
  if constexpr (HOLD) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gp[k] = pk_load_keep<D, E>(gamma + static_cast<size_t>(vc[k]) * XB);
      bp[k] = beta ? pk_load_keep<D, E>(beta + static_cast<size_t>(vc[k]) * XB) : PD{};
    }
  }

  const int64_t step = static_cast<int64_t>(gridDim.x) * RPB;
  // the next row's x and residual are loaded while this row is reduced
  PD xn[NV];
  PR rn[NV];
  auto fetch = [&](int64_t r) {
    const size_t xo = static_cast<size_t>(r) * H * Vec<D>::BYTES;
    const size_t ro = static_cast<size_t>(r) * H * Vec<R>::BYTES;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      xn[k] = pk_load<D, E>(x + xo + static_cast<size_t>(vc[k]) * XB);
      rn[k] = pk_load<R, E>(res + ro + static_cast<size_t>(vc[k]) * RB);
    }
  };
  int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + sub;
  if (row < T) fetch(row);
  for (; row < T; row += step) {
    const size_t xo = static_cast<size_t>(row) * H * Vec<D>::BYTES;
    PD xp[NV];
    PR rp[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      xp[k] = xn[k];
      rp[k] = rn[k];
    }
    if constexpr (prefetch<TPR, NV>()) {
      if (row + step < T) fetch(row + step);
    }
    PD hp[NV];  // h, rounded to D
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float xv[E], rv[E];
      pk_unpack<D, E>(xp[k], xv);
      pk_unpack<R, E>(rp[k], rv);
#pragma unroll
      for (int e = 0; e < E; ++e) xv[e] += R == D ? rv[e] : round_to<D>(rv[e]);
      hp[k] = pk_pack<D, E>(xv);
      if (hout && ok[k]) pk_store<D, E>(hout + xo + static_cast<size_t>(vc[k]) * XB, hp[k]);
      float hv[E];
      pk_unpack<D, E>(hp[k], hv);
#pragma unroll
      for (int e = 0; e < E; ++e) s += ok[k] ? hv[e] : 0.0f;
    }
    const float mean = row_sum<W, RPB>(s, lds, sub, wr, lane, 0) / fh;
#pragma unroll
    for (int k = 0; k < NV; ++k) opaque(hp[k]);
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float hv[E];
      pk_unpack<D, E>(hp[k], hv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = hv[e] - mean;
        ss += ok[k] ? d * d : 0.0f;
      }
    }
    const float var = row_sum<W, RPB>(ss, lds, sub, wr, lane, 1) / fh;
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);
#pragma unroll
    for (int k = 0; k < NV; ++k) opaque(hp[k]);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!ok[k]) continue;
      float hv[E], g[E], b[E];
      pk_unpack<D, E>(hp[k], hv);
      if constexpr (HOLD) {
        pk_unpack<D, E>(gp[k], g);
        pk_unpack<D, E>(bp[k], b);
      } else {
        pk_unpack<D, E>(pk_load_keep<D, E>(gamma + static_cast<size_t>(vc[k]) * XB), g);
        if (beta) {
          pk_unpack<D, E>(pk_load_keep<D, E>(beta + static_cast<size_t>(vc[k]) * XB), b);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) b[e] = 0.0f;
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) hv[e] = __builtin_fmaf((hv[e] - mean) * rstd, g[e] + gshift, b[e]);
      pk_store<D, E>(y + xo + static_cast<size_t>(vc[k]) * XB, pk_pack<D, E>(hv));
    }
    if (lt == 0 && mean_out) {
      mean_out[row] = mean;
      rstd_out[row] = rstd;
    }
    if constexpr (!prefetch<TPR, NV>()) {
      if (row + step < T) fetch(row + step);
    }
  }
}

// The forward of the widest rows (8192 vectors): h goes to LDS (each thread
// writes and reads only its own vectors, slot k TPR + l, so it needs no
// barrier of its own), which leaves the registers to the next row's x and
// residual, loaded while this row is reduced and its y stored. Blocks stay
// resident (one per CU) and walk rows. LDS: TPR NV h pieces (128 KiB for a
// 65536-element bf16 row).
template <DT D, DT R, int TPR, int NV>
__global__ __launch_bounds__(TPR) void ln_fwd_lds_kernel(const char* __restrict__ x, const char* __restrict__ res,
                                                         const char* __restrict__ gamma, const char* __restrict__ beta,
                                                         char* hout, char* y, float* __restrict__ mean_out,
                                                         float* __restrict__ rstd_out, int64_t T, int H, float eps,
                                                         float gshift) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ RowLds<W, 1> lds;
  extern __shared__ __align__(16) unsigned char hrow_raw[];
  PD* hrow = reinterpret_cast<PD*>(hrow_raw);
  const int lt = threadIdx.x, wr = lt / 64, lane = lt & 63;
  const int nvec = H / E;
  const float fh = static_cast<float>(H);
  // Vector k of this thread is lt + k TPR (clamped to 0 past the row, where
  // it is loaded but neither stored nor counted). Addresses are a row base,
  // the same for the whole block, plus a 32-bit offset: the per-vector
  // offsets are then one register each, where 64-bit addresses of every
  // vector of two tensors, hoisted out of the row loop, would not fit.
  auto in_row = [&](int k) { return lt + k * TPR < nvec; };
  auto vec_of = [&](int k) { return static_cast<uint32_t>(in_row(k) ? lt + k * TPR : 0); };
  const int64_t step = gridDim.x;
  const size_t px = static_cast<size_t>(H) * Vec<D>::BYTES, pr = static_cast<size_t>(H) * Vec<R>::BYTES;
  PD xn[NV];
  PR rn[NV];
  const uint32_t xbytes = static_cast<uint32_t>(nvec) * XB, rbytes = static_cast<uint32_t>(nvec) * RB;
  auto fetch = [&](int64_t r) {
    const char* xr = x + static_cast<size_t>(r) * px;
    const char* rr = res + static_cast<size_t>(r) * pr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {  // past the row: zeros, neither stored nor counted
      xn[k] = pk_load_rsrc<D, E>(xr, xbytes, lt * XB, k * TPR * XB, MB_NT_LOAD);
      rn[k] = pk_load_rsrc<R, E>(rr, rbytes, lt * RB, k * TPR * RB, MB_NT_LOAD);
    }
  };
  int64_t row = blockIdx.x;
  if (row < T) fetch(row);
  for (; row < T; row += step) {
    char* hr = hout ? hout + static_cast<size_t>(row) * px : nullptr;
    char* yr = y + static_cast<size_t>(row) * px;
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float xv[E], rv[E];
      pk_unpack<D, E>(xn[k], xv);
      pk_unpack<R, E>(rn[k], rv);
#pragma unroll
      for (int e = 0; e < E; ++e) xv[e] += R == D ? rv[e] : round_to<D>(rv[e]);
      const PD hp = pk_pack<D, E>(xv);
      hrow[k * TPR + lt] = hp;
      if (hr && in_row(k)) pk_store<D, E>(hr + vec_of(k) * static_cast<uint32_t>(XB), hp);
      float hv[E];
      pk_unpack<D, E>(hp, hv);
#pragma unroll
      for (int e = 0; e < E; ++e) s += in_row(k) ? hv[e] : 0.0f;
    }
    // the registers are free: the next row's loads go out now (the scheduling
    // barrier keeps the compiler from hoisting them above the pass that still
    // reads this row's registers, which would need both rows in registers)
    __builtin_amdgcn_sched_barrier(0);
    if (row + step < T) fetch(row + step);
    const float mean = row_sum<W, 1>(s, lds, 0, wr, lane, 0) / fh;
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float hv[E];
      pk_unpack<D, E>(hrow[k * TPR + lt], hv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = hv[e] - mean;
        ss += in_row(k) ? d * d : 0.0f;
      }
    }
    const float var = row_sum<W, 1>(ss, lds, 0, wr, lane, 1) / fh;
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      const uint32_t cv = vec_of(k) * static_cast<uint32_t>(XB);
      float hv[E], g[E], b[E];
      pk_unpack<D, E>(hrow[k * TPR + lt], hv);
      pk_unpack<D, E>(pk_load_rsrc<D, E>(gamma, xbytes, lt * XB, k * TPR * XB, false), g);
      if (beta) {
        pk_unpack<D, E>(pk_load_rsrc<D, E>(beta, xbytes, lt * XB, k * TPR * XB, false), b);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) b[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) hv[e] = __builtin_fmaf((hv[e] - mean) * rstd, g[e] + gshift, b[e]);
      pk_store<D, E>(yr + cv, pk_pack<D, E>(hv));
    }
    if (lt == 0 && mean_out) {
      mean_out[row] = mean;
      rstd_out[row] = rstd;
    }
  }
}

template <DT D, DT R, int TPR, int NV, int RPB, bool DGB>
__global__ __launch_bounds__(TPR* RPB) void ln_bwd_kernel(const char* __restrict__ dy, const char* __restrict__ h,
                                                           const char* __restrict__ gamma,
                                                           const float* __restrict__ mean,
                                                           const float* __restrict__ rstd, const char* dh_in,
                                                           char* dx, char* dres, float* __restrict__ pg,
                                                           float* __restrict__ pb, int64_t T, int H, float gshift) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  constexpr bool HOLD = hold_params<NV>();
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ RowLds<W, RPB> lds;
  const int tid = threadIdx.x, sub = tid / TPR, lt = tid % TPR, wr = lt / 64, lane = tid & 63;
  const int nvec = H / E;
  const float fh = static_cast<float>(H);

  int vc[NV];
  bool ok[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = lt + k * TPR;
    ok[k] = v < nvec;
    vc[k] = ok[k] ? v : 0;
  }
  PD gp[HOLD ? NV : 1];
  if constexpr (HOLD) {
#pragma unroll
    for (int k = 0; k < NV; ++k) gp[k] = pk_load_keep<D, E>(gamma + static_cast<size_t>(vc[k]) * XB);
  }
  // parameter-gradient sums in registers, added every kFlushRows rows into a
  // second level in LDS ([RPB][2][H] floats, each touched by its owning
  // thread only, so no barrier is needed), so that their rounding error does
  // not grow with the rows a block visits
  constexpr bool REG = DGB;
  extern __shared__ float lds_acc[];
  float ag[REG ? NV : 1][E], ab[REG ? NV : 1][E];
  float* hig = lds_acc + static_cast<size_t>(sub) * 2 * H;
  float* hib = hig + H;
  int nrows = 0;
  if constexpr (REG) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) ag[k][e] = ab[k][e] = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (ok[k])
#pragma unroll
        for (int e = 0; e < E; ++e) hig[vc[k] * E + e] = hib[vc[k] * E + e] = 0.0f;
  }

  int slot = 0;  // alternates between the two pairs of LDS slots by row
  const int64_t step = static_cast<int64_t>(gridDim.x) * RPB;
  // the next row's dy, h (and dh_in) are loaded while this row is reduced
  PD gyn[NV], hn[NV];
  PR upn[HOLD ? NV : 1];
  float mun = 0.0f, rsn = 0.0f;
  auto fetch = [&](int64_t r) {
    const size_t xo = static_cast<size_t>(r) * H * Vec<D>::BYTES;
    const size_t ro = static_cast<size_t>(r) * H * Vec<R>::BYTES;
    mun = mean[r];
    rsn = rstd[r];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gyn[k] = pk_load<D, E>(dy + xo + static_cast<size_t>(vc[k]) * XB);
      hn[k] = pk_load<D, E>(h + xo + static_cast<size_t>(vc[k]) * XB);
    }
    if constexpr (HOLD) {
      if (dh_in) {
#pragma unroll
        for (int k = 0; k < NV; ++k) upn[k] = pk_load<R, E>(dh_in + ro + static_cast<size_t>(vc[k]) * RB);
      }
    }
  };
  int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + sub;
  if (row < T) fetch(row);
  for (; row < T; row += step) {
    const size_t xo = static_cast<size_t>(row) * H * Vec<D>::BYTES;
    const size_t ro = static_cast<size_t>(row) * H * Vec<R>::BYTES;
    const float mu = mun, rs = rsn;
    PD gyp[NV], hp[NV];
    PR up[HOLD ? NV : 1];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gyp[k] = gyn[k];
      hp[k] = hn[k];
      if constexpr (HOLD) up[k] = upn[k];
    }
    if constexpr (prefetch<TPR, NV>()) {
      if (row + step < T) fetch(row + step);
    }
    // pass 1: the two row sums (and the parameter-gradient terms)
    float sa = 0.0f, sax = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float gv[E], hv[E], g[E];
      pk_unpack<D, E>(gyp[k], gv);
      pk_unpack<D, E>(hp[k], hv);
      pk_unpack<D, E>(HOLD ? gp[k] : pk_load_keep<D, E>(gamma + static_cast<size_t>(vc[k]) * XB), g);
      float xa[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = (hv[e] - mu) * rs;
        const float dyv = ok[k] ? gv[e] : 0.0f;
        const float a = dyv * (g[e] + gshift);
        sa += a;
        sax = __builtin_fmaf(a, xv, sax);
        xa[e] = xv;
        gv[e] = dyv;
      }
      if constexpr (REG) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ag[k][e] = __builtin_fmaf(gv[e], xa[e], ag[k][e]);
          ab[k][e] += gv[e];
        }
      }
    }
    row_sum2<W, RPB>(sa, sax, lds, sub, wr, lane, slot);
    slot ^= 2;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      opaque(gyp[k]);
      opaque(hp[k]);
      if constexpr (HOLD) opaque(gp[k]);
    }
    const float ma = sa / fh, mx = sax / fh;
    // pass 2: recompute a and xhat from the packed row, form dh
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!ok[k]) continue;
      float gv[E], hv[E], g[E], u[E];
      pk_unpack<D, E>(gyp[k], gv);
      pk_unpack<D, E>(hp[k], hv);
      pk_unpack<D, E>(HOLD ? gp[k] : pk_load_keep<D, E>(gamma + static_cast<size_t>(vc[k]) * XB), g);
      if (dh_in) {
        if constexpr (HOLD) pk_unpack<R, E>(up[k], u);
        else pk_unpack<R, E>(pk_load<R, E>(dh_in + ro + static_cast<size_t>(vc[k]) * RB), u);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) u[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = (hv[e] - mu) * rs;
        const float a = gv[e] * (g[e] + gshift);
        gv[e] = __builtin_fmaf(rs, __builtin_fmaf(-xv, mx, a - ma), u[e]);
      }
      pk_store<D, E>(dx + xo + static_cast<size_t>(vc[k]) * XB, pk_pack<D, E>(gv));
      if (dres) pk_store<R, E>(dres + ro + static_cast<size_t>(vc[k]) * RB, pk_pack<R, E>(gv));
    }
    if constexpr (REG) {
      if (++nrows == kFlushRows) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          if (ok[k]) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              hig[vc[k] * E + e] += ag[k][e];
              hib[vc[k] * E + e] += ab[k][e];
            }
          }
#pragma unroll
          for (int e = 0; e < E; ++e) ag[k][e] = ab[k][e] = 0.0f;
        }
        nrows = 0;
      }
    }
    if constexpr (!prefetch<TPR, NV>()) {
      if (row + step < T) fetch(row + step);
    }
  }

  if constexpr (REG) {
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (ok[k])
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ag[k][e] += hig[vc[k] * E + e];
          ab[k][e] += hib[vc[k] * E + e];
        }
  }
  if constexpr (DGB) {
    // one partial row per block: the RPB rows in flight combined in order
    float* rowg = pg + static_cast<size_t>(blockIdx.x) * H;
    float* rowb = pb + static_cast<size_t>(blockIdx.x) * H;
    if constexpr (RPB == 1) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if (!ok[k]) continue;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          store_f32x4(rowg + static_cast<size_t>(vc[k]) * E + 4 * q, ag[k] + 4 * q);
          store_f32x4(rowb + static_cast<size_t>(vc[k]) * E + 4 * q, ab[k] + 4 * q);
        }
      }
    } else {
      __shared__ float buf[RPB][TPR][E];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          const float* src = which ? ab[k] : ag[k];
#pragma unroll
          for (int e = 0; e < E; ++e) buf[sub][lt][e] = src[e];
          __syncthreads();
          if (sub == 0 && ok[k]) {
            float sum[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              float t = buf[0][lt][e];
#pragma unroll
              for (int r = 1; r < RPB; ++r) t += buf[r][lt][e];
              sum[e] = t;
            }
            float* dst = (which ? rowb : rowg) + static_cast<size_t>(vc[k]) * E;
#pragma unroll
            for (int q = 0; q < E / 4; ++q) store_f32x4(dst + 4 * q, sum + 4 * q);
          }
          __syncthreads();
        }
      }
    }
  }
}

// Sum over the wave, the same in every lane: each 32-lane half by swizzles
// (xor of the lane index with 16, 8, 4, 2, 1; the pattern is an immediate),
// then the two halves' totals read as scalars and added. Unlike a permute
// butterfly it keeps no lane-address registers, which a row loop would hoist.
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (16 << 10) | 0x1F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (8 << 10) | 0x1F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (4 << 10) | 0x1F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (2 << 10) | 0x1F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (1 << 10) | 0x1F));
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return lo + hi;
}

// Backward of rows of up to NV TPR vectors (1024 < vectors <= 2048 with 512
// threads of 4): a resident block walks a contiguous range of rows with the
// whole row in registers (each thread its NV vectors of dy, h, dh_in) and the
// next row's loaded while this one is reduced; each thread owns the same
// columns on every row, so its dgamma / dbeta sums stay in registers, added
// into the block's partial row (its own columns: no reduction across threads)
// every kFlushRows rows and at the end. Loads go through buffer descriptors
// (row base + 32-bit lane offset, the per-vector step a scalar), so no 64-bit
// address per vector is kept in registers.
template <DT D, DT R, int TPR, int NV>
__global__ __launch_bounds__(TPR) void ln_bwd_block_kernel(LnArgs a, int64_t rows_per_block) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ RowLds<W, 1> lds;
  const int lt = threadIdx.x, wr = lt / 64, lane = lt & 63;
  const int nvec = static_cast<int>(a.H / E);
  const float fh = static_cast<float>(a.H);
  auto in_row = [&](int k) { return lt + k * TPR < nvec; };
  const uint32_t xbytes = static_cast<uint32_t>(nvec) * XB, rbytes = static_cast<uint32_t>(nvec) * RB;
  const size_t px = static_cast<size_t>(a.H) * Vec<D>::BYTES, pr = static_cast<size_t>(a.H) * Vec<R>::BYTES;
  const char* dy = static_cast<const char*>(a.dy);
  const char* hh = static_cast<const char*>(a.h);
  const char* up = static_cast<const char*>(a.dh_in);
  char* dx = static_cast<char*>(a.dx);
  char* dres = static_cast<char*>(a.dres);
  PD gp[NV];  // gamma, packed (unpacked where used: fewer registers)
#pragma unroll
  for (int k = 0; k < NV; ++k)
    gp[k] = pk_load_rsrc<D, E>(static_cast<const char*>(a.gamma), xbytes, lt * XB, k * TPR * XB, false);
  const bool dgb = a.pg != nullptr;
  float sg[NV][E], sb[NV][E];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) sg[k][e] = sb[k][e] = 0.0f;
  float* pgr = dgb ? a.pg + static_cast<size_t>(blockIdx.x) * a.H : nullptr;
  float* pbr = dgb ? a.pb + static_cast<size_t>(blockIdx.x) * a.H : nullptr;
  bool first_flush = true;
  auto flush = [&]() {  // add the sums into the block's partial row (this thread's columns)
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      uint32_t ci = static_cast<uint32_t>(lt + k * TPR) * E;
      opaque(ci);  // formed here, not kept in registers across the row loop
      const size_t c = ci;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        float tg[4], tb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tg[e] = first_flush ? sg[k][4 * q + e] : pgr[c + 4 * q + e] + sg[k][4 * q + e];
          tb[e] = first_flush ? sb[k][4 * q + e] : pbr[c + 4 * q + e] + sb[k][4 * q + e];
        }
        store_f32x4(pgr + c + 4 * q, tg);
        store_f32x4(pbr + c + 4 * q, tb);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) sg[k][e] = sb[k][e] = 0.0f;
    }
    first_flush = false;
  };
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < a.T ? r0 + rows_per_block : a.T;
  PD gyn[NV], hn[NV];
  auto fetch = [&](int64_t r) {
    const char* dyr = dy + static_cast<size_t>(r) * px;
    const char* hr = hh + static_cast<size_t>(r) * px;
#pragma unroll
    for (int k = 0; k < NV; ++k) {  // past the row: zeros, neither stored nor summed
      gyn[k] = pk_load_rsrc<D, E>(dyr, xbytes, lt * XB, k * TPR * XB, MB_NT_LOAD);
      hn[k] = pk_load_rsrc<D, E>(hr, xbytes, lt * XB, k * TPR * XB, MB_NT_LOAD);
    }
  };
  int nrows = 0;
  if (r0 < r1) fetch(r0);
  for (int64_t row = r0; row < r1; ++row) {
    PD gy[NV], hp[NV];
    PR uu[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gy[k] = gyn[k];
      hp[k] = hn[k];
    }
    // dh_in is first used after the row sums: loaded for this row, ahead of
    // the next row's dy and h (one row of it in registers, not two)
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (up) uu[k] = pk_load_rsrc<R, E>(up + static_cast<size_t>(row) * pr, rbytes, lt * RB, k * TPR * RB, MB_NT_LOAD);
    if (row + 1 < r1) fetch(row + 1);
#pragma unroll
    for (int k = 0; k < NV; ++k) opaque(gp[k]);  // unpacked per row, not kept unpacked across rows
    const float mu = a.cmean[row], rs = a.crstd[row];
    float sa = 0.0f, sax = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float gv[E], hv[E], g[E];
      pk_unpack<D, E>(gy[k], gv);
      pk_unpack<D, E>(hp[k], hv);
      pk_unpack<D, E>(gp[k], g);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = (hv[e] - mu) * rs;
        const float av = gv[e] * (g[e] + a.gshift);
        sa += av;
        sax = __builtin_fmaf(av, xv, sax);
        sg[k][e] = __builtin_fmaf(gv[e], xv, sg[k][e]);
        sb[k][e] += gv[e];
      }
      __builtin_amdgcn_sched_barrier(0);  // one vector unpacked at a time
    }
    {
      // the two row sums: the waves' sums through LDS in wave order (slots
      // alternate by row, so a wave ahead never overwrites a slot still read)
      const int slot = static_cast<int>(row & 1) * 2;
      sa = wave_sum_uniform(sa);
      sax = wave_sum_uniform(sax);
      if (lane == 0) {
        lds.v[0][slot][wr] = sa;
        lds.v[0][slot + 1][wr] = sax;
      }
      __syncthreads();
      sa = lds.v[0][slot][0];
      sax = lds.v[0][slot + 1][0];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        sa += lds.v[0][slot][w];
        sax += lds.v[0][slot + 1][w];
      }
    }
    const float ma = sa / fh, mx = sax / fh;
#pragma unroll
    for (int k = 0; k < NV; ++k) {  // unpacked again below, not kept unpacked across the row sums
      opaque(gy[k]);
      opaque(hp[k]);
      opaque(gp[k]);
    }
    const size_t xo = static_cast<size_t>(row) * px, ro = static_cast<size_t>(row) * pr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      float gv[E], hv[E], uv[E], g[E];
      pk_unpack<D, E>(gy[k], gv);
      pk_unpack<D, E>(hp[k], hv);
      pk_unpack<D, E>(gp[k], g);
      if (up) {
        pk_unpack<R, E>(uu[k], uv);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) uv[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = (hv[e] - mu) * rs;
        gv[e] = __builtin_fmaf(rs, __builtin_fmaf(-xv, mx, gv[e] * (g[e] + a.gshift) - ma), uv[e]);
      }
      const uint32_t v = static_cast<uint32_t>(lt + k * TPR);
      pk_store<D, E>(dx + xo + v * XB, pk_pack<D, E>(gv));
      if (dres) pk_store<R, E>(dres + ro + v * RB, pk_pack<R, E>(gv));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (dgb && ++nrows == kFlushRows) {
      flush();
      nrows = 0;
    }
  }
  if (dgb && (nrows > 0 || first_flush)) flush();
}

// Waits until at most n vector-memory operations of this wave are
// outstanding, n rounded down to a multiple of 4 up to 32 (waiting longer is
// always safe: the counter retires in issue order).
__device__ __forceinline__ void vm_wait_at_most(int n) {
  if (n >= 32) __builtin_amdgcn_s_waitcnt(0x8F70);
  else if (n >= 28) __builtin_amdgcn_s_waitcnt(0x4F7C);
  else if (n >= 24) __builtin_amdgcn_s_waitcnt(0x4F78);
  else if (n >= 20) __builtin_amdgcn_s_waitcnt(0x4F74);
  else if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);
  else if (n >= 12) __builtin_amdgcn_s_waitcnt(0x0F7C);
  else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// A workgroup barrier that leaves outstanding vector loads in flight: the
// caller has waited for its LDS writes; the asm keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The block backward above with the row loads staged through LDS (rows of
// 16-byte pieces): two stages of dy and h (128 KiB for 2048 vectors) are
// filled by buffer loads that write LDS directly; at the start of a row the
// block copies its stage into registers and refills the stage with the row
// after next, so two rows of loads are in flight where registers alone hold
// one (the per-thread dgamma / dbeta sums leave no room for a second). Each
// lane reads back only the 16 bytes its own load wrote, so a wait on the
// wave's vector-memory counter (the loads retire in issue order; the count
// of those issued since is a fixed lower bound, every row issuing the same
// loads) is all the row needs; the row-sum barrier leaves them in flight.
// The row's mean and rstd reach it through LDS as well and its dh_in a row
// ahead in registers, so that no load is waited for before it is needed.
template <DT D, DT R, int TPR, int NV>
__global__ __launch_bounds__(TPR) void ln_bwd_block_lds_kernel(LnArgs a, int64_t rows_per_block) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  static_assert(XB == 16, "16-byte pieces of dy and h");
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ RowLds<W, 1> lds;
  // [2 stages][dy, h][NV][W] chunks of 64 x 16 B, then the row statistics
  extern __shared__ __align__(16) unsigned char stage_raw[];
  const int lt = threadIdx.x, wr = lt / 64, lane = lt & 63;
  const int nvec = static_cast<int>(a.H / E);
  const float fh = static_cast<float>(a.H);
  auto in_row = [&](int k) { return lt + k * TPR < nvec; };
  const uint32_t xbytes = static_cast<uint32_t>(nvec) * XB, rbytes = static_cast<uint32_t>(nvec) * RB;
  const size_t px = static_cast<size_t>(a.H) * Vec<D>::BYTES, pr = static_cast<size_t>(a.H) * Vec<R>::BYTES;
  const char* dy = static_cast<const char*>(a.dy);
  const char* hh = static_cast<const char*>(a.h);
  const char* up = static_cast<const char*>(a.dh_in);
  char* dx = static_cast<char*>(a.dx);
  char* dres = static_cast<char*>(a.dres);
  auto chunk = [&](int st, int t, int k) {  // this wave's 1 KiB chunk
    return stage_raw + static_cast<size_t>(((st * 2 + t) * NV + k) * W + wr) * 1024;
  };
  PD gp[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k)
    gp[k] = pk_load_rsrc<D, E>(static_cast<const char*>(a.gamma), xbytes, lt * XB, k * TPR * XB, false);
  vm_wait_at_most(0);  // gamma in registers before the row loads start counting
  const bool dgb = a.pg != nullptr;
  float sg[NV][E], sb[NV][E];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) sg[k][e] = sb[k][e] = 0.0f;
  float* pgr = dgb ? a.pg + static_cast<size_t>(blockIdx.x) * a.H : nullptr;
  float* pbr = dgb ? a.pb + static_cast<size_t>(blockIdx.x) * a.H : nullptr;
  bool first_flush = true;
  auto flush = [&]() {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      uint32_t ci = static_cast<uint32_t>(lt + k * TPR) * E;
      opaque(ci);
      const size_t c = ci;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        float tg[4], tb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tg[e] = first_flush ? sg[k][4 * q + e] : pgr[c + 4 * q + e] + sg[k][4 * q + e];
          tb[e] = first_flush ? sb[k][4 * q + e] : pbr[c + 4 * q + e] + sb[k][4 * q + e];
        }
        store_f32x4(pgr + c + 4 * q, tg);
        store_f32x4(pbr + c + 4 * q, tb);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) sg[k][e] = sb[k][e] = 0.0f;
    }
    first_flush = false;
  };
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < a.T ? r0 + rows_per_block : a.T;
  // row r's dy and h into stage st: always 2 NV vector-memory operations (a
  // row past the range gets an empty buffer: nothing is read), so that the
  // wait counts below hold on every path
  auto dma = [&](int64_t r, int st) {
    const bool real = r < r1;
    const size_t ro = real ? static_cast<size_t>(r) * px : 0;
    const uint32_t nb = real ? xbytes : 0u;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(dy + ro), 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(hh + ro), 0, nb, 0x00020000);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)chunk(st, 0, k), 16,
                                               lt * XB, k * TPR * XB, 0, 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (__attribute__((address_space(3))) void*)chunk(st, 1, k), 16,
                                               lt * XB, k * TPR * XB, 0, 2);
    }
  };
  // mean and rstd come through LDS too: every 64 rows each wave copies the
  // next 64 rows' statistics into its own ring of two chunks, so that a row
  // reads them from LDS; as vector loads, the wait for them would also wait
  // for the dh_in loads issued after them (the ring follows the stages:
  // [W][2 chunks][mean, rstd][64] floats)
  float* const ring = reinterpret_cast<float*>(stage_raw + static_cast<size_t>(2 * 2 * NV * W) * 1024);
  auto stats = [&](int buf, int which) { return ring + ((wr * 2 + buf) * 2 + which) * 64; };
  auto stats_dma = [&](int64_t c0, int buf) {  // rows c0 .. c0 + 63, clipped at r1
    const int64_t n = r1 - c0;
    const bool real = n > 0;
    const uint32_t nb = real ? static_cast<uint32_t>(n < 64 ? n : 64) * 4u : 0u;
    const size_t off = real ? static_cast<size_t>(c0) : 0;
    const __amdgpu_buffer_rsrc_t rm =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.cmean + off), 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.crstd + off), 0, nb, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (__attribute__((address_space(3))) void*)stats(buf, 0), 4, lane * 4,
                                             0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (__attribute__((address_space(3))) void*)stats(buf, 1), 4, lane * 4,
                                             0, 0, 0);
  };
  // dh_in, first used after the row sums, is loaded a row ahead into one of
  // two register sets; always NV loads (an empty buffer past r1 or without
  // dh_in: zeros, nothing read)
  PR ua[NV], ub[NV];
  auto load_up = [&](int64_t r, PR(&u)[NV]) {
    const bool real = up != nullptr && r < r1;
    const char* base = real ? up + static_cast<size_t>(r) * pr : up;
#pragma unroll
    for (int k = 0; k < NV; ++k)
      u[k] = pk_load_rsrc<R, E>(base, real ? rbytes : 0u, lt * RB, k * TPR * RB, MB_NT_LOAD);
  };
  int nrows = 0;
  // the loads of one row, in issue order: [statistics of the next 64 rows,
  // every 64th row], the next row's dh_in (NV), the dy and h of the row after
  // next (2 NV), this row's stores
  auto do_row = [&](int64_t row, PR(&cur)[NV], PR(&nxt)[NV]) {
    const int64_t i = row - r0;
    const int st = static_cast<int>(i & 1);
    // this row's dy and h were issued two rows ago; the next row's dh_in, dy
    // and h, issued since, may stay outstanding
    vm_wait_at_most(i == 0 ? 2 * NV : 3 * NV);
    if ((i & 63) == 0) stats_dma(row + 64, static_cast<int>(((i >> 6) + 1) & 1));
    PD gy[NV], hp[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gy[k] = *reinterpret_cast<const PD*>(chunk(st, 0, k) + lane * 16);
      hp[k] = *reinterpret_cast<const PD*>(chunk(st, 1, k) + lane * 16);
    }
    const int cb = static_cast<int>((i >> 6) & 1), ci = static_cast<int>(i & 63);
    const float mu = stats(cb, 0)[ci], rs = stats(cb, 1)[ci];
    load_up(row + 1, nxt);
    lgkm_wait0();  // the stage is read: it may be filled again
    asm volatile("" ::: "memory");
    dma(row + 2, st);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < NV; ++k) opaque(gp[k]);
    float sa = 0.0f, sax = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      float gv[E], hv[E], g[E];
      pk_unpack<D, E>(gy[k], gv);
      pk_unpack<D, E>(hp[k], hv);
      pk_unpack<D, E>(gp[k], g);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = (hv[e] - mu) * rs;
        const float av = gv[e] * (g[e] + a.gshift);
        sa += av;
        sax = __builtin_fmaf(av, xv, sax);
        sg[k][e] = __builtin_fmaf(gv[e], xv, sg[k][e]);
        sb[k][e] += gv[e];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const int slot = static_cast<int>(row & 1) * 2;
      sa = wave_sum_uniform(sa);
      sax = wave_sum_uniform(sax);
      if (lane == 0) {
        lds.v[0][slot][wr] = sa;
        lds.v[0][slot + 1][wr] = sax;
      }
      lgkm_wait0();
      bare_barrier();
      sa = lds.v[0][slot][0];
      sax = lds.v[0][slot + 1][0];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        sa += lds.v[0][slot][w];
        sax += lds.v[0][slot + 1][w];
      }
    }
    const float ma = sa / fh, mx = sax / fh;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      opaque(gy[k]);
      opaque(hp[k]);
      opaque(gp[k]);
    }
    const size_t xo = static_cast<size_t>(row) * px, ro = static_cast<size_t>(row) * pr;
    // this row's dh_in was issued before the next row's dy and h, the next
    // row's dh_in and the dy and h of the row after
    vm_wait_at_most(5 * NV);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      float gv[E], hv[E], uv[E], g[E];
      pk_unpack<D, E>(gy[k], gv);
      pk_unpack<D, E>(hp[k], hv);
      pk_unpack<D, E>(gp[k], g);
      pk_unpack<R, E>(cur[k], uv);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xv = (hv[e] - mu) * rs;
        gv[e] = __builtin_fmaf(rs, __builtin_fmaf(-xv, mx, gv[e] * (g[e] + a.gshift) - ma), uv[e]);
      }
      const uint32_t v = static_cast<uint32_t>(lt + k * TPR);
      pk_store<D, E>(dx + xo + v * XB, pk_pack<D, E>(gv));
      if (dres) pk_store<R, E>(dres + ro + v * RB, pk_pack<R, E>(gv));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (dgb && ++nrows == kFlushRows) {
      flush();
      nrows = 0;
    }
  };
  stats_dma(r0, 0);
  load_up(r0, ua);
  asm volatile("" ::: "memory");
  dma(r0, 0);
  dma(r0 + 1, 1);
  // two rows per trip, so that the two dh_in register sets alternate
  // without copies (the odd last row after the loop: inside it, the path
  // that skips the second row would leave a load in flight at the back edge)
  const int n = static_cast<int>(r1 - r0);
  int i = 0;
  for (; i + 1 < n; i += 2) {
    do_row(r0 + i, ua, ub);
    do_row(r0 + i + 1, ub, ua);
  }
  if (i < n) do_row(r0 + i, ua, ub);
  if (dgb && (nrows > 0 || first_flush)) flush();
  vm_wait_at_most(0);  // no LDS write of the (empty) loads past the range still in flight at exit
}

// ---------------------------------------------------------------- team rows
// The backward of rows too wide for one block's registers (2049-8192
// vectors): a row is split over a team of `members` blocks, member m holding
// the `slice` vectors from m slice on of every row the team walks (its part
// of dy and h staged through LDS two rows ahead as in the block kernel above,
// its part of gamma and of the dgamma / dbeta sums in registers). The two row
// sums need the whole row: each member publishes its partial pair as one
// 64-bit atomic store (agent scope) into the row's slot, and wave 0 polls the
// other members' slots with atomic loads; every member then adds the pairs in
// member order, so all get the same sums. A fill kernel sets the slots to
// kTeamEmpty (and the row flags to 0) before the launch. The grid is sized to
// the blocks the device holds at once, so a partner's pair normally arrives
// within microseconds; the wait is still bounded: after `spin_limit` polls
// (and for the rest of the launch once that happened) a block flags the row
// (its dx from the incomplete sums is then rewritten) for
// ln_team_fixup_kernel, launched after, which recomputes every member's pair
// of each flagged row from the row's slices, with the same per-thread,
// per-wave and member-order arithmetic, and writes the row's dx: the result
// is the same bit for bit whether the pairs arrive or not (when other work
// holds part of the device, say). Kept out of the row loop, that path costs
// the loop nothing (inside it, even as a call, it cost 6 %).

// No published pair has this bit pattern: a NaN sum is published as the
// canonical quiet NaN, whose high word differs.
constexpr uint64_t kTeamEmpty = ~0ull;

__global__ __launch_bounds__(256) void team_fill_kernel(uint64_t* slots, int64_t nslots, uint32_t* flags,
                                                        int64_t rows) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nslots; i += step)
    slots[i] = kTeamEmpty;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < rows; i += step) flags[i] = 0;
}

__device__ __forceinline__ uint32_t canonical_bits(float v) { return v != v ? 0x7FC00000u : __float_as_uint(v); }

// A thread's terms of the two row sums over its vectors of a slice (k < nk,
// the vectors that exist): sum a and sum a xhat with a = dy gamma', xhat =
// (h - mean) rstd; with SUMS also its dgamma / dbeta terms (dy xhat, dy). No
// contraction, so that both kernels round them alike.
template <DT D, int E, int NV, bool SUMS>
__device__ __forceinline__ void team_terms(const typename Pk<D, E>::T* gy, const typename Pk<D, E>::T* hp,
                                           const typename Pk<D, E>::T* gp, int nk, float mu, float rs,
                                           float gshift, float& sa, float& sax, float (*sg)[E], float (*sb)[E]) {
#pragma clang fp contract(off)
  sa = 0.0f;
  sax = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (k >= nk) break;
    float gv[E], hv[E], g[E];
    pk_unpack<D, E>(gy[k], gv);
    pk_unpack<D, E>(hp[k], hv);
    pk_unpack<D, E>(gp[k], g);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float xv = (hv[e] - mu) * rs;
      const float av = gv[e] * (g[e] + gshift);
      sa = sa + av;
      sax = __builtin_fmaf(av, xv, sax);
      if constexpr (SUMS) {
        sg[k][e] = __builtin_fmaf(gv[e], xv, sg[k][e]);
        sb[k][e] = sb[k][e] + gv[e];
      }
    }
  }
}

// dh of one vector from the row's means ma = mean_j a, mx = mean_j a xhat
// (into gv), every fused step written out (both kernels round it alike).
template <int E>
__device__ __forceinline__ void team_dh(float* gv, const float* hv, const float* g, const float* uv, float mu,
                                        float rs, float gshift, float ma, float mx) {
#pragma clang fp contract(off)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float xv = (hv[e] - mu) * rs;
    const float t = __builtin_fmaf(gv[e], g[e] + gshift, -ma);
    gv[e] = __builtin_fmaf(rs, __builtin_fmaf(-xv, mx, t), uv[e]);
  }
}

// The block's sum of per-wave values in wave order, in every thread (two
// barriers; `buf` holds W pairs).
template <int W>
__device__ __forceinline__ void team_block_pair(float& a, float& b, float (*buf)[2]) {
  const int wr = threadIdx.x / 64, lane = threadIdx.x & 63;
  a = wave_sum_uniform(a);
  b = wave_sum_uniform(b);
  if (lane == 0) {
    buf[wr][0] = a;
    buf[wr][1] = b;
  }
  __syncthreads();
  a = buf[0][0];
  b = buf[0][1];
#pragma unroll
  for (int w = 1; w < W; ++w) {
    a += buf[w][0];
    b += buf[w][1];
  }
  __syncthreads();
}

template <DT D, DT R, int TPR, int NV>
__global__ __launch_bounds__(TPR, 2) void ln_bwd_team_kernel(LnArgs a, int members, int slice,
                                                              int64_t rows_per_team, int spin_limit,
                                                              uint32_t* flags) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ RowLds<W, 1> lds;
  __shared__ float pairs[2][kLnTeamMaxMembers][2];  // the members' pairs, by row parity
  extern __shared__ __align__(16) unsigned char stage_raw[];  // [2 stages][dy, h][NV][W] chunks of 64 x 16 B
  const int lt = threadIdx.x, wr = lt / 64, lane = lt & 63;
  const int m = static_cast<int>(blockIdx.x) % members, team = static_cast<int>(blockIdx.x) / members;
  const int nvec = static_cast<int>(a.H / E);
  const float fh = static_cast<float>(a.H);
  const int nvm = nvec - m * slice < slice ? nvec - m * slice : slice;  // >= 1
  const int nk = lt < nvm ? (nvm - lt + TPR - 1) / TPR : 0;           // this thread's vectors in the slice
  auto in_row = [&](int k) { return k < nk; };
  const size_t px = static_cast<size_t>(a.H) * Vec<D>::BYTES, pr = static_cast<size_t>(a.H) * Vec<R>::BYTES;
  const size_t xs = static_cast<size_t>(m) * slice * XB, rsl = static_cast<size_t>(m) * slice * RB;
  const uint32_t xbytes = static_cast<uint32_t>(nvm) * XB, rbytes = static_cast<uint32_t>(nvm) * RB;
  const char* dy = static_cast<const char*>(a.dy) + xs;
  const char* hh = static_cast<const char*>(a.h) + xs;
  const char* up = a.dh_in ? static_cast<const char*>(a.dh_in) + rsl : nullptr;
  char* dx = static_cast<char*>(a.dx) + xs;
  char* dres = a.dres ? static_cast<char*>(a.dres) + rsl : nullptr;
  uint64_t* slots = reinterpret_cast<uint64_t*>(a.rowsums);
  PD gp[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k)
    gp[k] = pk_load_rsrc<D, E>(static_cast<const char*>(a.gamma) + xs, xbytes, lt * XB, k * TPR * XB, false);
  vm_wait_at_most(0);  // gamma in registers before the row loads start counting
  const bool dgb = a.pg != nullptr;
  float sg[NV][E], sb[NV][E];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) sg[k][e] = sb[k][e] = 0.0f;
  float* pgr = dgb ? a.pg + static_cast<size_t>(team) * a.H + static_cast<size_t>(m) * slice * E : nullptr;
  float* pbr = dgb ? a.pb + static_cast<size_t>(team) * a.H + static_cast<size_t>(m) * slice * E : nullptr;
  bool first_flush = true;
  auto flush = [&]() {  // add the sums into the team's partial row (this thread's columns)
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!in_row(k)) continue;
      uint32_t ci = static_cast<uint32_t>(lt + k * TPR) * E;
      opaque(ci);
      const size_t c = ci;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        float tg[4], tb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tg[e] = first_flush ? sg[k][4 * q + e] : pgr[c + 4 * q + e] + sg[k][4 * q + e];
          tb[e] = first_flush ? sb[k][4 * q + e] : pbr[c + 4 * q + e] + sb[k][4 * q + e];
        }
        store_f32x4(pgr + c + 4 * q, tg);
        store_f32x4(pbr + c + 4 * q, tb);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) sg[k][e] = sb[k][e] = 0.0f;
    }
    first_flush = false;
  };
  const int64_t r0 = static_cast<int64_t>(team) * rows_per_team;
  const int64_t r1 = r0 + rows_per_team < a.T ? r0 + rows_per_team : a.T;
  // rows staged through LDS as in ln_bwd_block_lds_kernel: the slice's dy and
  // h of row r into stage st, always 2 NV vector-memory operations (a row past
  // the range reads nothing); its lane reads back only what it loaded. LDS
  // loads come in 16 bytes: an 8-byte piece (16-bit rows beside an fp32
  // residual) is loaded with the next piece's 8 bytes (or zeros past the
  // slice) and the lane keeps the first 8, the same cache lines either way
  auto chunk = [&](int st, int t, int k) {
    return stage_raw + static_cast<size_t>(((st * 2 + t) * NV + k) * W + wr) * 1024;
  };
  auto dma = [&](int64_t r, int st) {
    const bool real = r < r1;
    const size_t ro = real ? static_cast<size_t>(r) * px : 0;
    const uint32_t nb = real ? xbytes : 0u;
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(dy + ro), 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(hh + ro), 0, nb, 0x00020000);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)chunk(st, 0, k), 16,
                                               lt * XB, k * TPR * XB, 0, 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (__attribute__((address_space(3))) void*)chunk(st, 1, k), 16,
                                               lt * XB, k * TPR * XB, 0, 2);
    }
  };
  const int U = up ? NV : 0;  // dh_in loads per row
  bool waiting = true;  // wave 0: false once a wait has run out (the rest of the launch is left to the fix-up)
  int nrows = 0;
  // the row's mean and rstd are loaded a row ahead, before the row after
  // next goes out, so that waiting for them leaves those loads in flight
  float mu_n = a.cmean[r0], rs_n = a.crstd[r0];
  asm volatile("" ::: "memory");  // issued before the first rows' loads
  dma(r0, 0);
  dma(r0 + 1, 1);
  for (int64_t row = r0; row < r1; ++row) {
    const int st = static_cast<int>((row - r0) & 1);
    // this row's loads were issued during the row before last; the dh_in and
    // row loads issued since may stay outstanding
    vm_wait_at_most(row == r0 ? 2 * NV : U + 2 * NV);
    PD gy[NV], hp[NV];
    PR uu[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      gy[k] = *reinterpret_cast<const PD*>(chunk(st, 0, k) + lane * 16);
      hp[k] = *reinterpret_cast<const PD*>(chunk(st, 1, k) + lane * 16);
    }
    const float mu = mu_n, rs = rs_n;
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (up) uu[k] = pk_load_rsrc<R, E>(up + static_cast<size_t>(row) * pr, rbytes, lt * RB, k * TPR * RB, MB_NT_LOAD);
#pragma unroll
    for (int k = 0; k < NV; ++k) opaque(gp[k]);
    float sa, sax;
    team_terms<D, E, NV, true>(gy, hp, gp, nk, mu, rs, a.gshift, sa, sax, sg, sb);
    const int par = static_cast<int>(row & 1);
    // this member's pair: the waves' sums in wave order through LDS
    sa = wave_sum_uniform(sa);
    sax = wave_sum_uniform(sax);
    if (lane == 0) {
      lds.v[0][2 * par][wr] = sa;
      lds.v[0][2 * par + 1][wr] = sax;
    }
    lgkm_wait0();
    bare_barrier();  // the row loads in flight stay in flight
    if (wr == 0) {
      float pa = lds.v[0][2 * par][0], pax = lds.v[0][2 * par + 1][0];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        pa += lds.v[0][2 * par][w];
        pax += lds.v[0][2 * par + 1][w];
      }
      uint64_t* rslots = slots + static_cast<size_t>(row) * members;
      if (lane == 0)
        __hip_atomic_store(rslots + m, (static_cast<uint64_t>(canonical_bits(pax)) << 32) | canonical_bits(pa),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint64_t got = kTeamEmpty;
      const bool partner = lane < members && lane != m;
      if (partner && waiting) {
        got = __hip_atomic_load(rslots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int spins = 0; got == kTeamEmpty && spins < spin_limit; ++spins) {
          __builtin_amdgcn_s_sleep(2);
          got = __hip_atomic_load(rslots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      const bool miss = __ballot(partner && got == kTeamEmpty) != 0;  // the same in every lane of wave 0
      if (miss) waiting = false;
      if (lane < members) {
        pairs[par][lane][0] = lane == m ? pa : __uint_as_float(static_cast<uint32_t>(got));
        pairs[par][lane][1] = lane == m ? pax : __uint_as_float(static_cast<uint32_t>(got >> 32));
      }
      if (lane == 0 && miss) flags[row] = 1u;  // its dx is rewritten by the fix-up
    }
    lgkm_wait0();
    bare_barrier();
    // the stage is read (its registers were loaded before the first barrier)
    // and the polls are done: the row after next goes out now (issued before
    // the polls, wave 0 would have waited for it to land)
    {
      const int64_t nx = row + 1 < r1 ? row + 1 : row;
      mu_n = a.cmean[nx];
      rs_n = a.crstd[nx];
    }
    asm volatile("" ::: "memory");
    dma(row + 2, st);
    asm volatile("" ::: "memory");
    {
      // the team's sums in member order (the same in every member)
      float ta = 0.0f, tax = 0.0f;
      for (int j = 0; j < members; ++j) {
        ta += pairs[par][j][0];
        tax += pairs[par][j][1];
      }
      const float ma = ta / fh, mx = tax / fh;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        opaque(gy[k]);
        opaque(hp[k]);
        opaque(gp[k]);
      }
      const size_t xo = static_cast<size_t>(row) * px, ro = static_cast<size_t>(row) * pr;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if (!in_row(k)) continue;
        float gv[E], hv[E], uv[E], g[E];
        pk_unpack<D, E>(gy[k], gv);
        pk_unpack<D, E>(hp[k], hv);
        pk_unpack<D, E>(gp[k], g);
        if (up) {
          pk_unpack<R, E>(uu[k], uv);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) uv[e] = 0.0f;
        }
        team_dh<E>(gv, hv, g, uv, mu, rs, a.gshift, ma, mx);
        const uint32_t v = static_cast<uint32_t>(lt + k * TPR);
        pk_store<D, E>(dx + xo + v * XB, pk_pack<D, E>(gv));
        if (dres) pk_store<R, E>(dres + ro + v * RB, pk_pack<R, E>(gv));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (dgb && ++nrows == kFlushRows) {
      flush();
      nrows = 0;
    }
  }
  if (dgb && (nrows > 0 || first_flush)) flush();
}

// dx (and dresidual) of the rows ln_bwd_team_kernel flagged: each member's
// pair recomputed from its slice exactly as the member computes it (the same
// thread layout, terms, wave sums and wave order), the pairs added in member
// order, then dh of every vector of the row. Block b looks after rows
// [b TPR, (b + 1) TPR): its threads read their flags at once, and a block
// without a flagged row returns after one barrier.
template <DT D, DT R, int TPR, int NV>
__global__ __launch_bounds__(TPR) void ln_team_fixup_kernel(LnArgs a, int members, int slice,
                                                            const uint32_t* flags) {
  constexpr int E = ln_epl<D, R>();
  constexpr int W = TPR / 64;
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES;
  using PD = typename Pk<D, E>::T;
  __shared__ float buf[W][2];
  __shared__ uint32_t fl[TPR];
  const int lt = threadIdx.x;
  const int nvec = static_cast<int>(a.H / E);
  const float fh = static_cast<float>(a.H);
  const size_t px = static_cast<size_t>(a.H) * Vec<D>::BYTES, pr = static_cast<size_t>(a.H) * Vec<R>::BYTES;
  const char* dy0 = static_cast<const char*>(a.dy);
  const char* h0 = static_cast<const char*>(a.h);
  const char* gm0 = static_cast<const char*>(a.gamma);
  const char* up0 = static_cast<const char*>(a.dh_in);
  char* dx0 = static_cast<char*>(a.dx);
  char* dres0 = static_cast<char*>(a.dres);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * TPR;
  const uint32_t mine = base + lt < a.T ? flags[base + lt] : 0u;
  fl[lt] = mine;
  if (__syncthreads_count(mine != 0) == 0) return;  // the same in every thread
  for (int i = 0; i < TPR && base + i < a.T; ++i) {
    if (fl[i] == 0) continue;  // the same in every thread
    const int64_t row = base + i;
    const float mu = a.cmean[row], rs = a.crstd[row];
    float ta = 0.0f, tax = 0.0f;
    for (int j = 0; j < members; ++j) {
      const int nj = nvec - j * slice < slice ? nvec - j * slice : slice;
      const int nk = lt < nj ? (nj - lt + TPR - 1) / TPR : 0;
      const uint32_t jb = static_cast<uint32_t>(nj) * XB;
      const size_t jo = static_cast<size_t>(j) * slice * XB;
      PD ty[NV], th[NV], tg[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        ty[k] = pk_load_rsrc<D, E>(dy0 + static_cast<size_t>(row) * px + jo, jb, lt * XB, k * TPR * XB, false);
        th[k] = pk_load_rsrc<D, E>(h0 + static_cast<size_t>(row) * px + jo, jb, lt * XB, k * TPR * XB, false);
        tg[k] = pk_load_rsrc<D, E>(gm0 + jo, jb, lt * XB, k * TPR * XB, false);
      }
      float ja, jax;
      team_terms<D, E, NV, false>(ty, th, tg, nk, mu, rs, a.gshift, ja, jax, nullptr, nullptr);
      team_block_pair<W>(ja, jax, buf);
      ta += ja;
      tax += jax;
    }
    const float ma = ta / fh, mx = tax / fh;
    for (int j = 0; j < members; ++j) {
      const int nj = nvec - j * slice < slice ? nvec - j * slice : slice;
      const size_t jo = static_cast<size_t>(j) * slice;
      for (int v = lt; v < nj; v += TPR) {
        const size_t xo = static_cast<size_t>(row) * px + (jo + v) * XB;
        const size_t ro = static_cast<size_t>(row) * pr + (jo + v) * RB;
        float gv[E], hv[E], uv[E], g[E];
        pk_unpack<D, E>(pk_load<D, E>(dy0 + xo), gv);
        pk_unpack<D, E>(pk_load<D, E>(h0 + xo), hv);
        pk_unpack<D, E>(pk_load_keep<D, E>(gm0 + (jo + v) * XB), g);
        if (up0) {
          pk_unpack<R, E>(pk_load<R, E>(up0 + ro), uv);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) uv[e] = 0.0f;
        }
        team_dh<E>(gv, hv, g, uv, mu, rs, a.gshift, ma, mx);
        pk_store<D, E>(dx0 + xo, pk_pack<D, E>(gv));
        if (dres0) pk_store<R, E>(dres0 + ro, pk_pack<R, E>(gv));
      }
    }
  }
}

// ---------------------------------------------------------------- wide rows
// The backward of rows of 2048 or more vectors, whose parameter-gradient sums
// do not fit beside a register-resident row, runs as two kernels:
//   ln2_rowsums_kernel, one block per row: mean_j a and mean_j a xhat, read
//     from dy and h;
//   ln2_dx_kernel, column strips (a wave keeps the same columns on every row,
//     so gamma and the dgamma / dbeta sums stay in registers): dx (and
//     dresidual) from the row sums, reading dy and h a second time.
// The second kernel walks the rows from the last one down: the rows the first
// kernel read last are still in the memory-side cache (256 MB on MI355X), so
// part of the second read of dy and h does not reach HBM.

#ifndef MB_LN2_A_THREADS
#define MB_LN2_A_THREADS 256  // threads per row in ln2_rowsums_kernel
#endif
#ifndef MB_LN2_A_UNROLL
#define MB_LN2_A_UNROLL 4  // vectors in flight per thread there
#endif
#ifndef MB_LN2_B_UNROLL
#define MB_LN2_B_UNROLL 2  // rows in flight per wave in ln2_dx_kernel
#endif

template <DT D, DT R>
__global__ __launch_bounds__(MB_LN2_A_THREADS) void ln2_rowsums_kernel(LnArgs a, int nvec) {
  constexpr int E = ln_epl<D, R>();
  constexpr int XB = E * Vec<D>::BYTES, U = MB_LN2_A_UNROLL, TA = MB_LN2_A_THREADS, W = TA / 64;
  using PD = typename Pk<D, E>::T;
  __shared__ float part[W][2];
  const int lt = threadIdx.x, lane = lt & 63, w = lt >> 6;
  const char* gm = static_cast<const char*>(a.gamma);
  for (int64_t row = blockIdx.x; row < a.T; row += gridDim.x) {
    const size_t ro = static_cast<size_t>(row) * a.H * Vec<D>::BYTES;
    const char* dyr = static_cast<const char*>(a.dy) + ro;
    const char* hr = static_cast<const char*>(a.h) + ro;
    const float mu = a.cmean[row], rs = a.crstd[row];
    float sa = 0.0f, sax = 0.0f;
    for (int v0 = lt; v0 < nvec; v0 += U * TA) {
      PD gy[U], hp[U], gp[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * TA;
        if (v < nvec) {
          gy[u] = pk_load_keep<D, E>(dyr + static_cast<size_t>(v) * XB);
          hp[u] = pk_load_keep<D, E>(hr + static_cast<size_t>(v) * XB);
          gp[u] = pk_load_keep<D, E>(gm + static_cast<size_t>(v) * XB);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v0 + u * TA >= nvec) break;
        float gv[E], hv[E], g[E];
        pk_unpack<D, E>(gy[u], gv);
        pk_unpack<D, E>(hp[u], hv);
        pk_unpack<D, E>(gp[u], g);
        // the vector's own sums first, then the thread's: a term passes
        // through at most E - 1 + nvec / TA additions in the thread
        float va = 0.0f, vx = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xv = (hv[e] - mu) * rs;
          const float av = gv[e] * (g[e] + a.gshift);
          va += av;
          vx = __builtin_fmaf(av, xv, vx);
        }
        sa += va;
        sax += vx;
      }
    }
    sa = wave_sum(sa);
    sax = wave_sum(sax);
    if (lane == 0) {
      part[w][0] = sa;
      part[w][1] = sax;
    }
    __syncthreads();
    if (lt == 0) {
      float ta = part[0][0], tx = part[0][1];
#pragma unroll
      for (int k = 1; k < W; ++k) {
        ta += part[k][0];
        tx += part[k][1];
      }
      const float fh = static_cast<float>(a.H);
      a.rowsums[2 * row] = ta / fh;
      a.rowsums[2 * row + 1] = tx / fh;
    }
    __syncthreads();  // part is reused by the block's next row
  }
}

// dx (and dresidual) for the strip's columns on every row, and the strip's
// dgamma / dbeta sums as partial row rg ([G][H] in a.pg / a.pb). Wave w of row
// group rg takes the rows T - 1 - (4 rg + w + 4 G k).
template <DT D, DT R> __global__ __launch_bounds__(kThreads) void ln2_dx_kernel(LnArgs a, int nvec) {
  constexpr int E = ln_epl<D, R>();
  constexpr int XB = E * Vec<D>::BYTES, RB = E * Vec<R>::BYTES, U = MB_LN2_B_UNROLL;
  using PD = typename Pk<D, E>::T;
  using PR = typename Pk<R, E>::T;
  __shared__ float red[kWaves][2 * E][64];
  const int lane = threadIdx.x & 63, w = wave_index<true>();
  const TileIdx ti = tile_idx();
  const int cv = ti.strip * kStrip + lane;
  const bool active = cv < nvec;
  const size_t cx = static_cast<size_t>(cv) * XB, cr = static_cast<size_t>(cv) * RB;
  ColAcc<E> cg, cb;
  cg.init();
  cb.init();
  if (active) {
    float g[E];
    pk_unpack<D, E>(pk_load_keep<D, E>(static_cast<const char*>(a.gamma) + cx), g);
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] += a.gshift;
    const size_t px = static_cast<size_t>(a.H) * Vec<D>::BYTES, pr = static_cast<size_t>(a.H) * Vec<R>::BYTES;
    const char* dy = static_cast<const char*>(a.dy);
    const char* h = static_cast<const char*>(a.h);
    const char* up = static_cast<const char*>(a.dh_in);
    char* dx = static_cast<char*>(a.dx);
    char* dres = static_cast<char*>(a.dres);
    const int64_t T = a.T, S = static_cast<int64_t>(kWaves) * ti.G;
    for (int64_t t = static_cast<int64_t>(ti.rg) * kWaves + w; t < T; t += U * S) {
      PD gy[U], hp[U];
      PR uu[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t + u * S < T) {
          const int64_t tt = T - 1 - (t + u * S);
          gy[u] = pk_load_keep<D, E>(dy + tt * px + cx);
          hp[u] = pk_load_keep<D, E>(h + tt * px + cx);
          if (up) uu[u] = pk_load<R, E>(up + tt * pr + cr);
        }
      }
      int rows = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t + u * S >= T) break;
        const int64_t tt = T - 1 - (t + u * S);
        ++rows;
        const float mu = a.cmean[tt], rs = a.crstd[tt], ma = a.rowsums[2 * tt], mx = a.rowsums[2 * tt + 1];
        float gv[E], hv[E], uv[E];
        pk_unpack<D, E>(gy[u], gv);
        pk_unpack<D, E>(hp[u], hv);
        if (up) {
          pk_unpack<R, E>(uu[u], uv);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) uv[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float xv = (hv[e] - mu) * rs;
          cg.lo[e] = __builtin_fmaf(gv[e], xv, cg.lo[e]);
          cb.lo[e] += gv[e];
          gv[e] = __builtin_fmaf(rs, __builtin_fmaf(-xv, mx, gv[e] * g[e] - ma), uv[e]);
        }
        pk_store<D, E>(dx + tt * px + cx, pk_pack<D, E>(gv));
        if (dres) pk_store<R, E>(dres + tt * pr + cr, pk_pack<R, E>(gv));
      }
      cg.tick(rows);
      cb.tick(rows);
    }
  }
  if (!a.pg) return;  // uniform over the launch
  float sg[E], sb[E];
  cg.total(sg);
  cb.total(sb);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    red[w][e][lane] = sg[e];
    red[w][E + e][lane] = sb[e];
  }
  __syncthreads();
  if (w == 0 && active) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sg[e] = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
      sb[e] = ((red[0][E + e][lane] + red[1][E + e][lane]) + red[2][E + e][lane]) + red[3][E + e][lane];
    }
    const size_t o = static_cast<size_t>(ti.rg) * a.H + static_cast<size_t>(cv) * E;
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      store_f32x4(a.pg + o + 4 * q, sg + 4 * q);
      store_f32x4(a.pb + o + 4 * q, sb + 4 * q);
    }
  }
}

template <DT D, DT R> hipError_t ln2_bwd_run(const LnArgs& a, const Ln2Plan& p, hipStream_t s) {
  hipLaunchKernelGGL((ln2_rowsums_kernel<D, R>), dim3(p.rows_grid), dim3(MB_LN2_A_THREADS), 0, s, a, p.nvec);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL((ln2_dx_kernel<D, R>), tile_grid(p.strips, p.G), dim3(kThreads), 0, s, a, p.nvec);
  return hipGetLastError();
}

// Row-group shapes of this many vectors or more keep h in LDS: 512 threads of
// 16 (65536 bf16, 32768 fp32) ran 234 -> 208 us at [2048, 65536] bf16; at
// 4096 vectors (512 threads of 8) the register-resident row was as fast.
#ifndef MB_LN_FWD_LDS_MIN_VEC
#define MB_LN_FWD_LDS_MIN_VEC 8192
#endif
#ifndef MB_LN_FWD_LDS_BLOCKS_PER_CU
#define MB_LN_FWD_LDS_BLOCKS_PER_CU 1
#endif
template <int S> constexpr bool fwd_lds_shape() {
  return kLnShapes[S].tpr * kLnShapes[S].nv >= MB_LN_FWD_LDS_MIN_VEC && kLnShapes[S].rpb == 1;
}

template <DT D, DT R, int S>
hipError_t fwd_shape(const LnArgs& a, const LnPlan& p, hipStream_t s) {
  constexpr LnShape sh = kLnShapes[S];
  if constexpr (fwd_lds_shape<S>()) {
    constexpr int E = ln_epl<D, R>();
    const size_t shm = static_cast<size_t>(sh.tpr) * sh.nv * E * Vec<D>::BYTES;
    const int64_t resident = static_cast<int64_t>(p.cus) * MB_LN_FWD_LDS_BLOCKS_PER_CU;
    const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(a.T, resident)));
    hipLaunchKernelGGL((ln_fwd_lds_kernel<D, R, sh.tpr, sh.nv>), dim3(grid), dim3(sh.tpr), shm, s,
                       static_cast<const char*>(a.x), static_cast<const char*>(a.res),
                       static_cast<const char*>(a.gamma), static_cast<const char*>(a.beta),
                       static_cast<char*>(a.hout), static_cast<char*>(a.y), a.mean, a.rstd, a.T,
                       static_cast<int>(a.H), a.eps, a.gshift);
  } else {
    hipLaunchKernelGGL((ln_fwd_kernel<D, R, sh.tpr, sh.nv, sh.rpb>), dim3(p.grid), dim3(sh.tpr * sh.rpb), 0, s,
                       static_cast<const char*>(a.x), static_cast<const char*>(a.res),
                       static_cast<const char*>(a.gamma), static_cast<const char*>(a.beta),
                       static_cast<char*>(a.hout), static_cast<char*>(a.y), a.mean, a.rstd, a.T,
                       static_cast<int>(a.H), a.eps, a.gshift);
  }
  return hipGetLastError();
}

// Backward rows of at most 1024 vectors (wider ones take the wide-row kernels),
// so the row kernel's shapes hold at most 1024 vectors here.
template <int S> constexpr bool bwd_shape_used() { return kLnShapes[S].tpr * kLnShapes[S].nv <= MB_LN2_ROW_VEC; }

template <DT D, DT R, int S>
hipError_t bwd_shape(const LnArgs& a, const LnPlan& p, hipStream_t s) {
  constexpr LnShape sh = kLnShapes[S];
  if constexpr (!bwd_shape_used<S>()) {
    return hipErrorInvalidValue;
  } else {
    const auto dy = static_cast<const char*>(a.dy);
    const auto h = static_cast<const char*>(a.h);
    const auto gamma = static_cast<const char*>(a.gamma);
    const auto dh_in = static_cast<const char*>(a.dh_in);
    const auto dx = static_cast<char*>(a.dx);
    const auto dres = static_cast<char*>(a.dres);
    const int H = static_cast<int>(a.H);
    const dim3 grid(p.grid), block(sh.tpr * sh.rpb);
    if (a.pg) {
      const size_t shm = sh.rpb * 2 * static_cast<size_t>(H) * sizeof(float);
      hipLaunchKernelGGL((ln_bwd_kernel<D, R, sh.tpr, sh.nv, sh.rpb, true>), grid, block, shm, s, dy, h, gamma,
                         a.cmean, a.crstd, dh_in, dx, dres, a.pg, a.pb, a.T, H, a.gshift);
    } else {
      hipLaunchKernelGGL((ln_bwd_kernel<D, R, sh.tpr, sh.nv, sh.rpb, false>), grid, block, 0, s, dy, h, gamma,
                         a.cmean, a.crstd, dh_in, dx, dres, nullptr, nullptr, a.T, H, a.gshift);
    }
    return hipGetLastError();
  }
}

template <DT D, DT R, bool BWD, int S = 0>
hipError_t by_shape(const LnArgs& a, const LnPlan& p, hipStream_t s) {
  if constexpr (S < kLnNumShapes) {
    if (p.shape == S) return BWD ? bwd_shape<D, R, S>(a, p, s) : fwd_shape<D, R, S>(a, p, s);
    return by_shape<D, R, BWD, S + 1>(a, p, s);
  } else {
    return hipErrorInvalidValue;
  }
}

template <bool BWD>
hipError_t by_dtype(const LnArgs& a, const LnPlan& p, hipStream_t s) {
  const DT d = static_cast<DT>(a.dt), r = static_cast<DT>(a.rdt);
  if (d == DT::F32 && r == DT::F32) return by_shape<DT::F32, DT::F32, BWD>(a, p, s);
  if (d == DT::BF16 && r == DT::BF16) return by_shape<DT::BF16, DT::BF16, BWD>(a, p, s);
  if (d == DT::BF16 && r == DT::F32) return by_shape<DT::BF16, DT::F32, BWD>(a, p, s);
  if (d == DT::F16 && r == DT::F16) return by_shape<DT::F16, DT::F16, BWD>(a, p, s);
  if (d == DT::F16 && r == DT::F32) return by_shape<DT::F16, DT::F32, BWD>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ln_fwd(const LnArgs& a, const LnPlan& p, hipStream_t s) { return by_dtype<false>(a, p, s); }
hipError_t launch_ln_bwd(const LnArgs& a, const LnPlan& p, hipStream_t s) { return by_dtype<true>(a, p, s); }
// Threads of the resident-block backward (each holds 2048 / MB_LN_BLOCK_TPR
// vectors of a row). 1024 threads of 2 leave 128 registers a thread, which
// the fp16 / bf16 builds overflow into scratch: 1.7-1.8x slower than 512.
#ifndef MB_LN_BLOCK_TPR
#define MB_LN_BLOCK_TPR 512
#endif
#ifndef MB_LN_BLOCK_LDS
#define MB_LN_BLOCK_LDS 1  // rows of 16-byte pieces staged through LDS (+4 to +9 %)
#endif
template <DT D, DT R> hipError_t ln_block_run(const LnArgs& a, const LnBlockPlan& p, hipStream_t s) {
  constexpr int TPR = MB_LN_BLOCK_TPR, NV = 2048 / TPR;
  if constexpr (MB_LN_BLOCK_LDS && ln_epl<D, R>() * Vec<D>::BYTES == 16) {
    // two stages of dy and h, and two chunks of 64 rows' mean and rstd per wave
    const size_t shm = static_cast<size_t>(2 * 2 * NV * TPR) * 16 + static_cast<size_t>(TPR / 64) * 2 * 2 * 64 * 4;
    static_assert(2 * 2 * NV * TPR * 16 + (TPR / 64) * 2 * 2 * 64 * 4 <= 160 * 1024, "fits a CU's LDS");
    hipLaunchKernelGGL((ln_bwd_block_lds_kernel<D, R, TPR, NV>), dim3(p.grid), dim3(TPR), shm, s, a,
                       p.rows_per_block);
  } else {
    hipLaunchKernelGGL((ln_bwd_block_kernel<D, R, TPR, NV>), dim3(p.grid), dim3(TPR), 0, s, a, p.rows_per_block);
  }
  return hipGetLastError();
}

hipError_t launch_ln_block_bwd(const LnArgs& a, const LnBlockPlan& p, hipStream_t s) {
  if (p.nvec > 2048) return hipErrorInvalidValue;  // the kernel holds 2048 vectors per block
  const DT d = static_cast<DT>(a.dt), r = static_cast<DT>(a.rdt);
  if (d == DT::F32 && r == DT::F32) return ln_block_run<DT::F32, DT::F32>(a, p, s);
  if (d == DT::BF16 && r == DT::BF16) return ln_block_run<DT::BF16, DT::BF16>(a, p, s);
  if (d == DT::BF16 && r == DT::F32) return ln_block_run<DT::BF16, DT::F32>(a, p, s);
  if (d == DT::F16 && r == DT::F16) return ln_block_run<DT::F16, DT::F16>(a, p, s);
  if (d == DT::F16 && r == DT::F32) return ln_block_run<DT::F16, DT::F32>(a, p, s);
  return hipErrorInvalidValue;
}

namespace {

std::atomic<int> g_team_spin_limit{MB_LN_TEAM_SPIN_LIMIT};
int team_spin_limit() { return g_team_spin_limit.load(std::memory_order_relaxed); }

constexpr int kTeamTpr = 256, kTeamNv = kLnTeamVec / kTeamTpr;  // 256 threads of 4 vectors
constexpr size_t team_stage_bytes() { return static_cast<size_t>(2 * 2 * kTeamNv * kTeamTpr) * 16; }  // 64 KiB

template <DT D, DT R> hipError_t ln_team_run(const LnArgs& a, const LnTeamPlan& p, hipStream_t s) {
  constexpr int TPR = kTeamTpr, NV = kTeamNv;
  const int64_t nslots = a.T * p.members;
  uint64_t* slots = reinterpret_cast<uint64_t*>(a.rowsums);
  uint32_t* flags = reinterpret_cast<uint32_t*>(slots + nslots);
  const unsigned fill_grid = static_cast<unsigned>(std::min<int64_t>((nslots + 255) / 256, 4096));
  hipLaunchKernelGGL(team_fill_kernel, dim3(fill_grid), dim3(256), 0, s, slots, nslots, flags, a.T);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL((ln_bwd_team_kernel<D, R, TPR, NV>), dim3(p.grid), dim3(TPR), team_stage_bytes(), s, a,
                     p.members, p.slice, p.rows_per_team, team_spin_limit(), flags);
  if (hipError_t e = hipGetLastError()) return e;
  const unsigned fix_grid = static_cast<unsigned>((a.T + TPR - 1) / TPR);
  hipLaunchKernelGGL((ln_team_fixup_kernel<D, R, TPR, NV>), dim3(fix_grid), dim3(TPR), 0, s, a, p.members, p.slice,
                     static_cast<const uint32_t*>(flags));
  return hipGetLastError();
}

// Asked of the runtime once per dtype pair (the workspace query and every
// launch use it); 1 when no device answers, and then asked again next time.
template <DT D, DT R> int team_occupancy() {
  constexpr int TPR = kTeamTpr, NV = kTeamNv;
  static std::atomic<int> cached{0};
  if (const int c = cached.load(std::memory_order_relaxed)) return c;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ln_bwd_team_kernel<D, R, TPR, NV>, TPR,
                                                   team_stage_bytes()) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return 1;
  }
  n = std::min(n, kLnTeamMaxBlocksPerCu);
  cached.store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

void set_ln_team_spin_limit(int polls) {
  g_team_spin_limit.store(polls < 0 ? MB_LN_TEAM_SPIN_LIMIT : polls, std::memory_order_relaxed);
}

int ln_team_blocks_per_cu(int dt, int rdt) {
  const DT d = static_cast<DT>(dt), r = static_cast<DT>(rdt);
  if (d == DT::F32 && r == DT::F32) return team_occupancy<DT::F32, DT::F32>();
  if (d == DT::BF16 && r == DT::BF16) return team_occupancy<DT::BF16, DT::BF16>();
  if (d == DT::BF16 && r == DT::F32) return team_occupancy<DT::BF16, DT::F32>();
  if (d == DT::F16 && r == DT::F16) return team_occupancy<DT::F16, DT::F16>();
  if (d == DT::F16 && r == DT::F32) return team_occupancy<DT::F16, DT::F32>();
  return 1;
}

hipError_t launch_ln_team_bwd(const LnArgs& a, const LnTeamPlan& p, hipStream_t s) {
  if (p.members < 1 || p.members > kLnTeamMaxMembers || p.slice < 1 || p.slice > kLnTeamVec ||
      static_cast<int64_t>(p.members) * p.slice < p.nvec || static_cast<int64_t>(p.members - 1) * p.slice >= p.nvec)
    return hipErrorInvalidValue;  // the slices cover the row, each holds at least one vector
  const DT d = static_cast<DT>(a.dt), r = static_cast<DT>(a.rdt);
  if (d == DT::F32 && r == DT::F32) return ln_team_run<DT::F32, DT::F32>(a, p, s);
  if (d == DT::BF16 && r == DT::BF16) return ln_team_run<DT::BF16, DT::BF16>(a, p, s);
  if (d == DT::BF16 && r == DT::F32) return ln_team_run<DT::BF16, DT::F32>(a, p, s);
  if (d == DT::F16 && r == DT::F16) return ln_team_run<DT::F16, DT::F16>(a, p, s);
  if (d == DT::F16 && r == DT::F32) return ln_team_run<DT::F16, DT::F32>(a, p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_ln2_bwd(const LnArgs& a, const Ln2Plan& p, hipStream_t s) {
  const DT d = static_cast<DT>(a.dt), r = static_cast<DT>(a.rdt);
  if (d == DT::F32 && r == DT::F32) return ln2_bwd_run<DT::F32, DT::F32>(a, p, s);
  if (d == DT::BF16 && r == DT::BF16) return ln2_bwd_run<DT::BF16, DT::BF16>(a, p, s);
  if (d == DT::BF16 && r == DT::F32) return ln2_bwd_run<DT::BF16, DT::F32>(a, p, s);
  if (d == DT::F16 && r == DT::F16) return ln2_bwd_run<DT::F16, DT::F16>(a, p, s);
  if (d == DT::F16 && r == DT::F32) return ln2_bwd_run<DT::F16, DT::F32>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace mb
