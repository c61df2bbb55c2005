// mb_device.hpp -- device-side building blocks shared by the epilogue kernels
// (gfx950, wave64).
//
// 16-byte vector I/O with streaming (non-temporal) hints, fp32 <-> bf16/fp16
// conversion (round to nearest even in hardware), Philox4x32-10, and the
// logistic function in a cancellation- and overflow-free form that the GeLU
// and SiLU paths use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mb {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

enum class DT : int { F32 = 0, F16 = 1, BF16 = 2 };

// Elements per 16-byte vector.
template <DT D> struct Vec;
template <> struct Vec<DT::F32> { static constexpr int N = 4; static constexpr int BYTES = 4; };
template <> struct Vec<DT::F16> { static constexpr int N = 8; static constexpr int BYTES = 2; };
template <> struct Vec<DT::BF16> { static constexpr int N = 8; static constexpr int BYTES = 2; };

// Geometry of every tiled kernel: a block is 4 waves; a wave covers one strip
// of 64 consecutive 16-byte column vectors (1 KiB of a row) and walks rows.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStrip = 64;

// Block order. Workgroups are dealt to the 8 XCDs round-robin by linear block
// id. With the row group as the fast grid dimension, every XCD works on all
// column strips (and so on all memory channels a row spans) rather than on a
// fixed 1-in-8 subset of columns.
#ifndef MB_RG_MAJOR
#define MB_RG_MAJOR 0
#endif
struct TileIdx {
  int strip;  // column strip of 64 vectors
  int rg;     // row group
  int G;      // row groups in the grid
};
__device__ __forceinline__ TileIdx tile_idx() {
  if constexpr (MB_RG_MAJOR) return TileIdx{static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.x),
                                            static_cast<int>(gridDim.x)};
  return TileIdx{static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), static_cast<int>(gridDim.y)};
}
// The wave's index in its block as a scalar, so that rows chosen from it are
// known to be wave-uniform (buffer-store descriptors need that). With it the
// compiler moves the row loop's arithmetic to the scalar unit, which measured
// 13 % slower for the exact GeLU forward (global stores), so kernels take the
// scalar form only when their stores need it: wave_index<true>().
template <bool SCALAR = true> __device__ __forceinline__ int wave_index() {
  if constexpr (SCALAR) return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  return static_cast<int>(threadIdx.x >> 6);
}
__host__ __forceinline__ dim3 tile_grid(int strips, int G) {
  if constexpr (MB_RG_MAJOR) return dim3(G, strips);
  return dim3(strips, G);
}

// ---------------------------------------------------------------- vector I/O

// Streaming tensors are read and written once: non-temporal hints keep them
// from displacing reused lines (bias) in the caches.
#ifndef MB_NT_LOAD
#define MB_NT_LOAD 1
#endif
#ifndef MB_NT_STORE
#define MB_NT_STORE 1
#endif
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  if constexpr (MB_NT_LOAD) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_stream(void* p, u32x4 v) {
  if constexpr (MB_NT_STORE)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ u32x4 ld_keep(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Bit casts always take a plain scalar or whole vector: clang lowers a
// __builtin_bit_cast of an ext_vector element expression (v[k]) as a cast of
// element 0, so vector elements are first copied into scalars.
__device__ __forceinline__ float as_float(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned as_uint(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  const f32x2 x = {a, b};
  const bf16x2 h = __builtin_convertvector(x, bf16x2);  // v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(unsigned, h);
}
__device__ __forceinline__ unsigned pk_f16(float a, float b) {
  const f32x2 x = {a, b};
  const f16x2 h = __builtin_convertvector(x, f16x2);  // v_cvt_pk_f16_f32, nearest even
  return __builtin_bit_cast(unsigned, h);
}

template <DT D> __device__ __forceinline__ void unpack(u32x4 v, float* f);

template <> __device__ __forceinline__ void unpack<DT::F32>(u32x4 v, float* f) {
  const unsigned w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
  f[0] = as_float(w0);
  f[1] = as_float(w1);
  f[2] = as_float(w2);
  f[3] = as_float(w3);
}
template <> __device__ __forceinline__ void unpack<DT::BF16>(u32x4 v, float* f) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = as_float(w[k] << 16);
    f[2 * k + 1] = as_float(w[k] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void unpack<DT::F16>(u32x4 v, float* f) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned u = w[k];
    const f16x2 h = __builtin_bit_cast(f16x2, u);
    const f32x2 x = __builtin_convertvector(h, f32x2);
    f[2 * k] = x.x;
    f[2 * k + 1] = x.y;
  }
}

template <DT D> __device__ __forceinline__ u32x4 pack(const float* f);

template <> __device__ __forceinline__ u32x4 pack<DT::F32>(const float* f) {
  return u32x4{as_uint(f[0]), as_uint(f[1]), as_uint(f[2]), as_uint(f[3])};
}
template <> __device__ __forceinline__ u32x4 pack<DT::BF16>(const float* f) {
  return u32x4{pk_bf16(f[0], f[1]), pk_bf16(f[2], f[3]), pk_bf16(f[4], f[5]), pk_bf16(f[6], f[7])};
}
template <> __device__ __forceinline__ u32x4 pack<DT::F16>(const float* f) {
  return u32x4{pk_f16(f[0], f[1]), pk_f16(f[2], f[3]), pk_f16(f[4], f[5]), pk_f16(f[6], f[7])};
}

// Four fp32 values to a 16-byte aligned address.
__device__ __forceinline__ void store_f32x4(float* dst, const float* s) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{s[0], s[1], s[2], s[3]};
}

// N consecutive elements of storage type D as fp32, for groups of 8 or 16
// bytes (4 bf16/fp16, or a full 16-byte vector). Used where a lane's element
// count is set by a wider tensor next to this one (an fp32 residual beside
// bf16 activations), so that every load and store instruction of the wave
// still covers one contiguous span of memory.
template <DT D, int N> __device__ __forceinline__ void ld_elems(const char* p, float* f) {
  if constexpr (N * Vec<D>::BYTES == 16) {
    unpack<D>(ld_stream(p), f);
  } else {
    static_assert(N == 4 && Vec<D>::BYTES == 2, "8-byte groups hold 4 bf16/fp16 values");
    u32x2 v;
    if constexpr (MB_NT_LOAD) v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    else v = *reinterpret_cast<const u32x2*>(p);
    const u32x4 w = {v.x, v.y, 0u, 0u};
    float t[8];
    unpack<D>(w, t);
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = t[k];
  }
}
// Streaming stores through a buffer descriptor whose base is a wave-uniform
// row address (any tensor size works: only the lane's offset within the row
// is 32-bit), so that the cache policy can be chosen: AUX 2 = nt, 18 = nt sc1
// (non-temporal at system scope, written through the device caches). The
// compiler tracks these stores like any other (waits, register reuse).
// Buffer stores alone streamed 1-2.5 % faster than the global nt stores in
// the dropout-add forward, and sc1 another 1-2.5 % (MI355X, same-process A/B
// under two allocation layouts); each kernel picks by measurement. The row
// address must be the same in every lane of the wave. (An inline-asm global
// store with these bits is not an option: the compiler does not know that such
// a store still reads its data registers after issue and may reuse them.)
template <int AUX> __device__ __forceinline__ void st_buf(char* row, uint32_t off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}
template <int AUX> __device__ __forceinline__ void st_buf(char* row, uint32_t off, u32x2 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, AUX);
}

// Streaming loads through a buffer descriptor on a wave-uniform row, with the
// cache policy AUX (as st_buf), and ld_row: AUX < 0 loads at `at` with the
// global non-temporal load (at == row + off).
template <int AUX> __device__ __forceinline__ u32x4 ld_buf(const char* row, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), 0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
}
template <int AUX> __device__ __forceinline__ u32x4 ld_row(const char* at, const char* row, uint32_t off) {
  if constexpr (AUX < 0)
    return ld_stream(at);
  else
    return ld_buf<AUX>(row, off);
}

template <DT D, int N> __device__ __forceinline__ u32x2 pack4(const float* f) {
  static_assert(N == 4 && Vec<D>::BYTES == 2, "8-byte groups hold 4 bf16/fp16 values");
  const unsigned w0 = D == DT::BF16 ? pk_bf16(f[0], f[1]) : pk_f16(f[0], f[1]);
  const unsigned w1 = D == DT::BF16 ? pk_bf16(f[2], f[3]) : pk_f16(f[2], f[3]);
  return u32x2{w0, w1};
}
// N elements of D at byte `off` of a wave-uniform row, through st_buf
template <DT D, int N, int AUX> __device__ __forceinline__ void st_elems_buf(char* row, uint32_t off, const float* f) {
  if constexpr (N * Vec<D>::BYTES == 16)
    st_buf<AUX>(row, off, pack<D>(f));
  else
    st_buf<AUX>(row, off, pack4<D, N>(f));
}
// Store of a 16-byte vector or of N elements: AUX < 0 stores at `at` with the
// global non-temporal store, else at byte `off` of the wave-uniform row `row`
// with st_buf<AUX>. Callers pass both forms of the same address (at == row +
// off); the global path keeps the per-lane address form the kernels had
// before the buffer stores, which the compiler turns into faster code for the
// exact GeLU forward (5 %) than row + off.
template <int AUX> __device__ __forceinline__ void st_row(char* at, char* row, uint32_t off, u32x4 v) {
  if constexpr (AUX < 0)
    st_stream(at, v);
  else
    st_buf<AUX>(row, off, v);
}
template <DT D, int N, int AUX>
__device__ __forceinline__ void st_row_elems(char* at, char* row, uint32_t off, const float* f);

template <DT D, int N> __device__ __forceinline__ void st_elems(char* p, const float* f) {
  if constexpr (N * Vec<D>::BYTES == 16) {
    st_stream(p, pack<D>(f));
  } else {
    const u32x2 v = pack4<D, N>(f);
    if constexpr (MB_NT_STORE) __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
    else *reinterpret_cast<u32x2*>(p) = v;
  }
}
template <DT D, int N, int AUX>
__device__ __forceinline__ void st_row_elems(char* at, char* row, uint32_t off, const float* f) {
  if constexpr (AUX < 0)
    st_elems<D, N>(at, f);
  else
    st_elems_buf<D, N, AUX>(row, off, f);
}

// Value of fp32 x after rounding to storage type D (the residual cast).
template <DT D> __device__ __forceinline__ float round_to(float x);
template <> __device__ __forceinline__ float round_to<DT::F32>(float x) { return x; }
template <> __device__ __forceinline__ float round_to<DT::BF16>(float x) {
  return as_float(pk_bf16(x, 0.0f) << 16);
}
template <> __device__ __forceinline__ float round_to<DT::F16>(float x) {
  return static_cast<float>(static_cast<_Float16>(x));
}

// ---------------------------------------------------------------- Philox

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit products and an xor with the round key; the key advances by
// the Weyl increments after every round. On gfx950 each product is a single
// v_mad_u64_u32 and each three-way xor a single v_bitop3_b32 (truth table
// 0x96 = a ^ b ^ c, new in CDNA4); the key lives in scalar registers.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t m0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
    const uint64_t m1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
    const uint32_t n0 = xor3(static_cast<uint32_t>(m1 >> 32), c[1], k0);
    const uint32_t n2 = xor3(static_cast<uint32_t>(m0 >> 32), c[3], k1);
    c[1] = static_cast<uint32_t>(m1);
    c[3] = static_cast<uint32_t>(m0);
    c[0] = n0;
    c[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Keep flags of the 4 consecutive elements 4q .. 4q+3: counter (q, offset),
// key seed; element 4q+k keeps iff word k >= theta, given as a 32-bit
// threshold and a drop-everything flag (theta = 2^32).
__device__ __forceinline__ void keep4(uint64_t q, uint32_t o0, uint32_t o1, uint32_t k0, uint32_t k1,
                                      uint32_t theta32, uint32_t drop_all, bool* keep) {
  uint32_t c[4] = {static_cast<uint32_t>(q), static_cast<uint32_t>(q >> 32), o0, o1};
  philox4x32_10(c, k0, k1);
#pragma unroll
  for (int k = 0; k < 4; ++k) keep[k] = c[k] >= theta32 && !drop_all;
}

// Scheduling fence after a software pipeline's prefetch (emits no code): the
// compiler may not move instructions across it, so the next rows' loads all
// issue before this rows' arithmetic instead of being spread through it.
#ifndef MB_PREFETCH_FENCE
#define MB_PREFETCH_FENCE 1
#endif
__device__ __forceinline__ void prefetch_fence() {
  if constexpr (MB_PREFETCH_FENCE) __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------- activations

// An opaque VGPR copy of a constant. On gfx950 a VALU instruction that reads
// an SGPR operand issues at about 60 % of the rate of the same instruction
// with VGPR, inline-constant or literal operands (measured on MI355X: 1.9
// against 2.8-3.5 wave instructions per CU per ns), and the compiler keeps
// loop-invariant constants of three-operand instructions in SGPRs. The asm
// has no side effects, so the compiler hoists the copy out of loops but cannot
// fold it back into an SGPR. Used only where it costs no occupancy (one VGPR
// per constant) and measured faster: the exact GeLU forward (+4.6 %).
__device__ __forceinline__ float vconst(float c) {
  float v;
  asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(c));
  return v;
}

// Value with a deferred scale: the product of `v` and `sc` (1 or a power of
// two below 1), applied by the caller to its final product, so that results
// in the fp32 subnormal range are rounded only once however large the factors
// they are multiplied by (the up half, the gradient, the router weight).
struct ScaledF {
  float v;
  float sc;
};

// The logistic function sigma(t) goes through e = 2^-|x|, x = t log2(e) the
// argument in base-2 units, and r = 1 / (1 + e):
//   sigma(t) = t >= 0 ? r : e r,    sigma(t) (1 - sigma(t)) = e r^2
// so neither 1 - sigma nor exp of a large positive number is ever formed. The
// hardware exp2 flushes subnormal results, so it is taken as 2^(32 - |x|) =
// 2^32 e, which stays normal down to |x| = 158, and quantities that carry the
// factor e for t < 0 are kept scaled by 2^32, with the deferred scale
// sc = 2^-32 (1 for t >= 0). Below |x| = 158 they are flushed to zero; the
// activation there is below 2^-158 |t|.
struct Logistic {
  float r;   // 1 / (1 + e)
  float s;   // sigma(t) / sc
  float er;  // e r / sc
  float sc;  // 1 or 2^-32
};

// w = 32 - |x|
__device__ __forceinline__ Logistic logistic_scaled(float w, bool pos) {
  const float es = __builtin_amdgcn_exp2f(w);
  Logistic L;
  L.r = __builtin_amdgcn_rcpf(__builtin_fmaf(es, 0x1p-32f, 1.0f));
  const float esr = es * L.r;
  L.s = pos ? L.r : esr;
  L.er = pos ? esr * 0x1p-32f : esr;
  L.sc = pos ? 1.0f : 0x1p-32f;
  return L;
}

constexpr double kLog2e = 1.4426950408889634;
// tanh-approximation constants as printed with the Megatron-LM fusions
// (bias_gelu): sqrt(2/pi), the cubic coefficient, and sqrt(2/pi) * 3 * 0.044715.
constexpr double kGeluK = 0.79788456;
constexpr double kGeluC = 0.044715;
constexpr double kGeluKD = 0.1070322243;
// 0.5 (1 + tanh(u)) = sigma(2u): the logistic argument in base-2 units is
// x = z * (A0 + A1 z^2) with A0 = 2 k log2(e), A1 = 2 k c log2(e); the factor
// A0 + A1 z^2 is positive, so |x| = |z| (A0 + A1 z^2) and x has the sign of z.
constexpr float kGeluA0 = static_cast<float>(2.0 * kGeluK * kLog2e);
constexpr float kGeluA1 = static_cast<float>(2.0 * kGeluK * kGeluC * kLog2e);
constexpr float kSiluA = static_cast<float>(kLog2e);

// Forward only: gelu_tanh(z) = 0.5 z (1 + tanh u) = z sigma(2u) as z r, or
// (z r 2^32 e) with the scale 2^-32 below zero. For z = +-inf or NaN the
// products give what the formula gives (inf, NaN, NaN).
__device__ __forceinline__ ScaledF gelu_tanh_scaled(float z) {
  const float x = z * __builtin_fmaf(z * z, kGeluA1, kGeluA0);
  const float es = __builtin_amdgcn_exp2f(32.0f - __builtin_fabsf(x));
  const float zr = z * __builtin_amdgcn_rcpf(__builtin_fmaf(es, 0x1p-32f, 1.0f));
  ScaledF o;
  o.v = x >= 0.0f ? zr : zr * es;
  o.sc = x >= 0.0f ? 1.0f : 0x1p-32f;
  return o;
}

// Forward only, silu(a) = a sigma(a), in the same form.
__device__ __forceinline__ ScaledF silu_scaled(float a) {
  const float x = a * kSiluA;
  const float es = __builtin_amdgcn_exp2f(32.0f - __builtin_fabsf(x));
  const float ar = a * __builtin_amdgcn_rcpf(__builtin_fmaf(es, 0x1p-32f, 1.0f));
  ScaledF o;
  o.v = x >= 0.0f ? ar : ar * es;
  o.sc = x >= 0.0f ? 1.0f : 0x1p-32f;
  return o;
}

// gelu_tanh and its derivative (the GeLU and gated backward kernels). With
// s = sigma(2u), 1 - t^2 = 4 s (1 - s) and s (1 - s) = e r^2, the derivative
// 0.5 (1+t) + 0.5 z (1-t^2)(k + k' z^2) is
//   d = s + q e r,    q = 2 z r (k + k' z^2)
// evaluated at z clamped to +-1e4, where sigma is exactly 1 or 0 in fp32, so
// that no 0 * inf arises; the value z s takes the unclamped z and is exact
// there too. v and d carry the deferred scale sc. `nan` is z - z (+0, or NaN
// for a NaN or infinite z, where the formula's 0 * inf gives NaN): callers
// add it to their scaled product with d.
struct GeluB {
  float v;    // gelu_tanh(z) / sc
  float d;    // gelu_tanh'(z) / sc, finite for every input
  float nan;  // +0 or NaN
  float sc;
};
__device__ __forceinline__ GeluB gelu_tanh_fwd_bwd(float z) {
  const float zc = __builtin_amdgcn_fmed3f(z, -1e4f, 1e4f);
  const float z2 = zc * zc;
  const Logistic L = logistic_scaled(
      __builtin_fmaf(-__builtin_fabsf(zc), __builtin_fmaf(z2, kGeluA1, kGeluA0), 32.0f), zc >= 0.0f);
  const float q = (zc * L.r) * __builtin_fmaf(z2, static_cast<float>(2.0 * kGeluKD), static_cast<float>(2.0 * kGeluK));
  GeluB o;
  o.v = z * L.s;
  o.d = __builtin_fmaf(q, L.er, L.s);
  o.nan = z - z;
  o.sc = L.sc;
  return o;
}

// silu(a) = a s with s = sigma(a); silu'(a) = s (1 + a (1 - s)) = s + (a r) (e r),
// both carrying the deferred scale sc. For a = +-inf or NaN both give what
// the formula gives.
struct SiluB {
  float v;  // silu(a) / sc
  float d;  // silu'(a) / sc
  float sc;
};
__device__ __forceinline__ SiluB silu_fwd_bwd(float a) {
  const Logistic L = logistic_scaled(__builtin_fmaf(-__builtin_fabsf(a), kSiluA, 32.0f), a >= 0.0f);
  SiluB o;
  o.v = a * L.s;
  o.d = __builtin_fmaf(a * L.r, L.er, L.s);
  o.sc = L.sc;
  return o;
}

// Exact GeLU, 0.5 z (1 + erf(k z)) = z Phi(z), with the constants printed with
// Megatron-LM's fusions: k = 0.70710678 (1/sqrt 2) and 0.3989423 (1/sqrt(2 pi)).
// 1 + erf(k z) = erfc(-k z), and for x = k |z| >= 0 the complementary error
// function is evaluated branch-free as
//   0.5 erfc(x) = t Q(t) exp(-z^2 / 2),   t = 1 / (1 + x / 2),
// with Q a degree-8 polynomial fitted for relative error (fit_erfc.py beside
// this file: least squares on t in [1/8, 1], i.e. x <= 14; the fp32 Horner
// evaluation is within 1.9e-7 relative of 0.5 erfc(x) exp(z^2/2) / t, and the
// small difference between k^2 and 1/2 is part of the fitted function). The
// factor exp(-z^2/2) is the Gaussian of the derivative too, so the backward
// needs one exponential. Then
//   z >= 0:  Phi = 1 - 0.5 erfc(x)        z < 0:  Phi = 0.5 erfc(x)
// so the negative tail is a product, never a difference. Below z = -12 the
// exponent is shifted by 64 (results are subnormal there) and the caller
// multiplies by the deferred scale 2^-64 last. (Unlike the logistic forms,
// whose exponent is shifted by a constant, the shift here depends on z: a
// constant shift of 64 would round the exponent's argument near 63, a relative
// error up to 1.3e-6 near z = 0, too close to the fp32 tolerance.)
constexpr float kErfK = 0.70710678f;
constexpr float kErfPdf = 0.3989423f;
constexpr float kErfQ[9] = {1.410423517e-01f, 1.412065774e-01f, 1.213941872e-01f, 1.020300612e-01f, -1.505985670e-02f,
                            1.417247653e-01f, -2.460705340e-01f, 1.435308009e-01f, -2.979838476e-02f};
// the degree-5 fit (fit_erfc.py: within 3.5e-5 relative) for the forward
// with bf16/fp16 outputs, whose half ulp is 2e-3 or 5e-4 relative
constexpr float kErfQ5[6] = {1.408312619e-01f, 1.445789635e-01f, 1.034489125e-01f,
                             1.344528794e-01f, 1.098317560e-02f, -3.431227431e-02f};
constexpr float kErfTail = -12.0f;
constexpr float kErfShift = 64.0f;
constexpr float kErfScaleDown = 0x1p-64f;

// t Q(t) for x = k |z|; k is kErfK, passed in so that the forward can hold it
// in a VGPR. HALF: the degree-5 polynomial.
template <bool HALF = false>
__device__ __forceinline__ float erf_tq(float z, float k) {
  const float x = __builtin_fabsf(z) * k;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, x, 1.0f));
  constexpr int n = HALF ? 5 : 8;
  float q = HALF ? kErfQ5[n] : kErfQ[n];
#pragma unroll
  for (int j = n - 1; j >= 0; --j) q = __builtin_fmaf(q, t, HALF ? kErfQ5[j] : kErfQ[j]);
  return t * q;
}

// exp(-z^2 / 2) times 2^shift
__device__ __forceinline__ float gauss_scaled(float z, float shift) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(z * z, static_cast<float>(-0.5 * kLog2e), shift));
}

// value and derivative below z = -12 carry the deferred scale 2^-64. HALF
// (bf16/fp16 outputs): erfc from the degree-5 polynomial.
template <bool HALF = false>
__device__ __forceinline__ ScaledF gelu_erf_fwd(float z) {
  const bool tail = z < kErfTail;
  const float h = erf_tq<HALF>(z, vconst(kErfK)) * gauss_scaled(z, tail ? kErfShift : 0.0f);
  ScaledF o;
  o.v = z * (z < 0.0f ? h : 1.0f - h);  // not z - z h: inf * 0 at z = inf
  o.sc = tail ? kErfScaleDown : 1.0f;
  return o;
}

// gelu_erf'(z) = Phi(z) + z * 0.3989423 * exp(-z^2 / 2), both terms carrying the
// same deferred scale
__device__ __forceinline__ ScaledF gelu_erf_grad(float z) {
  const bool tail = z < kErfTail;
  const float E = gauss_scaled(z, tail ? kErfShift : 0.0f);
  const float h = erf_tq(z, kErfK) * E;
  ScaledF o;
  o.v = (z < 0.0f ? h : 1.0f - h) + (z * kErfPdf) * E;
  o.sc = tail ? kErfScaleDown : 1.0f;
  return o;
}

// ---------------------------------------------------------------- reductions

// Combine the 4 waves' per-lane column sums of one block in LDS, in a fixed
// order, and write them as one partial row: dst[0 .. N) for this lane's
// columns (dst already offset to the block's row group and the lane's
// columns; 16-byte aligned). Every thread of the block must call it.
template <int N>
__device__ __forceinline__ void block_column_partials(const float* acc, int wave, int lane, bool active, float* dst) {
  __shared__ float red[kWaves][N][64];
#pragma unroll
  for (int k = 0; k < N; ++k) red[wave][k][lane] = acc[k];
  __syncthreads();
  if (wave == 0 && active) {
    float sum[N];
#pragma unroll
    for (int k = 0; k < N; ++k) sum[k] = ((red[0][k][lane] + red[1][k][lane]) + red[2][k][lane]) + red[3][k][lane];
#pragma unroll
    for (int q = 0; q < N / 4; ++q) store_f32x4(dst + 4 * q, sum + 4 * q);
  }
}

// Two-level fp32 column sums for a lane that visits many rows: the terms go
// into `lo`, which is added into `hi` and cleared every kFlushRows rows, so
// the rounding error of the lane's sum grows with kFlushRows + rows /
// kFlushRows instead of with the number of rows (2^14 rows per lane at 2^24
// tokens). The row count is the same in every lane of a wave.
#ifndef MB_COL_FLUSH_ROWS
#define MB_COL_FLUSH_ROWS 64
#endif
constexpr int kFlushRows = MB_COL_FLUSH_ROWS;
template <int N> struct ColAcc {
  float hi[N], lo[N];
  int rows;
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < N; ++k) hi[k] = lo[k] = 0.0f;
    rows = 0;
  }
  __device__ __forceinline__ void tick(int r) {
    rows += r;
    if (rows >= kFlushRows) {
#pragma unroll
      for (int k = 0; k < N; ++k) {
        hi[k] += lo[k];
        lo[k] = 0.0f;
      }
      rows = 0;
    }
  }
  __device__ __forceinline__ void total(float* out) const {
#pragma unroll
    for (int k = 0; k < N; ++k) out[k] = hi[k] + lo[k];
  }
};

// Sum over the 64 lanes of a wave, in a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace mb
