// mb_abi.cpp -- the C ABI declared in include/mb.h: argument validation (on
// the host, before any HIP call), workspace sizing, and the launches.
#include "mb.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <limits>

#include "mb_launch.hpp"

namespace {

size_t esize(mb_dtype_t dt) {
  switch (dt) {
    case MB_F32: return 4;
    case MB_F16: return 2;
    case MB_BF16: return 2;
    default: return 0;  // any other value a caller passes through the C ABI
  }
}

bool dt_ok(mb_dtype_t dt) { return esize(dt) != 0; }

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

struct Buf {
  const void* p;
  size_t bytes;
};

bool overlap(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool identical(const Buf& a, const Buf& b) { return a.p == b.p && a.bytes == b.bytes; }

// An allowed alias: output `out` may coincide exactly with input `in`.
struct Alias {
  int out;
  int in;
};

// Outputs must not overlap each other; an output may overlap an input only as
// an exact, listed alias.
bool aliasing_ok(std::initializer_list<Buf> outs, std::initializer_list<Buf> ins, std::initializer_list<Alias> ok) {
  const Buf* o = outs.begin();
  const Buf* in = ins.begin();
  const int no = static_cast<int>(outs.size()), ni = static_cast<int>(ins.size());
  for (int a = 0; a < no; ++a) {
    for (int b = a + 1; b < no; ++b)
      if (overlap(o[a], o[b])) return false;
    for (int b = 0; b < ni; ++b) {
      if (!overlap(o[a], in[b])) continue;
      bool allowed = false;
      for (const Alias& al : ok)
        if (al.out == a && al.in == b && identical(o[a], in[b])) allowed = true;
      if (!allowed) return false;
    }
  }
  return true;
}

// Shape rule shared by every op: T >= 0, H > 0, rows made of whole 16-byte
// vectors, byte sizes (up to `width` columns of up to 4-byte elements) that
// fit in int64, and vectors per row that fit in int.
mb_status_t check_shape(int64_t T, int64_t H, mb_dtype_t dt, int width = 1) {
  if (T < 0 || H <= 0) return MB_ERR_SHAPE;
  const size_t es = esize(dt);
  if ((static_cast<uint64_t>(H) * es) % 16 != 0) return MB_ERR_SHAPE;
  const int64_t maxi = std::numeric_limits<int64_t>::max();
  if (H > maxi / (8 * width)) return MB_ERR_SHAPE;
  if (T > 0 && T > maxi / (H * 8 * width)) return MB_ERR_SHAPE;
  if (static_cast<uint64_t>(H) * es * width / 16 > static_cast<uint64_t>(std::numeric_limits<int>::max()))
    return MB_ERR_SHAPE;
  if (T > (int64_t{1} << 40)) return MB_ERR_SHAPE;  // row index bound of the kernels' 64-bit math
  // column strips of 64 vectors form one grid dimension (at most 65535)
  if (static_cast<uint64_t>(H) * es / 16 > uint64_t{65535} * 64) return MB_ERR_SHAPE;
  return MB_OK;
}

bool need(const void* p, size_t bytes) { return bytes == 0 || p != nullptr; }

mb_status_t hip_status(hipError_t e) { return e == hipSuccess ? MB_OK : MB_ERR_HIP; }

// Compute units of the device that runs the work: the device of stream s
// (for_stream), else the calling thread's current device (the workspace
// queries take no stream). Queried once per device; mb::kTunedCUs when no
// device answers (no GPU: the queries and the host-side checks still work,
// and the failed query's error is cleared so that no later call reports it).
int device_cus(hipStream_t s, bool for_stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = -1;
  const hipError_t e = for_stream ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return mb::kTunedCUs;
  }
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
    (void)hipGetLastError();
    return mb::kTunedCUs;
  }
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

int stream_cus(hipStream_t s) { return device_cus(s, true); }
int current_cus() { return device_cus(nullptr, false); }

mb_status_t finish() { return hip_status(hipGetLastError()); }

int nvec_of(int64_t H, mb_dtype_t dt) { return static_cast<int>(static_cast<uint64_t>(H) * esize(dt) / 16); }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool prob_ok(float p) { return !std::isnan(p) && p >= 0.0f && p <= 1.0f; }

mb::DropoutArgs dropout_args(float p, uint64_t seed, uint64_t offset) {
  mb::DropoutArgs d;
  const double t = std::floor(static_cast<double>(p) * 4294967296.0);
  const uint64_t theta = t >= 4294967296.0 ? (uint64_t{1} << 32) : (t <= 0.0 ? 0 : static_cast<uint64_t>(t));
  d.drop_all = theta == (uint64_t{1} << 32) ? 1u : 0u;
  d.theta32 = d.drop_all ? 0u : static_cast<uint32_t>(theta);
  d.scale = p < 1.0f ? static_cast<float>(1.0 / (1.0 - static_cast<double>(p))) : 0.0f;
  d.k0 = static_cast<uint32_t>(seed);
  d.k1 = static_cast<uint32_t>(seed >> 32);
  d.o0 = static_cast<uint32_t>(offset);
  d.o1 = static_cast<uint32_t>(offset >> 32);
  return d;
}

// Row groups of the gated backward: the bias gradient's per-lane column sums
// want a persistent grid; without them (the weights gradient is summed per row)
// the launch shape is its own.
static mb::Tiling glu_bwd_tiling(int64_t tokens, int64_t hidden, mb_dtype_t dt, bool dbias, int cus) {
  return mb::plan_tiling(tokens, nvec_of(hidden, dt), dbias ? MB_GLU_BWD_BLOCKS : MB_GLU_BWD_NODBIAS_BLOCKS, cus);
}

// Partial-row workspace of a column reduction.
size_t col_partials_bytes(const mb::Tiling& t, int64_t cols) { return static_cast<size_t>(t.G) * cols * 4; }

// Second pass of a column reduction over `cols` fp32 columns.
hipError_t reduce_columns(const float* partials, const mb::Tiling& t, int64_t cols, float* out, hipStream_t s) {
  return mb::launch_colsum(partials, t.G, cols, out, s);
}

}  // namespace

extern "C" {

const char* mb_status_string(mb_status_t status) {
  switch (status) {
    case MB_OK: return "MB_OK";
    case MB_ERR_NULL: return "MB_ERR_NULL: a required pointer is NULL";
    case MB_ERR_SHAPE: return "MB_ERR_SHAPE: bad tokens/hidden (rows must be whole 16-byte vectors)";
    case MB_ERR_DTYPE: return "MB_ERR_DTYPE: unsupported dtype combination";
    case MB_ERR_ALIGN: return "MB_ERR_ALIGN: pointer not aligned as required";
    case MB_ERR_ALIAS: return "MB_ERR_ALIAS: buffers overlap in a way this entry point forbids";
    case MB_ERR_PROB: return "MB_ERR_PROB: dropout probability is NaN or outside [0, 1]";
    case MB_ERR_WORKSPACE: return "MB_ERR_WORKSPACE: workspace missing or too small";
    case MB_ERR_HIP: return "MB_ERR_HIP: the HIP runtime reported an error";
    case MB_ERR_SCRATCH:
      return "MB_ERR_SCRATCH: the problem needs more than the static scratch of the no-allocation entry point";
  }
  return "unknown mb_status_t";
}

int mb_abi_version(void) { return 1; }

// ------------------------------------------------------------------ GeLU

static mb_status_t gelu_fwd_common(bool exact, const void* y, const void* bias, void* out, int64_t tokens,
                                   int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  if (!dt_ok(dt)) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  const size_t tb = static_cast<size_t>(tokens) * hidden * esize(dt), bb = hidden * esize(dt);
  if (!need(y, tb) || !need(out, tb)) return MB_ERR_NULL;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(bias, 16)) return MB_ERR_ALIGN;
  if (!aliasing_ok({{out, tb}}, {{y, tb}, {bias, bias ? bb : 0}}, {{0, 0}})) return MB_ERR_ALIAS;
  if (tokens == 0) return MB_OK;
  const mb::Tiling t = mb::plan_tiling(tokens, nvec_of(hidden, dt), MB_GELU_FWD_BLOCKS, stream_cus(s));
  if (hipError_t e = mb::launch_gelu_fwd(dt, exact, y, bias, out, t, s)) return hip_status(e);
  return finish();
}

mb_status_t mb_bias_gelu_fwd(const void* y, const void* bias, void* out, int64_t tokens, int64_t hidden,
                             mb_dtype_t dt, hipStream_t s) {
  return gelu_fwd_common(false, y, bias, out, tokens, hidden, dt, s);
}

mb_status_t mb_bias_gelu_erf_fwd(const void* y, const void* bias, void* out, int64_t tokens, int64_t hidden,
                                 mb_dtype_t dt, hipStream_t s) {
  return gelu_fwd_common(true, y, bias, out, tokens, hidden, dt, s);
}

// The tanh and the exact forms have their own launch shapes (the exact form,
// heavier on the ALU, runs many more row groups), so each has its workspace
// query: the partial rows, then (for more than 32 of them) the chunk sums of
// the ordered two-level column sum.
static mb::Tiling gelu_bwd_tiling(bool exact, int64_t tokens, int64_t hidden, mb_dtype_t dt, int cus) {
  return mb::plan_tiling(tokens, nvec_of(hidden, dt), exact ? MB_GELU_ERF_BWD_BLOCKS : MB_GELU_BWD_BLOCKS, cus,
                         exact ? MB_GELU_ERF_BWD_MIN_ROWS : MB_GELU_BWD_MIN_ROWS);
}

static size_t gelu_bwd_ws(bool exact, int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias, int cus) {
  if (!with_dbias || !dt_ok(dt) || check_shape(tokens, hidden, dt) != MB_OK || tokens == 0) return 0;
  const mb::Tiling t = gelu_bwd_tiling(exact, tokens, hidden, dt, cus);
  return round_up(col_partials_bytes(t, hidden), 256) +
         static_cast<size_t>(mb::colsum_tall_tmp_floats(t.G, hidden)) * 4;
}

size_t mb_bias_gelu_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias) {
  return gelu_bwd_ws(false, tokens, hidden, dt, with_dbias, current_cus());
}

size_t mb_bias_gelu_erf_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias) {
  return gelu_bwd_ws(true, tokens, hidden, dt, with_dbias, current_cus());
}

// Checks shared by the GeLU backward entry points, apart from the workspace
// size: dtype, shape, required pointers, alignment and aliasing (wsb: the
// caller's workspace, or none).
static mb_status_t gelu_bwd_check(const void* g, const void* y, const void* bias, void* dgrad, float* dbias,
                                  const Buf& wsb, int64_t tokens, int64_t hidden, mb_dtype_t dt) {
  if (!dt_ok(dt)) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  const size_t tb = static_cast<size_t>(tokens) * hidden * esize(dt), bb = hidden * esize(dt);
  if (!need(g, tb) || !need(y, tb) || !need(dgrad, tb)) return MB_ERR_NULL;
  if (!aligned(g, 16) || !aligned(y, 16) || !aligned(dgrad, 16) || !aligned(bias, 16) || !aligned(dbias, 4) ||
      (wsb.bytes && !aligned(wsb.p, 16)))
    return MB_ERR_ALIGN;
  if (!aliasing_ok({{dgrad, tb}, {dbias, dbias ? static_cast<size_t>(hidden) * 4 : 0}, wsb},
                   {{g, tb}, {y, tb}, {bias, bias ? bb : 0}}, {{0, 0}, {0, 1}}))
    return MB_ERR_ALIAS;
  return MB_OK;
}

// The launches of a checked GeLU backward with tokens > 0: the fused pass
// (partial rows into `partials` when dbias is requested), then the ordered
// column sum (through `tmp` when there are more than 512 partial rows).
static mb_status_t gelu_bwd_run(bool exact, const void* g, const void* y, const void* bias, void* dgrad,
                                float* dbias, float* partials, float* tmp, const mb::Tiling& t, int64_t hidden,
                                mb_dtype_t dt, hipStream_t s) {
  if (hipError_t e = mb::launch_gelu_bwd(dt, exact, g, y, bias, dgrad, dbias ? partials : nullptr, t, s))
    return hip_status(e);
  if (dbias)
    if (hipError_t e = mb::launch_colsum_tall(partials, t.G, hidden, tmp, dbias, s)) return hip_status(e);
  return finish();
}

static mb_status_t gelu_bwd_common(bool exact, const void* g, const void* y, const void* bias, void* dgrad,
                                   float* dbias, void* ws, size_t ws_bytes, int64_t tokens, int64_t hidden,
                                   mb_dtype_t dt, hipStream_t s) {
  if (!dt_ok(dt)) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  const int cus = stream_cus(s);
  const size_t need_ws = gelu_bwd_ws(exact, tokens, hidden, dt, dbias != nullptr, cus);
  if (mb_status_t st = gelu_bwd_check(g, y, bias, dgrad, dbias, Buf{need_ws ? ws : nullptr, need_ws}, tokens,
                                      hidden, dt))
    return st;
  if (need_ws && (!ws || ws_bytes < need_ws)) return MB_ERR_WORKSPACE;
  if (tokens == 0) {
    if (!dbias) return MB_OK;
    if (hipError_t e = mb::launch_fill_zero(dbias, hidden, s)) return hip_status(e);
    return finish();
  }
  const mb::Tiling t = gelu_bwd_tiling(exact, tokens, hidden, dt, cus);
  float* partials = static_cast<float*>(ws);
  float* tmp = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up(col_partials_bytes(t, hidden), 256));
  return gelu_bwd_run(exact, g, y, bias, dgrad, dbias, partials, tmp, t, hidden, dt, s);
}

mb_status_t mb_bias_gelu_bwd(const void* g, const void* y, const void* bias, void* dgrad, float* dbias, void* ws,
                             size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  return gelu_bwd_common(false, g, y, bias, dgrad, dbias, ws, ws_bytes, tokens, hidden, dt, s);
}

mb_status_t mb_bias_gelu_erf_bwd(const void* g, const void* y, const void* bias, void* dgrad, float* dbias,
                                 void* ws, size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                 hipStream_t s) {
  return gelu_bwd_common(true, g, y, bias, dgrad, dbias, ws, ws_bytes, tokens, hidden, dt, s);
}

// The variant that allocates nothing: the partial rows go to the library's
// static device scratch (MB_NOALLOC_SCRATCH_BYTES per device, mb_noalloc.hip).
// Its launch shape is the tanh backward's, with the row groups capped so that
// their partial rows fit the scratch and stay within one column-sum launch
// (at most 512), so no chunk-sum buffer is needed. Nothing in the scratch has
// to start at zero: the fused pass writes every partial row the column sum
// reads.
mb_status_t mb_bias_gelu_bwd_noalloc(const void* g, const void* y, const void* bias, void* dgrad, float* dbias,
                                     int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  if (mb_status_t st = gelu_bwd_check(g, y, bias, dgrad, dbias, Buf{nullptr, 0}, tokens, hidden, dt)) return st;
  const int64_t row_bytes = hidden * 4;  // one fp32 partial row
  const int64_t max_rows = static_cast<int64_t>(MB_NOALLOC_SCRATCH_BYTES) / row_bytes;
  if (dbias && max_rows < 1) return MB_ERR_SCRATCH;
  if (tokens == 0) {
    if (!dbias) return MB_OK;
    if (hipError_t e = mb::launch_fill_zero(dbias, hidden, s)) return hip_status(e);
    return finish();
  }
  mb::Tiling t = gelu_bwd_tiling(false, tokens, hidden, dt, stream_cus(s));
  if (!dbias) return gelu_bwd_run(false, g, y, bias, dgrad, nullptr, nullptr, nullptr, t, hidden, dt, s);
  int64_t G = t.G;
  if (G > max_rows) G = max_rows;
  if (G > 512) G = 512;
  t.G = static_cast<int>(G);
  void* scratch = nullptr;
  if (hipError_t e = mb::noalloc_scratch(s, &scratch)) return hip_status(e);
  return gelu_bwd_run(false, g, y, bias, dgrad, dbias, static_cast<float*>(scratch), nullptr, t, hidden, dt, s);
}

// ------------------------------------------------------------------ dropout-add

static mb_status_t bda_common(const void* x, const void* bias, const void* residual, mb_dtype_t residual_dt,
                              void* out, int64_t tokens, int64_t hidden, mb_dtype_t dt, bool train, float p,
                              uint64_t seed, uint64_t offset, hipStream_t s) {
  if (!dt_ok(dt) || !dt_ok(residual_dt)) return MB_ERR_DTYPE;
  if (residual_dt != dt && residual_dt != MB_F32) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  if (train && !prob_ok(p)) return MB_ERR_PROB;
  const size_t tb = static_cast<size_t>(tokens) * hidden * esize(dt);
  const size_t rb = static_cast<size_t>(tokens) * hidden * esize(residual_dt);
  const size_t bb = hidden * esize(dt);
  if (!need(x, tb) || !need(residual, rb) || !need(out, tb)) return MB_ERR_NULL;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(out, 16) || !aligned(bias, 16)) return MB_ERR_ALIGN;
  if (!aliasing_ok({{out, tb}}, {{x, tb}, {residual, rb}, {bias, bias ? bb : 0}}, {{0, 0}, {0, 1}}))
    return MB_ERR_ALIAS;
  if (tokens == 0) return MB_OK;
  const int lanes = static_cast<int>(hidden / mb::bda_elems_per_lane(dt, residual_dt));
  const bool mixed = residual_dt == MB_F32 && dt != MB_F32;
  const mb::Tiling t =
      mb::plan_tiling(tokens, lanes, !mixed ? MB_BDA_BLOCKS : train ? MB_BDA_MIXED_TRAIN_BLOCKS : MB_BDA_MIXED_BLOCKS,
                      stream_cus(s));
  const mb::DropoutArgs d = train ? dropout_args(p, seed, offset) : mb::DropoutArgs{};
  if (hipError_t e = mb::launch_bda(dt, residual_dt, train, x, bias, residual, out, hidden, t, d, s))
    return hip_status(e);
  return finish();
}

mb_status_t mb_bias_dropout_add_train(const void* x, const void* bias, const void* residual, mb_dtype_t residual_dt,
                                      void* out, int64_t tokens, int64_t hidden, mb_dtype_t dt, float p,
                                      uint64_t seed, uint64_t offset, hipStream_t s) {
  return bda_common(x, bias, residual, residual_dt, out, tokens, hidden, dt, true, p, seed, offset, s);
}

mb_status_t mb_bias_dropout_add_infer(const void* x, const void* bias, const void* residual, mb_dtype_t residual_dt,
                                      void* out, int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  return bda_common(x, bias, residual, residual_dt, out, tokens, hidden, dt, false, 0.0f, 0, 0, s);
}

// Row groups of the dropout-add backward. The lane layout and the launch
// shape depend on the residual dtype (fp32 beside bf16/fp16 or not), which the
// workspace query does not take: it returns the larger of the two layouts'
// partial rows. Without the bias gradient the launch shape is its own.
static mb::Tiling bda_bwd_tiling(int64_t tokens, int64_t hidden, mb_dtype_t dt, mb_dtype_t residual_dt, bool dbias,
                                 int cus) {
  const int lanes = static_cast<int>(hidden / mb::bda_elems_per_lane(dt, residual_dt));
  const bool mixed = residual_dt == MB_F32 && dt != MB_F32;
  const int blocks = !dbias ? MB_BDA_BWD_NODBIAS_BLOCKS : mixed ? MB_BDA_BWD_MIXED_BLOCKS : MB_BDA_BWD_BLOCKS;
  return mb::plan_tiling(tokens, lanes, blocks, cus);
}

static size_t bda_bwd_ws(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias, int cus) {
  if (!with_dbias || !dt_ok(dt) || check_shape(tokens, hidden, dt) != MB_OK || tokens == 0) return 0;
  const size_t same = col_partials_bytes(bda_bwd_tiling(tokens, hidden, dt, dt, true, cus), hidden);
  const size_t mixed = col_partials_bytes(bda_bwd_tiling(tokens, hidden, dt, MB_F32, true, cus), hidden);
  return same > mixed ? same : mixed;
}

size_t mb_bias_dropout_add_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias) {
  return bda_bwd_ws(tokens, hidden, dt, with_dbias, current_cus());
}

mb_status_t mb_bias_dropout_add_bwd(const void* g, void* dx, void* dresidual, mb_dtype_t residual_dt, float* dbias,
                                    void* ws, size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                    float p, uint64_t seed, uint64_t offset, hipStream_t s) {
  if (!dt_ok(dt) || !dt_ok(residual_dt)) return MB_ERR_DTYPE;
  if (residual_dt != dt && residual_dt != MB_F32) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  if (!prob_ok(p)) return MB_ERR_PROB;
  const size_t tb = static_cast<size_t>(tokens) * hidden * esize(dt);
  const size_t rb = static_cast<size_t>(tokens) * hidden * esize(residual_dt);
  if (!need(g, tb) || !need(dx, tb)) return MB_ERR_NULL;
  const int cus = stream_cus(s);
  const size_t need_ws = bda_bwd_ws(tokens, hidden, dt, dbias != nullptr, cus);
  if (!aligned(g, 16) || !aligned(dx, 16) || !aligned(dresidual, 16) || !aligned(dbias, 4) ||
      (need_ws && !aligned(ws, 16)))
    return MB_ERR_ALIGN;
  if (need_ws && (!ws || ws_bytes < need_ws)) return MB_ERR_WORKSPACE;
  const Buf wsb{need_ws ? ws : nullptr, need_ws};
  const Buf resb{dresidual, dresidual ? rb : 0};
  const Buf dbb{dbias, dbias ? static_cast<size_t>(hidden) * 4 : 0};
  if (residual_dt == dt) {
    if (!aliasing_ok({{dx, tb}, resb, dbb, wsb}, {{g, tb}}, {{0, 0}, {1, 0}})) return MB_ERR_ALIAS;
  } else {
    if (!aliasing_ok({{dx, tb}, resb, dbb, wsb}, {{g, tb}}, {{0, 0}})) return MB_ERR_ALIAS;
  }
  if (tokens == 0) {
    if (!dbias) return MB_OK;
    if (hipError_t e = mb::launch_fill_zero(dbias, hidden, s)) return hip_status(e);
    return finish();
  }
  const mb::Tiling t = bda_bwd_tiling(tokens, hidden, dt, residual_dt, dbias != nullptr, cus);
  float* partials = dbias ? static_cast<float*>(ws) : nullptr;
  if (hipError_t e = mb::launch_bda_bwd(dt, residual_dt, g, dx, dresidual, partials, hidden, t,
                                        dropout_args(p, seed, offset), s))
    return hip_status(e);
  if (dbias)
    if (hipError_t e = reduce_columns(partials, t, hidden, dbias, s)) return hip_status(e);
  return finish();
}

mb_status_t mb_dropout_mask(uint8_t* bits, int64_t tokens, int64_t hidden, float p, uint64_t seed, uint64_t offset,
                            hipStream_t s) {
  if (tokens < 0 || hidden <= 0 || hidden % 4 != 0) return MB_ERR_SHAPE;
  if (tokens > 0 && tokens > std::numeric_limits<int64_t>::max() / hidden) return MB_ERR_SHAPE;
  if (!prob_ok(p)) return MB_ERR_PROB;
  const int64_t n = tokens * hidden;
  const int64_t nbytes = (n + 7) / 8;
  if ((nbytes + 255) / 256 > std::numeric_limits<int>::max()) return MB_ERR_SHAPE;
  if (!need(bits, static_cast<size_t>(nbytes))) return MB_ERR_NULL;
  if (n == 0) return MB_OK;
  if (hipError_t e = mb::launch_dropout_mask(bits, n, dropout_args(p, seed, offset), s)) return hip_status(e);
  return finish();
}

// ------------------------------------------------------------------ gated units

static mb_status_t glu_fwd_common(int act, const void* in, const void* bias, const void* weights,
                                  mb_dtype_t weights_dt, void* out, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                  hipStream_t s) {
  if (!dt_ok(dt)) return MB_ERR_DTYPE;
  if (weights && weights_dt != dt && weights_dt != MB_F32) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt, 2)) return st;
  const size_t ob = static_cast<size_t>(tokens) * hidden * esize(dt), ib = 2 * ob;
  const size_t bb = 2 * hidden * esize(dt);
  const size_t wb = weights ? static_cast<size_t>(tokens) * esize(weights_dt) : 0;
  if (!need(in, ib) || !need(out, ob)) return MB_ERR_NULL;
  if (!aligned(in, 16) || !aligned(out, 16) || !aligned(bias, 16) ||
      (weights && !aligned(weights, esize(weights_dt))))
    return MB_ERR_ALIGN;
  if (!aliasing_ok({{out, ob}}, {{in, ib}, {bias, bias ? bb : 0}, {weights, wb}}, {})) return MB_ERR_ALIAS;
  if (tokens == 0) return MB_OK;
  const mb::Tiling t = mb::plan_tiling(tokens, nvec_of(hidden, dt), MB_GLU_FWD_BLOCKS, stream_cus(s));
  if (hipError_t e = mb::launch_glu_fwd(act, dt, in, bias, weights, weights ? weights_dt : dt, out, hidden, t, s))
    return hip_status(e);
  return finish();
}

mb_status_t mb_bias_swiglu_fwd(const void* in, const void* bias, const void* weights, mb_dtype_t weights_dt,
                               void* out, int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  return glu_fwd_common(mb::kSwiGLU, in, bias, weights, weights_dt, out, tokens, hidden, dt, s);
}

mb_status_t mb_bias_geglu_fwd(const void* in, const void* bias, void* out, int64_t tokens, int64_t hidden,
                              mb_dtype_t dt, hipStream_t s) {
  return glu_fwd_common(mb::kGEGLU, in, bias, nullptr, dt, out, tokens, hidden, dt, s);
}

namespace {
struct GluWs {
  size_t bias_off, bias_bytes, w_off, w_bytes, total;
};
GluWs glu_ws(int64_t tokens, int64_t hidden, mb_dtype_t dt, bool with_dbias, bool with_dw, int cus) {
  GluWs w{0, 0, 0, 0, 0};
  if (tokens == 0) return w;
  const mb::Tiling t = glu_bwd_tiling(tokens, hidden, dt, with_dbias, cus);
  w.bias_bytes = with_dbias ? col_partials_bytes(t, 2 * hidden) : 0;
  w.w_off = round_up(w.bias_bytes, 256);
  w.w_bytes = with_dw ? static_cast<size_t>(t.strips) * tokens * 4 : 0;
  w.total = w.w_bytes ? w.w_off + w.w_bytes : w.bias_bytes;
  return w;
}
}  // namespace

size_t mb_bias_glu_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dbias, int with_dweights) {
  if (!dt_ok(dt) || check_shape(tokens, hidden, dt, 2) != MB_OK) return 0;
  return glu_ws(tokens, hidden, dt, with_dbias != 0, with_dweights != 0, current_cus()).total;
}

static mb_status_t glu_bwd_common(int act, const void* g, const void* in, const void* bias, const void* weights,
                                  mb_dtype_t weights_dt, void* din, float* dbias, float* dweights, void* ws,
                                  size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  if (!dt_ok(dt)) return MB_ERR_DTYPE;
  if (weights && weights_dt != dt && weights_dt != MB_F32) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt, 2)) return st;
  const size_t gb = static_cast<size_t>(tokens) * hidden * esize(dt), ib = 2 * gb;
  const size_t bb = 2 * hidden * esize(dt);
  const size_t wb = weights ? static_cast<size_t>(tokens) * esize(weights_dt) : 0;
  if (!need(g, gb) || !need(in, ib) || !need(din, ib)) return MB_ERR_NULL;
  if (dweights && !weights) return MB_ERR_NULL;
  const int cus = stream_cus(s);
  const GluWs w = glu_ws(tokens, hidden, dt, dbias != nullptr, dweights != nullptr, cus);
  if (!aligned(g, 16) || !aligned(in, 16) || !aligned(din, 16) || !aligned(bias, 16) || !aligned(dbias, 4) ||
      !aligned(dweights, 4) || (weights && !aligned(weights, esize(weights_dt))) || (w.total && !aligned(ws, 16)))
    return MB_ERR_ALIGN;
  if (w.total && (!ws || ws_bytes < w.total)) return MB_ERR_WORKSPACE;
  const Buf wsb{w.total ? ws : nullptr, w.total};
  if (!aliasing_ok({{din, ib}, {dbias, dbias ? static_cast<size_t>(hidden) * 8 : 0},
                    {dweights, dweights ? static_cast<size_t>(tokens) * 4 : 0}, wsb},
                   {{g, gb}, {in, ib}, {bias, bias ? bb : 0}, {weights, wb}}, {{0, 1}}))
    return MB_ERR_ALIAS;
  if (tokens == 0) {
    if (!dbias) return MB_OK;
    if (hipError_t e = mb::launch_fill_zero(dbias, 2 * hidden, s)) return hip_status(e);
    return finish();
  }
  const mb::Tiling t = glu_bwd_tiling(tokens, hidden, dt, dbias != nullptr, cus);
  float* bp = dbias ? static_cast<float*>(ws) : nullptr;
  float* wp = dweights ? reinterpret_cast<float*>(static_cast<char*>(ws) + w.w_off) : nullptr;
  if (hipError_t e = mb::launch_glu_bwd(act, dt, g, in, bias, weights, weights ? weights_dt : dt, din, bp, wp, hidden,
                                        t, s))
    return hip_status(e);
  if (dbias && dweights) {
    if (hipError_t e = mb::launch_colsum2(mb::ColSum{bp, t.G, 2 * hidden, dbias},
                                          mb::ColSum{wp, t.strips, tokens, dweights}, s))
      return hip_status(e);
  } else if (dbias) {
    if (hipError_t e = reduce_columns(bp, t, 2 * hidden, dbias, s)) return hip_status(e);
  } else if (dweights) {
    if (hipError_t e = mb::launch_colsum(wp, t.strips, tokens, dweights, s)) return hip_status(e);
  }
  return finish();
}

mb_status_t mb_bias_swiglu_bwd(const void* g, const void* in, const void* bias, const void* weights,
                               mb_dtype_t weights_dt, void* din, float* dbias, float* dweights, void* ws,
                               size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  return glu_bwd_common(mb::kSwiGLU, g, in, bias, weights, weights_dt, din, dbias, dweights, ws, ws_bytes, tokens,
                        hidden, dt, s);
}

mb_status_t mb_bias_geglu_bwd(const void* g, const void* in, const void* bias, void* din, float* dbias, void* ws,
                              size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  return glu_bwd_common(mb::kGEGLU, g, in, bias, nullptr, dt, din, dbias, nullptr, ws, ws_bytes, tokens, hidden, dt,
                        s);
}

// ------------------------------------------------------------------ weighted squared ReLU

mb_status_t mb_weighted_squared_relu_fwd(const void* x, const void* weights, mb_dtype_t weights_dt, void* out,
                                         int64_t tokens, int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  if (!dt_ok(dt) || (weights && !dt_ok(weights_dt))) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  const size_t tb = static_cast<size_t>(tokens) * hidden * esize(dt);
  const size_t wb = weights ? static_cast<size_t>(tokens) * esize(weights_dt) : 0;
  if (!need(x, tb) || !need(out, tb)) return MB_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 16) || (weights && !aligned(weights, esize(weights_dt)))) return MB_ERR_ALIGN;
  if (!aliasing_ok({{out, tb}}, {{x, tb}, {weights, wb}}, {{0, 0}})) return MB_ERR_ALIAS;
  if (tokens == 0) return MB_OK;
  const mb::Tiling t = mb::plan_tiling(tokens, nvec_of(hidden, dt), MB_SRELU_FWD_BLOCKS, stream_cus(s));
  if (hipError_t e = mb::launch_srelu_fwd(dt, weights_dt, x, weights, out, t, s)) return hip_status(e);
  return finish();
}

static mb::Tiling srelu_bwd_tiling(int64_t tokens, int64_t hidden, mb_dtype_t dt, int cus) {
  return mb::plan_tiling(tokens, nvec_of(hidden, dt), MB_SRELU_BWD_BLOCKS, cus);
}

static size_t srelu_bwd_ws(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dweights, int cus) {
  if (!with_dweights || !dt_ok(dt) || check_shape(tokens, hidden, dt) != MB_OK || tokens == 0) return 0;
  const mb::Tiling t = srelu_bwd_tiling(tokens, hidden, dt, cus);
  return static_cast<size_t>(t.strips) * tokens * 4;
}

size_t mb_weighted_squared_relu_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, int with_dweights) {
  return srelu_bwd_ws(tokens, hidden, dt, with_dweights, current_cus());
}

mb_status_t mb_weighted_squared_relu_bwd(const void* g, const void* x, const void* weights, mb_dtype_t weights_dt,
                                         void* dx, float* dweights, void* ws, size_t ws_bytes, int64_t tokens,
                                         int64_t hidden, mb_dtype_t dt, hipStream_t s) {
  if (!dt_ok(dt) || (weights && !dt_ok(weights_dt))) return MB_ERR_DTYPE;
  if (mb_status_t st = check_shape(tokens, hidden, dt)) return st;
  if (dweights && !weights) return MB_ERR_NULL;
  const size_t tb = static_cast<size_t>(tokens) * hidden * esize(dt);
  const size_t wb = weights ? static_cast<size_t>(tokens) * esize(weights_dt) : 0;
  if (!need(g, tb) || !need(x, tb) || !need(dx, tb)) return MB_ERR_NULL;
  if (!aligned(g, 16) || !aligned(x, 16) || !aligned(dx, 16) || (weights && !aligned(weights, esize(weights_dt))) ||
      !aligned(dweights, 4) || !aligned(ws, 16))
    return MB_ERR_ALIGN;
  const int cus = stream_cus(s);
  const size_t need_ws = dweights ? srelu_bwd_ws(tokens, hidden, dt, 1, cus) : 0;
  if (need_ws && (!ws || ws_bytes < need_ws)) return MB_ERR_WORKSPACE;
  if (!aliasing_ok({{dx, tb}, {dweights, dweights ? static_cast<size_t>(tokens) * 4 : 0}, {ws, need_ws}},
                   {{g, tb}, {x, tb}, {weights, wb}}, {{0, 0}, {0, 1}}))
    return MB_ERR_ALIAS;
  if (tokens == 0) return MB_OK;
  const mb::Tiling t = srelu_bwd_tiling(tokens, hidden, dt, cus);
  float* wpart = dweights ? static_cast<float*>(ws) : nullptr;
  if (hipError_t e = mb::launch_srelu_bwd(dt, weights_dt, g, x, weights, dx, wpart, t, s)) return hip_status(e);
  if (dweights)
    if (hipError_t e = mb::launch_colsum(wpart, t.strips, tokens, dweights, s)) return hip_status(e);
  return finish();
}

// ------------------------------------------------------------------ residual add + LayerNorm

static bool ln_dtypes_ok(mb_dtype_t dt, mb_dtype_t rdt) { return dt_ok(dt) && (rdt == dt || rdt == MB_F32); }

// Shape rule of the LayerNorm rows: whole vectors, a row-group shape that holds
// the row, sizes within the kernels' index math.
static mb_status_t ln_shape(int64_t T, int64_t H, mb_dtype_t dt, mb_dtype_t rdt, int cus, mb::LnPlan* plan) {
  if (T < 0 || H <= 0 || T > (int64_t{1} << 40) || H > (int64_t{1} << 20)) return MB_ERR_SHAPE;
  const int E = mb::ln_elems_per_vector(dt, rdt);
  if (H % E != 0) return MB_ERR_SHAPE;
  const int blocks = H / E >= 1024 ? MB_LN_BWD_BLOCKS_WIDE : MB_LN_BWD_BLOCKS;
  *plan = mb::plan_ln(T, H, dt, rdt, blocks, MB_LN_BWD_NV, cus);
  if (plan->shape < 0) return MB_ERR_SHAPE;
  return MB_OK;
}

static bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

mb_status_t mb_add_layer_norm_fwd(const void* x, const void* residual, mb_dtype_t residual_dt, const void* gamma,
                                  const void* beta, float eps, int zero_centered_gamma, void* h_out, void* y,
                                  float* mean, float* rstd, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                  hipStream_t s) {
  if (!ln_dtypes_ok(dt, residual_dt)) return MB_ERR_DTYPE;
  mb::LnPlan plan;
  const int cus = stream_cus(s);
  if (mb_status_t st = ln_shape(tokens, hidden, dt, residual_dt, cus, &plan)) return st;
  if (!eps_ok(eps)) return MB_ERR_PROB;
  const size_t n = static_cast<size_t>(tokens) * hidden;
  const size_t tb = n * esize(dt), rb = n * esize(residual_dt), hb = static_cast<size_t>(hidden) * esize(dt),
               sb = static_cast<size_t>(tokens) * 4;
  if (!gamma || !need(x, tb) || !need(residual, rb) || !need(y, tb)) return MB_ERR_NULL;
  if ((mean == nullptr) != (rstd == nullptr)) return MB_ERR_NULL;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gamma, 16) || !aligned(beta, 16) ||
      !aligned(h_out, 16) || !aligned(y, 16) || !aligned(mean, 4) || !aligned(rstd, 4))
    return MB_ERR_ALIGN;
  if (!aliasing_ok({{h_out, h_out ? tb : 0}, {y, tb}, {mean, mean ? sb : 0}, {rstd, rstd ? sb : 0}},
                   {{x, tb}, {residual, rb}, {gamma, hb}, {beta, beta ? hb : 0}}, {{0, 0}, {1, 0}, {0, 1}, {1, 1}}))
    return MB_ERR_ALIAS;
  if (tokens == 0) return MB_OK;
  mb::LnArgs a;
  a.dt = dt;
  a.rdt = residual_dt;
  a.T = tokens;
  a.H = hidden;
  a.eps = eps;
  a.gshift = zero_centered_gamma ? 1.0f : 0.0f;
  a.x = x;
  a.res = residual;
  a.gamma = gamma;
  a.beta = beta;
  a.hout = h_out;
  a.y = y;
  a.mean = mean;
  a.rstd = rstd;
  mb::LnPlan fp = mb::plan_ln(tokens, hidden, dt, residual_dt, MB_LN_FWD_BLOCKS, MB_LN_FWD_NV, cus);
  if (MB_LN_FWD_WIDE_HALF && mb::ln_plan_is(fp, 1024, 4)) {
    const mb::LnPlan half = mb::plan_ln(tokens, hidden, dt, residual_dt, MB_LN_FWD_BLOCKS, 8, cus);
    if (mb::ln_plan_is(half, 512, 8)) fp = half;
  }
  if (mb::ln_plan_is(fp, 1024, 8)) {
    // rows of more than 4096 vectors: 512 threads of 16 (the LDS-staged kernel
    // fits that in registers; 1024 threads of 8 would spill)
    const mb::LnPlan half = mb::plan_ln(tokens, hidden, dt, residual_dt, MB_LN_FWD_BLOCKS, 16, cus);
    if (mb::ln_plan_is(half, 512, 16)) fp = half;
  }
  if (fp.shape < 0) return MB_ERR_SHAPE;
  if (hipError_t e = mb::launch_ln_fwd(a, fp, s)) return hip_status(e);
  return finish();
}

// Workspace layout: for the wide-row backward, the row sums ([T][2] floats);
// then, with parameter gradients, partial rows of dgamma, of dbeta, and the
// chunk sums of each when there are more than 32 partial rows (256-byte
// aligned pieces).
struct LnWs {
  bool wide = false, block = false, team = false;
  mb::LnTeamPlan tp;
  int partial_rows = 0;
  size_t rows = 0, pg = 0, pb = 0, tg = 0, tb = 0, total = 0;
};
// team_ok: the team backward may be used (no output overwrites an input:
// its fix-up pass rereads whole rows of dy, h and dh_in)
static LnWs ln_ws_layout(int64_t T, int64_t H, mb_dtype_t dt, mb_dtype_t rdt, const mb::LnPlan& p, int cus,
                         bool params, bool team_ok) {
  LnWs w;
  w.team = team_ok && mb::ln_team_applies(H, dt, rdt);
  w.wide = mb::ln2_applies(H, dt, rdt) && !w.team;
  w.block = mb::ln_block_applies(H, dt, rdt);
  if (w.team) w.tp = mb::plan_ln_team(T, H, dt, rdt, cus, mb::ln_team_blocks_per_cu(dt, rdt));
  w.partial_rows = w.wide    ? mb::plan_ln2(T, H, dt, rdt, cus).G
                   : w.block ? mb::plan_ln_block(T, H, dt, rdt, cus).grid
                   : w.team  ? w.tp.teams
                             : p.partial_rows;
  // the wide rows' two row sums, or the team rows' exchange slots (one pair
  // of floats per row and member) and a flag per row
  const size_t rows = w.wide   ? round_up(static_cast<size_t>(T) * 8, 256)
                      : w.team ? round_up(static_cast<size_t>(T) * (w.tp.members * 8 + 4), 256)
                               : 0;
  const size_t part = params ? round_up(static_cast<size_t>(w.partial_rows) * H * 4, 256) : 0;
  const size_t tmp =
      params ? round_up(static_cast<size_t>(mb::colsum_tall_tmp_floats(w.partial_rows, H)) * 4, 256) : 0;
  w.rows = 0;
  w.pg = rows;
  w.pb = rows + part;
  w.tg = rows + 2 * part;
  w.tb = rows + 2 * part + tmp;
  w.total = rows + 2 * part + 2 * tmp;
  return w;
}

size_t mb_add_layer_norm_bwd_workspace(int64_t tokens, int64_t hidden, mb_dtype_t dt, mb_dtype_t residual_dt,
                                       int with_param_grads) {
  if (!ln_dtypes_ok(dt, residual_dt) || tokens <= 0) return 0;
  mb::LnPlan plan;
  const int cus = current_cus();
  if (ln_shape(tokens, hidden, dt, residual_dt, cus, &plan) != MB_OK) return 0;
  // enough for either backward of the widest rows (in place or not)
  return std::max(ln_ws_layout(tokens, hidden, dt, residual_dt, plan, cus, with_param_grads != 0, true).total,
                  ln_ws_layout(tokens, hidden, dt, residual_dt, plan, cus, with_param_grads != 0, false).total);
}

mb_status_t mb_add_layer_norm_bwd(const void* dy, const void* h, const void* gamma, const float* mean,
                                  const float* rstd, int zero_centered_gamma, const void* dh_in,
                                  mb_dtype_t residual_dt, void* dx, void* dresidual, float* dgamma, float* dbeta,
                                  void* ws, size_t ws_bytes, int64_t tokens, int64_t hidden, mb_dtype_t dt,
                                  hipStream_t s) {
  if (!ln_dtypes_ok(dt, residual_dt)) return MB_ERR_DTYPE;
  mb::LnPlan plan;
  const int cus = stream_cus(s);
  if (mb_status_t st = ln_shape(tokens, hidden, dt, residual_dt, cus, &plan)) return st;
  const size_t n = static_cast<size_t>(tokens) * hidden;
  const size_t tb = n * esize(dt), rb = n * esize(residual_dt), hb = static_cast<size_t>(hidden) * esize(dt),
               sb = static_cast<size_t>(tokens) * 4;
  if (!gamma || !need(dy, tb) || !need(h, tb) || !need(dx, tb) || !need(mean, sb) || !need(rstd, sb))
    return MB_ERR_NULL;
  if (!aligned(dy, 16) || !aligned(h, 16) || !aligned(gamma, 16) || !aligned(dh_in, 16) || !aligned(dx, 16) ||
      !aligned(dresidual, 16) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(dgamma, 16) ||
      !aligned(dbeta, 16) || !aligned(ws, 16))
    return MB_ERR_ALIGN;
  const bool params = dgamma || dbeta;
  const bool in_place = dx == dy || dx == h || (dresidual && (dresidual == dy || dresidual == h || dresidual == dh_in));
  const LnWs lay = ln_ws_layout(tokens, hidden, dt, residual_dt, plan, cus, params, !in_place);
  const size_t need_ws = tokens > 0 ? lay.total : 0;
  if (need_ws && (!ws || ws_bytes < need_ws)) return MB_ERR_WORKSPACE;
  const size_t pb4 = static_cast<size_t>(hidden) * 4;
  if (!aliasing_ok({{dx, tb}, {dresidual, dresidual ? rb : 0}, {dgamma, dgamma ? pb4 : 0},
                    {dbeta, dbeta ? pb4 : 0}, {ws, need_ws}},
                   {{dy, tb}, {h, tb}, {gamma, hb}, {mean, sb}, {rstd, sb}, {dh_in, dh_in ? rb : 0}},
                   {{0, 0}, {0, 1}, {1, 5}, {1, 0}, {1, 1}}))
    return MB_ERR_ALIAS;
  if (tokens == 0) {
    if (dgamma)
      if (hipError_t e = mb::launch_fill_zero(dgamma, hidden, s)) return hip_status(e);
    if (dbeta)
      if (hipError_t e = mb::launch_fill_zero(dbeta, hidden, s)) return hip_status(e);
    return dgamma || dbeta ? finish() : MB_OK;
  }
  mb::LnArgs a;
  a.dt = dt;
  a.rdt = residual_dt;
  a.T = tokens;
  a.H = hidden;
  a.gshift = zero_centered_gamma ? 1.0f : 0.0f;
  a.dy = dy;
  a.h = h;
  a.gamma = gamma;
  a.cmean = mean;
  a.crstd = rstd;
  a.dh_in = dh_in;
  a.dx = dx;
  a.dres = dresidual;
  char* w = static_cast<char*>(ws);
  if (params) {
    a.pg = reinterpret_cast<float*>(w + lay.pg);
    a.pb = reinterpret_cast<float*>(w + lay.pb);
  }
  if (lay.wide) {
    a.rowsums = reinterpret_cast<float*>(w + lay.rows);
    const mb::Ln2Plan p2 = mb::plan_ln2(tokens, hidden, dt, residual_dt, cus);
    if (hipError_t e = mb::launch_ln2_bwd(a, p2, s)) return hip_status(e);
  } else if (lay.block) {
    if (hipError_t e = mb::launch_ln_block_bwd(a, mb::plan_ln_block(tokens, hidden, dt, residual_dt, cus), s))
      return hip_status(e);
  } else if (lay.team) {
    a.rowsums = reinterpret_cast<float*>(w + lay.rows);
    if (hipError_t e = mb::launch_ln_team_bwd(a, lay.tp, s)) return hip_status(e);
  } else {
    if (hipError_t e = mb::launch_ln_bwd(a, plan, s)) return hip_status(e);
  }
  const int R = lay.partial_rows;
  float* tg = reinterpret_cast<float*>(w + lay.tg);
  float* tbeta = reinterpret_cast<float*>(w + lay.tb);
  if (dgamma && dbeta) {
    if (hipError_t e = mb::launch_colsum_tall2(a.pg, a.pb, R, hidden, tg, tbeta, dgamma, dbeta, s))
      return hip_status(e);
  } else if (dgamma) {
    if (hipError_t e = mb::launch_colsum_tall(a.pg, R, hidden, tg, dgamma, s)) return hip_status(e);
  } else if (dbeta) {
    if (hipError_t e = mb::launch_colsum_tall(a.pb, R, hidden, tbeta, dbeta, s)) return hip_status(e);
  }
  return finish();
}

void mb_set_layer_norm_team_wait(int polls) { mb::set_ln_team_spin_limit(polls); }

}  // extern "C"
