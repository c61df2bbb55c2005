// mb_launch.hpp -- host-side launch interface between the C ABI (mb_abi.cpp)
// and the kernels. Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mb_plan.hpp"

namespace mb {


// Bytes of the static device scratch that holds the bias gradient's partial
// rows for the entry point that allocates nothing (one copy per device).
#ifndef MB_NOALLOC_SCRATCH_BYTES
#define MB_NOALLOC_SCRATCH_BYTES (16u << 20)
#endif
// Device address of that scratch on the device of stream s; looked up once
// per device (thread-safe), never allocated.
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
// One column sum: out[c] = sum over r < R of in[r * C + c], r ascending (fp32).
struct ColSum {
  const float* in;
  int R;
  int64_t C;
  float* out;
};
// Two independent column sums (any shapes) in one launch.
hipError_t launch_colsum2(const ColSum& a, const ColSum& b, hipStream_t s);
// As launch_colsum for many partial rows: rows are first summed in ascending
// chunks of 32 into tmp ([ceil(R / 32), C]), then the chunk sums in order.
hipError_t launch_colsum_tall(const float* in, int R, int64_t C, float* tmp, float* out, hipStream_t s);
// Two such sums of the same shape in the same launches (in0 -> out0 through
// tmp0, in1 -> out1 through tmp1).
hipError_t launch_colsum_tall2(const float* in0, const float* in1, int R, int64_t C, float* tmp0, float* tmp1,
                               float* out0, float* out1, hipStream_t s);
// out[c] = sum over r < R of in[r * C + c], r ascending (fp32).
hipError_t launch_colsum(const float* in, int R, int64_t C, float* out, hipStream_t s);

// exact = false: tanh approximation; true: the erf form
hipError_t launch_gelu_fwd(int dt, bool exact, const void* y, const void* bias, void* out, const Tiling& t,
                           hipStream_t s);
// partials: [G, H] fp32 or nullptr (no bias gradient)
hipError_t launch_gelu_bwd(int dt, bool exact, const void* g, const void* y, const void* bias, void* dgrad,
                           float* partials, const Tiling& t, hipStream_t s);

struct DropoutArgs {
  // keep iff word >= theta, theta in [0, 2^32]: theta32 = theta and
  // drop_all = 0, or drop_all = 1 for theta = 2^32 (p = 1), so that the
  // kernels compare in 32 bits
  uint32_t theta32;
  uint32_t drop_all;
  float scale;     // survivor scale
  uint32_t k0, k1; // key = seed
  uint32_t o0, o1; // counter high words = offset
};
hipError_t launch_bda(int dt, int res_dt, bool train, const void* x, const void* bias,
                      const void* residual, void* out, int64_t H, const Tiling& t,
                      const DropoutArgs& d, hipStream_t s);
hipError_t launch_dropout_mask(uint8_t* bits, int64_t n, const DropoutArgs& d, hipStream_t s);
// dres (residual dtype res_dt) and partials ([G, H]) are optional
hipError_t launch_bda_bwd(int dt, int res_dt, const void* g, void* dx, void* dres, float* partials, int64_t H,
                          const Tiling& t, const DropoutArgs& d, hipStream_t s);

enum Act { kSwiGLU = 0, kGEGLU = 1 };
hipError_t launch_glu_fwd(int act, int dt, const void* in, const void* bias, const void* w,
                          int w_dt, void* out, int64_t H, const Tiling& t, hipStream_t s);
// bias_partials: [G, 2H] or nullptr; w_partials: [strips, T] or nullptr
hipError_t launch_glu_bwd(int act, int dt, const void* g, const void* in, const void* bias,
                          const void* w, int w_dt, void* din, float* bias_partials,
                          float* w_partials, int64_t H, const Tiling& t, hipStream_t s);

// ---- weighted squared ReLU. w: per-token weights of dtype wdt, or nullptr;
// wpart: [strips, T] fp32 row partials of the weights gradient, or nullptr.
hipError_t launch_srelu_fwd(int dt, int wdt, const void* x, const void* w, void* out, const Tiling& t,
                            hipStream_t s);
hipError_t launch_srelu_bwd(int dt, int wdt, const void* g, const void* x, const void* w, void* dx, float* wpart,
                            const Tiling& t, hipStream_t s);

// ---- residual add + LayerNorm
struct LnArgs {
  int dt = 0, rdt = 0;  // activation and residual dtypes (DT values)
  int64_t T = 0, H = 0;
  float eps = 0.0f, gshift = 0.0f;  // gshift: 1 for a zero-centred gamma, else 0
  // forward
  const void* x = nullptr;
  const void* res = nullptr;
  const void* gamma = nullptr;
  const void* beta = nullptr;  // nullable
  void* hout = nullptr;        // nullable
  void* y = nullptr;
  float* mean = nullptr;  // nullable (with rstd)
  float* rstd = nullptr;
  // backward
  const void* dy = nullptr;
  const void* h = nullptr;
  const float* cmean = nullptr;
  const float* crstd = nullptr;
  const void* dh_in = nullptr;  // nullable
  void* dx = nullptr;
  void* dres = nullptr;  // nullable
  float* pg = nullptr;   // partial rows of dgamma / dbeta [partial_rows, H]; nullable
  float* pb = nullptr;
  float* rowsums = nullptr;  // wide-row backward: [T][2] (mean_j a, mean_j a xhat) per row
};
hipError_t launch_ln_fwd(const LnArgs& a, const LnPlan& p, hipStream_t s);
hipError_t launch_ln_bwd(const LnArgs& a, const LnPlan& p, hipStream_t s);
// backward of wide rows (plan_ln2): needs a.rowsums, and a.pg / a.pb
// ([p.G, H]) for the parameter gradients
hipError_t launch_ln2_bwd(const LnArgs& a, const Ln2Plan& p, hipStream_t s);
// backward of rows of 1025-2048 vectors (plan_ln_block): a.pg / a.pb
// ([p.grid, H]) for the parameter gradients
hipError_t launch_ln_block_bwd(const LnArgs& a, const LnBlockPlan& p, hipStream_t s);
// backward of rows split over teams of blocks (plan_ln_team): a.rowsums holds
// the exchange slots ([T][p.members] pairs of floats) and then T row flags,
// both set by the launch itself; a.pg / a.pb ([p.teams, H]) the parameter
// gradients
hipError_t launch_ln_team_bwd(const LnArgs& a, const LnTeamPlan& p, hipStream_t s);
// blocks of the team kernel one compute unit holds (dtype pair dt, rdt); 1
// when the device cannot be asked
int ln_team_blocks_per_cu(int dt, int rdt);
// polls of a team's wait before a block recomputes a partner's terms
// (negative: the default); later launches use it
void set_ln_team_spin_limit(int polls);

}  // namespace mb
