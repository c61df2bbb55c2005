/*
 * oracle32.c -- the oracle's formulas evaluated in IEEE binary32 ("oracle32").
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c beside it (linked into the same
 * liboracle.so): only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it. It shares nothing with the HIP library.
 *
 * What it is for: the plain fp32 scalar evaluation of every op, reported as a
 * secondary statistic next to the parity reference (oracle.c, fp64) and timed
 * as the fp32 CPU baseline. It is NOT the parity reference: the literal tanh
 * GeLU derivative cancels in float once tanh(u) rounds to -1, and float row
 * sums lose digits that the fp64 oracle keeps.
 *
 * Evaluation rules:
 *   - inputs decode exactly to float (bf16 and fp16 are subsets of binary32);
 *   - every formula is evaluated in float, in the order the Megatron-LM
 *     fusions walkthrough (wmrh.cn/news/51426) prints it where it prints one
 *     ([fusions §4.2]: x * 0.5 * (1 + tanh(0.79788456 x (1 + 0.044715 x x)))
 *     and x * 0.5 * (1 + erf(x * 0.70710678))), else in the order oracle.c
 *     writes the formula; no FMA contraction (-ffp-contract=off), the C
 *     library's float functions (tanhf, erff, expf, sqrtf);
 *   - each output is rounded once from its float value to the output dtype;
 *   - bias, weight and parameter gradients are float sums in row (column)
 *     order, returned unrounded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* format helpers and the dropout definition, from oracle.c */
uint16_t orc_round_bf16(double v);
uint16_t orc_round_f16(double v);
double orc_bf16_to_double(uint16_t h);
double orc_f16_to_double(uint16_t h);
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint64_t orc_drop_threshold(float p);
float orc_keep_scale(float p);

enum { O32_F32 = 0, O32_F16 = 1, O32_BF16 = 2 };
enum { O32_SWIGLU = 0, O32_GEGLU = 1 };
enum { O32_OK = 0, O32_BAD = 1 };

static int dt_ok(int dt) { return dt == O32_F32 || dt == O32_F16 || dt == O32_BF16; }

static float ld(int dt, const void* p, int64_t i) {
  switch (dt) {
    case O32_F32: return ((const float*)p)[i];
    case O32_F16: return (float)orc_f16_to_double(((const uint16_t*)p)[i]);
    default: return (float)orc_bf16_to_double(((const uint16_t*)p)[i]);
  }
}

/* round the float v once to dt (float -> double is exact, then nearest-even) */
static void st(int dt, void* p, int64_t i, float v) {
  switch (dt) {
    case O32_F32: ((float*)p)[i] = v; break;
    case O32_F16: ((uint16_t*)p)[i] = orc_round_f16((double)v); break;
    default: ((uint16_t*)p)[i] = orc_round_bf16((double)v); break;
  }
}

/* the value a dt tensor holds after storing v */
static float as_dt(int dt, float v) {
  switch (dt) {
    case O32_F32: return v;
    case O32_F16: return (float)orc_f16_to_double(orc_round_f16((double)v));
    default: return (float)orc_bf16_to_double(orc_round_bf16((double)v));
  }
}

static int kept(uint64_t gi, uint64_t theta, uint64_t seed, uint64_t offset) {
  const uint64_t block = gi >> 2;
  const uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (uint64_t)out[gi & 3] >= theta;
}

/* ---------------------------------------------------------------- activations [fusions §4.2] */

static float gelu_tanh(float x) { return x * 0.5f * (1.0f + tanhf(0.79788456f * x * (1.0f + 0.044715f * x * x))); }

/* the derivative with t = tanh(u) in its literal form (cancels for u << 0) */
static float gelu_tanh_grad(float x) {
  const float t = tanhf(0.79788456f * x * (1.0f + 0.044715f * x * x));
  return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * (0.79788456f + 0.1070322243f * x * x);
}

static float gelu_erf(float x) { return x * 0.5f * (1.0f + erff(x * 0.70710678f)); }

static float gelu_erf_grad(float x) { return 0.5f * (1.0f + erff(x * 0.70710678f)) + x * 0.3989423f * expf(-0.5f * x * x); }

static float sigmoid(float a) { return 1.0f / (1.0f + expf(-a)); }
static float silu(float a) { return a * sigmoid(a); }
static float silu_grad(float a) {
  const float s = sigmoid(a);
  return s * (1.0f + a * (1.0f - s));
}

/* ---------------------------------------------------------------- fused ops */

int orc32_bias_gelu_fwd(int dt, int exact, const void* y, const void* bias, void* out, int64_t T, int64_t H) {
  if (!dt_ok(dt) || T < 0 || H <= 0) return O32_BAD;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      const float x = ld(dt, y, i) + (bias ? ld(dt, bias, j) : 0.0f);
      st(dt, out, i, exact ? gelu_erf(x) : gelu_tanh(x));
    }
  return O32_OK;
}

int orc32_bias_gelu_bwd(int dt, int exact, const void* g, const void* y, const void* bias, void* dgrad,
                        float* dbias, int64_t T, int64_t H) {
  if (!dt_ok(dt) || T < 0 || H <= 0) return O32_BAD;
  if (dbias)
    for (int64_t j = 0; j < H; ++j) dbias[j] = 0.0f;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      const float x = ld(dt, y, i) + (bias ? ld(dt, bias, j) : 0.0f);
      const float v = ld(dt, g, i) * (exact ? gelu_erf_grad(x) : gelu_tanh_grad(x));
      st(dt, dgrad, i, v);
      if (dbias) dbias[j] += v;
    }
  return O32_OK;
}

/* [fusions §3.2]: z = x + bias, then * s on kept elements, then + r' */
int orc32_bias_dropout_add(int dt, const void* x, const void* bias, const void* res, int res_dt, void* out,
                           int64_t T, int64_t H, int train, float p, uint64_t seed, uint64_t offset, int64_t row0) {
  if (!dt_ok(dt) || !dt_ok(res_dt) || T < 0 || H <= 0 || row0 < 0) return O32_BAD;
  if (train && (isnan(p) || p < 0.0f || p > 1.0f)) return O32_BAD;
  const uint64_t theta = train ? orc_drop_threshold(p) : 0;
  const float s = train ? orc_keep_scale(p) : 1.0f;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      float r = ld(res_dt, res, i);
      if (res_dt != dt) r = as_dt(dt, r);
      const float z = ld(dt, x, i) + (bias ? ld(dt, bias, j) : 0.0f);
      float v;
      if (train) {
        const uint64_t gi = (uint64_t)(row0 + t) * (uint64_t)H + (uint64_t)j;
        const float d = kept(gi, theta, seed, offset) ? z * s : 0.0f;
        v = r + d;
      } else {
        v = r + z;
      }
      st(dt, out, i, v);
    }
  return O32_OK;
}

int orc32_bias_dropout_add_bwd(int dt, const void* g, int res_dt, void* dx, void* dres, float* dbias, int64_t T,
                               int64_t H, float p, uint64_t seed, uint64_t offset, int64_t row0) {
  if (!dt_ok(dt) || !dt_ok(res_dt) || T < 0 || H <= 0 || row0 < 0 || isnan(p) || p < 0.0f || p > 1.0f)
    return O32_BAD;
  const uint64_t theta = orc_drop_threshold(p);
  const float s = orc_keep_scale(p);
  if (dbias)
    for (int64_t j = 0; j < H; ++j) dbias[j] = 0.0f;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      const float gv = ld(dt, g, i);
      const uint64_t gi = (uint64_t)(row0 + t) * (uint64_t)H + (uint64_t)j;
      const float v = kept(gi, theta, seed, offset) ? gv * s : 0.0f;
      st(dt, dx, i, v);
      if (dres) st(res_dt, dres, i, gv);
      if (dbias) dbias[j] += v;
    }
  return O32_OK;
}

static float act_fwd(int act, float a) { return act == O32_SWIGLU ? silu(a) : gelu_tanh(a); }
static float act_grad(int act, float a) { return act == O32_SWIGLU ? silu_grad(a) : gelu_tanh_grad(a); }

/* in [T, 2H]: a = in[t, j] + bias[j], b = in[t, H + j] + bias[H + j];
 * out = act(a) * b (* w[t] when weighted) */
int orc32_bias_glu_fwd(int act, int dt, const void* in, const void* bias, const void* w, int w_dt, void* out,
                       int64_t T, int64_t H) {
  if ((act != O32_SWIGLU && act != O32_GEGLU) || !dt_ok(dt) || (w && !dt_ok(w_dt)) || T < 0 || H <= 0)
    return O32_BAD;
  for (int64_t t = 0; t < T; ++t) {
    const float wt = w ? ld(w_dt, w, t) : 1.0f;
    for (int64_t j = 0; j < H; ++j) {
      const float a = ld(dt, in, t * 2 * H + j) + (bias ? ld(dt, bias, j) : 0.0f);
      const float b = ld(dt, in, t * 2 * H + H + j) + (bias ? ld(dt, bias, H + j) : 0.0f);
      float v = act_fwd(act, a) * b;
      if (w) v = v * wt;
      st(dt, out, t * H + j, v);
    }
  }
  return O32_OK;
}

int orc32_bias_glu_bwd(int act, int dt, const void* g, const void* in, const void* bias, const void* w, int w_dt,
                       void* din, float* dbias, float* dw, int64_t T, int64_t H) {
  if ((act != O32_SWIGLU && act != O32_GEGLU) || !dt_ok(dt) || (w && !dt_ok(w_dt)) || T < 0 || H <= 0)
    return O32_BAD;
  if (dbias)
    for (int64_t c = 0; c < 2 * H; ++c) dbias[c] = 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    const float wt = w ? ld(w_dt, w, t) : 1.0f;
    float acc = 0.0f;
    for (int64_t j = 0; j < H; ++j) {
      const float a = ld(dt, in, t * 2 * H + j) + (bias ? ld(dt, bias, j) : 0.0f);
      const float b = ld(dt, in, t * 2 * H + H + j) + (bias ? ld(dt, bias, H + j) : 0.0f);
      const float gv = ld(dt, g, t * H + j);
      const float fa = act_fwd(act, a);
      const float da = gv * wt * b * act_grad(act, a);
      const float db = gv * wt * fa;
      st(dt, din, t * 2 * H + j, da);
      st(dt, din, t * 2 * H + H + j, db);
      if (dbias) {
        dbias[j] += da;
        dbias[H + j] += db;
      }
      acc += gv * fa * b;
    }
    if (dw && w) dw[t] = acc;
  }
  return O32_OK;
}

/* [fusions §5] behind a residual add: h = x + r' (rounded to dt); mean and the
 * biased variance of the rounded h in two float passes; y = xhat gamma' + beta */
int orc32_add_layer_norm_fwd(int dt, const void* x, const void* res, int res_dt, const void* gamma,
                             const void* beta, int zc, float eps, void* h_out, void* y, float* mean_out,
                             float* rstd_out, int64_t T, int64_t H) {
  if (!dt_ok(dt) || !dt_ok(res_dt) || !gamma || T < 0 || H <= 0 || isnan(eps) || eps < 0.0f) return O32_BAD;
  float* h = (float*)malloc(sizeof(float) * (size_t)H);
  if (!h) return O32_BAD;
  const float fh = (float)H;
  for (int64_t t = 0; t < T; ++t) {
    float sum = 0.0f;
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      float r = ld(res_dt, res, i);
      if (res_dt != dt) r = as_dt(dt, r);
      h[j] = as_dt(dt, ld(dt, x, i) + r);
      if (h_out) st(dt, h_out, i, h[j]);
      sum += h[j];
    }
    const float mean = sum / fh;
    float var = 0.0f;
    for (int64_t j = 0; j < H; ++j) var += (h[j] - mean) * (h[j] - mean);
    var = var / fh;
    const float rstd = 1.0f / sqrtf(var + eps);
    for (int64_t j = 0; j < H; ++j) {
      const float gj = ld(dt, gamma, j) + (zc ? 1.0f : 0.0f);
      const float bj = beta ? ld(dt, beta, j) : 0.0f;
      st(dt, y, t * H + j, (h[j] - mean) * rstd * gj + bj);
    }
    if (mean_out) mean_out[t] = mean;
    if (rstd_out) rstd_out[t] = rstd;
  }
  free(h);
  return O32_OK;
}

/* dh = rstd (a - mean_j a - xhat mean_j (a xhat)) + dh_in with a = dy gamma',
 * the statistics recomputed from h in float as the forward computes them */
int orc32_add_layer_norm_bwd(int dt, const void* dy, const void* h_in, const void* gamma, int zc, float eps,
                             const void* dh_in, int res_dt, void* dx, void* dres, float* dgamma, float* dbeta,
                             int64_t T, int64_t H) {
  if (!dt_ok(dt) || !dt_ok(res_dt) || !gamma || T < 0 || H <= 0 || isnan(eps) || eps < 0.0f) return O32_BAD;
  float* h = (float*)malloc(sizeof(float) * (size_t)H);
  float* a = (float*)malloc(sizeof(float) * (size_t)H);
  if (!h || !a) {
    free(h);
    free(a);
    return O32_BAD;
  }
  if (dgamma)
    for (int64_t j = 0; j < H; ++j) dgamma[j] = 0.0f;
  if (dbeta)
    for (int64_t j = 0; j < H; ++j) dbeta[j] = 0.0f;
  const float fh = (float)H;
  for (int64_t t = 0; t < T; ++t) {
    float sum = 0.0f;
    for (int64_t j = 0; j < H; ++j) {
      h[j] = ld(dt, h_in, t * H + j);
      sum += h[j];
    }
    const float mean = sum / fh;
    float var = 0.0f;
    for (int64_t j = 0; j < H; ++j) var += (h[j] - mean) * (h[j] - mean);
    var = var / fh;
    const float rstd = 1.0f / sqrtf(var + eps);
    float sa = 0.0f, sax = 0.0f;
    for (int64_t j = 0; j < H; ++j) {
      const float xhat = (h[j] - mean) * rstd;
      const float dyv = ld(dt, dy, t * H + j);
      a[j] = dyv * (ld(dt, gamma, j) + (zc ? 1.0f : 0.0f));
      sa += a[j];
      sax += a[j] * xhat;
      if (dgamma) dgamma[j] += dyv * xhat;
      if (dbeta) dbeta[j] += dyv;
    }
    const float ma = sa / fh, mx = sax / fh;
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      const float xhat = (h[j] - mean) * rstd;
      const float up = dh_in ? ld(res_dt, dh_in, i) : 0.0f;
      const float v = rstd * (a[j] - ma - xhat * mx) + up;
      st(dt, dx, i, v);
      if (dres) st(res_dt, dres, i, v);
    }
  }
  free(h);
  free(a);
  return O32_OK;
}

/* out = relu(x)^2 * w[t]; dx = g * w[t] * 2 relu(x); dw[t] = sum_j g relu(x)^2 */
static float relu(float x) { return x > 0.0f ? x : (isnan(x) ? x : 0.0f); }

int orc32_weighted_squared_relu_fwd(int dt, const void* x, const void* w, int w_dt, void* out, int64_t T,
                                    int64_t H) {
  if (!dt_ok(dt) || (w && !dt_ok(w_dt)) || T < 0 || H <= 0) return O32_BAD;
  for (int64_t t = 0; t < T; ++t) {
    const float wt = w ? ld(w_dt, w, t) : 1.0f;
    for (int64_t j = 0; j < H; ++j) {
      const float r = relu(ld(dt, x, t * H + j));
      st(dt, out, t * H + j, r * r * wt);
    }
  }
  return O32_OK;
}

int orc32_weighted_squared_relu_bwd(int dt, const void* g, const void* x, const void* w, int w_dt, void* dx,
                                    float* dw, int64_t T, int64_t H) {
  if (!dt_ok(dt) || (w && !dt_ok(w_dt)) || T < 0 || H <= 0 || (dw && !w)) return O32_BAD;
  for (int64_t t = 0; t < T; ++t) {
    const float wt = w ? ld(w_dt, w, t) : 1.0f;
    float acc = 0.0f;
    for (int64_t j = 0; j < H; ++j) {
      const int64_t i = t * H + j;
      const float r = relu(ld(dt, x, i));
      const float gv = ld(dt, g, i);
      st(dt, dx, i, gv * wt * 2.0f * r);
      acc += gv * r * r;
    }
    if (dw) dw[t] = acc;
  }
  return O32_OK;
}
