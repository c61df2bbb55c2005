/*
 * oracle.c -- plain scalar CPU oracle for the fused Transformer epilogues.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct
 * reference that the GPU kernels are checked against. It shares no code,
 * header, table or constant with the HIP library. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it.
 *
 * Source of the method: the wmrh.cn article walking through Megatron-LM's
 * megatron/core/fusions package (wmrh.cn/news/51426), cited below as
 * [fusions §N] for its section N:
 *   §3.2  bias + dropout + residual add, residual cast to x's dtype
 *   §3.3  separate train and inference functions
 *   §4.2  exact and tanh-approximated GeLU with their literal constants,
 *         bias folded into the forward and backward
 *   §4.3  the bias gradient is the per-element gradient reduced over tokens
 *   §2    bias-SwiGLU / bias-GEGLU gated activations, weighted SwiGLU
 *   §9    weighted SwiGLU equals unweighted SwiGLU times the weights
 *   §5    the fused LayerNorm (eps, zero-centred gamma), here behind a
 *         residual add
 *   §2/§8 the MoE weighted squared ReLU (named only)
 *
 * Evaluation rules (readings where the pages are silent):
 *   - every input is decoded exactly to double; every formula is evaluated in
 *     IEEE double (compile with -ffp-contract=off, no fast-math);
 *   - each output is rounded ONCE, round-to-nearest-even, to the output
 *     dtype (fp32, fp16 or bf16); NaN stays a quiet NaN;
 *   - 1 + tanh(u) and 1 - tanh(u)^2 are evaluated through the exact
 *     identities 1 + tanh(u) = 2 / (1 + exp(-2u)) and
 *     1 - tanh(u)^2 = 1 / cosh(u)^2, because the literal forms cancel to
 *     zero in double once tanh(u) rounds to -1 (u < -18.7);
 *   - gated ops split the [T, 2H] input row into a = columns [0, H) (the
 *     half that goes through the activation) and b = columns [H, 2H);
 *   - gradients of the bias and of the per-token weights are accumulated in
 *     double in row/column order and returned unrounded.
 *
 * Dropout mask: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11).  Element i = (row0 + t) * H + j of a
 * [T, H] tensor uses 32-bit word (i mod 4) of the block generated with
 *   counter = (lo32(i/4), hi32(i/4), lo32(offset), hi32(offset)),
 *   key     = (lo32(seed), hi32(seed)).
 * It is kept iff word >= floor(p * 2^32) (computed in double from the float
 * p, capped at 2^32), and a kept value is scaled by the float
 * s = (float)(1 / (1 - p)).
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

/* ORC_F64 (double storage, no rounding) exists only so that tests can take
 * finite differences through the fused ops themselves. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_F64 = 3 };
enum { ORC_SWIGLU = 0, ORC_GEGLU = 1 };
enum { ORC_OK = 0, ORC_BAD = 1 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static double f32_bits_to_double(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

static uint32_t float_to_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* bfloat16: 1 sign, 8 exponent, 7 fraction bits; the upper half of a float. */
double orc_bf16_to_double(uint16_t h) { return f32_bits_to_double((uint32_t)h << 16); }

/* IEEE binary16: 1 sign, 5 exponent, 10 fraction bits, bias 15. */
double orc_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = (m == 0) ? INFINITY : NAN;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

/* Round a finite, non-zero magnitude a to a binary format with `prec`
 * significant bits and minimum normal exponent `emin`, nearest-even.
 * Returns the rounded magnitude (possibly 2^(emax+1), i.e. an overflow). */
static double round_mag(double a, int prec, int emin) {
  int e;
  frexp(a, &e);            /* a = m * 2^e with m in [0.5, 1): floor(log2 a) = e-1 */
  int ex = e - 1;
  if (ex < emin) ex = emin; /* subnormal range: fixed quantum */
  double q = ldexp(1.0, ex - (prec - 1));
  return nearbyint(a / q) * q; /* a/q is exact; nearbyint is ties-to-even */
}

uint16_t orc_round_bf16(double v) {
  if (isnan(v)) return (uint16_t)(0x7fc0 | (signbit(v) ? 0x8000 : 0));
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return s;
  if (isinf(a)) return (uint16_t)(s | 0x7f80);
  double r = round_mag(a, 8, -126);
  if (r >= 0x1p128) return (uint16_t)(s | 0x7f80);
  /* r is a bf16 value, hence exactly a float whose low 16 bits are zero */
  return (uint16_t)(s | (float_to_bits((float)r) >> 16));
}

uint16_t orc_round_f16(double v) {
  if (isnan(v)) return (uint16_t)(0x7e00 | (signbit(v) ? 0x8000 : 0));
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return s;
  if (isinf(a)) return (uint16_t)(s | 0x7c00);
  double r = round_mag(a, 11, -14);
  if (r >= 65536.0) return (uint16_t)(s | 0x7c00);
  if (r < 0x1p-14) return (uint16_t)(s | (uint16_t)(r * 0x1p24)); /* subnormal */
  int e;
  frexp(r, &e);
  int ex = e - 1; /* r in [2^ex, 2^(ex+1)) */
  uint16_t mant = (uint16_t)(ldexp(r, 10 - ex) - 1024.0);
  return (uint16_t)(s | ((ex + 15) << 10) | mant);
}

/* double -> float conversion in C is IEEE round-to-nearest-even. */
float orc_round_f32(double v) { return (float)v; }

static double load_elem(int dt, const void* p, int64_t i) {
  switch (dt) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_F16: return orc_f16_to_double(((const uint16_t*)p)[i]);
    case ORC_F64: return ((const double*)p)[i];
    default: return orc_bf16_to_double(((const uint16_t*)p)[i]);
  }
}

static void store_elem(int dt, void* p, int64_t i, double v) {
  switch (dt) {
    case ORC_F32: ((float*)p)[i] = orc_round_f32(v); break;
    case ORC_F16: ((uint16_t*)p)[i] = orc_round_f16(v); break;
    case ORC_F64: ((double*)p)[i] = v; break;
    default: ((uint16_t*)p)[i] = orc_round_bf16(v); break;
  }
}

/* Round v to dtype dt and decode it back: the value a dt tensor holds. */
static double to_dtype(int dt, double v) {
  switch (dt) {
    case ORC_F32: return (double)orc_round_f32(v);
    case ORC_F16: return orc_f16_to_double(orc_round_f16(v));
    case ORC_F64: return v;
    default: return orc_bf16_to_double(orc_round_bf16(v));
  }
}

double orc_decode(int dt, const void* p, int64_t i) { return load_elem(dt, p, i); }

static int dtype_ok(int dt) { return dt == ORC_F32 || dt == ORC_F16 || dt == ORC_BF16 || dt == ORC_F64; }

/* ------------------------------------------------------------------------ */
/* Activations [fusions §4.2]                                                */
/* ------------------------------------------------------------------------ */

/* Constants exactly as printed in [fusions §4.2]. */
#define K_TANH 0.79788456      /* sqrt(2/pi) */
#define K_CUBIC 0.044715
#define K_TANH_GRAD 0.1070322243 /* sqrt(2/pi) * 3 * 0.044715 */
#define K_ERF 0.70710678       /* 1/sqrt(2) */
#define K_PDF 0.3989423        /* 1/sqrt(2*pi) */

/* tanh argument of the approximation: u(z) = 0.79788456 z (1 + 0.044715 z^2) */
static double tanh_arg(double z) { return K_TANH * z * (1.0 + K_CUBIC * z * z); }

/* 1 + tanh(u), written as 2 / (1 + exp(-2u)) */
static double one_plus_tanh(double u) { return 2.0 / (1.0 + exp(-2.0 * u)); }

/* 1 - tanh(u)^2, written as sech(u)^2 */
static double one_minus_tanh2(double u) {
  double c = cosh(u);
  return 1.0 / (c * c);
}

/* gelu_tanh(z) = 0.5 z (1 + tanh(u(z))) */
double orc_gelu_tanh(double z) { return 0.5 * z * one_plus_tanh(tanh_arg(z)); }

/* d/dz gelu_tanh = 0.5 (1 + t) + 0.5 z (1 - t^2)(0.79788456 + 0.1070322243 z^2),
 * t = tanh(u(z))  [fusions §4.2, backward with the printed constant] */
double orc_gelu_tanh_grad(double z) {
  double u = tanh_arg(z);
  return 0.5 * one_plus_tanh(u) + 0.5 * z * one_minus_tanh2(u) * (K_TANH + K_TANH_GRAD * z * z);
}

/* Magnitude of the larger of the two summands of orc_gelu_tanh_grad. */
static double gelu_tanh_grad_mag(double z) {
  double u = tanh_arg(z);
  double t1 = fabs(0.5 * one_plus_tanh(u));
  double t2 = fabs(0.5 * z * one_minus_tanh2(u) * (K_TANH + K_TANH_GRAD * z * z));
  return t1 > t2 ? t1 : t2;
}

/* exact GeLU: 0.5 z (1 + erf(0.70710678 z)); 1 + erf(x) written as erfc(-x) */
double orc_gelu_erf(double z) { return 0.5 * z * erfc(-K_ERF * z); }

/* d/dz gelu_erf = 0.5 (1 + erf(0.70710678 z)) + z 0.3989423 exp(-z^2/2) */
double orc_gelu_erf_grad(double z) { return 0.5 * erfc(-K_ERF * z) + z * K_PDF * exp(-0.5 * z * z); }

/* logistic sigmoid */
static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* silu(a) = a * sigmoid(a) */
double orc_silu(double a) { return a * sigmoid(a); }

/* silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))), with 1 - sigmoid(a) = sigmoid(-a) */
double orc_silu_grad(double a) { return sigmoid(a) * (1.0 + a * sigmoid(-a)); }

static double silu_grad_mag(double a) {
  double x = fabs(a * sigmoid(-a));
  return sigmoid(a) * (x > 1.0 ? x : 1.0);
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (SC'11)                                                     */
/* ------------------------------------------------------------------------ */

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* One Philox4x32 round: two 32x32->64 products, then the S-box permutation
 * (c0, c1, c2, c3) <- (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)). */
static void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

/* Ten rounds; the key is bumped by the Weyl constants between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k[0] += PHILOX_W0;
      k[1] += PHILOX_W1;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

/* The 32-bit random word of global element index i. */
static uint32_t element_word(uint64_t i, uint64_t seed, uint64_t offset) {
  uint64_t block = i >> 2;
  uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[i & 3];
}

/* floor(p * 2^32) in double from the float p, capped at 2^32 */
static uint64_t drop_threshold(float p) {
  double t = floor((double)p * 4294967296.0);
  if (t >= 4294967296.0) return (uint64_t)1 << 32;
  if (t <= 0.0) return 0;
  return (uint64_t)t;
}

uint64_t orc_drop_threshold(float p) { return drop_threshold(p); }

/* survivor scale, a float, as the kernel receives it */
float orc_keep_scale(float p) { return p < 1.0f ? (float)(1.0 / (1.0 - (double)p)) : 0.0f; }

static int element_kept(uint64_t i, uint64_t theta, uint64_t seed, uint64_t offset) {
  return (uint64_t)element_word(i, seed, offset) >= theta;
}

static int prob_ok(float p) { return !isnan(p) && p >= 0.0f && p <= 1.0f; }

/* Keep bits of a [T, H] tensor, LSB-first by element index t*H + j
 * (global index (row0 + t)*H + j for the Philox counter). */
int orc_dropout_mask(uint8_t* bits, int64_t T, int64_t H, float p, uint64_t seed, uint64_t offset,
                     int64_t row0) {
  if (T < 0 || H <= 0 || row0 < 0 || !prob_ok(p)) return ORC_BAD;
  uint64_t theta = drop_threshold(p);
  int64_t n = T * H;
  memset(bits, 0, (size_t)((n + 7) / 8));
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t local = t * H + j;
      uint64_t gi = (uint64_t)(row0 + t) * (uint64_t)H + (uint64_t)j;
      if (element_kept(gi, theta, seed, offset)) bits[local >> 3] |= (uint8_t)(1u << (local & 7));
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Fused ops                                                                 */
/* ------------------------------------------------------------------------ */

/* Bias-GeLU forward [fusions §4.2]: out = gelu_tanh(y + bias).
 * bias may be NULL (zero). out64 (nullable) receives the unrounded value. */
int orc_bias_gelu_fwd(int dt, const void* y, const void* bias, void* out, double* out64, int64_t T,
                      int64_t H) {
  if (!dtype_ok(dt) || T < 0 || H <= 0) return ORC_BAD;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double z = load_elem(dt, y, i) + (bias ? load_elem(dt, bias, j) : 0.0);
      double v = orc_gelu_tanh(z);
      store_elem(dt, out, i, v);
      if (out64) out64[i] = v;
    }
  return ORC_OK;
}

/* Bias-GeLU backward [fusions §4.2, §4.3]: dgrad = g * gelu_tanh'(y + bias),
 * dbias[j] = sum over t of the unrounded dgrad[t, j] (double, nullable).
 * mag (nullable): |g| times the larger summand of gelu_tanh', the scale of
 * the cancellation in the derivative. */
int orc_bias_gelu_bwd(int dt, const void* g, const void* y, const void* bias, void* dgrad,
                      double* dgrad64, double* mag, double* dbias, int64_t T, int64_t H) {
  if (!dtype_ok(dt) || T < 0 || H <= 0) return ORC_BAD;
  if (dbias)
    for (int64_t j = 0; j < H; ++j) dbias[j] = 0.0;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double z = load_elem(dt, y, i) + (bias ? load_elem(dt, bias, j) : 0.0);
      double gv = load_elem(dt, g, i);
      double v = gv * orc_gelu_tanh_grad(z);
      store_elem(dt, dgrad, i, v);
      if (dgrad64) dgrad64[i] = v;
      if (mag) mag[i] = fabs(gv) * gelu_tanh_grad_mag(z);
      if (dbias) dbias[j] += v;
    }
  return ORC_OK;
}

/* Magnitude of the larger of the two summands of orc_gelu_erf_grad. */
static double gelu_erf_grad_mag(double z) {
  double t1 = fabs(0.5 * erfc(-K_ERF * z));
  double t2 = fabs(z * K_PDF * exp(-0.5 * z * z));
  return t1 > t2 ? t1 : t2;
}

/* Exact (erf) bias-GeLU forward [fusions §4.2]: out = gelu_erf(y + bias). */
int orc_bias_gelu_erf_fwd(int dt, const void* y, const void* bias, void* out, double* out64, int64_t T,
                          int64_t H) {
  if (!dtype_ok(dt) || T < 0 || H <= 0) return ORC_BAD;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double z = load_elem(dt, y, i) + (bias ? load_elem(dt, bias, j) : 0.0);
      double v = orc_gelu_erf(z);
      store_elem(dt, out, i, v);
      if (out64) out64[i] = v;
    }
  return ORC_OK;
}

/* Exact (erf) bias-GeLU backward: dgrad = g * gelu_erf'(y + bias), dbias as for
 * the tanh form; mag = |g| times the larger summand of gelu_erf'. */
int orc_bias_gelu_erf_bwd(int dt, const void* g, const void* y, const void* bias, void* dgrad,
                          double* dgrad64, double* mag, double* dbias, int64_t T, int64_t H) {
  if (!dtype_ok(dt) || T < 0 || H <= 0) return ORC_BAD;
  if (dbias)
    for (int64_t j = 0; j < H; ++j) dbias[j] = 0.0;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double z = load_elem(dt, y, i) + (bias ? load_elem(dt, bias, j) : 0.0);
      double gv = load_elem(dt, g, i);
      double v = gv * orc_gelu_erf_grad(z);
      store_elem(dt, dgrad, i, v);
      if (dgrad64) dgrad64[i] = v;
      if (mag) mag[i] = fabs(gv) * gelu_erf_grad_mag(z);
      if (dbias) dbias[j] += v;
    }
  return ORC_OK;
}

/* Bias-dropout-add [fusions §3.2, §3.3].
 *   r' = residual rounded to dt when its dtype differs (the AMP-O1 cast);
 *   z  = x + bias;
 *   train: out = r' + (kept ? z * s : 0);  infer: out = r' + z.
 * mag (nullable): the largest magnitude among r', z*s, x*s, bias*s. */
int orc_bias_dropout_add(int dt, const void* x, const void* bias, const void* residual, int res_dt,
                         void* out, double* out64, double* mag, int64_t T, int64_t H, int train,
                         float p, uint64_t seed, uint64_t offset, int64_t row0) {
  if (!dtype_ok(dt) || !dtype_ok(res_dt) || T < 0 || H <= 0 || row0 < 0) return ORC_BAD;
  if (train && !prob_ok(p)) return ORC_BAD;
  uint64_t theta = train ? drop_threshold(p) : 0;
  double s = train ? (double)orc_keep_scale(p) : 1.0;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double xv = load_elem(dt, x, i);
      double bv = bias ? load_elem(dt, bias, j) : 0.0;
      double rv = load_elem(res_dt, residual, i);
      if (res_dt != dt) rv = to_dtype(dt, rv);
      double z = xv + bv;
      double v;
      int kept = 1;
      if (train) {
        uint64_t gi = (uint64_t)(row0 + t) * (uint64_t)H + (uint64_t)j;
        kept = element_kept(gi, theta, seed, offset);
        v = rv + (kept ? z * s : 0.0);
      } else {
        v = rv + z;
      }
      store_elem(dt, out, i, v);
      if (out64) out64[i] = v;
      if (mag) {
        double m = fabs(rv);
        if (kept) {
          double c[3] = {fabs(z * s), fabs(xv * s), fabs(bv * s)};
          for (int k = 0; k < 3; ++k)
            if (c[k] > m) m = c[k];
        }
        mag[i] = m;
      }
    }
  return ORC_OK;
}

/* Backward of bias-dropout-add, train [fusions §3.2, §3.3; the unit test of
 * §9 compares gradients too]. With out = r' + keep * (x + bias) * s:
 *   dx[t, j]        = g * s if kept, else 0                    (dtype dt)
 *   dresidual[t, j] = g, in the residual's dtype (nullable); the cast of the
 *                     residual to dt passes the gradient straight through
 *   dbias[j]        = sum over t of the unrounded dx[t, j]     (double, nullable)
 * The keep decisions are regenerated from (p, seed, offset) exactly as the
 * forward made them. */
int orc_bias_dropout_add_bwd(int dt, const void* g, int res_dt, void* dx, double* dx64, void* dres,
                             double* dbias, int64_t T, int64_t H, float p, uint64_t seed,
                             uint64_t offset, int64_t row0) {
  if (!dtype_ok(dt) || !dtype_ok(res_dt) || T < 0 || H <= 0 || row0 < 0 || !prob_ok(p)) return ORC_BAD;
  uint64_t theta = drop_threshold(p);
  double s = (double)orc_keep_scale(p);
  if (dbias)
    for (int64_t j = 0; j < H; ++j) dbias[j] = 0.0;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double gv = load_elem(dt, g, i);
      uint64_t gi = (uint64_t)(row0 + t) * (uint64_t)H + (uint64_t)j;
      double v = element_kept(gi, theta, seed, offset) ? gv * s : 0.0;
      store_elem(dt, dx, i, v);
      if (dx64) dx64[i] = v;
      if (dres) store_elem(res_dt, dres, i, gv);
      if (dbias) dbias[j] += v;
    }
  return ORC_OK;
}

/* Residual add + LayerNorm [fusions §5: the fused LayerNorm wrapped for the
 * listed hidden sizes, eps (default 1e-5) in the denominator, and the
 * zero-centred gamma applied as weight + 1]. The pages do not print the
 * normalisation itself; it is the standard LayerNorm over the hidden
 * dimension with the biased (1/H) variance. The residual add in front reads
 * the residual as §3.2 does (cast to x's dtype when they differ), so
 *   h[t, j] = x + r'                                   rounded to dt (stored)
 *   mean_t  = (1/H) sum_j h,   var_t = (1/H) sum_j (h - mean_t)^2
 *   rstd_t  = 1 / sqrt(var_t + eps)
 *   xhat    = (h - mean_t) * rstd_t
 *   y[t, j] = xhat * gamma'_j + beta_j,  gamma' = gamma (+ 1 if zero_centered)
 * The normalisation reads the ROUNDED h, as an unfused LayerNorm applied to
 * the stored sum would. gamma, beta (nullable: 0) are dt vectors; eps is the
 * float the caller passes, widened exactly.
 * Outputs: h (dt, nullable), y (dt), y64, mean/rstd (double [T], nullable),
 * mag (nullable): |gamma'| * (|xhat| + rstd * mean_j |h|) + |beta|, the size
 * of the terms an fp32 evaluation of y combines. */
static double ln_gamma(int dt, const void* gamma, int64_t j, int zero_centered) {
  return load_elem(dt, gamma, j) + (zero_centered ? 1.0 : 0.0);
}

int orc_add_layer_norm_fwd(int dt, const void* x, const void* residual, int res_dt, const void* gamma,
                           const void* beta, int zero_centered, float eps, void* h_out, void* y, double* y64,
                           double* mag, double* mean_out, double* rstd_out, int64_t T, int64_t H) {
  if (!dtype_ok(dt) || !dtype_ok(res_dt) || T < 0 || H <= 0 || !gamma || isnan(eps) || eps < 0.0f) return ORC_BAD;
  double* h = (double*)malloc(sizeof(double) * (size_t)H);
  if (!h) return ORC_BAD;
  for (int64_t t = 0; t < T; ++t) {
    double sum = 0.0, asum = 0.0;
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double rv = load_elem(res_dt, residual, i);
      if (res_dt != dt) rv = to_dtype(dt, rv);
      h[j] = to_dtype(dt, load_elem(dt, x, i) + rv);
      if (h_out) store_elem(dt, h_out, i, h[j]);
      sum += h[j];
      asum += fabs(h[j]);
    }
    double mean = sum / (double)H, var = 0.0;
    for (int64_t j = 0; j < H; ++j) var += (h[j] - mean) * (h[j] - mean);
    var /= (double)H;
    double rstd = 1.0 / sqrt(var + (double)eps);
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double xhat = (h[j] - mean) * rstd;
      double gj = ln_gamma(dt, gamma, j, zero_centered);
      double bj = beta ? load_elem(dt, beta, j) : 0.0;
      double v = xhat * gj + bj;
      store_elem(dt, y, i, v);
      if (y64) y64[i] = v;
      if (mag) mag[i] = fabs(gj) * (fabs(xhat) + rstd * asum / (double)H) + fabs(bj);
    }
    if (mean_out) mean_out[t] = mean;
    if (rstd_out) rstd_out[t] = rstd;
  }
  free(h);
  return ORC_OK;
}

/* Backward of residual add + LayerNorm. With a = dy * gamma' and xhat as in
 * the forward (recomputed here from h):
 *   dh[t, j]   = rstd_t * (a - mean_j a - xhat * mean_j (a * xhat)) + dh_in
 *   dx         = dh rounded to dt;  dresidual = dh rounded to res_dt (nullable)
 *   dgamma[j]  = sum_t dy * xhat,   dbeta[j] = sum_t dy        (double, nullable)
 * dh_in (res_dt, nullable) is the gradient reaching h from its other use as
 * the next residual; h = x + r' passes dh unchanged to both x and the
 * residual. mag (nullable): rstd * (|a| + mean|a| + (|xhat| + rstd mean|h|)
 * * mean|a xhat|) + |dh_in|. */
int orc_add_layer_norm_bwd(int dt, const void* dy, const void* h_in, const void* gamma, int zero_centered,
                           float eps, const void* dh_in, int res_dt, void* dx, double* dx64, double* mag,
                           void* dres, double* dgamma, double* dbeta, int64_t T, int64_t H) {
  if (!dtype_ok(dt) || !dtype_ok(res_dt) || T < 0 || H <= 0 || !gamma || isnan(eps) || eps < 0.0f) return ORC_BAD;
  double* h = (double*)malloc(sizeof(double) * (size_t)H);
  double* a = (double*)malloc(sizeof(double) * (size_t)H);
  if (!h || !a) {
    free(h);
    free(a);
    return ORC_BAD;
  }
  if (dgamma)
    for (int64_t j = 0; j < H; ++j) dgamma[j] = 0.0;
  if (dbeta)
    for (int64_t j = 0; j < H; ++j) dbeta[j] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    double sum = 0.0, asum_h = 0.0;
    for (int64_t j = 0; j < H; ++j) {
      h[j] = load_elem(dt, h_in, t * H + j);
      sum += h[j];
      asum_h += fabs(h[j]);
    }
    double mean = sum / (double)H, var = 0.0;
    for (int64_t j = 0; j < H; ++j) var += (h[j] - mean) * (h[j] - mean);
    var /= (double)H;
    double rstd = 1.0 / sqrt(var + (double)eps);
    double sa = 0.0, sax = 0.0, abs_a = 0.0, abs_ax = 0.0;
    for (int64_t j = 0; j < H; ++j) {
      double xhat = (h[j] - mean) * rstd;
      double dyv = load_elem(dt, dy, t * H + j);
      a[j] = dyv * ln_gamma(dt, gamma, j, zero_centered);
      sa += a[j];
      sax += a[j] * xhat;
      abs_a += fabs(a[j]);
      abs_ax += fabs(a[j] * xhat);
      if (dgamma) dgamma[j] += dyv * xhat;
      if (dbeta) dbeta[j] += dyv;
    }
    double ma = sa / (double)H, max = sax / (double)H;
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double xhat = (h[j] - mean) * rstd;
      double up = dh_in ? load_elem(res_dt, dh_in, i) : 0.0;
      double v = rstd * (a[j] - ma - xhat * max) + up;
      store_elem(dt, dx, i, v);
      if (dx64) dx64[i] = v;
      if (dres) store_elem(res_dt, dres, i, v);
      if (mag)
        mag[i] = rstd * (fabs(a[j]) + abs_a / (double)H + (fabs(xhat) + rstd * asum_h / (double)H) * abs_ax / (double)H) +
                 fabs(up);
    }
  }
  free(h);
  free(a);
  return ORC_OK;
}

/* Weighted squared ReLU for MoE experts [fusions §2 and §8 name the fused
 * op and its switch, §9 its unit test; the formula is not printed]. Read as
 * the weighted-SwiGLU pattern of §9 applied to the squared ReLU:
 *   out[t, j] = relu(x)^2 * w[t]          (w NULL: 1, the plain squared ReLU)
 * relu passes NaN through as torch's does (NaN > 0 is false, but NaN is not 0).
 * Backward:
 *   dx[t, j]  = g * w[t] * 2 relu(x)
 *   dw[t]     = sum_j g * relu(x)^2      (double, nullable; needs w)    */
static double relu(double x) { return x > 0.0 ? x : (isnan(x) ? x : 0.0); }

int orc_weighted_squared_relu_fwd(int dt, const void* x, const void* w, int w_dt, void* out, double* out64,
                                  int64_t T, int64_t H) {
  if (!dtype_ok(dt) || (w && !dtype_ok(w_dt)) || T < 0 || H <= 0) return ORC_BAD;
  for (int64_t t = 0; t < T; ++t) {
    double wt = w ? load_elem(w_dt, w, t) : 1.0;
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double r = relu(load_elem(dt, x, i));
      double v = r * r * wt;
      store_elem(dt, out, i, v);
      if (out64) out64[i] = v;
    }
  }
  return ORC_OK;
}

int orc_weighted_squared_relu_bwd(int dt, const void* g, const void* x, const void* w, int w_dt, void* dx,
                                  double* dx64, double* dw, int64_t T, int64_t H) {
  if (!dtype_ok(dt) || (w && !dtype_ok(w_dt)) || T < 0 || H <= 0 || (dw && !w)) return ORC_BAD;
  for (int64_t t = 0; t < T; ++t) {
    double wt = w ? load_elem(w_dt, w, t) : 1.0;
    double acc = 0.0;
    for (int64_t j = 0; j < H; ++j) {
      int64_t i = t * H + j;
      double r = relu(load_elem(dt, x, i));
      double gv = load_elem(dt, g, i);
      double v = gv * wt * 2.0 * r;
      store_elem(dt, dx, i, v);
      if (dx64) dx64[i] = v;
      acc += gv * r * r;
    }
    if (dw) dw[t] = acc;
  }
  return ORC_OK;
}

static double act_fwd(int act, double a) { return act == ORC_SWIGLU ? orc_silu(a) : orc_gelu_tanh(a); }
static double act_grad(int act, double a) {
  return act == ORC_SWIGLU ? orc_silu_grad(a) : orc_gelu_tanh_grad(a);
}
static double act_grad_mag(int act, double a) {
  return act == ORC_SWIGLU ? silu_grad_mag(a) : gelu_tanh_grad_mag(a);
}

/* Bias + gated activation forward [fusions §2, §9].
 * in is [T, 2H]; a = in[t, j] + bias[j], b = in[t, H + j] + bias[H + j];
 * out[t, j] = act(a) * b, times w[t] when w is given (weighted SwiGLU). */
int orc_bias_glu_fwd(int act, int dt, const void* in, const void* bias, const void* w, int w_dt,
                     void* out, double* out64, int64_t T, int64_t H) {
  if ((act != ORC_SWIGLU && act != ORC_GEGLU) || !dtype_ok(dt) || T < 0 || H <= 0) return ORC_BAD;
  if (w && !dtype_ok(w_dt)) return ORC_BAD;
  for (int64_t t = 0; t < T; ++t) {
    double wt = w ? load_elem(w_dt, w, t) : 1.0;
    for (int64_t j = 0; j < H; ++j) {
      double a = load_elem(dt, in, t * 2 * H + j) + (bias ? load_elem(dt, bias, j) : 0.0);
      double b = load_elem(dt, in, t * 2 * H + H + j) + (bias ? load_elem(dt, bias, H + j) : 0.0);
      double v = act_fwd(act, a) * b;
      if (w) v *= wt;
      store_elem(dt, out, t * H + j, v);
      if (out64) out64[t * H + j] = v;
    }
  }
  return ORC_OK;
}

/* Bias + gated activation backward.
 *   da = g * w * b * act'(a),  db = g * w * act(a)      -> din[t, j], din[t, H + j]
 *   dbias[c] = sum over t of the unrounded din[t, c]     (c in [0, 2H), nullable)
 *   dw[t]    = sum over j of g * act(a) * b              (weighted only, nullable)
 * mag (nullable, [T, 2H]): for da, |g w b| times the larger summand of act';
 * for db, |g w act(a)|. */
int orc_bias_glu_bwd(int act, int dt, const void* g, const void* in, const void* bias, const void* w,
                     int w_dt, void* din, double* din64, double* mag, double* dbias, double* dw,
                     int64_t T, int64_t H) {
  if ((act != ORC_SWIGLU && act != ORC_GEGLU) || !dtype_ok(dt) || T < 0 || H <= 0) return ORC_BAD;
  if (w && !dtype_ok(w_dt)) return ORC_BAD;
  if (dbias)
    for (int64_t c = 0; c < 2 * H; ++c) dbias[c] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    double wt = w ? load_elem(w_dt, w, t) : 1.0;
    double acc_w = 0.0;
    for (int64_t j = 0; j < H; ++j) {
      double a = load_elem(dt, in, t * 2 * H + j) + (bias ? load_elem(dt, bias, j) : 0.0);
      double b = load_elem(dt, in, t * 2 * H + H + j) + (bias ? load_elem(dt, bias, H + j) : 0.0);
      double gv = load_elem(dt, g, t * H + j);
      double fa = act_fwd(act, a);
      double da = gv * wt * b * act_grad(act, a);
      double db = gv * wt * fa;
      int64_t ia = t * 2 * H + j, ib = t * 2 * H + H + j;
      store_elem(dt, din, ia, da);
      store_elem(dt, din, ib, db);
      if (din64) {
        din64[ia] = da;
        din64[ib] = db;
      }
      if (mag) {
        mag[ia] = fabs(gv * wt * b) * act_grad_mag(act, a);
        mag[ib] = fabs(db);
      }
      if (dbias) {
        dbias[j] += da;
        dbias[H + j] += db;
      }
      acc_w += gv * fa * b;
    }
    if (dw && w) dw[t] = acc_w;
  }
  return ORC_OK;
}

int orc_version(void) { return 1; }
