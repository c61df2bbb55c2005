/* Runs every oracle entry point on small inputs, edge cases included (no
 * rows, one column, NaN and infinite inputs, p = 0 and 1, every dtype), so
 * that an address- and undefined-behaviour-sanitized build of oracle.c can
 * check the oracle's own memory accesses and arithmetic. Prints "ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_bias_gelu_fwd(int, const void*, const void*, void*, double*, int64_t, int64_t);
int orc_bias_gelu_bwd(int, const void*, const void*, const void*, void*, double*, double*, double*, int64_t, int64_t);
int orc_bias_gelu_erf_fwd(int, const void*, const void*, void*, double*, int64_t, int64_t);
int orc_bias_gelu_erf_bwd(int, const void*, const void*, const void*, void*, double*, double*, double*, int64_t,
                          int64_t);
int orc_bias_dropout_add(int, const void*, const void*, const void*, int, void*, double*, double*, int64_t, int64_t,
                         int, float, uint64_t, uint64_t, int64_t);
int orc_bias_dropout_add_bwd(int, const void*, int, void*, double*, void*, double*, int64_t, int64_t, float,
                             uint64_t, uint64_t, int64_t);
int orc_dropout_mask(uint8_t*, int64_t, int64_t, float, uint64_t, uint64_t, int64_t);
int orc_add_layer_norm_fwd(int, const void*, const void*, int, const void*, const void*, int, float, void*, void*,
                           double*, double*, double*, double*, int64_t, int64_t);
int orc_add_layer_norm_bwd(int, const void*, const void*, const void*, int, float, const void*, int, void*, double*,
                           double*, void*, double*, double*, int64_t, int64_t);
int orc_weighted_squared_relu_fwd(int, const void*, const void*, int, void*, double*, int64_t, int64_t);
int orc_weighted_squared_relu_bwd(int, const void*, const void*, const void*, int, void*, double*, double*, int64_t,
                                  int64_t);
int orc_bias_glu_fwd(int, int, const void*, const void*, const void*, int, void*, double*, int64_t, int64_t);
int orc_bias_glu_bwd(int, int, const void*, const void*, const void*, const void*, int, void*, double*, double*,
                     double*, double*, int64_t, int64_t);
uint16_t orc_round_bf16(double);
uint16_t orc_round_f16(double);
double orc_bf16_to_double(uint16_t);
double orc_f16_to_double(uint16_t);

static size_t esz(int dt) { return dt == 0 ? 4 : dt == 3 ? 8 : 2; }

/* n elements of dtype dt holding a mix of ordinary and special values */
static void* fill(int dt, size_t n, unsigned seed) {
  void* p = malloc(n * esz(dt) + 1);
  for (size_t i = 0; i < n; ++i) {
    seed = seed * 1664525u + 1013904223u;
    double v = ((double)(seed >> 8) / 16777216.0 - 0.5) * 16.0;
    if (i % 97 == 3) v = NAN;
    if (i % 89 == 5) v = INFINITY;
    if (i % 83 == 7) v = -INFINITY;
    if (i % 79 == 11) v = 0.0;
    if (i % 73 == 13) v = -1e-40;
    switch (dt) {
      case 0: ((float*)p)[i] = (float)v; break;
      case 1: ((uint16_t*)p)[i] = orc_round_f16(v); break;
      case 2: ((uint16_t*)p)[i] = orc_round_bf16(v); break;
      default: ((double*)p)[i] = v;
    }
  }
  return p;
}

int main(void) {
  int bad = 0;
  const int64_t shapes[][2] = {{0, 8}, {1, 4}, {3, 8}, {5, 12}};
  for (int s = 0; s < 4; ++s) {
    const int64_t T = shapes[s][0], H = shapes[s][1], n = T * H;
    for (int dt = 0; dt < 4; ++dt) {
      void *x = fill(dt, (size_t)(n + 1), 1), *g = fill(dt, (size_t)(n + 1), 2), *b = fill(dt, (size_t)(2 * H), 3);
      void *r32 = fill(0, (size_t)(n + 1), 4), *w = fill(dt, (size_t)(T + 1), 5), *in2 = fill(dt, (size_t)(2 * n + 1), 6);
      void* out = malloc((size_t)(2 * n + 1) * 8);
      void* out2 = malloc((size_t)(2 * n + 1) * 8);
      double* o64 = malloc((size_t)(2 * n + 1) * sizeof(double));
      double* mag = malloc((size_t)(2 * n + 1) * sizeof(double));
      double* red = malloc((size_t)(2 * H + T + 1) * sizeof(double));
      double* red2 = malloc((size_t)(2 * H + T + 1) * sizeof(double));
      double* st = malloc((size_t)(2 * T + 2) * sizeof(double));
      uint8_t* bits = malloc((size_t)(n / 8 + 2));
      bad |= orc_bias_gelu_fwd(dt, x, b, out, o64, T, H);
      bad |= orc_bias_gelu_fwd(dt, x, NULL, out, NULL, T, H);
      bad |= orc_bias_gelu_bwd(dt, g, x, b, out, o64, mag, red, T, H);
      bad |= orc_bias_gelu_erf_fwd(dt, x, b, out, o64, T, H);
      bad |= orc_bias_gelu_erf_bwd(dt, g, x, b, out, o64, mag, red, T, H);
      const float ps[] = {0.0f, 0.1f, 0.5f, 1.0f};
      for (int k = 0; k < 4; ++k) {
        bad |= orc_bias_dropout_add(dt, x, b, x, dt, out, o64, mag, T, H, 1, ps[k], 1234, 7, 3);
        bad |= orc_bias_dropout_add(dt, x, NULL, r32, 0, out, o64, mag, T, H, 1, ps[k], 1, (uint64_t)1 << 32, 0);
        bad |= orc_bias_dropout_add_bwd(dt, g, dt, out, o64, out2, red, T, H, ps[k], 99, 0, 0);
        bad |= orc_bias_dropout_add_bwd(dt, g, 0, out, o64, out2, red, T, H, ps[k], 99, 0, 0);
        bad |= orc_dropout_mask(bits, T, H, ps[k], 5, 6, 2);
      }
      bad |= orc_bias_dropout_add(dt, x, b, r32, 0, out, NULL, NULL, T, H, 0, 0.0f, 0, 0, 0);
      bad |= orc_add_layer_norm_fwd(dt, x, x, dt, b, b, 1, 1e-5f, out2, out, o64, mag, st, st + T + 1, T, H);
      bad |= orc_add_layer_norm_fwd(dt, x, r32, 0, b, NULL, 0, 0.0f, NULL, out, NULL, NULL, NULL, NULL, T, H);
      bad |= orc_add_layer_norm_bwd(dt, g, x, b, 1, 1e-5f, g, dt, out, o64, mag, out2, red, red2, T, H);
      bad |= orc_add_layer_norm_bwd(dt, g, x, b, 0, 1e-5f, NULL, 0, out, NULL, NULL, NULL, NULL, NULL, T, H);
      bad |= orc_weighted_squared_relu_fwd(dt, x, w, dt, out, o64, T, H);
      bad |= orc_weighted_squared_relu_fwd(dt, x, NULL, dt, out, NULL, T, H);
      bad |= orc_weighted_squared_relu_bwd(dt, g, x, w, dt, out, o64, red, T, H);
      for (int act = 0; act < 2; ++act) {
        bad |= orc_bias_glu_fwd(act, dt, in2, b, w, dt, out, o64, T, H);
        bad |= orc_bias_glu_fwd(act, dt, in2, NULL, NULL, dt, out, NULL, T, H);
        bad |= orc_bias_glu_bwd(act, dt, g, in2, b, w, dt, out, o64, mag, red, red2, T, H);
        bad |= orc_bias_glu_bwd(act, dt, g, in2, NULL, NULL, dt, out, NULL, NULL, NULL, NULL, T, H);
      }
      free(x); free(g); free(b); free(r32); free(w); free(in2); free(out); free(out2); free(o64); free(mag);
      free(red); free(red2); free(st); free(bits);
    }
  }
  /* refused arguments */
  bad |= orc_bias_gelu_fwd(7, NULL, NULL, NULL, NULL, 1, 4) == 0;
  bad |= orc_bias_gelu_fwd(0, NULL, NULL, NULL, NULL, -1, 4) == 0;
  bad |= orc_dropout_mask(NULL, 1, 4, NAN, 0, 0, 0) == 0;
  bad |= orc_dropout_mask(NULL, 1, 4, 1.5f, 0, 0, 0) == 0;
  /* every 16-bit pattern round-trips through the decoders and rounders */
  for (uint32_t h = 0; h < 65536; ++h) {
    double v = orc_bf16_to_double((uint16_t)h), u = orc_f16_to_double((uint16_t)h);
    if (!isnan(v)) bad |= orc_round_bf16(v) != (uint16_t)h;
    if (!isnan(u)) bad |= orc_round_f16(u) != (uint16_t)h;
  }
  printf("%s\n", bad ? "FAIL" : "ok");
  return bad;
}
