/* Runs every oracle32 entry point (oracle/oracle32.c) on small inputs with
 * edge cases (no rows, one column, NaN and infinite inputs, p = 0 and 1,
 * every dtype it takes), so that an address- and undefined-behaviour-
 * sanitized build checks its memory accesses and arithmetic. Prints "ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc32_bias_gelu_fwd(int, int, const void*, const void*, void*, int64_t, int64_t);
int orc32_bias_gelu_bwd(int, int, const void*, const void*, const void*, void*, float*, int64_t, int64_t);
int orc32_bias_dropout_add(int, const void*, const void*, const void*, int, void*, int64_t, int64_t, int, float,
                           uint64_t, uint64_t, int64_t);
int orc32_bias_dropout_add_bwd(int, const void*, int, void*, void*, float*, int64_t, int64_t, float, uint64_t,
                               uint64_t, int64_t);
int orc32_bias_glu_fwd(int, int, const void*, const void*, const void*, int, void*, int64_t, int64_t);
int orc32_bias_glu_bwd(int, int, const void*, const void*, const void*, const void*, int, void*, float*, float*,
                       int64_t, int64_t);
int orc32_add_layer_norm_fwd(int, const void*, const void*, int, const void*, const void*, int, float, void*, void*,
                             float*, float*, int64_t, int64_t);
int orc32_add_layer_norm_bwd(int, const void*, const void*, const void*, int, float, const void*, int, void*, void*,
                             float*, float*, int64_t, int64_t);
int orc32_weighted_squared_relu_fwd(int, const void*, const void*, int, void*, int64_t, int64_t);
int orc32_weighted_squared_relu_bwd(int, const void*, const void*, const void*, int, void*, float*, int64_t, int64_t);
uint16_t orc_round_bf16(double);
uint16_t orc_round_f16(double);

static size_t esz(int dt) { return dt == 0 ? 4 : 2; }

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
      default: ((uint16_t*)p)[i] = orc_round_bf16(v); break;
    }
  }
  return p;
}

int main(void) {
  int bad = 0;
  const int64_t shapes[][2] = {{0, 8}, {1, 4}, {3, 8}, {5, 12}};
  for (int s = 0; s < 4; ++s) {
    const int64_t T = shapes[s][0], H = shapes[s][1], n = T * H;
    for (int dt = 0; dt < 3; ++dt) {
      void *x = fill(dt, (size_t)(n + 1), 1), *g = fill(dt, (size_t)(n + 1), 2), *b = fill(dt, (size_t)(2 * H), 3);
      void *r32 = fill(0, (size_t)(n + 1), 4), *w = fill(dt, (size_t)(T + 1), 5), *in2 = fill(dt, (size_t)(2 * n + 1), 6);
      void* out = malloc((size_t)(2 * n + 1) * 4);
      void* out2 = malloc((size_t)(2 * n + 1) * 4);
      float* red = malloc((size_t)(2 * H + T + 1) * sizeof(float));
      float* red2 = malloc((size_t)(2 * H + T + 1) * sizeof(float));
      float* st = malloc((size_t)(2 * T + 2) * sizeof(float));
      for (int exact = 0; exact < 2; ++exact) {
        bad |= orc32_bias_gelu_fwd(dt, exact, x, b, out, T, H);
        bad |= orc32_bias_gelu_fwd(dt, exact, x, NULL, out, T, H);
        bad |= orc32_bias_gelu_bwd(dt, exact, g, x, b, out, red, T, H);
        bad |= orc32_bias_gelu_bwd(dt, exact, g, x, NULL, out, NULL, T, H);
      }
      const float ps[] = {0.0f, 0.1f, 0.5f, 1.0f};
      for (int k = 0; k < 4; ++k) {
        bad |= orc32_bias_dropout_add(dt, x, b, x, dt, out, T, H, 1, ps[k], 1234, 7, 3);
        bad |= orc32_bias_dropout_add(dt, x, NULL, r32, 0, out, T, H, 1, ps[k], 1, (uint64_t)1 << 32, 0);
        bad |= orc32_bias_dropout_add_bwd(dt, g, dt, out, out2, red, T, H, ps[k], 99, 0, 0);
        bad |= orc32_bias_dropout_add_bwd(dt, g, 0, out, NULL, NULL, T, H, ps[k], 99, 0, 0);
      }
      bad |= orc32_bias_dropout_add(dt, x, b, r32, 0, out, T, H, 0, 0.0f, 0, 0, 0);
      bad |= orc32_add_layer_norm_fwd(dt, x, x, dt, b, b, 1, 1e-5f, out2, out, st, st + T + 1, T, H);
      bad |= orc32_add_layer_norm_fwd(dt, x, r32, 0, b, NULL, 0, 0.0f, NULL, out, NULL, NULL, T, H);
      bad |= orc32_add_layer_norm_bwd(dt, g, x, b, 1, 1e-5f, g, dt, out, out2, red, red2, T, H);
      bad |= orc32_add_layer_norm_bwd(dt, g, x, b, 0, 1e-5f, NULL, 0, out, NULL, NULL, NULL, T, H);
      bad |= orc32_weighted_squared_relu_fwd(dt, x, w, dt, out, T, H);
      bad |= orc32_weighted_squared_relu_fwd(dt, x, NULL, dt, out, T, H);
      bad |= orc32_weighted_squared_relu_bwd(dt, g, x, w, dt, out, red, T, H);
      for (int act = 0; act < 2; ++act) {
        bad |= orc32_bias_glu_fwd(act, dt, in2, b, w, dt, out, T, H);
        bad |= orc32_bias_glu_fwd(act, dt, in2, NULL, NULL, dt, out, T, H);
        bad |= orc32_bias_glu_bwd(act, dt, g, in2, b, w, dt, out, red, red2, T, H);
        bad |= orc32_bias_glu_bwd(act, dt, g, in2, NULL, NULL, dt, out, NULL, NULL, T, H);
      }
      free(x); free(g); free(b); free(r32); free(w); free(in2); free(out); free(out2); free(red); free(red2);
      free(st);
    }
  }
  /* refused arguments: fp64 storage, bad shapes, probabilities, dw without weights */
  bad |= orc32_bias_gelu_fwd(3, 0, NULL, NULL, NULL, 1, 4) == 0;
  bad |= orc32_bias_gelu_fwd(0, 0, NULL, NULL, NULL, -1, 4) == 0;
  bad |= orc32_bias_dropout_add(0, NULL, NULL, NULL, 0, NULL, 1, 4, 1, NAN, 0, 0, 0) == 0;
  bad |= orc32_bias_dropout_add_bwd(0, NULL, 0, NULL, NULL, NULL, 1, 4, 1.5f, 0, 0, 0) == 0;
  bad |= orc32_weighted_squared_relu_bwd(0, NULL, NULL, NULL, 0, NULL, (float*)&bad, 1, 4) == 0;
  printf("%s\n", bad ? "FAIL" : "ok");
  return bad;
}
