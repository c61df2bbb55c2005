// Drives the C ABI's host code (argument validation, workspace queries,
// launch planning) through every entry point with ordinary, edge and hostile
// arguments: null and misaligned pointers, overlapping buffers, unknown
// dtypes, NaN and out-of-range probabilities, row counts and widths up to the
// int64 limits. Built with the address and undefined-behaviour sanitizers
// against launch stand-ins (abi_stubs.cpp), so it needs no GPU; prints "ok".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "mb.h"

namespace mb {
extern int stub_launches;
}

namespace {

void* P(uintptr_t k) { return reinterpret_cast<void*>(k << 32); }  // fake, 4 GiB apart, never dereferenced
float* F(uintptr_t k) { return reinterpret_cast<float*>(k << 32); }
const hipStream_t S = nullptr;
int bad = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("unexpected: %s\n", what);
    bad = 1;
  }
}

}  // namespace

int main() {
  const int64_t maxi = std::numeric_limits<int64_t>::max();
  const int64_t Ts[] = {0, 1, 3, 4096, 1 << 20, int64_t{1} << 40, (int64_t{1} << 40) + 1, maxi, -1};
  const int64_t Hs[] = {4, 8, 12, 1040, 32768, 65536, 4194312, int64_t{1} << 31, maxi / 4, maxi, 0, -8};
  const mb_dtype_t dts[] = {MB_F32, MB_F16, MB_BF16, static_cast<mb_dtype_t>(7)};
  for (int64_t T : Ts)
    for (int64_t H : Hs)
      for (mb_dtype_t dt : dts) {
        // workspace queries: pure host arithmetic at any size
        for (int w = 0; w < 2; ++w) {
          (void)mb_bias_gelu_bwd_workspace(T, H, dt, w);
          (void)mb_bias_gelu_erf_bwd_workspace(T, H, dt, w);
          (void)mb_bias_dropout_add_bwd_workspace(T, H, dt, w);
          (void)mb_bias_glu_bwd_workspace(T, H, dt, w, 1 - w);
          (void)mb_weighted_squared_relu_bwd_workspace(T, H, dt, w);
          (void)mb_add_layer_norm_bwd_workspace(T, H, dt, MB_F32, w);
          (void)mb_add_layer_norm_bwd_workspace(T, H, dt, dt, w);
        }
        const size_t big = std::numeric_limits<size_t>::max();
        (void)mb_bias_gelu_fwd(P(1), P(2), P(3), T, H, dt, S);
        (void)mb_bias_gelu_fwd(P(1), nullptr, P(1), T, H, dt, S);
        (void)mb_bias_gelu_erf_fwd(P(1), P(2), P(3), T, H, dt, S);
        (void)mb_bias_gelu_bwd(P(1), P(2), P(3), P(4), F(5), P(6), big, T, H, dt, S);
        (void)mb_bias_gelu_bwd(P(1), P(2), nullptr, P(1), nullptr, nullptr, 0, T, H, dt, S);
        (void)mb_bias_gelu_erf_bwd(P(1), P(2), P(3), P(4), F(5), P(6), big, T, H, dt, S);
        (void)mb_bias_gelu_bwd_noalloc(P(1), P(2), P(3), P(4), F(5), T, H, dt, S);
        for (float p : {0.0f, 0.1f, 1.0f, 1.5f, -0.1f, NAN, INFINITY}) {
          (void)mb_bias_dropout_add_train(P(1), P(2), P(3), MB_F32, P(4), T, H, dt, p, 1, 2, S);
          (void)mb_bias_dropout_add_train(P(1), nullptr, P(3), dt, P(1), T, H, dt, p, ~0ull, ~0ull, S);
          (void)mb_bias_dropout_add_bwd(P(1), P(2), P(3), MB_F32, F(4), P(5), big, T, H, dt, p, 1, 2, S);
          (void)mb_bias_dropout_add_bwd(P(1), P(1), nullptr, dt, nullptr, nullptr, 0, T, H, dt, p, 1, 2, S);
          (void)mb_dropout_mask(static_cast<uint8_t*>(P(1)), T, H, p, 1, 2, S);
        }
        (void)mb_bias_dropout_add_infer(P(1), P(2), P(3), dt, P(1), T, H, dt, S);
        (void)mb_bias_swiglu_fwd(P(1), P(2), P(3), MB_F32, P(4), T, H, dt, S);
        (void)mb_bias_geglu_fwd(P(1), P(2), P(4), T, H, dt, S);
        (void)mb_bias_swiglu_bwd(P(1), P(2), P(3), P(4), dt, P(5), F(6), F(7), P(8), big, T, H, dt, S);
        (void)mb_bias_swiglu_bwd(P(1), P(2), nullptr, nullptr, dt, P(2), nullptr, F(7), nullptr, 0, T, H, dt, S);
        (void)mb_bias_geglu_bwd(P(1), P(2), P(3), P(5), F(6), P(8), big, T, H, dt, S);
        for (float eps : {1e-5f, 0.0f, -1.0f, NAN, INFINITY}) {
          (void)mb_add_layer_norm_fwd(P(1), P(2), MB_F32, P(3), P(4), eps, 1, P(5), P(6), F(7), F(8), T, H, dt, S);
          (void)mb_add_layer_norm_fwd(P(1), P(2), dt, P(3), nullptr, eps, 0, P(1), P(2), nullptr, nullptr, T, H, dt, S);
        }
        (void)mb_add_layer_norm_bwd(P(1), P(2), P(3), F(4), F(5), 1, P(6), MB_F32, P(7), P(8), F(9), F(10), P(11), big, T,
                                    H, dt, S);
        (void)mb_add_layer_norm_bwd(P(1), P(2), P(3), F(4), F(5), 0, nullptr, dt, P(1), nullptr, nullptr, nullptr,
                                    nullptr, 0, T, H, dt, S);
        (void)mb_weighted_squared_relu_fwd(P(1), P(2), MB_F32, P(3), T, H, dt, S);
        (void)mb_weighted_squared_relu_bwd(P(1), P(2), P(3), MB_BF16, P(4), F(5), P(6), big, T, H, dt, S);
      }
  // a few exact answers
  expect(mb_bias_gelu_fwd(nullptr, nullptr, P(1), 4, 8, MB_BF16, S) == MB_ERR_NULL, "null y");
  expect(mb_bias_gelu_fwd(P(1), nullptr, P(2), 4, 7, MB_BF16, S) == MB_ERR_SHAPE, "ragged row");
  expect(mb_bias_gelu_fwd(P(1), nullptr, P(2), maxi, 8, MB_BF16, S) == MB_ERR_SHAPE, "size overflow");
  expect(mb_bias_dropout_add_train(P(1), nullptr, P(2), MB_BF16, P(3), 4, 8, MB_BF16, NAN, 1, 2, S) == MB_ERR_PROB,
         "NaN p");
  expect(mb_bias_gelu_bwd_noalloc(P(1), P(2), nullptr, P(3), F(4), 1, 4194312, MB_BF16, S) == MB_ERR_SCRATCH,
         "scratch too small");
  expect(mb_add_layer_norm_fwd(P(1), P(2), MB_BF16, P(3), nullptr, NAN, 0, nullptr, P(4), nullptr, nullptr, 4, 64,
                               MB_BF16, S) == MB_ERR_PROB,
         "NaN eps");
  expect(mb::stub_launches > 0, "no call reached a launch");
  std::printf("%s\n", bad ? "FAIL" : "ok");
  return bad;
}
