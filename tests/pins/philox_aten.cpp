// Host program: prints Philox4x32-10 blocks from ATen's header-only philox_engine.
// Usage: philox_aten seed subsequence q0 count -> count lines "w0 w1 w2 w3" for blocks q0..
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  if (argc != 5) return 2;
  unsigned long long seed = strtoull(argv[1], 0, 0), sub = strtoull(argv[2], 0, 0);
  unsigned long long q0 = strtoull(argv[3], 0, 0), cnt = strtoull(argv[4], 0, 0);
  for (unsigned long long q = q0; q < q0 + cnt; ++q) {
    at::philox_engine e(seed, sub, q);
    uint32_t w[4];
    for (int k = 0; k < 4; ++k) w[k] = e();
    printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
