// Host program: prints Philox4x32-10 blocks from rocRAND's header-only engine.
// Usage: philox_rocrand seed subsequence q0 count  -> prints count lines "w0 w1 w2 w3"
// for blocks q0 .. q0+count-1 (engine offset 4q: word 4q of the subsequence).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  if (argc != 5) return 2;
  unsigned long long seed = strtoull(argv[1], 0, 0), sub = strtoull(argv[2], 0, 0);
  unsigned long long q0 = strtoull(argv[3], 0, 0), cnt = strtoull(argv[4], 0, 0);
  for (unsigned long long q = q0; q < q0 + cnt; ++q) {
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ull * q);
    uint4 v = e.next4();
    printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
