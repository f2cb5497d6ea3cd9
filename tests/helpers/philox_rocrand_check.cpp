// Prints Philox4x32-10 blocks produced by rocRAND's engine, for checking the
// oracle's own implementation against an independent one.  Reads lines
// "seed pos" from stdin; for each prints the four 32-bit words of
// philox(counter = (pos, 0, 0, 0), key = (seed lo, seed hi)).  rocRAND's
// (seed, subsequence 0, offset 4*pos) start position is that same block.
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
  unsigned long long seed, pos;
  while (std::scanf("%llu %llu", &seed, &pos) == 2) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, 0ull, 4ull * pos, &st);
    uint4 r = rocrand4(&st);
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
