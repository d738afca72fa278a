// Host-only driver that evaluates rocRAND's Philox4x32-10 (an installed,
// independently written library) for counters/keys read from stdin.
// Each input line: c0 c1 c2 c3 k0 k1 (decimal); output: four words (decimal).
// Counter words (c0, c1) are reached through the engine's offset (4 draws per
// counter value) and (c2, c3) through its subsequence; the key is the seed.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const unsigned long long seed = k0 | (k1 << 32);
    const unsigned long long sub = c2 | (c3 << 32);
    const unsigned long long ctr01 = c0 | (c1 << 32);
    rocrand_device::philox4x32_10_engine e(seed, sub, 0ull);
    // advance the 64-bit low counter by ctr01 blocks of four outputs
    for (int i = 0; i < 4; ++i) e.discard(ctr01);
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
