// Host-only reference for the Philox4x32-10 pin: drives rocRAND's own
// Philox4x32-10 engine (an implementation independent of this project) so the
// oracle's generator can be checked against it.  Input lines: c0 c1 c2 c3 k0 k1
// (hex, 32-bit each).  Output lines: the four 32-bit words for that counter/key.
// The engine is positioned with seed = k0 | k1<<32, subsequence = c2 | c3<<32 and
// offset = 4 * (c0 | c1<<32), which places its counter block at (c0, c1, c2, c3).
#include <cstdio>
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    rocrand_state_philox4x32_10 st;
    unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
    unsigned long long subseq = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long offset = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
    rocrand_init(seed, subseq, offset, &st);
    unsigned a = rocrand(&st), b = rocrand(&st), c = rocrand(&st), d = rocrand(&st);
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
