// Test-only helper: exposes rocRAND's Philox4x32-10 engine (a library
// routine, used here from its public header and run on the host) so the
// oracle's pure-Python Philox can be pinned against it.
#include <rocrand/rocrand_kernel.h>

extern "C" void rocrand_philox4x32_10_block(unsigned int c0, unsigned int c1, unsigned int c2,
                                            unsigned int c3, unsigned int k0, unsigned int k1,
                                            unsigned int* out4) {
  // rocRAND places the 64-bit "subsequence" in counter words 2..3 and
  // skips offset/4 blocks in words 0..1.
  const unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
  const unsigned long long subsequence = ((unsigned long long)c3 << 32) | c2;
  const unsigned long long block = ((unsigned long long)c1 << 32) | c0;
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, subsequence, block * 4ull, &st);
  uint4 r = rocrand4(&st);
  out4[0] = r.x; out4[1] = r.y; out4[2] = r.z; out4[3] = r.w;
}
