// Test-only cross-check: Philox4x32-10 blocks from rocRAND's host-callable
// engine (rocrand/rocrand_philox4x32_10.h), independent of this repository's
// oracle and GPU library.  rocRAND's subsequence fills counter words 2,3 and
// its offset counts 32-bit outputs, so counter words (c0,c1) are reached with
// offset = 4 * ((c1 << 32) | c0); that stays below 2^64 for c1 < 2^30.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdint>

extern "C" void rocrand_philox_batch(uint64_t seed, const uint32_t* ctr, uint32_t* out,
                                     int64_t n) {
  for (int64_t b = 0; b < n; ++b) {
    const uint32_t* c = ctr + 4 * b;
    const unsigned long long offset = 4ull * (((unsigned long long)c[1] << 32) | c[0]);
    const unsigned long long subseq = ((unsigned long long)c[3] << 32) | c[2];
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    for (int k = 0; k < 4; ++k) out[4 * b + k] = eng();
  }
}
