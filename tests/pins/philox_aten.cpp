// Test-only cross-check: Philox4x32-10 blocks from ATen's host engine
// (torch/include/ATen/core/PhiloxRNGEngine.h), an implementation independent
// of this repository's oracle and GPU library.  Counter words (c0,c1,c2,c3)
// map to ATen's offset = (c1 << 32) | c0 and subsequence = (c3 << 32) | c2.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>

extern "C" void aten_philox_batch(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n) {
  for (int64_t b = 0; b < n; ++b) {
    const uint32_t* c = ctr + 4 * b;
    const uint64_t offset = ((uint64_t)c[1] << 32) | c[0];
    const uint64_t subseq = ((uint64_t)c[3] << 32) | c[2];
    at::philox_engine eng(seed, subseq, offset);
    for (int k = 0; k < 4; ++k) out[4 * b + k] = eng();
  }
}
