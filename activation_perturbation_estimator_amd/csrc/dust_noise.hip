// dust_noise.hip -- the noise stage: raw Philox blocks and materialised
// standard-normal noise a^(i)_t[n] (laoyaoba analysis, mechanism section: each
// linear output is jittered by sigma times standard-normal noise, token by
// token).
//
// The estimator kernels never read noise from memory: they regenerate it from
// its counters.  These two kernels serve callers that apply the noise in their
// own perturbed forward, and the bit-exactness tests.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

__global__ void __launch_bounds__(256) philox_raw_kernel(const uint32_t* __restrict__ ctr,
                                                         uint32_t* __restrict__ out, int64_t n,
                                                         uint32_t k0, uint32_t k1) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n; b += stride) {
    const uint4 c = reinterpret_cast<const uint4*>(ctr)[b];
    const u32x4 x = philox10(c.x, c.y, c.z, c.w, k0, k1);
    reinterpret_cast<uint4*>(out)[b] = make_uint4(x.x, x.y, x.z, x.w);
  }
}

// One thread per Philox block (four consecutive columns of one (draw, token)
// row); consecutive threads write consecutive 16-byte chunks.
__global__ void __launch_bounds__(256) noise_fill_kernel(float* __restrict__ out,
                                                         int64_t ndraw, int64_t T, int64_t nblk,
                                                         uint32_t draw0, uint32_t stream,
                                                         uint32_t k0, uint32_t k1) {
  const int64_t total = ndraw * T * nblk;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < total; b += stride) {
    const int64_t row = b / nblk;
    const uint32_t j = (uint32_t)(b - row * nblk);
    const uint32_t t = (uint32_t)(row % T);
    const uint32_t i = draw0 + (uint32_t)(row / T);
    float4 v;
    normal4(j, t, i, stream, k0, k1, v.x, v.y, v.z, v.w);
    reinterpret_cast<float4*>(out)[b] = v;
  }
}

static int grid_for(int64_t work, int threads) {
  int64_t g = (work + threads - 1) / threads;
  if (g > 65536) g = 65536;  // grid-stride loops cover the rest
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_philox_raw(const uint32_t* ctr, uint32_t* out, int64_t n, uint64_t seed,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(philox_raw_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, ctr, out, n,
                     (uint32_t)seed, (uint32_t)(seed >> 32));
  return hipGetLastError();
}

hipError_t launch_noise_fill(float* out, int64_t ndraw, int64_t T, int64_t N, uint32_t draw0,
                             uint32_t stream, uint64_t seed, hipStream_t s) {
  const int64_t nblk = N / 4;
  const int64_t total = ndraw * T * nblk;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(noise_fill_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, out, ndraw,
                     T, nblk, draw0, stream, (uint32_t)seed, (uint32_t)(seed >> 32));
  return hipGetLastError();
}

}  // namespace dust
