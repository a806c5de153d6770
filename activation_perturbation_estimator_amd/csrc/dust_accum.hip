// dust_accum.hip -- the error estimate with regenerated noise.
//
// Paper digest, section 2.2: averaging the reward-weighted noise over K draws
// gives the output-error estimate
//     g_t = -(1/(K sigma)) sum_i r^(i)_t a^(i)_t .
// The noise a^(i)_t is never read from memory: each lane regenerates its
// columns' Philox blocks from (token, column/4, draw, stream), so the kernel
// moves only r (4 bytes per token-draw) and g (4 bytes per token-column).
//
// One workgroup per token (W waves split the columns as in the head kernels);
// the draws run in a loop with the token's row of g in registers.  The rewards
// of 64 draws are fetched at once (lane l holds draw i0+l), one block of 64
// ahead of their use, and broadcast one at a time with v_readlane.
#include "dust_device.hpp"
#include "dust_gemm16.hpp"
#include "dust_launch.hpp"

namespace dust {

template <int kNB, int kW>
__global__ void __launch_bounds__(64 * kW)
error_estimate_kernel(const float* __restrict__ r, int64_t K, int64_t T, int64_t N, float scale,
                      uint32_t stream, uint32_t draw0, uint32_t k0, uint32_t k1,
                      float* __restrict__ g_hat, Gemm16Out op) {
  constexpr int kCols = 4 * kNB;
  __shared__ float red[3 * kW];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = producer_token(blockIdx.x, T);
  const int64_t nblk = N >> 2;

  float acc[kCols];
#pragma unroll
  for (int q = 0; q < kCols; ++q) acc[q] = 0.f;

  float r_next = (lane < K) ? r[(int64_t)lane * T + t] : 0.f;
  float r_vec = 0.f;
  for (int64_t i = 0; i < K; ++i) {
    const int il = (int)(i & 63);
    if (il == 0) {
      r_vec = r_next;
      r_next = (i + 64 + lane < K) ? r[(i + 64 + lane) * T + t] : 0.f;
    }
    const float ri = lane_value(r_vec, il);
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const uint32_t j = (uint32_t)(b * 64 * kW + wave * 64 + lane);
      float a0, a1, a2, a3;
      normal4_scaled<true>(j, (uint32_t)t, draw0 + (uint32_t)i, stream, k0, k1, a0, a1, a2, a3);
      acc[4 * b] = fmaf(ri, a0, acc[4 * b]);
      acc[4 * b + 1] = fmaf(ri, a1, acc[4 * b + 1]);
      acc[4 * b + 2] = fmaf(ri, a2, acc[4 * b + 2]);
      acc[4 * b + 3] = fmaf(ri, a3, acc[4 * b + 3]);
    }
  }
  float* grow = g_hat + t * N;
#pragma unroll
  for (int q = 0; q < kCols; ++q) acc[q] *= scale;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int64_t j = (int64_t)b * 64 * kW + wave * 64 + lane;
    if (j < nblk)
      *reinterpret_cast<float4*>(grow + 4 * j) =
          make_float4(acc[4 * b], acc[4 * b + 1], acc[4 * b + 2], acc[4 * b + 3]);
  }
  // The fp16 operands of the G_W pass: this workgroup owns the token's whole row.
  if (op.g16 != nullptr) emit_operands<kNB, kW>(op, t, N, acc, red);
}

template <int kNB, int kW>
static hipError_t launch_ee_t(const float* r, int64_t K, int64_t T, int64_t N, float scale,
                              uint32_t stream, uint64_t seed, uint32_t draw0, float* g_hat,
                              const Gemm16Out& op, hipStream_t s) {
  hipLaunchKernelGGL((error_estimate_kernel<kNB, kW>), dim3((uint32_t)T), dim3(64 * kW), 0, s, r,
                     K, T, N, scale, stream, draw0, (uint32_t)seed, (uint32_t)(seed >> 32), g_hat,
                     op);
  return hipGetLastError();
}

hipError_t launch_error_estimate(const float* r, int64_t K, int64_t T, int64_t N, float sigma,
                                 uint32_t stream, uint64_t seed, uint32_t draw0, int64_t K_total,
                                 float* g_hat, const Gemm16Out& op, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // the noise comes divided by kBoxMullerScale (normal4_scaled)
  const float scale = -kBoxMullerScale / ((float)K_total * sigma);
  const HeadShape h = wide_shape(N);
#define DUST_EE_CASE(NB, W) \
  if (h.nb == NB && h.w == W)                                                                  \
    return launch_ee_t<NB, W>(r, K, T, N, scale, stream, seed, draw0, g_hat, op, s);
  DUST_EE_CASE(1, 1)
  DUST_EE_CASE(2, 1)
  DUST_EE_CASE(4, 1)
  DUST_EE_CASE(8, 1)
  DUST_EE_CASE(16, 1)
  DUST_EE_CASE(16, 2)
  DUST_EE_CASE(16, 4)
  DUST_EE_CASE(16, 8)
  DUST_EE_CASE(16, 16)
#undef DUST_EE_CASE
  return hipErrorInvalidValue;
}

}  // namespace dust
