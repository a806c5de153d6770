// dust_scan.hip -- centring and the discounted reward scan, both on [K,T]
// arrays (draw-major, token-contiguous), plus the target range check.
//
// Paper digest, section 2.2 (credit assignment): token s scores a draw by its
// centred loss decrease c_s, and token t's reward is
//     r_t = sum_{s >= t} gamma^(s-t) c_s          (gamma = 0: the token's own c).
// The sum runs inside one sequence: causal attention cannot carry a token's
// perturbation into another sequence, so the scan restarts at every sequence
// boundary.  Centring is read as: subtract the mean over the K draws of the
// same token.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

// c[i,t] = mean_j x[j,t] - x[i,t].  One thread per token; the mean is summed in
// fp64 over the draws (fixed order), so the result does not depend on K's size
// beyond fp32 rounding of the output.  Memory-bound: 12 bytes per element.
// c may be x (the estimator centres in place), so neither pointer is restrict.
__global__ void __launch_bounds__(256) centre_kernel(const float* x, int64_t K, int64_t T,
                                                     float* c) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  double s = 0.0;
  for (int64_t i = 0; i < K; ++i) s += (double)x[i * T + t];
  const double mean = s / (double)K;
  for (int64_t i = 0; i < K; ++i) c[i * T + t] = (float)(mean - (double)x[i * T + t]);
}

// Segmented reverse scan r_t = c_t + gamma r_{t+1}.  One wave per (draw,
// sequence) job, the waves striding over the jobs; the sequence is walked from its end in tiles of 64 lanes x kE
// elements (kE = 32 covers a 2048-token sequence in one tile, so each wave
// issues all its loads at once).  Per tile: a coalesced load into LDS, a serial
// scan of each lane's kE elements with zero carry, a wave-wide suffix scan of
// the lanes' affine maps x -> A + B x (B = gamma^kE), and a second serial pass
// with the true carry.
// r may be c (the estimator scans in place), so neither pointer is restrict.
template <int kE>
__global__ void __launch_bounds__(256) reward_scan_kernel(const float* c, int64_t K, int64_t T,
                                                          int64_t L, float gamma, float* r) {
  constexpr int kTile = 64 * kE;
  __shared__ float buf[4][64 * (kE + 1)];  // rows of kE + 1: conflict-free lane-major reads
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nseg = T / L;
  float* sb = buf[wave];
  float gE = 1.f;
#pragma unroll
  for (int k = 0; k < kE; ++k) gE *= gamma;

  // Waves stride over the jobs; a wave leaves on its own (no workgroup barrier).
  const int64_t njobs = K * nseg;
  for (int64_t job = (int64_t)blockIdx.x * 4 + wave; job < njobs; job += (int64_t)gridDim.x * 4) {
    const int64_t i = job / nseg;
    const int64_t seg = job - i * nseg;
    const int64_t base = i * T + seg * L;
    float carry = 0.f;  // r at the first position after the current tile
    for (int64_t tile_end = L; tile_end > 0; tile_end -= kTile) {
      const int64_t tile_start = tile_end > kTile ? tile_end - kTile : 0;
      const int n = (int)(tile_end - tile_start);
      const int off = kTile - n;  // a short tile is aligned to its end
#pragma unroll
      for (int k = 0; k < kE; ++k) {
        const int e = k * 64 + lane;
        const float v = (e >= off) ? c[base + tile_start + (e - off)] : 0.f;
        sb[(e / kE) * (kE + 1) + (e % kE)] = v;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
      float xv[kE];
#pragma unroll
      for (int k = 0; k < kE; ++k) xv[k] = sb[lane * (kE + 1) + k];
      // pass 1: this lane's chunk with zero carry
      float A = 0.f;
#pragma unroll
      for (int k = kE - 1; k >= 0; --k) A = fmaf(gamma, A, xv[k]);
      float B = gE;
      // suffix scan over lanes: (A,B) o (A',B') = (A + B A', B B')
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        const float An = __shfl_down(A, sh, 64);
        const float Bn = __shfl_down(B, sh, 64);
        if (lane + sh < 64) {
          A = fmaf(B, An, A);
          B = B * Bn;
        }
      }
      const float R = fmaf(B, carry, A);            // r at this lane's first element
      float cin = __shfl_down(R, 1, 64);            // r at the next lane's first element
      if (lane == 63) cin = carry;
      // pass 2: true values
      float rho = cin;
#pragma unroll
      for (int k = kE - 1; k >= 0; --k) {
        rho = fmaf(gamma, rho, xv[k]);
        sb[lane * (kE + 1) + k] = rho;
      }
      carry = lane_value(R, 0);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int k = 0; k < kE; ++k) {
        const int e = k * 64 + lane;
        if (e >= off) r[base + tile_start + (e - off)] = sb[(e / kE) * (kE + 1) + (e % kE)];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
}

__global__ void zero_flag_kernel(int32_t* flag) { *flag = 0; }

__global__ void __launch_bounds__(256) check_targets_kernel(const int32_t* __restrict__ y,
                                                            int64_t T, int64_t V,
                                                            int32_t* __restrict__ flag) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += stride)
    if (y[t] < 0 || (int64_t)y[t] >= V) *flag = 1;
}

hipError_t launch_centre(const float* x, int64_t K, int64_t T, float* c, hipStream_t s) {
  if (T == 0 || K == 0) return hipSuccess;
  hipLaunchKernelGGL(centre_kernel, dim3((uint32_t)((T + 255) / 256)), dim3(256), 0, s, x, K, T,
                     c);
  return hipGetLastError();
}

hipError_t launch_reward_scan(const float* c, int64_t K, int64_t T, int64_t L, float gamma,
                              float* r, hipStream_t s) {
  const int64_t jobs = K * (T / L);
  if (jobs == 0) return hipSuccess;
  const dim3 grid((uint32_t)((jobs + 3) / 4 < 65536 ? (jobs + 3) / 4 : 65536));
  if (L >= 2048)
    hipLaunchKernelGGL(reward_scan_kernel<32>, grid, dim3(256), 0, s, c, K, T, L, gamma, r);
  else if (L >= 512)
    hipLaunchKernelGGL(reward_scan_kernel<16>, grid, dim3(256), 0, s, c, K, T, L, gamma, r);
  else
    hipLaunchKernelGGL(reward_scan_kernel<8>, grid, dim3(256), 0, s, c, K, T, L, gamma, r);
  return hipGetLastError();
}

hipError_t launch_check_targets(const int32_t* targets, int64_t T, int64_t V, int32_t* flag,
                                hipStream_t s) {
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(1), 0, s, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  int64_t g = (T + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(check_targets_kernel, dim3((uint32_t)g), dim3(256), 0, s, targets, T, V,
                     flag);
  return hipGetLastError();
}

}  // namespace dust
