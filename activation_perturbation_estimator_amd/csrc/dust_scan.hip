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

// Segmented reverse scan r_t = c_t + gamma r_{t+1} (r = c at a segment's last
// token) over the flattened [K,T] array, whose segments are its runs of L
// consecutive elements.  One workgroup of 256 threads scans a tile of up to
// 2048 elements, 8 consecutive ones per thread:
//   - L <= 2048: a tile is m = floor(2048/L) whole segments (the tile's last
//     element ends a segment, so nothing flows in from the right);
//   - L > 2048: a workgroup walks one segment in tiles from its end, carrying
//     r of each tile's first element into the tile to its left.
// Per tile: coalesced loads into LDS; each thread reduces its 8 elements to an
// affine map r_first = A + B r_after (B = 0 when a segment ends inside them); a
// suffix scan of the maps, by shuffles inside each wave and through LDS
// across the four waves, gives every thread the r that follows its elements;
// a second pass over the 8 elements writes r to LDS; coalesced stores.  The
// whole tile is read before any of it is written, so r may be c.
// gamma^m underflows to 0 in fp32 for long distances (0.9^2048): harmless.
constexpr int kScanThreads = 256;
constexpr int kScanE = 8;
constexpr int kScanTile = kScanThreads * kScanE;

// kVec: every tile starts at a multiple of 4 elements of 16-byte aligned
// arrays (L % 4 == 0), so each thread moves its 8 elements with two 16-byte
// loads and stores of its own, without the LDS staging.
template <bool kVec>
__global__ void __launch_bounds__(kScanThreads) reward_scan_kernel(const float* c, int64_t nseg,
                                                                   int64_t L, float gamma,
                                                                   float* r) {
  __shared__ float buf[kVec ? 1 : kScanThreads * (kScanE + 1)];
  __shared__ float wa[4], wb[4], tile_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool long_seg = L > kScanTile;
  const int64_t m = long_seg ? 1 : kScanTile / L;  // segments per tile
  const int64_t njobs = (nseg + m - 1) / m;

  // One tile: elements [base, base + n); the tile's last element ends a
  // segment unless carry_in flows from a tile to its right.  The element at
  // local index j ends a segment when (pos0 + j) % L == L - 1.
  auto scan_tile = [&](int64_t base, int n, int64_t pos0, float carry_in) -> float {
    const int j0 = tid * kScanE;
    float xv[kScanE];
    if constexpr (kVec) {
      // n is a multiple of 4: each half of the thread's 8 is wholly in or out
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j0 + 4 * h < n) v = *reinterpret_cast<const float4*>(c + base + j0 + 4 * h);
        xv[4 * h] = v.x; xv[4 * h + 1] = v.y; xv[4 * h + 2] = v.z; xv[4 * h + 3] = v.w;
      }
    } else {
      for (int q = 0; q < kScanE; ++q) {
        const int j = q * kScanThreads + tid;
        if (j < n) buf[(j / kScanE) * (kScanE + 1) + (j % kScanE)] = c[base + j];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kScanE; ++k) xv[k] = buf[tid * (kScanE + 1) + k];
    }
    bool end[kScanE];
    int64_t p = (pos0 + j0) % L;  // position of the first element in its segment
#pragma unroll
    for (int k = 0; k < kScanE; ++k) {
      end[k] = (p == L - 1);
      p = end[k] ? 0 : p + 1;
    }
    // pass 1: this thread's map (identity for elements past the tile)
    float A = 0.f, B = 1.f;
#pragma unroll
    for (int k = kScanE - 1; k >= 0; --k) {
      if (j0 + k < n) {
        if (end[k]) {
          A = xv[k];
          B = 0.f;
        } else {
          A = fmaf(gamma, A, xv[k]);
          B *= gamma;
        }
      }
    }
    // inclusive suffix scan of the maps inside the wave: (A,B) o (A',B')
    // = (A + B A', B B'), the left map applied after the right one
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const float An = __shfl_down(A, sh, 64);
      const float Bn = __shfl_down(B, sh, 64);
      if (lane + sh < 64) {
        A = fmaf(B, An, A);
        B *= Bn;
      }
    }
    if (lane == 0) {
      wa[wave] = A;
      wb[wave] = B;
    }
    __syncthreads();
    // r after this wave's last element: the waves to the right applied to the
    // tile's carry, in order from the rightmost
    float X = carry_in;
    for (int w = 3; w > wave; --w) X = fmaf(wb[w], X, wa[w]);
    const float R = fmaf(B, X, A);  // r at this thread's first element
    float cin = __shfl_down(R, 1, 64);
    if (lane == 63) cin = X;
    if (tid == 0) tile_carry = R;
    // pass 2: the true values
    float rho = cin;
#pragma unroll
    for (int k = kScanE - 1; k >= 0; --k) {
      if (j0 + k < n) {  // elements past the tile's end do not exist
        rho = end[k] ? xv[k] : fmaf(gamma, rho, xv[k]);
        xv[k] = rho;
      }
    }
    if constexpr (kVec) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (j0 + 4 * h < n)
          *reinterpret_cast<float4*>(r + base + j0 + 4 * h) =
              make_float4(xv[4 * h], xv[4 * h + 1], xv[4 * h + 2], xv[4 * h + 3]);
      __syncthreads();  // wa, wb and tile_carry are read before the next tile
      return tile_carry;
    } else {
#pragma unroll
      for (int k = 0; k < kScanE; ++k) buf[tid * (kScanE + 1) + k] = xv[k];
      __syncthreads();
      for (int q = 0; q < kScanE; ++q) {
        const int j = q * kScanThreads + tid;
        if (j < n) r[base + j] = buf[(j / kScanE) * (kScanE + 1) + (j % kScanE)];
      }
      const float out = tile_carry;
      __syncthreads();  // buf and tile_carry are reused by the next tile
      return out;
    }
  };

  for (int64_t job = blockIdx.x; job < njobs; job += gridDim.x) {
    if (!long_seg) {
      const int64_t seg0 = job * m;
      const int64_t segs = nseg - seg0 < m ? nseg - seg0 : m;
      scan_tile(seg0 * L, (int)(segs * L), 0, 0.f);
    } else {
      const int64_t sbase = job * L;
      float carry = 0.f;
      for (int64_t tile_end = L; tile_end > 0; tile_end -= kScanTile) {
        const int64_t tile_start = tile_end > kScanTile ? tile_end - kScanTile : 0;
        carry = scan_tile(sbase + tile_start, (int)(tile_end - tile_start), tile_start, carry);
      }
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
  const int64_t nseg = K * (T / L);
  if (nseg == 0) return hipSuccess;
  const int64_t m = L > kScanTile ? 1 : kScanTile / L;
  const int64_t njobs = (nseg + m - 1) / m;
  const dim3 grid((uint32_t)(njobs < 65536 ? njobs : 65536));
  const bool vec = L % 4 == 0 && reinterpret_cast<uintptr_t>(c) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(r) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(reward_scan_kernel<true>, grid, dim3(kScanThreads), 0, s, c, nseg, L,
                       gamma, r);
  else
    hipLaunchKernelGGL(reward_scan_kernel<false>, grid, dim3(kScanThreads), 0, s, c, nseg, L,
                       gamma, r);
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
