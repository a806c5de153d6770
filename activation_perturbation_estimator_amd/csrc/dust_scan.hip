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
#include <mutex>

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
// 8192 elements, 32 consecutive ones (a chunk) per thread:
//   - L <= 8192: a tile is m = floor(8192/L) whole segments (the tile's last
//     element ends a segment, so nothing flows in from the right);
//   - L > 8192: a workgroup walks one segment in tiles from its end, carrying
//     r of each tile's first element into the tile to its left.
// Per tile: coalesced loads; each thread reduces its chunk to an affine map
// r_first = A + B r_after (B = 0 when a segment ends inside it); a suffix scan
// of the maps (inside each wave by DPP lane shifts, across the 4 waves through
// LDS) gives every thread the r that follows its chunk; a second pass over the
// chunk writes r; stores.  The whole tile is read before any of it is written,
// so r may be c.  Long chunks keep the wave count low: waves start at a few
// thousand per microsecond, and with 8 elements per thread the 32 MiB of the
// hidden-layer workload spent as long starting waves (and waiting at the
// barrier for a workgroup's last ones) as moving data.
// gamma^m underflows to 0 in fp32 for long distances (0.9^2048): harmless.
constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanE = 32;
constexpr int kScanTile = kScanThreads * kScanE;

// Maps compose as (A, B) o (A', B') = (A + B A', B B'): the left one is applied
// after the right one.  compose_dpp<ctrl, rows>: each lane of the enabled rows
// takes the map of the lane the DPP control names (the identity (0, 1) where
// there is none) and composes it on the right of its own.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void compose_dpp(float& A, float& B) {
  const float Ap = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(A), kCtrl, kRowMask,
                                                              0xf, false));
  const float Bp = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f),
                                                              __float_as_int(B), kCtrl, kRowMask,
                                                              0xf, false));
  A = fmaf(B, Ap, A);
  B *= Bp;
}

// Inclusive scan of the maps over the lanes of a wave, lane 0 first: lane l
// ends with f_l o f_(l-1) o ... o f_0.  Shifts by 1, 2, 4 and 8 lanes inside
// each row of 16, then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31
// into rows 2 and 3.
__device__ __forceinline__ void wave_scan_maps(float& A, float& B) {
  compose_dpp<0x111, 0xf>(A, B);  // row_shr:1
  compose_dpp<0x112, 0xf>(A, B);  // row_shr:2
  compose_dpp<0x114, 0xf>(A, B);  // row_shr:4
  compose_dpp<0x118, 0xf>(A, B);  // row_shr:8
  compose_dpp<0x142, 0xa>(A, B);  // row_bcast:15
  compose_dpp<0x143, 0xc>(A, B);  // row_bcast:31
}

// Tiles go through LDS, chunk by chunk ([chunk][36] floats: 16-byte aligned
// rows whose starts fall on different banks for the 16 lanes of a read
// phase), so that the global loads and stores stay coalesced.
// kVec: every tile starts at a multiple of 4 elements of 16-byte aligned
// arrays (L % 4 == 0), and its global accesses are 16 bytes per lane.
// P: the integer type of positions within a segment (int32_t when L < 2^30).
template <bool kVec, typename P>
__global__ void __launch_bounds__(kScanThreads) reward_scan_kernel(const float* c, int64_t nseg,
                                                                   int64_t L, float gamma,
                                                                   float* r) {
  constexpr int kRow = kScanE + 4;
  __shared__ __attribute__((aligned(16))) float buf[kScanThreads * kRow];
  __shared__ float wa[kScanWaves], wb[kScanWaves], tile_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The wave's chunks run right to left over its lanes, so that the suffix
  // scan over the wave's chunks is a prefix scan over its lanes.
  const int q = wave * 64 + (63 - lane);  // this thread's chunk of the tile
  const int j0 = q * kScanE;
  const bool long_seg = L > kScanTile;
  const int64_t m = long_seg ? 1 : kScanTile / L;  // segments per tile
  const int64_t njobs = (nseg + m - 1) / m;

  // One tile: elements [base, base + n); the tile's last element ends a
  // segment unless carry_in flows from a tile to its right.  The element at
  // local index j ends a segment when (pos0 + j) % L == L - 1.
  auto scan_tile = [&](int64_t base, int n, int64_t pos0, float carry_in) -> float {
    float xv[kScanE];
    if constexpr (kVec) {  // n is a multiple of 4
#pragma unroll
      for (int h = 0; h < kScanE / 4; ++h) {
        const int j = 4 * (h * kScanThreads + tid);
        if (j < n)
          *reinterpret_cast<float4*>(buf + (j / kScanE) * kRow + j % kScanE) =
              *reinterpret_cast<const float4*>(c + base + j);
      }
    } else {
#pragma unroll 8
      for (int k = 0; k < kScanE; ++k) {
        const int j = k * kScanThreads + tid;
        if (j < n) buf[(j / kScanE) * kRow + (j % kScanE)] = c[base + j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kScanE / 4; ++h) {  // past n: not used
      const float4 v = *reinterpret_cast<const float4*>(buf + q * kRow + 4 * h);
      xv[4 * h] = v.x; xv[4 * h + 1] = v.y; xv[4 * h + 2] = v.z; xv[4 * h + 3] = v.w;
    }
    // position in its segment of the chunk's last element; both passes walk
    // the chunk backwards, stepping the position down with it, and the element
    // at position L - 1 ends a segment
    const P Lp = (P)L;
    const P plast = (P)((pos0 + j0 + kScanE - 1) % L);
    // pass 1: this chunk's map (identity for elements past the tile)
    float A = 0.f, B = 1.f;
    P p = plast;
#pragma unroll
    for (int k = kScanE - 1; k >= 0; --k) {
      if (j0 + k < n) {
        if (p == Lp - 1) {
          A = xv[k];
          B = 0.f;
        } else {
          A = fmaf(gamma, A, xv[k]);
          B *= gamma;
        }
      }
      p = p == 0 ? Lp - 1 : p - 1;
    }
    wave_scan_maps(A, B);  // lane l: the wave's chunks from its right end to its own
    if (lane == 63) {      // the whole wave
      wa[wave] = A;
      wb[wave] = B;
    }
    __syncthreads();
    // r after this wave's last element: the waves to the right applied to the
    // tile's carry, in order from the rightmost
    float X = carry_in;
    for (int w = kScanWaves - 1; w > wave; --w) X = fmaf(wb[w], X, wa[w]);
    const float R = fmaf(B, X, A);  // r at this chunk's first element
    // r after this chunk: R of the chunk to its right (lane - 1), X for lane 0
    const float cin = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(X),
                                                                 __float_as_int(R), 0x138, 0xf,
                                                                 0xf, false));  // wave_shr:1
    if (q == 0) tile_carry = R;
    // pass 2: the true values
    float rho = cin;
    p = plast;
#pragma unroll
    for (int k = kScanE - 1; k >= 0; --k) {
      if (j0 + k < n) {  // elements past the tile's end do not exist
        rho = p == Lp - 1 ? xv[k] : fmaf(gamma, rho, xv[k]);
        xv[k] = rho;
      }
      p = p == 0 ? Lp - 1 : p - 1;
    }
#pragma unroll
    for (int h = 0; h < kScanE / 4; ++h)
      *reinterpret_cast<float4*>(buf + q * kRow + 4 * h) =
          make_float4(xv[4 * h], xv[4 * h + 1], xv[4 * h + 2], xv[4 * h + 3]);
    __syncthreads();
    if constexpr (kVec) {
#pragma unroll
      for (int h = 0; h < kScanE / 4; ++h) {
        const int j = 4 * (h * kScanThreads + tid);
        if (j < n)
          *reinterpret_cast<float4*>(r + base + j) =
              *reinterpret_cast<const float4*>(buf + (j / kScanE) * kRow + j % kScanE);
      }
    } else {
#pragma unroll 8
      for (int k = 0; k < kScanE; ++k) {
        const int j = k * kScanThreads + tid;
        if (j < n) r[base + j] = buf[(j / kScanE) * kRow + (j % kScanE)];
      }
    }
    const float out = tile_carry;
    __syncthreads();  // buf, wa, wb and tile_carry are reused by the next tile
    return out;
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

// The same scan for segments of kWaveBlock to kScanTile elements, one wave per
// segment and no LDS or barriers: the wave walks its segment from the end in
// blocks of 64 x 4 elements (lane 0 holds the block's last 4 elements, lane 63
// its first 4: every load and store of a block is one contiguous 1 KiB), in
// groups of kWaveDepth blocks held in registers.  Per block: each lane reduces
// its 4 elements to a map r_first = A + gamma^4 r_after, the wave's maps are
// scanned (wave_scan_maps), and r after the block comes in as the carry of the
// block to its right (0 at the segment's end, where r = c).  A group's loads
// are all issued at once, and the next group's loads go out before this
// group's stores: loads and stores may complete in any order relative to each
// other, so a wave can only wait for all of its memory operations, and this
// order makes one wait cover both.  Each wave depends on nothing but its own
// data, so waves whose loads arrive early store while others still load, as in
// a copy; the tile kernel above reads its whole tile (and waits at barriers for
// all of its waves) before it writes any of it.
constexpr int kWaveE = 4;
constexpr int kWaveBlock = 64 * kWaveE;
constexpr int kWaveDepth = 8;  // blocks per group: seq_len 2048 is one group
constexpr int kWaveSegs = 1;   // waves (segments) per workgroup
constexpr int kNonTemporal = 2;  // cache-policy bits of a buffer store: nt

typedef unsigned int scan_u32x4_t __attribute__((ext_vector_type(4)));
typedef float scan_f32x4_t __attribute__((ext_vector_type(4)));

// kDirect (L % kWaveBlock == 0 and 16-byte accesses): every lane's elements
// exist in every block, so loads and stores are plain and unconditional.
// Otherwise they go through buffer resources spanning the wave's segment:
// the elements before the segment's start, which only the first block has,
// read as zeros and are not written, with no branch and no mask (a masked
// store would make each store wait for the previous one).  The stores are
// non-temporal (nothing reads r again in this kernel): at the hidden-layer
// workload that takes a launch from 6.5 to 5.1 us.
template <bool kDirect, bool kVec>
__global__ void __launch_bounds__(64 * kWaveSegs) reward_scan_wave_kernel(const float* c,
                                                                         int64_t nseg, int64_t L,
                                                                         float gamma, float* r) {
  const int lane = threadIdx.x & 63;
  const int64_t seg =
      ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kWaveSegs + (threadIdx.x >> 6);
  if (seg >= nseg) return;  // whole wave
  const int64_t nblk = (L + kWaveBlock - 1) / kWaveBlock;
  const float g2 = gamma * gamma, g4 = g2 * g2;
  const int64_t s0 = seg * L;
  // this lane's elements of block b: [e0 - b kWaveBlock, + 4) of the segment,
  // negative indices past its start
  const int e0 = (int)L - kWaveE * (lane + 1);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(c + s0), 0, (int)(L * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc(r + s0, 0, (int)(L * 4), 0x00020000);
  auto load_group = [&](int64_t b0, float(&x)[kWaveDepth][kWaveE]) {
#pragma unroll
    for (int u = 0; u < kWaveDepth; ++u) {
      if (b0 + u < nblk) {
        const int e = e0 - (int)(b0 + u) * kWaveBlock;
        if constexpr (kDirect) {
          const float4 q = *reinterpret_cast<const float4*>(c + s0 + e);
          x[u][0] = q.x;
          x[u][1] = q.y;
          x[u][2] = q.z;
          x[u][3] = q.w;
        } else if constexpr (kVec) {  // L % 4 == 0: a lane's 4 elements all exist or none does
          const scan_u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(rc, 4 * e, 0, 0);
#pragma unroll
          for (int k = 0; k < kWaveE; ++k) x[u][k] = __uint_as_float(q[k]);
        } else {
#pragma unroll
          for (int k = 0; k < kWaveE; ++k)
            x[u][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, 4 * (e + k), 0, 0));
        }
      }
    }
  };
  float carry = 0.f;  // r after the block: nothing after the segment's end
  auto scan_group = [&](int64_t b0, float(&x)[kWaveDepth][kWaveE]) {
#pragma unroll
    for (int u = 0; u < kWaveDepth; ++u) {
      if (b0 + u < nblk) {
        float(&v)[kWaveE] = x[u];
        float A = 0.f, B = g4;
#pragma unroll
        for (int k = kWaveE - 1; k >= 0; --k) A = fmaf(gamma, A, v[k]);
        wave_scan_maps(A, B);  // lane l: the block's lanes 0..l, right to left
        const float R = fmaf(B, carry, A);  // r at this lane's first element
        // r after this lane's elements: R of lane - 1, the carry for lane 0
        float rho = __int_as_float(__builtin_amdgcn_update_dpp(
            __float_as_int(carry), __float_as_int(R), 0x138, 0xf, 0xf, false));  // wave_shr:1
#pragma unroll
        for (int k = kWaveE - 1; k >= 0; --k) {
          rho = fmaf(gamma, rho, v[k]);
          v[k] = rho;
        }
        carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(R), 63));
      }
    }
  };
  auto store_group = [&](int64_t b0, const float(&x)[kWaveDepth][kWaveE]) {
#pragma unroll
    for (int u = 0; u < kWaveDepth; ++u) {
      if (b0 + u < nblk) {
        const int e = e0 - (int)(b0 + u) * kWaveBlock;
        if constexpr (kDirect) {
          const scan_f32x4_t q = {x[u][0], x[u][1], x[u][2], x[u][3]};
          __builtin_nontemporal_store(q, reinterpret_cast<scan_f32x4_t*>(r + s0 + e));
        } else if constexpr (kVec) {
          const scan_u32x4_t q = {__float_as_uint(x[u][0]), __float_as_uint(x[u][1]),
                                  __float_as_uint(x[u][2]), __float_as_uint(x[u][3])};
          __builtin_amdgcn_raw_buffer_store_b128(q, rr, 4 * e, 0, kNonTemporal);
        } else {
#pragma unroll
          for (int k = 0; k < kWaveE; ++k)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[u][k]), rr, 4 * (e + k), 0,
                                                 kNonTemporal);
        }
      }
    }
  };
  float x[kWaveDepth][kWaveE], y[kWaveDepth][kWaveE];
  load_group(0, x);
  for (int64_t b0 = 0; b0 < nblk; b0 += 2 * kWaveDepth) {
    scan_group(b0, x);
    if (b0 + kWaveDepth < nblk) load_group(b0 + kWaveDepth, y);
    store_group(b0, x);
    if (b0 + kWaveDepth >= nblk) break;
    scan_group(b0 + kWaveDepth, y);
    if (b0 + 2 * kWaveDepth < nblk) load_group(b0 + 2 * kWaveDepth, x);
    store_group(b0 + kWaveDepth, y);
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
  const bool vec = L % 4 == 0 && reinterpret_cast<uintptr_t>(c) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(r) % 16 == 0;
  if (L >= kWaveBlock && L <= kScanTile) {  // one wave per segment
    // groups <= 2^32 (K T <= 2^40); grid x times the block stays below 2^32,
    // and the grid holds fewer than gy groups more than there are
    const int64_t groups = (nseg + kWaveSegs - 1) / kWaveSegs;
    const int64_t gy = (groups + ((int64_t)1 << 24) - 1) >> 24;
    const dim3 grid((uint32_t)((groups + gy - 1) / gy), (uint32_t)gy);
    const dim3 block(64 * kWaveSegs);
    if (vec && L % kWaveBlock == 0)
      hipLaunchKernelGGL((reward_scan_wave_kernel<true, true>), grid, block, 0, s, c, nseg, L,
                         gamma, r);
    else if (vec)
      hipLaunchKernelGGL((reward_scan_wave_kernel<false, true>), grid, block, 0, s, c, nseg, L,
                         gamma, r);
    else
      hipLaunchKernelGGL((reward_scan_wave_kernel<false, false>), grid, block, 0, s, c, nseg, L,
                         gamma, r);
    return hipGetLastError();
  }
  const int64_t m = L > kScanTile ? 1 : kScanTile / L;
  const int64_t njobs = (nseg + m - 1) / m;
  const dim3 grid((uint32_t)(njobs < 65536 ? njobs : 65536));
  const bool narrow = L < ((int64_t)1 << 30);
  if (vec && narrow)
    hipLaunchKernelGGL((reward_scan_kernel<true, int32_t>), grid, dim3(kScanThreads), 0, s, c,
                       nseg, L, gamma, r);
  else if (vec)
    hipLaunchKernelGGL((reward_scan_kernel<true, int64_t>), grid, dim3(kScanThreads), 0, s, c,
                       nseg, L, gamma, r);
  else if (narrow)
    hipLaunchKernelGGL((reward_scan_kernel<false, int32_t>), grid, dim3(kScanThreads), 0, s, c,
                       nseg, L, gamma, r);
  else
    hipLaunchKernelGGL((reward_scan_kernel<false, int64_t>), grid, dim3(kScanThreads), 0, s, c,
                       nseg, L, gamma, r);
  return hipGetLastError();
}

// The flag of dust_check_targets calls that pass none: one int32 per GPU, held
// until the process ends.  Host code takes each device's address of it once,
// with hipGetSymbolAddress, and passes that to the kernels.
static __device__ int32_t check_flag;

namespace {
constexpr int kMaxFlagDevices = 64;
std::mutex g_flag_mutex;
int32_t* g_flag_ptr[kMaxFlagDevices] = {};
}  // namespace

hipError_t check_targets_own_flag(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxFlagDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_flag_mutex);
  if (g_flag_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flag));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_flag_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_flag_ptr[dev];
  return hipSuccess;
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
