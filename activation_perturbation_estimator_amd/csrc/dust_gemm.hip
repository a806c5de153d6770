// dust_gemm.hip -- the weight gradient G_W = sum_t g_t x_t^T on the matrix cores.
//
// Paper digest, section 2.2: the error estimate's outer product with the layer
// input gives the weight gradient, in the same form as backprop.  As a matrix
// product, G[n][k] = sum_t g[t][n] X[t][k], contracting over the token axis,
// which is the slow axis of both row-major operands.
//
// Precision: g is fp32 and the product must keep ~fp32 accuracy.  Each fp32
// value v is split into two bf16 values hi = bf16(v), lo = bf16(v - hi) with
// |v - hi - lo| <= 2^-17 |v|, and the products run on the bf16 MFMA units with
// fp32 accumulation: g_hi X + g_lo X for bf16 X (exact in bf16), plus
// g_hi X_lo for fp32 X.  Every bf16 x bf16 product is exact in fp32.
//
// Tiling: a workgroup (4 waves) owns a 128 x 128 tile of G over one token range
// (split-K over tokens so that the grid fills the 256 CUs).  Per 32-token step
// the fp32 g tile is read with each lane walking 8 tokens of one column (every
// load instruction reads 64 consecutive floats), split to hi/lo and written to
// LDS transposed (token-contiguous), which is the operand layout of
// v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 and the 8 consecutive
// contraction indices 8*(l/32) .. 8*(l/32)+7.  Each wave computes 64 x 64 of
// the tile as 2 x 2 MFMA blocks.  Partial tiles of the token splits are summed
// in a fixed order by a second kernel, so results are deterministic.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kBM = 128;      // rows of G (layer outputs) per workgroup
constexpr int kBN = 128;      // columns of G (layer inputs) per workgroup
constexpr int kBT = 32;       // tokens per step
constexpr int kLdsRow = kBT + 8;  // bf16 per LDS row (80 bytes: 16-byte aligned, staggered banks)

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = bf16_bits(v);
  const float rest = v - __uint_as_float(hi << 16);  // exact
  lo = bf16_bits(rest);
}

template <bool kXF32>
__global__ void __launch_bounds__(256)
outer_sum_kernel(const float* __restrict__ g, const void* __restrict__ Xv, int64_t T, int64_t M,
                 int64_t Nd, int64_t t_per_split, float* __restrict__ out, int64_t split_stride) {
  __shared__ __attribute__((aligned(16))) uint16_t Ah[kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Al[kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bh[kBN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bl[kXF32 ? kBN * kLdsRow : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t tiles_m = (M + kBM - 1) / kBM;
  const int64_t m0 = (blockIdx.x % tiles_m) * kBM;
  const int64_t n0 = (blockIdx.x / tiles_m) * kBN;
  const int64_t t_begin = (int64_t)blockIdx.y * t_per_split;
  int64_t t_end = t_begin + t_per_split;
  if (t_end > T) t_end = T;

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int row = tid & 127;    // staging: this thread's row of the A / B tile
  const int qbase = tid >> 7;   // token groups qbase and qbase + 2 (8 tokens each)

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kBT) {
    // ---- stage g (A operand), transposed to token-contiguous rows ----
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = qbase + 2 * qq;
      const int64_t m = m0 + row;
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t tt = t0 + 8 * q + e;
        const float v = (tt < t_end && m < M) ? g[tt * M + m] : 0.f;
        split_bf16(v, hi[e], lo[e]);
      }
      uint4 ph, pl;
      ph.x = hi[0] | (hi[1] << 16); ph.y = hi[2] | (hi[3] << 16);
      ph.z = hi[4] | (hi[5] << 16); ph.w = hi[6] | (hi[7] << 16);
      pl.x = lo[0] | (lo[1] << 16); pl.y = lo[2] | (lo[3] << 16);
      pl.z = lo[4] | (lo[5] << 16); pl.w = lo[6] | (lo[7] << 16);
      *reinterpret_cast<uint4*>(&Ah[row * kLdsRow + 8 * q]) = ph;
      *reinterpret_cast<uint4*>(&Al[row * kLdsRow + 8 * q]) = pl;
    }
    // ---- stage X (B operand) ----
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = qbase + 2 * qq;
      const int64_t n = n0 + row;
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t tt = t0 + 8 * q + e;
        const bool ok = (tt < t_end && n < Nd);
        if constexpr (kXF32) {
          const float v = ok ? reinterpret_cast<const float*>(Xv)[tt * Nd + n] : 0.f;
          split_bf16(v, hi[e], lo[e]);
        } else {
          hi[e] = ok ? (uint32_t)reinterpret_cast<const uint16_t*>(Xv)[tt * Nd + n] : 0u;
          lo[e] = 0u;
        }
      }
      uint4 ph;
      ph.x = hi[0] | (hi[1] << 16); ph.y = hi[2] | (hi[3] << 16);
      ph.z = hi[4] | (hi[5] << 16); ph.w = hi[6] | (hi[7] << 16);
      *reinterpret_cast<uint4*>(&Bh[row * kLdsRow + 8 * q]) = ph;
      if constexpr (kXF32) {
        uint4 pl;
        pl.x = lo[0] | (lo[1] << 16); pl.y = lo[2] | (lo[3] << 16);
        pl.z = lo[4] | (lo[5] << 16); pl.w = lo[6] | (lo[7] << 16);
        *reinterpret_cast<uint4*>(&Bl[row * kLdsRow + 8 * q]) = pl;
      }
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < kBT; kk += 16) {
      const int koff = kk + 8 * (lane >> 5);
      bf16x8_t ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = wm * 64 + mb * 32 + (lane & 31);
        ah[mb] = *reinterpret_cast<const bf16x8_t*>(&Ah[r * kLdsRow + koff]);
        al[mb] = *reinterpret_cast<const bf16x8_t*>(&Al[r * kLdsRow + koff]);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int r = wn * 64 + nb * 32 + (lane & 31);
        bh[nb] = *reinterpret_cast<const bf16x8_t*>(&Bh[r * kLdsRow + koff]);
        if constexpr (kXF32) bl[nb] = *reinterpret_cast<const bf16x8_t*>(&Bl[r * kLdsRow + koff]);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh[nb], acc[mb][nb], 0, 0, 0);
          if constexpr (kXF32)
            acc[mb][nb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl[nb], acc[mb][nb], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // ---- write the 64 x 64 wave tile: register r of block (mb, nb) holds
  // row 8*(r/4) + 4*(lane/32) + r%4, column lane%32 ----
  float* o = out + (int64_t)blockIdx.y * split_stride;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + nb * 32 + (lane & 31);
        if (m < M && n < Nd) o[m * Nd + n] = acc[mb][nb][r];
      }
}

// G[e] = sum_s part[s][e] in split order.
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* __restrict__ part,
                                                           int64_t nsplit, int64_t n,
                                                           float* __restrict__ G) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    float s = part[e];
    for (int64_t q = 1; q < nsplit; ++q) s += part[q * n + e];
    G[e] = s;
  }
}

struct SplitPlan {
  int64_t tiles;
  int64_t nsplit;
  int64_t t_per_split;
};

static SplitPlan plan_splits(int64_t T, int64_t M, int64_t Nd) {
  SplitPlan p;
  p.tiles = ((M + kBM - 1) / kBM) * ((Nd + kBN - 1) / kBN);
  // Aim for >= 1024 workgroups (4 per CU) with >= 512 tokens per split.
  int64_t want = (1024 + p.tiles - 1) / p.tiles;
  int64_t cap = (T + 511) / 512;
  if (cap < 1) cap = 1;
  p.nsplit = want < cap ? want : cap;
  if (p.nsplit < 1) p.nsplit = 1;
  int64_t per = (T + p.nsplit - 1) / p.nsplit;
  per = (per + kBT - 1) / kBT * kBT;
  p.t_per_split = per > 0 ? per : kBT;
  p.nsplit = (T + p.t_per_split - 1) / p.t_per_split;
  if (p.nsplit < 1) p.nsplit = 1;
  return p;
}

size_t outer_sum_workspace_bytes(int64_t T, int64_t N, int64_t d) {
  const SplitPlan p = plan_splits(T, N, d);
  if (p.nsplit <= 1) return 0;
  return (size_t)p.nsplit * (size_t)N * (size_t)d * sizeof(float);
}

hipError_t launch_outer_sum(const float* g, const void* X, bool x_bf16, int64_t T, int64_t N,
                            int64_t d, float* G, void* workspace, hipStream_t s) {
  const SplitPlan p = plan_splits(T, N, d);
  float* out = (p.nsplit > 1) ? reinterpret_cast<float*>(workspace) : G;
  const int64_t split_stride = N * d;
  dim3 grid((uint32_t)p.tiles, (uint32_t)p.nsplit);
  if (x_bf16)
    hipLaunchKernelGGL(outer_sum_kernel<false>, grid, dim3(256), 0, s, g, X, T, N, d,
                       p.t_per_split, out, split_stride);
  else
    hipLaunchKernelGGL(outer_sum_kernel<true>, grid, dim3(256), 0, s, g, X, T, N, d,
                       p.t_per_split, out, split_stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit <= 1) return e;
  const int64_t n = N * d;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, out, p.nsplit,
                     n, G);
  return hipGetLastError();
}

}  // namespace dust
