// dust_forward.hip -- the caller's perturbed forward of a hidden linear layer,
// y_t + sigma a^(i)_t with y_t = W x_t (paper digest, sections 2 and 2.1: every
// linear layer's output is jittered per token; laoyaoba analysis, mechanism
// section).  This is the step just before the error estimate of that layer:
// the noise comes from the same counters (token, column/4, draw, stream) that
// dust_linear_estimate regenerates, so the caller never stores it.
//
// Y[k, t, n] = sum_j X[t, j] W[n, j] + sigma a^(draw0 + k)_t[n],  k < ndraw.
// X [T, d] and W [N, d] are both contraction-contiguous (PyTorch Linear layout),
// which is the operand layout of v_mfma_f32_32x32x16_bf16 (lane l supplies row
// l%32 and 8 consecutive contraction indices), so tiles go global -> LDS as
// 16-byte rows without transposition.  fp32 operands are split into bf16
// hi + lo and multiplied as hi*hi + lo*hi + hi*lo (fp32 accumulation).
//
// The product is formed once per tile (operands double buffered in LDS); the
// epilogue stages the fp32 tile in LDS, half a tile at a time, so that each
// thread owns 4 consecutive columns of a token -- one Philox block -- and
// writes that item for every draw (sigma a added, 16-byte streaming stores).
// bf16 operands fit four workgroups per CU (40 KiB of LDS, <= 128 VGPRs), so
// the product of one tile overlaps the stores of others.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

typedef __attribute__((ext_vector_type(8))) __bf16 fbf16x8_t;
typedef __attribute__((ext_vector_type(16))) float ff32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 fbf16x2_t;
typedef __attribute__((ext_vector_type(2))) float ff32x2_t;
typedef __attribute__((ext_vector_type(4))) float ff32x4_t;
typedef unsigned int fu32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFM = 128;        // tokens per workgroup tile
constexpr int kFN = 128;        // output columns per workgroup tile
constexpr int kFK = 32;         // contraction step
constexpr int kFRow = kFK + 8;  // bf16 per LDS row (80 bytes)

__device__ __forceinline__ void fsplit2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const ff32x2_t v = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, fbf16x2_t));
  const ff32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, fbf16x2_t));
}

// Loads 8 consecutive contraction elements of one row as bf16 hi (and lo for
// fp32) from a buffer resource; out-of-range reads give zeros.
template <bool kF32>
__device__ __forceinline__ void load_row8(__amdgpu_buffer_rsrc_t rs, int byte_off, uint4& hi,
                                          uint4& lo) {
  if constexpr (kF32) {
    const fu32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
    const fu32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off + 16, 0, 0);
    fsplit2(__uint_as_float(a.x), __uint_as_float(a.y), hi.x, lo.x);
    fsplit2(__uint_as_float(a.z), __uint_as_float(a.w), hi.y, lo.y);
    fsplit2(__uint_as_float(b.x), __uint_as_float(b.y), hi.z, lo.z);
    fsplit2(__uint_as_float(b.z), __uint_as_float(b.w), hi.w, lo.w);
  } else {
    const fu32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
    hi = make_uint4(a.x, a.y, a.z, a.w);
    lo = make_uint4(0, 0, 0, 0);
  }
}

template <bool kF32>
__global__ void __launch_bounds__(256, kF32 ? 2 : 4)
perturbed_linear_kernel(const void* __restrict__ Xv, const void* __restrict__ Wv, int64_t T,
                        int64_t N, int64_t d, float sigma, uint32_t draw0, int64_t ndraw,
                        uint32_t stream, uint32_t k0, uint32_t k1, float* __restrict__ Y) {
  // operand stages during the product; the fp32 result tile afterwards
  extern __shared__ __attribute__((aligned(16))) uint16_t flds[];
  constexpr int kA = kFM * kFRow, kB = kFN * kFRow;
  constexpr int kStage = kF32 ? 2 * kA + 2 * kB : kA + kB;  // Ah, Bh (and Al, Bl) of one step

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t tiles_m = (T + kFM - 1) / kFM;
  const int64_t t0 = (blockIdx.x % tiles_m) * kFM;
  const int64_t n0 = (blockIdx.x / tiles_m) * kFN;
  constexpr int kEs = kF32 ? 4 : 2;  // bytes per operand element

  const int64_t rows_a = min((int64_t)kFM, T - t0), rows_b = min((int64_t)kFN, N - n0);
  const __amdgpu_buffer_rsrc_t xa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(Xv) + t0 * d * kEs), 0,
      (int)(rows_a * d * kEs), 0x00020000);
  const __amdgpu_buffer_rsrc_t wb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(Wv) + n0 * d * kEs), 0,
      (int)(rows_b * d * kEs), 0x00020000);

  ff32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Staging: 128 rows x 4 chunks of 8 contraction elements per operand, two
  // chunks per thread; the next step's chunks are fetched into registers
  // while the matrix cores work on the current LDS stage (double buffered).
  uint4 rah[2], ral[2], rbh[2], rbl[2];
  auto fetch = [&](int64_t kc) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int chunk = tid + 256 * h;
      const int row = chunk >> 2, c = chunk & 3;
      const int64_t kk = kc + 8 * c;
      // a row's chunk is either inside [0, d) or past its end (d % 8 == 0)
      if (kk < d) {
        load_row8<kF32>(xa, (int)((row * d + kk) * kEs), rah[h], ral[h]);
        load_row8<kF32>(wb, (int)((row * d + kk) * kEs), rbh[h], rbl[h]);
      } else {
        rah[h] = ral[h] = rbh[h] = rbl[h] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stash = [&](int stage) {
    uint16_t* Ah = flds + stage * kStage;
    uint16_t* Bh = Ah + (kF32 ? 2 : 1) * kA;
    uint16_t* Al = Ah + kA;  // fp32 only
    uint16_t* Bl = Bh + kB;  // fp32 only
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int chunk = tid + 256 * h;
      const int row = chunk >> 2, c = chunk & 3;
      *reinterpret_cast<uint4*>(Ah + row * kFRow + 8 * c) = rah[h];
      *reinterpret_cast<uint4*>(Bh + row * kFRow + 8 * c) = rbh[h];
      if constexpr (kF32) {
        *reinterpret_cast<uint4*>(Al + row * kFRow + 8 * c) = ral[h];
        *reinterpret_cast<uint4*>(Bl + row * kFRow + 8 * c) = rbl[h];
      }
    }
  };
  auto compute = [&](int stage) {
    const uint16_t* Ah = flds + stage * kStage;
    const uint16_t* Bh = Ah + (kF32 ? 2 : 1) * kA;
    const uint16_t* Al = Ah + kA;  // fp32 only
    const uint16_t* Bl = Bh + kB;  // fp32 only
#pragma unroll
    for (int ks = 0; ks < kFK; ks += 16) {
      const int koff = ks + 8 * (lane >> 5);
      fbf16x8_t ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ra = wm * 64 + q * 32 + (lane & 31);
        const int rb = wn * 64 + q * 32 + (lane & 31);
        ah[q] = *reinterpret_cast<const fbf16x8_t*>(Ah + ra * kFRow + koff);
        bh[q] = *reinterpret_cast<const fbf16x8_t*>(Bh + rb * kFRow + koff);
        if constexpr (kF32) {
          al[q] = *reinterpret_cast<const fbf16x8_t*>(Al + ra * kFRow + koff);
          bl[q] = *reinterpret_cast<const fbf16x8_t*>(Bl + rb * kFRow + koff);
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bh[b], acc[a][b], 0, 0, 0);
          if constexpr (kF32) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[a], bh[b], acc[a][b], 0, 0, 0);
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[a], bl[b], acc[a][b], 0, 0, 0);
          }
        }
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  const int nk = (int)((d + kFK - 1) / kFK);
  for (int i = 0; i < nk; ++i) {
    if (i + 1 < nk) fetch((int64_t)(i + 1) * kFK);
    compute(i & 1);
    if (i + 1 < nk) stash((i + 1) & 1);
    __syncthreads();
  }

  // Result tile through LDS as fp32 [64][132] (padded rows), one half of the
  // tokens at a time (the waves with wm = h own half h), so that the staging
  // needs no more LDS than the operand stages.  Each thread then owns 8 items
  // of the half (one token, 4 columns: one Philox block) and writes every draw
  // of an item before moving on, so only one item's product is live.
  constexpr int kYRow = kFN + 4;
  const float sigma_s = sigma * kBoxMullerScale;  // the noise comes divided by it
  float* tile = reinterpret_cast<float*>(flds);
  const int64_t nblk = N >> 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = wn * 64 + b * 32 + (lane & 31);
            tile[row * kYRow + col] = acc[a][b][r];
          }
    }
    __syncthreads();
    for (int q = 0; q < 8; ++q) {
      const int item = tid + 256 * q;
      const float4 base = *reinterpret_cast<const float4*>(tile + (item >> 5) * kYRow + 4 * (item & 31));
      const int64_t t = t0 + 64 * h + (item >> 5);
      const int64_t j = (n0 >> 2) + (item & 31);
      if (t < T && j < nblk) {
        float* yt = Y + t * N + 4 * j;
#pragma unroll 2
        for (int64_t k = 0; k < ndraw; ++k) {
          float a0, a1, a2, a3;
          normal4_scaled((uint32_t)j, (uint32_t)t, draw0 + (uint32_t)k, stream, k0, k1, a0, a1,
                         a2, a3);
          ff32x4_t o;
          o.x = fmaf(sigma_s, a0, base.x);
          o.y = fmaf(sigma_s, a1, base.y);
          o.z = fmaf(sigma_s, a2, base.z);
          o.w = fmaf(sigma_s, a3, base.w);
          // streaming store: Y is written once and is far larger than the caches
          __builtin_nontemporal_store(o, reinterpret_cast<ff32x4_t*>(yt + k * T * N));
        }
      }
    }
    __syncthreads();
  }
}

bool perturbed_linear_supported(int64_t T, int64_t N) {
  // one workgroup of 256 threads per output tile: the grid must fit 32 bits
  return ((T + kFM - 1) / kFM) * ((N + kFN - 1) / kFN) < ((int64_t)1 << 24);
}

hipError_t launch_perturbed_linear(const void* X, const void* W, bool bf16, int64_t T, int64_t N,
                                   int64_t d, float sigma, uint64_t seed, uint32_t stream,
                                   uint32_t draw0, int64_t ndraw, float* Y, hipStream_t s) {
  if (T == 0 || ndraw == 0) return hipSuccess;
  const int64_t tiles = ((T + kFM - 1) / kFM) * ((N + kFN - 1) / kFN);
  const size_t operands =
      (size_t)2 * 2 * (bf16 ? 1 : 2) * (kFM * kFRow + kFN * kFRow);  // 2 stages (hi, + lo for fp32)
  const size_t result = (size_t)(kFM / 2) * (kFN + 4) * sizeof(float);  // half the result tile
  const size_t lds = operands > result ? operands : result;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  if (lds > 65536) {
    const void* fn = bf16 ? reinterpret_cast<const void*>(&perturbed_linear_kernel<false>)
                          : reinterpret_cast<const void*>(&perturbed_linear_kernel<true>);
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (bf16) {
    hipLaunchKernelGGL(perturbed_linear_kernel<false>, dim3((uint32_t)tiles), dim3(256), lds, s, X,
                       W, T, N, d, sigma, draw0, ndraw, stream, k0, k1, Y);
  } else {
    hipLaunchKernelGGL(perturbed_linear_kernel<true>, dim3((uint32_t)tiles), dim3(256), lds, s, X,
                       W, T, N, d, sigma, draw0, ndraw, stream, k0, k1, Y);
  }
  return hipGetLastError();
}

}  // namespace dust
