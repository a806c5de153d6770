// dust_gemm16.hpp -- the operand form of the G_W pass on the fp16 matrix cores,
// shared by the kernels that produce g (they write it as each token's row of g
// is finished) and by the G_W kernel that reads it.
//
// Paper digest, section 2.2: G_W = sum_t g_t x_t^T.  The product is exact if
// each token's pair (g_t, x_t) is replaced by (g_t 2^-s, x_t 2^s) for any
// integer s_t, so each token gets its own power of two that puts both rows in
// the range of fp16; the matrix cores then take both operands rounded to fp16
// (11 significant bits; bf16 inputs are exact there) and accumulate in fp32.
//
//   g16   [T][Mp] fp16 bits (Mp = N rounded up to 8, zero past N), row t is
//         g_t 2^-s_t: token-major, the layout the producers write;
//   x16   [ceil(T/8)][d][8] fp16 bits, x16[(t/8) d + k][t % 8] = x_t[k] 2^s_t:
//         eight consecutive tokens of one column side by side, the layout of a
//         matrix-core operand (zero for the padding tokens of the last group);
//   flags [T] bytes: 1 for a token left to an exact fp32 pass (non-finite
//         values, or a range no power of two fits into fp16); its rows above
//         are zero.
//
// Choice of s_t: with G = max |g_t| and X = max |x_t| written as 2^eg (1+f) and
// 2^ex (1+f'), s = floor((eg - ex) / 2) leaves the scaled maxima in
// [2^ceil(p/2), 2^(ceil(p/2)+1)) and [2^floor(p/2), 2^(floor(p/2)+1)), p = eg + ex.
// For kScaleExpMin <= p <= kScaleExpMax both lie in [2^-11, 2^14): no overflow
// (fp16 max 65504), and an element rounds to an fp16 subnormal (absolute error
// <= 2^-25) only when it is 2^-3 or less of its row's maximum.  Rows with G = 0
// or X = 0 contribute nothing and are written as zeros.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

constexpr int kScaleExpMin = -22;
constexpr int kScaleExpMax = 26;

__device__ __forceinline__ float load_x(const void* X, int bf16, int64_t i) {
  return bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(X)[i] << 16)
              : reinterpret_cast<const float*>(X)[i];
}

__device__ __forceinline__ uint16_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// 0: scale by 2^-s (g) and 2^s (x); 1: the token contributes nothing (zero
// rows); 2: exact fp32 pass (zero rows, flag set).
__device__ __forceinline__ int choose_scale(float gmax, float xmax, bool nonfinite, int& s) {
  s = 0;
  if (nonfinite) return 2;
  if (!(gmax > 0.f) || !(xmax > 0.f)) return 1;
  const int eg = __builtin_amdgcn_frexp_expf(gmax) - 1;  // gmax in [2^eg, 2^(eg+1))
  const int ex = __builtin_amdgcn_frexp_expf(xmax) - 1;
  const int p = eg + ex;
  if (p < kScaleExpMin || p > kScaleExpMax) return 2;
  s = (eg - ex) >> 1;  // floor
  return 0;
}

__device__ __forceinline__ bool not_finite(float v) { return !(__builtin_fabsf(v) <= 3.4e38f); }

// Workgroup maximum of three wave-uniform values (the waves' maxima of |g|,
// |x| and a non-finite marker); `red` holds 3 * kW floats.  One barrier.
template <int kW>
__device__ __forceinline__ void group_max3(float& a, float& b, float& c, float* red) {
  if constexpr (kW > 1) {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      red[w] = a;
      red[kW + w] = b;
      red[2 * kW + w] = c;
    }
    __syncthreads();
    a = red[0];
    b = red[kW];
    c = red[2 * kW];
#pragma unroll
    for (int q = 1; q < kW; ++q) {
      a = fmaxf(a, red[q]);
      b = fmaxf(b, red[kW + q]);
      c = fmaxf(c, red[2 * kW + q]);
    }
  }
}

// Token of workgroup b in a grid of T workgroups that produce one token each.
// Workgroups are dealt to the 8 XCDs in turn (XCD b % 8), and the 8 tokens of
// one x16 group write interleaved 2-byte slots of the same lines, so within
// each full block of 64 tokens the (turn, XCD) grid is transposed: XCD x then
// produces tokens 8x .. 8x+7 of the block, and its L2 merges their writes into
// whole lines instead of 8 XCDs each writing the lines back partially. Tokens
// past the last full block keep b.
__device__ __forceinline__ int64_t producer_token(uint32_t b, int64_t T) {
  if ((int64_t)b >= (T & ~(int64_t)63)) return (int64_t)b;
  return (int64_t)(b & ~63u) + 8 * (int64_t)(b & 7u) + (int64_t)((b >> 3) & 7u);
}

// Scaled copy of x_t into its column slots of x16 (every thread of the
// token's workgroup, threads striding over the columns), and the zero
// padding of the last token group when t is the last token.
__device__ __forceinline__ void emit_x_row(const Gemm16Out& o, int64_t t, int mode, int s,
                                           int nthreads) {
  const int64_t d = o.d;
  uint16_t* xg = o.x16 + ((t >> 3) * d) * 8 + (t & 7);
  for (int64_t k = threadIdx.x; k < d; k += nthreads) {
    const float v = mode == 0 ? __builtin_ldexpf(load_x(o.X, o.x_bf16, t * d + k), s) : 0.f;
    xg[k * 8] = f16_bits(v);
  }
  if (t == o.T - 1) {
    for (int64_t tt = o.T; tt < ((o.T + 7) & ~(int64_t)7); ++tt) {
      uint16_t* xp = o.x16 + ((tt >> 3) * d) * 8 + (tt & 7);
      for (int64_t k = threadIdx.x; k < d; k += nthreads) xp[k * 8] = 0;
    }
  }
}

// Called by all 64 kW threads of a producer's workgroup for token t once its
// row of g is final: this thread holds g[t][4j .. 4j+3] in gv[4b .. 4b+3] for
// j = b * 64 kW + (thread index), b < kNB, where j < N/4 (N % 4 == 0).
// `red` is workgroup shared memory of at least 3 kW floats not otherwise in
// use across this call.
template <int kNB, int kW>
__device__ __forceinline__ void emit_operands(const Gemm16Out& o, int64_t t, int64_t N,
                                              const float* gv, float* red) {
  const int tid = threadIdx.x;
  const int64_t nblk = N >> 2;
  float gm = 0.f, nf = 0.f;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int64_t j = (int64_t)b * 64 * kW + tid;
    if (j < nblk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gm = fmaxf(gm, __builtin_fabsf(gv[4 * b + e]));
        if (not_finite(gv[4 * b + e])) nf = 1.f;
      }
    }
  }
  float xm = 0.f;
  for (int64_t k = tid; k < o.d; k += 64 * kW) {
    const float v = load_x(o.X, o.x_bf16, t * o.d + k);
    xm = fmaxf(xm, __builtin_fabsf(v));
    if (not_finite(v)) nf = 1.f;
  }
  gm = wave_max(gm);
  xm = wave_max(xm);
  nf = wave_max(nf);
  group_max3<kW>(gm, xm, nf, red);
  int s;
  const int mode = choose_scale(gm, xm, nf > 0.f, s);

  uint16_t* grow = o.g16 + t * o.Mp;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int64_t j = (int64_t)b * 64 * kW + tid;
    if (j < nblk) {
      uint32_t w0, w1;
      if (mode == 0) {
        w0 = f16_bits(__builtin_ldexpf(gv[4 * b], -s)) |
             ((uint32_t)f16_bits(__builtin_ldexpf(gv[4 * b + 1], -s)) << 16);
        w1 = f16_bits(__builtin_ldexpf(gv[4 * b + 2], -s)) |
             ((uint32_t)f16_bits(__builtin_ldexpf(gv[4 * b + 3], -s)) << 16);
      } else {
        w0 = w1 = 0u;
      }
      *reinterpret_cast<uint2*>(grow + 4 * j) = make_uint2(w0, w1);
    }
  }
  if (tid < o.Mp - N) grow[N + tid] = 0;  // at most 4 padding columns (N % 4 == 0)
  emit_x_row(o, t, mode, s, 64 * kW);
  if (tid == 0) o.flags[t] = mode == 2 ? 1 : 0;
}

}  // namespace dust
