// dust_device.hpp -- device building blocks shared by the libdust kernels:
// the counter-based noise generator and wavefront reductions (gfx950, wave64).
//
// Noise: the pages (laoyaoba analysis, mechanism section; linlog explainer,
// "the core of Dust") ask for a_t ~ N(0, I), independent per token and per
// draw.  libdust draws it from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11) followed by Box-Muller
// (Box & Muller, 1958), so that any element can be recomputed from its
// coordinates (draw, token, column) instead of being stored.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dust {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;  // golden ratio
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;  // sqrt(3) - 1

struct u32x4 {
  uint32_t x, y, z, w;
};

// Three-input xor in one gfx950 instruction (v_bitop3_b32, truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// One Philox4x32 round: counter words 0 and 2 are multiplied by the two
// multipliers (full 64-bit products); the high halves are xor-ed with the other
// two counter words and the round key; the low halves are kept.  The modes only
// change how the xors are written for the compiler:
//   kXorPlain : two-input xors, so that lane-uniform operands can be combined
//               on the scalar unit first;
//   kXorBitop3: one v_bitop3 per three-input xor (every operand lane-varying
//               but the key);
//   kXorC3Uniform: as kXorBitop3 for the new word 0, but c3 ^ k1 grouped for
//               the new word 2, when c3 is lane-uniform (a vector instruction
//               can take only one scalar operand, so a bitop3 there would need
//               a copy of c3 into a vector register).
enum PhiloxXor { kXorPlain, kXorBitop3, kXorC3Uniform };

template <PhiloxXor kMode>
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                             uint32_t& c3, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)kPhiloxM0 * (uint64_t)c0;
  const uint64_t p1 = (uint64_t)kPhiloxM1 * (uint64_t)c2;
  uint32_t n0, n2;
  if constexpr (kMode == kXorBitop3) {
    n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
  } else if constexpr (kMode == kXorC3Uniform) {
    n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    n2 = (uint32_t)(p0 >> 32) ^ (c3 ^ k1);
  } else {
    n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
  }
  c1 = (uint32_t)p1;
  c3 = (uint32_t)p0;
  c0 = n0;
  c2 = n2;
}

// Philox4x32-10 on an arbitrary counter: 10 rounds, the key bumped by the Weyl
// increments between rounds.
__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r)
    philox_round<kXorBitop3>(c0, c1, c2, c3, k0 + (uint32_t)r * kPhiloxW0,
                             k1 + (uint32_t)r * kPhiloxW1);
  return u32x4{c0, c1, c2, c3};
}

// The same function for the counters of a noise row, (token, column/4, draw,
// stream).  With kColumnOnly, only the column word differs between lanes (one
// token and draw per wave): the column enters through a xor, so the first
// rounds are mostly lane-uniform; their uniform parts run on the scalar unit
// (plain xors let the compiler split them off), the vector work is 16 products
// instead of 20, and in the fourth round the fourth word is still uniform.
// From the fifth round on every word differs between lanes and each
// three-input xor is one bitop3.
template <bool kColumnOnly>
__device__ __forceinline__ u32x4 philox10_row(uint32_t token, uint32_t j, uint32_t draw,
                                              uint32_t stream, uint32_t k0, uint32_t k1) {
  uint32_t c0 = token, c1 = j, c2 = draw, c3 = stream;
#pragma unroll
  for (int r = 0; r < 3; ++r)
    philox_round<kXorPlain>(c0, c1, c2, c3, k0 + (uint32_t)r * kPhiloxW0,
                            k1 + (uint32_t)r * kPhiloxW1);
  philox_round<kColumnOnly ? kXorC3Uniform : kXorBitop3>(c0, c1, c2, c3, k0 + 3u * kPhiloxW0,
                                                         k1 + 3u * kPhiloxW1);
#pragma unroll
  for (int r = 4; r < 10; ++r)
    philox_round<kXorBitop3>(c0, c1, c2, c3, k0 + (uint32_t)r * kPhiloxW0,
                             k1 + (uint32_t)r * kPhiloxW1);
  return u32x4{c0, c1, c2, c3};
}

// u = ((x >> 9) + 1/2) * 2^-23, exactly.  The 23 top bits are placed under the
// exponent of 1.0f, giving 1 + m 2^-23 in [1, 2); subtracting 1 - 2^-24 is
// exact (Sterbenz) and yields m 2^-23 + 2^-24 in (0, 1).
__device__ __forceinline__ float unit_open(uint32_t x) {
  const uint32_t bits = __builtin_amdgcn_alignbit(0x7Fu, x, 9u);  // (x >> 9) | 0x3F800000
  return __uint_as_float(bits) - 0.999999940395355224609375f;
}

// The Box-Muller angle of a word, in revolutions: v = (x >> 9) 2^-23 in [0, 1).
// Returned as 1 + v, the same single instruction as unit_open without its
// subtraction: v_sin_f32 and v_cos_f32 take their argument in revolutions and
// reduce it modulo one, and 1 + v (exact in fp32) is the same point of the
// circle as v.
__device__ __forceinline__ float angle_rev_plus1(uint32_t x) {
  return __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, x, 9u));  // (x >> 9) | 0x3F800000
}

// Four standard normals from one Philox block, Box-Muller on the word pairs
// (0,1) and (2,3): radius sqrt(-2 ln u) from the even word's uniform, angle
// 2 pi v from the odd word's fraction, cosine first.  v_log_f32 is log2.
__device__ __forceinline__ void box_muller4(const u32x4& x, float& a0, float& a1, float& a2,
                                            float& a3) {
  constexpr float kMinus2Ln2 = -1.38629436111989061883f;
  const float u0 = unit_open(x.x), v1 = angle_rev_plus1(x.y);
  const float u2 = unit_open(x.z), v3 = angle_rev_plus1(x.w);
  const float r0 = __builtin_amdgcn_sqrtf(kMinus2Ln2 * __builtin_amdgcn_logf(u0));
  const float r1 = __builtin_amdgcn_sqrtf(kMinus2Ln2 * __builtin_amdgcn_logf(u2));
  a0 = r0 * __builtin_amdgcn_cosf(v1);
  a1 = r0 * __builtin_amdgcn_sinf(v1);
  a2 = r1 * __builtin_amdgcn_cosf(v3);
  a3 = r1 * __builtin_amdgcn_sinf(v3);
}

// The four normals of columns 4j .. 4j+3 of a^(draw)_token.
__device__ __forceinline__ void normal4(uint32_t j, uint32_t token, uint32_t draw,
                                        uint32_t stream, uint32_t k0, uint32_t k1,
                                        float& a0, float& a1, float& a2, float& a3) {
  box_muller4(philox10_row<false>(token, j, draw, stream, k0, k1), a0, a1, a2, a3);
}

// The same normals divided by sqrt(2 ln 2): the radius sqrt(-2 ln u) is
// sqrt(2 ln 2) sqrt(-log2 u), and sqrt(-log2 u) is one v_sqrt with a negated
// operand, one multiply fewer per pair.  Kernels that only ever scale the noise
// (sigma a in a perturbation, r a in the error estimate) use these and fold
// kBoxMullerScale into their scalar factor.
constexpr float kBoxMullerScale = 1.17741002251547469101f;  // sqrt(2 ln 2)

// kColumnOnly: the caller's token and draw are the same in every lane.
template <bool kColumnOnly = false>
__device__ __forceinline__ void normal4_scaled(uint32_t j, uint32_t token, uint32_t draw,
                                               uint32_t stream, uint32_t k0, uint32_t k1,
                                               float& a0, float& a1, float& a2, float& a3) {
  const u32x4 x = philox10_row<kColumnOnly>(token, j, draw, stream, k0, k1);
  const float u0 = unit_open(x.x), v1 = angle_rev_plus1(x.y);
  const float u2 = unit_open(x.z), v3 = angle_rev_plus1(x.w);
  const float r0 = __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(u0));
  const float r1 = __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(u2));
  a0 = r0 * __builtin_amdgcn_cosf(v1);
  a1 = r0 * __builtin_amdgcn_sinf(v1);
  a2 = r1 * __builtin_amdgcn_cosf(v3);
  a3 = r1 * __builtin_amdgcn_sinf(v3);
}

// ---------------------------------------------------------------------------
// Wavefront (64-lane) reductions.  DPP steps inside rows of 16 lanes, then the
// four row sums combined in a fixed order, so the result is deterministic and
// identical in every lane.
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Row sums R0..R3 in every lane of their row, then row_bcast:15 adds R0 into
// row 1 and R2 into row 3, and row_bcast:31 adds row 1's R0 + R1 into row 3:
// lane 63 holds (R2 + R3) + (R0 + R1).  The sum is left in lane 63 only, for a
// caller that stores it from that lane.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  // One v_add_f32_dpp each, written out because the compiler keeps a partial
  // row mask as v_mov + v_mov_dpp + v_add: the rows the mask leaves out keep
  // their value.  The s_nop gives the two wait states a DPP read needs after a
  // vector write of the same register.
  asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf"
               : "+v"(v));
  asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
               : "+v"(v));
  return v;
}

// The wave's sum in every lane (read from lane 63 into a scalar register).
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum_lane63(v)), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

}  // namespace dust
