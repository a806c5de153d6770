// dust_head.hip -- LM-head stages of the Dust estimator.
//
// The pages (laoyaoba analysis, mechanism section; linlog explainer, "the core
// of Dust"; paper digest, section 2.3) perturb the LM head directly on the
// cached logits and recompute only the per-token cross-entropy, which makes a
// draw far cheaper than a forward pass.  For token t and draw i:
//     l^(i)_t = logsumexp_v(z_tv + sigma a^(i)_tv) - (z_t,y + sigma a^(i)_t,y).
//
// One workgroup owns one token; each of its W waves owns an interleaved share of
// the vocabulary (Philox block j = columns 4j..4j+3 goes to lane j mod 64W), and
// the draws run in a loop.  The token's logits are read from HBM once, shifted
// by the clean row maximum M and scaled by log2(e) into ztilde, and kept in LDS
// for all K draws (in HBM/L2 for vocabularies too large for LDS).  A draw then
// costs, per column, one Philox share, one Box-Muller share, one FMA, one exp2
// and one add; the exp2 sum is reduced across the wave with DPP.
//
// Numerics: with S_i = sum_v 2^(ztilde_v + sigma log2(e) a_v) and S_0 the clean
// sum, the loss change is delta_i = l_i - l_0 = ln(S_i / S_0) - sigma a_y.  It is
// formed from the ratio, never as a difference of two ~log(V)-sized losses.
//
// Two variants share the code:
//   kFused = false: writes delta_i (and optionally l_i) to [K,T] arrays; the
//                   centring, gamma scan and error estimate run afterwards.
//   kFused = true : gamma = 0 only.  The token's reward is then its own
//                   centred decrease c_i = dbar - delta_i (paper digest,
//                   section 2.2), so
//                   sum_i c_i a_i = dbar sum_i a_i - sum_i delta_i a_i,
//                   and the kernel keeps the draw's noise in registers until
//                   delta_i is known, accumulates sum a and sum delta a, and
//                   writes g_t = (sum delta a - dbar sum a) / (K sigma) once.
//                   The noise is generated exactly once per (draw, token, column).
#include "dust_device.hpp"
#include "dust_gemm16.hpp"
#include "dust_launch.hpp"

namespace dust {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

template <typename ZT>
__device__ __forceinline__ void load4(const ZT* p, float& a, float& b, float& c, float& d);

template <>
__device__ __forceinline__ void load4<float>(const float* p, float& a, float& b, float& c,
                                             float& d) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  a = v.x; b = v.y; c = v.z; d = v.w;
}

// bf16 -> fp32 is exact: the 16 bits become the high half of the fp32 word.
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float& a, float& b, float& c,
                                                float& d) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  a = __uint_as_float(v.x << 16);
  b = __uint_as_float(v.x & 0xFFFF0000u);
  c = __uint_as_float(v.y << 16);
  d = __uint_as_float(v.y & 0xFFFF0000u);
}

// Workgroup-wide sum / max of one value per wave (wave results already uniform).
// `red` holds 2*W floats; `slot` alternates so that back-to-back reductions
// need one barrier each.
template <int W>
__device__ __forceinline__ float group_sum(float wave_val, float* red, int slot) {
  if constexpr (W == 1) {
    return wave_val;
  } else {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[slot * W + w] = wave_val;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < W; ++q) s += red[slot * W + q];
    return s;
  }
}

template <int W>
__device__ __forceinline__ float group_max(float wave_val, float* red, int slot) {
  if constexpr (W == 1) {
    return wave_val;
  } else {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[slot * W + w] = wave_val;
    __syncthreads();
    float s = red[slot * W];
#pragma unroll
    for (int q = 1; q < W; ++q) s = fmaxf(s, red[slot * W + q]);
    return s;
  }
}

// Workgroup sums of kN per-wave values at once (one barrier); each wave's value
// must be complete in its lane 63 (wave_sum_lane63), which stores it.  Slot
// `slot` of a kStride-wide layout; alternating slots need no second barrier.
template <int W, int kN, int kStride>
__device__ __forceinline__ void group_sum_n(float* v, float* red, int slot) {
  if constexpr (W > 1) {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 63) {  // the wave's sum is complete in lane 63
#pragma unroll
      for (int d = 0; d < kN; ++d) red[(slot * kStride + d) * W + w] = v[d];
    }
    __syncthreads();
#pragma unroll
    for (int d = 0; d < kN; ++d) {
      float s = red[(slot * kStride + d) * W];
#pragma unroll
      for (int q = 1; q < W; ++q) s += red[(slot * kStride + d) * W + q];
      v[d] = s;
    }
  }
}

// kNB    : Philox blocks per lane per draw (4 kNB columns per lane).
// kW     : waves per token.
// kZInLds: ztilde staged in LDS (V <= 32768); wider vocabularies re-read the
//          raw logits from global memory (L2-resident) every draw.
// kDraws : draws per loop iteration (they share one cross-wave reduction).
template <int kNB, int kW, bool kFused, typename ZT, bool kZInLds, int kDraws>
__global__ void __launch_bounds__(64 * kW)
head_kernel(const ZT* __restrict__ logits, const int32_t* __restrict__ targets, int64_t T,
            int64_t V, float sigma, int64_t K, uint32_t stream, uint32_t k0, uint32_t k1,
            float* __restrict__ g_hat, float* __restrict__ losses, float* __restrict__ delta_out,
            Gemm16Out op) {
  constexpr int kCols = 4 * kNB;
  extern __shared__ float smem[];
  float* red = smem;             // reductions: 2 kW + 2 kDraws kW <= 64 floats, then
                                 // 3 kW <= 48 at smem + 64 for the G_W operands
  float* zs = smem + 128;        // kNB * 64 * kW * 4 floats when kZInLds

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = producer_token(blockIdx.x, T);
  const int64_t nblk = V >> 2;
  const ZT* zrow = logits + t * V;

  // --- clean row: maximum, shifted/scaled logits, clean exp2 sum ----------
  float zt[kCols];  // ztilde of this lane's columns (dead after staging when in LDS)
  float mloc = -INFINITY;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int64_t j = (int64_t)b * 64 * kW + wave * 64 + lane;
    if (j < nblk) {
      load4<ZT>(zrow + 4 * j, zt[4 * b], zt[4 * b + 1], zt[4 * b + 2], zt[4 * b + 3]);
      mloc = fmaxf(mloc, fmaxf(fmaxf(zt[4 * b], zt[4 * b + 1]), fmaxf(zt[4 * b + 2], zt[4 * b + 3])));
    } else {
      zt[4 * b] = zt[4 * b + 1] = zt[4 * b + 2] = zt[4 * b + 3] = -INFINITY;
    }
  }
  const float M = group_max<kW>(wave_max(mloc), red, 0);
  const float Ml2e = M * kLog2e;
  float s0 = 0.f;
#pragma unroll
  for (int q = 0; q < kCols; ++q) {
    zt[q] = fmaf(zt[q], kLog2e, -Ml2e);  // -inf stays -inf (exp2 -> 0)
    s0 += __builtin_amdgcn_exp2f(zt[q]);
  }
  if constexpr (kZInLds) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int j = b * 64 * kW + wave * 64 + lane;
      *reinterpret_cast<float4*>(zs + 4 * j) =
          make_float4(zt[4 * b], zt[4 * b + 1], zt[4 * b + 2], zt[4 * b + 3]);
    }
  }
  const float S0 = group_sum<kW>(wave_sum(s0), red, 1);
  const float inv_S0 = 1.0f / S0;
  // An out-of-range target is clamped: the values are then meaningless, but
  // every access stays inside the logits row.
  const int32_t y = min(max(targets[t], 0), (int32_t)(V - 1));
  float zy;
  {
    float c0, c1, c2, c3;
    load4<ZT>(zrow + 4 * (y >> 2), c0, c1, c2, c3);
    const int q = y & 3;
    zy = q == 0 ? c0 : (q == 1 ? c1 : (q == 2 ? c2 : c3));
  }
  const float zty = fmaf(zy, kLog2e, -Ml2e);  // ztilde of the target column
  const float ell0 = kLn2 * (__builtin_amdgcn_logf(S0) - zty);
  // No barrier for the staged row: each lane reads back only the columns it
  // wrote itself, and a wave's LDS accesses complete in order.

  // The noise arrives divided by kBoxMullerScale (normal4_scaled): every use
  // scales it, so the constant rides on the scalar factors below and on g_t.
  const float sl2e = sigma * kLog2e * kBoxMullerScale;
  const float sigma_s = sigma * kBoxMullerScale;
  float acc_a[kFused ? kCols : 1];
  float acc_da[kFused ? kCols : 1];
  if constexpr (kFused) {
#pragma unroll
    for (int q = 0; q < kCols; ++q) { acc_a[q] = 0.f; acc_da[q] = 0.f; }
  }
  float sum_delta = 0.f;
  float ay_vec = 0.f;  // lane l: target-column noise of draw (i0 + l), i0 = i & ~63
  float* red_loop = red + 2 * kW;  // the prologue's reductions used red[0, 2 kW)

  // Noise of draw i for this lane's columns, and the lane's share of
  // S_i = sum_v 2^(ztilde_v + sigma log2(e) a_v).
  auto draw_noise = [&](int64_t i, float* a) -> float {
    float p0, p1, p2, p3;  // set by the first block (no add to a zero start)
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int j = b * 64 * kW + wave * 64 + lane;
      normal4_scaled<true>((uint32_t)j, (uint32_t)t, (uint32_t)i, stream, k0, k1, a[4 * b],
                           a[4 * b + 1], a[4 * b + 2], a[4 * b + 3]);
      float z0, z1, z2, z3;
      if constexpr (kZInLds) {
        const float4 zz = *reinterpret_cast<const float4*>(zs + 4 * j);
        z0 = zz.x; z1 = zz.y; z2 = zz.z; z3 = zz.w;
      } else {
        if (j < nblk) {
          load4<ZT>(zrow + 4 * (int64_t)j, z0, z1, z2, z3);
          z0 = fmaf(z0, kLog2e, -Ml2e); z1 = fmaf(z1, kLog2e, -Ml2e);
          z2 = fmaf(z2, kLog2e, -Ml2e); z3 = fmaf(z3, kLog2e, -Ml2e);
        } else {
          z0 = z1 = z2 = z3 = -INFINITY;
        }
      }
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sl2e, a[4 * b], z0));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sl2e, a[4 * b + 1], z1));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(sl2e, a[4 * b + 2], z2));
      const float e3 = __builtin_amdgcn_exp2f(fmaf(sl2e, a[4 * b + 3], z3));
      if (b == 0) {
        p0 = e0; p1 = e1; p2 = e2; p3 = e3;
      } else {
        p0 += e0; p1 += e1; p2 += e2; p3 += e3;
      }
    }
    return (p0 + p1) + (p2 + p3);
  };
  auto refresh_target_noise = [&](int64_t i) {
    if ((i & 63) == 0) {
      float a0, a1, a2, a3;
      normal4_scaled((uint32_t)(y >> 2), (uint32_t)t, (uint32_t)(i + lane), stream, k0, k1, a0,
                     a1, a2, a3);
      const int q = y & 3;
      ay_vec = q == 0 ? a0 : (q == 1 ? a1 : (q == 2 ? a2 : a3));
    }
  };
  // Loss change of draw i from its full sum S_i; accumulate or write it.
  auto finish = [&](int64_t i, float Si, const float* a) {
    const float ay = lane_value(ay_vec, (int)(i & 63));
    const float delta = kLn2 * __builtin_amdgcn_logf(Si * inv_S0) - sigma_s * ay;
    if constexpr (kFused) {
      sum_delta += delta;
#pragma unroll
      for (int q = 0; q < kCols; ++q) {
        acc_a[q] += a[q];
        acc_da[q] = fmaf(delta, a[q], acc_da[q]);
      }
    } else {
      if (delta_out != nullptr && threadIdx.x == 0) delta_out[i * T + t] = delta;
    }
    if (losses != nullptr && threadIdx.x == 0) losses[i * T + t] = ell0 + delta;
  };

  // kDraws draws per iteration share one cross-wave reduction (one barrier).
  int64_t i = 0;
  int parity = 0;
  for (; i + kDraws <= K; i += kDraws, parity ^= 1) {
    refresh_target_noise(i);
    float a[kDraws][kCols];
    float S[kDraws];
#pragma unroll
    for (int d = 0; d < kDraws; ++d) {
      if constexpr (kW > 1) S[d] = wave_sum_lane63(draw_noise(i + d, a[d]));
      else S[d] = wave_sum(draw_noise(i + d, a[d]));
    }
    group_sum_n<kW, kDraws, kDraws>(S, red_loop, parity);
#pragma unroll
    for (int d = 0; d < kDraws; ++d) finish(i + d, S[d], a[d]);
  }
  for (; i < K; ++i, parity ^= 1) {  // tail when kDraws does not divide K
    refresh_target_noise(i);
    float a[kCols];
    float S[1] = {wave_sum(draw_noise(i, a))};
    group_sum_n<kW, 1, kDraws>(S, red_loop, parity);
    finish(i, S[0], a);
  }

  if constexpr (kFused) {
    const float dbar = sum_delta / (float)K;
    const float scale = kBoxMullerScale / ((float)K * sigma);
    float* grow = g_hat + t * V;
    float gv[kCols];
#pragma unroll
    for (int q = 0; q < kCols; ++q) gv[q] = (acc_da[q] - dbar * acc_a[q]) * scale;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int64_t j = (int64_t)b * 64 * kW + wave * 64 + lane;
      if (j < nblk)
        *reinterpret_cast<float4*>(grow + 4 * j) =
            make_float4(gv[4 * b], gv[4 * b + 1], gv[4 * b + 2], gv[4 * b + 3]);
    }
    // The fp16 operands of the G_W pass: this workgroup owns the token's whole row.
    if (op.g16 != nullptr) emit_operands<kNB, kW>(op, t, V, gv, smem + 64);
  }
}

// --------------------------------------------------------------------------
// Host-side launch configuration.
// --------------------------------------------------------------------------
constexpr int64_t kLdsVocabMax = 32768;  // ztilde (4 bytes per column) fits LDS
// Draws per cross-wave reduction in the fused kernel.  Two draws per barrier
// cost more registers (two noise rows live at once) than the barrier they
// save: measured on MI355X at V=4096, one draw per reduction is faster.
constexpr int fused_draws(int /*nb*/) { return 1; }

// Fused kernel: 16 columns per lane and up to 16 waves per token, which keeps a
// lane's draw noise and both accumulators near 100 VGPRs (4 waves per SIMD).
// Wider rows use 64 columns per lane on 8 waves.
HeadShape fused_shape(int64_t V) {
  const int64_t nblk = V / 4;
  HeadShape h;
  if (nblk <= 64) { h.nb = 1; h.w = 1; }
  else if (nblk <= 128) { h.nb = 2; h.w = 1; }
  else if (nblk <= 256) { h.nb = 4; h.w = 1; }
  else if (nblk <= 512) { h.nb = 4; h.w = 2; }
  else if (nblk <= 1024) { h.nb = 4; h.w = 4; }
  else if (nblk <= 2048) { h.nb = 4; h.w = 8; }
  else if (nblk <= 4096) { h.nb = 4; h.w = 16; }
  else if (nblk <= 8192) { h.nb = 16; h.w = 8; }
  else { h.nb = 0; h.w = 0; }
  return h;
}

// Kernels that keep at most one value per column (per-draw losses, error
// estimate): up to 64 columns per lane on one wave, then more waves.
HeadShape wide_shape(int64_t V) {
  const int64_t nblk = V / 4;
  HeadShape h;
  if (nblk <= 64) { h.nb = 1; h.w = 1; }
  else if (nblk <= 128) { h.nb = 2; h.w = 1; }
  else if (nblk <= 256) { h.nb = 4; h.w = 1; }
  else if (nblk <= 512) { h.nb = 8; h.w = 1; }
  else {
    h.nb = 16;
    const int64_t w = (nblk + 1023) / 1024;
    h.w = w <= 1 ? 1 : w <= 2 ? 2 : w <= 4 ? 4 : w <= 8 ? 8 : 16;
  }
  return h;
}

bool head_fused_supported(int64_t V) { return fused_shape(V).nb != 0; }

template <int kNB, int kW, bool kFused, typename ZT, bool kZInLds>
static hipError_t launch_head_t(const void* logits, const int32_t* targets, int64_t T, int64_t V,
                                float sigma, int64_t K, uint32_t stream, uint64_t seed,
                                float* g_hat, float* losses, float* delta, const Gemm16Out& op,
                                hipStream_t s) {
  constexpr int kDraws = kFused ? fused_draws(kNB) : 1;
  const size_t lds = sizeof(float) * (128 + (kZInLds ? (size_t)kNB * 64 * kW * 4 : 0));
  if (lds > 65536) {  // above the default dynamic-LDS limit: raise it for this kernel
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&head_kernel<kNB, kW, kFused, ZT, kZInLds, kDraws>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((head_kernel<kNB, kW, kFused, ZT, kZInLds, kDraws>), dim3((uint32_t)T),
                     dim3(64 * kW),
                     lds, s, reinterpret_cast<const ZT*>(logits), targets, T, V, sigma, K, stream,
                     (uint32_t)seed, (uint32_t)(seed >> 32), g_hat, losses, delta, op);
  return hipGetLastError();
}

template <bool kFused, typename ZT>
static hipError_t launch_head_dispatch(const void* logits, const int32_t* targets, int64_t T,
                                       int64_t V, float sigma, int64_t K, uint32_t stream,
                                       uint64_t seed, float* g_hat, float* losses, float* delta,
                                       const Gemm16Out& op, hipStream_t s) {
  const HeadShape h = kFused ? fused_shape(V) : wide_shape(V);
  const bool lds = V <= kLdsVocabMax;
#define DUST_HEAD_CASE(NB, W, LDS)                                                              \
  if (h.nb == NB && h.w == W && lds == LDS)                                                     \
    return launch_head_t<NB, W, kFused, ZT, LDS>(logits, targets, T, V, sigma, K, stream, seed, \
                                                 g_hat, losses, delta, op, s);
  DUST_HEAD_CASE(1, 1, true)
  DUST_HEAD_CASE(2, 1, true)
  DUST_HEAD_CASE(4, 1, true)
  if constexpr (kFused) {
    DUST_HEAD_CASE(4, 2, true)
    DUST_HEAD_CASE(4, 4, true)
    DUST_HEAD_CASE(4, 8, true)
    DUST_HEAD_CASE(4, 16, true)
    DUST_HEAD_CASE(16, 8, true)
  } else {
    DUST_HEAD_CASE(8, 1, true)
    DUST_HEAD_CASE(16, 1, true)
    DUST_HEAD_CASE(16, 2, true)
    DUST_HEAD_CASE(16, 4, true)
    DUST_HEAD_CASE(16, 8, true)
    DUST_HEAD_CASE(16, 16, false)
  }
#undef DUST_HEAD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_head_fused(const void* logits, bool logits_bf16, const int32_t* targets,
                             int64_t T, int64_t V, float sigma, int64_t K, uint32_t stream,
                             uint64_t seed, float* g_hat, float* losses, const Gemm16Out& op,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  return logits_bf16
             ? launch_head_dispatch<true, uint16_t>(logits, targets, T, V, sigma, K, stream, seed,
                                                    g_hat, losses, nullptr, op, s)
             : launch_head_dispatch<true, float>(logits, targets, T, V, sigma, K, stream, seed,
                                                 g_hat, losses, nullptr, op, s);
}

hipError_t launch_head_losses(const void* logits, bool logits_bf16, const int32_t* targets,
                              int64_t T, int64_t V, float sigma, int64_t K, uint32_t stream,
                              uint64_t seed, float* losses, float* delta, hipStream_t s) {
  if (T == 0) return hipSuccess;
  Gemm16Out none{};
  return logits_bf16
             ? launch_head_dispatch<false, uint16_t>(logits, targets, T, V, sigma, K, stream, seed,
                                                     nullptr, losses, delta, none, s)
             : launch_head_dispatch<false, float>(logits, targets, T, V, sigma, K, stream, seed,
                                                  nullptr, losses, delta, none, s);
}

}  // namespace dust
