// dust_launch.hpp -- internal host-side launchers of the libdust kernels.
// Sizes have been validated by the C ABI layer before any of these is called;
// each returns the HIP status of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dust {

// Noise stage.
hipError_t launch_philox_raw(const uint32_t* ctr, uint32_t* out, int64_t n, uint64_t seed,
                             hipStream_t s);
hipError_t launch_noise_fill(float* out, int64_t ndraw, int64_t T, int64_t N, uint32_t draw0,
                             uint32_t stream, uint64_t seed, hipStream_t s);

// Where a kernel that produces g writes the fp16 operands of the G_W pass
// (layout and scale rule in dust_gemm16.hpp); g16 == nullptr: not wanted.
struct Gemm16Out {
  uint16_t* g16;   // [T][Mp]
  uint16_t* x16;   // [ceil(T/8)][d][8]
  uint8_t* flags;  // [T]
  const void* X;   // [T][d] layer input, bf16 (x_bf16) or fp32
  int64_t T, Mp, d;
  int x_bf16;
};

// LM head.  Work split: one workgroup of 64*w threads per token, nb Philox
// blocks per lane per draw.
struct HeadShape {
  int nb;
  int w;
};
HeadShape fused_shape(int64_t V);   // the fused gamma = 0 kernel (0 if unsupported)
HeadShape wide_shape(int64_t V);    // per-draw losses and the error estimate
bool head_fused_supported(int64_t V);
hipError_t launch_head_fused(const void* logits, bool logits_bf16, const int32_t* targets,
                             int64_t T, int64_t V, float sigma, int64_t K, uint32_t stream,
                             uint64_t seed, float* g_hat, float* losses, const Gemm16Out& op,
                             hipStream_t s);
hipError_t launch_head_losses(const void* logits, bool logits_bf16, const int32_t* targets,
                              int64_t T, int64_t V, float sigma, int64_t K, uint32_t stream,
                              uint64_t seed, float* losses, float* delta, hipStream_t s);

// Centring and the discounted-reward scan.
hipError_t launch_centre(const float* x, int64_t K, int64_t T, float* c, hipStream_t s);
hipError_t launch_reward_scan(const float* c, int64_t K, int64_t T, int64_t L, float gamma,
                              float* r, hipStream_t s);

// Error estimate from rewards with regenerated noise.
// Draws draw0 .. draw0 + K - 1 of a population of K_total (the 1/(K_total sigma)).
hipError_t launch_error_estimate(const float* r, int64_t K, int64_t T, int64_t N, float sigma,
                                 uint32_t stream, uint64_t seed, uint32_t draw0, int64_t K_total,
                                 float* g_hat, const Gemm16Out& op, hipStream_t s);

// Outer-product sum G = g^T X on the matrix cores.  The workspace starts with
// the fp16 operands (outer_sum_operands), written either by the kernel that
// produced g or, for a caller's g, by launch_outer_sum's own pass.
size_t outer_sum_workspace_bytes(int64_t T, int64_t N, int64_t d);
bool outer_sum_supported(int64_t T, int64_t N, int64_t d);  // the launch grid fits
Gemm16Out outer_sum_operands(void* workspace, int64_t T, int64_t N, int64_t d, const void* X,
                             bool x_bf16);
hipError_t launch_outer_sum16(const Gemm16Out& op, const float* g32, int64_t N, float* G,
                              void* workspace, hipStream_t s);
hipError_t launch_outer_sum(const float* g, const void* X, bool x_bf16, int64_t T, int64_t N,
                            int64_t d, float* G, void* workspace, hipStream_t s);

// Perturbed forward of a linear layer: Y[k] = X W^T + sigma a^(draw0+k).
bool perturbed_linear_supported(int64_t T, int64_t N);  // the launch grid fits
hipError_t launch_perturbed_linear(const void* X, const void* W, bool bf16, int64_t T, int64_t N,
                                   int64_t d, float sigma, uint64_t seed, uint32_t stream,
                                   uint32_t draw0, int64_t ndraw, float* Y, hipStream_t s);

// Embedding rows: G_E[v] = sum_{t: ids[t] = v} g_t, deterministic order.
size_t embedding_workspace_bytes(int64_t T, int64_t N, int64_t vocab);
hipError_t launch_embedding_grad(const int32_t* ids, const float* g, int64_t T, int64_t N,
                                 int64_t vocab, float* GE, void* workspace, hipStream_t s);
// The library's own scratch for the variant that allocates nothing: the
// current device's address of a fixed array of this many bytes.
constexpr size_t kEmbeddingStaticScratchBytes = (size_t)16 << 20;
hipError_t embedding_static_scratch(void** out);

// Optimiser steps and the closed-form head gradient.
hipError_t launch_sgd_momentum(float* W, const float* G, float* M, int64_t n, float lr, float mu,
                               float wd, hipStream_t s);
hipError_t launch_adam(float* W, const float* G, float* M, float* V, int64_t n, float lr, float b1,
                       float b2, float eps, float wd, float inv_bc1, float inv_sqrt_bc2,
                       hipStream_t s);
hipError_t launch_ce_grad(const void* logits, bool bf16, const int32_t* targets, int64_t T,
                          int64_t V, float* out, hipStream_t s);

// Target range check; flag must be a device int32.
// The library's own flag for dust_check_targets on the current device.
hipError_t check_targets_own_flag(int32_t** out);
hipError_t launch_check_targets(const int32_t* targets, int64_t T, int64_t V, int32_t* flag,
                                hipStream_t s);

}  // namespace dust
