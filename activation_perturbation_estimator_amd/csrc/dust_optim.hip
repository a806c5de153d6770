// dust_optim.hip -- consumers of the estimate: the optimiser step on G_W and
// the closed-form LM-head gradient used to measure the estimate's alignment.
//
// Optimisers (linlog explainer, experiment setup: SGD with momentum; paper
// digest, section 3.3 and laoyaoba analysis, engineering section: Adam works
// with the estimate unchanged).  G_W approximates +dL/dW (it has backprop's
// form, paper digest section 2.2), so both steps descend along it:
//   SGD + momentum : m = mu m + (G + wd W);   W -= lr m
//   Adam           : g = G + wd W; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
//                    W -= lr (m / (1 - b1^k)) / (sqrt(v / (1 - b2^k)) + eps)
// Elementwise and memory-bound (16 / 28 bytes per parameter).
//
// Closed-form head gradient: d CE / d z_t = softmax(z_t) - onehot(y_t), the
// backprop gradient the pages compare the estimate against (paper digest,
// section 4.2; linlog explainer, gradient-alignment section).
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

__global__ void __launch_bounds__(256) sgd_momentum_kernel(float* __restrict__ W,
                                                           const float* __restrict__ G,
                                                           float* __restrict__ M, int64_t n,
                                                           float lr, float mu, float wd) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float w = W[i];
    const float g = fmaf(wd, w, G[i]);
    const float m = fmaf(mu, M[i], g);
    M[i] = m;
    W[i] = fmaf(-lr, m, w);
  }
}

__global__ void __launch_bounds__(256) adam_kernel(float* __restrict__ W, const float* __restrict__ G,
                                                   float* __restrict__ M, float* __restrict__ Vv,
                                                   int64_t n, float lr, float b1, float b2,
                                                   float eps, float wd, float inv_bc1,
                                                   float inv_sqrt_bc2) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float w = W[i];
    const float g = fmaf(wd, w, G[i]);
    const float m = fmaf(b1, M[i], (1.0f - b1) * g);
    const float v = fmaf(b2, Vv[i], (1.0f - b2) * g * g);
    M[i] = m;
    Vv[i] = v;
    const float denom = sqrtf(v) * inv_sqrt_bc2 + eps;
    W[i] = w - lr * (m * inv_bc1) / denom;
  }
}

template <typename ZT>
__device__ __forceinline__ float ld1(const ZT* p);
template <>
__device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}

// One workgroup (256 threads) per token.
template <typename ZT>
__global__ void __launch_bounds__(256) ce_grad_kernel(const ZT* __restrict__ logits,
                                                      const int32_t* __restrict__ targets,
                                                      int64_t V, float* __restrict__ out) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const ZT* z = logits + t * V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m = -INFINITY;
  for (int64_t v = threadIdx.x; v < V; v += 256) m = fmaxf(m, ld1<ZT>(z + v));
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float s = 0.f;
  for (int64_t v = threadIdx.x; v < V; v += 256) s += expf(ld1<ZT>(z + v) - m);
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  s = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / s;
  const int32_t y = targets[t];
  float* o = out + t * V;
  for (int64_t v = threadIdx.x; v < V; v += 256)
    o[v] = expf(ld1<ZT>(z + v) - m) * inv - (v == y ? 1.0f : 0.0f);
}

static int grid1d(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_sgd_momentum(float* W, const float* G, float* M, int64_t n, float lr, float mu,
                               float wd, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sgd_momentum_kernel, dim3(grid1d(n)), dim3(256), 0, s, W, G, M, n, lr, mu,
                     wd);
  return hipGetLastError();
}

hipError_t launch_adam(float* W, const float* G, float* M, float* V, int64_t n, float lr, float b1,
                       float b2, float eps, float wd, float inv_bc1, float inv_sqrt_bc2,
                       hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(adam_kernel, dim3(grid1d(n)), dim3(256), 0, s, W, G, M, V, n, lr, b1, b2, eps,
                     wd, inv_bc1, inv_sqrt_bc2);
  return hipGetLastError();
}

hipError_t launch_ce_grad(const void* logits, bool bf16, const int32_t* targets, int64_t T,
                          int64_t V, float* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(ce_grad_kernel<uint16_t>, dim3((uint32_t)T), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(logits), targets, V, out);
  else
    hipLaunchKernelGGL(ce_grad_kernel<float>, dim3((uint32_t)T), dim3(256), 0, s,
                       reinterpret_cast<const float*>(logits), targets, V, out);
  return hipGetLastError();
}

}  // namespace dust
