// valu_rates.hip -- issue-rate probe of the gfx950 VALU instructions the
// estimator kernels use.  Each kernel runs CH independent dependency chains of
// one instruction (inline asm, register operands only) per lane; the time per
// lane-instruction at 8 and 16 waves per CU gives each instruction's issue
// cost relative to the full fp32 rate (256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz
// = 78.64e12 lane-instructions/s).  Build and run:
//   python -m activation_perturbation_estimator_amd.probes
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#define CH 16
#define K1(NAME, ASM) \
__global__ void __launch_bounds__(256) NAME(float* out, int iters) { \
  float v[CH]; for (int u = 0; u < CH; ++u) v[u] = threadIdx.x * 1e-3f + u + 1.0f; \
  for (int i = 0; i < iters; ++i) { _Pragma("unroll") for (int u = 0; u < CH; ++u) { asm volatile(ASM : "+v"(v[u])); } } \
  float s = 0; for (int u = 0; u < CH; ++u) s += v[u]; out[blockIdx.x * 256 + threadIdx.x] = s; }
K1(k_fma, "v_fma_f32 %0, %0, %0, %0")
K1(k_add, "v_add_f32 %0, 1.0, %0")
K1(k_xor, "v_xor_b32 %0, 0x1234, %0")
K1(k_bitop3, "v_bitop3_b32 %0, %0, %0, %0 bitop3:0x96")
K1(k_alignbit, "v_alignbit_b32 %0, %0, %0, 9")
K1(k_lshr, "v_lshrrev_b32 %0, 9, %0")
K1(k_cvt, "v_cvt_f32_u32 %0, %0")
K1(k_mulhi, "v_mul_hi_u32 %0, %0, %0")
K1(k_exp, "v_exp_f32 %0, %0")
K1(k_log, "v_log_f32 %0, %0")
K1(k_sqrt, "v_sqrt_f32 %0, %0")
K1(k_sin, "v_sin_f32 %0, %0")
K1(k_fma3exp, "v_fma_f32 %0, %0, %0, %0\n v_fma_f32 %0, %0, %0, %0\n v_fma_f32 %0, %0, %0, %0\n v_exp_f32 %0, %0")
K1(k_xor2bitop, "v_xor_b32 %0, 0x1234, %0\n v_bitop3_b32 %0, %0, %0, %0 bitop3:0x96")

__global__ void __launch_bounds__(256) k_mad64(float* out, int iters) {
  uint64_t v[CH]; for (int u = 0; u < CH; ++u) v[u] = threadIdx.x + u;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      uint64_t r;
      asm volatile("v_mad_u64_u32 %0, vcc, %1, %1, %2" : "=v"(r) : "v"((uint32_t)v[u]), "v"(v[u]) : "vcc");
      v[u] = r;
    }
  }
  uint64_t s = 0; for (int u = 0; u < CH; ++u) s += v[u]; out[blockIdx.x * 256 + threadIdx.x] = (float)s;
}
// mad64 followed by a dependent bitop3 on the high half (the Philox pattern)
__global__ void __launch_bounds__(256) k_mad64_bitop(float* out, int iters) {
  uint64_t v[CH]; for (int u = 0; u < CH; ++u) v[u] = threadIdx.x + u;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      uint64_t r; uint32_t hi;
      asm volatile("v_mad_u64_u32 %0, vcc, %1, %1, 0" : "=v"(r) : "v"((uint32_t)v[u]) : "vcc");
      hi = (uint32_t)(r >> 32);
      asm volatile("v_bitop3_b32 %0, %0, %1, %1 bitop3:0x96" : "+v"(hi) : "v"((uint32_t)r));
      v[u] = ((uint64_t)hi << 32) | (uint32_t)r;
    }
  }
  uint64_t s = 0; for (int u = 0; u < CH; ++u) s += v[u]; out[blockIdx.x * 256 + threadIdx.x] = (float)s;
}

void run(const char* name, void (*kern)(float*, int), int wpc, int ipi, int ncu) {
  int blocks = ncu * wpc / 4;
  float* d; (void)hipMalloc(&d, sizeof(float) * blocks * 256);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, d, 8);
  (void)hipDeviceSynchronize();
  hipEvent_t a, b; (void)hipEventCreate(&a); (void)hipEventCreate(&b);
  int iters = 2048;
  (void)hipEventRecord(a);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, 0, d, iters);
  (void)hipEventRecord(b); (void)hipEventSynchronize(b);
  float ms; (void)hipEventElapsedTime(&ms, a, b);
  double lane_instr = (double)blocks * 256 * iters * CH * ipi;
  double rate = lane_instr / (ms * 1e-3);
  printf("%-12s waves/CU=%2d  %7.3f ms  %6.2f T lane-instr/s  = %.3f of 78.64T\n", name, wpc, ms, rate / 1e12, rate / 78.64e12);
  (void)hipFree(d);
}

int main() {
  hipDeviceProp_t p; (void)hipGetDeviceProperties(&p, 0);
  int n = p.multiProcessorCount;
  for (int wpc : {8, 16}) {
    run("fma", k_fma, wpc, 1, n); run("add", k_add, wpc, 1, n); run("xor", k_xor, wpc, 1, n);
    run("bitop3", k_bitop3, wpc, 1, n); run("alignbit", k_alignbit, wpc, 1, n);
    run("lshr", k_lshr, wpc, 1, n); run("cvt_f32_u32", k_cvt, wpc, 1, n);
    run("mul_hi", k_mulhi, wpc, 1, n); run("mad_u64", k_mad64, wpc, 1, n);
    run("mad64+bitop", k_mad64_bitop, wpc, 2, n);
    run("exp", k_exp, wpc, 1, n); run("log", k_log, wpc, 1, n); run("sqrt", k_sqrt, wpc, 1, n);
    run("sin", k_sin, wpc, 1, n); run("3fma+exp", k_fma3exp, wpc, 4, n);
    run("xor+bitop3", k_xor2bitop, wpc, 2, n);
  }
  return 0;
}
