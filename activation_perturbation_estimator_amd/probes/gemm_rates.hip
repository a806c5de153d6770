// gemm_rates.hip -- throughput probes behind the design of the G_W kernel on
// gfx950: the bf16 and fp16 matrix-core rates, the LDS read rates of the
// instruction forms the kernel can use, the rate of buffer loads that write
// LDS directly, and the fp16 G_W inner loop in isolation (LDS operands, MFMA).  Build and run:
//   python -m activation_perturbation_estimator_amd.probes gemm
// Every LDS address stays inside the kernel's own shared array; the loaded
// buffer is 1 MiB and every load offset stays below 8 KiB.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x2_t lds_f32x2;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Clock of each workgroup's run: shader-clock ticks (s_memtime) and
// constant-rate ticks (s_memrealtime) between its first and last instruction,
// recorded by thread 0 of workgroups below 1024.
__device__ unsigned long long g_clk[1024 * 2];
struct ClockSpan {
  long long c0, w0;
  __device__ ClockSpan() : c0(clock64()), w0(wall_clock64()) {}
  __device__ void record() const {
    if (threadIdx.x == 0 && blockIdx.x < 1024) {
      g_clk[2 * blockIdx.x] = (unsigned long long)(clock64() - c0);
      g_clk[2 * blockIdx.x + 1] = (unsigned long long)(wall_clock64() - w0);
    }
  }
};

// 1. Matrix cores alone: 16 independent v_mfma_f32_32x32x16_bf16 per iteration.
__global__ void __launch_bounds__(256) mfma_only(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a[2], b[4];
  for (int i = 0; i < 8; ++i) {
    a[0][i] = (__bf16)(lane * 0.01f + i);
    a[1][i] = (__bf16)(i * 0.5f);
    for (int j = 0; j < 4; ++j) b[j][i] = (__bf16)(0.25f * j + i * 0.125f);
  }
  f32x16_t acc[2][4];
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
  for (int it = 0; it < iters; ++it)
    for (int p = 0; p < 2; ++p)
      for (int x = 0; x < 2; ++x)
        for (int y = 0; y < 4; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
  float s = 0.f;
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 16; ++r) s += acc[x][y][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// 1b. The same for fp16 (v_mfma_f32_32x32x16_f16) or bf16 operands, with kBlocks
// independent accumulator blocks (16: 256 accumulator registers per lane, as
// a 128 x 128 wave tile) used round-robin, 32 MFMAs per iteration.
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
template <bool kF16, int kBlocks>
__global__ void __launch_bounds__(256, 1) mfma_rate(float* out, int iters) {
  const ClockSpan span;
  const int lane = threadIdx.x & 63;
  f16x8_t ah[4], bh[4];
  bf16x8_t ab[4], bb[4];
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) {
      ah[j][i] = (_Float16)(lane * 0.01f + i + j);
      bh[j][i] = (_Float16)(0.25f * j + i * 0.125f);
      ab[j][i] = (__bf16)(lane * 0.01f + i + j);
      bb[j][i] = (__bf16)(0.25f * j + i * 0.125f);
    }
  f32x16_t acc[kBlocks];
  for (int x = 0; x < kBlocks; ++x)
    for (int r = 0; r < 16; ++r) acc[x][r] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int x = k % kBlocks;
      if constexpr (kF16)
        acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[k & 3], bh[(k >> 2) & 3], acc[x], 0, 0, 0);
      else
        acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[k & 3], bb[(k >> 2) & 3], acc[x], 0, 0, 0);
    }
  float s = 0.f;
  for (int x = 0; x < kBlocks; ++x)
    for (int r = 0; r < 16; ++r) s += acc[x][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  span.record();
}

// 2. LDS reads: 8 reads per iteration of one form, addresses moving with the
// iteration (so that nothing is hoisted), summed into a register.
//   kForm 0 ds_read_b32, 1 ds_read_b64, 2 ds_read_b128, 3 ds_read_b64_tr_b16
//   (the kernel's X pattern), 4 two b32 reads 512 bytes apart (ds_read2st64_b32).
template <int kForm>
__global__ void __launch_bounds__(256) lds_read(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  for (int i = threadIdx.x; i < 16384; i += 256) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 7);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    const int base = ((it * 4096) + w * 1024) & 65535;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int o = (base + u * 8192) & 49151;  // + at most 16 KiB - 1 below
      if constexpr (kForm == 0) acc += *(lds_f32*)((lds_u8*)lds + o + lane * 4);
      if constexpr (kForm == 1) {
        const f32x2_t v = *(lds_f32x2*)((lds_u8*)lds + o + lane * 8);
        acc += v.x + v.y;
      }
      if constexpr (kForm == 2) {
        const f32x4_t v = *(lds_f32x4*)((lds_u8*)lds + o + lane * 16);
        acc += v.x + v.w;
      }
      if constexpr (kForm == 3) {
        const int q = lane >> 4, j = lane & 15;
        const int t = 8 * (q >> 1) + (j >> 2);
        const int n = 16 * (q & 1) + 4 * (j & 3);
        const int off = t * 512 + (((n >> 3) ^ ((j >> 2) << 2)) << 4) + (n & 7) * 2;
        const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + o + off));
        acc += (float)(r.x + r.w);
      }
      if constexpr (kForm == 4) {
        const int oo = o + lane * 4;
        acc += *(lds_f32*)((lds_u8*)lds + oo) + *(lds_f32*)((lds_u8*)lds + oo + 512);
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// 3. Buffer loads that write LDS directly (16 bytes per lane), from a 1 MiB
// buffer that stays in L2.
__global__ void __launch_bounds__(256) lds_dma(const float* src, float* out, int iters) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[65536];
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), 0, 1 << 20, 0x00020000);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_u8*)lds + ((w * 16 + u) & 63) * 1024, 16,
                                               lane * 16 + (u & 7) * 1024, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0)
  }
  __syncthreads();
  out[blockIdx.x * 256 + threadIdx.x] = reinterpret_cast<float*>(lds)[threadIdx.x];
}

// 4. The G_W inner loop in isolation, per 16 tokens and wave (a 64 x 128 wave
// tile): A = 2 blocks of 32 rows of the token-major fp16 g operand, each by
// two transposed reads (ds_read_b64_tr_b16); B = 4 blocks of 32 columns of the
// 8-token-blocked fp16 x operand, one ds_read_b128 each; 8 MFMAs.  Two such
// steps per iteration (32 tokens, as one LDS stage of the kernel).  With
// kReads false the operands are read once before the loop, which leaves the
// matrix instructions and the loop's own overhead.
typedef __attribute__((address_space(3))) f16x8_t lds_f16x8;
template <bool kReads>
__global__ void __launch_bounds__(256) gw16_loop(float* out, int iters) {
  const ClockSpan span;
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  for (int i = threadIdx.x; i < 16384; i += 256) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 7);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  f32x16_t acc[2][4];
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
  const int aoff = (lane * 8) & 511;      // A reads end below 512 + 127 + 3072 + 8
  const int boff = 32768 + lane * 16;     // B reads end below 32768 + 1024 + 127 + 12288 + 16
  f16x8_t a[2][2], b[2][4];
  auto load = [&](int it, int h) {
    const int sw = ((it * 2 + h) & 7) << 4;
    for (int mb = 0; mb < 2; ++mb) {
      const i16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + (aoff ^ sw) + mb * 1024));
      const i16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + (aoff ^ sw) + mb * 1024 + 2048));
      a[h][mb] = __builtin_bit_cast(f16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    for (int nb = 0; nb < 4; ++nb)
      b[h][nb] = *(lds_f16x8*)((lds_u8*)lds + (boff ^ sw) + nb * 4096);
  };
  load(0, 0);
  load(0, 1);
  for (int it = 0; it < iters; ++it) {
    for (int h = 0; h < 2; ++h) {
      f16x8_t ah[2] = {a[h][0], a[h][1]}, bh[4] = {b[h][0], b[h][1], b[h][2], b[h][3]};
      if constexpr (kReads) load(it + 1, h);
      for (int mb = 0; mb < 2; ++mb)
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[mb], bh[nb], acc[mb][nb], 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 16; ++r) s += acc[x][y][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  span.record();
}

// Shader clock of the last timed launch, from the spans of its first `wgs`
// workgroups (at most 1024): s_memtime ticks over s_memrealtime time.
static double span_ghz(int wgs, double realtime_hz) {
  static unsigned long long h[1024 * 2];
  if (hipMemcpyFromSymbol(h, HIP_SYMBOL(g_clk), sizeof(h)) != hipSuccess) return 0.0;
  double c = 0.0, w = 0.0;
  for (int b = 0; b < wgs && b < 1024; ++b) {
    c += (double)h[2 * b];
    w += (double)h[2 * b + 1];
  }
  return w > 0.0 ? c / (w / realtime_hz) / 1e9 : 0.0;
}

static float time_ms(void (*launch)(float*, int, int), float* out, int wgs, int iters) {
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {  // the first run warms up
    (void)hipEventRecord(e0);
    launch(out, wgs, iters);
    (void)hipEventRecord(e1);
    (void)hipEventSynchronize(e1);
    (void)hipEventElapsedTime(&ms, e0, e1);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}

static const float* g_src = nullptr;

int main() {
  float* out;
  float* src;
  if (hipMalloc(&out, 4096 * 256 * sizeof(float)) != hipSuccess) return 1;
  if (hipMalloc(&src, 1 << 20) != hipSuccess) return 1;
  (void)hipMemset(src, 0, 1 << 20);
  g_src = src;
  const double mfma_flops = 2.0 * 32 * 32 * 16;  // per v_mfma_f32_32x32x16_bf16
  int rt_khz = 0;
  if (hipDeviceGetAttribute(&rt_khz, hipDeviceAttributeWallClockRate, 0) != hipSuccess || rt_khz <= 0)
    rt_khz = 100000;
  const double rt_hz = rt_khz * 1e3;

  printf("bf16 MFMA (v_mfma_f32_32x32x16_bf16), 16 independent per iteration:\n");
  for (int wgs : {256, 512, 1024}) {
    const int iters = 4096;
    const float ms = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(mfma_only, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters);
    const double fl = mfma_flops * 16.0 * iters * wgs * 4;
    printf("  %d wave(s)/SIMD  %.3f ms  %7.1f TFLOP/s  (%.2f GHz at 32 cycles per MFMA)\n",
           wgs / 256, ms, fl / ms / 1e9, 16.0 * iters * wgs * 4 / 1024 * 32 / (ms * 1e-3) / 1e9);
  }

  printf("MFMA 32x32x16 rate by operand type and accumulator blocks (32 per iteration, 1 wave/SIMD):\n");
  {
    const int iters = 2048, wgs = 256;
    const char* nm[4] = {"bf16,  8 blocks", "bf16, 16 blocks", "fp16,  8 blocks", "fp16, 16 blocks"};
    for (int v = 0; v < 4; ++v) {
      float ms = 0.f;
      switch (v) {
        case 0: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL((mfma_rate<false, 8>), dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        case 1: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL((mfma_rate<false, 16>), dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        case 2: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL((mfma_rate<true, 8>), dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        default: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL((mfma_rate<true, 16>), dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
      }
      const double fl = mfma_flops * 32.0 * iters * wgs * 4;
      printf("  %s  %.3f ms  %7.1f TFLOP/s  (%.2f GHz at 32 cycles per MFMA; s_memtime %.2f GHz)\n",
             nm[v], ms, fl / ms / 1e9, 32.0 * iters * wgs * 4 / 1024 * 32 / (ms * 1e-3) / 1e9,
             span_ghz(wgs, rt_hz));
    }
  }

  printf("LDS reads, bytes per clock per CU at 2.1 GHz (512 / 1024 workgroups of 256):\n");
  const char* names[5] = {"ds_read_b32", "ds_read_b64", "ds_read_b128", "ds_read_b64_tr_b16",
                          "ds_read2st64_b32"};
  const int bytes[5] = {4, 8, 16, 8, 8};
  for (int f = 0; f < 5; ++f)
    for (int wgs : {512, 1024}) {
      const int iters = 8192;
      float ms = 0.f;
      switch (f) {
        case 0: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL(lds_read<0>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        case 1: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL(lds_read<1>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        case 2: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL(lds_read<2>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        case 3: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL(lds_read<3>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
        default: ms = time_ms([](float* o, int g, int it) { hipLaunchKernelGGL(lds_read<4>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters); break;
      }
      const double b = (double)bytes[f] * 256 * 8 * iters * wgs;
      printf("  %-20s wgs %4d  %.3f ms  %6.1f TB/s  %6.1f B/clk/CU\n", names[f], wgs, ms,
             b / ms / 1e9, b / (ms * 1e-3) / 256 / 2.1e9);
    }

  printf("Buffer loads into LDS (16 B per lane, L2-resident source):\n");
  for (int wgs : {256, 512}) {
    const int iters = 2048;
    const float ms = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(lds_dma, dim3(g), dim3(256), 0, 0, g_src, o, it); }, out, wgs, iters);
    const double b = 1024.0 * 16 * 4 * iters * wgs;
    printf("  wgs %4d  %.3f ms  %6.1f TB/s  %6.1f B/clk/CU\n", wgs, ms, b / ms / 1e9,
           b / (ms * 1e-3) / 256 / 2.1e9);
  }

  printf("G_W inner loop alone (fp16, 64 x 128 per wave, 32 tokens per iteration):\n");
  for (int wgs : {256, 512}) {
    const int iters = 1024;
    const float ms0 = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(gw16_loop<true>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters);
    const double ghz0 = span_ghz(wgs, rt_hz);
    const float ms1 = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(gw16_loop<false>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters);
    const double ghz1 = span_ghz(wgs, rt_hz);
    const double fl = mfma_flops * 16.0 * iters * wgs * 4;
    printf("  %d wave(s)/SIMD, LDS reads in the loop  %.3f ms  %7.1f TFLOP/s  (s_memtime %.2f GHz)\n",
           wgs / 256, ms0, fl / ms0 / 1e9, ghz0);
    printf("  %d wave(s)/SIMD, matrix work only       %.3f ms  %7.1f TFLOP/s  (s_memtime %.2f GHz)\n",
           wgs / 256, ms1, fl / ms1 / 1e9, ghz1);
  }
  (void)hipFree(out);
  (void)hipFree(src);
  return 0;
}
