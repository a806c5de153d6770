// gemm_rates.hip -- throughput probes behind the design of the G_W kernel on
// gfx950: the bf16 matrix-core rate, the LDS read rates of the instruction
// forms the kernel can use, the rate of buffer loads that write LDS directly,
// and the G_W inner loop in isolation (LDS operands, MFMA), with the fp32 ->
// bf16 hi/lo split done in the loop or not.  Build and run:
//   python -m activation_perturbation_estimator_amd.probes gemm
// Every LDS address stays inside the kernel's own shared array; the loaded
// buffer is 1 MiB and every load offset stays below 8 KiB.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x2_t lds_f32x2;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2_t v = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  const f32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

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

// 4. The G_W inner loop in isolation, per 16 tokens and wave: A = 2 blocks of
// 32 rows (fp32, eight b32 reads each, split into hi/lo in the loop) or, with
// kPlanes, the same blocks as pre-split bf16 planes (transposed reads, no
// VALU); B = 4 blocks by transposed reads; 16 MFMAs.
template <bool kPlanes>
__global__ void __launch_bounds__(256, 1) gw_loop(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  for (int i = threadIdx.x; i < 16384; i += 256) reinterpret_cast<float*>(lds)[i] = 0.001f * (i & 7);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  f32x16_t acc[2][4];
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
  const int boff = 32768 + ((lane * 8) & 4095);                 // < 36864
  const int aoff = (lane & 31) * 4 + (lane >> 5) * 8192;        // < 8320
  float a[2][8];
  bf16x8_t ph[2], pl[2], b[4];
  auto load = [&](int it) {
    const int sw = (it & 7) << 4;
    for (int nb = 0; nb < 4; ++nb) {
      const i16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + (boff ^ sw) + nb * 1024));
      const i16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + (boff ^ sw) + nb * 1024 + 2048));
      b[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    for (int mb = 0; mb < 2; ++mb) {
      if constexpr (kPlanes) {
        const int o = ((boff - 32768) ^ sw) + mb * 1024;
        const i16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + o));
        const i16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + o + 2048));
        const i16x4_t l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + o + 16384));
        const i16x4_t l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_u8*)lds + o + 18432));
        ph[mb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        pl[mb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        for (int e = 0; e < 8; ++e) a[mb][e] = *(lds_f32*)((lds_u8*)lds + (aoff ^ sw) + mb * 128 + e * 1024);
      }
    }
  };
  load(0);
  for (int it = 0; it < iters; ++it) {
    bf16x8_t ah[2], al[2], bb[4];
    for (int mb = 0; mb < 2; ++mb) {
      if constexpr (kPlanes) {
        ah[mb] = ph[mb];
        al[mb] = pl[mb];
      } else {
        uint32_t h[4], l[4];
        for (int e = 0; e < 4; ++e) split2(a[mb][2 * e], a[mb][2 * e + 1], h[e], l[e]);
        ah[mb] = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
        al[mb] = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
      }
    }
    for (int nb = 0; nb < 4; ++nb) bb[nb] = b[nb];
    load(it + 1);
    for (int mb = 0; mb < 2; ++mb)
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bb[nb], acc[mb][nb], 0, 0, 0);
    for (int mb = 0; mb < 2; ++mb)
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bb[nb], acc[mb][nb], 0, 0, 0);
  }
  float s = 0.f;
  for (int x = 0; x < 2; ++x)
    for (int y = 0; y < 4; ++y)
      for (int r = 0; r < 16; ++r) s += acc[x][y][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
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

  printf("bf16 MFMA (v_mfma_f32_32x32x16_bf16), 16 independent per iteration:\n");
  for (int wgs : {256, 512, 1024}) {
    const int iters = 4096;
    const float ms = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(mfma_only, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters);
    const double fl = mfma_flops * 16.0 * iters * wgs * 4;
    printf("  %d wave(s)/SIMD  %.3f ms  %7.1f TFLOP/s  (%.2f GHz at 32 cycles per MFMA)\n",
           wgs / 256, ms, fl / ms / 1e9, 16.0 * iters * wgs * 4 / 1024 * 32 / (ms * 1e-3) / 1e9);
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

  printf("G_W inner loop alone (1 wave/SIMD, 64 x 128 per wave, 16 tokens per iteration):\n");
  {
    const int iters = 2048, wgs = 256;
    const float ms0 = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(gw_loop<false>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters);
    const float ms1 = time_ms([](float* o, int g, int it) {
      hipLaunchKernelGGL(gw_loop<true>, dim3(g), dim3(256), 0, 0, o, it); }, out, wgs, iters);
    const double fl = mfma_flops * 16.0 * iters * wgs * 4;
    printf("  fp32 A, hi/lo split in the loop   %.3f ms  %7.1f TFLOP/s\n", ms0, fl / ms0 / 1e9);
    printf("  bf16 hi/lo planes, no VALU        %.3f ms  %7.1f TFLOP/s\n", ms1, fl / ms1 / 1e9);
  }
  (void)hipFree(out);
  (void)hipFree(src);
  return 0;
}
