// dust_gemm.hip -- the weight gradient G_W = sum_t g_t x_t^T on the matrix cores.
//
// Paper digest, section 2.2: the error estimate's outer product with the layer
// input gives the weight gradient, in the same form as backprop.  As a matrix
// product, G[m][n] = sum_t g[t][m] X[t][n], contracting over the token axis,
// which is the slow axis of both row-major operands.
//
// Precision: g is fp32 and the product must keep ~fp32 accuracy.  Each fp32
// value v is split into two bf16 values hi = bf16(v), lo = bf16(v - hi) with
// |v - hi - lo| <= 2^-17 |v|, and the products run on the bf16 MFMA units with
// fp32 accumulation: g_hi X + g_lo X for bf16 X (exact in bf16), plus
// g_hi X_lo for fp32 X.  Every bf16 x bf16 product is exact in fp32.
//
// Data movement: both operands stay in their natural token-major layout.  Each
// pipeline step moves kBT token rows of a g tile (fp32) and of an X tile (bf16)
// straight from HBM into LDS with buffer loads that write LDS directly (no
// registers, hardware bounds checks give zeros past the end), into a ring of
// kS stages, so kS - 1 steps are in flight while the matrix cores work.  The
// operands of v_mfma_f32_32x32x16_bf16 want 8 consecutive tokens per lane:
//   X: ds_read_b64_tr_b16 gives each lane one column of a 4-token x 16-column
//      block of a token-major tile, two of them make the lane's 8 tokens;
//   g: eight ds_read_b32 (one per token) of the lane's column, then the hi/lo
//      split in registers.
// 16-byte chunks of each LDS row are xor-swizzled by the row index so that both
// read patterns hit distinct banks.
//
// Tiling: a workgroup (4 waves, one per SIMD) owns a 128 x 256 tile of G over
// one token range (split-K over tokens so that the grid fills the 256 CUs);
// each wave owns 64 x 128 as 2 x 4 MFMA blocks.  Partial tiles of the token
// splits are summed in a fixed order by a second kernel, so results are
// deterministic.  (Measured on MI355X: 128 x 256 tiles with a 4-stage ring beat
// 256 x 256 and 128 x 512 tiles; the loop is bound by the VALU work of the
// hi/lo split and the LDS reads issued between matrix instructions, not by
// HBM.)
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kBM = 128;   // rows of G (layer outputs) per workgroup
constexpr int kBN = 256;   // columns of G (layer inputs) per workgroup
constexpr int kWaveM = 64, kWaveN = 128;  // per wave: 2 x 4 blocks of 32 x 32
constexpr int kMB = kWaveM / 32, kNB = kWaveN / 32;
constexpr int kXcds = 8;   // MI355X: workgroups go round-robin to 8 XCDs
constexpr int kGRow = kBM * 4;  // bytes of one token row of the g tile (fp32)
constexpr int kXRow = kBN * 2;  // bytes of one token row of an X tile (bf16)
constexpr int kGRowsPerLoad = 1024 / kGRow;  // token rows per 1 KiB load
constexpr int kXRowsPerLoad = 1024 / kXRow;
static_assert((kBM / kWaveM) * (kBN / kWaveN) == 4, "four waves per workgroup, 2 x 2");
static_assert(kGRow >= 256 && kXRow >= 256 && kGRow <= 1024 && kXRow <= 1024, "row swizzles");

// Pipeline shape: tokens per step, stages in the LDS ring, workgroups per CU.
template <bool kXF32>
struct Pipe {
  static constexpr int kBT = 32;
  static constexpr int kS = kXF32 ? 3 : 4;
  static constexpr int kWgPerCu = 1;
  static constexpr int kPlanes = kXF32 ? 2 : 1;
  static constexpr int kGRegion = kBT * kGRow;   // bytes of g per step
  static constexpr int kXRegion = kBT * kXRow;   // bytes per X plane per step
  static constexpr int kStageBytes = kGRegion + kPlanes * kXRegion;
  static constexpr int kGLoads = kGRegion / 1024 / 4;  // 1 KiB loads per wave
  static constexpr int kXLoads = kXRegion / 1024 / 4;
  static constexpr int kLoadsPerStage = kGLoads + kPlanes * kXLoads;
};

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS ring.  The wait for this wave's LDS reads and
// the barrier are emitted as one asm statement with a memory clobber: the
// compiler keeps every memory access on its side of it, and no fence is
// involved (a release fence would also wait for the loads still in flight
// into the other stages).  Each wave has already waited for its own loads into
// the stage it is about to read (wait_vmcnt), so after the barrier every wave's
// part of that stage is in LDS.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from a buffer straight into LDS at lds + 16 * lane (the
// LDS base is taken from m0, so it must be uniform over the wave).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, lds_u8* lds, int voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, voff, soff, 0, 0);
}

// Two fp32 values -> packed bf16 hi and packed bf16 lo (v_cvt_pk_bf16_f32, round
// to nearest even): v = hi + lo + O(2^-17 |v|).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2_t v = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  const f32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

// Token-major copies for the operands the main kernel cannot read in place:
// X as bf16 planes [T][dp] (dp = d rounded up to 8; hi and, for fp32 X, lo),
// zero in the padding columns.  One thread per 8 columns of a row, grid-stride.
template <bool kXF32>
__global__ void __launch_bounds__(256) x_planes_kernel(const void* __restrict__ Xv, int64_t T,
                                                       int64_t d, int64_t dp,
                                                       uint16_t* __restrict__ hi,
                                                       uint16_t* __restrict__ lo) {
  const int64_t per_row = dp / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T * per_row; i += stride) {
    const int64_t t = i / per_row, c0 = (i % per_row) * 8;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t c = c0 + e;
      v[e] = 0.f;
      if (c < d) {
        if constexpr (kXF32) v[e] = reinterpret_cast<const float*>(Xv)[t * d + c];
        else v[e] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Xv)[t * d + c] << 16);
      }
    }
    uint4 h, l;
    if constexpr (kXF32) {
      split2(v[0], v[1], h.x, l.x);
      split2(v[2], v[3], h.y, l.y);
      split2(v[4], v[5], h.z, l.z);
      split2(v[6], v[7], h.w, l.w);
      *reinterpret_cast<uint4*>(lo + t * dp + c0) = l;
    } else {
      h.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xFFFF0000u);
      h.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xFFFF0000u);
      h.z = (__float_as_uint(v[4]) >> 16) | (__float_as_uint(v[5]) & 0xFFFF0000u);
      h.w = (__float_as_uint(v[6]) >> 16) | (__float_as_uint(v[7]) & 0xFFFF0000u);
    }
    *reinterpret_cast<uint4*>(hi + t * dp + c0) = h;
  }
}

// g [T][N] -> [T][Np] (Np = N rounded up to 4), zero padding; only for N % 4 != 0.
__global__ void __launch_bounds__(256) g_pad_kernel(const float* __restrict__ g, int64_t T,
                                                    int64_t N, int64_t Np, float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T * Np; i += stride) {
    const int64_t t = i / Np, c = i % Np;
    out[i] = c < N ? g[t * N + c] : 0.f;
  }
}

struct GemmGeom {
  int64_t M, Mp, Nd, dp, T, tiles_m, tiles_n, nsplit, t_per_split, groups, groups_per_xcd;
};

template <bool kXF32>
__global__ void __launch_bounds__(256, Pipe<kXF32>::kWgPerCu)
outer_sum_kernel(const float* __restrict__ g, const uint16_t* __restrict__ xh,
                 const uint16_t* __restrict__ xl, GemmGeom geo, float* __restrict__ out) {
  using P = Pipe<kXF32>;
  constexpr int kBT = P::kBT, kS = P::kS;
  // One array per ring stage: the compiler tracks the loads into each array
  // separately, so reading one stage waits only for the loads into that stage.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[P::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[P::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kS > 2 ? P::kStageBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kS > 3 ? P::kStageBytes : 16];
  lds_u8* const stages[4] = {(lds_u8*)st0, (lds_u8*)st1, (lds_u8*)st2, (lds_u8*)st3};

  // XCD-aware order (workgroup ids go round-robin over the 8 XCDs): each XCD
  // takes a contiguous range of (m tile, split) groups, split-major, so an XCD
  // works on as few token ranges as possible and reads their X rows from its
  // own L2; the tiles_n workgroups of one group share its g rows there too.
  const int64_t id = blockIdx.x;
  const int64_t xcd = id % kXcds, rank = id / kXcds;
  const int64_t group = xcd * geo.groups_per_xcd + rank / geo.tiles_n;
  if (group >= geo.groups) return;  // padding workgroup: leaves before any barrier
  const int64_t ntile = rank % geo.tiles_n;
  const int64_t mtile = group % geo.tiles_m, split = group / geo.tiles_m;
  const int m0 = (int)(mtile * kBM), n0 = (int)(ntile * kBN);
  const int64_t t_begin = split * geo.t_per_split;
  const int64_t t_end = min(geo.T, t_begin + geo.t_per_split);
  // Whole ring turns: the last split's extra steps read zeros.
  const int nsteps = (int)((t_end - t_begin + kS * kBT - 1) / (kS * kBT)) * kS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // Buffer resources over this split's token rows: loads past t_end read 0.
  // Columns past M (or d) in the last tile read the next row's values, which
  // reach only accumulator rows (columns) that are never stored.
  const int64_t t_rows = t_end - t_begin;
  const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(g + t_begin * geo.Mp), 0, (int)(t_rows * geo.Mp * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t xh_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xh + t_begin * geo.dp), 0, (int)(t_rows * geo.dp * 2), 0x00020000);
  __amdgpu_buffer_rsrc_t xl_rsrc = xh_rsrc;
  if constexpr (kXF32)
    xl_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xl + t_begin * geo.dp), 0,
                                                (int)(t_rows * geo.dp * 2), 0x00020000);

  // Loads: a 1 KiB load of a wave fills whole token rows of one tile; lane l
  // fetches the 16-byte chunk that lands at LDS position l.
  int g_voff[P::kGLoads], x_voff[P::kXLoads];
#pragma unroll
  for (int i = 0; i < P::kGLoads; ++i) {
    constexpr int kLanesPerRow = 64 / kGRowsPerLoad;
    const int row = (wave * P::kGLoads + i) * kGRowsPerLoad + lane / kLanesPerRow;
    const int gc = (lane % kLanesPerRow) ^ (((row >> 3) & 1) << 3);  // chunk = 4 fp32 columns
    g_voff[i] = (int)((row * geo.Mp + m0 + 4 * gc) * 4);
  }
#pragma unroll
  for (int i = 0; i < P::kXLoads; ++i) {
    constexpr int kLanesPerRow = 64 / kXRowsPerLoad;
    const int row = (wave * P::kXLoads + i) * kXRowsPerLoad + lane / kLanesPerRow;
    const int xc = (lane % kLanesPerRow) ^ ((row & 3) << 2);  // chunk = 8 bf16 columns
    x_voff[i] = (int)((row * geo.dp + n0 + 8 * xc) * 2);
  }
  auto issue = [&](lds_u8* st, int step) {
    const int tl = step * kBT;
    const int g_soff = (int)(tl * geo.Mp * 4), x_soff = (int)(tl * geo.dp * 2);
#pragma unroll
    for (int i = 0; i < P::kGLoads; ++i)
      load_lds16(g_rsrc, st + (wave * P::kGLoads + i) * 1024, g_voff[i], g_soff);
#pragma unroll
    for (int i = 0; i < P::kXLoads; ++i) {
      const int blk = P::kGRegion + (wave * P::kXLoads + i) * 1024;
      load_lds16(xh_rsrc, st + blk, x_voff[i], x_soff);
      if constexpr (kXF32) load_lds16(xl_rsrc, st + P::kXRegion + blk, x_voff[i], x_soff);
    }
  };

  // Fragment addresses (bytes within a stage, for kk = 0).
  //   g: lane reads column m = wm*128 + mb*32 + lane%32 of tokens 8*(lane/32) + e.
  //   X: lane group q = lane/16 reads tokens 8*(q/2) + 4*hh + (j/4) (j = lane%16)
  //      at columns wn*128 + nb*32 + 16*(q%2) + 4*(j%4) .. +3; the transposed read
  //      returns column wn*128 + nb*32 + lane%32 for tokens 8*(lane/32) + 4*hh + 0..3.
  int a_off[kMB], b_off[kNB];
  {
    const int h = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int m = wm * kWaveM + mb * 32 + (lane & 31);
      a_off[mb] = (8 * h) * kGRow + (((m >> 2) ^ (h << 3)) << 4) + (m & 3) * 4;
    }
    const int q = lane >> 4, j = lane & 15;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int t = 8 * (q >> 1) + (j >> 2);
      const int n = wn * kWaveN + nb * 32 + 16 * (q & 1) + 4 * (j & 3);
      b_off[nb] = P::kGRegion + t * kXRow + (((n >> 3) ^ ((j >> 2) << 2)) << 4) + (n & 7) * 2;
    }
  }

  f32x16_t acc[kMB][kNB];
#pragma unroll
  for (int a = 0; a < kMB; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Operands of 16 tokens: g as read (fp32, split just before use, so that the
  // reads stay in flight behind earlier matrix work) and X as bf16 fragments.
  struct Frag {
    float a[kMB][8];
    bf16x8_t bh[kNB], bl[kXF32 ? kNB : 1];
  };
  auto load = [&](lds_u8* st, int kk, Frag& f) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      lds_u8* p = st + b_off[nb] + kk * kXRow;
      const i16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * kXRow));
      f.bh[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (kXF32) {
        lds_u8* pl = p + P::kXRegion;
        const i16x4_t s0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pl);
        const i16x4_t s1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pl + 4 * kXRow));
        f.bl[nb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      lds_u8* p = st + a_off[mb] + kk * kGRow;
#pragma unroll
      for (int e = 0; e < 8; ++e) f.a[mb][e] = *(lds_f32*)(p + e * kGRow);
    }
  };
  auto mma = [&](const Frag& f) {
    bf16x8_t ah[kMB], al[kMB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split2(f.a[mb][2 * e], f.a[mb][2 * e + 1], h[e], l[e]);
      ah[mb] = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
      al[mb] = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], f.bh[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], f.bh[nb], acc[mb][nb], 0, 0, 0);
    if constexpr (kXF32) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], f.bl[nb], acc[mb][nb], 0, 0, 0);
    }
  };

  // Software pipeline over steps of kBT = 32 tokens (two halves of 16).  The
  // ring holds kS steps; every load is issued unconditionally (steps past the
  // split read zeros), so the wait counts are the same in every step and the
  // loop has no branches.  Step s, with the first half's operands already in
  // registers:
  //   read the second half of stage s;  matrix work on the first half;
  //   wait for this wave's loads of step s+1 (kS-2 later steps stay in flight);
  //   barrier: every wave's part of stage s+1 has landed and every wave has
  //   finished reading stage s;  refill stage s with step s+kS;
  //   read the first half of stage s+1;  matrix work on the second half.
  static_assert(kBT == 32, "two halves of 16 tokens per step");
  static_assert(kS >= 2 && kS <= 4, "ring of 2 to 4 stages");
  Frag f0, f1;
  auto step = [&](int i, int s) {  // i = s % kS, a constant at every call
    load(stages[i], 16, f1);
    mma(f0);
    wait_vmcnt<(kS - 2) * P::kLoadsPerStage>();
    ring_barrier();
    issue(stages[i], s + kS);
    load(stages[(i + 1) % kS], 0, f0);
    mma(f1);
  };

  issue(stages[0], 0);
  issue(stages[1], 1);
  if constexpr (kS > 2) issue(stages[2], 2);
  if constexpr (kS > 3) issue(stages[3], 3);
  wait_vmcnt<(kS - 1) * P::kLoadsPerStage>();
  ring_barrier();
  load(stages[0], 0, f0);
  for (int s0 = 0; s0 < nsteps; s0 += kS) {
    step(0, s0);
    step(1, s0 + 1);
    if constexpr (kS > 2) step(2, s0 + 2);
    if constexpr (kS > 3) step(3, s0 + 3);
  }
  wait_vmcnt<0>();  // the last kS (zero) loads land before the LDS is released

  // Register r of block (mb, nb) holds row 8*(r/4) + 4*(lane/32) + r%4 and
  // column lane%32 of that 32 x 32 block.
  float* o = out + split * geo.M * geo.Nd;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * kWaveM + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * kWaveN + nb * 32 + (lane & 31);
        if (m < geo.M && n < geo.Nd) o[m * geo.Nd + n] = acc[mb][nb][r];
      }
}

// G[e] = sum_s part[s][e] in split order (four elements per thread).
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* __restrict__ part,
                                                           int64_t nsplit, int64_t n,
                                                           float* __restrict__ G) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += stride) {
    float4 s = reinterpret_cast<const float4*>(part)[e];
    for (int64_t q = 1; q < nsplit; ++q) {
      const float4 v = reinterpret_cast<const float4*>(part + q * n)[e];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    reinterpret_cast<float4*>(G)[e] = s;
  }
  for (int64_t e = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    float s = part[e];
    for (int64_t q = 1; q < nsplit; ++q) s += part[q * n + e];
    G[e] = s;
  }
}

template <bool kXF32>
static GemmGeom plan_t(int64_t T, int64_t M, int64_t Nd) {
  using P = Pipe<kXF32>;
  GemmGeom g;
  g.M = M;
  g.Mp = (M + 3) / 4 * 4;
  g.Nd = Nd;
  g.dp = (Nd + 7) / 8 * 8;
  g.T = T;
  g.tiles_m = (M + kBM - 1) / kBM;
  g.tiles_n = (Nd + kBN - 1) / kBN;
  const int64_t tiles = g.tiles_m * g.tiles_n;
  // One wave of workgroups over the 256 CUs, with >= 1024 tokens per split.
  const int64_t slots = 256 * P::kWgPerCu;
  int64_t want = (slots + tiles - 1) / tiles;
  int64_t cap = (T + 1023) / 1024;
  if (cap < 1) cap = 1;
  int64_t ns = want < cap ? want : cap;
  if (ns < 1) ns = 1;
  int64_t per = (T + ns - 1) / ns;
  constexpr int64_t gran = P::kS * P::kBT;  // whole ring turns per split
  per = (per + gran - 1) / gran * gran;
  // 32-bit buffer offsets: one split's rows of g (and of X) stay below 2^31 bytes.
  const int64_t row_bytes = 4 * (g.Mp + kBM) > 2 * (g.dp + kBN) ? 4 * (g.Mp + kBM) : 2 * (g.dp + kBN);
  const int64_t per_max = ((((int64_t)1 << 31) - 1) / row_bytes - 3 * gran) / gran * gran;
  if (per > per_max) per = per_max > gran ? per_max : gran;
  g.t_per_split = per > 0 ? per : gran;
  g.nsplit = (T + g.t_per_split - 1) / g.t_per_split;
  if (g.nsplit < 1) g.nsplit = 1;
  g.groups = g.tiles_m * g.nsplit;
  g.groups_per_xcd = (g.groups + kXcds - 1) / kXcds;
  return g;
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace: X planes [T][dp] bf16 (hi, lo; used for fp32 X or d % 8 != 0),
// padded g [T][Np] (N % 4 != 0 only), split partials [S][N][d] fp32.
struct WsLayout {
  size_t plane, gpad, part;
};
static WsLayout ws_layout(int64_t T, int64_t N, int64_t d) {
  const GemmGeom a = plan_t<false>(T, N, d), b = plan_t<true>(T, N, d);
  const int64_t ns = a.nsplit > b.nsplit ? a.nsplit : b.nsplit;
  WsLayout w;
  w.plane = align256((size_t)T * (size_t)a.dp * 2);
  w.gpad = N % 4 ? align256((size_t)T * (size_t)a.Mp * 4) : 0;
  w.part = ns > 1 ? (size_t)ns * (size_t)N * (size_t)d * sizeof(float) : 0;
  return w;
}

bool outer_sum_supported(int64_t T, int64_t N, int64_t d) {
  // one workgroup per (tile, split): the grid's work-items must fit 32 bits
  const GemmGeom a = plan_t<false>(T, N, d), b = plan_t<true>(T, N, d);
  const int64_t na = a.groups_per_xcd * kXcds * a.tiles_n;
  const int64_t nb = b.groups_per_xcd * kXcds * b.tiles_n;
  return (na > nb ? na : nb) < ((int64_t)1 << 24);
}

size_t outer_sum_workspace_bytes(int64_t T, int64_t N, int64_t d) {
  const WsLayout w = ws_layout(T, N, d);
  return 2 * w.plane + w.gpad + w.part;
}

template <bool kXF32>
static hipError_t launch_gemm_t(const GemmGeom& geo, const float* g, const uint16_t* xh,
                                const uint16_t* xl, float* out, hipStream_t s) {
  const int64_t nwg = geo.groups_per_xcd * kXcds * geo.tiles_n;
  hipLaunchKernelGGL(outer_sum_kernel<kXF32>, dim3((uint32_t)nwg), dim3(256), 0, s, g, xh, xl, geo,
                     out);
  return hipGetLastError();
}

hipError_t launch_outer_sum(const float* g, const void* X, bool x_bf16, int64_t T, int64_t N,
                            int64_t d, float* G, void* workspace, hipStream_t s) {
  const GemmGeom geo = x_bf16 ? plan_t<false>(T, N, d) : plan_t<true>(T, N, d);
  const WsLayout w = ws_layout(T, N, d);
  char* ws = reinterpret_cast<char*>(workspace);
  uint16_t* ph = reinterpret_cast<uint16_t*>(ws);
  uint16_t* pl = reinterpret_cast<uint16_t*>(ws + w.plane);
  float* gpad = reinterpret_cast<float*>(ws + 2 * w.plane);
  float* part = reinterpret_cast<float*>(ws + 2 * w.plane + w.gpad);
  float* out = (geo.nsplit > 1) ? part : G;

  const uint16_t* xh = reinterpret_cast<const uint16_t*>(X);
  if (!x_bf16 || d % 8 != 0) {
    const int64_t n = T * (geo.dp / 8);
    const dim3 grid((uint32_t)(n / 256 < 16384 ? n / 256 + 1 : 16384));
    if (x_bf16)
      hipLaunchKernelGGL(x_planes_kernel<false>, grid, dim3(256), 0, s, X, T, d, geo.dp, ph, nullptr);
    else
      hipLaunchKernelGGL(x_planes_kernel<true>, grid, dim3(256), 0, s, X, T, d, geo.dp, ph, pl);
    xh = ph;
  }
  const float* gg = g;
  if (N % 4 != 0) {
    int64_t blocks = (T * geo.Mp + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(g_pad_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, g, T, N, geo.Mp, gpad);
    gg = gpad;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = x_bf16 ? launch_gemm_t<false>(geo, gg, xh, nullptr, out, s)
             : launch_gemm_t<true>(geo, gg, ph, pl, out, s);
  if (e != hipSuccess || geo.nsplit <= 1) return e;
  const int64_t n = N * d;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, part,
                     geo.nsplit, n, G);
  return hipGetLastError();
}

}  // namespace dust
