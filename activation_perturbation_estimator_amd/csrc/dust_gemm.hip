// dust_gemm.hip -- the weight gradient G_W = sum_t g_t x_t^T on the matrix cores.
//
// Paper digest, section 2.2: the error estimate's outer product with the layer
// input gives the weight gradient, in the same form as backprop.  As a matrix
// product, G[m][n] = sum_t g[t][m] X[t][n], contracting over the token axis.
//
// Precision: one pass of v_mfma_f32_32x32x16_f16 (fp32 accumulation) over the
// fp16 operand form of dust_gemm16.hpp: every token's rows rescaled by a power
// of two (exact) and rounded to fp16 (11 significant bits; bf16 X is exact),
// so each product g_t[m] x_t[n] carries a relative error <= 2^-11 (2^-10 for
// fp32 X), independent between tokens.  Tokens whose range fits no power of
// two (or with non-finite values) are added afterwards in fp32 from the
// original g and X.
//
// Data movement: the kernel reads only the fp16 operands, written by the
// kernels that produce g (or by prep16_kernel for a caller's fp32 g):
//   g16 [T][Mp] token-major: each pipeline step moves 32 token rows of a
//       256-column tile into LDS; ds_read_b64_tr_b16 gives a lane one column
//       of a 4-token x 16-column block, two of them the lane's 8 tokens of a
//       v_mfma_f32_32x32x16_f16 operand.  16-byte chunks of each LDS row are
//       xor-swizzled by the row index so that the reads hit distinct banks.
//   x16 [T/8][d][8] blocked: each column's 8 tokens are one 16-byte chunk,
//       exactly a lane's operand, read with one ds_read_b128.
// Both go from HBM straight into LDS with buffer loads that write LDS (no
// registers), into a ring of kS stages, so kS - 1 steps are in flight while
// the matrix cores work.  Every offset of a load is in its vector offset, so
// the buffer's bounds check covers all of it: loads past a token split's rows
// return zeros.
//
// Tiling: a workgroup of kWavesM x kWavesN waves owns a kWavesM kWM x kWavesN kWN
// tile of G over one token range (split-K over tokens so that the grid fills
// the 256 CUs); each wave owns kWM x kWN as kWM/32 x kWN/32 MFMA blocks.  The
// built configurations (WideCfg, NarrowCfg below): waves of 64 x 128 on
// 256 x 256 or 256 x 128 tiles, 32 tokens per pipeline step, a ring of 4
// steps (128 or 96 KiB of LDS).  Partial tiles of the token splits are summed
// in a fixed order by a second kernel, so results are deterministic.
#include <type_traits>

#include "dust_device.hpp"
#include "dust_gemm16.hpp"
#include "dust_launch.hpp"

namespace dust {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) f16x8_t lds_f16x8;

constexpr int kXcds = 8;  // MI355X: workgroups go round-robin to 8 XCDs

// A workgroup of kWavesM x kWavesN waves owns a (kWavesM kWM) x (kWavesN kWN)
// tile of G; each wave owns kWM x kWN as (kWM/32) x (kWN/32) MFMA blocks.  A
// pipeline step moves kBT tokens of both operands into one of kS LDS stages.
template <int kWavesM_, int kWavesN_, int kWM_, int kWN_, int kBT_, int kS_>
struct Cfg {
  static constexpr int kWavesM = kWavesM_, kWavesN = kWavesN_;
  static constexpr int kWaves = kWavesM * kWavesN, kThreads = 64 * kWaves;
  static constexpr int kWM = kWM_, kWN = kWN_;
  static constexpr int kBM = kWavesM * kWM, kBN = kWavesN * kWN;
  static constexpr int kMB = kWM / 32, kNB = kWN / 32;
  static constexpr int kBT = kBT_, kS = kS_;
  static constexpr int kSub = kBT / 16;           // MFMA k-steps of 16 tokens per step
  static constexpr int kARow = kBM * 2;           // bytes of one token row of the g tile
  static constexpr int kARegion = kBT * kARow;    // g bytes per stage
  static constexpr int kXRegion = (kBT / 8) * kBN * 16;  // x bytes per stage
  static constexpr int kStage = kARegion + kXRegion;
  static constexpr int kALoads = kARegion / (1024 * kWaves);  // 1 KiB loads per wave, stage
  static constexpr int kXLoads = kXRegion / (1024 * kWaves);
  static constexpr int kLoads = kALoads + kXLoads;
  static constexpr int kARowsPerLoad = 1024 / kARow;
  static constexpr int kALanesPerRow = 64 / kARowsPerLoad;  // 16-byte chunks per g-tile row
  static_assert(kALanesPerRow >= 16, "the row swizzle xors chunk indices with up to 12");
  static_assert(kARow <= 1024, "a 1 KiB load holds whole g-tile rows");
  static_assert(kARegion % (1024 * kWaves) == 0 && kXRegion % (1024 * kWaves) == 0,
                "whole 1 KiB loads per wave");
  static_assert(kBT % 16 == 0 && kSub >= 2, "at least two MFMA k-steps per pipeline step");
  static_assert(kS >= 2 && kS <= 4, "ring of 2 to 4 stages");
  static_assert(kS * kStage <= 160 * 1024, "LDS of one CU");
};

// Workgroups per launch: one per two CUs.  On a full grid the burst of
// matrix work at the end of each estimate (changing fp16 data through LDS on
// every CU) pulls the shader clock of some MI355X parts down, from about 2.38
// to 2.12-2.16 GHz, for the whole of the next call's VALU-bound head kernel
// (10% of the step); on half the CUs the same parts keep 2.37-2.39 GHz, and
// the G_W stage itself takes about 20 us longer.
constexpr int64_t kGemmGridTarget = 128;

// Two tile shapes, chosen per call (plan16): 256 x 256 tiles (8 waves, two per
// SIMD, of 64 x 128) reach the grid target with at most 8 token splits when
// the output has at least 16 such tiles (N d >= 2^20); smaller outputs take
// 256 x 128 tiles (4 waves of 64 x 128), which need half the splits and so
// half the partial bytes.
using WideCfg = Cfg<4, 2, 64, 128, 32, 4>;
using NarrowCfg = Cfg<4, 1, 64, 128, 32, 4>;

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
// LDS base is taken from m0, so it must be uniform over the wave).  The whole
// offset is the lane's vector offset: a chunk at or past the buffer's size
// reads as zeros.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, lds_u8* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, voff, 0, 0, 0);
}

// fp16 operand form of a caller's fp32 g (dust_outer_sum): one workgroup of
// 256 threads per token, the same scale rule as the producer kernels.
__global__ void __launch_bounds__(256) prep16_kernel(const float* __restrict__ g, int64_t N,
                                                     Gemm16Out o) {
  __shared__ float red[12];
  const int64_t t = blockIdx.x;
  const float* grow = g + t * N;
  float gm = 0.f, xm = 0.f, nf = 0.f;
  for (int64_t c = threadIdx.x; c < N; c += 256) {
    const float v = grow[c];
    gm = fmaxf(gm, __builtin_fabsf(v));
    if (not_finite(v)) nf = 1.f;
  }
  for (int64_t k = threadIdx.x; k < o.d; k += 256) {
    const float v = load_x(o.X, o.x_bf16, t * o.d + k);
    xm = fmaxf(xm, __builtin_fabsf(v));
    if (not_finite(v)) nf = 1.f;
  }
  gm = wave_max(gm);
  xm = wave_max(xm);
  nf = wave_max(nf);
  group_max3<4>(gm, xm, nf, red);
  int s;
  const int mode = choose_scale(gm, xm, nf > 0.f, s);
  uint16_t* out = o.g16 + t * o.Mp;
  for (int64_t c = threadIdx.x; c < o.Mp; c += 256)
    out[c] = (mode == 0 && c < N) ? f16_bits(__builtin_ldexpf(grow[c], -s)) : (uint16_t)0;
  emit_x_row(o, t, mode, s, 256);
  if (threadIdx.x == 0) o.flags[t] = mode == 2 ? 1 : 0;
}

struct Gemm16Geom {
  int64_t M, Mp, d, T, tiles_m, tiles_n, nsplit, t_per_split, groups, groups_per_xcd;
  int64_t pstride;  // elements between the partial tiles of consecutive splits
  int wide;         // WideCfg (1) or NarrowCfg (0)
};

template <typename C>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm16_kernel(const uint16_t* __restrict__ g16, const uint16_t* __restrict__ x16,
              const uint8_t* __restrict__ flags, Gemm16Geom geo, float* __restrict__ part,
              int32_t* __restrict__ list, int32_t* __restrict__ count) {
  constexpr int kBT = C::kBT, kS = C::kS, kMB = C::kMB, kNB = C::kNB, kWM = C::kWM;
  // One array per ring stage: the compiler tracks the loads into each array
  // separately, so reading one stage waits only for the loads into that stage.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[C::kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kS > 2 ? C::kStage : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kS > 3 ? C::kStage : 16];
  lds_u8* const stages[4] = {(lds_u8*)st0, (lds_u8*)st1, (lds_u8*)st2, (lds_u8*)st3};

  // XCD-aware order (workgroup ids go round-robin over the 8 XCDs): each XCD
  // takes a contiguous range of (m tile, split) groups, split-major, so an XCD
  // works on as few token ranges as possible and reads their x rows from its
  // own L2; the tiles_n workgroups of one group share its g rows there too.
  const int64_t id = blockIdx.x;
  const int64_t xcd = id % kXcds, rank = id / kXcds;
  const int64_t group = xcd * geo.groups_per_xcd + rank / geo.tiles_n;
  if (group >= geo.groups) return;  // padding workgroup: leaves before any barrier
  const int64_t ntile = rank % geo.tiles_n;
  const int64_t mtile = group % geo.tiles_m, split = group / geo.tiles_m;
  const int m0 = (int)(mtile * C::kBM), n0 = (int)(ntile * C::kBN);
  const int64_t t_begin = split * geo.t_per_split;  // a multiple of 8
  const int64_t t_end = min(geo.T, t_begin + geo.t_per_split);
  const int64_t t_rows = t_end - t_begin;
  // Whole ring turns: the last split's extra steps read zeros.
  const int nsteps = (int)((t_rows + kS * kBT - 1) / (kS * kBT)) * kS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::kWavesM, wn = wave / C::kWavesM;

  // The split's flags (4 per word; bytes past the split read as 0), the first
  // kEarlyWords words per thread loaded now by the workgroup that lists them.
  const bool lister = (mtile == 0 && ntile == 0);
  auto flag_word = [&](int64_t i) -> uint32_t {  // flags of tokens t_begin + i .. + 3
    const uint32_t v = *reinterpret_cast<const uint32_t*>(flags + t_begin + i);
    return (t_rows - i >= 4) ? v : (v & ((1u << (8 * (t_rows - i))) - 1u));
  };
  constexpr int kEarlyWords = (2048 / 4 + C::kThreads - 1) / C::kThreads;
  uint32_t fbits = 0u;
  if (lister) {
#pragma unroll
    for (int w = 0; w < kEarlyWords; ++w) {
      const int64_t i = ((int64_t)w * C::kThreads + tid) * 4;
      if (i < t_rows) fbits |= flag_word(i);
    }
  }

  // Buffer resources over this split's rows of g16 and token groups of x16.
  // Columns past M (or d) in the last tile read the next row's (group's)
  // values, which reach only accumulator rows (columns) that are never stored.
  const int64_t Mp = geo.Mp, d = geo.d;
  const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(g16 + t_begin * Mp), 0, (int)(t_rows * Mp * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x16 + (t_begin >> 3) * d * 8), 0, (int)(((t_rows + 7) >> 3) * d * 16),
      0x00020000);

  // Load offsets at step 0; a 1 KiB load of a wave fills whole token rows of
  // the g tile (lane l fetches the chunk that lands at LDS position l), or 64
  // consecutive column chunks of one token group of the x tile.
  int a_voff[C::kALoads], x_voff[C::kXLoads];
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i) {
    const int row = (wave * C::kALoads + i) * C::kARowsPerLoad + lane / C::kALanesPerRow;
    const int gc = (lane % C::kALanesPerRow) ^ ((row & 3) << 2);  // chunk = 8 fp16 columns
    a_voff[i] = (int)((row * Mp + m0 + 8 * gc) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::kXLoads; ++i) {
    const int chunk = (wave * C::kXLoads + i) * 64 + lane;
    const int grp = chunk / C::kBN, col = chunk % C::kBN;
    x_voff[i] = (int)((grp * d + n0 + col) * 16);
  }
  const int a_step = (int)(kBT * Mp * 2), x_step = (int)((kBT / 8) * d * 16);
  auto issue = [&](lds_u8* st, int step) {
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i)
      load_lds16(g_rsrc, st + (wave * C::kALoads + i) * 1024, a_voff[i] + step * a_step);
#pragma unroll
    for (int i = 0; i < C::kXLoads; ++i)
      load_lds16(x_rsrc, st + C::kARegion + (wave * C::kXLoads + i) * 1024,
                 x_voff[i] + step * x_step);
  };

  // Fragment addresses (bytes within a stage, first 16 tokens).
  //   g: lane group q = lane/16 reads tokens 8*(q/2) + (j/4) (j = lane%16), and
  //      4 tokens later, at columns wm*kWM + mb*32 + 16*(q%2) + 4*(j%4) .. +3;
  //      the transposed reads return column wm*kWM + mb*32 + lane%32 for tokens
  //      8*(lane/32) + 0..7.
  //   x: lane reads the chunk of token group lane/32 and column
  //      wn*128 + nb*32 + lane%32: tokens 8*(lane/32) + 0..7 of that column.
  int a_off[kMB], b_off[kNB];
  {
    const int q = lane >> 4, j = lane & 15;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int t = 8 * (q >> 1) + (j >> 2);
      const int m = wm * kWM + mb * 32 + 16 * (q & 1) + 4 * (j & 3);
      a_off[mb] = t * C::kARow + (((m >> 3) ^ ((j >> 2) << 2)) << 4) + (m & 7) * 2;
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      b_off[nb] = C::kARegion + ((lane >> 5) * C::kBN + wn * C::kWN + nb * 32 + (lane & 31)) * 16;
  }

  f32x16_t acc[kMB][kNB];
#pragma unroll
  for (int a = 0; a < kMB; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  struct Frag {
    f16x4_t a[kMB][2];  // tokens 0..3 and 4..7 of the lane's eight
    f16x8_t b[kNB];
  };
  // Read number k (< kReads) of one k-step's fragments from stage st, in the
  // order the k-step's matrix instructions use them (row block by row block,
  // each against every column block): the two transposed reads of g block 0,
  // the x chunk of every column block, then the g blocks 1, 2, ...
  constexpr int kReads = kMB * 2 + kNB;  // LDS read instructions per k-step
  constexpr int kMfma = kMB * kNB;       // matrix instructions per k-step
  auto read = [&](lds_u8* st, int kk, Frag& f, int k) {
    if (k < 2 || k >= 2 + kNB) {
      const int ka = k < 2 ? k : k - kNB;  // index among the 2 kMB g reads
      const int mb = ka >> 1;
      lds_u8* p = st + a_off[mb] + kk * 16 * C::kARow + (ka & 1) * 4 * C::kARow;
      f.a[mb][ka & 1] =
          __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
    } else {
      const int nb = k - 2;
      f.b[nb] = *(lds_f16x8*)(st + b_off[nb] + kk * 2 * C::kBN * 16);
    }
  };
  auto mfma = [&](const Frag& f, int k) {
    const int mb = k / kNB, nb = k % kNB;
    const f16x8_t a = __builtin_shufflevector(f.a[mb][0], f.a[mb][1], 0, 1, 2, 3, 4, 5, 6, 7);
    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, f.b[nb], acc[mb][nb], 0, 0, 0);
  };
  auto refill = [&](lds_u8* st, int q, int step) {  // load q (< kLoads) of a stage refill
    if (q < C::kALoads)
      load_lds16(g_rsrc, st + (wave * C::kALoads + q) * 1024, a_voff[q] + step * a_step);
    else
      load_lds16(x_rsrc, st + C::kARegion + (wave * C::kXLoads + (q - C::kALoads)) * 1024,
                 x_voff[q - C::kALoads] + step * x_step);
  };

  // Software pipeline over steps of kBT tokens (kSub k-steps of 16).  The ring
  // holds kS steps; every load is issued unconditionally (steps past the split
  // read zeros), so the wait counts are the same in every step and the loop
  // has no branches.  Step s, with its first k-step's operands in registers:
  //   k-steps 0 .. kSub-2: matrix work, each instruction followed by its share
  //   of the reads of the next k-step of stage s;
  //   wait for this wave's loads of step s+1 (kS-2 later steps stay in flight);
  //   barrier: every wave's part of stage s+1 has landed and every wave has
  //   finished reading stage s;
  //   k-step kSub-1: matrix work, each instruction followed by its share of
  //   the loads refilling stage s with step s+kS and of the reads of the first
  //   k-step of stage s+1.
  // sched_barrier keeps this order: the reads are in flight behind independent
  // matrix work, not issued next to the instruction that consumes them.
  Frag f[2];
  auto step = [&](int i, int s) {  // i = s % kS, a constant at every call
    lds_u8* st = stages[i];
    lds_u8* nx = stages[(i + 1) % kS];
#pragma unroll
    for (int j = 0; j + 1 < C::kSub; ++j) {
#pragma unroll
      for (int k = 0; k < kMfma; ++k) {
        mfma(f[j & 1], k);
#pragma unroll
        for (int r = k * kReads / kMfma; r < (k + 1) * kReads / kMfma; ++r)
          read(st, j + 1, f[(j + 1) & 1], r);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vmcnt<(kS - 2) * C::kLoads>();
    ring_barrier();
    constexpr int jl = C::kSub - 1;
#pragma unroll
    for (int k = 0; k < kMfma; ++k) {
      mfma(f[jl & 1], k);
#pragma unroll
      for (int q = k * C::kLoads / kMfma; q < (k + 1) * C::kLoads / kMfma; ++q)
        refill(st, q, s + kS);
#pragma unroll
      for (int r = k * kReads / kMfma; r < (k + 1) * kReads / kMfma; ++r)
        read(nx, 0, f[(jl + 1) & 1], r);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  static_assert(C::kSub % 2 == 0, "the fragment buffers alternate, so a step holds an even "
                "number of k-steps");

  issue(stages[0], 0);
  issue(stages[1], 1);
  if constexpr (kS > 2) issue(stages[2], 2);
  if constexpr (kS > 3) issue(stages[3], 3);
  wait_vmcnt<(kS - 1) * C::kLoads>();
  ring_barrier();
#pragma unroll
  for (int k = 0; k < kReads; ++k) read(stages[0], 0, f[0], k);
  for (int s0 = 0; s0 < nsteps; s0 += kS) {
    step(0, s0);
    step(1, s0 + 1);
    if constexpr (kS > 2) step(2, s0 + 2);
    if constexpr (kS > 3) step(3, s0 + 3);
  }
  wait_vmcnt<0>();  // the last kS (zero) loads land before the LDS is released

  // Register r of block (mb, nb) holds row 8*(r/4) + 4*(lane/32) + r%4 and
  // column lane%32 of that 32 x 32 block.
  auto row_of = [&](int mb, int r) {
    return (int64_t)m0 + wm * kWM + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  };
  auto col_of = [&](int nb) { return (int64_t)n0 + wn * C::kWN + nb * 32 + (lane & 31); };

  float* o = part + split * geo.pstride;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = row_of(mb, r), n = col_of(nb);
        if (m < geo.M && n < d) o[m * d + n] = acc[mb][nb][r];
      }

  // One workgroup per split lists the split's tokens left out of the fp16
  // operands, in token order, for the exact fp32 pass of split_finish_kernel.
  // Its first flag words were loaded before the main loop (fbits); a split with
  // no flag set (the usual case) only writes its count.
  if (lister) {
    for (int64_t i = ((int64_t)kEarlyWords * C::kThreads + tid) * 4; i < t_rows;
         i += (int64_t)C::kThreads * 4)
      fbits |= flag_word(i);
    if (!__syncthreads_or(fbits != 0u)) {
      if (tid == 0) count[split] = 0;
      return;
    }
  }
  if (lister) {
    __shared__ int wsum[C::kWaves];
    int base = 0;
    for (int64_t c0 = 0; c0 < t_rows; c0 += C::kThreads) {
      const int64_t i = c0 + tid;
      const int fl = (i < t_rows) ? flags[t_begin + i] : 0;
      const uint64_t bal = __ballot(fl);
      if (lane == 0) wsum[wave] = __popcll(bal);
      __syncthreads();
      int off = base, all = 0;
      for (int w = 0; w < C::kWaves; ++w) {
        off += w < wave ? wsum[w] : 0;
        all += wsum[w];
      }
      if (fl) list[t_begin + off + __popcll(bal & ((1ull << lane) - 1ull))] = (int32_t)(t_begin + i);
      base += all;
      __syncthreads();
    }
    if (tid == 0) count[split] = base;
  }
}

// G[e] = sum_s part[s][e] in split order, then plus g[t][m] x[t][n] in fp32 for
// each token the fp16 operands left out (split by split, in token order).
// Four elements per thread.
__global__ void __launch_bounds__(256) split_finish_kernel(const float* __restrict__ part,
                                                     int64_t nsplit, int64_t pstride, int64_t M,
                                                     int64_t d, const int32_t* __restrict__ list,
                                                     const int32_t* __restrict__ count,
                                                     int64_t t_per_split,
                                                     const float* __restrict__ g32,
                                                     const void* __restrict__ X, int x_bf16,
                                                     float* __restrict__ G) {
  // Whether any split left tokens to the exact pass: the counts are the same
  // for every thread, read without a barrier so that their latency overlaps the
  // partial loads below; the first 8 in one go (the count region holds at
  // least 64 entries, so reading 8 stays inside it).
  int any = 0;
  {
    const int4 c0 = reinterpret_cast<const int4*>(count)[0];
    const int4 c1 = reinterpret_cast<const int4*>(count)[1];
    const int c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) any |= (q < nsplit) ? c[q] : 0;
    for (int64_t q = 8; q < nsplit; ++q) any |= count[q];
  }
  const int64_t n = M * d;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 4 * e4 < n; e4 += stride) {
    const int64_t e = 4 * e4;
    float v[4];
    if (e + 4 <= n) {
      // split order (0 + p0 = p0 exactly); four partials loaded at a time so
      // that their reads overlap: the usual 4 or 8 splits take 1 or 2 round trips
      float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
      int64_t q = 0;
      for (; q + 4 <= nsplit; q += 4) {
        float4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = reinterpret_cast<const float4*>(part + (q + u) * pstride)[e4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s.x += w[u].x; s.y += w[u].y; s.z += w[u].z; s.w += w[u].w;
        }
      }
      for (; q < nsplit; ++q) {
        const float4 w = reinterpret_cast<const float4*>(part + q * pstride)[e4];
        s.x += w.x; s.y += w.y; s.z += w.z; s.w += w.w;
      }
      v[0] = s.x; v[1] = s.y; v[2] = s.z; v[3] = s.w;
    } else {
      for (int k = 0; k < 4; ++k) {
        v[k] = 0.f;
        if (e + k < n)
          for (int64_t q = 0; q < nsplit; ++q) v[k] += part[q * pstride + e + k];
      }
    }
    if (any) {
      for (int k = 0; k < 4 && e + k < n; ++k) {
        const int64_t m = (e + k) / d, c = (e + k) % d;
        for (int64_t q = 0; q < nsplit; ++q) {
          const int32_t* lq = list + q * t_per_split;
          for (int i = 0; i < count[q]; ++i) {
            const int64_t t = lq[i];
            v[k] = fmaf(g32[t * M + m], load_x(X, x_bf16, t * d + c), v[k]);
          }
        }
      }
    }
    if (e + 4 <= n) {
      reinterpret_cast<float4*>(G)[e4] = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int k = 0; k < 4 && e + k < n; ++k) G[e + k] = v[k];
    }
  }
}

template <typename C>
static Gemm16Geom plan16_t(int64_t T, int64_t M, int64_t d) {
  Gemm16Geom g;
  g.M = M;
  g.Mp = (M + 7) / 8 * 8;
  g.d = d;
  g.T = T;
  g.tiles_m = (M + C::kBM - 1) / C::kBM;
  g.tiles_n = (d + C::kBN - 1) / C::kBN;
  const int64_t tiles = g.tiles_m * g.tiles_n;
  // kGemmGridTarget workgroups, with >= 1024 tokens per split.
  int64_t want = (kGemmGridTarget + tiles - 1) / tiles;
  int64_t cap = (T + 1023) / 1024;
  if (cap < 1) cap = 1;
  int64_t ns = want < cap ? want : cap;
  if (ns < 1) ns = 1;
  int64_t per = (T + ns - 1) / ns;
  constexpr int64_t gran = C::kS * C::kBT;  // whole ring turns per split
  per = (per + gran - 1) / gran * gran;
  // 32-bit buffer offsets: over a split's rows of g16 and token groups of
  // x16, plus the three ring steps of prefetch past them and the column
  // overrun of the last tile (one row of g16, one group of x16), every offset
  // stays below 2^31 bytes: 2 W (per + 3 gran) + o (W + tile width) < 2^31,
  // W = Mp and o = 2 for g16, W = d and o = 16 for x16.
  auto per_limit = [&](int64_t W, int64_t B, int64_t o) {
    return ((((int64_t)1 << 31) - 1 - o * (W + B)) / (2 * W) - 3 * gran) / gran * gran;
  };
  const int64_t lim_g = per_limit(g.Mp, C::kBM, 2), lim_x = per_limit(d, C::kBN, 16);
  const int64_t per_max = lim_g < lim_x ? lim_g : lim_x;
  if (per > per_max) per = per_max > gran ? per_max : gran;
  g.t_per_split = per > 0 ? per : gran;
  g.nsplit = (T + g.t_per_split - 1) / g.t_per_split;
  if (g.nsplit < 1) g.nsplit = 1;
  g.groups = g.tiles_m * g.nsplit;
  g.groups_per_xcd = (g.groups + kXcds - 1) / kXcds;
  g.pstride = (M * d + 63) / 64 * 64;
  g.wide = std::is_same<C, WideCfg>::value ? 1 : 0;
  return g;
}

static Gemm16Geom plan16(int64_t T, int64_t M, int64_t d) {
  const Gemm16Geom w = plan16_t<WideCfg>(T, M, d);
  return w.nsplit <= 8 ? w : plan16_t<NarrowCfg>(T, M, d);
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace: g16 [T][Mp], x16 [ceil(T/8)][d][8], flags [T], the per-split
// lists of left-out tokens [T] int32 and their counts [S], the split partials
// [S][pstride] fp32.
struct WsLayout {
  size_t g16, x16, flags, list, count, part;
  size_t total() const { return g16 + x16 + flags + list + count + part; }
};
static WsLayout ws_layout(int64_t T, int64_t N, int64_t d) {
  const Gemm16Geom a = plan16(T, N, d);
  WsLayout w;
  w.g16 = align256((size_t)T * (size_t)a.Mp * 2);
  w.x16 = align256((size_t)((T + 7) / 8) * (size_t)d * 16);
  w.flags = align256((size_t)T);
  w.list = align256((size_t)T * 4);
  w.count = align256((size_t)a.nsplit * 4);
  w.part = (size_t)a.nsplit * (size_t)a.pstride * sizeof(float);
  return w;
}

bool outer_sum_supported(int64_t T, int64_t N, int64_t d) {
  // one workgroup per (tile, split): the grid's work-items must fit 32 bits
  const Gemm16Geom a = plan16(T, N, d);
  return a.groups_per_xcd * kXcds * a.tiles_n < ((int64_t)1 << 24);
}

size_t outer_sum_workspace_bytes(int64_t T, int64_t N, int64_t d) {
  return ws_layout(T, N, d).total();
}

Gemm16Out outer_sum_operands(void* workspace, int64_t T, int64_t N, int64_t d, const void* X,
                             bool x_bf16) {
  const WsLayout w = ws_layout(T, N, d);
  char* ws = reinterpret_cast<char*>(workspace);
  Gemm16Out o;
  o.g16 = reinterpret_cast<uint16_t*>(ws);
  o.x16 = reinterpret_cast<uint16_t*>(ws + w.g16);
  o.flags = reinterpret_cast<uint8_t*>(ws + w.g16 + w.x16);
  o.X = X;
  o.T = T;
  o.Mp = (N + 7) / 8 * 8;
  o.d = d;
  o.x_bf16 = x_bf16 ? 1 : 0;
  return o;
}

hipError_t launch_outer_sum16(const Gemm16Out& o, const float* g32, int64_t N, float* G,
                              void* workspace, hipStream_t s) {
  const Gemm16Geom geo = plan16(o.T, N, o.d);
  const WsLayout w = ws_layout(o.T, N, o.d);
  char* ws = reinterpret_cast<char*>(workspace) + w.g16 + w.x16 + w.flags;
  int32_t* list = reinterpret_cast<int32_t*>(ws);
  int32_t* count = reinterpret_cast<int32_t*>(ws + w.list);
  float* part = reinterpret_cast<float*>(ws + w.list + w.count);
  const int64_t nwg = geo.groups_per_xcd * kXcds * geo.tiles_n;
  if (geo.wide)
    hipLaunchKernelGGL(gemm16_kernel<WideCfg>, dim3((uint32_t)nwg), dim3(WideCfg::kThreads), 0, s,
                       o.g16, o.x16, o.flags, geo, part, list, count);
  else
    hipLaunchKernelGGL(gemm16_kernel<NarrowCfg>, dim3((uint32_t)nwg), dim3(NarrowCfg::kThreads), 0,
                       s, o.g16, o.x16, o.flags, geo, part, list, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = N * o.d;
  int64_t blocks = ((n + 3) / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(split_finish_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, part, geo.nsplit,
                     geo.pstride, N, o.d, list, count, geo.t_per_split, g32, o.X, o.x_bf16, G);
  return hipGetLastError();
}

hipError_t launch_outer_sum(const float* g, const void* X, bool x_bf16, int64_t T, int64_t N,
                            int64_t d, float* G, void* workspace, hipStream_t s) {
  const Gemm16Out o = outer_sum_operands(workspace, T, N, d, X, x_bf16);
  hipLaunchKernelGGL(prep16_kernel, dim3((uint32_t)T), dim3(256), 0, s, g, N, o);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_outer_sum16(o, g, N, G, workspace, s);
}

}  // namespace dust
