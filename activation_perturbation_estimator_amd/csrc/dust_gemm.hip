// dust_gemm.hip -- the weight gradient G_W = sum_t g_t x_t^T on the matrix cores.
//
// Paper digest, section 2.2: the error estimate's outer product with the layer
// input gives the weight gradient, in the same form as backprop.  As a matrix
// product, G[n][k] = sum_t g[t][n] X[t][k], contracting over the token axis,
// which is the slow axis of both row-major operands.
//
// Precision: g is fp32 and the product must keep ~fp32 accuracy.  Each fp32
// value v is split into two bf16 values hi = bf16(v), lo = bf16(v - hi) with
// |v - hi - lo| <= 2^-17 |v|, and the products run on the bf16 MFMA units with
// fp32 accumulation: g_hi X + g_lo X for bf16 X (exact in bf16), plus
// g_hi X_lo for fp32 X.  Every bf16 x bf16 product is exact in fp32.
//
// Layout: both operands are needed token-contiguous (the operand layout of
// v_mfma_f32_32x32x16_bf16: lane l supplies row l%32 and the 8 consecutive
// contraction indices 8*(l/32) .. 8*(l/32)+7).  X is small and read by every
// tile, so a prologue transposes it once to Xt [d][T] bf16.  g is large and read
// once: each lane walks 8 tokens of one column (every load instruction reads 64
// consecutive floats), splits to hi/lo and writes 16-byte rows to LDS.
//
// Tiling: a workgroup (4 waves) owns a 128 x 256 tile of G over one token range
// (split-K over tokens so that the grid fills the 256 CUs), double-buffered in
// LDS.  Partial tiles of the token splits are summed in a fixed order by a
// second kernel, so results are deterministic.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

constexpr int kBM = 128;          // rows of G (layer outputs) per workgroup
constexpr int kBN = 256;          // columns of G (layer inputs) per workgroup
constexpr int kBT = 32;           // tokens per pipeline step
constexpr int kRow = kBT + 8;     // bf16 per LDS row: 80 bytes, 16-byte aligned
constexpr int kXcds = 8;          // MI355X: workgroups go round-robin to 8 XCDs
constexpr int kGemmDepth = 1;     // steps of g / X^T loads in flight per thread (2 measured slower: 1 wave per SIMD)

// Two fp32 values -> packed bf16 hi and packed bf16 lo (v_cvt_pk_bf16_f32, round
// to nearest even): v = hi + lo + O(2^-17 |v|).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2_t v = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  const f32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

// X [T,d] -> Xt [d][Tp] bf16 (token-contiguous, zero beyond T), and for fp32 X
// its hi/lo split.  64 x 64 tiles through LDS; every thread reads 4 consecutive
// columns of one token and writes 4 consecutive tokens of one column.
template <bool kXF32>
__global__ void __launch_bounds__(256) x_transpose_kernel(const void* __restrict__ Xv, int64_t T,
                                                          int64_t d, int64_t Tp,
                                                          uint16_t* __restrict__ xt_hi,
                                                          uint16_t* __restrict__ xt_lo) {
  __shared__ float tile[64][65];
  const int64_t t0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64;
  const int c4 = (threadIdx.x & 15) * 4, r = threadIdx.x >> 4;  // 16 x 16 threads
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int tt = r + 16 * k;
    const int64_t t = t0 + tt;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < T) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t n = n0 + c4 + e;
        if (n < d) {
          if constexpr (kXF32) v[e] = reinterpret_cast<const float*>(Xv)[t * d + n];
          else v[e] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Xv)[t * d + n] << 16);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[tt][c4 + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int nn = r + 16 * k;
    const int64_t n = n0 + nn;
    const int64_t t = t0 + c4;
    if (n >= d || t >= Tp) continue;
    const float a = tile[c4][nn], b = tile[c4 + 1][nn], c = tile[c4 + 2][nn], e = tile[c4 + 3][nn];
    uint2 hi;
    if constexpr (kXF32) {
      uint2 lo;
      split2(a, b, hi.x, lo.x);
      split2(c, e, hi.y, lo.y);
      *reinterpret_cast<uint2*>(xt_lo + n * Tp + t) = lo;
    } else {
      hi.x = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
      hi.y = (__float_as_uint(c) >> 16) | (__float_as_uint(e) & 0xFFFF0000u);
    }
    *reinterpret_cast<uint2*>(xt_hi + n * Tp + t) = hi;
  }
}

struct GemmGeom {
  int64_t M, Nd, T, Tp, tiles_m, tiles_n, nsplit, t_per_split, groups, groups_per_xcd;
};

// Main kernel.  Workgroup = 4 waves on a 128 x 256 tile of G for one token
// split; each wave owns 64 x 128 as 2 x 4 MFMA blocks.  Tokens advance 32 at a
// time through two LDS stages: the next step's g and Xt are fetched into
// registers while the matrix cores work on the current stage.
// kDepth: steps of global loads in flight (register sets).
template <bool kXF32, int kDepth>
__global__ void __launch_bounds__(256, kDepth > 1 || kXF32 ? 1 : 2)
outer_sum_kernel(const float* __restrict__ g, const uint16_t* __restrict__ xt_hi,
                 const uint16_t* __restrict__ xt_lo, GemmGeom geo, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  constexpr int kA = kBM * kRow, kB = kBN * kRow;
  constexpr int kStage = 2 * kA + (kXF32 ? 2 : 1) * kB;

  // XCD-aware order: the tiles_n workgroups that share one (m tile, split) are
  // consecutive on the same XCD, so the second reads g from that XCD's L2.
  const int64_t id = blockIdx.x;
  const int64_t xcd = id % kXcds, rank = id / kXcds;
  const int64_t group = (rank / geo.tiles_n) * kXcds + xcd;
  if (group >= geo.groups) return;  // padding workgroup: leaves before any barrier
  const int64_t ntile = rank % geo.tiles_n;
  const int64_t mtile = group % geo.tiles_m, split = group / geo.tiles_m;
  const int64_t m0 = mtile * kBM, n0 = ntile * kBN;
  const int64_t t_begin = split * geo.t_per_split;
  const int64_t t_end = min(geo.T, t_begin + geo.t_per_split);
  const int nsteps = (int)((t_end - t_begin + kBT - 1) / kBT);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int arow = tid & 127, aq = tid >> 7;  // A staging: row, token groups aq and aq + 2

  f32x16_t acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Buffer loads: out-of-range offsets read as 0.  The g window of this split
  // ends at min(split end, T), so the last partial step of the last split reads
  // zeros; rows m >= M read the next token's values, which only reach
  // accumulator rows that are never stored.
  const int64_t t_rows = t_end - t_begin;
  const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(g + t_begin * geo.M), 0, (int)(t_rows * geo.M * 4), 0x00020000);
  const int64_t n_rows = min((int64_t)kBN, geo.Nd - n0);
  const __amdgpu_buffer_rsrc_t xh_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xt_hi + n0 * geo.Tp), 0, (int)(n_rows * geo.Tp * 2), 0x00020000);
  __amdgpu_buffer_rsrc_t xl_rsrc = xh_rsrc;
  if constexpr (kXF32)
    xl_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xt_lo + n0 * geo.Tp), 0,
                                                (int)(n_rows * geo.Tp * 2), 0x00020000);
  const int a_voff = (int)((m0 + arow) * 4);
  const int a_tstride = (int)(geo.M * 4);

  float av[kDepth][16];
  uint4 bh[kDepth][4], bl[kDepth][kXF32 ? 4 : 1];
  auto fetch = [&](int set, int64_t t0) {
    const int tl = (int)(t0 - t_begin);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = tl + 8 * (aq + 2 * qq) + e;
        av[set][8 * qq + e] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(g_rsrc, a_voff + tt * a_tstride, 0, 0));
      }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int chunk = tid + 256 * k;
      const int off = (int)(((chunk >> 2) * geo.Tp + t0 + 8 * (chunk & 3)) * 2);
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xh_rsrc, off, 0, 0);
      bh[set][k] = make_uint4(v.x, v.y, v.z, v.w);
      if constexpr (kXF32) {
        u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(xl_rsrc, off, 0, 0);
        bl[set][k] = make_uint4(w.x, w.y, w.z, w.w);
      }
    }
  };
  auto stash = [&](int set, int stage) {
    uint16_t* base = lds + stage * kStage;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      uint4 ph, pl;
      split2(av[set][8 * qq + 0], av[set][8 * qq + 1], ph.x, pl.x);
      split2(av[set][8 * qq + 2], av[set][8 * qq + 3], ph.y, pl.y);
      split2(av[set][8 * qq + 4], av[set][8 * qq + 5], ph.z, pl.z);
      split2(av[set][8 * qq + 6], av[set][8 * qq + 7], ph.w, pl.w);
      const int off = arow * kRow + 8 * (aq + 2 * qq);
      *reinterpret_cast<uint4*>(base + off) = ph;
      *reinterpret_cast<uint4*>(base + kA + off) = pl;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int chunk = tid + 256 * k;
      const int off = (chunk >> 2) * kRow + 8 * (chunk & 3);
      *reinterpret_cast<uint4*>(base + 2 * kA + off) = bh[set][k];
      if constexpr (kXF32) *reinterpret_cast<uint4*>(base + 2 * kA + kB + off) = bl[set][k];
    }
  };

  auto compute = [&](int stage) {
    const uint16_t* base = lds + stage * kStage;
#pragma unroll
    for (int kk = 0; kk < kBT; kk += 16) {
      const int koff = kk + 8 * (lane >> 5);
      bf16x8_t fah[2], fal[2], fbh[4], fbl[kXF32 ? 4 : 1];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = wm * 64 + mb * 32 + (lane & 31);
        fah[mb] = *reinterpret_cast<const bf16x8_t*>(base + r * kRow + koff);
        fal[mb] = *reinterpret_cast<const bf16x8_t*>(base + kA + r * kRow + koff);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = wn * 128 + nb * 32 + (lane & 31);
        fbh[nb] = *reinterpret_cast<const bf16x8_t*>(base + 2 * kA + r * kRow + koff);
        if constexpr (kXF32)
          fbl[nb] = *reinterpret_cast<const bf16x8_t*>(base + 2 * kA + kB + r * kRow + koff);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fah[mb], fbh[nb], acc[mb][nb], 0, 0, 0);
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fal[mb], fbh[nb], acc[mb][nb], 0, 0, 0);
          if constexpr (kXF32)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fah[mb], fbl[nb], acc[mb][nb], 0, 0, 0);
        }
    }
  };

  // Software pipeline: step s computes from LDS stage s%2 while register set
  // (s+1)%kDepth is in flight from global memory and set s%kDepth, already
  // stashed, is refilled with step s+kDepth.
  for (int d = 0; d < kDepth; ++d)
    if (d < nsteps) fetch(d, t_begin + (int64_t)d * kBT);
  if (nsteps > 0) stash(0, 0);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int s = s0 + d;
      if (s < nsteps) {
        if (s + kDepth < nsteps) fetch(d, t_begin + (int64_t)(s + kDepth) * kBT);
        compute(s & 1);
        if (s + 1 < nsteps) stash((d + 1) % kDepth, (s + 1) & 1);
        __syncthreads();
      }
    }
  }

  // Register r of block (mb, nb) holds row 8*(r/4) + 4*(lane/32) + r%4 and
  // column lane%32 of that 32 x 32 block.
  float* o = out + split * geo.M * geo.Nd;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 128 + nb * 32 + (lane & 31);
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

static GemmGeom plan(int64_t T, int64_t M, int64_t Nd) {
  GemmGeom g;
  g.M = M;
  g.Nd = Nd;
  g.T = T;
  g.Tp = (T + kBT - 1) / kBT * kBT;
  if (g.Tp == 0) g.Tp = kBT;
  g.tiles_m = (M + kBM - 1) / kBM;
  g.tiles_n = (Nd + kBN - 1) / kBN;
  const int64_t tiles = g.tiles_m * g.tiles_n;
  // Aim for >= 512 workgroups (2 per CU) with >= 512 tokens per split.
  int64_t want = (512 + tiles - 1) / tiles;
  int64_t cap = (T + 511) / 512;
  if (cap < 1) cap = 1;
  int64_t ns = want < cap ? want : cap;
  if (ns < 1) ns = 1;
  int64_t per = (T + ns - 1) / ns;
  per = (per + kBT - 1) / kBT * kBT;
  // 32-bit buffer offsets: one split's slice of g stays below 2^31 bytes.
  const int64_t mm = M > 0 ? M : 1;
  const int64_t per_max = ((((int64_t)1 << 31) - 1 - 4 * (mm + kBM)) / (4 * mm)) / kBT * kBT;
  if (per > per_max) per = per_max > kBT ? per_max : kBT;
  g.t_per_split = per > 0 ? per : kBT;
  g.nsplit = (T + g.t_per_split - 1) / g.t_per_split;
  if (g.nsplit < 1) g.nsplit = 1;
  g.groups = g.tiles_m * g.nsplit;
  g.groups_per_xcd = (g.groups + kXcds - 1) / kXcds;
  return g;
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace: Xt_hi [d][Tp] bf16, Xt_lo (fp32 X only), split partials [S][N][d] fp32.
static void ws_layout(const GemmGeom& g, bool x_f32, size_t& xt_bytes, size_t& part_bytes) {
  xt_bytes = align256((size_t)g.Nd * (size_t)g.Tp * 2);
  part_bytes = g.nsplit > 1 ? (size_t)g.nsplit * (size_t)g.M * (size_t)g.Nd * sizeof(float) : 0;
  (void)x_f32;
}

size_t outer_sum_workspace_bytes(int64_t T, int64_t N, int64_t d) {
  const GemmGeom g = plan(T, N, d);
  size_t xt, part;
  ws_layout(g, true, xt, part);
  return 2 * xt + part;  // sized for fp32 X (hi and lo); bf16 X uses the first half
}

template <bool kXF32>
static hipError_t launch_gemm_t(const GemmGeom& geo, const float* g, const uint16_t* xh,
                                const uint16_t* xl, float* out, hipStream_t s) {
  constexpr int kStageBytes = 2 * (2 * kBM * kRow + (kXF32 ? 2 : 1) * kBN * kRow);
  const size_t lds = 2 * (size_t)kStageBytes;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&outer_sum_kernel<kXF32, kGemmDepth>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t nwg = geo.groups_per_xcd * kXcds * geo.tiles_n;
  hipLaunchKernelGGL((outer_sum_kernel<kXF32, kGemmDepth>), dim3((uint32_t)nwg), dim3(256), lds, s, g,
                     xh, xl, geo, out);
  return hipGetLastError();
}

hipError_t launch_outer_sum(const float* g, const void* X, bool x_bf16, int64_t T, int64_t N,
                            int64_t d, float* G, void* workspace, hipStream_t s) {
  const GemmGeom geo = plan(T, N, d);
  size_t xt_bytes, part_bytes;
  ws_layout(geo, !x_bf16, xt_bytes, part_bytes);
  char* ws = reinterpret_cast<char*>(workspace);
  uint16_t* xh = reinterpret_cast<uint16_t*>(ws);
  uint16_t* xl = reinterpret_cast<uint16_t*>(ws + xt_bytes);
  float* part = reinterpret_cast<float*>(ws + 2 * xt_bytes);
  float* out = (geo.nsplit > 1) ? part : G;

  dim3 tgrid((uint32_t)((geo.Tp + 63) / 64), (uint32_t)((d + 63) / 64));
  if (x_bf16)
    hipLaunchKernelGGL(x_transpose_kernel<false>, tgrid, dim3(256), 0, s, X, T, d, geo.Tp, xh,
                       nullptr);
  else
    hipLaunchKernelGGL(x_transpose_kernel<true>, tgrid, dim3(256), 0, s, X, T, d, geo.Tp, xh, xl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = x_bf16 ? launch_gemm_t<false>(geo, g, xh, nullptr, out, s)
             : launch_gemm_t<true>(geo, g, xh, xl, out, s);
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
