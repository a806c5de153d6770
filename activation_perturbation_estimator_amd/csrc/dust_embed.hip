// dust_embed.hip -- the embedding layer's weight gradient.
//
// Paper digest, section 2.2: an embedding layer's input is one-hot, so the
// outer product sum_t g_t x_t^T becomes a scatter-add of the error estimates
// into the rows of the token ids: G_E[v] = sum_{t : id_t = v} g_t.
//
// Deterministic without float atomics: the tokens are ordered by id with a
// stable counting sort (chunk histograms with in-chunk ranks, a scan, a
// scatter); the sorted order is then cut into segments of kSeg positions that
// are summed in parallel, and an id whose tokens span several segments adds
// its per-segment partial sums in segment order.  Every row is therefore the
// sum of its tokens' rows in increasing token order, grouped by segment.
//   1. rank_kernel     : one workgroup per chunk of kChunk tokens; each token's
//                        rank among equal ids earlier in its chunk, and the
//                        chunk's per-id counts.
//   2. row_offsets     : per id, the exclusive prefix of the chunk counts and
//                        the id's total.
//   3. id_scan         : exclusive scan of the totals (one workgroup).
//   4. scatter_kernel  : order[start[id] + chunk offset + rank] = t, with the
//                        id (and whether its range fits one segment) beside it.
//   5. segment_kernel  : one wave per segment of the sorted order and block of
//                        256 columns: the sum of each run of equal ids in it,
//                        written to G_E when the run is the id's whole range,
//                        else kept as a partial (at most the first and the
//                        last run).
//   6. finish_kernel   : per id, the zero row of an absent id, or the in-order
//                        sum of the partials of an id that spans segments.
// Ids outside [0, vocab) are skipped.
#include <mutex>

#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

constexpr int kChunk = 512;   // tokens per rank workgroup (a power of two)
constexpr int kSeg = 32;      // sorted positions per segment workgroup
constexpr int kSegCols = 64;  // float4 columns per segment workgroup (one wave)
constexpr int kFinishBatch = 32;  // partial rows in flight when an id's partials are summed
constexpr int kRankRowMax = 8192;  // vocabularies whose counts rows the rank pass writes whole

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// The chunk's (id, position) pairs are sorted by a bitonic network (keys
// id * 2^32 + position, out-of-range ids last): the stages whose partners sit
// in the same wave exchange keys by shuffles, the others through LDS (two
// buffers, one barrier per stage).  A token's rank is its sorted position
// minus the first sorted position of its id, and the last token of each run
// holds the run length, the chunk's count of that id.  With full_row
// (vocab <= kRankRowMax) the counts are gathered in LDS and the workgroup
// writes its whole row of counts, zeros included; otherwise only present ids
// are written and the row must have been cleared before.
__global__ void __launch_bounds__(kChunk) rank_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int64_t vocab, int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ counts, int full_row) {
  __shared__ uint64_t key[2][kChunk];
  __shared__ int32_t cnt[kRankRowMax];
  const int64_t c = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t t = c * kChunk + tid;
  if (full_row)
    for (int v = tid; v < vocab; v += kChunk) cnt[v] = 0;  // ordered by the barriers below
  uint64_t k = ~0ull;
  if (t < T) {
    const int32_t v = ids[t];
    if (v >= 0 && v < vocab) k = ((uint64_t)(uint32_t)v << 32) | (uint32_t)tid;
  }
  int buf = 0;
  for (int size = 2; size <= kChunk; size <<= 1)
    for (int j = size >> 1; j > 0; j >>= 1) {
      uint64_t other;
      if (j >= 64) {
        key[buf][tid] = k;
        __syncthreads();
        other = key[buf][tid ^ j];
        buf ^= 1;
      } else {
        other = shfl_xor64(k, j);
      }
      const bool keep_min = ((tid & j) == 0) == ((tid & size) == 0);
      k = keep_min ? (other < k ? other : k) : (other < k ? k : other);
    }
  key[buf][tid] = k;
  __syncthreads();
  const uint64_t* sk = key[buf];
  if (k != ~0ull) {
    const uint32_t v = (uint32_t)(k >> 32);
    // first sorted position with this id (lower bound of v * 2^32)
    int lo = 0, hi = tid;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((uint32_t)(sk[mid] >> 32) < v) lo = mid + 1;
      else hi = mid;
    }
    rank[c * kChunk + (int64_t)(uint32_t)k] = tid - lo;
    if (tid + 1 == kChunk || (uint32_t)(sk[tid + 1] >> 32) != v) {
      if (full_row) cnt[v] = tid - lo + 1;
      else counts[c * vocab + v] = tid - lo + 1;
    }
  }
  if (full_row) {
    __syncthreads();
    for (int v = tid; v < vocab; v += kChunk) counts[c * vocab + v] = cnt[v];
  }
}

// counts [C][vocab] -> in place exclusive prefix over chunks; total[id].
__global__ void __launch_bounds__(256) row_offsets_kernel(int32_t* __restrict__ counts,
                                                          int64_t C, int64_t vocab,
                                                          int32_t* __restrict__ total) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= vocab) return;
  int32_t run = 0;
  for (int64_t c0 = 0; c0 < C; c0 += 32) {
    int32_t n[32];  // unconditional loads: past the last chunk re-read it
#pragma unroll
    for (int u = 0; u < 32; ++u) n[u] = counts[(c0 + u < C ? c0 + u : C - 1) * vocab + v];
#pragma unroll
    for (int u = 0; u < 32; ++u)
      if (c0 + u < C) {
        counts[(c0 + u) * vocab + v] = run;
        run += n[u];
      }
  }
  total[v] = run;
}

// start[v] = sum_{u < v} total[u], start[vocab] = number of valid tokens.
// One workgroup of 1024 threads, 4096 ids per pass: 4 per thread, a wave
// inclusive scan of the thread sums (shuffles), then the 16 wave totals.
__global__ void __launch_bounds__(1024) id_scan_kernel(const int32_t* __restrict__ total,
                                                       int64_t vocab,
                                                       int32_t* __restrict__ start) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t carry = 0;
  for (int64_t base = 0; base < vocab; base += 4096) {
    int32_t x[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t v = base + 4 * tid + e;
      x[e] = v < vocab ? total[v] : 0;
      sum += x[e];
    }
    int32_t incl = sum;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int32_t run = before + incl - sum;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t v = base + 4 * tid + e;
      if (v < vocab) start[v] = run;
      run += x[e];
    }
    int32_t all = 0;
    for (int w = 0; w < 16; ++w) all += wsum[w];
    carry += all;
    __syncthreads();
  }
  if (tid == 0) start[vocab] = carry;
}

// order[p] = t and info[p] = id | whole << 31 for sorted position p, where
// whole says that the id's positions all lie in one segment.
__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int64_t vocab,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ start,
                                                      int32_t* __restrict__ order,
                                                      uint32_t* __restrict__ info) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int32_t v = ids[t];
  if (v < 0 || v >= vocab) return;
  const int64_t c = t / kChunk;
  const int32_t lo = start[v], hi = start[v + 1];
  const int64_t pos = lo + counts[c * vocab + v] + rank[t];
  order[pos] = (int32_t)t;
  info[pos] = (uint32_t)v | ((lo / kSeg == (hi - 1) / kSeg) ? 0x80000000u : 0u);
}

// Steps 1-4 in one launch, for T <= kOneT tokens and vocabularies of up to
// kOneVocab ids: one workgroup per chunk of kChunk tokens, each of which also
// counts every id in LDS over all T tokens and over the tokens before its
// chunk (integer atomics: the counts do not depend on their order) -- the ids
// are only 4T bytes, so every workgroup reading all of them costs less than
// the three launches that would otherwise share the counts.  The totals'
// exclusive scan gives the ids' starts.  Within the chunk, each wave ranks its
// 64 tokens among equal ids by ballots over the id's bits (a lane's peers are
// the AND over bits b of ballot(bit b set) or its complement), and its count of
// each id goes to an LDS row of the wave; a token's position is then
//   start[id] + (the id's tokens in earlier chunks) + (in earlier waves of the
//   chunk) + (its peers in lower lanes):
// ascending id, and ascending token within an id.
constexpr int64_t kOneT = 32768;
constexpr int64_t kOneVocab = 4096;
constexpr int kOneWaves = kChunk / 64;

__global__ void __launch_bounds__(kChunk) one_pass_sort_kernel(const int32_t* __restrict__ ids,
                                                               int64_t T, int64_t vocab,
                                                               int32_t* __restrict__ order,
                                                               uint32_t* __restrict__ info,
                                                               int32_t* __restrict__ start) {
  __shared__ __attribute__((aligned(16))) uint16_t wcnt[kOneWaves * kOneVocab];
  __shared__ int32_t hall[kOneVocab + 1], hbefore[kOneVocab];
  __shared__ int32_t wsum[kOneWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int V = (int)vocab, Ti = (int)T;
  const int c0 = (int)blockIdx.x * kChunk;  // this chunk's first token
  const int t = c0 + tid;
  const int mine = t < Ti ? ids[t] : -1;
  for (int i = tid; i < kOneWaves * kOneVocab / 8; i += kChunk)
    reinterpret_cast<uint4*>(wcnt)[i] = make_uint4(0, 0, 0, 0);
  for (int v = tid; v < V; v += kChunk) {
    hall[v] = 0;
    hbefore[v] = 0;
  }
  __syncthreads();
  // counts of every id, over all tokens and over those before the chunk; the
  // chunks in the second half count the tokens from the chunk on instead (fewer)
  // and subtract
  const bool before = 2 * c0 <= Ti;
  constexpr int kU = 16;
  for (int b = 0; b < Ti; b += kChunk * kU) {
    int v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tt = b + u * kChunk + tid;
      v[u] = tt < Ti ? ids[tt] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (v[u] >= 0 && v[u] < V) {
        atomicAdd(&hall[v[u]], 1);
        if ((b + u * kChunk + tid < c0) == before) atomicAdd(&hbefore[v[u]], 1);
      }
  }
  __syncthreads();
  if (!before)  // hbefore holds the counts from the chunk on: subtract them
    for (int v = tid; v < V; v += kChunk) hbefore[v] = hall[v] - hbefore[v];
  // exclusive scan of the totals: kChunk threads, 8 consecutive ids each
  constexpr int kPer = kOneVocab / kChunk;
  {
    int x[kPer], sum = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int v = kPer * tid + e;
      x[e] = v < V ? hall[v] : 0;
      sum += x[e];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int ww = 0; ww < w; ++ww) run += wsum[ww];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int v = kPer * tid + e;
      if (v < V) hall[v] = run;
      run += x[e];
    }
    if (tid == kChunk - 1) hall[V] = run;  // the number of valid tokens
  }
  // this wave's peers of each token, and the wave's count of each id
  const bool valid = mine >= 0 && mine < V;
  const int nbits = V > 1 ? 32 - __clz(V - 1) : 0;
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((mine >> b) & 1);
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  if (valid && (m >> lane) == 1ull) wcnt[w * kOneVocab + mine] = (uint16_t)__popcll(m);
  __syncthreads();
  if (blockIdx.x == 0)
    for (int v = tid; v <= V; v += kChunk) start[v] = hall[v];
  if (valid) {
    int pos = hall[mine] + hbefore[mine] + __popcll(m & ((1ull << lane) - 1));
    for (int ww = 0; ww < w; ++ww) pos += wcnt[ww * kOneVocab + mine];
    const int lo = hall[mine], hi = hall[mine + 1];
    order[pos] = t;
    info[pos] = (uint32_t)mine | ((lo / kSeg == (hi - 1) / kSeg) ? 0x80000000u : 0u);
  }
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// The partials of an id spanning segments s0..s1 summed in segment order: its
// run is the last one of s0 (slot 1, unless it starts the segment: slot 0) and
// the first one (slot 0) of every later segment.  kFinishBatch partials in
// flight at a time.
__device__ __forceinline__ void combine_partials(const float* __restrict__ part, int64_t N,
                                                 int64_t c4, int64_t lo, int64_t hi,
                                                 float* __restrict__ row) {
  const int64_t s0 = lo / kSeg, s1 = (hi - 1) / kSeg;
  float4 acc = reinterpret_cast<const float4*>(part + (s0 * 2 + (lo % kSeg == 0 ? 0 : 1)) * N)[c4];
  for (int64_t sb = s0 + 1; sb <= s1; sb += kFinishBatch) {
    float4 x[kFinishBatch];  // unconditional loads: past s1 re-read s1
#pragma unroll
    for (int u = 0; u < kFinishBatch; ++u)
      x[u] = reinterpret_cast<const float4*>(part + (sb + u <= s1 ? sb + u : s1) * 2 * N)[c4];
#pragma unroll
    for (int u = 0; u < kFinishBatch; ++u)
      if (sb + u <= s1) acc = add4(acc, x[u]);
  }
  reinterpret_cast<float4*>(row)[c4] = acc;
}

// One wave per (segment [kSeg s, kSeg s + kSeg) of the sorted order, block of
// kSegCols float4 columns); n_valid = start[vocab] sorted positions in all.
// Lane p < kSeg holds position p's token and info; each lane issues the loads
// of all the segment's rows for its 4 columns at once, then adds the rows of
// each run in position order.  A run that is its id's whole range is written
// to G_E; otherwise it is a partial (at most the segment's first and last
// run) and goes to part[s][0] (the run at the segment's first position) or
// part[s][1] (the run at its last position).
__global__ void __launch_bounds__(kSegCols) segment_kernel(const float* __restrict__ g, int64_t N,
                                                           int64_t T,
                                                           const int32_t* __restrict__ start,
                                                           int64_t vocab,
                                                           const int32_t* __restrict__ order,
                                                           const uint32_t* __restrict__ info,
                                                           float* __restrict__ GE,
                                                           float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int64_t seg = blockIdx.x, p0 = seg * kSeg;
  int32_t my_t = 0;
  uint32_t my_info = 0;
  if (lane < kSeg && p0 + lane < T) {
    my_t = order[p0 + lane];
    my_info = info[p0 + lane];
  }
  const int64_t nvalid = start[vocab];
  if (p0 >= nvalid) return;  // whole wave
  const int n = (int)min((int64_t)kSeg, nvalid - p0);
  const int64_t nc4 = N / 4;
  const int64_t c4 = (int64_t)blockIdx.y * kSegCols + lane;
  const bool col = c4 < nc4;
  const int64_t cl = col ? c4 : nc4 - 1;  // lanes past the last column load a valid one
  float4 x[kSeg];  // every row of the segment in flight (past n: the last row again)
#pragma unroll
  for (int u = 0; u < kSeg; ++u) {
    const int32_t t = __builtin_amdgcn_readlane(my_t, u < n ? u : n - 1);
    x[u] = reinterpret_cast<const float4*>(g + (int64_t)t * N)[cl];
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int a = 0;  // first position of the current run
#pragma unroll
  for (int p = 0; p < kSeg; ++p) {
    if (p < n) {
      acc = add4(acc, x[p]);
      const uint32_t inf = (uint32_t)__builtin_amdgcn_readlane((int)my_info, p);
      const uint32_t v = inf & 0x7FFFFFFFu;
      const uint32_t vn =
          (uint32_t)__builtin_amdgcn_readlane((int)my_info, p + 1 < kSeg ? p + 1 : p) & 0x7FFFFFFFu;
      if (p + 1 == n || vn != v) {  // run [a, p] ends
        if (inf >> 31) {
          if (col) reinterpret_cast<float4*>(GE + (int64_t)v * N)[c4] = acc;
        } else {
          const int slot = a == 0 ? 0 : 1;
          if (col) reinterpret_cast<float4*>(part + (seg * 2 + slot) * N)[c4] = acc;
        }
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
        a = p + 1;
      }
    }
  }
}

// Per id: the zero row of an absent id, or the in-order sum of the partials of
// an id whose range spans segments; ids written whole by segment_kernel return.
__global__ void __launch_bounds__(128) finish_kernel(int64_t N, const int32_t* __restrict__ start,
                                                     int64_t vocab, const float* __restrict__ part,
                                                     float* __restrict__ GE) {
  for (int64_t v = blockIdx.x; v < vocab; v += gridDim.x) {
    const int64_t lo = start[v], hi = start[v + 1];
    if (hi == lo) {
      for (int64_t c4 = threadIdx.x; c4 < N / 4; c4 += blockDim.x)
        reinterpret_cast<float4*>(GE + v * N)[c4] = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    if (lo / kSeg == (hi - 1) / kSeg) continue;  // written whole by segment_kernel
    for (int64_t c4 = threadIdx.x; c4 < N / 4; c4 += blockDim.x)
      combine_partials(part, N, c4, lo, hi, GE + v * N);
  }
}

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

static size_t a256(size_t v) { return (v + 255) / 256 * 256; }

static int64_t seg_col_blocks(int64_t N) { return (N / 4 + kSegCols - 1) / kSegCols; }

size_t embedding_workspace_bytes(int64_t T, int64_t N, int64_t vocab) {
  const int64_t C = (T + kChunk - 1) / kChunk, S = (T + kSeg - 1) / kSeg;
  return a256((size_t)C * vocab * 4) + a256((size_t)T * 4) * 3 + a256((size_t)vocab * 4) +
         a256((size_t)(vocab + 1) * 4) + a256((size_t)S * 2 * N * 4);
}

hipError_t launch_embedding_grad(const int32_t* ids, const float* g, int64_t T, int64_t N,
                                 int64_t vocab, float* GE, void* workspace, hipStream_t s) {
  const int64_t C = (T + kChunk - 1) / kChunk, S = (T + kSeg - 1) / kSeg;
  const int64_t CB = seg_col_blocks(N);
  char* w = reinterpret_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)C * vocab * 4);
  int32_t* rank = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)T * 4);
  int32_t* order = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)T * 4);
  uint32_t* info = reinterpret_cast<uint32_t*>(w);
  w += a256((size_t)T * 4);
  int32_t* total = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)vocab * 4);
  int32_t* start = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)(vocab + 1) * 4);
  float* part = reinterpret_cast<float*>(w);

  if (T <= kOneT && vocab <= kOneVocab) {  // steps 1-4 in one launch
    hipLaunchKernelGGL(one_pass_sort_kernel, dim3((uint32_t)(C > 0 ? C : 1)), dim3(kChunk), 0, s,
                       ids, T, vocab, order, info, start);
  } else {
    // small vocabularies: each rank workgroup writes its whole row of counts
    const int full_row = vocab <= kRankRowMax;
    if (!full_row) {
      const int64_t ncnt = C * vocab;
      int64_t zb = (ncnt + 255) / 256;
      if (zb > 4096) zb = 4096;
      hipLaunchKernelGGL(zero_i32_kernel, dim3((uint32_t)(zb > 0 ? zb : 1)), dim3(256), 0, s,
                         counts, ncnt);
    }
    if (T > 0)
      hipLaunchKernelGGL(rank_kernel, dim3((uint32_t)C), dim3(kChunk), 0, s, ids, T, vocab, rank,
                         counts, full_row);
    hipLaunchKernelGGL(row_offsets_kernel, dim3((uint32_t)((vocab + 255) / 256)), dim3(256), 0, s,
                       counts, C, vocab, total);
    hipLaunchKernelGGL(id_scan_kernel, dim3(1), dim3(1024), 0, s, total, vocab, start);
    if (T > 0)
      hipLaunchKernelGGL(scatter_kernel, dim3((uint32_t)((T + 255) / 256)), dim3(256), 0, s, ids,
                         T, vocab, rank, counts, start, order, info);
  }
  if (T > 0) {
    hipLaunchKernelGGL(segment_kernel, dim3((uint32_t)S, (uint32_t)CB), dim3(kSegCols), 0, s, g, N,
                       T, start, vocab, order, info, GE, part);
  }
  const int64_t fb = vocab < 65536 ? vocab : 65536;
  hipLaunchKernelGGL(finish_kernel, dim3((uint32_t)fb), dim3(128), 0, s, N, start, vocab, part, GE);
  return hipGetLastError();
}

// Scratch memory of the variant that allocates nothing (for callers that
// cannot allocate: graph capture, tight loops): a fixed device array, one per
// GPU, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol); it takes each
// device's address of it once, with hipGetSymbolAddress, and uses that.
static __device__ __align__(256) uint8_t scratch[kEmbeddingStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t embedding_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dust
