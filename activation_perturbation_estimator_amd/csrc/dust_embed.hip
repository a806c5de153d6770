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
//   4. scatter_kernel  : order[start[id] + chunk offset + rank] = t.
//   5. segment_kernel  : one workgroup per segment of the sorted order: the
//                        sum of each run of equal ids in it, written to G_E
//                        when the run is the id's whole range, else kept as a
//                        partial (at most the first and the last run).
//   6. finish_kernel   : per id, zero rows for absent ids and the in-order sum
//                        of the partials for ids that span segments.
// Ids outside [0, vocab) are skipped.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

constexpr int kChunk = 512;   // tokens per rank workgroup (a power of two)
constexpr int kSeg = 32;      // sorted positions per segment workgroup

// The chunk's (id, position) pairs are sorted in LDS (bitonic network, keys
// id * 2^32 + position, out-of-range ids last); a token's rank is its sorted
// position minus the first sorted position of its id, and the last token of
// each run records the run length as the chunk's count of that id.
__global__ void __launch_bounds__(kChunk) rank_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int64_t vocab, int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ counts) {
  __shared__ uint64_t key[kChunk];
  const int64_t c = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t t = c * kChunk + tid;
  uint64_t k = ~0ull;
  if (t < T) {
    const int32_t v = ids[t];
    if (v >= 0 && v < vocab) k = ((uint64_t)(uint32_t)v << 32) | (uint32_t)tid;
  }
  key[tid] = k;
  for (int size = 2; size <= kChunk; size <<= 1)
    for (int j = size >> 1; j > 0; j >>= 1) {
      __syncthreads();
      const int partner = tid ^ j;
      if (partner > tid) {
        const uint64_t a = key[tid], b = key[partner];
        const bool ascending = (tid & size) == 0;
        if ((a > b) == ascending) {
          key[tid] = b;
          key[partner] = a;
        }
      }
    }
  __syncthreads();
  const uint64_t mine = key[tid];
  if (mine == ~0ull) return;
  const uint32_t v = (uint32_t)(mine >> 32);
  // first sorted position with this id (lower bound of v * 2^32)
  int lo = 0, hi = tid;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((uint32_t)(key[mid] >> 32) < v) lo = mid + 1;
    else hi = mid;
  }
  rank[c * kChunk + (int64_t)(uint32_t)mine] = tid - lo;
  if (tid + 1 == kChunk || (uint32_t)(key[tid + 1] >> 32) != v)
    counts[c * vocab + v] = tid - lo + 1;
}

// counts [C][vocab] -> in place exclusive prefix over chunks; total[id].
__global__ void __launch_bounds__(256) row_offsets_kernel(int32_t* __restrict__ counts,
                                                          int64_t C, int64_t vocab,
                                                          int32_t* __restrict__ total) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= vocab) return;
  int32_t run = 0;
  for (int64_t c0 = 0; c0 < C; c0 += 8) {
    int32_t n[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) n[u] = c0 + u < C ? counts[(c0 + u) * vocab + v] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
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

__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int64_t vocab,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ start,
                                                      int32_t* __restrict__ order) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int32_t v = ids[t];
  if (v < 0 || v >= vocab) return;
  const int64_t c = t / kChunk;
  order[start[v] + counts[c * vocab + v] + rank[t]] = (int32_t)t;
}

// One workgroup per segment [kSeg s, kSeg s + kSeg) of the sorted order (n_valid
// = start[vocab] positions in all).  Threads own 4 columns each; the rows of a
// run are added in position order.  Partial runs go to part[s][0] (the run at
// the segment's first position) and part[s][1] (the run at its last position,
// when that is a different run).
__global__ void __launch_bounds__(128) segment_kernel(const float* __restrict__ g, int64_t N,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ start,
                                                      int64_t vocab,
                                                      const int32_t* __restrict__ order,
                                                      float* __restrict__ GE,
                                                      float* __restrict__ part) {
  __shared__ int32_t s_tok[kSeg], s_id[kSeg];
  const int64_t nvalid = start[vocab];
  const int64_t p0 = (int64_t)blockIdx.x * kSeg;
  if (p0 >= nvalid) return;
  const int n = (int)min((int64_t)kSeg, nvalid - p0);
  if (threadIdx.x < n) {
    const int32_t t = order[p0 + threadIdx.x];
    s_tok[threadIdx.x] = t;
    s_id[threadIdx.x] = ids[t];
  }
  __syncthreads();
  for (int64_t c4 = threadIdx.x; c4 < N / 4; c4 += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int a = 0;  // first position of the current run
    for (int pb = 0; pb < n; pb += 8) {
      float4 x[8];  // eight rows in flight
#pragma unroll
      for (int u = 0; u < 8; ++u)
        x[u] = pb + u < n ? reinterpret_cast<const float4*>(g + (int64_t)s_tok[pb + u] * N)[c4]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int p = pb + u;
        if (p >= n) break;
        acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w;
        const int v = s_id[p];
        if (p + 1 == n || s_id[p + 1] != v) {  // run [a, p] ends
          const int64_t lo = start[v], hi = start[v + 1];
          float* dst;
          if (lo >= p0 && hi <= p0 + n) dst = GE + (int64_t)v * N;                // whole id
          else dst = part + ((int64_t)blockIdx.x * 2 + (a == 0 ? 0 : 1)) * N;     // partial
          reinterpret_cast<float4*>(dst)[c4] = acc;
          acc = make_float4(0.f, 0.f, 0.f, 0.f);
          a = p + 1;
        }
      }
    }
  }
}

// Per id: rows of absent ids are zero; an id whose range spans segments s0..s1
// sums its partials in segment order (its run is the last one of s0, slot 1
// unless it starts the segment, and the first one of every later segment).
__global__ void __launch_bounds__(128) finish_kernel(int64_t N, const int32_t* __restrict__ start,
                                                     int64_t vocab, const float* __restrict__ part,
                                                     float* __restrict__ GE) {
  for (int64_t v = blockIdx.x; v < vocab; v += gridDim.x) {
    const int64_t lo = start[v], hi = start[v + 1];
    float4* row = reinterpret_cast<float4*>(GE + v * N);
    if (hi == lo) {
      for (int64_t c4 = threadIdx.x; c4 < N / 4; c4 += blockDim.x)
        row[c4] = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    const int64_t s0 = lo / kSeg, s1 = (hi - 1) / kSeg;
    if (s0 == s1) continue;  // written whole by segment_kernel
    for (int64_t c4 = threadIdx.x; c4 < N / 4; c4 += blockDim.x) {
      float4 acc = reinterpret_cast<const float4*>(part + (s0 * 2 + (lo % kSeg == 0 ? 0 : 1)) * N)[c4];
      for (int64_t sb = s0 + 1; sb <= s1; sb += 8) {
        float4 x[8];  // eight partials in flight, added in segment order
#pragma unroll
        for (int u = 0; u < 8; ++u)
          x[u] = sb + u <= s1 ? reinterpret_cast<const float4*>(part + (sb + u) * 2 * N)[c4]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w;
        }
      }
      row[c4] = acc;
    }
  }
}

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

static size_t a256(size_t v) { return (v + 255) / 256 * 256; }

size_t embedding_workspace_bytes(int64_t T, int64_t N, int64_t vocab) {
  const int64_t C = (T + kChunk - 1) / kChunk, S = (T + kSeg - 1) / kSeg;
  return a256((size_t)C * vocab * 4) + a256((size_t)T * 4) * 2 + a256((size_t)vocab * 4) +
         a256((size_t)(vocab + 1) * 4) + a256((size_t)S * 2 * N * 4);
}

hipError_t launch_embedding_grad(const int32_t* ids, const float* g, int64_t T, int64_t N,
                                 int64_t vocab, float* GE, void* workspace, hipStream_t s) {
  const int64_t C = (T + kChunk - 1) / kChunk, S = (T + kSeg - 1) / kSeg;
  char* w = reinterpret_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)C * vocab * 4);
  int32_t* rank = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)T * 4);
  int32_t* order = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)T * 4);
  int32_t* total = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)vocab * 4);
  int32_t* start = reinterpret_cast<int32_t*>(w);
  w += a256((size_t)(vocab + 1) * 4);
  float* part = reinterpret_cast<float*>(w);

  const int64_t ncnt = C * vocab;
  int64_t zb = (ncnt + 255) / 256;
  if (zb > 4096) zb = 4096;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((uint32_t)(zb > 0 ? zb : 1)), dim3(256), 0, s, counts,
                     ncnt);
  if (T > 0)
    hipLaunchKernelGGL(rank_kernel, dim3((uint32_t)C), dim3(kChunk), 0, s, ids, T, vocab, rank,
                       counts);
  hipLaunchKernelGGL(row_offsets_kernel, dim3((uint32_t)((vocab + 255) / 256)), dim3(256), 0, s,
                     counts, C, vocab, total);
  hipLaunchKernelGGL(id_scan_kernel, dim3(1), dim3(1024), 0, s, total, vocab, start);
  if (T > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3((uint32_t)((T + 255) / 256)), dim3(256), 0, s, ids, T,
                       vocab, rank, counts, start, order);
    hipLaunchKernelGGL(segment_kernel, dim3((uint32_t)S), dim3(128), 0, s, g, N, ids, start, vocab,
                       order, GE, part);
  }
  const int64_t fb = vocab < 2048 ? vocab : 2048;
  hipLaunchKernelGGL(finish_kernel, dim3((uint32_t)fb), dim3(128), 0, s, N, start, vocab, part, GE);
  return hipGetLastError();
}

}  // namespace dust
