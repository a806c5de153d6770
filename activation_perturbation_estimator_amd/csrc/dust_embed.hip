// dust_embed.hip -- the embedding layer's weight gradient.
//
// Paper digest, section 2.2: an embedding layer's input is one-hot, so the
// outer product sum_t g_t x_t^T becomes a scatter-add of the error estimates
// into the rows of the token ids: G_E[v] = sum_{t : id_t = v} g_t.
//
// Deterministic without float atomics: the tokens are ordered by id with a
// stable counting sort (chunk histograms with in-chunk ranks, a scan, a
// scatter), and each vocabulary row then sums its tokens' rows in increasing
// token order.
//   1. rank_kernel     : one workgroup per chunk of 1024 tokens; each token's
//                        rank among equal ids earlier in its chunk, and the
//                        chunk's per-id counts.
//   2. row_offsets     : per id, the exclusive prefix of the chunk counts and
//                        the id's total.
//   3. id_scan         : exclusive scan of the totals (one workgroup).
//   4. scatter_kernel  : order[start[id] + chunk offset + rank] = t.
//   5. gather_kernel   : one workgroup per id, sum of g rows in that order.
// Ids outside [0, vocab) are skipped.
#include "dust_device.hpp"
#include "dust_launch.hpp"

namespace dust {

constexpr int kChunk = 1024;

__global__ void __launch_bounds__(kChunk) rank_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                      int64_t vocab, int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ counts) {
  __shared__ int32_t sid[kChunk];
  const int64_t c = blockIdx.x;
  const int64_t t = c * kChunk + threadIdx.x;
  int32_t my = -1;
  if (t < T) {
    my = ids[t];
    if (my < 0 || my >= vocab) my = -1;
  }
  sid[threadIdx.x] = my;
  __syncthreads();
  if (my >= 0) {
    int r = 0;
    for (int j = 0; j < (int)threadIdx.x; ++j) r += (sid[j] == my);
    rank[t] = r;
    // the last occurrence of the id in this chunk records the chunk count
    bool last = true;
    for (int j = threadIdx.x + 1; j < kChunk; ++j)
      if (sid[j] == my) { last = false; break; }
    if (last) counts[c * vocab + my] = r + 1;
  }
}

// counts [C][vocab] -> in place exclusive prefix over chunks; total[id].
__global__ void __launch_bounds__(256) row_offsets_kernel(int32_t* __restrict__ counts,
                                                          int64_t C, int64_t vocab,
                                                          int32_t* __restrict__ total) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= vocab) return;
  int32_t run = 0;
  for (int64_t c = 0; c < C; ++c) {
    const int32_t n = counts[c * vocab + v];
    counts[c * vocab + v] = run;
    run += n;
  }
  total[v] = run;
}

// start[v] = sum_{u < v} total[u], start[vocab] = number of valid tokens.
__global__ void __launch_bounds__(1024) id_scan_kernel(const int32_t* __restrict__ total,
                                                       int64_t vocab,
                                                       int32_t* __restrict__ start) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < vocab; base += 1024) {
    const int64_t v = base + threadIdx.x;
    const int32_t x = v < vocab ? total[v] : 0;
    part[threadIdx.x] = x;
    __syncthreads();
    // Hillis-Steele inclusive scan in LDS
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t y = threadIdx.x >= (unsigned)off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += y;
      __syncthreads();
    }
    if (v < vocab) start[v] = carry + part[threadIdx.x] - x;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) start[vocab] = carry;
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

// One workgroup per id; 4 columns per thread per pass.
__global__ void __launch_bounds__(256) gather_kernel(const float* __restrict__ g, int64_t N,
                                                     const int32_t* __restrict__ start,
                                                     const int32_t* __restrict__ order,
                                                     float* __restrict__ GE) {
  const int64_t v = blockIdx.x;
  const int32_t b = start[v], e = start[v + 1];
  float* row = GE + v * N;
  for (int64_t n4 = threadIdx.x; n4 < N / 4; n4 += blockDim.x) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int32_t p = b; p < e; ++p) {
      const float4 x = reinterpret_cast<const float4*>(g + (int64_t)order[p] * N)[n4];
      s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
    }
    reinterpret_cast<float4*>(row)[n4] = s;
  }
}

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

static size_t a256(size_t v) { return (v + 255) / 256 * 256; }

size_t embedding_workspace_bytes(int64_t T, int64_t vocab) {
  const int64_t C = (T + kChunk - 1) / kChunk;
  return a256((size_t)C * vocab * 4) + a256((size_t)T * 4) * 2 + a256((size_t)vocab * 4) +
         a256((size_t)(vocab + 1) * 4);
}

hipError_t launch_embedding_grad(const int32_t* ids, const float* g, int64_t T, int64_t N,
                                 int64_t vocab, float* GE, void* workspace, hipStream_t s) {
  const int64_t C = (T + kChunk - 1) / kChunk;
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
  if (T > 0)
    hipLaunchKernelGGL(scatter_kernel, dim3((uint32_t)((T + 255) / 256)), dim3(256), 0, s, ids, T,
                       vocab, rank, counts, start, order);
  hipLaunchKernelGGL(gather_kernel, dim3((uint32_t)vocab), dim3(256), 0, s, g, N, start, order,
                     GE);
  return hipGetLastError();
}

}  // namespace dust
