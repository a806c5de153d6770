// dust_api.cpp -- the C ABI of libdust: argument validation, workspace layout
// and the launch sequence of each call.  Every check runs on the host before
// the first HIP call, so a rejected call touches neither the device nor the
// stream.  Nothing here allocates memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "dust.h"
#include "dust_launch.hpp"

static_assert(DUST_EMBEDDING_NOALLOC_BYTES == dust::kEmbeddingStaticScratchBytes,
              "the header states the size of the library's own scratch");

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool sigma_ok(float sigma) {
  return std::isfinite(sigma) && sigma > 0.f && sigma <= DUST_SIGMA_MAX;
}
bool gamma_ok(float gamma) { return std::isfinite(gamma) && gamma >= 0.f && gamma <= 1.f; }
// Enum arguments come from C callers, who may pass any int; in C++ loading an
// enum object whose value lies outside its enumerators' range is undefined, so
// the value is read from the object's bytes as an int before it is checked.
static_assert(sizeof(dust_dtype) == sizeof(int) && sizeof(dust_status) == sizeof(int),
              "the ABI's enums are passed as int");
template <typename E>
int enum_value(const E& e) {
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}
bool dtype_ok(const dust_dtype& dt) {
  const int v = enum_value(dt);
  return v == DUST_F32 || v == DUST_BF16;
}

// Index products stay far below 2^62, the 32-bit counter words hold t and i,
// token positions of the G_W and embedding calls fit int32, and the kernels
// that take one workgroup (at most 256 threads) per token keep their grid's
// work-item count inside the 32 bits of a dispatch.
constexpr int64_t kMaxT = (int64_t)1 << 22;          // calls that form G_W
constexpr int64_t kMaxWidth = (int64_t)1 << 20;      // N and d of the calls that form G_W
constexpr int64_t kMaxTokens = ((int64_t)1 << 24) - 1;  // the other per-token calls
constexpr int64_t kMaxK = ((int64_t)1 << 31) - 64;
constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int64_t kMaxVocab = (int64_t)1 << 24;      // the embedding calls

bool width_ok(int64_t N) { return N > 0 && N % 4 == 0 && N <= DUST_N_MAX; }

// A range of draws draw0 .. draw0 + K - 1 of a population of K_total: the
// draw is a 32-bit counter word of the noise.
bool draws_ok(int64_t draw0, int64_t K, int64_t K_total) {
  return draw0 >= 0 && K >= 0 && K <= kMaxK && K_total >= 1 && K_total <= kMaxK &&
         draw0 <= ((int64_t)1 << 32) - K;
}

// a * b <= lim for a, b >= 0, without forming a product that could overflow.
bool prod_le(int64_t a, int64_t b, int64_t lim) { return b == 0 || a <= lim / b; }

dust_status hip_status(hipError_t e) { return e == hipSuccess ? DUST_OK : DUST_ERR_HIP; }

hipStream_t as_stream(dust_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

hipError_t record(const dust_event_t* ev, int k, hipStream_t s) {
  if (ev == nullptr || ev[k] == nullptr) return hipSuccess;  // a NULL entry is not recorded
  return hipEventRecord(reinterpret_cast<hipEvent_t>(ev[k]), s);
}

// Workspace layout of the LM-head call:
//   [0, a)       per-draw loss changes delta [K,T] (non-fused path only),
//                later centred in place (c) and scanned in place (r)
//   [a, a + b)   split-K partials of the outer product
struct HeadPlan {
  bool fused;
  size_t delta_bytes;
  size_t gemm_bytes;
  size_t total() const { return align_up(delta_bytes) + align_up(gemm_bytes) + kAlign; }
};

HeadPlan head_plan(int64_t T, int64_t V, int64_t d, int64_t K, float gamma) {
  HeadPlan p;
  p.fused = (gamma == 0.f) && dust::head_fused_supported(V);
  p.delta_bytes = p.fused ? 0 : (size_t)K * (size_t)T * sizeof(float);
  p.gemm_bytes = dust::outer_sum_workspace_bytes(T, V, d);
  return p;
}

struct LinearPlan {
  size_t r_bytes;
  size_t gemm_bytes;
  size_t total() const { return align_up(r_bytes) + align_up(gemm_bytes) + kAlign; }
};

LinearPlan linear_plan(int64_t T, int64_t d_in, int64_t N, int64_t K, float gamma) {
  LinearPlan p;
  p.r_bytes = (gamma == 0.f) ? 0 : (size_t)K * (size_t)T * sizeof(float);
  p.gemm_bytes = dust::outer_sum_workspace_bytes(T, N, d_in);
  return p;
}

void* aligned_base(void* ws) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(ws);
  return reinterpret_cast<void*>((p + kAlign - 1) / kAlign * kAlign);
}

}  // namespace

extern "C" {

const char* dust_status_string(dust_status st) {
  switch (enum_value(st)) {
    case DUST_OK: return "DUST_OK";
    case DUST_ERR_INVALID_ARG: return "DUST_ERR_INVALID_ARG";
    case DUST_ERR_WORKSPACE: return "DUST_ERR_WORKSPACE";
    case DUST_ERR_HIP: return "DUST_ERR_HIP";
    case DUST_ERR_UNSUPPORTED: return "DUST_ERR_UNSUPPORTED";
    case DUST_ERR_TARGETS: return "DUST_ERR_TARGETS";
  }
  return "DUST_ERR_UNKNOWN";
}

const char* dust_version(void) { return "libdust 1.0 gfx950"; }

// The size queries answer the minimum for sizes the calls reject (invalid, or
// beyond the size limits), so that no size arithmetic runs on them.
size_t dust_head_workspace_size(int64_t T, int64_t V, int64_t d, int64_t K, float gamma) {
  if (T < 0 || V <= 0 || d <= 0 || K <= 0) return kAlign;
  if (T > kMaxT || V > kMaxWidth || d > kMaxWidth || K > kMaxK) return kAlign;
  return head_plan(T, V, d, K, gamma).total();
}

size_t dust_linear_workspace_size(int64_t T, int64_t d_in, int64_t N, int64_t K, float gamma) {
  if (T < 0 || N <= 0 || d_in <= 0 || K <= 0) return kAlign;
  if (T > kMaxT || N > kMaxWidth || d_in > kMaxWidth || K > kMaxK) return kAlign;
  return linear_plan(T, d_in, N, K, gamma).total();
}

size_t dust_outer_sum_workspace_size(int64_t T, int64_t N, int64_t d) {
  if (T < 0 || N <= 0 || d <= 0) return kAlign;
  if (T > kMaxT || N > kMaxWidth || d > kMaxWidth) return kAlign;
  return align_up(dust::outer_sum_workspace_bytes(T, N, d)) + kAlign;
}

dust_status dust_head_estimate(const void* logits, dust_dtype logits_dt, const int32_t* targets,
                               const void* X, dust_dtype x_dt, int64_t T, int64_t V, int64_t d,
                               int64_t seq_len, float sigma, int64_t K, float gamma,
                               uint64_t seed, uint32_t stream, float* g_hat, float* G_W,
                               float* losses_opt, void* workspace, size_t workspace_bytes,
                               dust_stream_t s_, const dust_event_t* stage_events) {
  if (!logits || !targets || !X || !g_hat || !G_W) return DUST_ERR_INVALID_ARG;
  if (!dtype_ok(logits_dt) || !dtype_ok(x_dt)) return DUST_ERR_INVALID_ARG;
  if (T <= 0 || !width_ok(V) || d <= 0 || K <= 0 || K > kMaxK) return DUST_ERR_INVALID_ARG;
  if (T > kMaxT || d > kMaxWidth) return DUST_ERR_UNSUPPORTED;
  if (seq_len <= 0 || T % seq_len != 0) return DUST_ERR_INVALID_ARG;
  if (!sigma_ok(sigma) || !gamma_ok(gamma)) return DUST_ERR_INVALID_ARG;
  if (T * V > kMaxElems || T * d > kMaxElems || K * T > kMaxElems || V * d > kMaxElems)
    return DUST_ERR_UNSUPPORTED;
  if (!dust::outer_sum_supported(T, V, d)) return DUST_ERR_UNSUPPORTED;
  const HeadPlan plan = head_plan(T, V, d, K, gamma);
  if (workspace == nullptr || workspace_bytes < plan.total()) return DUST_ERR_WORKSPACE;

  hipStream_t s = as_stream(s_);
  char* ws = reinterpret_cast<char*>(aligned_base(workspace));
  float* delta = reinterpret_cast<float*>(ws);
  void* gemm_ws = ws + align_up(plan.delta_bytes);
  const bool zbf16 = (logits_dt == DUST_BF16);

  // the kernel that finishes g_hat also writes the fp16 operands of the G_W pass
  const dust::Gemm16Out op = dust::outer_sum_operands(gemm_ws, T, V, d, X, x_dt == DUST_BF16);

  hipError_t e = record(stage_events, 0, s);
  if (e != hipSuccess) return DUST_ERR_HIP;
  if (plan.fused) {
    e = dust::launch_head_fused(logits, zbf16, targets, T, V, sigma, K, stream, seed, g_hat,
                                losses_opt, op, s);
    if (e != hipSuccess) return DUST_ERR_HIP;
    if ((e = record(stage_events, 1, s)) != hipSuccess) return DUST_ERR_HIP;
    if ((e = record(stage_events, 2, s)) != hipSuccess) return DUST_ERR_HIP;
  } else {
    e = dust::launch_head_losses(logits, zbf16, targets, T, V, sigma, K, stream, seed,
                                 losses_opt, delta, s);
    if (e != hipSuccess) return DUST_ERR_HIP;
    if ((e = dust::launch_centre(delta, K, T, delta, s)) != hipSuccess) return DUST_ERR_HIP;
    if (gamma != 0.f &&
        (e = dust::launch_reward_scan(delta, K, T, seq_len, gamma, delta, s)) != hipSuccess)
      return DUST_ERR_HIP;
    if ((e = record(stage_events, 1, s)) != hipSuccess) return DUST_ERR_HIP;
    e = dust::launch_error_estimate(delta, K, T, V, sigma, stream, seed, 0, K, g_hat, op, s);
    if (e != hipSuccess) return DUST_ERR_HIP;
    if ((e = record(stage_events, 2, s)) != hipSuccess) return DUST_ERR_HIP;
  }
  e = dust::launch_outer_sum16(op, g_hat, V, G_W, gemm_ws, s);
  if (e != hipSuccess) return DUST_ERR_HIP;
  return hip_status(record(stage_events, 3, s));
}

dust_status dust_linear_estimate(const void* X, dust_dtype x_dt, const float* c, int64_t T,
                                 int64_t d_in, int64_t N, int64_t seq_len, float sigma, int64_t K,
                                 float gamma, uint64_t seed, uint32_t stream, int64_t draw0,
                                 int64_t K_total, float* g_hat, float* G_W, void* workspace,
                                 size_t workspace_bytes, dust_stream_t s_,
                                 const dust_event_t* stage_events) {
  if (!X || !c || !g_hat || !G_W || !dtype_ok(x_dt)) return DUST_ERR_INVALID_ARG;
  if (!draws_ok(draw0, K, K_total)) return DUST_ERR_INVALID_ARG;
  if (T <= 0 || !width_ok(N) || d_in <= 0 || K <= 0 || K > kMaxK) return DUST_ERR_INVALID_ARG;
  if (T > kMaxT || d_in > kMaxWidth) return DUST_ERR_UNSUPPORTED;
  if (seq_len <= 0 || T % seq_len != 0) return DUST_ERR_INVALID_ARG;
  if (!sigma_ok(sigma) || !gamma_ok(gamma)) return DUST_ERR_INVALID_ARG;
  if (T * N > kMaxElems || T * d_in > kMaxElems || K * T > kMaxElems || N * d_in > kMaxElems)
    return DUST_ERR_UNSUPPORTED;
  if (!dust::outer_sum_supported(T, N, d_in)) return DUST_ERR_UNSUPPORTED;
  const LinearPlan plan = linear_plan(T, d_in, N, K, gamma);
  if (workspace == nullptr || workspace_bytes < plan.total()) return DUST_ERR_WORKSPACE;

  hipStream_t s = as_stream(s_);
  char* ws = reinterpret_cast<char*>(aligned_base(workspace));
  float* r = reinterpret_cast<float*>(ws);
  void* gemm_ws = ws + align_up(plan.r_bytes);

  hipError_t e = record(stage_events, 0, s);
  if (e != hipSuccess) return DUST_ERR_HIP;
  const float* rr = c;
  if (gamma != 0.f) {
    if ((e = dust::launch_reward_scan(c, K, T, seq_len, gamma, r, s)) != hipSuccess)
      return DUST_ERR_HIP;
    rr = r;
  }
  if ((e = record(stage_events, 1, s)) != hipSuccess) return DUST_ERR_HIP;
  const dust::Gemm16Out op = dust::outer_sum_operands(gemm_ws, T, N, d_in, X, x_dt == DUST_BF16);
  if ((e = dust::launch_error_estimate(rr, K, T, N, sigma, stream, seed, (uint32_t)draw0,
                                      K_total, g_hat, op, s)) != hipSuccess)
    return DUST_ERR_HIP;
  if ((e = record(stage_events, 2, s)) != hipSuccess) return DUST_ERR_HIP;
  if ((e = dust::launch_outer_sum16(op, g_hat, N, G_W, gemm_ws, s)) != hipSuccess)
    return DUST_ERR_HIP;
  return hip_status(record(stage_events, 3, s));
}

dust_status dust_noise(uint64_t seed, uint32_t stream, int64_t draw0, int64_t ndraw, int64_t T,
                       int64_t N, float* out, dust_stream_t s) {
  if (!out || ndraw < 0 || T < 0 || !width_ok(N) || draw0 < 0) return DUST_ERR_INVALID_ARG;
  if (draw0 > ((int64_t)1 << 32) - ndraw || T > ((int64_t)1 << 32)) return DUST_ERR_INVALID_ARG;
  if (!prod_le(ndraw, T, kMaxElems / N)) return DUST_ERR_UNSUPPORTED;
  return hip_status(dust::launch_noise_fill(out, ndraw, T, N, (uint32_t)draw0, stream, seed,
                                            as_stream(s)));
}

dust_status dust_philox4x32_10(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n,
                               dust_stream_t s) {
  if (n < 0 || n > kMaxElems) return DUST_ERR_INVALID_ARG;
  if (n > 0 && (!ctr || !out)) return DUST_ERR_INVALID_ARG;
  return hip_status(dust::launch_philox_raw(ctr, out, n, seed, as_stream(s)));
}

dust_status dust_head_losses(const void* logits, dust_dtype logits_dt, const int32_t* targets,
                             int64_t T, int64_t V, float sigma, int64_t K, uint64_t seed,
                             uint32_t stream, float* losses, dust_stream_t s) {
  if (!logits || !targets || !losses || !dtype_ok(logits_dt)) return DUST_ERR_INVALID_ARG;
  if (T <= 0 || !width_ok(V) || K <= 0 || K > kMaxK || !sigma_ok(sigma))
    return DUST_ERR_INVALID_ARG;
  if (T > kMaxTokens || T * V > kMaxElems || K * T > kMaxElems) return DUST_ERR_UNSUPPORTED;
  return hip_status(dust::launch_head_losses(logits, logits_dt == DUST_BF16, targets, T, V, sigma,
                                             K, stream, seed, losses, nullptr, as_stream(s)));
}

dust_status dust_centre(const float* x, int64_t K, int64_t T, float* c, dust_stream_t s) {
  if (!x || !c || K <= 0 || T <= 0) return DUST_ERR_INVALID_ARG;
  if (T > kMaxTokens || !prod_le(K, T, kMaxElems)) return DUST_ERR_UNSUPPORTED;
  return hip_status(dust::launch_centre(x, K, T, c, as_stream(s)));
}

dust_status dust_reward_scan(const float* c, int64_t K, int64_t T, int64_t seq_len, float gamma,
                             float* r, dust_stream_t s) {
  if (!c || !r || K <= 0 || T <= 0) return DUST_ERR_INVALID_ARG;
  if (seq_len <= 0 || T % seq_len != 0 || !gamma_ok(gamma)) return DUST_ERR_INVALID_ARG;
  if (!prod_le(K, T, kMaxElems)) return DUST_ERR_UNSUPPORTED;
  return hip_status(dust::launch_reward_scan(c, K, T, seq_len, gamma, r, as_stream(s)));
}

dust_status dust_error_estimate(const float* r, int64_t K, int64_t T, int64_t N, float sigma,
                                uint64_t seed, uint32_t stream, int64_t draw0, int64_t K_total,
                                float* g_hat, dust_stream_t s) {
  if (!r || !g_hat || K <= 0 || K > kMaxK || T <= 0 || !width_ok(N) || !sigma_ok(sigma))
    return DUST_ERR_INVALID_ARG;
  if (!draws_ok(draw0, K, K_total)) return DUST_ERR_INVALID_ARG;
  if (T > kMaxTokens || T * N > kMaxElems || K * T > kMaxElems) return DUST_ERR_UNSUPPORTED;
  const dust::Gemm16Out none{};  // no G_W operands wanted
  return hip_status(
      dust::launch_error_estimate(r, K, T, N, sigma, stream, seed, (uint32_t)draw0, K_total,
                                  g_hat, none, as_stream(s)));
}

dust_status dust_outer_sum(const float* g_hat, const void* X, dust_dtype x_dt, int64_t T,
                           int64_t N, int64_t d, float* G_W, void* workspace,
                           size_t workspace_bytes, dust_stream_t s) {
  if (!g_hat || !X || !G_W || !dtype_ok(x_dt)) return DUST_ERR_INVALID_ARG;
  if (T <= 0 || N <= 0 || d <= 0) return DUST_ERR_INVALID_ARG;
  if (T > kMaxT || N > kMaxWidth || d > kMaxWidth) return DUST_ERR_UNSUPPORTED;
  if (T * N > kMaxElems || T * d > kMaxElems || N * d > kMaxElems) return DUST_ERR_UNSUPPORTED;
  if (!dust::outer_sum_supported(T, N, d)) return DUST_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < dust_outer_sum_workspace_size(T, N, d))
    return DUST_ERR_WORKSPACE;
  return hip_status(dust::launch_outer_sum(g_hat, X, x_dt == DUST_BF16, T, N, d, G_W,
                                           aligned_base(workspace), as_stream(s)));
}

dust_status dust_perturbed_linear(const void* X, const void* W, dust_dtype dt, int64_t T,
                                  int64_t d, int64_t N, float sigma, uint64_t seed,
                                  uint32_t stream, int64_t draw0, int64_t ndraw, float* Y,
                                  dust_stream_t s) {
  if (!X || !W || !Y || !dtype_ok(dt)) return DUST_ERR_INVALID_ARG;
  if (T <= 0 || N <= 0 || N % 4 != 0 || d <= 0 || d % 8 != 0) return DUST_ERR_INVALID_ARG;
  if (T > kMaxTokens || N > kMaxWidth || d > kMaxWidth) return DUST_ERR_UNSUPPORTED;
  if (!dust::perturbed_linear_supported(T, N)) return DUST_ERR_UNSUPPORTED;
  if (!sigma_ok(sigma) || draw0 < 0 || ndraw < 0 || draw0 > ((int64_t)1 << 32) - ndraw)
    return DUST_ERR_INVALID_ARG;
  if (ndraw * T > kMaxElems / N) return DUST_ERR_UNSUPPORTED;
  // the operand windows of one 128-row tile stay inside 32-bit byte offsets
  if (128 * d * (dt == DUST_F32 ? 4 : 2) > (((int64_t)1 << 31) - 1)) return DUST_ERR_UNSUPPORTED;
  return hip_status(dust::launch_perturbed_linear(X, W, dt == DUST_BF16, T, N, d, sigma, seed,
                                                  stream, (uint32_t)draw0, ndraw, Y,
                                                  as_stream(s)));
}

size_t dust_embedding_workspace_size(int64_t T, int64_t N, int64_t vocab) {
  if (T < 0 || N <= 0 || vocab <= 0) return kAlign;
  if (T > kMaxT || N > kMaxWidth || vocab > kMaxVocab) return kAlign;
  return dust::embedding_workspace_bytes(T, N, vocab) + kAlign;
}

dust_status dust_embedding_grad(const int32_t* ids, const float* g_hat, int64_t T, int64_t N,
                                int64_t vocab, float* G_E, void* workspace,
                                size_t workspace_bytes, dust_stream_t s) {
  if (!ids || !g_hat || !G_E || T < 0 || N <= 0 || N % 4 != 0 || vocab <= 0)
    return DUST_ERR_INVALID_ARG;
  if (T > kMaxT || N > kMaxWidth || vocab > kMaxVocab || T * N > kMaxElems ||
      vocab * N > kMaxElems)
    return DUST_ERR_UNSUPPORTED;
  if (((T + 511) / 512) * vocab > ((int64_t)1 << 31)) return DUST_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < dust_embedding_workspace_size(T, N, vocab))
    return DUST_ERR_WORKSPACE;
  return hip_status(dust::launch_embedding_grad(ids, g_hat, T, N, vocab, G_E,
                                                aligned_base(workspace), as_stream(s)));
}

dust_status dust_embedding_grad_noalloc(const int32_t* ids, const float* g_hat, int64_t T,
                                        int64_t N, int64_t vocab, float* G_E, dust_stream_t s) {
  if (!ids || !g_hat || !G_E || T < 0 || N <= 0 || N % 4 != 0 || vocab <= 0)
    return DUST_ERR_INVALID_ARG;
  if (T > kMaxT || N > kMaxWidth || vocab > kMaxVocab || T * N > kMaxElems ||
      vocab * N > kMaxElems)
    return DUST_ERR_UNSUPPORTED;
  if (((T + 511) / 512) * vocab > ((int64_t)1 << 31)) return DUST_ERR_UNSUPPORTED;
  if (dust::embedding_workspace_bytes(T, N, vocab) > DUST_EMBEDDING_NOALLOC_BYTES)
    return DUST_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (dust::embedding_static_scratch(&scratch) != hipSuccess) return DUST_ERR_HIP;
  return hip_status(dust::launch_embedding_grad(ids, g_hat, T, N, vocab, G_E, scratch,
                                                as_stream(s)));
}

size_t dust_embedding_noalloc_bytes(int64_t T, int64_t N, int64_t vocab) {
  if (T < 0 || N <= 0 || vocab <= 0) return 0;
  if (T > kMaxT || N > kMaxWidth || vocab > kMaxVocab) return 0;
  return dust::embedding_workspace_bytes(T, N, vocab);
}

dust_status dust_sgd_momentum(float* W, const float* G, float* m, int64_t n, float lr,
                              float momentum, float weight_decay, dust_stream_t s) {
  if (n < 0 || (n > 0 && (!W || !G || !m))) return DUST_ERR_INVALID_ARG;
  if (n > kMaxElems) return DUST_ERR_UNSUPPORTED;
  if (!std::isfinite(lr) || !std::isfinite(momentum) || !std::isfinite(weight_decay))
    return DUST_ERR_INVALID_ARG;
  return hip_status(dust::launch_sgd_momentum(W, G, m, n, lr, momentum, weight_decay,
                                              as_stream(s)));
}

dust_status dust_adam(float* W, const float* G, float* m, float* v, int64_t n, float lr,
                      float beta1, float beta2, float eps, float weight_decay, int64_t step,
                      dust_stream_t s) {
  if (n < 0 || (n > 0 && (!W || !G || !m || !v)) || step < 1) return DUST_ERR_INVALID_ARG;
  if (n > kMaxElems) return DUST_ERR_UNSUPPORTED;
  if (!std::isfinite(lr) || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) ||
      !(eps > 0.f) || !std::isfinite(eps) || !std::isfinite(weight_decay))
    return DUST_ERR_INVALID_ARG;
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  if (!(bc1 > 0.0) || !(bc2 > 0.0)) return DUST_ERR_INVALID_ARG;
  return hip_status(dust::launch_adam(W, G, m, v, n, lr, beta1, beta2, eps, weight_decay,
                                      (float)(1.0 / bc1), (float)(1.0 / std::sqrt(bc2)),
                                      as_stream(s)));
}

dust_status dust_ce_grad(const void* logits, dust_dtype dt, const int32_t* targets, int64_t T,
                         int64_t V, float* out, dust_stream_t s) {
  if (!logits || !targets || !out || !dtype_ok(dt) || T < 0 || V <= 0) return DUST_ERR_INVALID_ARG;
  if (T > kMaxTokens || !prod_le(T, V, kMaxElems)) return DUST_ERR_UNSUPPORTED;
  return hip_status(dust::launch_ce_grad(logits, dt == DUST_BF16, targets, T, V, out,
                                         as_stream(s)));
}

dust_status dust_check_targets(const int32_t* targets, int64_t T, int64_t V, int32_t* flag,
                               dust_stream_t s_) {
  if (!targets || T < 0 || V <= 0) return DUST_ERR_INVALID_ARG;
  if (flag == nullptr && dust::check_targets_own_flag(&flag) != hipSuccess) return DUST_ERR_HIP;
  hipStream_t s = as_stream(s_);
  if (dust::launch_check_targets(targets, T, V, flag, s) != hipSuccess) return DUST_ERR_HIP;
  int32_t h = 0;
  if (hipMemcpyAsync(&h, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
    return DUST_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DUST_ERR_HIP;
  return h ? DUST_ERR_TARGETS : DUST_OK;
}

}  // extern "C"
