// C ABI of libdspark (declared in include/dspark.h): host-side argument
// validation, workspace sizing, status reporting and dispatch to the HIP
// launchers.  Every check runs before anything is enqueued, so argument
// errors are reported synchronously and without touching the GPU.
#include <atomic>
#include <cstdio>
#include <cstring>

#include "../../include/dspark.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

dspark_status fail(dspark_status s, const char* fmt, const char* detail = nullptr) {
  if (detail)
    std::snprintf(g_last_error, sizeof g_last_error, fmt, detail);
  else
    std::snprintf(g_last_error, sizeof g_last_error, "%s", fmt);
  return s;
}

dspark_status hip_fail(hipError_t e) {
  std::snprintf(g_last_error, sizeof g_last_error, "HIP error %d: %s", int(e), hipGetErrorString(e));
  return DSPARK_ERR_HIP;
}

std::atomic<int> g_draft_launch{DSPARK_LAUNCH_COOPERATIVE};

constexpr int kMaxGamma = 64;
constexpr int kMaxD = 65536;
constexpr int kMaxV = 1 << 24;

}  // namespace

extern "C" {

const char* dspark_status_string(dspark_status s) {
  switch (s) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_INVALID_ARG: return "invalid argument";
    case DSPARK_ERR_UNSUPPORTED: return "unsupported shape or type";
    case DSPARK_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case DSPARK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dspark_last_error(void) { return g_last_error; }

dspark_status dspark_set_draft_launch(dspark_launch mode) {
  g_last_error[0] = '\0';
  if (mode != DSPARK_LAUNCH_COOPERATIVE && mode != DSPARK_LAUNCH_EXCLUSIVE)
    return fail(DSPARK_ERR_INVALID_ARG, "unknown launch mode");
  g_draft_launch.store(int(mode));
  return DSPARK_OK;
}

dspark_launch dspark_get_draft_launch(void) { return dspark_launch(g_draft_launch.load()); }

size_t dspark_draft_workspace_bytes(int B, int gamma, int V, int r) {
  (void)V;
  (void)r;
  if (B <= 0 || gamma <= 0) return 0;
  return dspark::draft_workspace_layout(B, gamma, 0).total;
}

size_t dspark_serve_workspace_bytes(int B, int gamma, int V, int r) {
  const size_t draft = dspark_draft_workspace_bytes(B, gamma, V, r);
  if (draft == 0) return 0;
  return draft + dspark::schedule_workspace_bytes(B, gamma);
}

size_t dspark_rnn_draft_workspace_bytes(int B, int gamma, int V, int r) {
  (void)V;
  if (B <= 0 || gamma <= 0 || r <= 0) return 0;
  return dspark::draft_workspace_layout(B, gamma, r).total;
}

namespace {

// Shared by the Markov-head and RNN-head entry points (decay == nullptr: Markov).
dspark_status draft_impl(int B, int gamma, int V, int r, int d, dspark_dtype dtype, const int32_t* anchor,
                         const void* U, const void* h, const void* W1, const void* W2, const float* decay,
                         bool rnn, const float* conf_w, float conf_b, const float* sts_T, dspark_sampling mode,
                         uint64_t seed, int32_t* tokens, float* logit, float* conf, float* surv, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, bool noalloc = false,
                         const dspark::StepArgs* step = nullptr, bool* fused = nullptr) {
  g_last_error[0] = '\0';
  if (B < 0 || gamma < 0 || V < 0 || r < 0 || d < 0)
    return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return fail(DSPARK_ERR_INVALID_ARG, "unknown dtype");
  if (mode != DSPARK_GREEDY && mode != DSPARK_GUMBEL) return fail(DSPARK_ERR_INVALID_ARG, "unknown sampling mode");
  if (rnn && dtype != DSPARK_BF16) return fail(DSPARK_ERR_UNSUPPORTED, "the RNN head needs bf16 storage");
  if (B == 0 || gamma == 0) return DSPARK_OK;
  if (V < 1 || r < 1) return fail(DSPARK_ERR_INVALID_ARG, "V and r must be positive");
  if (!anchor || !U || !W1 || !W2 || !conf_w || !sts_T || !tokens || !logit || !conf || !surv ||
      (d > 0 && !h) || (rnn && !decay))
    return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (gamma > kMaxGamma) return fail(DSPARK_ERR_UNSUPPORTED, "gamma > 64");
  if (d > kMaxD) return fail(DSPARK_ERR_UNSUPPORTED, "d > 65536");
  if (V > kMaxV) return fail(DSPARK_ERR_UNSUPPORTED, "V > 2^24");
  const int elem = dtype == DSPARK_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(W1) % 16 || reinterpret_cast<uintptr_t>(U) % elem ||
      reinterpret_cast<uintptr_t>(W2) % elem || (h && reinterpret_cast<uintptr_t>(h) % elem) ||
      (rnn && reinterpret_cast<uintptr_t>(decay) % 4))
    return fail(DSPARK_ERR_INVALID_ARG, "misaligned tensor (W1 needs 16-byte alignment)");
  const size_t need = rnn ? dspark_rnn_draft_workspace_bytes(B, gamma, V, r) : dspark_draft_workspace_bytes(B, gamma, V, r);
  if (noalloc) {
    // allocation-free entry point: the launcher takes the static per-device
    // scratch in place of a workspace, once every check has passed
    if (need > dspark::kNoAllocScratchBytes)
      return fail(DSPARK_ERR_UNSUPPORTED, "shape needs more workspace than the 8 MiB static scratch");
  } else if (!workspace || workspace_bytes < need)
    return fail(DSPARK_ERR_WORKSPACE, rnn ? "workspace missing or smaller than dspark_rnn_draft_workspace_bytes()"
                                          : "workspace missing or smaller than dspark_draft_workspace_bytes()");
  if (!noalloc && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(DSPARK_ERR_WORKSPACE, "workspace not 256-byte aligned");

  dspark::DraftArgs a;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.d = d;
  a.bf16 = dtype == DSPARK_BF16;
  a.gumbel = mode == DSPARK_GUMBEL;
  a.seed = seed;
  a.anchor = anchor;
  a.U = U;
  a.h = h;
  a.W1 = W1;
  a.W2 = W2;
  a.conf_w = conf_w;
  a.conf_b = conf_b;
  a.sts_T = sts_T;
  a.tokens = tokens;
  a.logit = logit;
  a.conf = conf;
  a.surv = surv;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.exclusive = g_draft_launch.load() == DSPARK_LAUNCH_EXCLUSIVE;
  a.decay = rnn ? decay : nullptr;
  a.noalloc = noalloc;
  a.step = step;
  const char* why = nullptr;
  hipError_t e = dspark::launch_markov_draft(a, stream, &why, fused);
  if (why) return fail(DSPARK_ERR_UNSUPPORTED, "%s", why);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

}  // namespace

dspark_status dspark_markov_draft(int B, int gamma, int V, int r, int d, dspark_dtype dtype,
                                  const int32_t* anchor, const void* U, const void* h, const void* W1,
                                  const void* W2, const float* conf_w, float conf_b, const float* sts_T,
                                  dspark_sampling mode, uint64_t seed, int32_t* tokens, float* logit,
                                  float* conf, float* surv, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return draft_impl(B, gamma, V, r, d, dtype, anchor, U, h, W1, W2, nullptr, false, conf_w, conf_b, sts_T, mode, seed,
                    tokens, logit, conf, surv, workspace, workspace_bytes, stream);
}

dspark_status dspark_markov_draft_noalloc(int B, int gamma, int V, int r, int d, dspark_dtype dtype,
                                          const int32_t* anchor, const void* U, const void* h, const void* W1,
                                          const void* W2, const float* conf_w, float conf_b, const float* sts_T,
                                          dspark_sampling mode, uint64_t seed, int32_t* tokens, float* logit,
                                          float* conf, float* surv, hipStream_t stream) {
  return draft_impl(B, gamma, V, r, d, dtype, anchor, U, h, W1, W2, nullptr, false, conf_w, conf_b, sts_T, mode, seed,
                    tokens, logit, conf, surv, nullptr, 0, stream, /*noalloc=*/true);
}

dspark_status dspark_rnn_draft(int B, int gamma, int V, int r, int d, dspark_dtype dtype, const int32_t* anchor,
                               const void* U, const void* h, const void* W1, const void* W2, const float* decay,
                               const float* conf_w, float conf_b, const float* sts_T, dspark_sampling mode,
                               uint64_t seed, int32_t* tokens, float* logit, float* conf, float* surv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return draft_impl(B, gamma, V, r, d, dtype, anchor, U, h, W1, W2, decay, true, conf_w, conf_b, sts_T, mode, seed,
                    tokens, logit, conf, surv, workspace, workspace_bytes, stream);
}

size_t dspark_schedule_workspace_bytes(int B, int gamma) {
  if (B < 0 || gamma < 0) return 0;
  return dspark::schedule_workspace_bytes(B, gamma);
}

dspark_status dspark_schedule(int B, int gamma, const float* surv, const double* t_step, int n_min, int n_count,
                              int32_t* lens, int32_t* m_out, double* objective, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (B < 0 || gamma < 0 || n_count < 1) return fail(DSPARK_ERR_INVALID_ARG, "negative size or empty step-cost table");
  if (!t_step || !m_out || (B > 0 && (!lens || (gamma > 0 && !surv))))
    return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (n_min > B || (long long)n_min + n_count - 1 < B)
    return fail(DSPARK_ERR_INVALID_ARG, "step-cost table must cover n = B (n_min <= B <= n_min + n_count - 1)");
  if ((long long)B * gamma > dspark::kMaxScheduleItems)
    return fail(DSPARK_ERR_UNSUPPORTED, "B * gamma > 16384");
  if (workspace) {
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(DSPARK_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (workspace_bytes < dspark::schedule_workspace_bytes(B, gamma))
      return fail(DSPARK_ERR_WORKSPACE, "workspace smaller than dspark_schedule_workspace_bytes(B, gamma)");
  }
  hipError_t e =
      dspark::launch_schedule(B, gamma, surv, t_step, n_min, n_count, lens, m_out, objective, workspace, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

dspark_status dspark_parallel_draft(int B, int gamma, int V, dspark_dtype dtype, const void* U,
                                    dspark_sampling mode, uint64_t seed, int32_t* tokens, float* logit,
                                    hipStream_t stream) {
  g_last_error[0] = '\0';
  if (B < 0 || gamma < 0 || V < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return fail(DSPARK_ERR_INVALID_ARG, "unknown dtype");
  if (mode != DSPARK_GREEDY && mode != DSPARK_GUMBEL) return fail(DSPARK_ERR_INVALID_ARG, "unknown sampling mode");
  if (B == 0 || gamma == 0) return DSPARK_OK;
  if (V < 1) return fail(DSPARK_ERR_INVALID_ARG, "V must be positive");
  if (!U || !tokens || !logit) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (V > kMaxV) return fail(DSPARK_ERR_UNSUPPORTED, "V > 2^24");
  if ((long long)B * gamma > 0x7FFFFFFFLL) return fail(DSPARK_ERR_UNSUPPORTED, "B * gamma > 2^31 - 1");
  const int elem = dtype == DSPARK_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(U) % elem) return fail(DSPARK_ERR_INVALID_ARG, "misaligned U");
  hipError_t e = dspark::launch_parallel_draft(B, gamma, V, dtype == DSPARK_BF16, U, mode == DSPARK_GUMBEL, seed,
                                               tokens, logit, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

dspark_status dspark_gumbel_from_words(int n, const uint32_t* words, float* out, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (n < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (n == 0) return DSPARK_OK;
  if (!words || !out) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(words) % 4 || reinterpret_cast<uintptr_t>(out) % 4)
    return fail(DSPARK_ERR_INVALID_ARG, "misaligned array");
  hipError_t e = dspark::launch_gumbel_words(n, words, out, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

dspark_status dspark_schedule_threshold(int B, int gamma, const float* surv, float tau, int32_t* lens,
                                        int32_t* m_out, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (B < 0 || gamma < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (!m_out || (B > 0 && (!lens || (gamma > 0 && !surv)))) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if ((long long)B * gamma > 0x7FFFFFFFLL) return fail(DSPARK_ERR_UNSUPPORTED, "B * gamma > 2^31 - 1");
  hipError_t e = dspark::launch_schedule_threshold(B, gamma, surv, tau, lens, m_out, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

dspark_status dspark_serve(int iters, int B, int gamma, int V, int r, int d, dspark_dtype dtype,
                           const int32_t* anchor0, const void* U, const void* h, const void* W1, const void* W2,
                           const float* conf_w, float conf_b, const float* sts_T, dspark_sampling mode,
                           uint64_t seed, const int32_t* target, const double* t_step, int n_min, int n_count,
                           dspark_policy policy, float tau, int32_t* tokens, float* logit, float* conf,
                           float* surv, int32_t* lens, int32_t* accepted, int32_t* bonus, int32_t* m_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (iters < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative iteration count");
  if (policy != DSPARK_POLICY_GLOBAL && policy != DSPARK_POLICY_GLOBAL_DELAYED2 && policy != DSPARK_POLICY_THRESHOLD)
    return fail(DSPARK_ERR_INVALID_ARG, "unknown scheduling policy");
  if (B < 0 || gamma < 0 || V < 0 || r < 0 || d < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (iters == 0 || B == 0 || gamma == 0) return DSPARK_OK;
  if (!target || !lens || !accepted || !bonus || !m_out || (policy != DSPARK_POLICY_THRESHOLD && !t_step))
    return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (policy != DSPARK_POLICY_THRESHOLD) {
    if (n_count < 1) return fail(DSPARK_ERR_INVALID_ARG, "empty step-cost table");
    if (n_min > B || (long long)n_min + n_count - 1 < B)
      return fail(DSPARK_ERR_INVALID_ARG, "step-cost table must cover n = B (n_min <= B <= n_min + n_count - 1)");
    if ((long long)B * gamma > dspark::kMaxScheduleItems) return fail(DSPARK_ERR_UNSUPPORTED, "B * gamma > 16384");
  }
  // the draft's workspace first, the scheduler's after it
  const size_t draft_bytes = dspark_draft_workspace_bytes(B, gamma, V, r);
  const size_t sched_bytes = policy == DSPARK_POLICY_THRESHOLD ? 0 : dspark::schedule_workspace_bytes(B, gamma);
  if (workspace && workspace_bytes >= draft_bytes && workspace_bytes - draft_bytes < sched_bytes)
    return fail(DSPARK_ERR_WORKSPACE, "workspace smaller than dspark_serve_workspace_bytes(B, gamma, V, r)");
  void* sched_ws = workspace ? static_cast<unsigned char*>(workspace) + draft_bytes : nullptr;
  const size_t elem = dtype == DSPARK_BF16 ? 2 : 4;
  const size_t bg = size_t(B) * size_t(gamma);
  for (int t = 0; t < iters; ++t) {
    const int32_t* anchor = t == 0 ? anchor0 : bonus + size_t(t - 1) * B;
    const unsigned char* Ut = static_cast<const unsigned char*>(U) + size_t(t) * bg * size_t(V) * elem;
    const unsigned char* ht = h ? static_cast<const unsigned char*>(h) + size_t(t) * bg * size_t(d) * elem : nullptr;
    float* surv_t = surv + size_t(t) * bg;
    // iteration 0 validates the draft arguments before anything is enqueued;
    // later iterations differ only by offsets that keep the same alignment
    dspark_status st = dspark_markov_draft(B, gamma, V, r, d, dtype, anchor, Ut, ht, W1, W2, conf_w, conf_b, sts_T,
                                           mode, seed + uint64_t(t), tokens + size_t(t) * bg, logit + size_t(t) * bg,
                                           conf + size_t(t) * bg, surv_t, workspace, workspace_bytes, stream);
    if (st != DSPARK_OK) return st;
    hipError_t e;
    if (policy == DSPARK_POLICY_THRESHOLD) {
      e = dspark::launch_schedule_threshold(B, gamma, surv_t, tau, lens + size_t(t) * B, m_out + t, stream);
    } else {
      const float* src = (policy == DSPARK_POLICY_GLOBAL_DELAYED2 && t >= 2) ? surv + size_t(t - 2) * bg : surv_t;
      e = dspark::launch_schedule(B, gamma, src, t_step, n_min, n_count, lens + size_t(t) * B, m_out + t, nullptr,
                                  sched_ws, stream);
    }
    if (e != hipSuccess) return hip_fail(e);
    e = dspark::launch_verify(B, gamma, tokens + size_t(t) * bg, target + size_t(t) * bg + size_t(t) * B,
                              lens + size_t(t) * B, accepted + size_t(t) * B, bonus + size_t(t) * B, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return DSPARK_OK;
}

size_t dspark_sts_workspace_bytes(int N, int G, int n_bins) {
  if (N < 0 || G < 1 || n_bins < 1 || G > dspark::kMaxStsGrid || n_bins > dspark::kMaxStsBins) return 0;
  return dspark::sts_workspace_layout(N, G, n_bins).total;
}

dspark_status dspark_sts_fit(int N, int gamma, const float* logit, const int32_t* accepted, const float* grid,
                             int G, int n_bins, int32_t* choice, float* T_out, double* ece, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (N < 0 || gamma < 0 || G < 0 || n_bins < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (gamma == 0) return DSPARK_OK;
  if (G < 1 || n_bins < 1) return fail(DSPARK_ERR_INVALID_ARG, "G and n_bins must be positive");
  if (!grid || !choice || !T_out || !ece || (N > 0 && (!logit || !accepted)))
    return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (G > dspark::kMaxStsGrid) return fail(DSPARK_ERR_UNSUPPORTED, "G > 4096");
  if (n_bins > dspark::kMaxStsBins) return fail(DSPARK_ERR_UNSUPPORTED, "n_bins > 256");
  if ((long long)G * n_bins > dspark::kMaxStsHist) return fail(DSPARK_ERR_UNSUPPORTED, "G * n_bins > 8192");
  if (N > dspark::kMaxStsBlocks) return fail(DSPARK_ERR_UNSUPPORTED, "N > 2^24");
  if ((long long)N * gamma > 0x7FFFFFFFLL) return fail(DSPARK_ERR_UNSUPPORTED, "N * gamma > 2^31 - 1");
  if (reinterpret_cast<uintptr_t>(logit) % 4 || reinterpret_cast<uintptr_t>(accepted) % 4 ||
      reinterpret_cast<uintptr_t>(grid) % 4 || reinterpret_cast<uintptr_t>(ece) % 8)
    return fail(DSPARK_ERR_INVALID_ARG, "misaligned tensor");
  const size_t need = dspark_sts_workspace_bytes(N, G, n_bins);
  if (!workspace || workspace_bytes < need)
    return fail(DSPARK_ERR_WORKSPACE, "workspace missing or smaller than dspark_sts_workspace_bytes()");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(DSPARK_ERR_WORKSPACE, "workspace not 256-byte aligned");
  dspark::StsArgs a;
  a.N = N;
  a.gamma = gamma;
  a.G = G;
  a.nbins = n_bins;
  a.logit = logit;
  a.accepted = accepted;
  a.grid = grid;
  a.choice = choice;
  a.T_out = T_out;
  a.ece = ece;
  a.ws = workspace;
  hipError_t e = dspark::launch_sts_fit(a, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

dspark_status dspark_verify(int B, int gamma, const int32_t* tokens, const int32_t* target, const int32_t* lens,
                            int32_t* accepted, int32_t* bonus, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (B < 0 || gamma < 0) return fail(DSPARK_ERR_INVALID_ARG, "negative size");
  if (B == 0) return DSPARK_OK;
  if (!target || !lens || !accepted || !bonus || (gamma > 0 && !tokens))
    return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  hipError_t e = dspark::launch_verify(B, gamma, tokens, target, lens, accepted, bonus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

size_t dspark_step_workspace_bytes(int B, int gamma, int V, int r) { return dspark_serve_workspace_bytes(B, gamma, V, r); }

dspark_status dspark_step(int B, int gamma, int V, int r, int d, dspark_dtype dtype, const int32_t* anchor,
                          const void* U, const void* h, const void* W1, const void* W2, const float* conf_w,
                          float conf_b, const float* sts_T, dspark_sampling mode, uint64_t seed,
                          const int32_t* target, const double* t_step, int n_min, int n_count, int32_t* tokens,
                          float* logit, float* conf, float* surv, int32_t* lens, int32_t* m_out, int32_t* accepted,
                          int32_t* bonus, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (B < 0 || gamma < 0 || V < 0 || r < 0 || d < 0 || n_count < 1)
    return fail(DSPARK_ERR_INVALID_ARG, "negative size or empty step-cost table");
  if (B == 0) return DSPARK_OK;
  if (!target || !t_step || !lens || !m_out || !accepted || !bonus)
    return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
  if (n_min > B || (long long)n_min + n_count - 1 < B)
    return fail(DSPARK_ERR_INVALID_ARG, "step-cost table must cover n = B (n_min <= B <= n_min + n_count - 1)");
  if ((long long)B * gamma > dspark::kMaxScheduleItems) return fail(DSPARK_ERR_UNSUPPORTED, "B * gamma > 16384");
  // the drafting workspace first, the scheduler's after it
  const size_t draft_bytes = dspark_draft_workspace_bytes(B, gamma, V, r);
  const size_t sched_bytes = dspark::schedule_workspace_bytes(B, gamma);
  if (workspace && workspace_bytes >= draft_bytes && workspace_bytes - draft_bytes < sched_bytes)
    return fail(DSPARK_ERR_WORKSPACE, "workspace smaller than dspark_step_workspace_bytes(B, gamma, V, r)");
  if (gamma == 0) {   // nothing to draft or schedule: every length 0, bonus = target[b][0]
    hipError_t e = dspark::launch_schedule(B, 0, nullptr, t_step, n_min, n_count, lens, m_out, nullptr, nullptr,
                                           stream);
    if (e == hipSuccess) e = dspark::launch_verify(B, 0, nullptr, target, lens, accepted, bonus, stream);
    if (e != hipSuccess) return hip_fail(e);
    return DSPARK_OK;
  }
  dspark::StepArgs st;
  st.t_step = t_step;
  st.n_min = n_min;
  st.n_count = n_count;
  st.target = target;
  st.lens = lens;
  st.m_out = m_out;
  st.accepted = accepted;
  st.bonus = bonus;
  st.sched_ws = workspace ? static_cast<unsigned char*>(workspace) + draft_bytes : nullptr;
  bool fused = false;
  dspark_status ds = draft_impl(B, gamma, V, r, d, dtype, anchor, U, h, W1, W2, nullptr, false, conf_w, conf_b,
                                sts_T, mode, seed, tokens, logit, conf, surv, workspace, workspace_bytes, stream,
                                false, &st, &fused);
  if (ds != DSPARK_OK || fused) return ds;
  hipError_t e = dspark::launch_schedule(B, gamma, surv, t_step, n_min, n_count, lens, m_out, nullptr, st.sched_ws,
                                         stream);
  if (e == hipSuccess) e = dspark::launch_verify(B, gamma, tokens, target, lens, accepted, bonus, stream);
  if (e != hipSuccess) return hip_fail(e);
  return DSPARK_OK;
}

}  // extern "C"
