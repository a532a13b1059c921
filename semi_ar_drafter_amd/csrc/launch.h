// Host-side launch interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// Upper bound on the draft kernel's grid (one workgroup per compute unit).
constexpr int kMaxDraftWorkgroups = 512;
// Largest number of requests one workgroup can own for the confidence epilogue.
constexpr int kMaxOwnedRows = 64;
// Requests per group in the draft kernel (LDS holds one group's embeddings).
constexpr int kMaxGroupRows = 128;
// Batches of at most this many requests (one group of at most 16 rows)
// synchronise the draft positions through per-workgroup winner keys instead
// of arrival counters.
constexpr int kSmallBatch = 16;
// Distance (in 32-bit words) between the per-group arrival counters (one
// 128-byte line each: every workgroup polls them).
constexpr int kBarStride = 32;
// Scheduler: one workgroup sorts all (request, position) keys in LDS.
constexpr int kMaxScheduleItems = 16384;
// dspark_step runs draft, schedule and verify in one launch up to this many
// verify candidates (B * gamma), and makes three launches above it.
constexpr int kFusedStepItems = 1024;

// The schedule and verify part of a fused step (dspark_step).
struct StepArgs {
  const double* t_step;
  int n_min, n_count;
  const int32_t* target;
  int32_t *lens, *m_out, *accepted, *bonus;
  void* sched_ws;   // the scheduler's workspace (schedule_workspace_bytes)
};

struct DraftArgs {
  int B, gamma, V, r, d;
  bool bf16, gumbel;
  uint64_t seed;
  const int32_t* anchor;
  const void *U, *h, *W1, *W2;
  const float* conf_w;
  float conf_b;
  const float* sts_T;
  int32_t* tokens;
  float *logit, *conf, *surv;
  void* ws;
  size_t ws_bytes;
  bool exclusive;   // plain launch: the caller guarantees nothing else runs on the device
  const float* decay = nullptr;   // non-null: RNN head with this per-channel state decay [r] (bf16 only)
  bool noalloc = false;           // ws ignored: the per-device static scratch is used (Markov head)
  const StepArgs* step = nullptr;  // non-null: schedule and verify in the same launch when the shape allows
};

// Workspace carve-up of the draft call (byte offsets, 256-aligned).  Every
// section before zpart must be zero when a call starts (each call leaves it
// so); wkeys and wz are empty unless B <= kSmallBatch.
struct DraftWorkspace {
  size_t ctrl, bar, slots, wkeys, wz, zpart, hdot, state, total;
};
// r_state: the RNN head's rank (its bf16 state [2][B][r] is carved out too), 0 for the Markov head.
DraftWorkspace draft_workspace_layout(int B, int gamma, int r_state);

// Returns hipSuccess or the first HIP error; sets *unsupported (with a reason)
// when the shape is outside what the kernels handle.
// *fused (optional) tells whether the schedule and verify of a.step ran in the
// same launch (else the caller launches them).
hipError_t launch_markov_draft(const DraftArgs& a, hipStream_t stream, const char** unsupported,
                               bool* fused = nullptr);

// Allocation-free draft entry point: size of the per-device static scratch
// that replaces the caller's workspace, and its device address (set up and
// zero-filled on `stream` at the first call on the current device).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
// A call whose shape (B << 32 | gamma) differs from the previous one on the
// device clears the first zero_bytes (its counters and slots) first.
hipError_t noalloc_scratch(hipStream_t stream, void** out, uint64_t shape, size_t zero_bytes);

// Bytes of the multi-workgroup scheduler's workspace (0 for B*gamma == 0 or
// above kMaxScheduleItems).
size_t schedule_workspace_bytes(int B, int gamma);
// workspace == nullptr: the one-workgroup kernel; else the multi-workgroup
// kernel on a workspace of schedule_workspace_bytes(B, gamma) bytes.
hipError_t launch_schedule(int B, int gamma, const float* surv, const double* t_step, int n_min, int n_count,
                           int32_t* lens, int32_t* m_out, double* objective, void* workspace, hipStream_t stream);

hipError_t launch_schedule_threshold(int B, int gamma, const float* surv, float tau, int32_t* lens, int32_t* m_out,
                                    hipStream_t stream);

hipError_t launch_parallel_draft(int B, int gamma, int V, bool bf16, const void* U, bool gumbel, uint64_t seed,
                                 int32_t* tokens, float* logit, hipStream_t stream);
hipError_t launch_gumbel_words(int n, const uint32_t* words, float* out, hipStream_t stream);

// Sequential-temperature fit: limits of one workgroup's LDS histogram.
constexpr int kMaxStsGrid = 4096;
constexpr int kMaxStsBins = 256;
constexpr int kMaxStsHist = 8192;     // nbins * G
constexpr int kMaxStsBlocks = 1 << 24;

struct StsArgs {
  int N, gamma, G, nbins;
  const float* logit;
  const int32_t* accepted;
  const float* grid;
  int32_t* choice;
  float* T_out;
  double* ece;
  void* ws;
};

struct StsWorkspace {
  size_t ctrl, hist, S, total;
};
StsWorkspace sts_workspace_layout(int N, int G, int nbins);
size_t sts_lds_bytes(int G, int nbins);

hipError_t launch_sts_fit(const StsArgs& a, hipStream_t stream);

hipError_t launch_verify(int B, int gamma, const int32_t* tokens, const int32_t* target,
                         const int32_t* lens, int32_t* accepted, int32_t* bonus, hipStream_t stream);

}  // namespace dspark
