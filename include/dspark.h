/*
 * dspark.h — C ABI of libdspark: the DSpark Markov-head draft, the
 * hardware-aware prefix scheduler and the prefix-match verify step, as
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles and sections only):
 *   [P-blog] "DSpark: DeepSeek's new speculative decoding work (Video + Blog)"
 *   [P-wisp] "DSpark: Overcoming the Efficiency Wall in LLM Speculative Decoding"
 *   [P-news] "DeepSeek's DSpark just fixed the two things that held back
 *             faster AI inference"
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers to contiguous row-major storage
 *     owned by the caller.  The library keeps no pointer once the enqueued
 *     work has finished and allocates no device memory on these calls; all
 *     scratch memory comes from the caller's `workspace`.
 *   - Work is enqueued on `stream` and the call returns; outputs are valid
 *     once the stream has been synchronised.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     an error nothing is launched and outputs are left untouched.  Errors
 *     are reported by the return code; dspark_last_error() gives a
 *     thread-local message for the last failing call of the calling thread.
 *   - Nothing aborts or prints.
 *   - Token ids outside [0, V) are clamped to the vocabulary before any
 *     memory access (results are then meaningless but memory stays in
 *     bounds).  Inputs must be finite.
 *   - Calls are reentrant; concurrent calls need separate workspaces.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int dspark_status;
enum {
  DSPARK_OK = 0,
  DSPARK_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad enum      */
  DSPARK_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle  */
  DSPARK_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
  DSPARK_ERR_HIP = 4           /* a HIP runtime call or launch failed        */
};

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;     /* storage of U, h, W1, W2 */
typedef enum { DSPARK_GREEDY = 0, DSPARK_GUMBEL = 1 } dspark_sampling;
/* How dspark_markov_draft launches its persistent kernel (process-wide). */
typedef enum {
  DSPARK_LAUNCH_COOPERATIVE = 0,  /* cooperative launch: every workgroup is guaranteed resident (default) */
  DSPARK_LAUNCH_EXCLUSIVE = 1     /* plain launch; the caller guarantees no other kernel runs meanwhile */
} dspark_launch;
/* Verify-length policy of dspark_serve. */
typedef enum {
  DSPARK_POLICY_GLOBAL = 0,           /* dspark_schedule on the iteration's own survivals */
  DSPARK_POLICY_GLOBAL_DELAYED2 = 1,  /* dspark_schedule on the survivals of iteration t - 2 */
  DSPARK_POLICY_THRESHOLD = 2         /* dspark_schedule_threshold on the iteration's survivals */
} dspark_policy;

/* Bytes of workspace dspark_markov_draft needs for this shape (a multiple of
 * 256).  Returns 0 for B*gamma == 0.  Needs no GPU. */
size_t dspark_draft_workspace_bytes(int B, int gamma, int V, int r);

/* Bytes of workspace dspark_rnn_draft needs: the Markov-head workspace plus
 * the recurrent state (2 x B x r bf16).  Returns 0 for B*gamma == 0 or
 * r <= 0.  Needs no GPU. */
size_t dspark_rnn_draft_workspace_bytes(int B, int gamma, int V, int r);

/*
 * dspark_markov_draft — one block of semi-autoregressive drafting with the
 * Markov sequential head, its confidence head, Sequential Temperature
 * Scaling and the prefix-survival product.
 *
 * Defined by: [P-blog] §4 "Semi-Autoregressive Generation" (parallel stage:
 * the anchor is the first prediction position, so gamma positions give gamma
 * base logit vectors U_k; sequential stage: transition bias added to U_k;
 * Markov head: first-order transition B(x_{k-1}, x_k), low-rank B = W1 W2
 * with W1 an embedding lookup and W2 a logits projection); [P-blog] §5
 * "Confidence-Scheduled Verification" (c_k from a linear projection and a
 * sigmoid of the backbone hidden state at k and the Markov embedding of the
 * previous draft token; Sequential Temperature Scaling with one temperature
 * per position; the cumulative product as the prefix survival); [P-news]
 * "How DSpark combines the best of both worlds" (rank-256 factorisation).
 *
 * For every request b and k = 1..gamma, with x_0 = anchor[b]:
 *   e       = W1[x_{k-1}]                                    (gather)
 *   z_k(v)  = U[b][k-1][v] + sum_j e[j] * W2[j][v]           (fp32 accumulate)
 *   x_k     = smallest v maximising z_k(v)            (GREEDY)
 *           = smallest v maximising z_k(v) + G(seed,b,k,v)   (GUMBEL)
 *   c_k     = 1 / (1 + exp(-(conf_w . [h[b][k-1] ; e] + conf_b) / sts_T[k-1]))
 *   S_k     = S_{k-1} * c_k   (S_0 = 1, fp32 multiply)
 * G is standard Gumbel noise -ln(-ln u) from the Philox4x32-10 counter-based
 * generator: key = (seed low 32 bits, seed high 32 bits), counter =
 * (v >> 2, k, b, 0), output word v & 3, u = (2 * (word >> 9) + 1) * 2^-24.
 *
 * Arguments
 *   B, gamma      requests, draft positions per request (0 is a no-op)
 *   V, r, d       vocabulary size, Markov rank, backbone hidden size
 *   dtype         storage of U, h, W1, W2: DSPARK_F32 (r % 4 == 0, r <= 64)
 *                 or DSPARK_BF16 (r % 32 == 0, r <= 256)
 *   anchor  int32 [B]                x_0 per request
 *   U             [B][gamma][V]      base logits U_k
 *   h             [B][gamma][d]      backbone hidden states h_k
 *   W1            [V][r]             transition embedding table
 *   W2            [r][V]             transition logits projection
 *   conf_w  fp32  [d + r]            hidden-state weights first, then embedding weights
 *   conf_b        confidence bias
 *   sts_T   fp32  [gamma]            T_1..T_gamma (> 0)
 *   mode, seed    sampling rule; seed used only for DSPARK_GUMBEL
 *   tokens  int32 [B][gamma] out     x_1..x_gamma
 *   logit   fp32  [B][gamma] out     z_k(x_k), without Gumbel noise
 *   conf    fp32  [B][gamma] out     c_k
 *   surv    fp32  [B][gamma] out     S_k
 *   workspace     >= dspark_draft_workspace_bytes(B, gamma, V, r) bytes,
 *                 256-byte aligned, zero-filled (e.g. hipMemsetAsync) before
 *                 its first use and before any call whose B or gamma differs
 *                 from the previous call's on it: its counters and arg-max
 *                 slots (for B <= 16 also every workgroup's winner keys, up
 *                 to gamma * B * 512 * 12 bytes) sit at offsets that depend
 *                 on B and gamma.  A call
 *                 leaves them zero again, so calls of the same B and gamma
 *                 reuse it without clearing.  A workspace found dirty by the
 *                 barrier check (for B <= 16: a non-zero winner key of the
 *                 first position) is cleaned by the call, whose tokens are
 *                 then all -1 (stale arg-max slots are not detected).
 * The call is one kernel launch.  If the kernel cannot synchronise its
 * workgroups (it never can deadlock: its waits are bounded) every token of
 * the call is -1.
 * Limits: gamma <= 64, d <= 65536, V <= 2^24 and V small enough that the
 * GPU's compute units can hold W2 on chip (V <= 163840 on MI355X);
 * otherwise DSPARK_ERR_UNSUPPORTED.
 */
dspark_status dspark_markov_draft(
    int B, int gamma, int V, int r, int d, dspark_dtype dtype,
    const int32_t* anchor, const void* U, const void* h, const void* W1, const void* W2,
    const float* conf_w, float conf_b, const float* sts_T,
    dspark_sampling mode, uint64_t seed,
    int32_t* tokens, float* logit, float* conf, float* surv,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_markov_draft_noalloc — dspark_markov_draft without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments (minus workspace / workspace_bytes), outputs, errors and
 * limits as dspark_markov_draft; the kernels are the same.  The scratch
 * memory comes from a static device array of DSPARK_NOALLOC_SCRATCH_BYTES
 * per GPU, held by the library until the process ends.  Its device address
 * is looked up on the first call on each device (that call also zero-fills
 * it with a small kernel on `stream`); every completed call leaves its
 * counters and slots zero again, and a call whose B or gamma differs from the
 * previous call's on the device first clears the part it needs with the same
 * small kernel.  Nothing is allocated on any call.
 *   - Shapes whose dspark_draft_workspace_bytes(B, gamma, V, r) exceeds
 *     DSPARK_NOALLOC_SCRATCH_BYTES return DSPARK_ERR_UNSUPPORTED before
 *     anything is enqueued (B = 256, gamma = 16 needs about 1.1 MiB).
 *   - All calls on one GPU share its scratch: calls that can overlap (other
 *     streams, threads or processes on the same device) race and must not
 *     be issued; calls on one stream are ordered and safe.
 *   - A call whose kernel could not synchronise (tokens all -1) leaves the
 *     scratch dirty; the next call cleans it and also returns all -1, as a
 *     dirty workspace does for dspark_markov_draft.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

dspark_status dspark_markov_draft_noalloc(
    int B, int gamma, int V, int r, int d, dspark_dtype dtype,
    const int32_t* anchor, const void* U, const void* h, const void* W1, const void* W2,
    const float* conf_w, float conf_b, const float* sts_T,
    dspark_sampling mode, uint64_t seed,
    int32_t* tokens, float* logit, float* conf, float* surv, hipStream_t stream);

/*
 * dspark_schedule — hardware-aware prefix scheduler: per-request verify
 * lengths that maximise expected committed tokens per unit of verify-step
 * cost.
 *
 * Defined by: [P-wisp] "2. The Hardware-Aware Prefix Scheduler" (throughput
 * maximisation from calibrated survival probabilities and the current
 * steps-per-second curve; per-request verify lengths); [P-blog] §6 (global
 * throughput maximisation; verify cost depends on load); [P-blog] §3 (the
 * low-confidence suffix is dropped); [P-news] "Confidence-scheduled
 * verification" (strict prefix-matching survival).
 *
 * With n = B + M verify tokens (each request's anchor plus M drafts), choose
 * lens in {0..gamma}^B with sum lens = M maximising
 *   Phi = (B + sum_i sum_{k <= lens_i} S_{i,k}) / t_step[n - n_min].
 * Exactly: all (i, k) are ranked by (S desc, i asc, k asc); gains are the
 * fixed-point values rint(S * 2^32) (ties to even) summed in int64; Phi(M)
 * is one IEEE fp64 division of (B * 2^32 + sum of the top-M gains) by
 * t_step[B + M - n_min]; M* is the smallest M with the largest Phi over
 * M = 0..min(B*gamma, n_min + n_count - 1 - B); lens_i counts request i's
 * entries among the top M*.
 *
 * Arguments
 *   surv   fp32 [B][gamma]   prefix survivals, each row non-increasing, in [0, 1]
 *   t_step fp64 [n_count]    verify-step cost for n = n_min .. n_min + n_count - 1 (> 0)
 *   n_min, n_count           need n_min <= B <= n_min + n_count - 1
 *   lens      int32 [B] out
 *   m_out     int32 [1] out  M*
 *   objective fp64  [1] out  Phi(M*) / 2^32 (may be NULL)
 *   workspace  NULL, or >= dspark_schedule_workspace_bytes(B, gamma) bytes,
 *              256-byte aligned, its first 2048 bytes (ticket counters) zero
 *              before its first use; every call leaves them zero again,
 *              whatever B and gamma (the rest is scratch).  Calls sharing a
 *              workspace must not overlap.
 * With a workspace the call is one launch of about B*gamma/16 workgroups
 * that rank the entries by comparison (no sort) and hand the scan, the
 * divisions and the arg-max to the last workgroup to finish; without one, a
 * single workgroup sorts in LDS (slower, no workspace).  Both give the same
 * result bit for bit for survivals that are not NaN; rows need not be
 * non-increasing for either.
 * Errors: DSPARK_ERR_WORKSPACE for a workspace that is too small or
 * misaligned.  Limits: B * gamma <= 16384, else DSPARK_ERR_UNSUPPORTED.
 */
dspark_status dspark_schedule(
    int B, int gamma, const float* surv, const double* t_step, int n_min, int n_count,
    int32_t* lens, int32_t* m_out, double* objective, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/* Bytes of workspace dspark_schedule needs (a multiple of 256); 0 for
 * B*gamma == 0 or B*gamma > 16384.  Needs no GPU. */
size_t dspark_schedule_workspace_bytes(int B, int gamma);

/*
 * dspark_verify — strict prefix-match verification of the scheduled drafts.
 *
 * Defined by: [P-news] opening (the target checks the whole draft block in
 * one forward pass and keeps the drafts up to the first disagreement; the
 * disagreeing draft and all later ones are discarded); [P-blog] §3 (the
 * target verifies the scheduled prefix; the next anchor is the target's
 * bonus token).
 *
 *   accepted[b] = largest a <= lens[b] with tokens[b][j] == target[b][j] for all j < a
 *   bonus[b]    = target[b][accepted[b]]
 *
 * Arguments
 *   tokens int32 [B][gamma]      drafts x_1..x_gamma
 *   target int32 [B][gamma + 1]  the target model's tokens at positions 1..gamma+1
 *   lens   int32 [B]             scheduled lengths (clamped to [0, gamma])
 *   accepted, bonus int32 [B] out
 */
dspark_status dspark_verify(
    int B, int gamma, const int32_t* tokens, const int32_t* target, const int32_t* lens,
    int32_t* accepted, int32_t* bonus, hipStream_t stream);

/*
 * dspark_rnn_draft — dspark_markov_draft with the RNN sequential head in
 * place of the Markov head.
 *
 * Defined by: [P-blog] §4 "Semi-Autoregressive Generation" (sequential stage:
 * the transition bias B_k(x_0, x_{<k}, x_k) may depend on the anchor and the
 * whole draft prefix; "Two instantiations of the sequential block", RNN head:
 * its state carries information from every earlier position of the draft
 * block) and [P-blog] §5 (confidence head inputs: the hidden state and the
 * Markov embedding of the previous draft token).  The pages give no
 * equations for the RNN head; this library's reading is a per-channel
 * decayed state, computed in fp32 and stored in bf16:
 *   s_0     = 0
 *   s_k[j]  = bf16( fp32( fp32(decay[j] * s_{k-1}[j]) + W1[x_{k-1}][j] ) )
 *             (product and sum rounded separately, bf16 round to nearest even)
 *   z_k(v)  = U[b][k-1][v] + sum_j s_k[j] * W2[j][v]      (fp32 accumulate)
 * and x_k, c_k (with e = W1[x_{k-1}], not s_k) and S_k as in
 * dspark_markov_draft.  decay = 0 gives exactly the Markov head; decay = 1
 * sums the embeddings of x_0 .. x_{k-1}.
 *
 * Arguments as dspark_markov_draft, plus
 *   decay   fp32  [r]     per-channel decay of the recurrent state
 * with dtype DSPARK_BF16 only (DSPARK_ERR_UNSUPPORTED otherwise) and
 *   workspace     >= dspark_rnn_draft_workspace_bytes(B, gamma, V, r) bytes,
 *                 with the same zero-fill rule as dspark_markov_draft (the
 *                 state section needs none).
 * Errors and limits as dspark_markov_draft.
 */
dspark_status dspark_rnn_draft(
    int B, int gamma, int V, int r, int d, dspark_dtype dtype,
    const int32_t* anchor, const void* U, const void* h, const void* W1, const void* W2,
    const float* decay, const float* conf_w, float conf_b, const float* sts_T,
    dspark_sampling mode, uint64_t seed,
    int32_t* tokens, float* logit, float* conf, float* surv,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_gumbel_from_words — the Gumbel noise of the drafting kernels
 * (dspark_markov_draft, dspark_rnn_draft, dspark_parallel_draft in
 * DSPARK_GUMBEL mode) for given 32-bit hash words, computed by the same
 * device function: out[i] = -ln(-ln u), u = (2 * (words[i] >> 9) + 1) * 2^-24.
 *
 * Defined by: Gumbel-max sampling from softmax(z_k) (the reading of the
 * drafting distribution of [P-blog] §4, whose formula the pages lose); the
 * words themselves come from the Philox4x32-10 counter layout documented at
 * dspark_markov_draft.  For checking the noise arithmetic on its own.
 *
 * Arguments
 *   n             number of words (0 is a no-op)
 *   words  uint32 [n]   device, 4-byte aligned
 *   out    fp32   [n] out device, 4-byte aligned
 * Errors: DSPARK_ERR_INVALID_ARG for n < 0 or null / misaligned arrays.
 */
dspark_status dspark_gumbel_from_words(int n, const uint32_t* words, float* out, hipStream_t stream);

/*
 * dspark_parallel_draft — drafting with the parallel stage alone: the
 * baseline without a sequential head, for measuring what the Markov head
 * adds to the drafting time.
 *
 * Defined by: [P-blog] §1 "Autoregressive vs Parallel Drafting" (parallel
 * drafters emit the logits of every block position in one pass); §4
 * "Semi-Autoregressive Generation", parallel stage (base logits U_k); §2
 * "Speedup formula" (drafting time and acceptance as separate levers).
 *
 * For every request b and k = 1..gamma, independently:
 *   x_k = smallest v maximising U[b][k-1][v]                 (GREEDY)
 *       = smallest v maximising U[b][k-1][v] + G(seed,b,k,v)  (GUMBEL)
 * with G the Gumbel noise of dspark_markov_draft (same generator, key and
 * counter layout), i.e. the tokens dspark_markov_draft produces when W2 = 0.
 *
 * Arguments
 *   B, gamma, V   requests, positions, vocabulary (B * gamma == 0 is a no-op)
 *   dtype         storage of U (DSPARK_F32 or DSPARK_BF16)
 *   U             [B][gamma][V]      base logits, element-aligned
 *   mode, seed    sampling rule; seed used only for DSPARK_GUMBEL
 *   tokens  int32 [B][gamma] out     x_k
 *   logit   fp32  [B][gamma] out     U[b][k-1][x_k], without noise
 * No workspace.  Rows are read with 16-byte loads when V is a multiple of
 * 8 (bf16) or 4 (fp32) and U is 16-byte aligned, element by element
 * otherwise.  Limits: V <= 2^24, B * gamma < 2^31.
 */
dspark_status dspark_parallel_draft(
    int B, int gamma, int V, dspark_dtype dtype, const void* U,
    dspark_sampling mode, uint64_t seed,
    int32_t* tokens, float* logit, hipStream_t stream);

/*
 * dspark_sts_fit — fits the confidence head's per-position temperatures
 * T_1..T_gamma, left to right, on a calibration set.
 *
 * Defined by: [P-blog] §5 "Sequential Temperature Scaling" (raw confidence
 * is overconfident; the joint probability is calibrated position by
 * position, each by a 1-D grid search for the temperature minimising the
 * expected calibration error of the cumulative product, earlier positions
 * held at their calibrated values); [P-wisp] "Critical Insights"
 * (calibration is required for the scheduler); [P-news] (calibration
 * against empirical acceptance).
 *
 * For k = 1..gamma, in order, with S_{n,0} = 1 and y_n = (accepted[n] >= k):
 *   p_n(T)  = S_{n,k-1} * sigmoid(logit[n][k-1] / T)       for every T in grid
 *   ECE(T)  = sum_m |sum_{n: bin(p_n) = m} rint((y_n - p_n) 2^32)| / (2^32 N),
 *             bin(p) = min(floor(p * n_bins), n_bins - 1)
 *   T_k     = the first grid entry with the smallest ECE (compared exactly,
 *             on the integer sums)
 *   S_{n,k} = p_n(T_k)
 * in fp64.  The result is independent of thread and workgroup order.
 *
 * Arguments
 *   N             calibration blocks (0 allowed: every ECE is 0, T_k = grid[0])
 *   gamma         positions (0: no-op)
 *   logit  fp32  [N][gamma]  raw confidence logits (pre-sigmoid, bias included, T = 1)
 *   accepted int32 [N]       accepted drafts per block; values above gamma act
 *                            as gamma, negative ones as 0
 *   grid   fp32  [G]         candidate temperatures, positive and finite
 *   n_bins                   calibration-error bins over [0, 1]
 *   choice int32 [gamma] out grid index of T_k
 *   T_out  fp32  [gamma] out T_k (ready to pass as sts_T to dspark_markov_draft)
 *   ece    fp64  [gamma][G] out the ECE of every candidate at every position
 *   workspace     device memory of dspark_sts_workspace_bytes(N, G, n_bins)
 *                 bytes, 256-byte aligned, any contents (the call clears what
 *                 it needs).  Calls sharing a workspace must not overlap.
 * All arrays are device memory owned by the caller.  Limits: G <= 4096,
 * n_bins <= 256, G * n_bins <= 8192, N <= 2^24, N * gamma < 2^31, else
 * DSPARK_ERR_UNSUPPORTED.  Non-positive or non-finite temperatures and
 * non-finite logits are outside the contract (results unspecified; memory
 * accesses stay in bounds).  Runs gamma + 1 kernel launches on `stream`.
 */
size_t dspark_sts_workspace_bytes(int N, int G, int n_bins);

dspark_status dspark_sts_fit(
    int N, int gamma, const float* logit, const int32_t* accepted, const float* grid,
    int G, int n_bins, int32_t* choice, float* T_out, double* ece,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_schedule_threshold — the static confidence-threshold verify
 * lengths that the hardware-aware scheduler replaces.
 *
 * Defined by: [P-blog] §6 "Hardware-Aware Prefix Scheduler" (existing work
 * verifies by a static confidence threshold); [P-news] "Confidence-scheduled
 * verification" (offline threshold sweeps).
 *
 *   lens[b] = largest l <= gamma with surv[b][j] >= tau for all j < l   (fp32)
 *   m_out[0] = sum of lens
 * The threshold ignores the batch size and the step cost.
 *
 * Arguments
 *   surv fp32 [B][gamma]  prefix survivals;  tau  the threshold
 *   lens int32 [B] out;  m_out int32 [1] out
 * Limits: B * gamma < 2^31.
 */
dspark_status dspark_schedule_threshold(
    int B, int gamma, const float* surv, float tau, int32_t* lens, int32_t* m_out, hipStream_t stream);

/*
 * dspark_serve — `iters` drafting iterations of one batch chained as in
 * serving: draft (dspark_markov_draft), choose the verify lengths, verify
 * (dspark_verify); the bonus tokens of iteration t are the anchors of
 * iteration t + 1.  Everything is enqueued on `stream` without host
 * synchronisation; each kernel is the one the single-call entry points run.
 *
 * Defined by: [P-blog] §3 "Speculative decoding" (draft, verify, keep the
 * accepted prefix and the target's token, repeat) and §4 parallel stage
 * (the anchor opens the next block); [P-blog] §6 and [P-wisp] "2. The
 * Hardware-Aware Prefix Scheduler" (policy GLOBAL); [P-wisp] "Key
 * Takeaways" (asynchrony: scheduling from the predictions of two steps
 * earlier, policy GLOBAL_DELAYED2; iterations 0 and 1 use their own
 * survivals); [P-blog] §6 (the static threshold, policy THRESHOLD).
 *
 * Arguments (t = 0..iters-1; per-iteration arrays are stacked, iteration-major)
 *   iters                      iterations (0: no-op)
 *   B, gamma, V, r, d, dtype   as dspark_markov_draft
 *   anchor0 int32 [B]          anchors of iteration 0
 *   U  [iters][B][gamma][V], h [iters][B][gamma][d]     base logits and hidden states
 *   W1, W2, conf_w, conf_b, sts_T, mode                 as dspark_markov_draft
 *   seed                       iteration t samples with seed + t (GUMBEL)
 *   target int32 [iters][B][gamma + 1]                  the target's tokens
 *   t_step, n_min, n_count     step-cost table as dspark_schedule (unused by THRESHOLD)
 *   policy, tau                verify-length policy; tau used by THRESHOLD
 *   tokens, logit, conf, surv  [iters][B][gamma] out   draft outputs
 *   lens, accepted, bonus      int32 [iters][B] out
 *   m_out                      int32 [iters] out       scheduled drafts per iteration
 *   workspace                  >= dspark_serve_workspace_bytes(B, gamma, V, r) bytes, 256-byte
 *                              aligned: the drafting workspace, then the scheduler's (whose
 *                              counters follow the drafting part), zero-filled as the
 *                              drafting workspace (before the first use and on a change of B
 *                              or gamma)
 * Every argument is checked before the first launch; a HIP error later
 * leaves the iterations before it enqueued.  Limits: those of
 * dspark_markov_draft, and B * gamma <= 16384 for the GLOBAL policies.
 */
/*
 * dspark_step — one step of the path in one call: dspark_markov_draft, then
 * dspark_schedule on the drafted survivals (with its workspace), then
 * dspark_verify of the drafts against the target's tokens.
 *
 * Defined by: the three operations it chains (see dspark_markov_draft,
 * dspark_schedule and dspark_verify for the passages); [P-blog] §3 (draft,
 * schedule by confidence, verify the scheduled prefix).
 *
 * Outputs are exactly those of the three calls made in order on the same
 * stream: tokens, logit, conf, surv [B][gamma]; lens, accepted, bonus [B];
 * m_out [1] (the objective is not returned).
 *
 * Arguments: those of dspark_markov_draft (Markov head), followed by target
 * [B][gamma + 1] and the step-cost table (t_step, n_min, n_count) as in
 * dspark_verify and dspark_schedule, then the outputs.
 *   workspace  >= dspark_step_workspace_bytes(B, gamma, V, r) bytes, 256-byte
 *              aligned: the drafting workspace, then the scheduler's, zero-filled
 *              as dspark_serve's (before the first use and on a change of B or
 *              gamma).
 * For bf16 storage at r = 256 on the whole-tile path with 16 < B and
 * B * gamma <= 1024, the three run in one launch: after the last draft position every workgroup
 * ranks its share of the survivals, and the workgroup that finishes last runs
 * the scheduler's remaining steps and the verify (this saves the two launch
 * gaps that dominate small batches).  Otherwise the call makes the three
 * launches.  Errors and limits: the union of the three calls'.
 */
dspark_status dspark_step(
    int B, int gamma, int V, int r, int d, dspark_dtype dtype,
    const int32_t* anchor, const void* U, const void* h, const void* W1, const void* W2,
    const float* conf_w, float conf_b, const float* sts_T, dspark_sampling mode, uint64_t seed,
    const int32_t* target, const double* t_step, int n_min, int n_count,
    int32_t* tokens, float* logit, float* conf, float* surv,
    int32_t* lens, int32_t* m_out, int32_t* accepted, int32_t* bonus,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace dspark_step needs (the same as dspark_serve's): the
 * drafting workspace plus the scheduler's.  Returns 0 for B*gamma == 0.  Needs
 * no GPU. */
size_t dspark_step_workspace_bytes(int B, int gamma, int V, int r);

/* Bytes of workspace dspark_serve needs: dspark_draft_workspace_bytes plus
 * dspark_schedule_workspace_bytes.  Returns 0 for B*gamma == 0.  Needs no
 * GPU. */
size_t dspark_serve_workspace_bytes(int B, int gamma, int V, int r);

dspark_status dspark_serve(
    int iters, int B, int gamma, int V, int r, int d, dspark_dtype dtype,
    const int32_t* anchor0, const void* U, const void* h, const void* W1, const void* W2,
    const float* conf_w, float conf_b, const float* sts_T, dspark_sampling mode, uint64_t seed,
    const int32_t* target, const double* t_step, int n_min, int n_count,
    dspark_policy policy, float tau,
    int32_t* tokens, float* logit, float* conf, float* surv,
    int32_t* lens, int32_t* accepted, int32_t* bonus, int32_t* m_out,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_set_draft_launch / dspark_get_draft_launch — how the drafting
 * kernel is launched, for the whole process (dspark_markov_draft and
 * dspark_serve).  Not an operation of the pages: a property of this
 * implementation.
 *
 * The drafting kernel keeps one workgroup per compute unit resident for the
 * whole call and synchronises them between draft positions, so every
 * workgroup must run at the same time.  DSPARK_LAUNCH_COOPERATIVE (the
 * default) asks the runtime for that guarantee; on ROCm 7 the cooperative
 * launch path costs about 13 us more per launch than a plain launch and does
 * not overlap a launch with the preceding kernel (measured on an almost empty
 * kernel of the same grid shape).  DSPARK_LAUNCH_EXCLUSIVE launches plainly: the caller
 * guarantees that no other kernel (from any stream or process) runs on the
 * device while a drafting call runs, so the idle device places every
 * workgroup at once — the usual situation of one serving loop per GPU.  If
 * that guarantee is broken the kernel's bounded waits end the call after a
 * few seconds with every token set to -1, and the workspace must be
 * zero-filled again before its next use.
 * Returns DSPARK_ERR_INVALID_ARG for an unknown mode.
 */
dspark_status dspark_set_draft_launch(dspark_launch mode);
dspark_launch dspark_get_draft_launch(void);

/* Static description of a status code. */
const char* dspark_status_string(dspark_status s);

/* Message for the calling thread's last failing call ("" if none). */
const char* dspark_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
