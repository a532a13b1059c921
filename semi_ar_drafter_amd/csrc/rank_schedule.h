// Shared by the scheduler kernels and the fused draft-schedule-verify step:
// the scheduler's sort key and fixed-point gains, DPP wave reductions, and
// the multi-workgroup ranking scheduler as two device functions (every
// workgroup's ranking phase, and the tail run by the workgroup that draws
// the last ticket).  Sources: "DSpark: Overcoming the Efficiency Wall in LLM
// Speculative Decoding", "2. The Hardware-Aware Prefix Scheduler"; "DSpark:
// DeepSeek's new speculative decoding work", §6.
#pragma once
#include "device_util.h"
#include "launch.h"

namespace dspark {

// Sort key: ascending key order = descending survival, then ascending flat
// index (request-major), so the first M keys are the scheduler's top M.
__device__ __forceinline__ uint64_t sched_key(float s, uint32_t flat) {
  return (uint64_t(~ord_f32(s)) << 32) | uint64_t(flat);
}
__device__ __forceinline__ long long gain_fixed(uint64_t key) {
  const float s = unord_f32(~uint32_t(key >> 32));
  return (long long)rint(double(s) * 4294967296.0);
}

// Wave-wide scan and arg-max with DPP lane shifts (no LDS crossbar): row_shr
// by 1, 2, 4 and 8 within each row of 16 lanes, then row_bcast:15 into rows
// 1 and 3 and row_bcast:31 into rows 2 and 3.  Lanes whose source is outside
// the row, or whose row is masked, receive the identity passed as `old`.
template <int CTRL, int ROWM>
__device__ __forceinline__ uint32_t dpp32(uint32_t old, uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(x), CTRL, ROWM, 0xF, false));
}
template <int CTRL, int ROWM>
__device__ __forceinline__ long long dpp_i64(long long v) {
  const uint64_t u = uint64_t(v);
  return (long long)((uint64_t(dpp32<CTRL, ROWM>(0u, uint32_t(u >> 32))) << 32) | dpp32<CTRL, ROWM>(0u, uint32_t(u)));
}
// inclusive prefix sum over the lanes of the wave
__device__ __forceinline__ long long wave_scan_i64(long long v) {
  v += dpp_i64<0x111, 0xF>(v);
  v += dpp_i64<0x112, 0xF>(v);
  v += dpp_i64<0x114, 0xF>(v);
  v += dpp_i64<0x118, 0xF>(v);
  v += dpp_i64<0x142, 0xA>(v);
  v += dpp_i64<0x143, 0xC>(v);
  return v;
}
template <int CTRL, int ROWM>
__device__ __forceinline__ void dpp_argmax_step(double& b, int& m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, b);
  const uint32_t lo = dpp32<CTRL, ROWM>(0u, uint32_t(u));
  const uint32_t hi = dpp32<CTRL, ROWM>(0xFFF00000u, uint32_t(u >> 32));   // -inf where no source
  const int om = int(dpp32<CTRL, ROWM>(0x7FFFFFFFu, uint32_t(m)));
  const double ob = __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
  if (ob > b || (ob == b && om < m)) {
    b = ob;
    m = om;
  }
}
// larger value, then smaller index, over the wave; the result is in lane 63
__device__ __forceinline__ void wave_argmax_to_lane63(double& b, int& m) {
  dpp_argmax_step<0x111, 0xF>(b, m);
  dpp_argmax_step<0x112, 0xF>(b, m);
  dpp_argmax_step<0x114, 0xF>(b, m);
  dpp_argmax_step<0x118, 0xF>(b, m);
  dpp_argmax_step<0x142, 0xA>(b, m);
  dpp_argmax_step<0x143, 0xC>(b, m);
}

// Multi-workgroup scheduler.  No sort: the rank of a key is the number of
// keys below it, and with every key distinct the ranks are a permutation, so
// a key stored at its rank lands where a sort would put it.  Workgroup g
// ranks keys g*K .. g*K + K - 1 against all n keys, which its threads hold
// in registers (E per thread): per key, a wave compares against its 64*E
// keys, and the ballot's population count is the wave's share of the rank.
//
// The compares are 32-bit.  A key is (h, i): h = ~ord(S) (high word), i =
// the flat index; (h', i') < (h, i) iff h' < h, or h' == h and i' < i.
// Threads hold entries in 64-entry blocks of consecutive i, and a
// workgroup's K <= 64 keys all fall in one block c.  For an entry of a block
// wholly below c (i' < i for every key), "less" is h' <= h, i.e. h' - 1 < h;
// for an entry above c it is h' < h.  So each held entry is stored as h' - 1
// or h' by its block, one unsigned compare per (key, entry) gives the rank
// apart from ties inside block c, and those are added per key from a ballot
// of h' == h over block c masked to the lanes i' < i.  Exact for every
// survival that is not NaN (h then lies in [2^23 - 1, 2^32 - 2^23], so h' - 1
// and the padding value 2^32 - 1 stay in range).
// Each workgroup stores its keys at their ranks, each beside the step cost
// t_step[B + rank + 1 - n_min] that the division at M = rank + 1 needs,
// then takes a ticket; the workgroup that draws the last ticket has the
// whole sorted array visible, and does the rest as the one-workgroup kernel:
// the scan of gains, one fp64 division per M, the arg-max, and per-request
// counts of the first M* sorted keys (LDS counters).
//
// The last workgroup's thread t takes the Q = ceil(n / T) consecutive ranks
// t*Q .. t*Q + Q - 1, so the sorted array is stored transposed (rank r at
// entry (r % Q) * T + r / Q) and that workgroup's j-th load is contiguous
// across threads.  Tickets are taken in two levels (per group of
// workgroups, then per group) so that no counter sees more than a few dozen
// atomics at once; the last workgroup puts every counter back to zero, so a
// workspace whose first kRankHeader bytes start zero has them zero again
// after each call.
constexpr int kRankThreads = 512;
constexpr int kRankWaves = kRankThreads / 64;
constexpr int kTicketGroups = 8;
constexpr int kTicketStride = 32;   // counters 128 bytes apart
constexpr size_t kRankHeader = 2048;
static_assert((kTicketGroups + 1) * kTicketStride * 4 <= int(kRankHeader), "ticket counters fit the header");
static_assert(kMaxScheduleItems <= 32 * kRankThreads, "at most 32 keys per thread (the largest instance)");

struct RankEntry {
  uint64_t key;
  double t;   // t_step[B + rank + 1 - n_min] (1.0 past m_max)
};

// LDS bytes of the per-request counters: four 8-bit counters per word when a
// count cannot pass 255 (gamma <= 255), else one per word (then B <= 64).
__host__ __device__ inline int rank_counter_words(int B, int gamma) { return gamma <= 255 ? (B + 3) / 4 : B; }
__device__ __forceinline__ int rank_count(const unsigned int* counters, int b, int gamma) {
  return gamma <= 255 ? int((counters[b >> 2] >> (8 * (b & 3))) & 255u) : int(counters[b]);
}

// LDS the ranking functions use, provided by the calling kernel.
template <int K>
struct RankShared {
  int (*wcnt)[kRankWaves];   // [K][kRankWaves] per-wave counts of each key
  long long* wave_tot;       // [kRankWaves]
  double* red_phi;           // [kRankWaves]
  int* red_m;                // [kRankWaves]
  int* flag;                 // [1]
  unsigned int* counters;    // [rank_counter_words(B, gamma)]
};

// Every participating workgroup (index gidx < G = ceil(n / K)): ranks keys
// gidx*K .. gidx*K + K - 1, stores them with their step costs at their
// ranks, and takes a ticket.  Returns true (uniform over the workgroup) in
// the one workgroup that drew the last ticket.  DEV_IN: the survivals were
// written earlier in the same kernel by other workgroups (device-scope
// stores), so they are read with device-scope loads.  kRankThreads threads.
template <int E, int K, bool DEV_IN>
__device__ __forceinline__ bool rank_phase(int gidx, int G, int B, int gamma, const float* __restrict__ surv,
                                           const double* __restrict__ t_step, int n_min, int n_count,
                                           unsigned int* tickets, RankEntry* sorted, const RankShared<K>& sh) {
  static_assert((K & (K - 1)) == 0 && K >= 4 && K <= 64, "keys per workgroup: a power of two, one per lane");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B * gamma;
  const int g0 = gidx * K;
  const int m_max = min(n, n_min + n_count - 1 - B);
  const int Q = (n + kRankThreads - 1) / kRankThreads;   // ranks per thread of the last workgroup, <= E
  auto in = [&](int i) -> float {
    if constexpr (DEV_IN)
      return load_dev(&surv[i]);
    else
      return surv[i];
  };

  // every entry's high word, E per thread (entry j*T + tid in slot j),
  // lowered by one in blocks wholly below this workgroup's block c0; past n
  // the largest value.  Loads are unconditional (clamped index) so that they
  // all issue before the first wait; n >= 1.
  const int c0 = g0 & ~63;
  uint32_t hw[E];
  float sv[E];
#pragma unroll
  for (int j = 0; j < E; ++j) sv[j] = in(min(j * kRankThreads + tid, n - 1));
  // this workgroup's keys, one per lane (past n: copies of the last key,
  // ranked but never stored), and block c0, one entry per lane
  const float kv = in(min(g0 + (lane & (K - 1)), n - 1));
  const float cv = in(min(c0 + lane, n - 1));
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = j * kRankThreads + tid;
    const uint32_t below = (j * kRankThreads + wave * 64 + 64 <= c0) ? 1u : 0u;   // wave-uniform
    hw[j] = e < n ? ~ord_f32(sv[j]) - below : ~0u;
  }
  const uint32_t hc = c0 + lane < n ? ~ord_f32(cv) : ~0u;
  // KG keys at a time, so that their compares and counts interleave (KG * E
  // compare masks live at once: at most 32, which keeps them in SGPRs)
  constexpr int KG = E >= 32 ? 1 : E >= 16 ? 2 : 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KG) {
    uint32_t h[KG];
    int cnt[KG];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      h[u] = ~ord_f32(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(kv), k0 + u)));
      // ties inside block c0 at lower flat index, counted once (by wave 0)
      const int below_lanes = g0 + k0 + u - c0;   // in [0, 64)
      cnt[u] = wave == 0 ? __popcll(__ballot(hc == h[u]) & ((1ull << below_lanes) - 1)) : 0;
    }
#pragma unroll
    for (int j = 0; j < E; ++j)
#pragma unroll
      for (int u = 0; u < KG; ++u) cnt[u] += __popcll(__ballot(hw[j] < h[u]));
    int mine_cnt = cnt[0];
#pragma unroll
    for (int u = 1; u < KG; ++u)
      if (lane == u) mine_cnt = cnt[u];
    if (lane < KG) sh.wcnt[k0 + lane][wave] = mine_cnt;
  }
  __syncthreads();
  if (tid < K && g0 + tid < n) {
    int rank = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) rank += sh.wcnt[tid][w];
    const double t = rank + 1 <= m_max ? t_step[B + rank + 1 - n_min] : 1.0;
    RankEntry* slot = &sorted[(rank % Q) * kRankThreads + rank / Q];
    store_dev(&slot->key, sched_key(kv, uint32_t(g0 + tid)));
    store_dev(&slot->t, t);
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const int grp = gidx % kTicketGroups;
    const unsigned int in_group = unsigned((G - grp + kTicketGroups - 1) / kTicketGroups);
    const unsigned int groups = unsigned(min(G, kTicketGroups));
    bool last = false;
    if (__hip_atomic_fetch_add(&tickets[(1 + grp) * kTicketStride], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == in_group - 1)
      last = __hip_atomic_fetch_add(&tickets[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
    sh.flag[0] = last;
  }
  __syncthreads();
  return sh.flag[0] != 0;
}

// The workgroup that drew the last ticket: scan of gains, one fp64 division
// per M, arg-max, per-request counts of the first M* sorted keys (left in
// sh.counters, read with rank_count) and lens / m_out / objective (may be
// null); puts every ticket counter back to zero.
template <int E, int K>
__device__ __forceinline__ void rank_tail(int B, int gamma, const double* __restrict__ t_step, int n_min,
                                          int n_count, unsigned int* tickets, const RankEntry* sorted,
                                          int32_t* lens, int32_t* m_out, double* objective,
                                          const RankShared<K>& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B * gamma;
  const int m_max = min(n, n_min + n_count - 1 - B);
  const int Q = (n + kRankThreads - 1) / kRankThreads;
  unsigned int* counters = sh.counters;
  // Every other workgroup's stores completed before its ticket.  Up to 8
  // entries per thread they are read with device-scope loads (past any stale
  // copy of an earlier call's array in this L2); for larger arrays it is
  // cheaper to drop this L2's stale lines once (an acquire fence, about
  // 0.7 us) and read through it.
  constexpr bool kDeviceLoads = E <= 8;
  if constexpr (!kDeviceLoads) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ranks [p0, p1) per thread, M = p + 1
  const int p0 = min(tid * Q, m_max), p1 = min(p0 + Q, m_max);
  uint64_t kp[E];
  double tv[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const RankEntry* v = &sorted[min(j, Q - 1) * kRankThreads + tid];
    if constexpr (kDeviceLoads) {
      kp[j] = load_dev(&v->key);
      tv[j] = __builtin_bit_cast(double, load_dev(reinterpret_cast<const uint64_t*>(&v->t)));
    } else {
      kp[j] = v->key;
      tv[j] = v->t;
    }
  }
  const double t0 = t_step[B - n_min];
  const bool packed = gamma <= 255;
  for (int w = tid; w < rank_counter_words(B, gamma); w += kRankThreads) counters[w] = 0u;
  long long local = 0;
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (p0 + j < p1) local += gain_fixed(kp[j]);
  const long long incl = wave_scan_i64(local);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  long long before = 0;
#pragma unroll
  for (int w = 0; w < kRankWaves; ++w)
    if (w < wave) before += sh.wave_tot[w];
  long long G = before + incl - local;   // sum of gains at ranks < p0

  const long long base = (long long)B << 32;
  double best = -INFINITY;
  int best_m = 0x7FFFFFFF;
  if (tid == 0) {
    best = double(base) / t0;
    best_m = 0;
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (p0 + j >= p1) break;
    G += gain_fixed(kp[j]);
    const double phi = double(base + G) / tv[j];
    if (phi > best) {
      best = phi;
      best_m = p0 + j + 1;
    }
  }
  // arg-max: larger phi, then smaller M (a total order, M being distinct)
  wave_argmax_to_lane63(best, best_m);
  if (lane == 63) {
    sh.red_phi[wave] = best;
    sh.red_m[wave] = best_m;
  }
  __syncthreads();
  // every thread reduces the per-wave winners itself (no broadcast barrier)
  double bb = sh.red_phi[0];
  int bm = sh.red_m[0];
#pragma unroll
  for (int w = 1; w < kRankWaves; ++w) {
    const double ob = sh.red_phi[w];
    const int om = sh.red_m[w];
    if (ob > bb || (ob == bb && om < bm)) {
      bb = ob;
      bm = om;
    }
  }
  const int mstar = bm;
  if (wave == 0) {
    if (lane == 0) {
      m_out[0] = bm;
      if (objective) objective[0] = bb / 4294967296.0;
    }
    if (lane <= kTicketGroups) store_dev(&tickets[lane * kTicketStride], 0u);
  }
  // lens[b] = how many of the first M* sorted keys belong to request b
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (p0 + j >= min(p1, mstar)) break;
    const uint32_t b = uint32_t(kp[j]) / uint32_t(gamma);
    if (packed)
      atomicAdd(&counters[b >> 2], 1u << (8 * (b & 3)));
    else
      atomicAdd(&counters[b], 1u);
  }
  __syncthreads();
  for (int b = tid; b < B; b += kRankThreads) lens[b] = rank_count(counters, b, gamma);
}

}  // namespace dspark
