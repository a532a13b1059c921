// Hardware-aware prefix scheduler and prefix-match verify for gfx950.
//
// Scheduler ("DSpark: Overcoming the Efficiency Wall in LLM Speculative
// Decoding", "2. The Hardware-Aware Prefix Scheduler"; "DSpark: DeepSeek's
// new speculative decoding work", §6): choose per-request verify lengths
// maximising (B + sum of scheduled survivals) / t_step(B + M).  Survival is
// non-increasing along each request, so the best set of M drafts is the top
// M by (S desc, request asc, position asc) and only M has to be searched.
// Two kernels give the same result bit for bit:
//  * with a workspace (schedule_rank_kernel): every entry's rank counted by
//    comparison across about B*gamma/16 workgroups, the keys stored at their
//    ranks, and the last workgroup to finish does the scan of fixed-point
//    gains, one fp64 division per candidate M, the arg-max and the
//    per-request counts;
//  * without one (schedule_kernel): one workgroup of 1024 threads sorts the
//    64-bit keys in LDS (merge sort, bitonic above 8192 items), then the same
//    scan, divisions, arg-max and counts.
// Verify takes one lane per draft position (gamma < 64) or one thread per
// request.
//
// Static-threshold scheduler (the baseline of "DSpark: DeepSeek's new
// speculative decoding work", §6): each request verifies the longest prefix
// whose survival is at least a fixed threshold.
//
// Verify ("DeepSeek's DSpark just fixed the two things that held back faster
// AI inference", opening; "DSpark: DeepSeek's new speculative decoding
// work", §3): longest matching prefix of the scheduled drafts and the
// target's token right after it.
#include "device_util.h"
#include "launch.h"
#include "rank_schedule.h"

namespace dspark {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kPrefetchSteps = 4;   // step costs per thread held in registers across the sort

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(int B, int gamma, const float* __restrict__ surv,
                                                                 const double* __restrict__ t_step, int n_min,
                                                                 int n_count, int32_t* lens, int32_t* m_out,
                                                                 double* objective) {
  __shared__ uint64_t keys[kMaxScheduleItems];
  __shared__ long long wave_tot[kSchedWaves];
  __shared__ double red_phi[kSchedWaves];
  __shared__ int red_m[kSchedWaves];
  __shared__ uint64_t s_tau;
  __shared__ int s_mstar;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = B * gamma;
  int n2 = 4;
  while (n2 < n) n2 <<= 1;

  // The step costs this thread divides by, read before the sort so that
  // their latency hides behind it.
  const int m_max = min(n, n_min + n_count - 1 - B);
  const int C = (m_max + kSchedThreads - 1) / kSchedThreads;
  const int p0 = min(tid * C, m_max), p1 = min(p0 + C, m_max);
  const double t0 = tid == 0 ? t_step[B - n_min] : 1.0;
  double ts[kPrefetchSteps];
#pragma unroll
  for (int j = 0; j < kPrefetchSteps; ++j) ts[j] = (p0 + j < p1) ? t_step[B + p0 + j + 1 - n_min] : 1.0;

  // Sort the keys ascending.  Up to half the key array, a merge sort: runs
  // of 4 sorted in registers, then merge levels that ping-pong between the
  // two halves of `keys`, each thread placing 4 outputs after a search for
  // where its output range splits the two input runs (merge path).  Every
  // level reads and writes the keys once; the bitonic network used for
  // larger inputs passes over them once per stage.  Keys are distinct apart
  // from the padding, so the order is the same either way.
  //
  // Survival rows are non-increasing by construction (the documented input),
  // so each request's keys are usually in order already: if every row is
  // (checked), runs of gamma keys are sorted and, with gamma a power of two,
  // the merge starts at runs of gamma.
  const uint64_t* sorted = keys;
  bool merged = false;   // the sorted keys are in one half of `keys`, the other half is free
  if (n2 <= kMaxScheduleItems / 2) {
    merged = true;
    uint64_t* src = keys;
    uint64_t* dst = keys + kMaxScheduleItems / 2;
    bool in_order = true;   // this thread's keys continue their rows in order
    for (int q = tid * 4; q < n2; q += kSchedThreads * 4) {
      uint64_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (q + j < n) ? sched_key(surv[q + j], uint32_t(q + j)) : ~0ull;
      // the next key of the same row (the first key of the next quad)
      const bool cont = q + 4 < n && (q + 4) % gamma != 0;
      const uint64_t nx = cont ? sched_key(surv[q + 4], uint32_t(q + 4)) : ~0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool same_row = q + j + 1 < n && (q + j + 1) % gamma != 0;
        const uint64_t next = (j < 3) ? v[j + 1] : nx;
        if (same_row && next < v[j]) in_order = false;
      }
      auto cs = [](uint64_t& a, uint64_t& b) {
        const uint64_t lo = a < b ? a : b, hi = a < b ? b : a;
        a = lo;
        b = hi;
      };
      cs(v[0], v[1]);
      cs(v[2], v[3]);
      cs(v[0], v[2]);
      cs(v[1], v[3]);
      cs(v[1], v[2]);
#pragma unroll
      for (int j = 0; j < 4; ++j) src[q + j] = v[j];
    }
    const bool rows_in_order = __syncthreads_and(in_order) != 0;
    int L0 = 4;
    if (rows_in_order && (gamma & (gamma - 1)) == 0 && gamma > 4) L0 = gamma < n2 ? gamma : n2;
    for (int L = L0; L < n2; L <<= 1) {
      __syncthreads();
      for (int o = tid * 4; o < n2; o += kSchedThreads * 4) {
        const int base = o & ~(2 * L - 1);
        const int d = o - base;
        const uint64_t* A = src + base;
        const uint64_t* Bv = src + base + L;
        // i = outputs before o that come from A: the first i with A[i] > B[d-1-i],
        // searched four ways at a time (three probes per round trip)
        int lo = d > L ? d - L : 0, hi = d < L ? d : L;
        while (hi - lo > 3) {
          const int step = (hi - lo) >> 2;
          const int m1 = lo + step, m2 = lo + 2 * step, m3 = lo + 3 * step;
          const bool g1 = A[m1] > Bv[d - 1 - m1];
          const bool g2 = A[m2] > Bv[d - 1 - m2];
          const bool g3 = A[m3] > Bv[d - 1 - m3];
          if (g1) {
            hi = m1;
          } else if (g2) {
            lo = m1 + 1;
            hi = m2;
          } else if (g3) {
            lo = m2 + 1;
            hi = m3;
          } else {
            lo = m3 + 1;
          }
        }
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (A[mid] > Bv[d - 1 - mid])
            hi = mid;
          else
            lo = mid + 1;
        }
        int i = lo, j = d - lo;
        // the next four candidates of each run in registers (past a run's
        // end: the largest key, never taken before a real one)
        uint64_t ra[4], rb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          ra[t] = (i + t < L) ? A[i + t] : ~0ull;
          rb[t] = (j + t < L) ? Bv[j + t] : ~0ull;
        }
        int ia = 0, ib = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint64_t ka = ra[0], kb = rb[0];
          const bool take_a = (j + ib >= L) || (i + ia < L && ka <= kb);
          dst[o + t] = take_a ? ka : kb;
          // shift the run that was taken
          if (take_a) {
            ra[0] = ra[1]; ra[1] = ra[2]; ra[2] = ra[3]; ra[3] = ~0ull;
            ++ia;
          } else {
            rb[0] = rb[1]; rb[1] = rb[2]; rb[2] = rb[3]; rb[3] = ~0ull;
            ++ib;
          }
        }
      }
      uint64_t* tmp = src;
      src = dst;
      dst = tmp;
    }
    sorted = src;
  } else {
    for (int i = tid; i < n2; i += kSchedThreads)
      keys[i] = (i < n) ? sched_key(surv[i], uint32_t(i)) : ~0ull;
    // bitonic sort, ascending
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        __syncthreads();
        for (int t = tid; t < (n2 >> 1); t += kSchedThreads) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = keys[lo], b = keys[hi];
          if ((a > b) == up) {
            keys[lo] = b;
            keys[hi] = a;
          }
        }
      }
    }
  }
  __syncthreads();

  // M ranges over 0..m_max; thread t scans positions [t*C, (t+1)*C).
  long long local = 0;
  for (int p = p0; p < p1; ++p) local += gain_fixed(sorted[p]);
  // block exclusive scan of the per-thread sums
  const long long incl = wave_scan_i64(local);
  if (lane == 63) wave_tot[wave] = incl;
  // the per-request counts of the last phase live in the free half of `keys`
  int* counts = reinterpret_cast<int*>(keys + (sorted == keys ? kMaxScheduleItems / 2 : 0));
  if (merged)
    for (int b = tid; b < B; b += kSchedThreads) counts[b] = 0;
  __syncthreads();
  long long before = 0;
#pragma unroll
  for (int w = 0; w < kSchedWaves; ++w)
    if (w < wave) before += wave_tot[w];
  long long G = before + incl - local;   // sum of gains at positions < p0

  const long long base = (long long)B << 32;
  double best = -INFINITY;
  int best_m = 0x7FFFFFFF;
  if (tid == 0) {
    best = double(base) / t0;
    best_m = 0;
  }
  for (int p = p0; p < p1; ++p) {
    G += gain_fixed(sorted[p]);
    const int M = p + 1;
    const int k = p - p0;
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < kPrefetchSteps; ++j)
      if (k == j) t = ts[j];
    if (k >= kPrefetchSteps) t = t_step[B + M - n_min];
    const double phi = double(base + G) / t;
    if (phi > best) {
      best = phi;
      best_m = M;
    }
  }
  // block arg-max: larger phi, then smaller M (a total order, M being distinct)
  wave_argmax_to_lane63(best, best_m);
  if (lane == 63) {
    red_phi[wave] = best;
    red_m[wave] = best_m;
  }
  __syncthreads();
  if (wave == 0) {
    double bb = red_phi[0];
    int bm = red_m[0];
#pragma unroll
    for (int w = 1; w < kSchedWaves; ++w) {
      const double ob = red_phi[w];
      const int om = red_m[w];
      if (ob > bb || (ob == bb && om < bm)) {
        bb = ob;
        bm = om;
      }
    }
    if (lane == 0) {
      s_mstar = bm;
      s_tau = (bm < n) ? sorted[bm] : ~0ull;
      m_out[0] = bm;
      if (objective) objective[0] = bb / 4294967296.0;
    }
  }
  __syncthreads();
  if (merged) {
    // lens[b] = how many of the first M* sorted keys belong to request b
    const int mstar = s_mstar;
    for (int p = tid; p < mstar; p += kSchedThreads) atomicAdd(&counts[uint32_t(sorted[p]) / uint32_t(gamma)], 1);
    __syncthreads();
    for (int b = tid; b < B; b += kSchedThreads) lens[b] = counts[b];
  } else {
    const uint64_t tau = s_tau;
    for (int b = tid; b < B; b += kSchedThreads) {
      int cnt = 0;
      for (int k = 0; k < gamma; ++k) {
        const int i = b * gamma + k;
        cnt += sched_key(surv[i], uint32_t(i)) < tau ? 1 : 0;
      }
      lens[b] = cnt;
    }
  }
}

template <int E, int K>
__global__ __launch_bounds__(kRankThreads) void schedule_rank_kernel(
    int B, int gamma, const float* __restrict__ surv, const double* __restrict__ t_step, int n_min, int n_count,
    int32_t* lens, int32_t* m_out, double* objective, unsigned int* tickets, RankEntry* sorted) {
  extern __shared__ unsigned int counters[];
  __shared__ int wcnt[K][kRankWaves];
  __shared__ long long wave_tot[kRankWaves];
  __shared__ double red_phi[kRankWaves];
  __shared__ int red_m[kRankWaves];
  __shared__ int flag;
  const RankShared<K> sh{wcnt, wave_tot, red_phi, red_m, &flag, counters};
  const int n = B * gamma;
  if (!rank_phase<E, K, false>(blockIdx.x, (n + K - 1) / K, B, gamma, surv, t_step, n_min, n_count, tickets, sorted,
                               sh))
    return;
  rank_tail<E, K>(B, gamma, t_step, n_min, n_count, tickets, sorted, lens, m_out, objective, sh);
}

// One workgroup: a thread per request (looping for B > 1024) scans its
// survivals until the first one below tau; M is a block sum of the lengths.
__global__ __launch_bounds__(kSchedThreads) void schedule_threshold_kernel(int B, int gamma,
                                                                         const float* __restrict__ surv, float tau,
                                                                         int32_t* lens, int32_t* m_out) {
  __shared__ int part[kSchedWaves];
  const int tid = threadIdx.x;
  int acc = 0;
  for (int b = tid; b < B; b += kSchedThreads) {
    const float* row = surv + size_t(b) * gamma;
    int l = 0;
    while (l < gamma && row[l] >= tau) ++l;
    lens[b] = l;
    acc += l;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < kSchedWaves; ++w) total += part[w];
    m_out[0] = total;
  }
}

// Verify with one lane per position: request b takes a segment of S lanes
// (S a power of two > gamma, S <= 64), lane k loads tokens[b][k] and
// target[b][k] together, so every load of the call is in flight at once;
// the accepted length is the first flagged lane of the segment's ballot
// (k >= lens[b] or a mismatch, and k = gamma always), and the bonus token is
// the target word that lane already holds.
template <int S>
__global__ __launch_bounds__(256) void verify_lanes_kernel(int B, int gamma, const int32_t* __restrict__ tokens,
                                                           const int32_t* __restrict__ target,
                                                           const int32_t* __restrict__ lens, int32_t* accepted,
                                                           int32_t* bonus) {
  const int gl = blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int b = gl / S, k = gl % S;
  const bool live = b < B && k <= gamma;
  int32_t tg = 0, tk = 0, L = 0;
  if (live) {
    tg = target[size_t(b) * (gamma + 1) + k];
    if (k < gamma) tk = tokens[size_t(b) * gamma + k];
    L = min(max(int(lens[b]), 0), gamma);
  }
  const bool stop = live && (k >= L || tk != tg);
  const uint64_t m = __ballot(stop);
  const int seg = lane & ~(S - 1);
  const uint64_t mine = (S == 64) ? m : (m >> seg) & ((1ull << S) - 1);
  const int a = __builtin_ctzll(mine | (1ull << (S - 1)));   // k = gamma always stops, so a <= gamma for live b
  const int32_t bon = __shfl(tg, seg + a, 64);
  if (live && k == 0) {
    accepted[b] = a;
    bonus[b] = bon;
  }
}

__global__ __launch_bounds__(256) void verify_kernel(int B, int gamma, const int32_t* __restrict__ tokens,
                                                     const int32_t* __restrict__ target,
                                                     const int32_t* __restrict__ lens, int32_t* accepted,
                                                     int32_t* bonus) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int L = min(max(int(lens[b]), 0), gamma);
  const int32_t* tk = tokens + size_t(b) * gamma;
  const int32_t* tg = target + size_t(b) * (gamma + 1);
  int a = 0;
  while (a < L && tk[a] == tg[a]) ++a;
  accepted[b] = a;
  bonus[b] = tg[a];
}

}  // namespace

size_t schedule_workspace_bytes(int B, int gamma) {
  const size_t n = size_t(B) * size_t(gamma);
  if (n == 0 || n > size_t(kMaxScheduleItems)) return 0;
  const size_t q = (n + kRankThreads - 1) / kRankThreads;   // the transposed array: q rows of kRankThreads
  return kRankHeader + q * kRankThreads * sizeof(RankEntry);
}

hipError_t launch_schedule(int B, int gamma, const float* surv, const double* t_step, int n_min, int n_count,
                           int32_t* lens, int32_t* m_out, double* objective, void* workspace, hipStream_t stream) {
  const int n = B * gamma;
  if (!workspace || n == 0) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, B, gamma, surv, t_step, n_min,
                       n_count, lens, m_out, objective);
    return hipGetLastError();
  }
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  auto* tickets = reinterpret_cast<unsigned int*>(ws);
  auto* sorted = reinterpret_cast<RankEntry*>(ws + kRankHeader);
  const size_t lds = sizeof(unsigned int) * size_t(rank_counter_words(B, gamma));
  const int per = (n + kRankThreads - 1) / kRankThreads;   // keys per thread
  // keys ranked per workgroup grow with n: fewer workgroups re-reading all n
  // keys, at the price of a longer compare loop
#define DSPARK_RANK_LAUNCH(E, K)                                                                              \
  hipLaunchKernelGGL((schedule_rank_kernel<E, K>), dim3((n + K - 1) / K), dim3(kRankThreads), lds, stream, B, \
                     gamma, surv, t_step, n_min, n_count, lens, m_out, objective, tickets, sorted)
  if (per <= 1)
    DSPARK_RANK_LAUNCH(1, 16);
  else if (per <= 2)
    DSPARK_RANK_LAUNCH(2, 16);
  else if (per <= 4)
    DSPARK_RANK_LAUNCH(4, 16);
  else if (per <= 8)
    DSPARK_RANK_LAUNCH(8, 16);
  else if (per <= 16)
    DSPARK_RANK_LAUNCH(16, 16);
  else
    DSPARK_RANK_LAUNCH(32, 64);
#undef DSPARK_RANK_LAUNCH
  return hipGetLastError();
}

hipError_t launch_schedule_threshold(int B, int gamma, const float* surv, float tau, int32_t* lens, int32_t* m_out,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(schedule_threshold_kernel, dim3(1), dim3(kSchedThreads), 0, stream, B, gamma, surv, tau, lens,
                     m_out);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int gamma, const int32_t* tokens, const int32_t* target, const int32_t* lens,
                         int32_t* accepted, int32_t* bonus, hipStream_t stream) {
  // lanes per request: the smallest power of two above gamma, up to a wave
  int S = 4;
  while (S <= gamma && S < 64) S <<= 1;
  if (gamma >= 64 || size_t(B) * S > size_t(0x7FFFFFFF)) {
    hipLaunchKernelGGL(verify_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, gamma, tokens, target, lens,
                       accepted, bonus);
    return hipGetLastError();
  }
  const dim3 grid(unsigned((size_t(B) * S + 255) / 256)), block(256);
  switch (S) {
    case 4:
      hipLaunchKernelGGL(verify_lanes_kernel<4>, grid, block, 0, stream, B, gamma, tokens, target, lens, accepted,
                         bonus);
      break;
    case 8:
      hipLaunchKernelGGL(verify_lanes_kernel<8>, grid, block, 0, stream, B, gamma, tokens, target, lens, accepted,
                         bonus);
      break;
    case 16:
      hipLaunchKernelGGL(verify_lanes_kernel<16>, grid, block, 0, stream, B, gamma, tokens, target, lens, accepted,
                         bonus);
      break;
    case 32:
      hipLaunchKernelGGL(verify_lanes_kernel<32>, grid, block, 0, stream, B, gamma, tokens, target, lens, accepted,
                         bonus);
      break;
    default:
      hipLaunchKernelGGL(verify_lanes_kernel<64>, grid, block, 0, stream, B, gamma, tokens, target, lens, accepted,
                         bonus);
      break;
  }
  return hipGetLastError();
}

}  // namespace dspark
