// Hardware-aware prefix scheduler and prefix-match verify for gfx950.
//
// Scheduler ("DSpark: Overcoming the Efficiency Wall in LLM Speculative
// Decoding", "2. The Hardware-Aware Prefix Scheduler"; "DSpark: DeepSeek's
// new speculative decoding work", §6): choose per-request verify lengths
// maximising (B + sum of scheduled survivals) / t_step(B + M).  Survival is
// non-increasing along each request, so the best set of M drafts is the top
// M by (S desc, request asc, position asc) and only M has to be searched.
// One workgroup of 1024 threads: merge sort (bitonic above 8192 items) of
// 64-bit keys in LDS, a block scan of fixed-point gains, one fp64 division per candidate M, a
// block arg-max, and a per-request count below the M*-th key.
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

namespace dspark {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / 64;

// Sort key: ascending key order = descending survival, then ascending flat
// index (request-major), so the first M keys are the scheduler's top M.
__device__ __forceinline__ uint64_t sched_key(float s, uint32_t flat) {
  return (uint64_t(~ord_f32(s)) << 32) | uint64_t(flat);
}
__device__ __forceinline__ long long gain_fixed(uint64_t key) {
  const float s = unord_f32(~uint32_t(key >> 32));
  return (long long)rint(double(s) * 4294967296.0);
}

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

  // Sort the keys ascending.  Up to half the key array, a merge sort: runs
  // of 4 sorted in registers, then merge levels that ping-pong between the
  // two halves of `keys`, each thread placing 4 outputs after a binary
  // search for where its output range splits the two input runs (merge
  // path).  Every level reads and writes the keys once; the bitonic network
  // used for larger inputs passes over them once per stage.  Keys are
  // distinct apart from the padding, so the order is the same either way.
  const uint64_t* sorted = keys;
  if (n2 <= kMaxScheduleItems / 2) {
    uint64_t* src = keys;
    uint64_t* dst = keys + kMaxScheduleItems / 2;
    for (int q = tid * 4; q < n2; q += kSchedThreads * 4) {
      uint64_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (q + j < n) ? sched_key(surv[q + j], uint32_t(q + j)) : ~0ull;
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
    for (int L = 4; L < n2; L <<= 1) {
      __syncthreads();
      for (int o = tid * 4; o < n2; o += kSchedThreads * 4) {
        const int base = o & ~(2 * L - 1);
        const int d = o - base;
        const uint64_t* A = src + base;
        const uint64_t* Bv = src + base + L;
        // i = outputs before o that come from A: the first i with A[i] > B[d-1-i]
        int lo = d > L ? d - L : 0, hi = d < L ? d : L;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (A[mid] > Bv[d - 1 - mid])
            hi = mid;
          else
            lo = mid + 1;
        }
        int i = lo, j = d - lo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool take_a = j >= L || (i < L && A[i] <= Bv[j]);
          dst[o + t] = take_a ? A[i++] : Bv[j++];
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
  const int m_max = min(n, n_min + n_count - 1 - B);
  const int C = (m_max + kSchedThreads - 1) / kSchedThreads;
  const int p0 = min(tid * C, m_max), p1 = min(p0 + C, m_max);
  long long local = 0;
  for (int p = p0; p < p1; ++p) local += gain_fixed(sorted[p]);
  // block exclusive scan of the per-thread sums
  long long incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  long long G = before + incl - local;   // sum of gains at positions < p0

  const long long base = (long long)B << 32;
  double best = -INFINITY;
  int best_m = 0x7FFFFFFF;
  if (tid == 0) {
    best = double(base) / t_step[B - n_min];
    best_m = 0;
  }
  for (int p = p0; p < p1; ++p) {
    G += gain_fixed(sorted[p]);
    const int M = p + 1;
    const double phi = double(base + G) / t_step[B + M - n_min];
    if (phi > best) {
      best = phi;
      best_m = M;
    }
  }
  // block arg-max: larger phi, then smaller M
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double ob = __shfl_xor(best, m, 64);
    const int om = __shfl_xor(best_m, m, 64);
    if (ob > best || (ob == best && om < best_m)) {
      best = ob;
      best_m = om;
    }
  }
  if (lane == 0) {
    red_phi[wave] = best;
    red_m[wave] = best_m;
  }
  __syncthreads();
  if (tid == 0) {
    double bb = red_phi[0];
    int bm = red_m[0];
    for (int w = 1; w < kSchedWaves; ++w)
      if (red_phi[w] > bb || (red_phi[w] == bb && red_m[w] < bm)) {
        bb = red_phi[w];
        bm = red_m[w];
      }
    s_mstar = bm;
    s_tau = (bm < n) ? sorted[bm] : ~0ull;
    m_out[0] = bm;
    if (objective) objective[0] = bb / 4294967296.0;
  }
  __syncthreads();
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

hipError_t launch_schedule(int B, int gamma, const float* surv, const double* t_step, int n_min, int n_count,
                           int32_t* lens, int32_t* m_out, double* objective, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, B, gamma, surv, t_step, n_min,
                     n_count, lens, m_out, objective);
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
  hipLaunchKernelGGL(verify_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, B, gamma, tokens, target, lens,
                     accepted, bonus);
  return hipGetLastError();
}

}  // namespace dspark
