// Fitting the sequential temperatures of the confidence head: for each draft
// position k = 1..gamma in order, a grid search over candidate temperatures
// for the one whose cumulative-product confidence has the smallest expected
// calibration error against the observed prefix acceptance, the positions
// before k held at their fitted temperatures ("DSpark: DeepSeek's new
// speculative decoding work", §5 "Sequential Temperature Scaling").
//
// One launch per position.  A launch splits the calibration blocks into
// rounds of staged blocks, several workgroups per compute unit; within a
// workgroup the lanes of a wave hold different candidate temperatures and
// read the same staged block (an LDS broadcast).  For block n and candidate g:
//     p = S_{n,k-1} * sigmoid(logit[n][k-1] / T_g)          (fp64)
//     bin = min(floor(p * nbins), nbins - 1)
//     hist[bin][g] += rint((y_n - p) * 2^32)                 (exact int64)
// with y_n = (accepted[n] >= k).  The workgroup keeps one LDS column of bins
// per candidate and adds to it with 64-bit LDS atomics (for G >= 128 the 64
// lanes of a wave hold 64 different candidates); workgroup histograms are
// added to the device histogram with 64-bit atomics; the last workgroup to
// arrive turns the device histogram into ECE_g = sum_bin |hist| / (2^32 N),
// picks the first g with the smallest integer sum, and clears the histogram
// and the arrival counter for the next launch (a small kernel clears them
// before the first one, so the workspace may hold anything on entry).  The
// prefix products S_{n,k} are carried in the workspace: the launch for
// position k+1 applies the temperature chosen at k while it stages the blocks.
//
// The integer sums make the choice independent of the order in which lanes
// and workgroups add: the same inputs always give the same temperatures.
#include "device_util.h"
#include "launch.h"

namespace dspark {
namespace {

struct StsParams {
  const float* logit;          // [N][gamma] raw confidence logits
  const int32_t* accepted;     // [N] accepted drafts per block
  const float* grid;           // [G] candidate temperatures
  int N, gamma, G, nbins;
  int k;                       // position fitted by this launch (1-based)
  int32_t* choice;             // [gamma] out: grid index of T_k
  float* T_out;                // [gamma] out: T_k
  double* ece;                 // [gamma][G] out
  unsigned int* done;          // workgroups that have added their histogram
  unsigned long long* hist;    // [nbins][G] two's-complement int64 sums
  double* S;                   // [N] prefix products of the fitted positions
};

constexpr double kMagic = 6755399441055744.0;   // 1.5 * 2^52: x + kMagic rounds x to an integer

// q * r + c with the coefficient c in scalar registers: a three-operand fma
// that leaves every vector register of the chain in place (the compiler
// otherwise copies the coefficient into the accumulator of a two-operand fma).
__device__ __forceinline__ double horner_step(double q, double r, double c) {
  double out;
  asm("v_fma_f64 %0, %1, %2, %3" : "=v"(out) : "v"(q), "v"(r), "s"(c));
  return out;
}

// e^x for x in [-745, 708] (the caller clamps), about 2 ulp.  x = n ln2 + r
// with n = rint(x / ln2), read from the low word of x log2(e) + 1.5 * 2^52,
// and r = x - n ln2 in two steps (ln2 split into a 32-bit head, so n times
// the head is exact, and a tail); |r| <= ln2 / 2, where the Taylor series of
// e^r to degree 13 is within 2^-54 relative; the result is scaled by 2^n.
__device__ __forceinline__ double exp_clamped(double x) {
  constexpr double kLog2e = 1.4426950408889634;
  constexpr double kLn2Hi = 6.93147180369123816490e-01;   // 0x3FE62E42FEE00000
  constexpr double kLn2Lo = 1.90821492927058770002e-10;   // ln2 - kLn2Hi
  const double t = __builtin_fma(x, kLog2e, kMagic);
  const int n = static_cast<int>(static_cast<uint32_t>(__double_as_longlong(t)));
  const double nf = t - kMagic;
  double r = __builtin_fma(-nf, kLn2Hi, x);
  r = __builtin_fma(-nf, kLn2Lo, r);
  double q = horner_step(1.0 / 6227020800.0, r, 1.0 / 479001600.0);   // 1/13!, 1/12!
  q = horner_step(q, r, 1.0 / 39916800.0);
  q = horner_step(q, r, 1.0 / 3628800.0);
  q = horner_step(q, r, 1.0 / 362880.0);
  q = horner_step(q, r, 1.0 / 40320.0);
  q = horner_step(q, r, 1.0 / 5040.0);
  q = horner_step(q, r, 1.0 / 720.0);
  q = horner_step(q, r, 1.0 / 120.0);
  q = horner_step(q, r, 1.0 / 24.0);
  q = horner_step(q, r, 1.0 / 6.0);
  q = __builtin_fma(q, r, 0.5);
  q = __builtin_fma(q, r, 1.0);
  q = __builtin_fma(q, r, 1.0);
  return ldexp(q, n);
}

// sigmoid(l / T) = 1 / (1 + e^{l * (-1/T)}), the argument clamped to the range
// where e^x is finite (1 + e^x then stays finite; beyond it the sigmoid is 0
// or 1 to within 1e-300).  The reciprocal is the hardware estimate refined by
// two Newton steps.  Scoring and the prefix product carried to the next
// position both come from here, so they agree bit for bit.
__device__ __forceinline__ double sigmoid_scaled(double l, double neg_inv_t) {
  const double x = fmin(fmax(l * neg_inv_t, -745.0), 708.0);
  const double a = 1.0 + exp_clamped(x);
  double r = __builtin_amdgcn_rcp(a);
  r = __builtin_fma(r, __builtin_fma(-a, r, 1.0), r);
  r = __builtin_fma(r, __builtin_fma(-a, r, 1.0), r);
  return r;
}

// One candidate's contribution for one staged block: the bin of
// p = S * sigmoid(l / T) and rint((y - p) * 2^32).  p and y - p are rounded
// separately (no contraction); the product by 2^32 is exact, so
// fma(y - p, 2^32, 1.5 * 2^52) rounds once, to the nearest integer (ties to
// even), which sits in the low mantissa bits.
struct Scored {
  unsigned int bin;
  unsigned long long q;   // two's-complement int64
};
__device__ __forceinline__ Scored score(double l, double S, double y, double neg_inv_t, int nbins) {
#pragma clang fp contract(off)
  const double pr = S * sigmoid_scaled(l, neg_inv_t);
  const double biased = __builtin_fma(y - pr, 4294967296.0, kMagic);
  Scored r;
  r.q = static_cast<unsigned long long>(__double_as_longlong(biased) - __double_as_longlong(kMagic));
  const unsigned int b = static_cast<unsigned int>(pr * double(nbins));   // pr >= 0; NaN -> 0
  r.bin = min(b, unsigned(nbins - 1));
  return r;
}

// Histogram bytes rounded up to 16 (the staged pairs that follow are 16-byte loads).
__host__ __device__ constexpr size_t sts_hist_lds_bytes(int nh) { return (size_t(nh) * 8 + 15) & ~size_t(15); }

constexpr int kStsThreads = 1024;   // threads per workgroup = blocks staged per round

__global__ void __launch_bounds__(kStsThreads) sts_clear_kernel(unsigned int* done, unsigned long long* hist,
                                                                 int nh) {
  for (int i = threadIdx.x; i < nh; i += kStsThreads) hist[i] = 0ull;
  if (threadIdx.x == 0) *done = 0u;
}

__device__ __forceinline__ void add_dev(unsigned long long* p, unsigned long long v) {
  if (v != 0ull) __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(kStsThreads) sts_pass_kernel(StsParams p) {
  constexpr int T = kStsThreads;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int G = p.G, nbins = p.nbins, k = p.k;
  const int nh = nbins * G;
  // LDS: histogram [nbins][G], then the round's blocks {logit, S_{k-1}} and labels
  unsigned long long* h = reinterpret_cast<unsigned long long*>(smem);
  double2* stage_ls = reinterpret_cast<double2*>(smem + sts_hist_lds_bytes(nh));
  double* stage_y = reinterpret_cast<double*>(stage_ls + T);
  __shared__ int last;
  __shared__ long long best_e[T];
  __shared__ int best_g[T];

  for (int i = tid; i < nh; i += T) h[i] = 0ull;

  // temperature fitted at the previous position (applied while staging)
  double ninv_prev = 0.0;
  if (k >= 2) ninv_prev = -1.0 / double(p.grid[p.choice[k - 2]]);

  // A thread scores two candidates, g and g + slots, of one slot; slot =
  // tid % slots when slots <= T (tid / slots picks which staged blocks),
  // else slots tid, tid + T, ...
  const int slots = (G + 1) / 2;
  const bool resident = slots <= T;
  const int nsub = resident ? T / slots : 1;
  const int sub = resident ? tid / slots : 0;
  const bool active = sub < nsub;
  const unsigned int row_bytes = unsigned(G) * 8u;   // < 2^24: a 24-bit multiply addresses a bin row

  const int nchunks = (p.N + T - 1) / T;
  for (int c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int n0 = c * T;
    const int cnt = min(T, p.N - n0);
    __syncthreads();   // the previous round's readers are done with the stage
    if (tid < cnt) {
      const int n = n0 + tid;
      const size_t row = size_t(n) * size_t(p.gamma);
      double sv = 1.0;
      if (k >= 2) {
        const double s_prev = k >= 3 ? p.S[n] : 1.0;
        sv = s_prev * sigmoid_scaled(double(p.logit[row + k - 2]), ninv_prev);
        p.S[n] = sv;
      }
      stage_ls[tid] = make_double2(double(p.logit[row + k - 1]), sv);
      stage_y[tid] = p.accepted[n] >= k ? 1.0 : 0.0;
    }
    __syncthreads();
    if (!active) continue;
    for (int sl = resident ? tid % slots : tid; sl < slots; sl += T) {
      const int g1 = sl + slots;
      const bool two = g1 < G;
      const double ninv0 = -1.0 / double(p.grid[sl]);
      const double ninv1 = two ? -1.0 / double(p.grid[g1]) : ninv0;
      unsigned char* h0 = reinterpret_cast<unsigned char*>(h + sl);
      unsigned char* h1 = reinterpret_cast<unsigned char*>(h + g1);
      for (int j = sub; j < cnt; j += nsub) {
        const double2 ls = stage_ls[j];
        const double y = stage_y[j];
        const Scored s0 = score(ls.x, ls.y, y, ninv0, nbins);
        atomicAdd(reinterpret_cast<unsigned long long*>(h0 + __umul24(s0.bin, row_bytes)), s0.q);
        if (two) {
          const Scored s1 = score(ls.x, ls.y, y, ninv1, nbins);
          atomicAdd(reinterpret_cast<unsigned long long*>(h1 + __umul24(s1.bin, row_bytes)), s1.q);
        }
      }
    }
  }
  __syncthreads();

  // add this workgroup's histogram to the device one, then arrive
  for (int i = tid; i < nh; i += T) add_dev(&p.hist[i], h[i]);
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const unsigned int prior = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prior == gridDim.x - 1u ? 1 : 0;
  }
  __syncthreads();
  if (!last) return;

  // last workgroup: every other one has added its histogram (each waited for
  // its atomics before arriving); device-scope loads see the totals.
  long long my_e = -1;
  int my_g = 0;
  const double denom = 4294967296.0 * double(p.N);
  for (int g = tid; g < G; g += T) {
    long long e = 0;
    for (int m = 0; m < nbins; ++m) {
      const long long v = static_cast<long long>(load_dev(&p.hist[size_t(m) * G + g]));
      e += v < 0 ? -v : v;
    }
    p.ece[size_t(k - 1) * G + g] = p.N > 0 ? double(e) / denom : 0.0;
    if (my_e < 0 || e < my_e) {   // g increases: strict < keeps the first
      my_e = e;
      my_g = g;
    }
  }
  best_e[tid] = my_e;
  best_g[tid] = my_g;
  __syncthreads();
  for (int i = tid; i < nh; i += T) store_dev(&p.hist[i], 0ull);
  if (tid == 0) {
    long long e = -1;
    int g = 0;
    for (int t = 0; t < T && t < G; ++t) {
      if (best_e[t] < 0) continue;
      if (e < 0 || best_e[t] < e || (best_e[t] == e && best_g[t] < g)) {
        e = best_e[t];
        g = best_g[t];
      }
    }
    p.choice[k - 1] = g;
    p.T_out[k - 1] = p.grid[g];
    store_dev(p.done, 0u);
  }
}

}  // namespace

StsWorkspace sts_workspace_layout(int N, int G, int nbins) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  StsWorkspace L;
  L.ctrl = 0;
  L.hist = 256;
  L.S = L.hist + up(size_t(nbins) * size_t(G) * 8);
  L.total = L.S + up(size_t(N > 0 ? N : 0) * 8);
  return L;
}

size_t sts_lds_bytes(int G, int nbins) {
  return sts_hist_lds_bytes(nbins * G) + size_t(kStsThreads) * (sizeof(double) * 3);
}

hipError_t launch_sts_fit(const StsArgs& a, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const StsWorkspace L = sts_workspace_layout(a.N, a.G, a.nbins);
  unsigned char* ws = static_cast<unsigned char*>(a.ws);
  StsParams p;
  p.logit = a.logit;
  p.accepted = a.accepted;
  p.grid = a.grid;
  p.N = a.N;
  p.gamma = a.gamma;
  p.G = a.G;
  p.nbins = a.nbins;
  p.choice = a.choice;
  p.T_out = a.T_out;
  p.ece = a.ece;
  p.done = reinterpret_cast<unsigned int*>(ws + L.ctrl);
  p.hist = reinterpret_cast<unsigned long long*>(ws + L.hist);
  p.S = reinterpret_cast<double*>(ws + L.S);
  const size_t lds = sts_lds_bytes(a.G, a.nbins);
  int per_cu = 1;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&sts_pass_kernel),
                                                   kStsThreads, lds);
  if (e != hipSuccess) return e;
  const int nchunks = (a.N + kStsThreads - 1) / kStsThreads;
  const int nwg = std::max(1, std::min(nchunks, std::max(cus, 1) * std::max(per_cu, 1)));
  hipLaunchKernelGGL(sts_clear_kernel, dim3(1), dim3(kStsThreads), 0, stream, p.done, p.hist, a.G * a.nbins);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int k = 1; k <= a.gamma; ++k) {
    p.k = k;
    hipLaunchKernelGGL(sts_pass_kernel, dim3(nwg), dim3(kStsThreads), lds, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
