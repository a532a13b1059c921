// Fitting the sequential temperatures of the confidence head: for each draft
// position k = 1..gamma in order, a grid search over candidate temperatures
// for the one whose cumulative-product confidence has the smallest expected
// calibration error against the observed prefix acceptance, the positions
// before k held at their fitted temperatures ("DSpark: DeepSeek's new
// speculative decoding work", §5 "Sequential Temperature Scaling").
//
// One launch per position.  A launch splits the calibration blocks into
// chunks, one workgroup per compute unit; within a workgroup every lane owns
// one candidate temperature, so all 64 lanes of a wave read the same staged
// block (an LDS broadcast) and update different histogram entries.  For block
// n and candidate g:
//     p = S_{n,k-1} * sigmoid(logit[n][k-1] / T_g)          (fp64)
//     bin = min(floor(p * nbins), nbins - 1)
//     hist[bin][g] += rint((y_n - p) * 2^32)                 (exact int64)
// with y_n = (accepted[n] >= k).  The workgroup's histogram lives in LDS and
// is added to the device histogram with 64-bit atomics; the last workgroup to
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

constexpr int kStsThreads = 1024;   // threads per workgroup = blocks staged per round

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

// sigmoid(l / T) with l / T taken as l * (1 / T), in the order the fit uses
// everywhere (no contraction, so the prefix product carried to the next
// position equals the value scored here).
__device__ __forceinline__ double sigmoid_scaled(double l, double inv_t) {
#pragma clang fp contract(off)
  const double x = l * inv_t;
  return 1.0 / (1.0 + exp(-x));
}

// rint(v) as an int64 for |v| < 2^51: adding 1.5 * 2^52 leaves the integer
// nearest to v (ties to even, the default rounding) in the low mantissa bits.
__device__ __forceinline__ long long rint_to_i64(double v) {
#pragma clang fp contract(off)
  constexpr double kMagic = 6755399441055744.0;   // 1.5 * 2^52
  return __double_as_longlong(v + kMagic) - __double_as_longlong(kMagic);
}

// Histogram bytes rounded up to 16 (the staged pairs that follow are 16-byte loads).
__host__ __device__ constexpr size_t sts_hist_lds_bytes(int nh) { return (size_t(nh) * 8 + 15) & ~size_t(15); }

__global__ void __launch_bounds__(kStsThreads) sts_clear_kernel(unsigned int* done, unsigned long long* hist,
                                                                 int nh) {
  for (int i = threadIdx.x; i < nh; i += kStsThreads) hist[i] = 0ull;
  if (threadIdx.x == 0) *done = 0u;
}

__global__ void __launch_bounds__(kStsThreads) sts_pass_kernel(StsParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int G = p.G, nbins = p.nbins, k = p.k;
  const int nh = nbins * G;
  unsigned long long* h = reinterpret_cast<unsigned long long*>(smem);             // [nbins][G]
  double2* stage_ls = reinterpret_cast<double2*>(smem + sts_hist_lds_bytes(nh));  // {logit, S_{k-1}}
  double* stage_y = reinterpret_cast<double*>(stage_ls + kStsThreads);            // label
  __shared__ int last;
  __shared__ long long best_e[kStsThreads];
  __shared__ int best_g[kStsThreads];

  for (int i = tid; i < nh; i += kStsThreads) h[i] = 0ull;

  // temperature fitted at the previous position (applied while staging)
  double inv_prev = 0.0;
  if (k >= 2) inv_prev = 1.0 / double(p.grid[p.choice[k - 2]]);

  // candidate(s) of this thread: g = tid % G for G <= kStsThreads (tid / G
  // picks which of the staged blocks it scores), else g = tid, tid + 1024, ...
  const int nsub = G <= kStsThreads ? kStsThreads / G : 1;
  const int sub = G <= kStsThreads ? tid / G : 0;
  const bool active = sub < nsub;

  const int nchunks = (p.N + kStsThreads - 1) / kStsThreads;
  for (int c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int n0 = c * kStsThreads;
    const int cnt = min(kStsThreads, p.N - n0);
    __syncthreads();   // the previous chunk's readers are done with the stage
    if (tid < cnt) {
      const int n = n0 + tid;
      const size_t row = size_t(n) * size_t(p.gamma);
      double s = 1.0;
      if (k >= 2) {
        const double s_prev = k >= 3 ? p.S[n] : 1.0;
        s = s_prev * sigmoid_scaled(double(p.logit[row + k - 2]), inv_prev);
        p.S[n] = s;
      }
      stage_ls[tid] = make_double2(double(p.logit[row + k - 1]), s);
      stage_y[tid] = p.accepted[n] >= k ? 1.0 : 0.0;
    }
    __syncthreads();
    if (!active) continue;
    for (int g = G <= kStsThreads ? tid % G : tid; g < G; g += kStsThreads) {
      const double inv_t = 1.0 / double(p.grid[g]);
      for (int j = sub; j < cnt; j += nsub) {
        const double2 ls = stage_ls[j];
        double pr, res;
        {
#pragma clang fp contract(off)
          pr = ls.y * sigmoid_scaled(ls.x, inv_t);
          res = (stage_y[j] - pr) * 4294967296.0;
        }
        unsigned int b = static_cast<unsigned int>(pr * double(nbins));   // pr >= 0; NaN -> 0
        b = min(b, unsigned(nbins - 1));
        atomicAdd(&h[b * unsigned(G) + unsigned(g)], static_cast<unsigned long long>(rint_to_i64(res)));
      }
    }
  }
  __syncthreads();

  // add this workgroup's histogram to the device one, then arrive
  for (int i = tid; i < nh; i += kStsThreads) {
    const unsigned long long v = h[i];
    if (v != 0ull) __hip_atomic_fetch_add(&p.hist[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
  for (int g = tid; g < G; g += kStsThreads) {
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
  for (int i = tid; i < nh; i += kStsThreads) store_dev(&p.hist[i], 0ull);
  if (tid == 0) {
    long long e = -1;
    int g = 0;
    for (int t = 0; t < kStsThreads && t < G; ++t) {
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
  const int nchunks = (a.N + kStsThreads - 1) / kStsThreads;
  const int nwg = std::max(1, std::min(nchunks, std::max(cus, 1)));
  const size_t lds = sts_lds_bytes(a.G, a.nbins);
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
