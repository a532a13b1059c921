// Markov-head drafting for gfx950: one persistent, cooperatively launched
// kernel runs all gamma dependent draft steps of a call.
//
// Method ("DSpark: DeepSeek's new speculative decoding work", §4 sequential
// stage and Markov head; §5 confidence head and Sequential Temperature
// Scaling): per request b and step k, e = W1[x_{k-1}], z_k = U_k + e W2,
// x_k = argmax z_k (or of z_k + Gumbel noise), c_k = sigmoid((w.[h_k; e] +
// b) / T_k), S_k = S_{k-1} c_k.
//
// Layout of the work on the chip:
//  * The vocabulary is cut into 16-wide tiles; every workgroup (one per
//    compute unit) owns a contiguous range of tiles and every wave a
//    contiguous sub-range of at most TPW tiles.  The wave loads its slice of
//    W2 once per call into registers, already in the A-operand layout of
//    v_mfma_f32_16x16x32_bf16 (rows = vocabulary ids, K = rank), so W2 is
//    read from memory once per call instead of once per step.
//  * Per step the gathered embeddings e (B rows of W1, selected by the
//    previous tokens) sit in LDS and feed the B operand (columns = requests).
//  * The accumulator is initialised with the base logits U_k, so the U add
//    is free; the argmax over the wave's tiles runs on the accumulator in
//    registers and z_k is never written to memory.
//  * Per-row winners are reduced across lanes (shuffles), waves (LDS 64-bit
//    atomic max) and workgroups (one device-scope 64-bit atomic max per row
//    and workgroup on a packed (value, ~index) key, which also makes the
//    lowest index win ties), followed by one grid barrier per step.
//  * The confidence epilogue of request b runs in workgroup b mod grid, off
//    the critical path; the hidden-state half of its dot product does not
//    depend on the drafted tokens and is precomputed by draft_init_kernel.
#include "device_util.h"
#include "launch.h"

namespace dspark {
namespace {

struct DraftParams {
  int B, gamma, V, d;
  int nwg, tiles, vec_ok;
  uint32_t seed_lo, seed_hi;
  unsigned int spin_limit;
  float conf_b;
  const int32_t* anchor;
  const void* U;
  const void* h;
  const void* W1;
  const void* W2;
  const float* conf_w;
  const float* sts_T;
  int32_t* tokens;
  float* logit;
  float* conf;
  float* surv;
  unsigned int* ctrl;  // [0] barrier arrivals, [1] error flag
  uint64_t* slots;     // [gamma][B] packed argmax keys
  float* zpart;        // [2][nwg][B] logit of each workgroup's local winner
  double* hdot;        // [B][gamma] hidden-state part of the confidence logit
};

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  typedef uint16_t store_t;
  typedef bf16x8_t frag_t;
  static constexpr int KS = 32;  // K per MFMA
  static constexpr int KPL = 8;  // K values per lane
  static constexpr int PAD = 8;  // LDS row padding (elements): conflict-free 16-byte reads
};
template <>
struct Elem<false> {
  typedef float store_t;
  typedef float frag_t;
  static constexpr int KS = 4;
  static constexpr int KPL = 1;
  static constexpr int PAD = 4;
};

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Raw storage of four consecutive base logits of one request.
template <bool BF16>
struct RawU;
template <>
struct RawU<true> {
  u32x2_t q;
};
template <>
struct RawU<false> {
  f32x4_t q;
};

__device__ __forceinline__ void load_u(RawU<true>& r, const uint16_t* row, int v0, int V, int vec_ok) {
  if (vec_ok) {
    r.q = (v0 < V) ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(row + v0)) : u32x2_t{0u, 0u};
  } else {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (v0 + i < V) ? uint32_t(row[v0 + i]) : 0u;
    r.q = u32x2_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }
}
__device__ __forceinline__ void load_u(RawU<false>& r, const float* row, int v0, int V, int vec_ok) {
  if (vec_ok) {
    r.q = (v0 < V) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(row + v0)) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = (v0 + i < V) ? row[v0 + i] : 0.f;
  }
}
__device__ __forceinline__ f32x4_t widen_u(const RawU<true>& r) {
  return f32x4_t{bf16_lo(r.q.x), bf16_hi(r.q.x), bf16_lo(r.q.y), bf16_hi(r.q.y)};
}
__device__ __forceinline__ f32x4_t widen_u(const RawU<false>& r) { return r.q; }

// Operand layout (v_mfma_f32_16x16x32_bf16 / _16x16x4f32): the A operand of
// a 16-row tile holds vocabulary ids tile*16 + (lane & 15); lane group
// (lane >> 4) holds K values ks*KS + KPL*(lane>>4) + 0..KPL-1.  The B operand
// read from LDS uses the same K assignment, so their product sums over
// exactly these K values whatever order the hardware uses inside a step.
__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ float lds_frag(const float* p) { return *p; }

// Start of part `i` when `n` items are split into `parts` contiguous parts.
__device__ __forceinline__ int part_start(int i, int n, int parts) {
  return int((long long)i * n / parts);
}
// Index of the part containing item t.
__device__ __forceinline__ int part_of(int t, int n, int parts) {
  int w = int((long long)t * parts / n);
  while (w + 1 < parts && part_start(w + 1, n, parts) <= t) ++w;
  while (w > 0 && part_start(w, n, parts) > t) --w;
  return w;
}

// Loads the base logits of request tile `bt` for this wave's vocabulary
// tiles: lane (li, lg) gets U[b][k-1][tile*16 + 4*lg .. +3] with
// b = g0 + 16*bt + li (clamped into the batch; such lanes are ignored).
template <bool BF16, int TPW>
__device__ __forceinline__ void load_tile(RawU<BF16> (&buf)[TPW], const typename Elem<BF16>::store_t* U, int g0,
                                          int bt, int li, int lg, int B, int gamma, int k, int V, int w_lo, int nt,
                                          int vec_ok) {
  const int b = min(g0 + bt * 16 + li, B - 1);
  const typename Elem<BF16>::store_t* urow = U + (size_t(b) * gamma + (k - 1)) * V;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if (t < nt) load_u(buf[t], urow, (w_lo + t) * 16 + 4 * lg, V, vec_ok);
}

// Zeroes the barrier counter, the error flag and the argmax slots, and
// precomputes hdot[b][k] = sum_j conf_w[j] h[b][k][j] in fp64 (one wave per
// (b, k)); this half of the confidence logit does not depend on the tokens.
template <bool BF16>
__global__ __launch_bounds__(256) void draft_init_kernel(DraftParams p) {
  typedef typename Elem<BF16>::store_t st_t;
  const int gtid = blockIdx.x * 256 + threadIdx.x;
  const int nthreads = gridDim.x * 256;
  const long long nslots = (long long)p.gamma * p.B;
  for (long long i = gtid; i < nslots; i += nthreads) p.slots[i] = 0ull;
  if (gtid < 2) p.ctrl[gtid] = 0u;
  const int lane = threadIdx.x & 63;
  const int nwaves = nthreads >> 6;
  const st_t* h = static_cast<const st_t*>(p.h);
  for (int bk = gtid >> 6; bk < p.B * p.gamma; bk += nwaves) {
    const st_t* row = h + size_t(bk) * p.d;
    double acc = 0.0;
    for (int j = lane; j < p.d; j += 64) acc += double(p.conf_w[j]) * double(to_f32(row[j]));
    acc = wave_sum_f64(acc);
    if (lane == 0) p.hdot[bk] = acc;
  }
}

template <bool BF16, int R, int NW, int TPW, int GR, bool GUMBEL>
__global__ __launch_bounds__(NW * 64, 1) void markov_draft_kernel(DraftParams p) {
  typedef Elem<BF16> E;
  typedef typename E::store_t st_t;
  typedef typename E::frag_t frag_t;
  constexpr int NKS = R / E::KS;
  constexpr int LDE = R + E::PAD;
  constexpr int NT = NW * 64;
  constexpr int CHUNKS = int(R * sizeof(st_t)) / 16;      // 16-byte pieces per W1 row
  static_assert(R % E::KS == 0, "rank must be a multiple of the MFMA K step");

  constexpr int CMAX = TPW * NW * 16;                       // widest column slice of a workgroup
  constexpr int SLD = CMAX + (BF16 ? 2 : 1);                // W2 staging row stride (elements)
  constexpr int EBUF = (GR * LDE > E::KS * SLD) ? GR * LDE : E::KS * SLD;
  __shared__ __attribute__((aligned(16))) st_t lds_e[EBUF];
  __shared__ uint64_t lds_key[GR];
  __shared__ float lds_z[NW][GR];
  __shared__ int lds_x[GR];
  __shared__ double lds_hd[GR];
  __shared__ float lds_S[kMaxOwnedRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15;   // request column of the MFMA tile / row of A
  const int lg = lane >> 4;   // lane group: K slice of the operands, 4-row slice of D
  const int wg = blockIdx.x;
  const int B = p.B, V = p.V, gamma = p.gamma, nwg = p.nwg;

  const int wg_lo = part_start(wg, p.tiles, nwg);
  const int wg_nt = part_start(wg + 1, p.tiles, nwg) - wg_lo;
  const int w_lo = wg_lo + part_start(wave, wg_nt, NW);
  const int nt = wg_lo + part_start(wave + 1, wg_nt, NW) - w_lo;   // <= TPW

  // W2 slice of this wave in MFMA A-operand layout, resident for the call.
  // The workgroup's columns [wg_lo*16, wg_hi*16) of W2 are staged through
  // LDS (the embedding buffer is still free) a chunk of K rows at a time with
  // coalesced row loads; each wave then picks its fragments out of LDS.
  frag_t A[TPW][NKS];
  {
    constexpr int KCH0 = int(sizeof(lds_e) / (SLD * sizeof(st_t)));
    constexpr int KCH = (KCH0 >= R) ? R : (KCH0 / E::KS) * E::KS;   // K rows per chunk
    static_assert(KCH >= E::KS, "staging buffer too small");
    st_t* stage = lds_e;
    const st_t* W2 = static_cast<const st_t*>(p.W2);
    const int col0 = wg_lo * 16;
    const int ncols = wg_nt * 16;
    for (int kc = 0; kc < R; kc += KCH) {
      const int kn = min(KCH, R - kc);
      for (int i = tid; i < kn * ncols; i += NT) {
        const int kr = i / ncols, c = i - kr * ncols;
        const int v = col0 + c;
        stage[kr * SLD + c] = (v < V) ? W2[size_t(kc + kr) * V + v] : st_t(0);
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (t < nt) {   // columns of tile t lie inside the staged slice
          const int c = (w_lo - wg_lo + t) * 16 + li;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int kr = ks * E::KS + E::KPL * lg - kc;   // kn is a multiple of KS: kr..kr+KPL-1 all staged
            if (kr >= 0 && kr < kn) {
              if constexpr (BF16) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  w[i] = uint32_t(stage[(kr + 2 * i) * SLD + c]) | (uint32_t(stage[(kr + 2 * i + 1) * SLD + c]) << 16);
                A[t][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
              } else {
                A[t][ks] = stage[kr * SLD + c];
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < kMaxOwnedRows; i += NT) lds_S[i] = 1.0f;
  for (int i = tid; i < GR; i += NT) lds_key[i] = 0ull;

  const st_t* U = static_cast<const st_t*>(p.U);
  const st_t* W1 = static_cast<const st_t*>(p.W1);
  const int ngroups = (B + GR - 1) / GR;

  // Publishes the drafted token of step kk (1-based) for a row this
  // workgroup owns; its logit comes from the workgroup whose tiles hold it.
  auto emit = [&](int b, int kk, uint64_t key) {
    uint32_t x = key_index(key);
    if (key == 0ull || x >= uint32_t(V)) x = uint32_t(V - 1);   // only after a barrier timeout
    const int owner = part_of(int(x >> 4), p.tiles, nwg);
    const float z = __hip_atomic_load(&p.zpart[(size_t((kk & 1) * nwg + owner)) * B + b],
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p.tokens[size_t(b) * gamma + kk - 1] = int32_t(x);
    p.logit[size_t(b) * gamma + kk - 1] = z;
    return int(x);
  };

  for (int k = 1; k <= gamma; ++k) {
    for (int grp = 0; grp < ngroups; ++grp) {
      const int g0 = grp * GR;
      const int rows = min(GR, B - g0);

      // 1. previous tokens of the group's rows (and the outputs of step k-1)
      if (tid < rows) {
        const int b = g0 + tid;
        const bool own = (b % nwg) == wg;
        int x;
        if (k == 1) {
          x = min(max(int(p.anchor[b]), 0), V - 1);
        } else {
          const uint64_t key = __hip_atomic_load(&p.slots[size_t(k - 2) * B + b], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
          if (own) {
            x = emit(b, k - 1, key);
          } else {
            x = int(key_index(key));
            if (key == 0ull || x >= V || x < 0) x = V - 1;
          }
        }
        lds_x[tid] = x;
        if (own) lds_hd[tid] = p.hdot[size_t(b) * gamma + (k - 1)];
      }
      __syncthreads();

      // 2. gather e = W1[x_{k-1}] for the group's rows into LDS
      for (int c = tid; c < GR * CHUNKS; c += NT) {
        const int row = c / CHUNKS, ch = c - row * CHUNKS;
        u32x4_t val = u32x4_t{0u, 0u, 0u, 0u};
        if (row < rows)
          val = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(W1 + size_t(lds_x[row]) * R) + ch * 16);
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(lds_e + row * LDE) + ch * 16) = val;
      }
      __syncthreads();

      // 3. confidence + STS + survival for the rows this workgroup owns
      {
        const int j_lo = (g0 > wg) ? (g0 - wg + nwg - 1) / nwg : 0;
        const int j_hi = (g0 + rows > wg) ? (g0 + rows - wg + nwg - 1) / nwg : 0;
        for (int j = j_lo + wave; j < j_hi; j += NW) {
          const int b = wg + j * nwg;
          const int row = b - g0;
          double acc = 0.0;
          for (int i = lane; i < R; i += 64) acc += double(p.conf_w[p.d + i]) * double(to_f32(lds_e[row * LDE + i]));
          acc = wave_sum_f64(acc);
          if (lane == 0) {
            const double ell = double(p.conf_b) + (lds_hd[row] + acc);
            const double c = 1.0 / (1.0 + exp(-ell / double(p.sts_T[k - 1])));
            const float cf = float(c);
            const float S = lds_S[j] * cf;
            lds_S[j] = S;
            p.conf[size_t(b) * gamma + k - 1] = cf;
            p.surv[size_t(b) * gamma + k - 1] = S;
          }
        }
      }

      // 4. z = U_k + e W2 on MFMA, argmax in registers, per request tile
      const int nbt = (rows + 15) >> 4;
      RawU<BF16> ubuf[TPW];
      load_tile<BF16, TPW>(ubuf, U, g0, 0, li, lg, B, gamma, k, V, w_lo, nt, p.vec_ok);
      for (int bt = 0; bt < nbt; ++bt) {
        f32x4_t acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t] = widen_u(ubuf[t]);
        if (bt + 1 < nbt) load_tile<BF16, TPW>(ubuf, U, g0, bt + 1, li, lg, B, gamma, k, V, w_lo, nt, p.vec_ok);
        const st_t* erow = lds_e + (bt * 16 + li) * LDE + E::KPL * lg;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const frag_t bfr = lds_frag(erow + ks * E::KS);
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            if (t < nt) acc[t] = mfma16(A[t][ks], bfr, acc[t]);
        }
        const int brow = bt * 16 + li;
        const int b = g0 + brow;
        float bs = -INFINITY, bz = 0.f;
        uint32_t bv = 0xFFFFFFFFu;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          if (t < nt) {
            const int v0 = (w_lo + t) * 16 + 4 * lg;
            f32x4_t s4 = acc[t];
            if constexpr (GUMBEL) {
              uint32_t c0 = uint32_t(v0) >> 2, c1 = uint32_t(k), c2 = uint32_t(b), c3 = 0u;
              philox4x32_10(c0, c1, c2, c3, p.seed_lo, p.seed_hi);
              s4 += f32x4_t{gumbel_from_word(c0), gumbel_from_word(c1), gumbel_from_word(c2),
                            gumbel_from_word(c3)};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (v0 + i < V && s4[i] > bs) {
                bs = s4[i];
                bv = uint32_t(v0 + i);
                bz = acc[t][i];
              }
            }
          }
        }
        uint64_t key = (bv == 0xFFFFFFFFu) ? 0ull : argmax_key(bs, bv);
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
          const uint64_t ok = shfl_xor_u64(key, m);
          const float oz = __shfl_xor(bz, m, 64);
          if (ok > key) {
            key = ok;
            bz = oz;
          }
        }
        if (lg == 0 && b < B && key != 0ull) {
          atomicMax(reinterpret_cast<unsigned long long*>(&lds_key[brow]), (unsigned long long)key);
          lds_z[wave][brow] = bz;
        }
      }
      __syncthreads();

      // 5. publish this workgroup's winner of every row of the group
      if (tid < rows) {
        const uint64_t key = lds_key[tid];
        lds_key[tid] = 0ull;
        if (key != 0ull) {
          const int b = g0 + tid;
          __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(&p.slots[size_t(k - 1) * B + b]),
                                 (unsigned long long)key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int tile = int(key_index(key) >> 4);
          const int w = part_of(tile - wg_lo, wg_nt, NW);
          p.zpart[(size_t((k & 1) * nwg + wg)) * B + b] = lds_z[w][tid];
        }
      }
      __syncthreads();
    }
    grid_barrier(&p.ctrl[0], &p.ctrl[1], unsigned(k) * unsigned(nwg), p.spin_limit);
  }
  // outputs of the last step
  for (int b = wg + tid * nwg; b < B; b += NT * nwg) {
    const uint64_t key = __hip_atomic_load(&p.slots[size_t(gamma - 1) * B + b], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    emit(b, gamma, key);
  }
}

struct KernelChoice {
  const void* fn;
  int threads;
  int tpw;
};

template <bool BF16, int R, bool G>
KernelChoice pick_r() {
  constexpr int NW = 8, GR = 256;
  constexpr int TPW = BF16 ? 5 : 4;
  return KernelChoice{reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, TPW, GR, G>), NW * 64, TPW};
}

template <bool G>
bool pick(bool bf16, int r, KernelChoice* out) {
  if (bf16) {
    switch (r) {
      case 32: *out = pick_r<true, 32, G>(); return true;
      case 64: *out = pick_r<true, 64, G>(); return true;
      case 128: *out = pick_r<true, 128, G>(); return true;
      case 256: *out = pick_r<true, 256, G>(); return true;
      default: return false;
    }
  }
  switch (r) {
    case 16: *out = pick_r<false, 16, G>(); return true;
    case 32: *out = pick_r<false, 32, G>(); return true;
    case 64: *out = pick_r<false, 64, G>(); return true;
    default: return false;
  }
}

struct DeviceInfo {
  int cus = 0;
};

hipError_t device_info(DeviceInfo* info) {
  static thread_local int cached_dev = -1;
  static thread_local int cached_cus = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != cached_dev) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached_dev = dev;
    cached_cus = cus;
  }
  info->cus = cached_cus;
  return hipSuccess;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

DraftWorkspace draft_workspace_layout(int B, int gamma) {
  DraftWorkspace w;
  size_t off = 0;
  w.ctrl = off;
  off += 256;
  w.slots = off;
  off = align256(off + size_t(gamma) * B * sizeof(uint64_t));
  w.zpart = off;
  off = align256(off + size_t(2) * kMaxDraftWorkgroups * B * sizeof(float));
  w.hdot = off;
  off = align256(off + size_t(B) * gamma * sizeof(double));
  w.total = off;
  return w;
}

hipError_t launch_markov_draft(const DraftArgs& a, hipStream_t stream, const char** unsupported) {
  *unsupported = nullptr;
  KernelChoice kc;
  const bool ok = a.gumbel ? pick<true>(a.bf16, a.r, &kc) : pick<false>(a.bf16, a.r, &kc);
  if (!ok) {
    *unsupported = a.bf16 ? "bf16 drafting supports r in {32, 64, 128, 256}"
                          : "fp32 drafting supports r in {16, 32, 64}";
    return hipSuccess;
  }
  DeviceInfo info;
  hipError_t e = device_info(&info);
  if (e != hipSuccess) return e;
  const int tiles = (a.V + 15) / 16;
  int nwg = info.cus < kMaxDraftWorkgroups ? info.cus : kMaxDraftWorkgroups;
  if (nwg > tiles) nwg = tiles;
  if (nwg < 1) nwg = 1;
  const int per_wg = (tiles + nwg - 1) / nwg;
  const int nwaves = kc.threads / 64;
  if ((per_wg + nwaves - 1) / nwaves > kc.tpw) {
    *unsupported = "vocabulary too large to keep W2 on chip on this GPU";
    return hipSuccess;
  }
  if ((a.B + nwg - 1) / nwg > kMaxOwnedRows) {
    *unsupported = "too many requests per workgroup for the confidence epilogue";
    return hipSuccess;
  }
  const DraftWorkspace L = draft_workspace_layout(a.B, a.gamma);
  char* ws = static_cast<char*>(a.ws);
  DraftParams p;
  p.B = a.B;
  p.gamma = a.gamma;
  p.V = a.V;
  p.d = a.d;
  p.nwg = nwg;
  p.tiles = tiles;
  p.vec_ok = (a.V % 4) == 0;
  p.seed_lo = uint32_t(a.seed);
  p.seed_hi = uint32_t(a.seed >> 32);
  p.spin_limit = 1u << 22;
  p.conf_b = a.conf_b;
  p.anchor = a.anchor;
  p.U = a.U;
  p.h = a.h;
  p.W1 = a.W1;
  p.W2 = a.W2;
  p.conf_w = a.conf_w;
  p.sts_T = a.sts_T;
  p.tokens = a.tokens;
  p.logit = a.logit;
  p.conf = a.conf;
  p.surv = a.surv;
  p.ctrl = reinterpret_cast<unsigned int*>(ws + L.ctrl);
  p.slots = reinterpret_cast<uint64_t*>(ws + L.slots);
  p.zpart = reinterpret_cast<float*>(ws + L.zpart);
  p.hdot = reinterpret_cast<double*>(ws + L.hdot);

  int init_blocks = (a.B * a.gamma + 3) / 4;
  if (init_blocks > 1024) init_blocks = 1024;
  if (init_blocks < 1) init_blocks = 1;
  if (a.bf16)
    hipLaunchKernelGGL(draft_init_kernel<true>, dim3(init_blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(draft_init_kernel<false>, dim3(init_blocks), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* args[] = {&p};
  return hipLaunchCooperativeKernel(kc.fn, dim3(nwg), dim3(kc.threads), args, 0, stream);
}

}  // namespace dspark
