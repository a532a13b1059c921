// Parallel-only drafting for gfx950: the baseline without a sequential head.
//
// Method ("DSpark: DeepSeek's new speculative decoding work", §1
// "Autoregressive vs Parallel Drafting": a parallel drafter emits logits for
// all block positions in one pass; §4 "Semi-Autoregressive Generation",
// parallel stage: the base logits U_k; §2 "Speedup formula": drafting time
// is one of the three levers): x_k = the lowest id maximising U_k(v), or
// U_k(v) + G(seed, b, k, v) with the Gumbel noise of the Markov-head draft.
// No step depends on another, so the whole [B][gamma][V] block is one
// streaming arg-max: the cost of the drafting stage before the sequential
// head is added.
//
// One workgroup of 256 threads per (request, position) row.  Rows whose
// length is a multiple of 8 (bf16) or 4 (fp32) elements and that start on a
// 16-byte boundary are read with 16-byte loads, four in flight per thread;
// others element by element.  Each thread sees its ids in increasing order
// and keeps the first maximum; the block then takes the largest packed
// (score, ~id) key, so the lowest id wins ties.
#include "device_util.h"
#include "launch.h"

#include <type_traits>

namespace dspark {
namespace {

constexpr int kPThreads = 256;

__device__ __forceinline__ float pd_val(const uint16_t* row, int v) { return bf16_to_f32(row[v]); }
__device__ __forceinline__ float pd_val(const float* row, int v) { return row[v]; }

template <bool BF16, bool GUMBEL>
__global__ __launch_bounds__(kPThreads) void parallel_draft_kernel(int gamma, int V, const void* __restrict__ Uv,
                                                                    uint32_t seed_lo, uint32_t seed_hi,
                                                                    int32_t* __restrict__ tokens,
                                                                    float* __restrict__ logit) {
  typedef typename std::conditional<BF16, uint16_t, float>::type st_t;
  constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  const size_t rowi = blockIdx.x;
  const int b = int(rowi / gamma), k = int(rowi % gamma) + 1;
  const st_t* row = static_cast<const st_t*>(Uv) + rowi * size_t(V);
  const int tid = threadIdx.x;

  float bs = -INFINITY, bz = 0.f;
  int bi = -1;
  auto noisy = [&](int v0, float* s, const float* z, int n) {
    // s = z + G + ln(ln 2) for ids v0 .. v0+n-1 (v0 a multiple of 4, n a multiple of 4)
    for (int g = 0; g < n; g += 4) {
      uint32_t c0 = uint32_t(v0 + g) >> 2, c1 = uint32_t(k), c2 = uint32_t(b), c3 = 0u;
      philox4x32_10(c0, c1, c2, c3, seed_lo, seed_hi);
      s[g + 0] = z[g + 0] + gumbel_shifted_from_word(c0);
      s[g + 1] = z[g + 1] + gumbel_shifted_from_word(c1);
      s[g + 2] = z[g + 2] + gumbel_shifted_from_word(c2);
      s[g + 3] = z[g + 3] + gumbel_shifted_from_word(c3);
    }
  };
  auto take_chunk = [&](int v0, const float* z) {
    float s[EPC];
    if constexpr (GUMBEL) {
      noisy(v0, s, z, EPC);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) s[i] = z[i];
    }
#pragma unroll
    for (int i = 0; i < EPC; ++i) {
      const bool take = s[i] > bs;
      bs = take ? s[i] : bs;
      bi = take ? v0 + i : bi;
      bz = take ? z[i] : bz;
    }
  };

  const bool vec = (V % EPC) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  if (vec) {
    const u32x4_t* r16 = reinterpret_cast<const u32x4_t*>(row);
    const int nch = V / EPC;
    int c = tid;
    for (; c + 3 * kPThreads < nch; c += 4 * kPThreads) {
      u32x4_t q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = __builtin_nontemporal_load(r16 + c + u * kPThreads);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float z[EPC];
        if constexpr (BF16) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            z[2 * j] = bf16_lo(q[u][j]);
            z[2 * j + 1] = bf16_hi(q[u][j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) z[j] = __uint_as_float(q[u][j]);
        }
        take_chunk((c + u * kPThreads) * EPC, z);
      }
    }
    for (; c < nch; c += kPThreads) {
      const u32x4_t q = __builtin_nontemporal_load(r16 + c);
      float z[EPC];
      if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[2 * j] = bf16_lo(q[j]);
          z[2 * j + 1] = bf16_hi(q[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = __uint_as_float(q[j]);
      }
      take_chunk(c * EPC, z);
    }
  } else {
    // element by element, four consecutive ids per thread (one noise call)
    for (int v0 = tid * 4; v0 < V; v0 += 4 * kPThreads) {
      float z[4], s[4];
      const int n = min(4, V - v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = (i < n) ? pd_val(row, v0 + i) : 0.f;
      if constexpr (GUMBEL) {
        noisy(v0, s, z, 4);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = z[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool take = i < n && s[i] > bs;
        bs = take ? s[i] : bs;
        bi = take ? v0 + i : bi;
        bz = take ? z[i] : bz;
      }
    }
  }

  // block reduction of (score, ~id) keys, the unperturbed logit travelling along
  uint64_t key = (bi < 0) ? 0ull : argmax_key(bs, uint32_t(bi));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t ok = shfl_xor_u64(key, m);
    const float oz = __shfl_xor(bz, m, 64);
    if (ok > key) {
      key = ok;
      bz = oz;
    }
  }
  __shared__ uint64_t wkey[kPThreads / 64];
  __shared__ float wz[kPThreads / 64];
  if ((tid & 63) == 0) {
    wkey[tid >> 6] = key;
    wz[tid >> 6] = bz;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t best = wkey[0];
    float z = wz[0];
    for (int w = 1; w < kPThreads / 64; ++w)
      if (wkey[w] > best) {
        best = wkey[w];
        z = wz[w];
      }
    tokens[rowi] = best == 0ull ? -1 : int32_t(key_index(best));
    logit[rowi] = z;
  }
}

// The Gumbel sample of the drafting kernels for given 32-bit hash words.
__global__ __launch_bounds__(256) void gumbel_words_kernel(int n, const uint32_t* __restrict__ words,
                                                           float* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = gumbel_from_word(words[i]);
}

}  // namespace

hipError_t launch_gumbel_words(int n, const uint32_t* words, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(gumbel_words_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, n, words, out);
  return hipGetLastError();
}

hipError_t launch_parallel_draft(int B, int gamma, int V, bool bf16, const void* U, bool gumbel, uint64_t seed,
                                 int32_t* tokens, float* logit, hipStream_t stream) {
  const uint32_t lo = uint32_t(seed), hi = uint32_t(seed >> 32);
  const dim3 grid(unsigned(size_t(B) * gamma)), block(kPThreads);
  if (bf16) {
    if (gumbel)
      hipLaunchKernelGGL((parallel_draft_kernel<true, true>), grid, block, 0, stream, gamma, V, U, lo, hi, tokens, logit);
    else
      hipLaunchKernelGGL((parallel_draft_kernel<true, false>), grid, block, 0, stream, gamma, V, U, lo, hi, tokens, logit);
  } else {
    if (gumbel)
      hipLaunchKernelGGL((parallel_draft_kernel<false, true>), grid, block, 0, stream, gamma, V, U, lo, hi, tokens, logit);
    else
      hipLaunchKernelGGL((parallel_draft_kernel<false, false>), grid, block, 0, stream, gamma, V, U, lo, hi, tokens, logit);
  }
  return hipGetLastError();
}

}  // namespace dspark
