// Device helpers shared by the libdspark kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bfloat16 is the upper half of an IEEE fp32: widening is a 16-bit shift.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Order-preserving map of an fp32 value to uint32 (larger value -> larger
// code); -0 is folded onto +0 so that equal values compare equal.
__device__ __forceinline__ uint32_t ord_f32(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Argmax key: the larger key has the larger value, and among equal values
// the smaller index.  Key 0 means "no candidate".
__device__ __forceinline__ uint64_t argmax_key(float s, uint32_t idx) {
  return (uint64_t(ord_f32(s)) << 32) | uint64_t(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~uint32_t(key); }
__device__ __forceinline__ float key_value(uint64_t key) { return unord_f32(uint32_t(key >> 32)); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  uint32_t lo = __shfl_xor(uint32_t(x), m, 64);
  uint32_t hi = __shfl_xor(uint32_t(x >> 32), m, 64);
  return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Three-input exclusive or in one gfx950 instruction (v_bitop3_b32 with the
// truth table 0x96: the output bit is set when an odd number of inputs are).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64-bit
// multiplies on counter words 0 and 2 with the result words crossed and
// xor-ed with the key; the key advances by the Weyl constants between rounds.
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;   // key increments
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                             uint32_t k1) {
  const uint32_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
  const uint64_t p0 = uint64_t(m0) * c0, p1 = uint64_t(m1) * c2;   // one 32x32->64 multiply each
  const uint32_t hi0 = uint32_t(p0 >> 32), lo0 = uint32_t(p0);
  const uint32_t hi1 = uint32_t(p1 >> 32), lo1 = uint32_t(p1);
  const uint32_t n0 = xor3(hi1, c1, k0);
  const uint32_t n2 = xor3(hi0, c3, k1);
  c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
}
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    philox_round(c0, c1, c2, c3, k0, k1);
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
}

// Standard Gumbel sample from one 32-bit hash word: u = (2*(w>>9)+1) * 2^-24
// lies in (0, 1) and is exact in fp32; G = -ln(-ln u).
//
// Both logarithms use the hardware base-2 logarithm (v_log_f32) times ln 2.
// Measured on gfx950 over all 2^23 values u of this form (against fp64):
// the relative error of -ln u stays below 1.7e-7 everywhere, including u
// within 2^-24 of 1, where 1 - u is tiny; L = -ln u >= 5.9e-8 is a normal
// number, so the outer logarithm is as accurate, and the absolute error of G
// stays around 1e-6.
//
// u is formed in two instructions: one funnel shift puts the top 23 bits of
// w under the exponent of 1.0 (the float 1 + (w >> 9) * 2^-23), and
// subtracting 1 - 2^-24 leaves (2 (w >> 9) + 1) * 2^-24 exactly (the operands
// are within a factor of two of each other, so the difference is exact).
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  const float one_plus = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
  const float u = one_plus - 0x1.fffffep-1f;
  const float ln2 = 0.693147180559945309f;
  const float l = -__builtin_amdgcn_logf(u) * ln2;
  return -__builtin_amdgcn_logf(l) * ln2;
}

// The arg-max of z + G only needs G up to a constant: with L2 = -log2 u
// (so that -ln u = L2 ln 2), G = -ln(L2) - ln(ln 2), and the score
// z - ln 2 * log2(L2) is z + G + ln(ln 2), the same shift for every id.  It
// takes one multiply fewer per id; the drafting kernels rank by it (the
// unperturbed logit travels with the winner separately).
__device__ __forceinline__ float gumbel_shifted_from_word(uint32_t w) {
  const float one_plus = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
  const float u = one_plus - 0x1.fffffep-1f;
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u)) * 0.693147180559945309f;
}

// 16-byte direct-to-LDS load (gfx950 global_load_lds_dwordx4): lane j of the
// wave copies 16 bytes from its own global address `src` to lds_base + 16 * j.
// lds_base must be the same for every lane.  Completion is tracked by the
// vector-memory counter only (see wait_vmem); the compiler does not order
// later LDS reads after it, so readers synchronise explicitly.
__device__ __forceinline__ void load_lds16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
#endif
}

// The same load at device scope (cache policy sc1, as a relaxed agent-scope
// atomic load uses): it reads what other workgroups published with
// device-scope stores.
__device__ __forceinline__ void load_lds16_dev(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 16);
#endif
}

// LDS 64-bit atomic max and 32-bit store issued as plain ds_* instructions.
// The compiler does not see them as LDS accesses, so it does not make them
// wait for unrelated direct-to-LDS loads still in flight; in exchange the
// caller waits for them explicitly (lds_wait) before any other wave reads
// the locations.
typedef __attribute__((address_space(3))) uint64_t lds_u64_t;
typedef __attribute__((address_space(3))) float lds_f32_t;
__device__ __forceinline__ void lds_max_u64(uint64_t* p, uint64_t v) {
  asm volatile("ds_max_u64 %0, %1" : : "v"((lds_u64_t*)p), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store_f32(float* p, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"((lds_f32_t*)p), "v"(v) : "memory");
}
// Byte address of an LDS location, as ds_* instructions take it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Waits until this wave's outstanding vector-memory operations (loads,
// stores, atomics) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Device-scope (all XCDs) accesses: they bypass the non-coherent caches, so
// no L2 write-back or invalidation is needed around them.
template <typename T>
__device__ __forceinline__ T load_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void store_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid-wide barrier for a co-resident (cooperatively launched) grid whose
// cross-workgroup data moves only through device-scope atomics, loads and
// stores, in two halves so that independent work can be issued in between.
// grid_arrive: every wave waits for its own memory operations to complete,
// the workgroup synchronises, and one thread arrives on the counter.
// grid_wait: that thread polls the counter; the workgroup synchronises.  The
// counter counts arrivals over the whole launch; barrier number n waits for
// n * gridDim.x arrivals.  The spin is bounded: after `limit` polls the
// error flag is raised, and once it is raised every barrier returns at once,
// so every wave always reaches the end of the kernel.
__device__ __forceinline__ void grid_arrive(unsigned int* counter) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void grid_wait(unsigned int* counter, unsigned int* err, unsigned int target,
                                          unsigned int limit) {
  if (threadIdx.x == 0) {
    unsigned int polls = 0;
    while (load_dev(counter) < target) {
      if (load_dev(err) != 0u) break;
      if (++polls > limit) {
        store_dev(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

}  // namespace dspark
