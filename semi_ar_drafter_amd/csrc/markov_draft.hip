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
//    depend on the drafted tokens and is computed in the kernel's prologue.
//  * Cross-workgroup data (argmax slots, per-workgroup winner logits, the
//    barrier counter) moves only through device-scope atomics, loads and
//    stores, so no L2 write-back or invalidation is ever issued.  The
//    workspace is left zeroed by every call: the last phase of the kernel
//    clears the slots and counters for the next call, so a call is a single
//    launch.
#include "device_util.h"
#include "rank_schedule.h"
#include "launch.h"

#include <mutex>
#include <type_traits>

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
  int grs;             // requests per group (multiple of 16, at most the kernel's GR)
  unsigned int* ctrl;  // [1] error flag, [2] exit arrivals
  unsigned int* bar;   // arrivals of request group g at bar[g * kBarStride]
  uint64_t* slots;     // [gamma][B] packed argmax keys
  float* zpart;        // [2][nwg][B] logit of each workgroup's local winner
  double* hdot;        // [B][gamma] hidden-state part of the confidence logit
  const float* decay;  // RNN head: per-channel decay of the recurrent state [r]
  uint16_t* state;     // RNN head: recurrent state, bf16 [2][B][r] (by step parity)
  // small batches (the SMALL kernels): every workgroup's winner key of (step k, request b) at
  // wkeys[(k * B + b) * nwg + wg], written once per call (0 = not yet written), and for Gumbel
  // sampling the winner's unperturbed logit as ~bits at the same index of wz
  uint64_t* wkeys;
  uint32_t* wz;
  // fused step (the STEP kernels): the ranking scheduler and verify after the last draft position
  unsigned int* sched_tickets;
  RankEntry* sched_sorted;
  const double* t_step;
  int n_min, n_count, sched_e;
  const int32_t* target;
  int32_t *lens, *m_out, *accepted, *bonus;
};

// RNN head state step for four channels (a reading of the RNN head, whose
// equations the pages do not give): s = bf16(fp32(a * s_prev) + e), the
// product and the sum rounded separately (no fused multiply-add), the bf16
// rounding to nearest even by the hardware conversion.
__device__ __forceinline__ u32x2_t rnn_step4(const float* a, u32x2_t sp, u32x2_t e) {
#pragma clang fp contract(off)
  const float spv[4] = {bf16_lo(sp.x), bf16_hi(sp.x), bf16_lo(sp.y), bf16_hi(sp.y)};
  const float ev[4] = {bf16_lo(e.x), bf16_hi(e.x), bf16_lo(e.y), bf16_hi(e.y)};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = a[i] * spv[i];
    const float u = t + ev[i];
    o[i] = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(u)));
  }
  return u32x2_t{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
}

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

// Layout of the gathered embeddings e in LDS.  bf16 rows are stored
// unpadded (R elements) and filled by 16-byte direct-to-LDS loads; the
// 16-byte chunks of a row are permuted by an XOR with a per-row code so that
// the B-operand reads of 8 consecutive rows fall on 8 different bank groups.
// fp32 rows are padded instead.
template <bool BF16, int R>
struct ELayout {
  static constexpr int LDE = BF16 ? R : R + Elem<BF16>::PAD;                      // row stride (elements)
  static constexpr int CPR = R * int(sizeof(typename Elem<BF16>::store_t)) / 16;  // 16-byte chunks per row
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (!BF16) return 0;
    else if constexpr (CPR >= 8) return row & 7;
    else return (row / (8 / CPR)) & (CPR - 1);
  }
  // offset (elements) of element i of row `row`
  __device__ static __forceinline__ int at(int row, int i) {
    if constexpr (!BF16) return row * LDE + i;
    else return row * LDE + (((i >> 3) ^ swz(row)) << 3) + (i & 7);
  }
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
    r.q = (v0 < V) ? *reinterpret_cast<const u32x2_t*>(row + v0) : u32x2_t{0u, 0u};
  } else {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (v0 + i < V) ? uint32_t(row[v0 + i]) : 0u;
    r.q = u32x2_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  }
}
__device__ __forceinline__ void load_u(RawU<false>& r, const float* row, int v0, int V, int vec_ok) {
  if (vec_ok) {
    r.q = (v0 < V) ? *reinterpret_cast<const f32x4_t*>(row + v0) : f32x4_t{0.f, 0.f, 0.f, 0.f};
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

// Column layout of the branch-free path.  Tiles are taken in pairs; lane
// group q of a pair holds 8 consecutive vocabulary ids, 4 in each tile of the
// pair, so a single 16-byte load per lane fetches the base logits of both
// tiles (16 requests x 64 contiguous bytes per load instruction instead of
// 16 x 32).  With TPW odd the last slot is an ordinary 16-wide tile.  A wave
// owning nt < TPW tiles (nt >= 2) fills its spare slots with exact copies of
// columns it already holds: a spare pair slot repeats pair 0, a spare last
// slot repeats the second half of the last real pair.  With TPW even (no
// last slot) and nt odd, the pair slot after the last complete pair covers
// the wave's last two tiles (its first half repeats the previous pair's
// second half).  Returns the first of the four consecutive columns (relative
// to the wave's first column) that lane group q holds in tile slot t.  Along
// t the ids a lane sees never decrease except for exact repeats, so a strict
// comparison in t order still picks the lowest id among equal scores.
__device__ __forceinline__ int pair_col(int t, int q, int nt, int tpw) {
  const int rp = nt >> 1;   // complete pairs the wave owns
  if (t < (tpw & ~1)) {
    const int pr = t >> 1;
    const int base = pr < rp ? 32 * pr : ((tpw & 1) == 0 && (nt & 1) && pr == rp) ? 32 * rp - 16 : 0;
    return base + 8 * q + 4 * (t & 1);
  }
  return (nt & 1) ? 32 * rp + 4 * q : 32 * (rp - 1) + 8 * q + 4;
}

// Phase 4 of a draft step for one wave: for every 16-request tile of the
// group, z = U_k + e W2 over the wave's NTF vocabulary tiles (accumulator
// initialised with U_k, MFMA over the rank), then the argmax over z (greedy)
// or z + Gumbel noise, merged into the workgroup's per-request LDS key.
//
// Per lane and request tile the argmax runs tile by tile: the tile maximum,
// a strict comparison with the running best (so the earliest tile wins
// ties) that keeps the best tile's index and its four scores, and at the end
// the first of those four equal to the best score: the lowest vocabulary id
// among equal maxima.
//
// The U loads of request tile bt + 3 are issued right after tile bt's data
// has been taken into the accumulators, into the same one of three fixed
// buffers, with the tile index clamped at the end so the issue never sits
// behind a branch; the B-operand fragment is read one K step ahead.  CHECKED
// (natural 16-wide tiles, U loaded into registers) handles a wave with fewer
// than NTF tiles, a tile crossing the end of the vocabulary and V % 4 != 0.
// The unchecked form (bf16, whole tiles, the pair layout above) has no
// per-tile branches and stages U through a per-wave ring of three LDS slots:
// the 16 rows x nt*32 bytes of a request tile are fetched row-major with
// 16-byte direct-to-LDS loads (whole 128-byte lines per row, three load
// instructions per tile), rows padded to an odd number of 16-byte chunks so
// that the fragment reads of 8 consecutive rows hit 8 different bank groups.
template <bool BF16, int R, int TPW, int GR, bool GUMBEL, int NTF, bool CHECKED>
struct TileWork {
  typedef Elem<BF16> E;
  typedef typename E::store_t st_t;
  typedef typename E::frag_t frag_t;
  static constexpr int NKS = R / E::KS;
  typedef ELayout<BF16, R> EL;
  static constexpr int LDE = EL::LDE;
  static constexpr int NP = TPW / 2;               // tile pairs (unchecked form)
  static constexpr bool LONE = (TPW & 1) != 0;     // unpaired last slot
  static_assert(CHECKED || (BF16 && NTF == TPW), "the pair layout is for bf16 whole tiles");

  struct CheckedBuf {
    RawU<BF16> t[NTF];
  };
  struct SlotBuf {};   // the data lives in the wave's LDS slot of the same index
  typedef typename std::conditional<CHECKED, CheckedBuf, SlotBuf>::type Buf;
  static constexpr int SLOT_U32 = 768;   // one LDS slot: 192 16-byte chunks

  const frag_t (&A)[TPW][NKS];
  const st_t* lds_e;
  uint64_t* lds_key;
  float* lds_zw;
  size_t row_stride;   // gamma * V elements between consecutive requests
  const st_t* ubase;   // CHECKED: U[g0][k-1][vlane]; else U[g0][k-1][wave's first column]
  int g0, rows, nbt, B, k, V, nt, vec_ok, li, lg;
  int vlane;           // CHECKED: first id of this lane's 4 in tile 0; else the wave's first column
  int oP0, oP1, oL;    // unchecked: columns (relative) of this lane's pair-0 / pair-1 / last-slot loads
  int fe, fo;          // bf16: offsets within a row of this lane's B fragment for even / odd K steps
  uint32_t* lds_u;     // unchecked: this wave's three staging slots
  int dr0, dr1, dr2;   // unchecked: request row (within the tile) of this lane's chunk in load instruction 0/1/2
  int dc0, dc1, dc2;   //            and its column (elements, relative to the wave's first column)
  int rP0, rP1, rL;    // unchecked: byte offsets within a slot of this lane's pair-0 / pair-1 / last-slot data
  uint32_t seed_lo, seed_hi;

  // B-operand fragment of request tile bt, K step ks (ks is a compile-time constant after unrolling).
  // bf16: chunk (4 ks + lg) of row bt*16 + li sits at chunk ((4 ks + lg) ^ swz(li)); with
  // s = swz(li) that is 4 (ks ^ (s >> 2)) + (lg ^ (s & 3)), i.e. a per-lane base for even and
  // for odd ks plus 64 (ks >> 1) elements.
  __device__ __forceinline__ frag_t bfrag(int bt, int ks) const {
    if constexpr (BF16)
      return lds_frag(lds_e + (bt * 16 + li) * LDE + ((ks & 1) ? fo : fe) + 64 * (ks >> 1));
    else
      return lds_frag(lds_e + (bt * 16 + li) * LDE + ks * E::KS + E::KPL * lg);
  }

  // first of this lane's four consecutive ids in tile slot t
  __device__ __forceinline__ int tile_id0(int t) const {
    if constexpr (CHECKED) {
      return vlane + 16 * t;
    } else {
      if (t < 2 * NP) return vlane + ((t >> 1) == 0 ? oP0 : oP1) + 4 * (t & 1);
      return vlane + oL;
    }
  }

  // CHECKED: load this lane's U values of request tile bt into registers.
  __device__ __forceinline__ void issue(Buf& bb, int bt) const {
    if constexpr (CHECKED) {
      const int r = min(min(bt, nbt - 1) * 16 + li, rows - 1);   // clamped into the group
      const st_t* p = ubase + size_t(r) * row_stride;
#pragma unroll
      for (int t = 0; t < NTF; ++t)
        if (t < nt) load_u(bb.t[t], p - vlane, vlane + 16 * t, V, vec_ok);   // row start, column
    }
  }

  // Unchecked: staging slot s (0..2) of this wave.
  __device__ __forceinline__ uint32_t* slot(int s) const { return lds_u + s * SLOT_U32; }

  // Unchecked: fetch request tile bt into slot s (three 16-byte direct-to-LDS loads per lane).
  __device__ __forceinline__ void stage(int s, int bt) const {
    const int r0 = min(bt, nbt - 1) * 16;
    uint32_t* sl = slot(s);
    load_lds16(ubase + size_t(min(r0 + dr0, rows - 1)) * row_stride + dc0, sl);
    load_lds16(ubase + size_t(min(r0 + dr1, rows - 1)) * row_stride + dc1, sl + 256);
    load_lds16(ubase + size_t(min(r0 + dr2, rows - 1)) * row_stride + dc2, sl + 512);
  }

  // Unchecked: this lane's 20 base logits of the tile in slot s, widened into
  // the accumulators.  `ahead` later tiles (three loads each) were staged
  // after this one and may still be in flight; every older load has landed
  // once at most that many are outstanding (vector-memory operations of a
  // wave complete in order).  The reads are written as plain ds_* so that
  // the compiler does not add a wait for every staging load in flight, and
  // they complete before the asm block ends, so the slot can be refilled
  // right after.
  __device__ __forceinline__ void unstage(int s, int ahead, f32x4_t (&acc)[NTF]) const {
    static_assert(NP == 2, "staging reads written for two pairs (and an optional last slot)");
    const uint32_t base = lds_addr(slot(s));
    const uint32_t a0 = base + rP0, a1 = base + rP1, a2 = base + rL;
    u32x4_t q0, q1;
    u32x2_t ql = u32x2_t{0u, 0u};
    if constexpr (LONE) {
#define DSPARK_UNSTAGE(WAIT)                                                                  \
  asm volatile("s_waitcnt " WAIT "\n\tds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\t"        \
               "ds_read_b64 %2, %5\n\ts_waitcnt lgkmcnt(0)"                                  \
               : "=&v"(q0), "=&v"(q1), "=&v"(ql)                                            \
               : "v"(a0), "v"(a1), "v"(a2)                                                  \
               : "memory")
      if (ahead >= 2)
        DSPARK_UNSTAGE("vmcnt(6)");
      else if (ahead == 1)
        DSPARK_UNSTAGE("vmcnt(3)");
      else
        DSPARK_UNSTAGE("vmcnt(0)");
#undef DSPARK_UNSTAGE
    } else {
#define DSPARK_UNSTAGE(WAIT)                                                                  \
  asm volatile("s_waitcnt " WAIT "\n\tds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\t"        \
               "s_waitcnt lgkmcnt(0)"                                                        \
               : "=&v"(q0), "=&v"(q1)                                                        \
               : "v"(a0), "v"(a1)                                                            \
               : "memory")
      if (ahead >= 2)
        DSPARK_UNSTAGE("vmcnt(6)");
      else if (ahead == 1)
        DSPARK_UNSTAGE("vmcnt(3)");
      else
        DSPARK_UNSTAGE("vmcnt(0)");
#undef DSPARK_UNSTAGE
      (void)a2;
    }
    acc[0] = f32x4_t{bf16_lo(q0.x), bf16_hi(q0.x), bf16_lo(q0.y), bf16_hi(q0.y)};
    acc[1] = f32x4_t{bf16_lo(q0.z), bf16_hi(q0.z), bf16_lo(q0.w), bf16_hi(q0.w)};
    acc[2] = f32x4_t{bf16_lo(q1.x), bf16_hi(q1.x), bf16_lo(q1.y), bf16_hi(q1.y)};
    acc[3] = f32x4_t{bf16_lo(q1.z), bf16_hi(q1.z), bf16_lo(q1.w), bf16_hi(q1.w)};
    if constexpr (LONE) acc[4] = f32x4_t{bf16_lo(ql.x), bf16_hi(ql.x), bf16_lo(ql.y), bf16_hi(ql.y)};
  }

  // CHECKED: one request tile from registers, then the loads of tile bt + 3 into the same buffer.
  __device__ __forceinline__ void step(Buf& bb, int bt) const {
    f32x4_t acc[NTF];
#pragma unroll
    for (int t = 0; t < NTF; ++t) acc[t] = widen_u(bb.t[t]);
    issue(bb, bt + 3);
    tile(acc, bt);
  }

  // z = U + e W2 for request tile bt: the accumulators hold U on entry.
  __device__ __forceinline__ void mfma_chain(f32x4_t (&acc)[NTF], int bt) const {
    frag_t bfr = bfrag(bt, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const frag_t cur = bfr;
      if (ks + 1 < NKS) bfr = bfrag(bt, ks + 1);
#pragma unroll
      for (int t = 0; t < NTF; ++t) {
        if constexpr (CHECKED) {
          if (t < nt) acc[t] = mfma16(A[t][ks], cur, acc[t]);
        } else {
          acc[t] = mfma16(A[t][ks], cur, acc[t]);
        }
      }
    }
  }

  // This lane's candidate for request tile bt (z, or z + Gumbel noise, in
  // acc): the packed key (0 if none) and, for Gumbel sampling, the winner's
  // unperturbed logit, already reduced over the lane groups.
  // (whole-tile path) Gumbel noise of every slot of request tile bt: the
  // slots' generator calls are independent chains of dependent multiplies,
  // advanced round by round side by side.  It does not depend on the
  // accumulators.
  __device__ __forceinline__ void noise(int bt, f32x4_t (&g)[NTF]) const {
    const int b = g0 + bt * 16 + li;
    uint32_t w[NTF][4];
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      w[t][0] = uint32_t(tile_id0(t)) >> 2;
      w[t][1] = uint32_t(k);
      w[t][2] = uint32_t(b);
      w[t][3] = 0u;
    }
    uint32_t k0 = seed_lo, k1 = seed_hi;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
#pragma unroll
      for (int t = 0; t < NTF; ++t) philox_round(w[t][0], w[t][1], w[t][2], w[t][3], k0, k1);
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
#pragma unroll
    for (int t = 0; t < NTF; ++t)
      g[t] = f32x4_t{gumbel_shifted_from_word(w[t][0]), gumbel_shifted_from_word(w[t][1]),
                     gumbel_shifted_from_word(w[t][2]), gumbel_shifted_from_word(w[t][3])};
  }

  // g: the whole-tile path's noise of request tile bt (unused otherwise).
  __device__ __forceinline__ uint64_t select(const f32x4_t (&acc)[NTF], const f32x4_t (&g)[NTF], int bt,
                                             float& bz) const {
    const int b = g0 + bt * 16 + li;
    float bs = -INFINITY;
    int btile = -1;
    f32x4_t bsel = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t bzsel = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      if (CHECKED && t >= nt) continue;
      f32x4_t s4 = acc[t];
      if constexpr (GUMBEL && !CHECKED) s4 += g[t];
      if constexpr (GUMBEL && CHECKED) {
        uint32_t c0 = uint32_t(tile_id0(t)) >> 2, c1 = uint32_t(k), c2 = uint32_t(b), c3 = 0u;
        philox4x32_10(c0, c1, c2, c3, seed_lo, seed_hi);
        s4 += f32x4_t{gumbel_shifted_from_word(c0), gumbel_shifted_from_word(c1), gumbel_shifted_from_word(c2),
                      gumbel_shifted_from_word(c3)};
      }
      if constexpr (CHECKED) {   // ids past the vocabulary never win
        const int v0 = tile_id0(t);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (v0 + i >= V) s4[i] = -INFINITY;
      }
      const float mt = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
      if (!CHECKED && t == 0) {   // finite scores: tile 0 always starts the running best
        bs = mt;
        btile = 0;
        bsel = s4;
        if constexpr (GUMBEL) bzsel = acc[0];
        continue;
      }
      const bool take = mt > bs;
      bs = take ? mt : bs;
      btile = take ? t : btile;
      bsel = take ? s4 : bsel;
      if constexpr (GUMBEL) bzsel = take ? acc[t] : bzsel;
    }
    int bi = (bsel[2] == bs) ? 2 : 3;
    bi = (bsel[1] == bs) ? 1 : bi;
    bi = (bsel[0] == bs) ? 0 : bi;
    int id0;
    if constexpr (CHECKED) {
      id0 = vlane + 16 * btile;
    } else {
      id0 = (btile >= 2 * NP) ? oL : ((btile >= 2) ? oP1 : oP0) + 4 * (btile & 1);
      id0 += vlane;
    }
    uint64_t key = (btile < 0) ? 0ull : argmax_key(bs, uint32_t(id0 + bi));
    bz = 0.f;
    if constexpr (GUMBEL) {
      // the winner's unperturbed logit travels with the key
      bz = (bi == 0) ? bzsel[0] : (bi == 1) ? bzsel[1] : (bi == 2) ? bzsel[2] : bzsel[3];
      // the four lane groups' candidates of a request reduced by the gfx950
      // row swaps: swapping a value with itself leaves rows 0 and 2 (16
      // apart) or the lower half (32 apart) in one register and their
      // partners in the other, so the larger of the two is the pair's best
      // in every lane
#pragma unroll
      for (int m = 16; m <= 32; m <<= 1) {
        uint32_t kl = uint32_t(key), kh = uint32_t(key >> 32), zb = __float_as_uint(bz);
        const auto sl = (m == 16) ? __builtin_amdgcn_permlane16_swap(kl, kl, false, false)
                                  : __builtin_amdgcn_permlane32_swap(kl, kl, false, false);
        const auto sh = (m == 16) ? __builtin_amdgcn_permlane16_swap(kh, kh, false, false)
                                  : __builtin_amdgcn_permlane32_swap(kh, kh, false, false);
        const auto sz = (m == 16) ? __builtin_amdgcn_permlane16_swap(zb, zb, false, false)
                                  : __builtin_amdgcn_permlane32_swap(zb, zb, false, false);
        const uint64_t a = (uint64_t(sh[0]) << 32) | sl[0], b = (uint64_t(sh[1]) << 32) | sl[1];
        const bool tb = b > a;
        key = tb ? b : a;
        bz = __uint_as_float(tb ? sz[1] : sz[0]);
      }
    }
    return key;
  }

  // Merges a candidate of request tile bt into the workgroup's LDS key
  // (greedy: every lane its own; Gumbel: lane group 0 after the reduction).
  __device__ __forceinline__ void merge(uint64_t key, float bz, int bt) const {
    const int brow = bt * 16 + li;
    if (g0 + brow < B && key != 0ull && (!GUMBEL || lg == 0)) {
      lds_max_u64(&lds_key[brow], key);
      if constexpr (GUMBEL) lds_store_f32(&lds_zw[brow], bz);
    }
  }

  // The argmax runs at raised wave priority: it is the wave's serial
  // stretch between two MFMA chains, and the other wave of the SIMD keeps
  // the matrix unit busy meanwhile (measured: about 1.5 % faster calls).
  // The whole-tile path's Gumbel noise is computed before, at normal
  // priority: it is most of the wave's vector work, and at raised priority
  // it held back the other wave's MFMA issue (B = 512, V = 129280: 1.32 ms
  // with the noise inside the raised section, 1.26 ms with it outside, 1.36
  // ms with no raised section at all).
  __device__ __forceinline__ void tile(f32x4_t (&acc)[NTF], int bt) const {
    mfma_chain(acc, bt);
    f32x4_t g[NTF];
    if constexpr (GUMBEL && !CHECKED) noise(bt, g);
    __builtin_amdgcn_s_setprio(1);
    float bz;
    const uint64_t key = select(acc, g, bt, bz);
    merge(key, bz, bt);
    __builtin_amdgcn_s_setprio(0);
  }

  // First three request tiles' loads, issued ahead of run() (possibly
  // before the grid barrier that precedes the step: U does not depend on
  // the drafted tokens).
  __device__ __forceinline__ void prefetch(Buf& b0, Buf& b1, Buf& b2) const {
    if constexpr (CHECKED) {
      issue(b0, 0);
      issue(b1, 1);
      issue(b2, 2);
    } else {
      for (int t = 0; t < 3 && t < nbt; ++t) stage(t, t);
    }
  }

  __device__ __forceinline__ void run(Buf& b0, Buf& b1, Buf& b2) const {
    if constexpr (CHECKED) {
      // Straight-line loop body (the compiler's wait counts stay exact across
      // the back edge: consuming a buffer waits only for its own loads); the
      // last one or two request tiles run after the loop.
      int bt = 0;
      for (; bt + 3 <= nbt; bt += 3) {
        step(b0, bt);
        step(b1, bt + 1);
        step(b2, bt + 2);
      }
      if (bt < nbt) step(b0, bt);
      if (bt + 1 < nbt) step(b1, bt + 1);
    } else {
      int s = 0;
      for (int bt = 0; bt < nbt; ++bt) {
        f32x4_t acc[NTF];
        unstage(s, min(2, nbt - 1 - bt), acc);
        if (bt + 3 < nbt) stage(s, bt + 3);
        tile(acc, bt);
        s = (s == 2) ? 0 : s + 1;
      }
    }
    lds_wait();   // this wave's key merges have landed
  }
};

template <bool BF16, int R, int TPW, int GR, bool GUMBEL, int NTF, bool CHECKED>
__device__ __forceinline__ TileWork<BF16, R, TPW, GR, GUMBEL, NTF, CHECKED> make_work(
    const typename Elem<BF16>::frag_t (&A)[TPW][R / Elem<BF16>::KS], const typename Elem<BF16>::store_t* lds_e,
    const typename Elem<BF16>::store_t* U, int g0, int rows, int B, int gamma, int k, int V, int w_lo, int nt,
    int vec_ok, int li, int lg, uint32_t seed_lo, uint32_t seed_hi, uint64_t* lds_key, float* lds_zw,
    uint32_t* lds_u) {
  const size_t row_stride = size_t(gamma) * V;
  const int vlane = CHECKED ? w_lo * 16 + 4 * lg : w_lo * 16;
  const int oP0 = CHECKED ? 0 : pair_col(0, lg, nt, TPW);
  const int oP1 = CHECKED ? 0 : pair_col(2 < 2 * (TPW / 2) ? 2 : 0, lg, nt, TPW);
  const int oL = CHECKED ? 0 : pair_col(TPW - 1, lg, nt, TPW);
  const int sw = ELayout<BF16, R>::swz(li);
  const int m = lg ^ (sw & 3), h = sw >> 2;
  // staging slot: 16 rows of RS 16-byte chunks, the last chunk of a row and
  // the positions past 16 rows being padding that receives a copy of chunk 0
  const int RS = 2 * nt + 1;
  const int lane = li + 16 * lg;
  int dr[3], dc[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int pos = 64 * i + lane;
    const int rr = pos / RS, cc = pos - rr * RS;
    const bool real = rr < 16 && cc < 2 * nt;
    dr[i] = real ? rr : 0;
    dc[i] = real ? 8 * cc : 0;
  }
  const int rP0 = (li * RS + oP0 / 8) * 16, rP1 = (li * RS + oP1 / 8) * 16;
  const int rL = (li * RS + oL / 8) * 16 + (oL & 7) * 2;
  return TileWork<BF16, R, TPW, GR, GUMBEL, NTF, CHECKED>{
      A, lds_e, lds_key, lds_zw, row_stride, U + (size_t(g0) * gamma + (k - 1)) * V + vlane,
      g0, rows, (rows + 15) >> 4, B, k, V, nt, vec_ok, li, lg, vlane, oP0, oP1, oL,
      8 * (4 * h + m), 8 * (4 * (1 - h) + m), lds_u, dr[0], dr[1], dr[2], dc[0], dc[1], dc[2],
      rP0, rP1, rL, seed_lo, seed_hi};
}

// Hidden-state half of the confidence logit, hdot[b][k] = sum_j conf_w[j] *
// h[b][k][j], accumulated in fp64 by one wave (it does not depend on the
// drafted tokens).  bf16 rows with d % 8 == 0 are read 16 bytes per lane,
// four chunks in flight at a time.
__device__ __forceinline__ double hidden_dot(const uint16_t* row, const float* w, int d, int lane) {
  double acc = 0.0;
  if ((d & 7) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    const u32x4_t* r16 = reinterpret_cast<const u32x4_t*>(row);
    const f32x4_t* w16 = reinterpret_cast<const f32x4_t*>(w);
    const int nch = d >> 3;
    int c = lane;
    for (; c + 192 < nch; c += 256) {
      u32x4_t q[4];
      f32x4_t wa[4], wb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        q[u] = r16[c + 64 * u];
        wa[u] = w16[2 * (c + 64 * u)];
        wb[u] = w16[2 * (c + 64 * u) + 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc += double(wa[u][0]) * double(bf16_lo(q[u][0])) + double(wa[u][1]) * double(bf16_hi(q[u][0]));
        acc += double(wa[u][2]) * double(bf16_lo(q[u][1])) + double(wa[u][3]) * double(bf16_hi(q[u][1]));
        acc += double(wb[u][0]) * double(bf16_lo(q[u][2])) + double(wb[u][1]) * double(bf16_hi(q[u][2]));
        acc += double(wb[u][2]) * double(bf16_lo(q[u][3])) + double(wb[u][3]) * double(bf16_hi(q[u][3]));
      }
    }
    for (; c < nch; c += 64) {
      const u32x4_t q = r16[c];
      const f32x4_t wa = w16[2 * c], wb = w16[2 * c + 1];
      acc += double(wa[0]) * double(bf16_lo(q[0])) + double(wa[1]) * double(bf16_hi(q[0]));
      acc += double(wa[2]) * double(bf16_lo(q[1])) + double(wa[3]) * double(bf16_hi(q[1]));
      acc += double(wb[0]) * double(bf16_lo(q[2])) + double(wb[1]) * double(bf16_hi(q[2]));
      acc += double(wb[2]) * double(bf16_lo(q[3])) + double(wb[3]) * double(bf16_hi(q[3]));
    }
  } else {
    for (int j = lane; j < d; j += 64) acc += double(w[j]) * double(bf16_to_f32(row[j]));
  }
  return wave_sum_f64(acc);
}
__device__ __forceinline__ double hidden_dot(const float* row, const float* w, int d, int lane) {
  double acc = 0.0;
  for (int j = lane; j < d; j += 64) acc += double(w[j]) * double(row[j]);
  return wave_sum_f64(acc);
}

// FULL (bf16 only): V % 16 == 0, so every vocabulary tile is whole and rows
// are 32-byte aligned, and every wave owns either no tile or at least two,
// so the branch-free pair layout applies; otherwise the guarded path.
// Fused step tail: the ranking scheduler (rank_phase / rank_tail) over the
// survivals this launch has just written, on workgroups 0 .. G-1, then
// verify of every request in the workgroup that ran the scheduler's tail.
// `lds` is the U staging ring, idle once the last draft position is done.
static_assert(kFusedStepItems <= 2 * kRankThreads, "the fused step ranks at most two keys per thread");

template <int E, int K>
__device__ __forceinline__ void step_tail(const DraftParams& p, int wg, uint32_t* lds) {
  static_assert(K * kRankWaves <= 512, "counts fit the first 512 words");
  const int n = p.B * p.gamma;
  const int G = (n + K - 1) / K;
  const RankShared<K> sh{reinterpret_cast<int(*)[kRankWaves]>(lds), reinterpret_cast<long long*>(lds + 512),
                         reinterpret_cast<double*>(lds + 528), reinterpret_cast<int*>(lds + 544),
                         reinterpret_cast<int*>(lds + 552), lds + 576};
  if (wg >= G) return;
  if (!rank_phase<E, K, true>(wg, G, p.B, p.gamma, p.surv, p.t_step, p.n_min, p.n_count, p.sched_tickets,
                              p.sched_sorted, sh))
    return;
  rank_tail<E, K>(p.B, p.gamma, p.t_step, p.n_min, p.n_count, p.sched_tickets, p.sched_sorted, p.lens, p.m_out,
                  nullptr, sh);
  // verify: the longest prefix of the first lens[b] drafts that agrees with
  // the target, and the target's token after it; a request's loads are
  // issued eight positions at a time
  const int gamma = p.gamma;
  for (int b = threadIdx.x; b < p.B; b += kRankThreads) {
    const int L = min(rank_count(sh.counters, b, gamma), gamma);
    const int32_t* tk = p.tokens + size_t(b) * gamma;
    const int32_t* tg = p.target + size_t(b) * (gamma + 1);
    int a = 0;
    bool go = true;
    for (int k0 = 0; k0 < L && go; k0 += 8) {
      int32_t x[8], y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = min(k0 + u, gamma - 1);
        x[u] = load_dev(&tk[kk]);
        y[u] = tg[kk];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (go && k0 + u < L) {
          if (x[u] == y[u])
            ++a;
          else
            go = false;
        }
    }
    p.accepted[b] = a;
    p.bonus[b] = tg[a];
  }
}

// Small batches: the largest of the n keys row[0..n) (one per workgroup,
// each written once per call with a device-scope store, never 0 once
// written), read by a whole wave, which polls until every entry is there.
// The spin is bounded like a grid barrier's: past `limit` polls the error
// flag is raised, and a raised flag ends the wait.
__device__ __forceinline__ uint64_t small_max(const uint64_t* row, int n, int lane, unsigned int* err,
                                              unsigned int limit) {
  constexpr int PER = kMaxDraftWorkgroups / 64;
  uint32_t need = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < n) need |= 1u << i;
  uint64_t best = 0ull;
  unsigned int polls = 0;
  for (;;) {
    uint64_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = ((need >> i) & 1u) ? load_dev(row + lane + 64 * i) : 0ull;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (v[i] != 0ull) {
        best = v[i] > best ? v[i] : best;
        need &= ~(1u << i);
      }
    if (!__any(need != 0u)) break;
    if (++polls > limit) {
      if (lane == 0) store_dev(err, 1u);
      break;
    }
    if ((polls & 15u) == 0u && load_dev(err) != 0u) break;
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(best, m);
    best = o > best ? o : best;
  }
  return best;
}

// Small batches, Gumbel sampling: the unperturbed logit a workgroup stored
// (as ~bits, never 0) beside its winner key; one thread polls, bounded.
__device__ __forceinline__ float small_logit(const uint32_t* at, unsigned int* err, unsigned int limit) {
  uint32_t v = load_dev(at);
  unsigned int polls = 0;
  while (v == 0u) {
    if (++polls > limit || load_dev(err) != 0u) {
      store_dev(err, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = load_dev(at);
  }
  return __uint_as_float(~v);
}

// SMALL (B <= kSmallBatch, one request group): instead of the per-step
// arrival counter and the arg-max slots, every workgroup stores its winner
// key of each request once (wkeys), and a reader waits for the keys
// themselves: no atomic to complete before an arrival, no counter round
// trip, no separate slot read.
template <bool BF16, int R, int NW, int TPW, int GR, bool GUMBEL, bool FULL, bool RNN, bool STEP = false,
          bool SMALL = false>
__global__ __launch_bounds__(NW * 64, 1) void markov_draft_kernel(DraftParams p) {
  static_assert(!STEP || (FULL && !RNN && NW * 64 == kRankThreads), "the fused step runs on the whole-tile kernel");
  static_assert(!SMALL || (!STEP && kSmallBatch <= 2 * NW && kSmallBatch <= 16),
                "at most two requests per wave, one group; no fused step");
  static_assert(!RNN || BF16, "the RNN head is built for bf16 storage");
  typedef Elem<BF16> E;
  typedef typename E::store_t st_t;
  typedef typename E::frag_t frag_t;
  constexpr int NKS = R / E::KS;
  typedef ELayout<BF16, R> EL;
  constexpr int LDE = EL::LDE;
  constexpr int NT = NW * 64;
  constexpr int CHUNKS = int(R * sizeof(st_t)) / 16;      // 16-byte pieces per W1 row
  static_assert(R % E::KS == 0, "rank must be a multiple of the MFMA K step");

  constexpr int CMAX = TPW * NW * 16;                       // widest column slice of a workgroup
  constexpr int SLD = CMAX + (BF16 ? 8 : 4);                // W2 staging row stride (16-byte multiple)
  constexpr int EBUF = (GR * LDE > E::KS * SLD) ? GR * LDE : E::KS * SLD;
  // the embedding buffer and the U staging ring share one array, the
  // embeddings first: B-fragment reads then address them with the LDS
  // instruction's immediate offset
  constexpr int EWORDS = int((EBUF * sizeof(st_t) + 15) / 16) * 4;
  constexpr int UWORDS = FULL ? NW * 3 * 768 : 4;
  __shared__ __attribute__((aligned(16))) uint32_t lds_eu[EWORDS + UWORDS];
  st_t* const lds_e = reinterpret_cast<st_t*>(lds_eu);
  __shared__ uint64_t lds_key[GR];
  __shared__ float lds_z[NW][GR];
  __shared__ int lds_x[GR];
  __shared__ uint64_t lds_sk[SMALL ? 2 * NW : 1];   // SMALL: the previous step's key of each request
  __shared__ double lds_hd[GR];
  __shared__ float lds_S[kMaxOwnedRows];
  __shared__ float lds_we[R];   // confidence weights of the Markov-embedding half
  __shared__ float lds_dec[RNN ? R : 1];                // RNN head: decay
  __shared__ double lds_ce[RNN ? kMaxOwnedRows : 1];    // RNN head: embedding half of owned rows' confidence dots
  // U staging ring of the whole-tile path: three slots of 3 KB per wave
  uint32_t* const lds_u = lds_eu + EWORDS;

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

  // A workspace left by a completed call has zero barrier counters; before
  // this workgroup's first arrival at most nwg - 1 others can have arrived.
  if (tid == 0 && load_dev(&p.bar[0]) >= unsigned(nwg)) store_dev(&p.ctrl[1], 2u);
  // (SMALL: likewise its winner keys are all zero; this workgroup's entry of
  // the first position and request is written by it alone, after this read)
  if constexpr (SMALL)
    if (tid == 0 && load_dev(&p.wkeys[wg]) != 0ull) store_dev(&p.ctrl[1], 2u);

  // hdot for every (owned request, position): one (b, k) per wave at a time.
  if constexpr (!FULL) {
    const st_t* h = static_cast<const st_t*>(p.h);
    const int nown = (B > wg) ? (B - 1 - wg) / nwg + 1 : 0;
    for (int q = wave; q < nown * gamma; q += NW) {
      const int b = wg + (q / gamma) * nwg, kk = q % gamma;
      const double v = hidden_dot(h + (size_t(b) * gamma + kk) * p.d, p.conf_w, p.d, lane);
      if (lane == 0) store_dev(&p.hdot[size_t(b) * gamma + kk], v);
    }
    wait_vmem();   // visible to the other waves after the next workgroup barrier
  }

  // W2 slice of this wave in MFMA A-operand layout, resident for the call.
  // The workgroup's columns [wg_lo*16, wg_hi*16) of W2 are staged through
  // LDS (the embedding buffer is still free) a chunk of K rows at a time with
  // coalesced row loads; each wave then picks its fragments out of LDS.
  frag_t A[TPW][NKS];
  if constexpr (!FULL) {
    constexpr int KCH0 = int(EBUF / SLD);
    constexpr int KCH = (KCH0 >= R) ? R : (KCH0 / E::KS) * E::KS;   // K rows per chunk
    static_assert(KCH >= E::KS, "staging buffer too small");
    st_t* stage = lds_e;
    const st_t* W2 = static_cast<const st_t*>(p.W2);
    const int col0 = wg_lo * 16;
    const int ncols = wg_nt * 16;
    for (int kc = 0; kc < R; kc += KCH) {
      const int kn = min(KCH, R - kc);
      constexpr int EPC = 16 / int(sizeof(st_t));             // elements per 16-byte chunk
      if (FULL && (V % EPC) == 0) {
        // whole tiles, 16-byte aligned rows: 16-byte loads, eight in flight
        const int cpr = ncols / EPC;                         // chunks per staged row
        const int nch = kn * cpr;
        for (int i0 = tid; i0 < nch; i0 += 8 * NT) {
          u32x4_t q[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NT;
            if (i < nch) {
              const int kr = i / cpr, c = i - kr * cpr;
              q[u] = *reinterpret_cast<const u32x4_t*>(W2 + size_t(kc + kr) * V + col0 + c * EPC);
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * NT;
            if (i < nch) {
              const int kr = i / cpr, c = i - kr * cpr;
              *reinterpret_cast<u32x4_t*>(stage + kr * SLD + c * EPC) = q[u];
            }
          }
        }
      } else {
        for (int i = tid; i < kn * ncols; i += NT) {
          const int kr = i / ncols, c = i - kr * ncols;
          const int v = col0 + c;
          stage[kr * SLD + c] = (v < V) ? W2[size_t(kc + kr) * V + v] : st_t(0);
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (nt > 0) {   // spare slots repeat columns the wave owns (pair layout when FULL)
          const int c = (w_lo - wg_lo) * 16 +
                        (FULL ? pair_col(t, li >> 2, nt, TPW) + (li & 3) : min(t, nt - 1) * 16 + li);
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
  if constexpr (FULL) {
    // Whole-tile path: W2 in chunks of one K step (32 rows) staged
    // alternately through the embedding buffer and the U staging ring (both
    // still free), with the global loads of the next two chunks in flight
    // while a chunk is picked apart, one workgroup barrier per chunk.  The
    // hidden-state dots run while the first two chunks load: the confidence
    // weights are staged in the U ring first, and each wave keeps every
    // 16-byte piece of a (b, k) row in flight at once.
    constexpr int EPC = 8;                                    // bf16 per 16-byte piece
    constexpr int PER = (E::KS * (CMAX / EPC) + NT - 1) / NT; // pieces per thread and chunk
    static_assert(E::KS * SLD <= EBUF && E::KS * SLD * int(sizeof(st_t)) <= UWORDS * int(sizeof(uint32_t)),
                  "W2 staging buffers");
    const st_t* W2 = static_cast<const st_t*>(p.W2);
    const int col0 = wg_lo * 16;
    const int cpr = wg_nt * 16 / EPC;                         // pieces per staged row
    const int npc = E::KS * cpr;                              // pieces per chunk
    // this thread's pieces of a chunk: element offsets in W2 (from the chunk's
    // first row) and in the staging buffer (-1: none; such a slot loads the
    // chunk's first piece again, unconditionally, so that the loads need no
    // branches and stay in flight together, and stores nothing)
    int goff[PER], loff[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      const int kr = i / cpr, c = i - kr * cpr;
      goff[u] = (i < npc) ? kr * V + col0 + c * EPC : col0;
      loff[u] = (i < npc) ? kr * SLD + c * EPC : -1;
    }
    auto issue = [&](u32x4_t (&q)[PER], int k0) {
      const st_t* base = W2 + size_t(k0) * V;
#pragma unroll
      for (int u = 0; u < PER; ++u) q[u] = *reinterpret_cast<const u32x4_t*>(base + goff[u]);
    };
    auto put = [&](const u32x4_t (&q)[PER], st_t* stg) {
#pragma unroll
      for (int u = 0; u < PER; ++u)
        if (loff[u] >= 0) *reinterpret_cast<u32x4_t*>(stg + loff[u]) = q[u];
    };
    u32x4_t qa[PER], qb[PER];
    issue(qa, 0);
    if (NKS > 1) issue(qb, E::KS);

    const st_t* h = static_cast<const st_t*>(p.h);
    const int nown = (B > wg) ? (B - 1 - wg) / nwg + 1 : 0;
    constexpr int HJ = 16;                                     // 16-byte pieces per lane and row
    const int hpc = p.d / 8;                                   // pieces per row
    // (d = 0, where h may be null and every dot is 0, takes the generic loop, which reads nothing)
    const bool fast_hd = p.d > 0 && (p.d % 8) == 0 && hpc <= 64 * HJ &&
                         p.d <= UWORDS && (reinterpret_cast<uintptr_t>(h) & 15) == 0;
    if (fast_hd) {
      float* wl = reinterpret_cast<float*>(lds_u);
      for (int i = tid; i < p.d; i += NT) wl[i] = p.conf_w[i];
      __syncthreads();
      for (int q = wave; q < nown * gamma; q += NW) {
        const size_t hrow = size_t(wg + (q / gamma) * nwg) * gamma + q % gamma;
        const u32x4_t* r = reinterpret_cast<const u32x4_t*>(h + hrow * p.d);
        u32x4_t x[HJ];   // loaded unconditionally (clamped piece index), used where c < hpc
#pragma unroll
        for (int j = 0; j < HJ; ++j) x[j] = r[min(lane + 64 * j, hpc - 1)];
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
          const int c = lane + 64 * j;
          if (c < hpc) {
            const f32x4_t wa = *reinterpret_cast<const f32x4_t*>(wl + 8 * c);
            const f32x4_t wb = *reinterpret_cast<const f32x4_t*>(wl + 8 * c + 4);
            acc += double(wa[0]) * double(bf16_lo(x[j][0])) + double(wa[1]) * double(bf16_hi(x[j][0]));
            acc += double(wa[2]) * double(bf16_lo(x[j][1])) + double(wa[3]) * double(bf16_hi(x[j][1]));
            acc += double(wb[0]) * double(bf16_lo(x[j][2])) + double(wb[1]) * double(bf16_hi(x[j][2]));
            acc += double(wb[2]) * double(bf16_lo(x[j][3])) + double(wb[3]) * double(bf16_hi(x[j][3]));
          }
        }
        acc = wave_sum_f64(acc);
        if (lane == 0) store_dev(&p.hdot[hrow], acc);
      }
    } else {
      for (int q = wave; q < nown * gamma; q += NW) {
        const int b = wg + (q / gamma) * nwg, kk = q % gamma;
        const double v = hidden_dot(h + (size_t(b) * gamma + kk) * p.d, p.conf_w, p.d, lane);
        if (lane == 0) store_dev(&p.hdot[size_t(b) * gamma + kk], v);
      }
    }
    // (the hidden-state dots are visible to the other waves after the
    // workgroup barriers below: wait_vmem orders the stores first)
    wait_vmem();

#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      st_t* stg = (ks & 1) ? reinterpret_cast<st_t*>(lds_u) : lds_e;
      if (ks & 1) {
        put(qb, stg);
        if (ks + 2 < NKS) issue(qb, (ks + 2) * E::KS);
      } else {
        put(qa, stg);
        if (ks + 2 < NKS) issue(qa, (ks + 2) * E::KS);
      }
      __syncthreads();   // chunk ks staged; the buffer's previous chunk was picked apart before the last barrier
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (nt > 0) {   // spare slots repeat columns the wave owns (pair layout)
          const int c = (w_lo - wg_lo) * 16 + pair_col(t, li >> 2, nt, TPW) + (li & 3);
          const int kr = E::KPL * lg;
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = uint32_t(stg[(kr + 2 * i) * SLD + c]) | (uint32_t(stg[(kr + 2 * i + 1) * SLD + c]) << 16);
          A[t][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
        }
      }
    }
    __syncthreads();   // both buffers are free again
  }
  for (int i = tid; i < kMaxOwnedRows; i += NT) lds_S[i] = 1.0f;
  for (int i = tid; i < R; i += NT) lds_we[i] = p.conf_w[p.d + i];
  if constexpr (RNN)
    for (int i = tid; i < R; i += NT) lds_dec[i] = p.decay[i];
  for (int i = tid; i < GR; i += NT) lds_key[i] = 0ull;

  const st_t* U = static_cast<const st_t*>(p.U);
  const st_t* W1 = static_cast<const st_t*>(p.W1);
  const int grs = p.grs;
  const int ngroups = (B + grs - 1) / grs;

  // Publishes the drafted token of step kk (1-based) for a row this
  // workgroup owns; its logit comes from the workgroup whose tiles hold it.
  auto emit = [&](int b, int kk, uint64_t key) {
    uint32_t x = key_index(key);
    if (key == 0ull || x >= uint32_t(V)) x = uint32_t(V - 1);   // only after a barrier timeout
    const int owner = part_of(int(x >> 4), p.tiles, nwg);
    float z;
    if constexpr (SMALL && !GUMBEL)
      z = key_value(key);   // the greedy key carries the logit itself
    else if constexpr (SMALL)
      z = small_logit(&p.wz[(size_t(kk - 1) * B + b) * nwg + owner], &p.ctrl[1], p.spin_limit);
    else
      z = __hip_atomic_load(&p.zpart[(size_t((kk & 1) * nwg + owner)) * B + b], __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (STEP)   // read by the fused verify of another workgroup
      store_dev(&p.tokens[size_t(b) * gamma + kk - 1], int32_t(x));
    else
      p.tokens[size_t(b) * gamma + kk - 1] = int32_t(x);
    p.logit[size_t(b) * gamma + kk - 1] = z;
    return int(x);
  };

  // Requests are processed in groups of grs rows, group by group within a
  // step.  Each group has its own arrival counter: step k of group g needs
  // only the tokens of step k-1 of group g, so while the slowest workgroups
  // finish a group, the others already compute the next group instead of
  // waiting.  A workgroup's arrival for a group is issued after the next
  // group's gather, whose completion wait also covers the publishing atomics
  // (with a single group it is issued at once).
  //
  // The next group's first three request tiles of U are loaded ahead of
  // time, before the slot reads and the gather that precede their use.
  typedef TileWork<BF16, R, TPW, GR, GUMBEL, TPW, !FULL> Work;
  // (RNN head: the lane's addressing constants are recomputed per unit, the
  // lane index being made opaque, instead of being kept live across the
  // unit's state update, where they would spill to memory)
  auto work = [&](int k, int g0, int rows) {
    int ln = lane;
    if constexpr (RNN) asm volatile("" : "+v"(ln));
    return make_work<BF16, R, TPW, GR, GUMBEL, TPW, !FULL>(A, lds_e, U, g0, rows, B, gamma, k, V, w_lo, nt,
                                                           p.vec_ok, ln & 15, ln >> 4, p.seed_lo, p.seed_hi, lds_key,
                                                           lds_z[wave], lds_u + (FULL ? wave * 3 * 768 : 0));
  };
  auto bar = [&](int g) { return p.bar + size_t(g) * kBarStride; };
  typename Work::Buf pf0, pf1, pf2;
  // (the whole-tile RNN kernel stages the previous states in the U ring at
  // the start of a unit, so it loads a unit's first U tiles after that)
  constexpr bool RING_STATE = RNN && FULL;
  if (nt > 0 && !RING_STATE) work(1, 0, min(grs, B)).prefetch(pf0, pf1, pf2);
  int pending = -1;   // group whose arrival is still to be issued

  for (int k = 1; k <= gamma; ++k) {
    for (int grp = 0; grp < ngroups; ++grp) {
      const int g0 = grp * grs;
      const int rows = min(grs, B - g0);

      // tokens of step k-1 of this group are final once every workgroup has arrived
      // (SMALL: once every workgroup's key of each request is there)
      if constexpr (SMALL) {
        if (k > 1) {
          // wave w takes rows w and w + NW
          if (wave < rows) {
            const uint64_t key =
                small_max(&p.wkeys[(size_t(k - 2) * B + g0 + wave) * nwg], nwg, lane, &p.ctrl[1], p.spin_limit);
            if (lane == 0) lds_sk[wave] = key;
          }
          if (wave + NW < rows) {
            const uint64_t key = small_max(&p.wkeys[(size_t(k - 2) * B + g0 + wave + NW) * nwg], nwg, lane,
                                           &p.ctrl[1], p.spin_limit);
            if (lane == 0) lds_sk[wave + NW] = key;
          }
          __syncthreads();
        }
      } else if (k > 1) {
        grid_wait(bar(grp), &p.ctrl[1], unsigned(k - 1) * unsigned(nwg), p.spin_limit);
      }

      // 1. previous tokens of the group's rows
      uint64_t own_key = 0ull;   // key of step k-1 for a row this workgroup owns (emitted below)
      bool own = false;
      if (tid < rows) {
        const int b = g0 + tid;
        own = (b % nwg) == wg;
        int x;
        if (k == 1) {
          x = min(max(int(p.anchor[b]), 0), V - 1);
        } else {
          const uint64_t key = SMALL ? lds_sk[tid]
                                     : __hip_atomic_load(&p.slots[size_t(k - 2) * B + b], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
          own_key = key;
          x = int(key_index(key));
          if (key == 0ull || x >= V || x < 0) x = V - 1;
        }
        lds_x[tid] = x;
        if (own) lds_hd[tid] = load_dev(&p.hdot[size_t(b) * gamma + (k - 1)]);
      }
      __syncthreads();

      // 2. gather e = W1[x_{k-1}] for the group's rows (rounded up to whole request tiles) into LDS
      const int rows16 = (rows + 15) & ~15;
      if constexpr (BF16) {
        // one 16-byte direct-to-LDS load per lane, 64 / CPR rows per instruction, all in flight at once;
        // lane -> (row, physical chunk p) holds logical chunk p ^ swz(row); rows past the group read row 0
        constexpr int CPR = EL::CPR;
        constexpr int RPI = 64 / CPR;
        static_assert(RPI * CPR == 64 && 16 % RPI == 0, "gather instruction shape");
        for (int i = wave; i < rows16 / RPI; i += NW) {
          const int row = i * RPI + lane / CPR;
          const int x = row < rows ? lds_x[row] : 0;
          const int c = (lane % CPR) ^ EL::swz(row);
          load_lds16(W1 + size_t(x) * R + c * 8, lds_e + i * RPI * R);
        }
      } else {
        // eight 16-byte loads in flight per thread before their LDS stores
        for (int c0 = tid; c0 < rows16 * CHUNKS; c0 += 8 * NT) {
          u32x4_t val[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int c = c0 + u * NT;
            const int row = c / CHUNKS, ch = c - row * CHUNKS;
            val[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (c < rows16 * CHUNKS && row < rows)
              val[u] = *reinterpret_cast<const u32x4_t*>(
                  reinterpret_cast<const char*>(W1 + size_t(lds_x[row]) * R) + ch * 16);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int c = c0 + u * NT;
            const int row = c / CHUNKS, ch = c - row * CHUNKS;
            if (c < rows16 * CHUNKS)
              *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(lds_e + row * LDE) + ch * 16) = val[u];
          }
        }
      }
      // whole-tile RNN kernel: the group's previous states s_{k-1} (rows
      // contiguous in the state buffer) into the U ring, 16 bytes per lane,
      // with the gather (device scope: written by the rows' owners before
      // their arrival)
      // Each wave takes the rows it updates (wave, wave + NW, ...) into its
      // own part of the ring (its three U slots), row after row.
      if constexpr (RING_STATE) {
        if (k > 1) {
          const char* src = reinterpret_cast<const char*>(p.state + (size_t((k - 1) & 1) * B + g0) * R);
          const int nrw = (rows > wave) ? (rows - 1 - wave) / NW + 1 : 0;   // this wave's rows
          const int nbytes = nrw * R * 2;
          char* region = reinterpret_cast<char*>(lds_u + wave * 3 * 768);
          for (int i = 0; i * 1024 < nbytes; ++i) {
            const int off = i * 1024 + lane * 16;
            const int rr = off / (R * 2);
            if (off < nbytes)
              load_lds16_dev(src + size_t(wave + rr * NW) * (R * 2) + (off - rr * R * 2), region + i * 1024);
          }
        }
      }
      // outputs of step k-1 for owned rows, overlapping the gather
      if (own && k > 1) emit(g0 + tid, k - 1, own_key);
      wait_vmem();   // this wave's direct-to-LDS loads have landed (and its earlier atomics are done)
      __syncthreads();
      if (pending >= 0) {
        if (tid == 0) __hip_atomic_fetch_add(bar(pending), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pending = -1;
      }

      // RNN head: the confidence head keeps the embedding e of the previous
      // token as its input, so its embedding half is taken now; then the
      // rows' states s_k = bf16(a s_{k-1} + e) replace e in LDS as the
      // B operand, and each row's owner publishes its state for step k + 1.
      if constexpr (RING_STATE) {
        // Whole-tile kernel: wave w owns rows w, w + NW, ... of the group;
        // for each it first takes the embedding half of the confidence dot
        // (owned requests), then replaces e by the state (program order
        // within the wave: no workgroup barrier in between), then stages its
        // first U tiles into its part of the ring, whose states it has read.
        const int j_lo = (g0 > wg) ? (g0 - wg + nwg - 1) / nwg : 0;
        constexpr int PPR = R / 4;                                 // 4-channel pieces per row
        const uint64_t* region = reinterpret_cast<const uint64_t*>(lds_u + wave * 3 * 768);
        uint64_t* dst = reinterpret_cast<uint64_t*>(p.state + size_t(k & 1) * B * R);
        for (int rr = 0; wave + rr * NW < rows; ++rr) {
          const int row = wave + rr * NW;
          const int b = g0 + row;
          const bool owned = (b % nwg) == wg;
          if (owned) {
            double acc = 0.0;
            for (int i = lane; i < R; i += 64) acc += double(lds_we[i]) * double(to_f32(lds_e[EL::at(row, i)]));
            acc = wave_sum_f64(acc);
            if (lane == 0) lds_ce[(b - wg) / nwg - j_lo] = acc;
          }
          for (int q = lane; q < PPR; q += 64) {
            st_t* ep = lds_e + EL::at(row, 4 * q);
            const uint64_t sp = (k > 1) ? region[rr * PPR + q] : 0ull;
            const u32x2_t sv = rnn_step4(&lds_dec[4 * q], __builtin_bit_cast(u32x2_t, sp),
                                         *reinterpret_cast<const u32x2_t*>(ep));
            *reinterpret_cast<u32x2_t*>(ep) = sv;
            if (owned) store_dev(dst + (size_t(b) * R + 4 * q) / 4, __builtin_bit_cast(uint64_t, sv));
          }
        }
        lds_wait();   // the states have been read before the ring is refilled
        if (nt > 0) work(k, g0, rows).prefetch(pf0, pf1, pf2);
        __syncthreads();   // every row's state is in place (B operand) and the confidence halves are visible
      } else if constexpr (RNN) {
        const int j_lo = (g0 > wg) ? (g0 - wg + nwg - 1) / nwg : 0;
        const int j_hi = (g0 + rows > wg) ? (g0 + rows - wg + nwg - 1) / nwg : 0;
        for (int j = j_lo + wave; j < j_hi; j += NW) {
          const int row = wg + j * nwg - g0;
          double acc = 0.0;
          for (int i = lane; i < R; i += 64) acc += double(lds_we[i]) * double(to_f32(lds_e[EL::at(row, i)]));
          acc = wave_sum_f64(acc);
          if (lane == 0) lds_ce[j - j_lo] = acc;
        }
        __syncthreads();   // every wave has read e before the states replace it
        // Guarded kernel: this thread's pieces (4 channels, 8 bytes) of the
        // previous states s_{k-1} from the state buffer, four in flight at a
        // time (device scope: written by the rows' owners before their
        // arrival); s_0 = 0
        constexpr int PPR = R / 4;                                // pieces per row
        constexpr int SPT = (GR * PPR + NT - 1) / NT;             // pieces per thread
        constexpr int BATCH = SPT < 4 ? SPT : 4;
        const uint64_t* src = reinterpret_cast<const uint64_t*>(p.state + size_t((k - 1) & 1) * B * R);
        uint64_t* dst = reinterpret_cast<uint64_t*>(p.state + size_t(k & 1) * B * R);
#pragma unroll 1
        for (int u0 = 0; u0 < SPT; u0 += BATCH) {
          uint64_t sprev[BATCH];
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int q = min(tid + (u0 + u) * NT, rows * PPR - 1);   // clamped: always a valid address
            const int row = q / PPR;
            sprev[u] = (k > 1) ? load_dev(src + (size_t(g0 + row) * R + (q - row * PPR) * 4) / 4) : 0ull;
          }
#pragma unroll
          for (int u = 0; u < BATCH; ++u) {
            const int q = tid + (u0 + u) * NT;
            if (q < rows * PPR) {
              const int row = q / PPR, c = (q - row * PPR) * 4;
              st_t* ep = lds_e + EL::at(row, c);
              const u32x2_t sv = rnn_step4(&lds_dec[c], __builtin_bit_cast(u32x2_t, sprev[u]),
                                           *reinterpret_cast<const u32x2_t*>(ep));
              *reinterpret_cast<u32x2_t*>(ep) = sv;
              if ((g0 + row) % nwg == wg)
                store_dev(dst + (size_t(g0 + row) * R + c) / 4, __builtin_bit_cast(uint64_t, sv));
            }
          }
        }
        __syncthreads();
      }

      // 4. z = U_k + e W2 on MFMA, argmax in registers, per request tile
      if (nt > 0) work(k, g0, rows).run(pf0, pf1, pf2);

      // 3. confidence + STS + survival for the rows this workgroup owns (after the
      //    MFMA phase: it only needs e, which stays in LDS until the next gather)
      {
        const int j_lo = (g0 > wg) ? (g0 - wg + nwg - 1) / nwg : 0;
        const int j_hi = (g0 + rows > wg) ? (g0 + rows - wg + nwg - 1) / nwg : 0;
        for (int j = j_lo + wave; j < j_hi; j += NW) {
          const int b = wg + j * nwg;
          const int row = b - g0;
          double acc = 0.0;
          if constexpr (RNN) {
            acc = lds_ce[j - j_lo];
          } else {
            for (int i = lane; i < R; i += 64) acc += double(lds_we[i]) * double(to_f32(lds_e[EL::at(row, i)]));
            acc = wave_sum_f64(acc);
          }
          if (lane == 0) {
            const double ell = double(p.conf_b) + (lds_hd[row] + acc);
            const double c = 1.0 / (1.0 + exp(-ell / double(p.sts_T[k - 1])));
            const float cf = float(c);
            const float S = lds_S[j] * cf;
            lds_S[j] = S;
            p.conf[size_t(b) * gamma + k - 1] = cf;
            if constexpr (STEP)   // ranked by every workgroup of the fused step
              store_dev(&p.surv[size_t(b) * gamma + k - 1], S);
            else
              p.surv[size_t(b) * gamma + k - 1] = S;
          }
        }
      }

      // (SMALL RNN head: the owners' state stores of this unit complete
      // before any key of it is stored, so a reader that has every key of
      // the step also reads the states)
      if constexpr (SMALL && RNN) wait_vmem();
      __syncthreads();

      // 5. publish this workgroup's winner of every row of the group
      if (tid < rows) {
        const uint64_t key = lds_key[tid];
        lds_key[tid] = 0ull;
        if constexpr (SMALL) {
          // every workgroup writes an entry (1, below any real key, when it has no candidate)
          const size_t e = (size_t(k - 1) * B + g0 + tid) * nwg + wg;
          if constexpr (GUMBEL) {
            uint32_t zb = 1u;
            if (key != 0ull) {
              const int w = part_of(int(key_index(key) >> 4) - wg_lo, wg_nt, NW);
              zb = ~__float_as_uint(lds_z[w][tid]);
              zb = zb ? zb : 1u;
            }
            store_dev(&p.wz[e], zb);
          }
          store_dev(&p.wkeys[e], key != 0ull ? key : uint64_t(1));
        } else if (key != 0ull) {
          const int b = g0 + tid;
          __hip_atomic_fetch_max(reinterpret_cast<unsigned long long*>(&p.slots[size_t(k - 1) * B + b]),
                                 (unsigned long long)key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int tile = int(key_index(key) >> 4);
          const int w = part_of(tile - wg_lo, wg_nt, NW);
          store_dev(&p.zpart[(size_t((k & 1) * nwg + wg)) * B + b], GUMBEL ? lds_z[w][tid] : key_value(key));
        }
      }
      const bool last = (k == gamma) && (grp + 1 == ngroups);
      if constexpr (SMALL) {
        __syncthreads();
      } else if (ngroups == 1 || last) {
        grid_arrive(bar(grp));
      } else {
        pending = grp;
        __syncthreads();
      }
      if (!last && nt > 0) {
        const int nk = (grp + 1 < ngroups) ? k : k + 1;
        const int ng0 = (grp + 1 < ngroups) ? g0 + grs : 0;
        if constexpr (!RING_STATE) work(nk, ng0, min(grs, B - ng0)).prefetch(pf0, pf1, pf2);
      }
    }
  }
  // every group's last step is final before its outputs are read
  if constexpr (SMALL) {
    // wave w takes this workgroup's owned requests number w and w + NW,
    // wg + w * nwg and wg + (w + NW) * nwg
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int bw = wg + (wave + h * NW) * nwg;
      if (bw < B) {
        const uint64_t key = small_max(&p.wkeys[(size_t(gamma - 1) * B + bw) * nwg], nwg, lane, &p.ctrl[1],
                                       p.spin_limit);
        if (lane == 0) lds_sk[wave + h * NW] = key;
      }
    }
    __syncthreads();
  } else {
    for (int g = 0; g < ngroups; ++g) grid_wait(bar(g), &p.ctrl[1], unsigned(gamma) * unsigned(nwg), p.spin_limit);
  }

  // outputs of the last step; a failed synchronisation marks every token -1
  const bool failed = load_dev(&p.ctrl[1]) != 0u;
  for (int b = wg + tid * nwg; b < B; b += NT * nwg) {
    const uint64_t key = SMALL ? lds_sk[tid] : load_dev(&p.slots[size_t(gamma - 1) * B + b]);
    emit(b, gamma, key);
    if (failed)
      for (int kk = 0; kk < gamma; ++kk) {
        if constexpr (STEP)
          store_dev(&p.tokens[size_t(b) * gamma + kk], -1);
        else
          p.tokens[size_t(b) * gamma + kk] = -1;
      }
  }

  if constexpr (STEP) {
    __syncthreads();   // the staging ring is idle from here on
    if (p.sched_e == 1)
      step_tail<1, 16>(p, wg, lds_u);
    else
      step_tail<2, 16>(p, wg, lds_u);
  }

  // Leave the workspace as a fresh call expects it: once every workgroup is
  // done reading, workgroup 0 clears the argmax slots and the counters.
  wait_vmem();
  __syncthreads();
  if (tid == 0) __hip_atomic_fetch_add(&p.ctrl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wg == 0) {
    if (tid == 0) {
      unsigned int polls = 0;
      while (load_dev(&p.ctrl[2]) < unsigned(nwg) && ++polls <= p.spin_limit) __builtin_amdgcn_s_sleep(1);
    }
    __syncthreads();
    const long long nslots = (long long)gamma * B;
    for (long long i = tid; i < nslots; i += NT) store_dev(&p.slots[i], uint64_t(0));
    if constexpr (SMALL) {
      const long long nw = nslots * nwg;
      for (long long i = tid; i < nw; i += NT) {
        store_dev(&p.wkeys[i], uint64_t(0));
        if constexpr (GUMBEL) store_dev(&p.wz[i], 0u);
      }
    }
    for (int g = tid; g < ngroups; g += NT) store_dev(bar(g), 0u);
    if (tid == 0) {
      store_dev(&p.ctrl[1], 0u);
      store_dev(&p.ctrl[2], 0u);
    }
  }
}

struct KernelChoice {
  const void* fn;
  int threads;
  int tpw;
};

constexpr int kDraftWaves = 8;

template <bool BF16, int R, bool G, bool RNN>
KernelChoice pick_r(bool full, int tiles_per_wave, bool step, bool small) {
  constexpr int NW = kDraftWaves, GR = kMaxGroupRows;
  constexpr int TPW = BF16 ? 5 : 4;
  // small batches: the SMALL instances (bf16 at rank 256, both heads; fp32 at rank 16)
  if constexpr ((BF16 && R == 256) || (!BF16 && R == 16 && !RNN)) {
    if (small) {   // (never with the fused step)
      if constexpr (BF16) {
        if (full && tiles_per_wave <= 4)
          return KernelChoice{
              reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, 4, GR, G, true, RNN, false, true>),
              NW * 64, 4};
        if (full)
          return KernelChoice{
              reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, TPW, GR, G, true, RNN, false, true>),
              NW * 64, TPW};
      }
      return KernelChoice{
          reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, TPW, GR, G, false, RNN, false, true>),
          NW * 64, TPW};
    }
  }
  if constexpr (BF16 && R == 256 && !RNN) {
    // the fused draft-schedule-verify step (whole tiles only)
    if (step && full) {
      if (tiles_per_wave <= 4)
        return KernelChoice{
            reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, 4, GR, G, true, RNN, true>), NW * 64, 4};
      return KernelChoice{
          reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, TPW, GR, G, true, RNN, true>), NW * 64, TPW};
    }
  }
  if constexpr (BF16) {
    // rank 256, Markov head: four tiles per wave when they cover the
    // vocabulary (W2 then takes 128 instead of 160 registers per lane and no
    // wave computes a fifth, repeated slot)
    if constexpr (R == 256 && !RNN)
      if (full && tiles_per_wave <= 4)
        return KernelChoice{reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, 4, GR, G, true, RNN>),
                            NW * 64, 4};
    if (full)
      return KernelChoice{reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, TPW, GR, G, true, RNN>),
                          NW * 64, TPW};
  }
  return KernelChoice{reinterpret_cast<const void*>(&markov_draft_kernel<BF16, R, NW, TPW, GR, G, false, RNN>),
                      NW * 64, TPW};
}

template <bool G>
bool pick(bool bf16, int r, bool full, bool rnn, int tpw_need, KernelChoice* out, bool step = false,
          bool small = false) {
  const int n = tpw_need;
  if (bf16) {
    switch (r) {
      case 32: *out = rnn ? pick_r<true, 32, G, true>(full, n, false, false) : pick_r<true, 32, G, false>(full, n, false, false); return true;
      case 64: *out = rnn ? pick_r<true, 64, G, true>(full, n, false, false) : pick_r<true, 64, G, false>(full, n, false, false); return true;
      case 128: *out = rnn ? pick_r<true, 128, G, true>(full, n, false, false) : pick_r<true, 128, G, false>(full, n, false, false); return true;
      case 256: *out = rnn ? pick_r<true, 256, G, true>(full, n, false, small) : pick_r<true, 256, G, false>(full, n, step, small); return true;
      default: return false;
    }
  }
  if (rnn) return false;
  switch (r) {
    case 16: *out = pick_r<false, 16, G, false>(full, n, false, small); return true;
    case 32: *out = pick_r<false, 32, G, false>(full, n, false, false); return true;
    case 64: *out = pick_r<false, 64, G, false>(full, n, false, false); return true;
    default: return false;
  }
}

// whether pick() has SMALL instances for this shape
inline bool small_kernel_exists(bool bf16, int r, bool rnn) { return bf16 ? r == 256 : (r == 16 && !rnn); }

// Scratch of the allocation-free entry point (dspark_markov_draft_noalloc):
// the draft workspace as a file-scope device array, one copy per GPU for the
// life of the process.  Host code never passes `scratch` itself to a kernel
// (its host-side name is not a device address); it takes the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

// Zero-fill of the scratch at its set-up (a kernel, not a memset node).
__global__ __launch_bounds__(256) void scratch_clear_kernel(u32x4_t* p, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = u32x4_t{0u, 0u, 0u, 0u};
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

DraftWorkspace draft_workspace_layout(int B, int gamma, int r_state) {
  DraftWorkspace w;
  size_t off = 0;
  w.ctrl = off;
  off += 256;
  w.bar = off;
  off = align256(off + size_t((B + 15) / 16) * kBarStride * sizeof(unsigned int));
  w.slots = off;
  off = align256(off + size_t(gamma) * B * sizeof(uint64_t));
  const size_t small_entries = (B <= kSmallBatch) ? size_t(gamma) * B * kMaxDraftWorkgroups : 0;
  w.wkeys = off;
  off = align256(off + small_entries * sizeof(uint64_t));
  w.wz = off;
  off = align256(off + small_entries * sizeof(uint32_t));
  w.zpart = off;
  off = align256(off + size_t(2) * kMaxDraftWorkgroups * B * sizeof(float));
  w.hdot = off;
  off = align256(off + size_t(B) * gamma * sizeof(double));
  w.state = off;
  off = align256(off + size_t(2) * B * size_t(r_state) * sizeof(uint16_t));
  w.total = off;
  return w;
}

hipError_t launch_markov_draft(const DraftArgs& a, hipStream_t stream, const char** unsupported, bool* fused) {
  *unsupported = nullptr;
  if (fused) *fused = false;
  KernelChoice kc;
  const bool rnn = a.decay != nullptr;
  // small batches synchronise through per-workgroup winner keys (SMALL kernels)
  const bool small = a.B <= kSmallBatch && small_kernel_exists(a.bf16, a.r, rnn);
  if (!(a.gumbel ? pick<true>(a.bf16, a.r, false, rnn, 0, &kc, false, small)
                 : pick<false>(a.bf16, a.r, false, rnn, 0, &kc, false, small))) {
    *unsupported = rnn ? "the RNN head supports bf16 storage with r in {32, 64, 128, 256}"
                       : a.bf16 ? "bf16 drafting supports r in {32, 64, 128, 256}"
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
  // the pair layout needs at least two tiles in every wave's range
  const bool full = (a.V % 16) == 0 && (tiles / nwg) / kDraftWaves >= 2;
  const int per_wg = (tiles + nwg - 1) / nwg;
  // The fused step, for at most kFusedStepItems verify candidates (one or
  // two ranking keys per thread, 16 keys per ranking workgroup): the ranking
  // workgroups must fit in the draft grid, and the last one's verify follows.
  // Larger batches take three launches: their drafting kernel is bandwidth
  // bound, and the fused kernel's extra registers slow its tile loop by about
  // as much as the two launches it saves.  So do small batches: their
  // drafting kernel has no per-step barrier, and the fused tail's barrier and
  // ranking cost more than the two launch gaps.
  const long long n_items = (long long)a.B * a.gamma;
  const int sched_e = n_items <= kRankThreads ? 1 : 2;
  const bool step = a.step != nullptr && full && a.bf16 && a.r == 256 && !rnn && !a.noalloc && !small &&
                    n_items <= kFusedStepItems && (n_items + 15) / 16 <= nwg;
  if (full) {
    const int tpw_need = (per_wg + kDraftWaves - 1) / kDraftWaves;   // most tiles any wave owns
    if (a.gumbel)
      pick<true>(a.bf16, a.r, true, rnn, tpw_need, &kc, step, small);
    else
      pick<false>(a.bf16, a.r, true, rnn, tpw_need, &kc, step, small);
  }
  const int nwaves = kc.threads / 64;
  if ((per_wg + nwaves - 1) / nwaves > kc.tpw) {
    *unsupported = "vocabulary too large to keep W2 on chip on this GPU";
    return hipSuccess;
  }
  if ((a.B + nwg - 1) / nwg > kMaxOwnedRows) {
    *unsupported = "too many requests per workgroup for the confidence epilogue";
    return hipSuccess;
  }
  const DraftWorkspace L = draft_workspace_layout(a.B, a.gamma, rnn ? a.r : 0);
  char* ws = static_cast<char*>(a.ws);
  if (a.noalloc) {   // every check has passed: set up (first call) and take this device's scratch
    if (rnn || L.total > kNoAllocScratchBytes) {
      *unsupported = "shape needs more workspace than the static scratch";
      return hipSuccess;
    }
    void* sp = nullptr;
    // the sections that must start at zero for this shape: [0, zpart)
    const size_t zero_bytes = L.zpart;
    e = noalloc_scratch(stream, &sp, (uint64_t(uint32_t(a.B)) << 32) | uint32_t(a.gamma), zero_bytes);
    if (e != hipSuccess) return e;
    ws = static_cast<char*>(sp);
  }
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
  p.bar = reinterpret_cast<unsigned int*>(ws + L.bar);
  // two groups (each group's barrier completes while the other computes), at most kMaxGroupRows rows
  int grs = ((a.B + 1) / 2 + 15) & ~15;
  if (grs > kMaxGroupRows) grs = kMaxGroupRows;
  if (grs < 16) grs = 16;
  p.grs = grs;
  p.slots = reinterpret_cast<uint64_t*>(ws + L.slots);
  p.zpart = reinterpret_cast<float*>(ws + L.zpart);
  p.hdot = reinterpret_cast<double*>(ws + L.hdot);
  p.decay = a.decay;
  p.state = rnn ? reinterpret_cast<uint16_t*>(ws + L.state) : nullptr;
  p.wkeys = reinterpret_cast<uint64_t*>(ws + L.wkeys);
  p.wz = reinterpret_cast<uint32_t*>(ws + L.wz);
  p.sched_tickets = nullptr;
  p.sched_sorted = nullptr;
  p.t_step = nullptr;
  p.n_min = p.n_count = p.sched_e = 0;
  p.target = nullptr;
  p.lens = p.m_out = p.accepted = p.bonus = nullptr;
  if (step) {
    unsigned char* sws = static_cast<unsigned char*>(a.step->sched_ws);
    p.sched_tickets = reinterpret_cast<unsigned int*>(sws);
    p.sched_sorted = reinterpret_cast<RankEntry*>(sws + kRankHeader);
    p.t_step = a.step->t_step;
    p.n_min = a.step->n_min;
    p.n_count = a.step->n_count;
    p.sched_e = sched_e;
    p.target = a.step->target;
    p.lens = a.step->lens;
    p.m_out = a.step->m_out;
    p.accepted = a.step->accepted;
    p.bonus = a.step->bonus;
    if (fused) *fused = true;
  }

  // Every workgroup must be resident at once (grid barriers between draft
  // positions; nwg <= one per compute unit).  The cooperative launch
  // guarantees it; a plain launch gets it from an otherwise idle device,
  // which the caller promises in exclusive mode.
  void* args[] = {&p};
  if (a.exclusive) return hipLaunchKernel(kc.fn, dim3(nwg), dim3(kc.threads), args, 0, stream);
  return hipLaunchCooperativeKernel(kc.fn, dim3(nwg), dim3(kc.threads), args, 0, stream);
}


// Address of this device's scratch, set up on the first call per device:
// hipGetSymbolAddress with the device current, then one zero-fill on
// `stream` (ordered before the draft launch that follows on the same stream).
// A later call of the same shape finds its counters and slots zero (left so
// by the previous call's last phase); a call of another shape (B, gamma) has
// them elsewhere, so the first `zero_bytes` are cleared again first.
hipError_t noalloc_scratch(hipStream_t stream, void** out, uint64_t shape, size_t zero_bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  static uint64_t last_shape[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidValue;
    const size_t n16 = kNoAllocScratchBytes / 16;
    scratch_clear_kernel<<<dim3(256), dim3(256), 0, stream>>>(static_cast<u32x4_t*>(p), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
    last_shape[dev] = shape;
  } else if (shape != last_shape[dev]) {
    const size_t n16 = (zero_bytes + 15) / 16;
    scratch_clear_kernel<<<dim3(64), dim3(256), 0, stream>>>(static_cast<u32x4_t*>(addr[dev]), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    last_shape[dev] = shape;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace dspark
