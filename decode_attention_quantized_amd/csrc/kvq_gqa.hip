// Fused sparse-V decode attention for grouped-query caches (q8_0, q4_0, LUT3)
// on gfx950. One launch per call (or one per share of the groups when they
// do not all fit one launch); all workgroups of a launch are resident at once
// (at most one per compute unit) and the workgroups of one (sequence, kv
// head) group exchange data through workspace words tagged with the call's
// epoch, so the scores of a whole context never leave the chip:
//
//  1. K pass. Each workgroup owns P consecutive positions of one (sequence,
//     kv head). Waves stream 16-position tiles of packed K rows, dequantize
//     the codes straight into MFMA operands and form the scores of all G
//     query heads of the group with v_mfma_f32_16x16x32_f16 (q split into
//     fp16 hi + lo halves, so the products keep ~22 bits of q). Scores stay in
//     LDS; the split's running (max, sum of exp) per head is published.
//  2. Every workgroup gathers the split statistics of its group and merges
//     them into the log-sum-exp (same order everywhere, so all workgroups of
//     a group hold bit-identical values).
//  3. V pass. p = exp(s - LSE) is the normalized weight; a head keeps a
//     position iff p >= threshold. Each wave ballots the union over the G
//     heads for its 64 positions and only those value rows are fetched;
//     every other row is never read (the sparse-V rule of "Пропуск 90% работы
//     по деквантизации…", tproger.ru, section "Решение — не ускорять, а
//     пропускать": skip V dequantization and accumulation when the attention
//     weight is below the threshold; weights are known from K before any V
//     work). Splits with kept rows publish a partial output and a flag.
//  4. Every workgroup of the group sums one slice of the group's output over
//     the flagged splits in fixed split order (deterministic).
//
// All waits are bounded: a wait that does not complete within ~0.5 s sets a
// status bit and lets the kernel finish.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// phase stamps are kept per workgroup of the whole call: a launch covers the
// groups bg0 .. bg0 + ngroups - 1, so its workgroup i is number bg0 * S + i
__device__ inline void stamp(const GqaArgs& a, int k) {
  if (a.times && threadIdx.x == 0) a.times[(int64_t(a.bg0) * a.S + blockIdx.x) * 16 + k] = wall_clock64();
}

// 2^x with the hardware instruction (results below the normal range flush
// to 0; used for softmax statistics, where such terms are below rounding)
__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two (max, sum-of-exp2) pairs of the log2 domain.
__device__ inline float2 lse_merge(float2 x, float2 y) {
  const float M = fmaxf(x.x, y.x);
  const float Ms = M == -INFINITY ? 0.f : M;         // both empty: every term is 0
  return make_float2(M, x.y * ex2(x.x - Ms) + y.y * ex2(y.x - Ms));
}

template <int CTRL>
__device__ inline float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline float2 dpp2(float2 v) { return make_float2(dppf<CTRL>(v.x), dppf<CTRL>(v.y)); }

// Sum over the 64 lanes of the wave in a fixed tree (rows with DPP, then the
// four row results); lane 0 holds the total.
__device__ inline float sum_wave(float v) {
  v += dppf<0xB1>(v);                                 // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);                                 // quad_perm [2,3,0,1]
  v += dppf<0x141>(v);                                // row_half_mirror
  v += dppf<0x140>(v);                                // row_mirror
  const float r1 = __shfl(v, 16), r2 = __shfl(v, 32), r3 = __shfl(v, 48);
  return (v + r1) + (r2 + r3);
}

// Maximum over the 64 lanes (rows with DPP, then the four rows with the
// lane-swap instructions); every lane holds the result.
__device__ inline float max_wave(float v) {
  v = fmaxf(v, dppf<0xB1>(v));                        // quad_perm [1,0,3,2]
  v = fmaxf(v, dppf<0x4E>(v));                        // quad_perm [2,3,0,1]
  v = fmaxf(v, dppf<0x141>(v));                       // row_half_mirror
  v = fmaxf(v, dppf<0x140>(v));                       // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                            false, false);
  v = fmaxf(__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1])));
  r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v), false,
                                       false);
  return fmaxf(__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1])));
}

// lse_merge over the lanes of equal lane mod C (C = 1, 2, 4 or 8): rotations
// by C, 2C, .. 8 inside each 16-lane row, then the two rows of each half and
// the two halves, each in one fixed order, so every lane of a class holds the
// same bits.
template <int O>
__device__ inline float2 row_ror(float2 v) { return dpp2<0x120 + O>(v); }
__device__ inline float2 swap16(float2 v) {
  const auto x = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v.x), __builtin_bit_cast(unsigned, v.x),
                                                  false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v.y), __builtin_bit_cast(unsigned, v.y),
                                                  false, false);
  return lse_merge(make_float2(__builtin_bit_cast(float, unsigned(x[0])), __builtin_bit_cast(float, unsigned(y[0]))),
                   make_float2(__builtin_bit_cast(float, unsigned(x[1])), __builtin_bit_cast(float, unsigned(y[1]))));
}
__device__ inline float2 swap32(float2 v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v.x), __builtin_bit_cast(unsigned, v.x),
                                                  false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v.y), __builtin_bit_cast(unsigned, v.y),
                                                  false, false);
  return lse_merge(make_float2(__builtin_bit_cast(float, unsigned(x[0])), __builtin_bit_cast(float, unsigned(y[0]))),
                   make_float2(__builtin_bit_cast(float, unsigned(x[1])), __builtin_bit_cast(float, unsigned(y[1]))));
}
template <int C>
__device__ inline float2 merge_class(float2 v) {
  if constexpr (C <= 1) v = lse_merge(v, row_ror<1>(v));
  if constexpr (C <= 2) v = lse_merge(v, row_ror<2>(v));
  if constexpr (C <= 4) v = lse_merge(v, row_ror<4>(v));
  v = lse_merge(v, row_ror<8>(v));
  v = swap16(v);
  return swap32(v);
}

// lse_merge over the 16 lanes of each row of the wave (quad neighbours, the
// other pair of the quad, mirrored quads, mirrored half rows); lane 0 of the
// row holds the merge of all 16.
__device__ inline float2 merge_row16(float2 x) {
  x = lse_merge(x, dpp2<0xB1>(x));                    // quad_perm [1,0,3,2]
  x = lse_merge(x, dpp2<0x4E>(x));                    // quad_perm [2,3,0,1]
  x = lse_merge(x, dpp2<0x141>(x));                   // row_half_mirror
  x = lse_merge(x, dpp2<0x140>(x));                   // row_mirror
  return x;
}

// The defined result of a value that depended on a wait that gave up. The
// kernels are compiled without NaN semantics (their arithmetic never makes
// one), so the NaN pattern is passed through an empty asm statement: the
// compiler cannot see that it is a NaN and fold the selection away.
constexpr uint32_t kNaNBits = 0x7FC00000u;
__device__ inline float poison_if(bool bad, float v) {
  uint32_t nan_bits = kNaNBits;
  asm volatile("" : "+v"(nan_bits));
  return __uint_as_float(bad ? nan_bits : __float_as_uint(v));
}

__device__ inline float bf16_to_f32(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

__device__ inline float half_lo(uint32_t w) {
  return float(__builtin_bit_cast(half2v, w)[0]);
}
__device__ inline float half_hi(uint32_t w) {
  return float(__builtin_bit_cast(half2v, w)[1]);
}

// ---------------------------------------------------------------- tagged words
// A hand-off value is one 64-bit word: the call's epoch in the high half and
// the payload in the low half, stored and loaded as a single relaxed
// agent-scope atomic (coherent across the XCDs' L2 caches). A reader spins
// (bounded) until the tag matches; no fence or counter orders the hand-off.
typedef unsigned long long u64;

__device__ inline void put_tagged(u64* p, uint32_t epoch, uint32_t payload) {
  __hip_atomic_store(p, (u64(epoch) << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void put_tagged_f(u64* p, uint32_t epoch, float v) { put_tagged(p, epoch, __float_as_uint(v)); }

// One relaxed load; pair with a settle so a batch of loads is in flight at once.
__device__ inline u64 peek(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two adjacent tagged words read by one 16-byte buffer load with the same
// agent-coherent cache policy as peek() (sc1). Each naturally aligned 8-byte
// word of it is read as a unit (the load is served from one cache line), so
// a word's tag still vouches for its payload. Threads that take consecutive
// 16-byte pieces make a wave read whole lines: polling a group's words costs
// one request per line instead of one per word.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCoherentLoad = 16;                    // buffer cache policy: sc1
__device__ inline __amdgpu_buffer_rsrc_t coherent_rsrc(const u64* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<u64*>(base), 0, bytes, 0x00020000);
}
__device__ inline u32x4 peek2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentLoad);
}
__device__ inline bool stale2(const u32x4& v, uint32_t epoch) { return v.y != epoch || v.w != epoch; }

// Bring M peeked pairs of words (16-byte loads at byte offsets off[] of r)
// plus N single words up to the current epoch, re-reading all stale ones
// together (one round trip per retry rather than one per word). Bounded:
// after `limit` retries the wait gives up, sets the sticky status bit and
// returns true (the caller then publishes and writes NaN instead of values
// that depended on the words).
template <int M, int N>
__device__ inline bool settle_mixed(u32x4 (&v)[M], const bool (&use_v)[M], __amdgpu_buffer_rsrc_t r,
                                    const int (&off)[M], u64 (&w)[N], const u64* const (&p)[N], const bool (&use)[N],
                                    uint32_t epoch, WsHeader* h, uint32_t limit) {
  uint32_t spins = 0;
  while (true) {
    bool stale = false;
#pragma unroll
    for (int k = 0; k < M; ++k) stale |= use_v[k] && stale2(v[k], epoch);
#pragma unroll
    for (int k = 0; k < N; ++k) stale |= use[k] && uint32_t(w[k] >> 32) != epoch;
    if (!stale) return false;
    __builtin_amdgcn_s_sleep(1);
    if (++spins > limit) {
      __hip_atomic_fetch_or(&h->status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return true;
    }
#pragma unroll
    for (int k = 0; k < M; ++k)
      if (use_v[k] && stale2(v[k], epoch)) v[k] = peek2(r, off[k]);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (use[k] && uint32_t(w[k] >> 32) != epoch) w[k] = peek(p[k]);
  }
}

// Online (max, sum of exp2) update with one more score; -inf scores are skipped.
__device__ inline void online_add(float& m, float& l, float s) {
  if (s == -INFINITY) return;
  if (s > m) { l = l * ex2(m - s) + 1.f; m = s; }
  else l += ex2(s - m);
}

// The same update with N more scores at once and no branch: the new maximum
// first, then the old sum rescaled to it plus the new terms (-inf scores add
// 0; while every score so far is -inf the reference is 0 and the sum stays 0).
template <int N>
__device__ inline void batch_stats(float& m, float& l, const float (&s)[N]) {
  float mx = m;
#pragma unroll
  for (int k = 0; k < N; ++k) mx = fmaxf(mx, s[k]);
  const float ref = mx == -INFINITY ? 0.f : mx;
  float acc = l * ex2(m - ref);
#pragma unroll
  for (int k = 0; k < N; ++k) acc += ex2(s[k] - ref);
  m = mx;
  l = acc;
}

// The pair table: 64 words in LDS, read with one ds_read_b32 per key (the
// byte address is 4 * key), or held one entry per lane and read with
// ds_bpermute.
constexpr bool kLdsTable = true;
struct Lut {
  uint32_t entry;                                  // this lane's entry (ds_bpermute form)
  const uint32_t* tab;                             // the table in LDS
};
__device__ inline uint32_t lut_pair(const Lut& L, uint32_t addr) {
  if constexpr (kLdsTable) return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(L.tab) + addr);
  else return uint32_t(__builtin_amdgcn_ds_bpermute(int(addr), int(L.entry)));
}

// K rows are read with buffer loads: the resource covers exactly the split's
// rows in the context, so a load past them (the pipelined loop requests
// batches beyond the split) returns zeros without touching memory; the row
// offset of a tile is a wave-uniform byte offset and the lane's part a
// 32-bit offset, so no 64-bit address arithmetic is needed per tile.
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3v __attribute__((ext_vector_type(3)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v.x, v.y);
}

// The K stream (every key row of the call, read once) uses the non-temporal
// cache policy, so it does not push out of L2 what the later phases read
// again: the kernel's code for those phases, the hand-off words, q. Measured
// on the LUT3 batch (52 MB of keys, more than the 4 MB L2 of each XCD holds):
// 26.2-26.5 us per call against 27.4-27.8 us; on the long shape 14.5 against
// 14.9 us.
constexpr int kStreamLoad = 2;                       // buffer cache policy: nt
__device__ inline uint4 bload16s(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamLoad);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 bload8s(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamLoad);
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------- format traits
// Each lane of a 16x16x32 MFMA supplies 8 consecutive K-slots of one column.
// For the K pass the column is a position and the 32 K-slots of one MFMA are
// the 32 elements of one quantization block (so a per-position, per-block
// scale can be applied to the fp32 result). Lane group kk = lane/16 takes
// elements 8kk..8kk+7 of the block; dim_of() gives the element order the
// dequantizer produces, which the q operand must follow.
template <int FMT> struct Traits;

template <> struct Traits<KVQ_Q4_0> {
  static constexpr int CB = 64, SB = 8;
  static constexpr bool kRowScale = false;        // one scale per 32-element block
  static constexpr float kRowMul = 1.0f;
  // codes c in 0..15 enter the MFMA as fp16 (16 + c); value = c - 8, so the
  // bias removed per block is 24 * sum(q)
  static constexpr float kBias = 24.0f;
  struct Raw { uint32_t c[4]; uint2 s; };
  __device__ static int dim_of(int bb, int kk, int e) { return 32 * bb + 8 * kk + (e >> 1) + 4 * (e & 1); }
  // inverse of dim_of: MFMA index, lane group and vector slot of dim d
  __device__ static void locate(int d, int& bb, int& kk, int& slot) {
    bb = d >> 5; kk = (d >> 3) & 3; slot = 2 * (d & 3) + ((d >> 2) & 1);
  }
  // Staged K load: lane group kg reads block kg of its row (16 contiguous
  // bytes, so one instruction covers a whole 16-row tile); the wave then
  // swaps the pieces through LDS so that lane group kk holds dword kk of
  // every block (the layout of Raw).
  static constexpr bool kStaged = true;
  static constexpr int NV = 1;                    // 16-byte pieces per lane and row
  static constexpr int PITCH = 80;                // staged row pitch in LDS (bytes)
  static constexpr int kLaneOff = 16;             // byte offset of lane group kg's piece in a row
  struct Raw16 { uint4 v[NV]; uint2 s; };
  __device__ static Raw16 bload(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int vc, int vs, int sc,
                                int ss) {
    Raw16 r;
    r.v[0] = bload16s(rc, vc, sc);
    r.s = bload8s(rs, vs, ss);
    return r;
  }
  __device__ static void stage(uint8_t* lrow, const Raw16& r, int kg) {
    *reinterpret_cast<uint4*>(lrow + 16 * kg) = r.v[0];
  }
  __device__ static Raw unstage(const uint8_t* lrow, int kk, uint2 s) {
    Raw r;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) r.c[bb] = *reinterpret_cast<const uint32_t*>(lrow + 16 * bb + 4 * kk);
    r.s = s;
    return r;
  }
  // one dword = 8 nibbles -> fp16 (16 + c), vector order elements 0,4,1,5,2,6,3,7
  __device__ static half8 deq(const Raw& r, int bb, const Lut&) {
    const uint32_t x = r.c[bb];
    uint4 u;
    u.x = ((x << 6) & 0x03C003C0u) | 0x4C004C00u;
    u.y = ((x << 2) & 0x03C003C0u) | 0x4C004C00u;
    u.z = ((x >> 2) & 0x03C003C0u) | 0x4C004C00u;
    u.w = ((x >> 6) & 0x03C003C0u) | 0x4C004C00u;
    return __builtin_bit_cast(half8, u);
  }
  __device__ static float scale(const Raw& r, int bb) {
    const uint32_t w = (bb < 2) ? r.s.x : r.s.y;
    return (bb & 1) ? half_hi(w) : half_lo(w);
  }
  // value pass: lane owns dims 2*lane, 2*lane+1
  struct VRaw { uint32_t code, sc; };
  __device__ static VRaw vload(const uint8_t* crow, const uint8_t* srow, int lane) {
    VRaw v;
    v.code = crow[lane];
    v.sc = *reinterpret_cast<const uint16_t*>(srow + 2 * (lane >> 4));
    return v;
  }
  __device__ static void vdeq(const VRaw& r, const Lut&, float& v0, float& v1) {
    const float d = float(__builtin_bit_cast(_Float16, uint16_t(r.sc)));
    v0 = float(int(r.code & 15u) - 8) * d;
    v1 = float(int(r.code >> 4) - 8) * d;
  }
};

template <> struct Traits<KVQ_Q8_0> {
  static constexpr int CB = 128, SB = 8;
  static constexpr bool kRowScale = false;
  static constexpr float kRowMul = 1.0f;
  // signed codes enter as fp16 (1024 + (c + 128)); bias 1152
  static constexpr float kBias = 1152.0f;
  struct Raw { uint2 c[4]; uint2 s; };
  __device__ static int dim_of(int bb, int kk, int e) { return 32 * bb + 8 * kk + e; }
  __device__ static void locate(int d, int& bb, int& kk, int& slot) { bb = d >> 5; kk = (d >> 3) & 3; slot = d & 7; }
  // staged K load (see the q4_0 traits): lane group kg reads block kg (32 bytes)
  static constexpr bool kStaged = true;
  static constexpr int NV = 2;
  static constexpr int PITCH = 144;
  static constexpr int kLaneOff = 32;
  struct Raw16 { uint4 v[NV]; uint2 s; };
  __device__ static Raw16 bload(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int vc, int vs, int sc,
                                int ss) {
    Raw16 r;
    r.v[0] = bload16s(rc, vc, sc);
    r.v[1] = bload16s(rc, vc + 16, sc);
    r.s = bload8s(rs, vs, ss);
    return r;
  }
  __device__ static void stage(uint8_t* lrow, const Raw16& r, int kg) {
    *reinterpret_cast<uint4*>(lrow + 32 * kg) = r.v[0];
    *reinterpret_cast<uint4*>(lrow + 32 * kg + 16) = r.v[1];
  }
  __device__ static Raw unstage(const uint8_t* lrow, int kk, uint2 s) {
    Raw r;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) r.c[bb] = *reinterpret_cast<const uint2*>(lrow + 32 * bb + 8 * kk);
    r.s = s;
    return r;
  }
  __device__ static half8 deq(const Raw& r, int bb, const Lut&) {
    const uint32_t x0 = r.c[bb].x ^ 0x80808080u, x1 = r.c[bb].y ^ 0x80808080u;
    uint4 u;
    u.x = __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u);
    u.y = __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u);
    u.z = __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u);
    u.w = __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u);
    return __builtin_bit_cast(half8, u);
  }
  __device__ static float scale(const Raw& r, int bb) {
    const uint32_t w = (bb < 2) ? r.s.x : r.s.y;
    return (bb & 1) ? half_hi(w) : half_lo(w);
  }
  struct VRaw { uint32_t code, sc; };
  __device__ static VRaw vload(const uint8_t* crow, const uint8_t* srow, int lane) {
    VRaw v;
    v.code = *reinterpret_cast<const uint16_t*>(crow + 2 * lane);
    v.sc = *reinterpret_cast<const uint16_t*>(srow + 2 * (lane >> 4));
    return v;
  }
  __device__ static void vdeq(const VRaw& r, const Lut&, float& v0, float& v1) {
    const float d = float(__builtin_bit_cast(_Float16, uint16_t(r.sc)));
    v0 = float(int(int8_t(r.code & 0xFFu))) * d;
    v1 = float(int(int8_t(r.code >> 8))) * d;
  }
};

// LUT3: 3-bit codes (sign << 2 | magnitude index) packed contiguously, element
// i at bits 3i..3i+2 of the 384-bit row, one fp16 nu per row; value =
// nu * (+-M[idx]) / sqrt(128) with M the four fp16 Lloyd-Max magnitudes.
// Two neighbouring codes form a 6-bit key; every lane holds one entry of the
// 64-entry table of fp16 value pairs, read with ds_bpermute (the LUT read of
// the turbo3 dequant, "14 попыток, которые провалились", done as one
// cross-lane read per two elements). The scale is per row, so the four MFMAs
// of a row accumulate into one result.
constexpr uint16_t kLut3Bits[4] = {0x33D8, 0x3A0C, 0x3D60, 0x404E};

__device__ inline uint32_t lut3_code_bits(uint32_t c) {
  return ((c & 4u) << 13) | kLut3Bits[c & 3u];
}
// entry k of the pair table: key k = c0 | c1 << 3 -> (value c0, value c1)
__device__ inline uint32_t lut3_pair_entry(int k) {
  return lut3_code_bits(uint32_t(k) & 7u) | (lut3_code_bits(uint32_t(k) >> 3) << 16);
}


template <> struct Traits<KVQ_LUT3> {
  static constexpr int CB = 48, SB = 2;
  static constexpr bool kRowScale = true;
  static constexpr bool kStaged = false;          // lane group kk already reads 12 contiguous bytes
  static constexpr int PITCH = 64;                // staged row pitch in LDS (value rows only)
  static constexpr float kBias = 0.0f;
  static constexpr float kRowMul = 0.08838834764831845f;   // 1/sqrt(128)
  struct Raw { uint32_t c[3]; uint32_t s; };
  // lane group kk holds elements 32kk..32kk+31 (bits 96kk..96kk+95 of the row);
  // MFMA bb takes elements 32kk + 8bb + e
  __device__ static int dim_of(int bb, int kk, int e) { return 32 * kk + 8 * bb + e; }
  __device__ static void locate(int d, int& bb, int& kk, int& slot) { kk = d >> 5; bb = (d >> 3) & 3; slot = d & 7; }
  static constexpr int kLaneOff = 12;             // lane group kk reads bytes 12kk .. 12kk + 11
  __device__ static Raw bload(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int vc, int vs, int sc,
                              int ss) {
    Raw r;
    const u32x3v v = __builtin_amdgcn_raw_buffer_load_b96(rc, vc, sc, kStreamLoad);
    r.c[0] = v.x; r.c[1] = v.y; r.c[2] = v.z;
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, vs, ss, kStreamLoad);
    return r;
  }
  // byte address (4 * key) of the 6-bit key at bit b of the lane's 96 bits
  __device__ static uint32_t key_addr(const Raw& r, int b) {
    const int w = b >> 5, o = b & 31;
    const uint32_t x = (o <= 26) ? (r.c[w] >> o) : __builtin_amdgcn_alignbit(r.c[w + 1], r.c[w], o);
    return (x << 2) & 0xFCu;
  }
  __device__ static half8 deq(const Raw& r, int bb, const Lut& L) {
    uint4 u;
    u.x = lut_pair(L, key_addr(r, 24 * bb + 0));
    u.y = lut_pair(L, key_addr(r, 24 * bb + 6));
    u.z = lut_pair(L, key_addr(r, 24 * bb + 12));
    u.w = lut_pair(L, key_addr(r, 24 * bb + 18));
    return __builtin_bit_cast(half8, u);
  }
  __device__ static float scale(const Raw& r, int) { return half_lo(r.s); }
  // value pass: lane owns dims 2*lane, 2*lane+1 = bits 6*lane..6*lane+5
  struct VRaw { uint32_t lo, hi, sc; };
  __device__ static VRaw vload(const uint8_t* crow, const uint8_t* srow, int lane) {
    VRaw v;
    const int b = 6 * lane, w = b >> 5;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(crow);
    v.lo = p[w];
    v.hi = ((b & 31) > 26) ? p[w + 1] : 0u;       // only when the key straddles two words
    v.sc = *reinterpret_cast<const uint16_t*>(srow);
    return v;
  }
  __device__ static void vdeq(const VRaw& r, const Lut& L, float& v0, float& v1) {
    const int lane = __lane_id();
    const int o = (6 * lane) & 31;
    const uint32_t x = __builtin_amdgcn_alignbit(r.hi, r.lo, o);
    const uint32_t pair = lut_pair(L, (x << 2) & 0xFCu);
    const float nu = float(__builtin_bit_cast(_Float16, uint16_t(r.sc))) * kRowMul;
    v0 = half_lo(pair) * nu;
    v1 = half_hi(pair) * nu;
  }
};

// LUT3 of Walsh-Hadamard-rotated rows: the stored rows decode as LUT3; the
// kernel rotates q once (scores are inner products, and the rotation is
// orthonormal and symmetric) and each workgroup's partial output once.
template <> struct Traits<KVQ_LUT3_WHT> : Traits<KVQ_LUT3> {};

// v plus the value of lane l ^ 16 (resp. l ^ 32), the same bits on both lanes
__device__ inline float sum_pairs16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return __builtin_bit_cast(float, unsigned(r[0])) + __builtin_bit_cast(float, unsigned(r[1]));
}
__device__ inline float sum_pairs32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return __builtin_bit_cast(float, unsigned(r[0])) + __builtin_bit_cast(float, unsigned(r[1]));
}

// ---------------------------------------------------------------- value rows on MFMA
// A wave with many value rows sums p * v with v_mfma_f32_16x16x16_f16, 16
// rows per batch: out[h][d] = sum_r (p[h][r] * s[r][d]) * c[r][d] with s the
// row's scale for dim d and c its code value (q4_0: c - 8, exact in fp16).
// A rows 0..7 hold the fp16 high parts of x = 2^sh * p * s for heads 0..7,
// rows 8..15 the low parts (x minus the high part); the products with the
// exact codes are formed and summed in fp32. The power of two 2^sh puts the
// largest x of the wave's rows so far in [2^14, 2^15), far inside the fp16
// normal range: a term within 2^18 of that largest one is represented within
// 2^-22 relative, a smaller one within 2^-25 of the fp16 unit of its batch
// (weights near 1/n at long contexts would otherwise fall among fp16
// subnormals and lose their low parts). When a batch holds a larger x than
// any before, the accumulators are rescaled by the exact power of two. Tile t (0..7) takes the dims n + 16t (n the
// MFMA column), all inside scale block t / 2, so each tile has one A operand.
// A row's 64 code bytes are staged transposed as an 8 x 8 byte matrix,
// T[8j + a] = R[8a + j], so that the lane of column n finds the nibbles of
// its dims n + 16a (a = 0..7) in the 8 bytes at 8 * (n / 2).
template <int FMT> struct VMfma {
  static constexpr bool kOn = false;
  __device__ static int dim(int, int) { return 0; }
};
template <> struct VMfma<KVQ_Q4_0> {
  static constexpr bool kOn = true;
  // code piece ch (row bytes 16ch .. 16ch + 15) -> its transposed places: for
  // each j the bytes (j, 8 + j) of the piece go to T[8j + 2ch], T[8j + 2ch + 1]
  __device__ static void stage(uint8_t* lrow, const uint4& cv, int ch) {
    const uint32_t p01 = __builtin_amdgcn_perm(cv.z, cv.x, 0x05010400u);   // pairs j = 0, 1
    const uint32_t p23 = __builtin_amdgcn_perm(cv.z, cv.x, 0x07030602u);   // j = 2, 3
    const uint32_t p45 = __builtin_amdgcn_perm(cv.w, cv.y, 0x05010400u);   // j = 4, 5
    const uint32_t p67 = __builtin_amdgcn_perm(cv.w, cv.y, 0x07030602u);   // j = 6, 7
    uint16_t* q = reinterpret_cast<uint16_t*>(lrow + 2 * ch);
    q[0] = uint16_t(p01); q[4] = uint16_t(p01 >> 16);
    q[8] = uint16_t(p23); q[12] = uint16_t(p23 >> 16);
    q[16] = uint16_t(p45); q[20] = uint16_t(p45 >> 16);
    q[24] = uint16_t(p67); q[28] = uint16_t(p67 >> 16);
  }
  __device__ static int dim(int n, int t) { return n + 16 * t; }
  // B operands of the 8 tiles for rows 4g .. 4g + 3 of the batch (column n)
  __device__ static void b_ops(const uint8_t* vst, int g, int n, const Lut&, half4 (&B)[8]) {
    const int sh = 4 * (n & 1);
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 x = *reinterpret_cast<const uint2*>(vst + (4 * g + i) * Traits<KVQ_Q4_0>::PITCH + 8 * (n >> 1));
      lo[i] = x.x >> sh;
      hi[i] = x.y >> sh;
    }
    const half2v bias = {_Float16(1032.f), _Float16(1032.f)};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t* w = t < 4 ? lo : hi;
      const uint32_t sel = 0x0C000C00u | (uint32_t(4 + (t & 3)) << 16) | uint32_t(t & 3);
      // bytes t of rows (0, 1) and (2, 3) -> nibbles -> fp16 1024 + c -> c - 8
      const uint32_t r01 = (__builtin_amdgcn_perm(w[1], w[0], sel) & 0x000F000Fu) | 0x64006400u;
      const uint32_t r23 = (__builtin_amdgcn_perm(w[3], w[2], sel) & 0x000F000Fu) | 0x64006400u;
      const half2v h01 = __builtin_bit_cast(half2v, r01) - bias;
      const half2v h23 = __builtin_bit_cast(half2v, r23) - bias;
      B[t] = half4{h01[0], h01[1], h23[0], h23[1]};
    }
  }
  // scale of block b (dims 32b .. 32b + 31) of a staged row
  __device__ static float scale(const uint8_t* lrow, int b) {
    return float(reinterpret_cast<const _Float16*>(lrow + Traits<KVQ_Q4_0>::CB)[b]);
  }
  static constexpr int kBlocks = 4;                  // scale blocks (A operands) per row
};

// LUT3: one scale per row, so the A operand is p * nu / sqrt(128) and tile t
// takes the dims 8n + t; rows are staged as they are. The lane of column n
// reads the 24 code bits of its dims 8n .. 8n + 7 from a row, looks up the
// four value pairs in the pair table and swaps them into the row order of
// the B operand. B holds the fp16 table values (exact).
template <> struct VMfma<KVQ_LUT3> {
  static constexpr bool kOn = true;
  static constexpr int kBlocks = 1;
  __device__ static void stage(uint8_t* lrow, const uint4& cv, int ch) {
    *reinterpret_cast<uint4*>(lrow + 16 * ch) = cv;
  }
  __device__ static int dim(int n, int t) { return 8 * n + t; }
  __device__ static void b_ops(const uint8_t* vst, int g, int n, const Lut& L, half4 (&B)[8]) {
    const int w = (24 * n) >> 5, o = (24 * n) & 31;
    uint32_t pr[4][4];                               // [row][dim pair] value pairs
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t* rw = reinterpret_cast<const uint32_t*>(vst + (4 * g + i) * Traits<KVQ_LUT3>::PITCH);
      // bits 24n .. 24n + 23 of the row (the word after it is still inside the row's pitch)
      const uint32_t bits = __builtin_amdgcn_alignbit(rw[w + 1], rw[w], o);
#pragma unroll
      for (int tp = 0; tp < 4; ++tp)
        pr[i][tp] = lut_pair(L, ((bits >> (6 * tp)) << 2) & 0xFCu);
    }
#pragma unroll
    for (int tp = 0; tp < 4; ++tp) {
      const uint32_t e01 = __builtin_amdgcn_perm(pr[1][tp], pr[0][tp], 0x05040100u);   // even dim, rows 0, 1
      const uint32_t o01 = __builtin_amdgcn_perm(pr[1][tp], pr[0][tp], 0x07060302u);   // odd dim
      const uint32_t e23 = __builtin_amdgcn_perm(pr[3][tp], pr[2][tp], 0x05040100u);
      const uint32_t o23 = __builtin_amdgcn_perm(pr[3][tp], pr[2][tp], 0x07060302u);
      B[2 * tp] = __builtin_bit_cast(half4, make_uint2(e01, e23));
      B[2 * tp + 1] = __builtin_bit_cast(half4, make_uint2(o01, o23));
    }
  }
  __device__ static float scale(const uint8_t* lrow, int) {
    return float(*reinterpret_cast<const _Float16*>(lrow + Traits<KVQ_LUT3>::CB)) * Traits<KVQ_LUT3>::kRowMul;
  }
};
template <> struct VMfma<KVQ_LUT3_WHT> : VMfma<KVQ_LUT3> {};

// y = H x / sqrt(128) in float32 on a 128-vector held as elements (lane,
// lane + 64) of a wave (H the Sylvester Hadamard matrix, as the packers)
__device__ inline void wht_wave(int lane, float& v0, float& v1) {
#pragma unroll
  for (int h = 1; h < 64; h *= 2) {
    const float p0 = __shfl_xor(v0, h), p1 = __shfl_xor(v1, h);
    const bool upper = lane & h;
    v0 = upper ? p0 - v0 : v0 + p0;
    v1 = upper ? p1 - v1 : v1 + p1;
  }
  const float a = v0, b = v1;
  v0 = (a + b) * 0.08838834764831845f;
  v1 = (a - b) * 0.08838834764831845f;
}

template <class T, bool kStaged> struct LoadedOf { using type = typename T::Raw; };
template <class T> struct LoadedOf<T, true> { using type = typename T::Raw16; };

// ---------------------------------------------------------------- the kernel
// Workgroup roles: every workgroup scores its split, merges its group's LSE,
// runs its own V pass and sums one slice of the group's output; split 0 of
// each group also counts its group towards publishing the next epoch (once
// past the LSE exchange every workgroup of the group has read the epoch).
//
// MODE 1 (RUN) selects the single-pass skip rule: a position is kept when its weight
// under the softmax of its split's positions up to the end of its 64-position
// block reaches the threshold (the weight an in-loop flash-attention kernel
// sees with its running max and sum). That decision needs nothing from other
// workgroups, so the V pass runs right after the scores with weights relative
// to the split's own max, and the group's LSE is gathered afterwards only to
// scale the partial output (its wait overlaps the V pass).
//
// MODE 2 (KSKIP) is key skipping (the default rule otherwise): the split first scores
// its candidate blocks (largest key norm at least half the context's
// largest), the group exchanges their statistics, which bound each head's
// LSE from below, and the split then drops every other block whose bound
// weight (64 positions or fewer, every score at most sigma * ||q_h|| * R)
// is at most 1e-7 for all heads, and scores the rest.
template <int FMT, int G, int MODE>
__global__ __launch_bounds__(kThreads) void gqa_fused(GqaArgs a) {
  constexpr bool RUN = MODE == 1;                      // single-pass rule
  constexpr bool KSKIP = MODE == 2;                    // key skipping
  using T = Traits<FMT>;
  constexpr bool kRot = FMT == KVQ_LUT3_WHT;           // rotate q in, partial outputs out
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  extern __shared__ __align__(16) unsigned char smem[];
  // LDS: scores [G][P] (then kept weights in place; then the cross-wave
  // reduction; then the merge inputs), q operands, small per-head values.
  const int P = a.P;
  const int sc_floats = gqa_sc_floats(G, P, a.S);
  float* sc = reinterpret_cast<float*>(smem);
  // scores (then weights) of head j at split position i: chunk-major, the G
  // heads' 64 values of a chunk contiguous, so one chunk's heads are read
  // from one base address with constant offsets
  auto sidx = [](int j, int i) { return (i >> 6) * (G * kChunk) + j * kChunk + (i & (kChunk - 1)); };
  _Float16* qop = reinterpret_cast<_Float16*>(sc + sc_floats);     // [16 rows][4 blk][4 kk][8]
  float* cst = reinterpret_cast<float*>(qop + 16 * 128);          // [4 blk][16 rows]
  float* hs = cst + 64;                                           // [8] per-head score scale
  float* lse = hs + 8;                                            // [8] log2-domain LSE
  float* qmax = lse + 8;                                          // [8]
  int* wcount = reinterpret_cast<int*>(qmax + 8);                 // [kWaves] kept pairs
  int* wrows = wcount + kWaves;                                   // [kWaves] rows fetched
  float* wmass = reinterpret_cast<float*>(wrows + kWaves);        // [kWaves][G]
  float2* wml = reinterpret_cast<float2*>(wmass + kWaves * G);    // [kWaves][8] per-wave (max, sum)
  int* wproc = reinterpret_cast<int*>(wml + kWaves * 8);          // [kWaves] value rows each wave summed
  int* wto = wproc + kWaves;                                      // [4]: [0] a wait of this workgroup gave up
  // per-wave lists of the kept rows a wave fetches: [kWaves][64 * ceil(P/64 / kWaves)]
  uint16_t* rowlist = reinterpret_cast<uint16_t*>(wto + 4);
  const int list_cap = 64 * ((P / kChunk + kWaves - 1) / kWaves);
  // per-wave K staging strip [kWaves][16 rows][PITCH] (16-byte aligned; the
  // offset is rounded, not the pointer, so accesses stay LDS instructions)
  const int stg_off = (int(reinterpret_cast<unsigned char*>(rowlist + kWaves * list_cap) - smem) + 15) & ~15;
  uint8_t* stg = smem + stg_off;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform across the wave: taken as a scalar, every
  // tile index and loop bound derived from it stays scalar (no exec-masked
  // branches around uniform per-tile tests)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bg = a.bg0 + int(blockIdx.x) / a.S;   // b * Hkv + g
  const int split = int(blockIdx.x) - (bg - a.bg0) * a.S;
  const int wg = bg * a.S + split;                 // workgroup number within the whole call
  const bool master = split == 0;                  // advances the epoch for its group
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int pos0 = split * P;
  const int ctx = a.ctx;
  const float tau = a.tau;
  const int64_t row0 = int64_t(bg) * a.cap;
  const uint32_t epoch = __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  stamp(a, 0);

  const int n16 = lane & 15;     // MFMA column (position within a tile)
  const int kg = lane >> 4;      // lane group
  constexpr bool kLut3 = FMT == KVQ_LUT3 || FMT == KVQ_LUT3_WHT;
  __shared__ uint32_t lut3_tab[kLut3 ? 64 : 1];      // LUT3 pair table (written in the set-up below)
  const Lut table{kLut3 ? lut3_pair_entry(lane) : 0u, lut3_tab};
  // issue the first K tiles before the q set-up so their latency overlaps it
  const int ntiles = P / 16;
  constexpr int U = 4;
  using Loaded = typename LoadedOf<T, T::kStaged>::type;
  // a wave's batches of U tiles are double-buffered (the next batch is
  // requested before the current one is scored) when two fit in registers
  // (a third buffer measured slower for LUT3)
  constexpr bool kDouble = sizeof(Loaded) <= 24;
  Loaded rawA[U], rawB[kDouble ? U : 1];
  // Every lane loads unconditionally (buffer loads over the split's rows in
  // the context: a position past them reads zeros, its score is masked to
  // -inf or never formed). No load sits behind a branch, so the next batch's
  // loads are issued before the current batch is waited for. Batch kb's
  // tile u is tile wave + (kb * U + u) * kWaves; its rows start
  // (kb * U + u) * kWaves * 16 rows after the wave's first tile.
  const int nvalid = min(P, ctx - pos0);
  const __amdgpu_buffer_rsrc_t krc = rows_rsrc(a.kc + (row0 + pos0) * T::CB, nvalid * T::CB);
  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(a.ks + (row0 + pos0) * T::SB, nvalid * T::SB);
  const int kvc = n16 * T::CB + T::kLaneOff * kg;
  const int kvs = n16 * T::SB;
  // Tile t of a K pass covers rows trow(t) .. trow(t) + 15 of the split: 16t,
  // or, in the listed passes of key skipping, 16 (t mod 4) rows into the
  // chunk klist[t / 4] (a listed tile past the pass's ntl tiles reads past
  // the split's rows: zeros, no memory access).
  const uint8_t* klist = nullptr;
  int ntl = ntiles;
  auto trow = [&](auto listed, int t) -> int {
    if constexpr (decltype(listed)::value)
      return t < ntl ? 64 * __builtin_amdgcn_readfirstlane(int(klist[t >> 2])) + 16 * (t & 3) : P;
    else
      return 16 * t;
  };
  auto load_tiles = [&](auto listed, Loaded* raw, int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int m = trow(listed, wave + (kb * U + u) * kWaves);     // uniform
      raw[u] = T::bload(krc, krs, kvc, kvs, m * T::CB, m * T::SB);
    }
  };
  // the operand layout of a loaded tile (through this wave's LDS strip when
  // staged; a wave's LDS accesses complete in order, so no barrier is needed)
  uint8_t* lrow = stg + (wave * 16 + n16) * T::PITCH;
  auto operands = [&](const Loaded& rl) -> typename T::Raw {
    if constexpr (T::kStaged) {
      T::stage(lrow, rl, kg);
      return T::unstage(lrow, kg, rl.s);
    } else {
      return rl;
    }
  };
  // q of this group first, then the first K tiles: loads complete in order,
  // so the set-up below waits for q only while the K tiles are in flight
  // (one unconditional 16-byte load per thread, whatever the element type: a
  // bf16 row uses the first 8 bytes; the buffer bounds make the bytes past
  // the end of q read as zeros)
  const int jq = tid >> 5, lnq = tid & 31;          // 32 threads per head, 4 dims each
  const int qesz = a.q_bf16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t qrc = rows_rsrc(static_cast<const uint8_t*>(a.q), a.B * a.Hq * 128 * qesz);
  const uint4 qraw = bload16(qrc, ((b * a.Hq + g * G + min(jq, G - 1)) * 128 + lnq * 4) * qesz, 0);
  // key skipping: this group's block summaries (the candidates' K tiles are
  // requested once they are known)
  float rmax = 0.f;
  int nb_ctx = 0;
  if constexpr (KSKIP) {
    nb_ctx = (ctx + kChunk - 1) / kChunk;
    const float* kn = a.knorm + int64_t(bg) * a.knorm_pitch;
    for (int i = tid; i < nb_ctx; i += kThreads) rmax = fmaxf(rmax, kn[i]);
  }
  __asm__ volatile("" ::: "memory");
  if constexpr (!KSKIP) load_tiles(std::false_type{}, rawA, 0);
  __asm__ volatile("" ::: "memory");

  // ---------------------------------------------------------------- setup
  if (blockIdx.x == 0 && tid == 0) {
    a.hdr->batch = a.B; a.hdr->q_heads = a.Hq; a.hdr->kv_heads = a.Hkv; a.hdr->ctx = ctx;
    a.hdr->splits = a.S; a.hdr->positions_per_split = P; a.hdr->fmt = FMT; a.hdr->v_dim = 128;
    a.hdr->nwg = a.B * a.Hkv * a.S;
    a.hdr->launches = a.launches;
    a.hdr->k_row_bytes = T::CB + T::SB;
    a.hdr->v_row_bytes = T::CB + T::SB;
    a.hdr->live_off = a.live_off;
    a.hdr->kdrop_off = KSKIP ? a.kdrop_off : 0;
  }
  if (tid == 0) wto[0] = 0;
  if (kLut3 && tid < 64) lut3_tab[tid] = lut3_pair_entry(tid);
  // q of this group: per-head max |q| -> power-of-two prescale, then fp16 hi/lo rows
  float qv[4];
  {
    const int j = jq, ln = lnq;
    float m = 0.f;
    if (j < G) {
      if (a.q_bf16) {
        qv[0] = __uint_as_float(qraw.x << 16); qv[1] = __uint_as_float(qraw.x & 0xFFFF0000u);
        qv[2] = __uint_as_float(qraw.y << 16); qv[3] = __uint_as_float(qraw.y & 0xFFFF0000u);
      } else {
        qv[0] = __uint_as_float(qraw.x); qv[1] = __uint_as_float(qraw.y);
        qv[2] = __uint_as_float(qraw.z); qv[3] = __uint_as_float(qraw.w);
      }
      if constexpr (KSKIP) {
        // sigma * log2(e) * ||q_j|| of the query as given (the rotation of the
        // LUT3_WHT path keeps the norm): the bound's factor per head
        float ss = qv[0] * qv[0] + qv[1] * qv[1] + qv[2] * qv[2] + qv[3] * qv[3];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 32);
        if (ln == 0) qmax[j] = a.sigma_log2e * sqrtf(ss);
      }
      if constexpr (kRot) {
        // q' = H q / sqrt(128): dims 4ln + e; stages 1 and 2 inside the
        // thread, stages 4..64 with the thread ln ^ (h / 4) of the same head
        float t0 = qv[0] + qv[1], t1 = qv[0] - qv[1], t2 = qv[2] + qv[3], t3 = qv[2] - qv[3];
        qv[0] = t0 + t2; qv[1] = t1 + t3; qv[2] = t0 - t2; qv[3] = t1 - t3;
#pragma unroll
        for (int hh = 1; hh < 32; hh *= 2) {
          const bool upper = ln & hh;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __shfl_xor(qv[e], hh, 32);
            qv[e] = upper ? p - qv[e] : qv[e] + p;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[e] *= 0.08838834764831845f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(qv[e]));
    }
    // The 32 threads of a head are one half of a wave: the butterfly leaves
    // the head's max |q| in each of them, so the prescale, the fp16 hi/lo
    // rows and their bias sums are formed without a barrier. A thread's four
    // dims lie in one scale block; the blocks of the biased formats (q4_0,
    // q8_0) are dims 32bb .. 32bb + 31, the threads ln = 8bb .. 8bb + 7.
    if (j < 8) {
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
      float shi = 0.f, slo = 0.f;                             // this thread's part of the bias sums
      if (j < G) {
        const int ex = (m > 0.f) ? ilogbf(m) + 1 : 0;         // m * 2^-ex in [0.5, 1)
        if (ln == 0) hs[j] = ldexpf(a.sigma_log2e, ex) * T::kRowMul;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = ln * 4 + e;
          const float qs = ldexpf(qv[e], -ex);
          const _Float16 hi = _Float16(qs);
          const _Float16 lo = _Float16(qs - float(hi));
          int bb, kk, slot;
          T::locate(d, bb, kk, slot);
          qop[((2 * j) * 16 + bb * 4 + kk) * 8 + slot] = hi;
          qop[((2 * j + 1) * 16 + bb * 4 + kk) * 8 + slot] = lo;
          shi += float(hi);
          slo += float(lo);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = ln * 4 + e;
          const int bb = d >> 5, kk = (d >> 3) & 3;
          const int slot = d & 7;
          qop[((2 * j) * 16 + bb * 4 + kk) * 8 + slot] = _Float16(0.f);
          qop[((2 * j + 1) * 16 + bb * 4 + kk) * 8 + slot] = _Float16(0.f);
        }
      }
      if constexpr (T::kBias != 0.f) {
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          shi += __shfl_xor(shi, o, 32);
          slo += __shfl_xor(slo, o, 32);
        }
      }
      if ((ln & 7) == 0) {                                    // bias correction per (block, row)
        const int bb = ln >> 3;
        cst[bb * 16 + 2 * j] = -T::kBias * shi;
        cst[bb * 16 + 2 * j + 1] = -T::kBias * slo;
      }
    }
  }
  // key skipping: per-chunk summaries of this split and the context's largest
  // (LDS that the value pass's row lists use later: free until then)
  float* rown = reinterpret_cast<float*>(rowlist);                // [nch] largest key norm per chunk
  int* kcnt = reinterpret_cast<int*>(rown + P / kChunk);          // [4] list lengths, dropped positions
  uint8_t* kl1 = reinterpret_cast<uint8_t*>(kcnt + 4);            // [nch] chunks of a listed K pass
  uint8_t* kl2 = kl1 + P / kChunk;                                // [nch] chunks that are not candidates
  uint8_t* kdr = kl2 + P / kChunk;                                // [nch] 1: chunk dropped
  if constexpr (KSKIP) {
    const float wmx = max_wave(rmax);
    if (lane == 0) reinterpret_cast<float*>(wml)[wave] = wmx;
    const float* kn = a.knorm + int64_t(bg) * a.knorm_pitch;
    for (int c = tid; c < P / kChunk; c += kThreads) {
      const int k = pos0 / kChunk + c;
      rown[c] = k < nb_ctx ? kn[k] : 0.f;
      kdr[c] = 0;
    }
  }
  __syncthreads();

  // MFMA operands of this lane
  half8 A[4];
  floatx4 C0[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    A[bb] = *reinterpret_cast<const half8*>(&qop[(n16 * 16 + bb * 4 + kg) * 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) C0[bb][i] = cst[bb * 16 + 4 * kg + i];
  }
  const int j0 = 2 * kg, j1 = 2 * kg + 1;   // the two heads whose rows this lane group holds
  const float hs0 = (j0 < G) ? hs[j0] : 0.f;
  const float hs1 = (j1 < G) ? hs[j1] : 0.f;
  stamp(a, 1);

  // ---------------------------------------------------------------- phase 1: scores
  // Scores go to LDS; each lane keeps a running (max, sum exp2) of its two
  // heads, updated once per batch of tiles without branches.
  float m0 = -INFINITY, l0 = 0.f, m1 = -INFINITY, l1 = 0.f;
  auto score_batch = [&](auto listed, const Loaded* raw, int t0) {
    float sa[U], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sa[u] = sb[u] = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * kWaves;
      if (t >= ntl) break;                      // uniform across the wave
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const typename T::Raw ru = operands(raw[u]);
      if constexpr (T::kRowScale) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bb], T::deq(ru, bb, table), acc, 0, 0, 0);
        const float s = T::scale(ru, 0);
        acc[0] *= s; acc[1] *= s; acc[2] *= s; acc[3] *= s;
      } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[bb], T::deq(ru, bb, table), C0[bb], 0, 0, 0);
          const float s = T::scale(ru, bb);
          acc[0] = fmaf(s, d[0], acc[0]);
          acc[1] = fmaf(s, d[1], acc[1]);
          acc[2] = fmaf(s, d[2], acc[2]);
          acc[3] = fmaf(s, d[3], acc[3]);
        }
      }
      const int lp = trow(listed, t) + n16;
      const bool valid = (pos0 + lp) < ctx;
      const float s0 = valid ? (acc[0] + acc[1]) * hs0 : -INFINITY;
      const float s1 = valid ? (acc[2] + acc[3]) * hs1 : -INFINITY;
      if (j0 < G) sc[sidx(j0, lp)] = s0;
      if (j1 < G) sc[sidx(j1, lp)] = s1;
      sa[u] = s0;
      sb[u] = s1;
    }
    batch_stats<U>(m0, l0, sa);
    batch_stats<U>(m1, l1, sb);
  };
  constexpr int STRIDE = kWaves * U;                  // tiles between a wave's batches
  // One K pass over ntl tiles (all of the split's, or a listed pass's): the
  // loads of the next batch are issued before the current batch is scored,
  // unconditionally (past the split they read zeros without a memory
  // access), so no load depends on a branch and two batches stay in flight;
  // tiles past the pass are skipped inside score_batch.
  auto k_pass = [&](auto listed, bool preloaded) {
    const int nbat = (ntl + STRIDE - 1) / STRIDE;      // uniform
    if (!preloaded) load_tiles(listed, rawA, 0);
    if constexpr (kDouble) {
      for (int kb = 0; kb < nbat; kb += 2) {
        load_tiles(listed, rawB, kb + 1);
        score_batch(listed, rawA, wave + kb * STRIDE);
        load_tiles(listed, rawA, kb + 2);
        score_batch(listed, rawB, wave + (kb + 1) * STRIDE);
      }
    } else {
      for (int kb = 0; kb < nbat; ++kb) {
        if (kb > 0) load_tiles(listed, rawA, kb);
        score_batch(listed, rawA, wave + kb * STRIDE);
      }
    }
  };
  // split statistics of the tiles scored so far: merged over the 16 lanes of
  // a lane group, then over the waves, and published to `base`
  auto publish_stats = [&](u64* base, bool withhold) {
    {
      const float2 x0 = merge_row16(make_float2(m0, l0));
      const float2 x1 = merge_row16(make_float2(m1, l1));
      if (n16 == 0) {
        wml[wave * 8 + j0] = x0;
        wml[wave * 8 + j1] = x1;
      }
    }
    __syncthreads();
    if (tid < 128) {                                 // row j of 16 lanes merges head j over the 16 waves
      const int j = tid >> 4, w = tid & 15;
      float2 acc = (j < G) ? wml[w * 8 + j] : make_float2(-INFINITY, 0.f);
      acc = merge_row16(acc);
      if (w == 0 && j < G && !withhold) {
        u64* dst = base + ((int64_t(bg) * a.S + split) * G + j) * 2;
        put_tagged_f(dst, epoch, acc.x);
        put_tagged_f(dst + 1, epoch, acc.y);
        if constexpr (RUN) lse[j] = acc.x;           // the split's max: reference of its weights
      }
    }
    __syncthreads();                                 // wml is reused below
  };

  // ---------------------------------------------------------------- phase 2: LSE of the group
  // ---------------------------------------------------------------- phase 2: LSE of the group
  // Every workgroup gathers all split statistics of its group and merges
  // them itself (128 threads per head, fixed pattern, so every workgroup of
  // the group computes the same bits); no workgroup waits on another's LSE.
  auto gather_lse = [&](const u64* src, float* dst) {
    // The group's S*G (max, sum) pairs are contiguous 16-byte pieces (split
    // sp, head j at piece sp*G + j). Thread t takes pieces t and t + kThreads
    // (S*G <= 2048: at most 256 splits of at most 8 heads), both of head
    // t mod G; a wave merges its lanes of equal head with xor steps, the
    // waves' results are merged in wave order. The pattern is fixed, so every
    // workgroup of the group computes the same bits.
    const int nc = a.S * G;
    const __amdgpu_buffer_rsrc_t r = coherent_rsrc(src + int64_t(bg) * nc * 2, nc * 16);
    u32x4 v[2];
    bool use[2];
    int off[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = tid + k * kThreads;
      use[k] = c < nc;
      off[k] = use[k] ? c * 16 : 0;
      v[k] = use[k] ? peek2(r, off[k]) : u32x4{0u, epoch, 0u, epoch};
    }
    u64 none[1] = {0ull};
    const u64* const nop[1] = {a.split_ml};
    const bool nouse[1] = {false};
    if (settle_mixed(v, use, r, off, none, nop, nouse, epoch, a.hdr, a.spin_limit)) wto[0] = 1;
    float2 acc = make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (use[k]) acc = lse_merge(acc, make_float2(__uint_as_float(v[k].x), __uint_as_float(v[k].z)));
    acc = merge_class<G>(acc);                       // every lane: its head's merge over the wave
    if (lane < G) wml[wave * 8 + lane] = acc;
    __syncthreads();
    if (tid < 128) {                                 // row j of 16 lanes merges head j over the waves
      const int j = tid >> 4, w = tid & 15;
      float2 m = (j < G) ? wml[w * 8 + j] : make_float2(-INFINITY, 0.f);
      m = merge_row16(m);
      if (w == 0 && j < G) dst[j] = m.x + log2f(m.y);
    }
    __syncthreads();
  };

  if constexpr (!KSKIP) {
    k_pass(std::false_type{}, true);
  } else {
    // candidates: chunks inside the context whose largest key norm is at
    // least half the context's largest; the others inside the context are
    // tested after the exchange of the candidates' statistics
    float R = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) R = fmaxf(R, reinterpret_cast<const float*>(wml)[w]);
    const float half = 0.5f * R;
    const int nchs = P / kChunk;
    if (wave == 0) {                                 // lists in chunk order, 64 chunks per ballot
      int n1 = 0, n2 = 0;
      for (int c0 = 0; c0 < nchs; c0 += 64) {
        const int c = c0 + lane;
        const bool in = c < nchs && pos0 + c * kChunk < ctx;
        const bool cand = in && rown[c] >= half;
        const bool other = in && !cand;
        const u64 b1 = __ballot(cand), b2 = __ballot(other);
        const u64 below = (1ull << lane) - 1ull;
        if (cand) kl1[n1 + __popcll(b1 & below)] = uint8_t(c);
        if (other) kl2[n2 + __popcll(b2 & below)] = uint8_t(c);
        n1 += __popcll(b1);
        n2 += __popcll(b2);
      }
      if (lane == 0) { kcnt[0] = n1; kcnt[1] = n2; kcnt[2] = 0; kcnt[3] = 0; }
    }
    __syncthreads();
    const int n1 = kcnt[0], n2 = kcnt[1];
    klist = kl1;
    ntl = 4 * n1;
    k_pass(std::true_type{}, false);
    publish_stats(a.pre_ml, false);
    if (n2 > 0) {
      // lower bounds of the heads' LSE from every split's candidates, then the
      // drop test of this split's other chunks: every score of chunk c is at
      // most sigma * log2(e) * ||q_j|| * R_c (log2 domain), so its weight
      // under head j is at most |c| * 2^(that - L_j)
      gather_lse(a.pre_ml, lse);
      const float leps = log2f(1e-7f);
      for (int i = tid; i < n2; i += kThreads) {
        const int c = kl2[i];
        const int size = min(kChunk, ctx - pos0 - c * kChunk);
        const float lim = leps - log2f(float(size));
        bool drop = true;
#pragma unroll
        for (int j = 0; j < G; ++j) drop = drop && qmax[j] * rown[c] <= lse[j] + lim;
        kdr[c] = drop ? 1 : 0;
      }
      __syncthreads();
      if (wave == 0) {                               // the chunks that stay, in order: pass 2's list
        int n3 = 0, nd = 0;
        for (int i0 = 0; i0 < n2; i0 += 64) {
          const int i = i0 + lane;
          const int c = i < n2 ? kl2[i] : 0;
          const bool stay = i < n2 && !kdr[c];
          const bool gone = i < n2 && kdr[c];
          const u64 bs = __ballot(stay);
          if (stay) kl1[n3 + __popcll(bs & ((1ull << lane) - 1ull))] = uint8_t(c);
          n3 += __popcll(bs);
          int sz = gone ? min(kChunk, ctx - pos0 - c * kChunk) : 0;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) sz += __shfl_xor(sz, o);
          nd += sz;
        }
        if (lane == 0) { kcnt[2] = n3; kcnt[3] = nd; }
      }
      __syncthreads();
      ntl = 4 * kcnt[2];
      k_pass(std::true_type{}, false);
    }
    // chunks never scored (dropped, or past the context) hold -inf scores
    for (int i = tid; i < nchs * G * kChunk; i += kThreads) {
      const int c = i / (G * kChunk);
      if (kdr[c] || pos0 + c * kChunk >= ctx) sc[i] = -INFINITY;
    }
    if (a.kskip_out)
      for (int c = tid; c < nchs; c += kThreads) {
        const int k = pos0 / kChunk + c;
        if (k < nb_ctx) a.kskip_out[int64_t(bg) * nb_ctx + k] = kdr[c];
      }
    if (tid == 0) a.kdrop[wg] = kcnt[3];
  }
  // (test aid: split 0 of the first group withholds its statistics, so
  // every workgroup of that group waits in vain)
  publish_stats(a.split_ml, a.withhold && bg == 0 && split == 0);
  stamp(a, 2);
  const int nch = P / kChunk;                        // 64-position blocks of the split
  // single-pass rule: running LSE per (head, block) [G][nch] after block
  // summaries [G][nch], both in the K staging strip (free until the V pass)
  float2* csum = reinterpret_cast<float2*>(stg);
  float* rl = reinterpret_cast<float*>(csum + G * nch);
  if constexpr (!RUN) {
    gather_lse(a.split_ml, lse);
  } else {
    // block summaries: four adjacent threads per (head, block), 16 positions
    // each, combined with two exchanges (kThreads is a multiple of 64, so the
    // four are lanes of one wave in every pass of the loop)
    for (int it = tid; it < G * nch * 4; it += kThreads) {
      const int q4 = it & 3, jc = it >> 2;
      const int j = jc / nch, c = jc - j * nch;
      float m = -INFINITY, l = 0.f;
      const float* src = sc + sidx(j, c * kChunk + 16 * q4);
#pragma unroll
      for (int i = 0; i < 16; ++i) online_add(m, l, src[i]);
      float2 v = make_float2(m, l);
      v = lse_merge(v, make_float2(__shfl_xor(v.x, 1), __shfl_xor(v.y, 1)));
      v = lse_merge(v, make_float2(__shfl_xor(v.x, 2), __shfl_xor(v.y, 2)));
      if (q4 == 0) csum[jc] = v;
    }
    __syncthreads();
    if (tid < G) {                                   // prefix over the blocks in position order
      float2 acc = make_float2(-INFINITY, 0.f);
      for (int c = 0; c < nch; ++c) {
        acc = lse_merge(acc, csum[tid * nch + c]);
        rl[tid * nch + c] = acc.x + log2f(acc.y);
      }
    }
    __syncthreads();
  }
  stamp(a, 3);

  // ---------------------------------------------------------------- phase 3: sparse V pass
  // Wave w takes the 64-position chunks c = w (mod kWaves). With fewer
  // chunks than waves, chunk c goes to the waves w = c (mod nchunks), which
  // share its kept rows by rank (wave w takes ranks w / nchunks modulo their
  // count); each of them decides the chunk.
  // (a) It decides the keep bits of every head of the group for its chunks:
  //     a head keeps a position iff its normalized weight 2^(s - LSE)
  //     reaches the threshold, decided on the score as s >= LSE +
  //     log2(threshold) (the two differ only for weights within float32
  //     rounding of the threshold). A value row is fetched iff some head
  //     keeps it: the union of the heads' ballots goes straight to the
  //     wave's own row list. The scores stay in place: the value pass forms
  //     the weights of the rows it fetches (the same decision, then
  //     2^(s - LSE)).
  // (b) The wave then fetches only those rows. No other wave reads its list,
  //     so no barrier separates the decision from the value pass.
  // the hardware exp flushes results below 2^-126: exact for weights that a
  // normal threshold keeps, and for threshold 0 (such weights add < 2^-126);
  // a subnormal threshold needs the full-range exp2f
  const bool hw_exp = tau >= 1.17549435e-38f || tau == 0.f;
  const float ltau = tau > 0.f ? log2f(tau) : -INFINITY;
  float o0[G], o1[G], mass[G];
#pragma unroll
  for (int j = 0; j < G; ++j) { o0[j] = 0.f; o1[j] = 0.f; mass[j] = 0.f; }
  int kept_cnt = 0;
  const int nchunks = P / kChunk;
  uint16_t* mylist = rowlist + wave * list_cap;
  int nmine = 0, nlive = 0;                          // rows in the wave's list, chunks holding one
  // (not under the single-pass rule, whose decision writes the weights over
  // the scores: a second wave could read them back as scores)
  const bool few = !RUN && nchunks < kWaves;         // uniform
  const int cfirst = few ? wave % nchunks : wave;
  const int sub = few ? wave / nchunks : 0;          // this wave's share of a shared chunk's rows
  const int nsub = few ? (kWaves - 1 - cfirst) / nchunks + 1 : 1;
  {
    // a score past the context (or of a dropped key block) is -inf, below
    // every threshold (threshold 0 compares with the lowest finite value)
    float lsej[G], th[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      lsej[j] = lse[j];
      th[j] = fmaxf(lsej[j] + ltau, -3.4028235e38f);
    }
    // two of the wave's chunks per step: their scores are read together,
    // so the LDS latency is paid once per two chunks
    constexpr int CB = 2;
    for (int c0 = cfirst; c0 < nchunks; c0 += CB * kWaves) {
      float sv2[CB][G];
#pragma unroll
      for (int q = 0; q < CB; ++q) {
        const int c = min(c0 + q * kWaves, nchunks - 1);
        const float* base = sc + c * (G * kChunk) + lane;
#pragma unroll
        for (int j = 0; j < G; ++j) sv2[q][j] = base[j * kChunk];
      }
#pragma unroll
      for (int q = 0; q < CB; ++q) {
        const int c = c0 + q * kWaves;
        if (c >= nchunks) break;                      // uniform
        float* base = sc + c * (G * kChunk) + lane;
        const float (&sv)[G] = sv2[q];
        unsigned long long bal[G], uni = 0ull;
#pragma unroll
        for (int j = 0; j < G; ++j) {
          // single-pass rule: the reference is the running LSE of the block
          const float t = RUN ? fmaxf(rl[j * nch + c] + ltau, -3.4028235e38f) : th[j];
          bal[j] = __ballot(sv[j] >= t);
          uni |= bal[j];
          if (sub == 0) kept_cnt += __popcll(bal[j]);
        }
        if (uni) {                                    // uniform
          const int rank = __popcll(uni & ((1ull << lane) - 1ull));
          if (((uni >> lane) & 1ull) && rank % nsub == sub) mylist[nmine + rank / nsub] = uint16_t(c * kChunk + lane);
          nmine += (__popcll(uni) - sub + nsub - 1) / nsub;
          if (sub == 0) ++nlive;
        }
        if constexpr (RUN) {
          // single-pass rule: the running LSE of the blocks lives in the K
          // staging strip, which the value pass reuses, so the weights
          // (relative to the split's max, 0 where a head skips) replace the
          // scores here
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const bool keep = (bal[j] >> lane) & 1ull;
            const float x = sv[j] - lsej[j];
            base[j * kChunk] = keep ? (hw_exp ? ex2(x) : exp2f(x)) : 0.f;
          }
        }
        if (a.mask_out && sub == 0 && lane < 2) {
          const int word = (pos0 + c * kChunk) / 32 + lane;
          if (word < a.mask_words)
#pragma unroll
            for (int j = 0; j < G; ++j)
              a.mask_out[(int64_t(b) * a.Hq + g * G + j) * a.mask_words + word] = uint32_t(bal[j] >> (32 * lane));
        }
      }
    }
  }
  // single-pass rule: the running LSE lives in the K staging strips, which
  // the value pass below overwrites; every wave must be done reading it
  if constexpr (RUN) __syncthreads();
  const int rows_cnt = nmine | (nlive << 16);        // rows | live chunks << 16
  const int64_t pbase = int64_t(bg) * a.S + split;
  stamp(a, 7);
  stamp(a, 8);
  using VM = VMfma<FMT>;
  // weight of head j at split position i: 2^(s - LSE) if the head keeps the
  // position, else 0 (single-pass rule: formed in the keep-decision pass)
  auto weight = [&](int j, int i) __attribute__((always_inline)) -> float {
    const float sv = sc[sidx(j, i)];
    if constexpr (RUN) return sv;                    // formed in the keep-decision pass
    const float ref = lse[j];
    const float th = fmaxf(ref + ltau, -3.4028235e38f);
    const float x = sv - ref;
    return sv >= th ? (hw_exp ? ex2(x) : exp2f(x)) : 0.f;
  };
  // a wave with at least 8 rows sums them on MFMA (wave-uniform choice)
  const bool use_mfma = VM::kOn && nmine >= 8;
  floatx4 vacc[8];
  float vmass = 0.f;                                  // lanes of high-part rows: their head's weights
  // exponent e with every x = p * s of the wave's rows so far below 2^e; the
  // A operands hold x * 2^(15 - e) (kNoExp: no nonzero x yet)
  constexpr int kNoExp = -100000;
  int vexp = kNoExp;
#pragma unroll
  for (int t = 0; t < 8; ++t) vacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  {
    // This wave's rows in batches of 16, read with 16-byte loads (one or two
    // instructions per batch) that are kept D batches ahead in registers, then
    // staged in this wave's LDS strip (the list and the strip are written and
    // read by this wave only, and its LDS accesses complete in order).
    constexpr int VB = 16;
    constexpr int NL = T::CB / 16;                  // 16-byte pieces per row
    constexpr int NI = (VB * NL + 63) / 64;         // load instructions per batch
    // batches of loads in flight: LUT3 value rows (long dense runs, slow
    // per-row decode) gain from four; for q4_0 one measured fastest, and
    // q8_0 (two load instructions per batch) has no registers to spare
    constexpr int D = (FMT == KVQ_LUT3 || FMT == KVQ_LUT3_WHT) ? 4 : 1;
    uint8_t* vst = stg + wave * 16 * T::PITCH;
    static_assert(NI == 1 || NI == 2, "value row pieces per batch");
    struct VBuf { uint4 cv0, cv1; uint2 sv; };       // cv1 only when NI == 2
    // every lane loads (pieces past the batch re-read the batch's first row),
    // so the loads are not branched around and stay in registers
    auto load_piece = [&](int i, int k) __attribute__((always_inline)) -> uint4 {
      const int piece = 64 * i + lane, rr = piece / NL, ch = piece - rr * NL;
      const bool ok = piece < VB * NL && k + rr < nmine;
      const int64_t row = row0 + pos0 + mylist[ok ? k + rr : k];
      return *reinterpret_cast<const uint4*>(a.vc + row * T::CB + 16 * (ok ? ch : 0));
    };
    auto load_batch = [&](VBuf& vb, int k) __attribute__((always_inline)) {
      vb.cv0 = load_piece(0, k);
      if constexpr (NI == 2) vb.cv1 = load_piece(1, k);
      const bool sok = lane < VB && k + lane < nmine;
      const int64_t srow = row0 + pos0 + mylist[sok ? k + lane : k];
      if constexpr (T::SB == 8) vb.sv = *reinterpret_cast<const uint2*>(a.vs + srow * 8);
      else vb.sv = make_uint2(*reinterpret_cast<const uint16_t*>(a.vs + srow * T::SB), 0u);
    };
    // codes to the strip (transposed for the MFMA path of q4_0), scales after them
    auto stage_piece = [&](int i, const uint4& cv, int k, bool mf) __attribute__((always_inline)) {
      const int piece = 64 * i + lane, rr = piece / NL, ch = piece - rr * NL;
      if (piece < VB * NL && k + rr < nmine) {
        if constexpr (VM::kOn) {
          if (mf) VM::stage(vst + rr * T::PITCH, cv, ch);
          else *reinterpret_cast<uint4*>(vst + rr * T::PITCH + 16 * ch) = cv;
        } else {
          *reinterpret_cast<uint4*>(vst + rr * T::PITCH + 16 * ch) = cv;
        }
      }
    };
    auto stage_batch = [&](const VBuf& vb, int k, bool mf) __attribute__((always_inline)) {
      stage_piece(0, vb.cv0, k, mf);
      if constexpr (NI == 2) stage_piece(1, vb.cv1, k, mf);
      if (lane < VB && k + lane < nmine) {
        if constexpr (T::SB == 8) *reinterpret_cast<uint2*>(vst + lane * T::PITCH + T::CB) = vb.sv;
        else *reinterpret_cast<uint16_t*>(vst + lane * T::PITCH + T::CB) = uint16_t(vb.sv.x);
      }
    };
    // the batches in order, loads D batches ahead (the ring is D named
    // buffers, so it stays in registers)
    auto run_batches = [&](bool mf, auto&& compute) __attribute__((always_inline)) {
      VBuf v0, v1, v2, v3;                           // the first D are used
      auto step = [&](VBuf& vb, int k) __attribute__((always_inline)) -> bool {
        if (k >= nmine) return false;                // uniform across the wave
        stage_batch(vb, k, mf);
        if (k + D * VB < nmine) load_batch(vb, k + D * VB);
        compute(k);
        return true;
      };
      if (nmine == 0) return;                        // no rows: mylist holds nothing to read
      static_assert(D == 1 || D == 2 || D == 4, "batches in flight");
      load_batch(v0, 0);
      if constexpr (D >= 2)
        if (VB < nmine) load_batch(v1, VB);
      if constexpr (D == 4) {
        if (2 * VB < nmine) load_batch(v2, 2 * VB);
        if (3 * VB < nmine) load_batch(v3, 3 * VB);
      }
      for (int k0 = 0; k0 < nmine; k0 += D * VB) {
        if (!step(v0, k0)) break;
        if constexpr (D >= 2)
          if (!step(v1, k0 + VB)) break;
        if constexpr (D == 4) {
          if (!step(v2, k0 + 2 * VB)) break;
          if (!step(v3, k0 + 3 * VB)) break;
        }
      }
    };
    if constexpr (VM::kOn) {
      if (use_mfma)
        run_batches(true, [&](int k) __attribute__((always_inline)) {
          // lane (g, n) holds rows 4g .. 4g + 3; A row m is head m & 7, high
          // (m < 8) or low part
          const int g4 = lane >> 4, n16v = lane & 15, hj = n16v & 7;
          const bool lo_part = n16v >= 8;
          half4 B[8];
          VM::b_ops(vst, g4, n16v, table, B);
          float w[4];
          bool okr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = k + 4 * g4 + i;
            okr[i] = kk < nmine;
            w[i] = (okr[i] && hj < G) ? weight(hj, mylist[okr[i] ? kk : k]) : 0.f;
            if (!lo_part) vmass += w[i];
          }
          float x[VM::kBlocks][4];
          float xm = 0.f;
#pragma unroll
          for (int b = 0; b < VM::kBlocks; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[b][i] = okr[i] ? w[i] * VM::scale(vst + (4 * g4 + i) * T::PITCH, b) : 0.f;
              xm = fmaxf(xm, fabsf(x[b][i]));
            }
          // wave-uniform exponent of the batch's largest term (xm < 2^e)
          xm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, max_wave(xm))));
          if (xm > 0.f) {
            const int e = __builtin_amdgcn_frexp_expf(xm);
            if (e > vexp) {                          // rescale the sums to the new exponent (exact)
              const float f = vexp == kNoExp ? 0.f : __builtin_ldexpf(1.f, vexp - e);
#pragma unroll
              for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) vacc[t][i] *= f;
              vexp = e;
            }
          }
          const int sh = 15 - vexp;
#pragma unroll
          for (int b = 0; b < VM::kBlocks; ++b) {
            half4 A;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float xs = __builtin_ldexpf(x[b][i], sh);    // |xs| < 2^15
              const _Float16 h = _Float16(xs);
              A[i] = lo_part ? _Float16(xs - float(h)) : h;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
              if (t * VM::kBlocks / 8 == b) vacc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, B[t], vacc[t], 0, 0, 0);
          }
        });
    }
    if (!use_mfma)
      run_batches(false, [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          if (k + u >= nmine) break;
          const uint8_t* lr = vst + u * T::PITCH;
          const typename T::VRaw vr = T::vload(lr, lr + T::CB, lane);
          float v0, v1;
          T::vdeq(vr, table, v0, v1);
          const int pr = mylist[k + u];
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float pj = weight(j, pr);         // same for every lane of the wave
            o0[j] = fmaf(pj, v0, o0[j]);
            o1[j] = fmaf(pj, v1, o1[j]);
            mass[j] += pj;
          }
        }
      });
  }
  if (use_mfma) {
    // head h's weights are on lanes h, h + 16, h + 32, h + 48; a head's high
    // and low part rows are on lanes l and l + 32
    vmass = sum_pairs16(vmass);
    vmass = sum_pairs32(vmass);
    // undo the operand scale 2^(15 - vexp) (a power of two: exact)
    const float unscale = vexp == kNoExp ? 0.f : __builtin_ldexpf(1.f, vexp - 15);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) vacc[t][i] = sum_pairs32(vacc[t][i]) * unscale;
  }
  stamp(a, 9);

  // per-wave counters and kept mass (mass is wave-uniform: summed over the
  // wave's rows in row order; on the MFMA path lane h holds head h's)
  if (lane == 0) {
    wcount[wave] = kept_cnt;
    wrows[wave] = rows_cnt;
    wproc[wave] = nmine;
    if (!use_mfma)
#pragma unroll
      for (int j = 0; j < G; ++j) wmass[wave * G + j] = mass[j];
  }
  if (use_mfma && lane < G) wmass[wave * G + lane] = vmass;
  __syncthreads();                                   // all waves done with sc
  int wg_rows = 0, wg_kept = 0, wg_live = 0, nact = 0;
  uint32_t act = 0;                                  // waves that summed value rows
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wg_rows += wrows[w] & 0xFFFF;
    wg_live += wrows[w] >> 16;
    wg_kept += wcount[w];
    if (wproc[w] > 0) act |= 1u << w;
  }
  nact = __popc(act);
  // Whether this split publishes a partial output: the merge reads this word
  // with the partials and skips the partial of a split that keeps nothing
  // (which never writes one). A split whose wait gave up publishes its NaN
  // partial; under the single-pass rule every split publishes (its factor to
  // the group's LSE is only known later).
  const bool publishes = RUN || wto[0] != 0 || nact > 0;
  if (tid == 0) put_tagged(a.act + pbase, epoch, publishes ? 1u : 0u);
  float* fac = qmax;                                  // single-pass rule: per-head factor to the group LSE
  if constexpr (RUN) {
    // every workgroup takes part (the exchange also proves to the epoch
    // counter below that the whole group has read the epoch)
    gather_lse(a.split_ml, fac);
    if (tid < G) fac[tid] = exp2f(lse[tid] - fac[tid]);
    __syncthreads();
  }
  // a wait of this workgroup gave up (its statistics and weights are not the
  // call's): publish NaN, so every sum that uses them is NaN as well
  const bool bad = wto[0] != 0;
  if (nact == 0) {                                    // uniform: nothing kept
    // zeros (NaN after a wait gave up) only where the merge expects a partial
    if (publishes)
      for (int i = tid; i < G * 128; i += kThreads)
        put_tagged_f(a.partial + pbase * G * 128 + i, epoch, poison_if(bad, 0.f));
    if (tid < G) put_tagged_f(a.pmass + pbase * G + tid, epoch, poison_if(bad, 0.f));
  } else {
    // the partials of the waves that summed rows meet in LDS and are added in
    // ascending wave order; every thread publishes one word
    float* red = sc;                                 // [nact][G][128]
    if ((act >> wave) & 1u) {
      const int slot = __popc(act & ((1u << wave) - 1u));
      if (use_mfma) {
        // lane (g, n), g < 2: heads 4g + i, dims n + 16t
        if (lane < 32)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = 4 * (lane >> 4) + i;
            if (h < G)
#pragma unroll
              for (int t = 0; t < 8; ++t) red[(slot * G + h) * 128 + VM::dim(lane & 15, t)] = vacc[t][i];
          }
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          red[(slot * G + j) * 128 + 2 * lane] = o0[j];
          red[(slot * G + j) * 128 + 2 * lane + 1] = o1[j];
        }
      }
    }
    __syncthreads();
    if constexpr (kRot) {
      // the summed partial of every head is rotated back by one wave
      float* rot = reinterpret_cast<float*>(qop);    // [G][128] (the q operands are in registers)
      for (int i = tid; i < G * 128; i += kThreads) {
        float s = 0.f;
        for (int k = 0; k < nact; ++k) s += red[k * G * 128 + i];
        if constexpr (RUN) s *= fac[i >> 7];
        rot[i] = s;
      }
      __syncthreads();
      if (wave < G) {
        float v0 = rot[wave * 128 + lane], v1 = rot[wave * 128 + 64 + lane];
        wht_wave(lane, v0, v1);
        put_tagged_f(a.partial + pbase * G * 128 + wave * 128 + lane, epoch, poison_if(bad, v0));
        put_tagged_f(a.partial + pbase * G * 128 + wave * 128 + 64 + lane, epoch, poison_if(bad, v1));
      }
    } else {
      for (int i = tid; i < G * 128; i += kThreads) {
        float s = 0.f;
        for (int k = 0; k < nact; ++k) s += red[k * G * 128 + i];
        if constexpr (RUN) s *= fac[i >> 7];
        put_tagged_f(a.partial + pbase * G * 128 + i, epoch, poison_if(bad, s));
      }
    }
    if (tid < G) {
      float s = 0.f;
      for (int w = 0; w < kWaves; ++w)
        if ((act >> w) & 1u) s += wmass[w * G + tid];
      if constexpr (RUN) s *= fac[tid];
      put_tagged_f(a.pmass + pbase * G + tid, epoch, poison_if(bad, s));
    }
  }
  if (tid == 0) {
    put_tagged(a.flags + pbase, epoch, (uint32_t(wg_rows) << 18) | uint32_t(wg_kept));
    a.live[wg] = wg_live;                            // read by the host after the call
  }
  stamp(a, 4);

  // ---------------------------------------------------------------- phase 4: merge
  // Workgroup `split` of the group sums the slice [split*E, split*E + E) of
  // the group's G*128 outputs over all splits (a split that keeps no row
  // publishes no partial and counts as zeros) in ascending split order,
  // which is deterministic, and the kept mass of heads split, split+S, ... ;
  // split 0 also sums the group's counters. All words are read in one batch
  // and stale ones are re-read together; a partial piece is waited for only
  // when its split's early word says it publishes one.
  {
    constexpr int NE = G * 128;
    const int S = a.S;
    const int E = gqa_merge_slice(G, S);
    const int e0 = split * E;
    const int ne = e0 < NE ? (NE - e0 < E ? NE - e0 : E) : 0;
    const int nh = split < G ? (G - split + S - 1) / S : 0;
    const int nf = master ? S : 0;
    float* pv = sc;                                  // [ne][S]
    float* pm = pv + ne * S;                         // [nh][S]
    uint32_t* fl = reinterpret_cast<uint32_t*>(pm + nh * S);   // [S] (split 0)
    const int64_t gb = int64_t(bg) * S;
    __syncthreads();                                 // sc is free again
    // partials: 16-byte pieces (two words); consecutive threads take the
    // pieces of one split's slice, so a wave reads whole lines
    const int hc = ne >> 1;                          // pieces per split (ne is even)
    const bool use_p = tid < hc * S;
    const int sp_p = use_p ? tid / (hc > 0 ? hc : 1) : 0;
    const int k_p = use_p ? tid - sp_p * hc : 0;
    const __amdgpu_buffer_rsrc_t rp = coherent_rsrc(a.partial + gb * NE, S * NE * 8);
    const int poff = (sp_p * NE + e0 + 2 * k_p) * 8;
    u32x4 pw = use_p ? peek2(rp, poff) : u32x4{0u, epoch, 0u, epoch};
    const u64* asrc = a.act + gb + sp_p;
    u64 aw = use_p ? peek(asrc) : (u64(epoch) << 32) | 1u;
    constexpr int NW = 2 + 2;                        // mass and flag words per thread
    u64 w[NW];
    const u64* src[NW];
    bool use[NW];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + k * kThreads;
      use[k] = i < nh * S;
      const int j = use[k] ? split + (i / S) * S : 0, sp = use[k] ? i % S : 0;
      src[k] = a.pmass + (gb + sp) * G + j;
      use[2 + k] = i < nf;
      src[2 + k] = a.flags + gb + (use[2 + k] ? i : 0);
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = use[k] ? peek(src[k]) : 0ull;
    // Every workgroup of this group is past its LSE exchange, so each has
    // read the epoch; the last group to get here publishes the next call's
    // epoch. The counter's round trip overlaps the merge loads.
    uint32_t prev = 0;
    const bool counts = master && tid == 0;
    if (counts) prev = __hip_atomic_fetch_add(&a.hdr->groups_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    {
      // settle: the split's early word, then its piece if it publishes one,
      // plus the mass and flag words (bounded like settle_mixed)
      uint32_t spins = 0;
      while (true) {
        const bool afresh = uint32_t(aw >> 32) == epoch;
        bool stale = !afresh || (uint32_t(aw) != 0u && stale2(pw, epoch));
#pragma unroll
        for (int k = 0; k < NW; ++k) stale |= use[k] && uint32_t(w[k] >> 32) != epoch;
        if (!stale) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.spin_limit) {
          __hip_atomic_fetch_or(&a.hdr->status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          wto[0] = 1;
          break;
        }
        if (!afresh) aw = peek(asrc);
        else if (uint32_t(aw) != 0u && stale2(pw, epoch)) pw = peek2(rp, poff);
#pragma unroll
        for (int k = 0; k < NW; ++k)
          if (use[k] && uint32_t(w[k] >> 32) != epoch) w[k] = peek(src[k]);
      }
      if (uint32_t(aw) == 0u) pw = u32x4{0u, epoch, 0u, epoch};   // no partial: zeros
    }
    if (counts && prev == uint32_t(a.ngroups) - 1) {
      __hip_atomic_store(&a.hdr->groups_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.hdr->epoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    stamp(a, 5);
    if (use_p) {
      pv[(2 * k_p) * S + sp_p] = __uint_as_float(pw.x);
      pv[(2 * k_p + 1) * S + sp_p] = __uint_as_float(pw.z);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (use[k]) pm[tid + k * kThreads] = __uint_as_float(uint32_t(w[k]));
      if (use[2 + k]) fl[tid + k * kThreads] = uint32_t(w[2 + k]);
    }
    __syncthreads();
    const bool mbad = wto[0] != 0;                   // a wait gave up: the slice is NaN
    // one wave per sum: lane l adds splits l, l+64, ... in order, then a
    // fixed tree over the lanes (deterministic)
    if (S <= 16) {                                   // few splits: one thread per sum, in split order
      for (int job = tid; job < ne + nh; job += kThreads) {
        const float* src = job < ne ? pv + job * S : pm + (job - ne) * S;
        float v = 0.f;
        for (int sp = 0; sp < S; ++sp) v += src[sp];
        v = poison_if(mbad, v);
        if (job < ne) a.out[int64_t(bg) * NE + e0 + job] = v;
        else a.kept_mass[int64_t(bg) * G + split + (job - ne) * S] = v;
      }
    } else {
      for (int job = wave; job < ne + nh; job += kWaves) {
        const float* src = job < ne ? pv + job * S : pm + (job - ne) * S;
        float v = 0.f;
        for (int sp = lane; sp < S; sp += 64) v += src[sp];
        v = poison_if(mbad, sum_wave(v));
        if (lane == 0) {
          if (job < ne) a.out[int64_t(bg) * NE + e0 + job] = v;
          else a.kept_mass[int64_t(bg) * G + split + (job - ne) * S] = v;
        }
      }
    }
    if (master && wave == kWaves - 1) {
      unsigned long long kept_sum = 0, rows_sum = 0;
      for (int sp = lane; sp < S; sp += 64) {
        kept_sum += fl[sp] & 0x3FFFFu;
        rows_sum += fl[sp] >> 18;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        kept_sum += __shfl_xor(kept_sum, o);
        rows_sum += __shfl_xor(rows_sum, o);
      }
      if (lane == 0) {
        a.bgstat[2 * bg] = kept_sum;
        a.bgstat[2 * bg + 1] = rows_sum;
      }
    }
    stamp(a, 6);
  }
}

// LDS bytes the kernel needs for P positions per split and group size G.
size_t gqa_lds_bytes(int fmt, int G, int P, int S) {
  const size_t sc = size_t(gqa_sc_floats(G, P, S));
  const size_t list_cap = 64 * ((P / kChunk + kWaves - 1) / kWaves);
  const size_t pitch = fmt == KVQ_Q4_0 ? Traits<KVQ_Q4_0>::PITCH
                     : fmt == KVQ_Q8_0 ? Traits<KVQ_Q8_0>::PITCH
                                       : Traits<KVQ_LUT3>::PITCH;     // LUT3 and LUT3_WHT
  return sc * 4 + 16 * 128 * 2 + 64 * 4 + 3 * 8 * 4 + 2 * kWaves * 4 + size_t(kWaves) * G * 4 +
         size_t(kWaves) * 8 * 8 + (kWaves + 4) * 4 + size_t(kWaves) * list_cap * 2 + 16 +
         size_t(kWaves) * 16 * pitch + 64;
}

const void* gqa_kernel(int fmt, int G, int mode) {
#define KVQ_SEL(F, GG)                                                                      \
  if (fmt == F && G == GG)                                                                  \
    return mode == 1 ? reinterpret_cast<const void*>(&gqa_fused<F, GG, 1>)                  \
         : mode == 2 ? reinterpret_cast<const void*>(&gqa_fused<F, GG, 2>)                  \
                     : reinterpret_cast<const void*>(&gqa_fused<F, GG, 0>);
  KVQ_SEL(KVQ_Q4_0, 1) KVQ_SEL(KVQ_Q4_0, 2) KVQ_SEL(KVQ_Q4_0, 4) KVQ_SEL(KVQ_Q4_0, 8)
  KVQ_SEL(KVQ_Q8_0, 1) KVQ_SEL(KVQ_Q8_0, 2) KVQ_SEL(KVQ_Q8_0, 4) KVQ_SEL(KVQ_Q8_0, 8)
  KVQ_SEL(KVQ_LUT3, 1) KVQ_SEL(KVQ_LUT3, 2) KVQ_SEL(KVQ_LUT3, 4) KVQ_SEL(KVQ_LUT3, 8)
  KVQ_SEL(KVQ_LUT3_WHT, 1) KVQ_SEL(KVQ_LUT3_WHT, 2) KVQ_SEL(KVQ_LUT3_WHT, 4) KVQ_SEL(KVQ_LUT3_WHT, 8)
#undef KVQ_SEL
  return nullptr;
}

}  // namespace kvq
