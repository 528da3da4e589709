// Sparse-V decode attention for the MLA shape on gfx950: H query heads (a
// multiple of 32, at most 128) share one latent cache per sequence, stored as
// fp8 e4m3 with one fp32 scale per 128-element group (BlockWise1x128 of "FP8
// MLA KV compression projection", kernelindex.com: a 576-wide latent =
// kv_lora_rank 512 + qk_rope_head_dim 64). Scores use all 576 dims; values
// are the first 512. The skip rule is that of "Пропуск 90% работы по
// деквантизации…" (tproger.ru, section "Решение — не ускорять, а
// пропускать"): value rows whose normalized weight is below the threshold for
// every head are never read.
//
// Two launches on the caller's stream:
//  mla_scores  (one workgroup per (sequence, split); two waves per 32-head
//              block, each holding the bf16 query of its block for one half
//              of the latent (288 dims) in registers as MFMA operands, so two
//              waves share every SIMD)
//    1. streams 32-row latent tiles into a 4-deep LDS ring with direct
//       global->LDS loads (three tiles in flight); each wave scores its half
//       with v_mfma_f32_32x32x16_bf16 (fp8 -> bf16 with the hardware
//       converter, exact), applies the per-group fp32 scales to the fp32
//       accumulators and hands the rows the other wave finishes over through
//       LDS; the finished scores feed per-head (max, sum exp2) and a
//       per-(head, 32-position tile) maximum, one tile behind the MFMAs (at
//       threshold 0 with mla_out_dense they are also stored, every row);
//    2. every workgroup merges the split statistics of its sequence into
//       per-head log-sum-exps (one exchange of epoch-tagged words);
//    3. re-scores only the tiles whose maximum can reach the threshold
//       (identical code, identical bits), computes the normalized weights
//       and publishes, per kept row, its position and the weights of all
//       heads (0 where a head skips it); at threshold 0 with the stored
//       scores it publishes the positions only.
//  mla_out     (one workgroup per (sequence, 32 heads, 128 value dims))
//    sums p * v over the published rows of the sequence in split order and
//    row order (deterministic), reading only the kept latent rows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned long long u64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCoherentLoad = 16;                // buffer cache policy: sc1 (device-coherent read)

constexpr int D = 576;          // latent width (scores)
constexpr int DV = 512;         // value width
constexpr int HPAIRS = 9;       // MFMA step pairs (32 dims each) per latent half
constexpr int HSTEPS = 2 * HPAIRS;  // MFMA k-steps of 16 dims per latent half
constexpr int NGROUPS = 5;      // scale groups: 4 x 128 + 1 x 64
constexpr int ROW_LDS = 592;    // LDS pitch of a staged latent row: 37 x 16 bytes (odd), so the 16-byte
                                // reads of 8 consecutive rows hit distinct bank groups
constexpr int TILE = 32;        // positions per MFMA tile

// LDS ring of staged tiles. A buffer holds 32 latent rows at ROW_LDS pitch
// (37 slots of 16 bytes, the last one padding) followed by the 32 x 5 scales.
// Direct global->LDS loads write 64 consecutive 16-byte slots per wave
// instruction, so the padded layout is produced by the lane -> chunk mapping.
constexpr int PITCH16 = ROW_LDS / 16;          // 37
constexpr int NCHUNK_I = 19;                   // chunk instructions per tile (19 x 64 >= 32 x 37 slots)
constexpr int NSCALE_I = 3;                    // scale instructions per tile (3 x 64 >= 160 dwords)
constexpr int NDMA = NCHUNK_I + NSCALE_I;      // wave instructions per tile
constexpr int SC_OFF = NCHUNK_I * 64 * 16;     // byte offset of the scales in a buffer
constexpr int BUF_BYTES = SC_OFF + NSCALE_I * 64 * 4;
constexpr int NBUF = 4;                        // ring depth: three tiles in flight while one is scored

__device__ inline void put_tagged_f(u64* p, uint32_t epoch, float v) {
  __hip_atomic_store(p, (u64(epoch) << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline u64 peek(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Payload of a peeked tagged word once its tag is the call's epoch. Bounded:
// after `limit` retries the wait gives up, sets the sticky status bit and
// sets `gave_up` (the caller then writes NaN instead of what depended on it).
__device__ inline float settle_f(u64 w, const u64* p, uint32_t epoch, WsHeader* h, uint32_t limit, bool& gave_up) {
  uint32_t spins = 0;
  while (uint32_t(w >> 32) != epoch) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > limit) {
      __hip_atomic_fetch_or(&h->status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      gave_up = true;
      break;
    }
    w = peek(p);
  }
  return __uint_as_float(uint32_t(w));
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
// A split whose statistics wait gave up publishes its kept-row count with
// this bit set; the output kernels then write NaN for the whole sequence.
constexpr uint32_t kCountPoison = 0x80000000u;

__device__ inline float2 lse_merge(float2 x, float2 y) {
  const float M = fmaxf(x.x, y.x);
  if (M == -INFINITY) return make_float2(M, 0.f);
  return make_float2(M, x.y * exp2f(x.x - M) + y.y * exp2f(y.x - M));
}

// 2^x with the hardware instruction (results below the normal range flush to 0)
__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// The values of lanes j and j ^ 16 (rows 0 and 1, 2 and 3 of the wave):
// permlane16 swap of v with itself gives row 0 in rows 0 and 1 and row 1 in
// the second result (likewise rows 2 and 3).
__device__ inline float2 rows16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, v),
                                                  false, false);
  return make_float2(__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1])));
}

// Reduce N independent values over the 32 lanes of each wave half (max or
// sum), every lane getting the same bits. Steps: neighbour in quad, other
// pair in quad, mirrored quad in the 8-lane half row, mirrored half row, then
// the two rows combined in one order for both.
template <bool MAX, int N>
__device__ inline void reduce32(float (&v)[N]) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  float t[N];
#pragma unroll
  for (int e = 0; e < N; ++e) t[e] = dpp<0xB1>(v[e]);     // quad_perm [1,0,3,2]
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < N; ++e) t[e] = dpp<0x4E>(v[e]);     // quad_perm [2,3,0,1]
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < N; ++e) t[e] = dpp<0x141>(v[e]);    // row_half_mirror
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < N; ++e) t[e] = dpp<0x140>(v[e]);    // row_mirror
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float2 r = rows16(v[e]);
    v[e] = op(r.x, r.y);
  }
}

// 8 fp8 e4m3 bytes -> 8 bf16 (exact: every e4m3 value, subnormals included,
// is a bf16 value)
__device__ inline bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  u.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  u.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  u.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, u);
}

template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));   // vmcnt(N), other counters untouched
}

// Wait until at most k later tiles' direct loads of this wave are in flight
// (loads complete in order, so the tile before them has landed in LDS).
// Wave w issues the instructions j = w, w + NW, ... < NDMA of every tile.
template <int NW>
__device__ inline void wait_tiles(int k, int wave) {
  constexpr int base = NDMA / NW, extra = NDMA % NW;
  if (wave < extra) {
    if (k >= 2) wait_vm<2 * (base + 1)>(); else if (k == 1) wait_vm<base + 1>(); else wait_vm<0>();
  } else {
    if (k >= 2) wait_vm<2 * base>(); else if (k == 1) wait_vm<base>(); else wait_vm<0>();
  }
}

// Where this lane's direct loads of a tile come from: the sequence's code and
// scale planes, and per wave instruction i (instruction j = wave + NW * i of
// the tile) the row within the tile (or, for a scale instruction, the float
// within the tile's scales) and the byte offset within the row.
template <int NW>
struct TileSrc {
  static constexpr int NI = (NDMA + NW - 1) / NW;
  const uint8_t* kc;                  // row 0 of the sequence
  const float* ks;
  int ctx;
  int r[NI];
  int c[NI];
  __device__ TileSrc(const uint8_t* kc_, const float* ks_, int ctx_, int wave, int lane) : kc(kc_), ks(ks_), ctx(ctx_) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = wave + NW * i;
      if (j < NCHUNK_I) {
        const int sl = 64 * j + lane;
        const int rr = sl / PITCH16;
        r[i] = min(rr, TILE - 1);
        c[i] = 16 * min(sl - rr * PITCH16, D / 16 - 1);
      } else {
        r[i] = min(64 * (j - NCHUNK_I) + lane, TILE * NGROUPS - 1);
        c[i] = 0;
      }
    }
  }
};

// Issue this wave's direct loads of the tile starting at position `first`
// into buffer `dst`. Rows at or past ctx (and padding slots) repeat a real
// chunk of row ctx-1, so every instruction runs with all lanes and the
// per-wave instruction count is the same for every tile.
template <int NW>
__device__ __attribute__((always_inline)) inline void issue_tile(uint8_t* __restrict__ dst, const TileSrc<NW>& src,
                                                                 int first, int wave) {
#pragma unroll
  for (int i = 0; i < TileSrc<NW>::NI; ++i) {
    const int j = wave + NW * i;
    if (j < NCHUNK_I) {
      const int pos = min(first + src.r[i], src.ctx - 1);
      const uint8_t* g = src.kc + int64_t(pos) * D + src.c[i];
      __builtin_amdgcn_global_load_lds(g, dst + j * 1024, 16, 0, 0);
    } else if (j < NDMA) {
      const int gi = min(first * NGROUPS + src.r[i], src.ctx * NGROUPS - 1);
      const float* g = src.ks + gi;
      __builtin_amdgcn_global_load_lds(g, dst + SC_OFF + (j - NCHUNK_I) * 256, 4, 0, 0);
    }
  }
}

// Partial scores of one staged tile over latent half dh for the 32 heads of
// this wave's block x 32 positions, the fp32 group scales applied (log2
// domain). Half 0 holds scale groups 0 and 1 and the first 32 dims of group
// 4, half 1 groups 2 and 3 and the last 32 dims of group 4, so both halves
// have the same shape (segments of 4, 4 and 1 step pairs) and the code has
// no branch on dh. MFMA k order: step pair p (dims 32p..32p+31) takes, in
// k-half kh, the 16-byte chunk 2p + kh of the row, whose low 8 bytes feed
// step 2p and high 8 bytes step 2p + 1. The lane's 16 results are rows
// 8i + 4kh + j (i = 0..3); rows i = 0, 1 are the ones this wave finishes and
// rows i = 2, 3 go to the other half's wave. The half-1 wave holds its heads
// in the order h ^ 16, so that its rows i = 0, 1 are the heads the half-0
// wave hands over and the other way round.
__device__ __attribute__((always_inline)) inline void score_half(const uint8_t* __restrict__ buf,
                                                                 const bf16x8 (&A)[HSTEPS], float hs, int col, int kh,
                                                                 int dh, float (&own)[8], float (&send)[8]) {
  const uint8_t* src = buf + col * ROW_LDS + 16 * kh;
  uint4 ch[HPAIRS];
#pragma unroll
  for (int j = 0; j < 8; ++j) ch[j] = *reinterpret_cast<const uint4*>(src + 256 * dh + 32 * j);
  ch[8] = *reinterpret_cast<const uint4*>(src + 512 + 32 * dh);
  floatx16 c0 = {}, c1 = {}, c2 = {};
#pragma unroll
  for (int j = 0; j < HPAIRS; ++j) {
    const bf16x8 lo = fp8x8_to_bf16(ch[j].x, ch[j].y), hi = fp8x8_to_bf16(ch[j].z, ch[j].w);
    if (j < 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * j], lo, c0, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * j + 1], hi, c0, 0, 0, 0);
    } else if (j < 8) {
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * j], lo, c1, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * j + 1], hi, c1, 0, 0, 0);
    } else {
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * j], lo, c2, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * j + 1], hi, c2, 0, 0, 0);
    }
  }
  const float* sc = reinterpret_cast<const float*>(buf + SC_OFF) + col * NGROUPS;
  const float ga = sc[2 * dh] * hs, gb = sc[2 * dh + 1] * hs, gc = sc[4] * hs;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float v = fmaf(gc, c2[e], fmaf(gb, c1[e], ga * c0[e]));
    if (e < 8) own[e] = v; else send[e - 8] = v;
  }
}

// Both halves of one tile: this wave's own partial plus the one the other
// half's wave handed over (the sum is the same whichever wave adds), -inf
// past the context.
__device__ inline void finish_scores(const float (&own)[8], const float4* __restrict__ xr, bool valid,
                                     float (&s)[8]) {
  const float4 p0 = xr[0], p1 = xr[64];
  s[0] = own[0] + p0.x; s[1] = own[1] + p0.y; s[2] = own[2] + p0.z; s[3] = own[3] + p0.w;
  s[4] = own[4] + p1.x; s[5] = own[5] + p1.y; s[6] = own[6] + p1.z; s[7] = own[7] + p1.w;
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = valid ? s[e] : -INFINITY;
}

__device__ inline void hand_over(const float (&send)[8], float4* __restrict__ xw) {
  xw[0] = make_float4(send[0], send[1], send[2], send[3]);
  xw[64] = make_float4(send[4], send[5], send[6], send[7]);
}

// Maximum over the 32 columns of a wave half of each group of four rows of v
// (rows 4i .. 4i + 3, i = col & 1 in the result). The group's rows are
// merged in the lane; the lane pair col, col ^ 1 halves the two groups (each
// keeps the group of its parity and sends the other); the lanes that carry
// the same group (equal parity) are then combined: col ^ 2, the quads 4 and
// 8 lanes away in the 16-lane row, and the other 16 lanes.
__device__ __attribute__((always_inline)) inline float max32_group(const float (&v)[8], int col) {
  const float g0 = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  const float g1 = fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7]));
  const bool c0 = col & 1;
  float z = fmaxf(c0 ? g1 : g0, dpp<0xB1>(c0 ? g0 : g1));   // quad_perm [1,0,3,2]
  z = fmaxf(z, dpp<0x4E>(z));                                 // quad_perm [2,3,0,1]
  z = fmaxf(z, dpp<0x124>(z));                                // row_ror:4
  z = fmaxf(z, dpp<0x128>(z));                                // row_ror:8
  const float2 r = rows16(z);
  return fmaxf(r.x, r.y);
}

// Split statistics of the finished tiles 2u and 2u + 1 (8 head rows of this
// lane x its column each): each tile's maximum over the 32 columns and a
// group of four heads goes to the tile-maximum table entry of every head of
// the group (an upper bound of the head's own maximum, so the live-tile test
// stays conservative; one entry per 32-position tile when it fits in LDS,
// else one per pair: fine = false), lane col writing head 8 (col & 1) +
// ((col >> 1) & 3) of its rows (lanes that write one entry hold equal
// values); every lane
// keeps a running maximum m of its own scores and adds exp2(s - m) of its two
// scores to its sum l (rescaled when m grows); the lanes are merged once, at
// the end of the pass. No branch: the table index and value are selected.
__device__ __attribute__((always_inline)) inline void tile_stats(int u, const float (&s0)[8], const float (&s1)[8],
                                                                 float* __restrict__ tslot, bool fine, int col,
                                                                 float (&m)[8], float (&l)[8]) {
  const float t0 = max32_group(s0, col), t1 = max32_group(s1, col);
  const float tb = fmaxf(t0, t1);
  tslot[fine ? 2 * u : u] = fine ? t0 : tb;
  tslot[fine ? 2 * u + 1 : u] = fine ? t1 : tb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float mn = fmaxf(m[e], fmaxf(s0[e], s1[e]));
    const float ms = mn == -INFINITY ? 0.f : mn;  // nothing valid yet: every term is 0
    l[e] = l[e] * ex2(m[e] - ms) + ex2(s0[e] - ms) + ex2(s1[e] - ms);
    m[e] = mn;
  }
}

// Every score of a finished tile (threshold 0 with the dense output kernel):
// dkp points at this lane's heads (hrow) in row 0 of the split's block of kp;
// rows 8i+4kh+j of the lane are heads hrow + 8 (e >> 2) + (e & 3), column col
// is position t * 32 + col of the split.
__device__ __attribute__((always_inline)) inline void store_scores(float* __restrict__ dkp, int t, int col, int H,
                                                                   const float (&s)[8]) {
  float* d = dkp + (int64_t(t) * TILE + col) * H;
  *reinterpret_cast<float4*>(d) = make_float4(s[0], s[1], s[2], s[3]);
  *reinterpret_cast<float4*>(d + 8) = make_float4(s[4], s[5], s[6], s[7]);
}

// One tile of the scoring pass: start the direct loads of a later tile into
// `wr` (when given), score this wave's half of the tile staged in `rd`, finish
// the previous tile with the half the other wave handed over through `xr`,
// and hand over this tile's other half through `xw`. CLOSE: the previous tile
// closes a pair of tiles (fold the pair into the statistics), else it opens
// one (keep its scores in sprev). The restrict qualifiers state that the
// buffer being filled, the buffer being read, the exchange slots and the
// tile-maximum table are disjoint, so the compiler adds no wait for the
// direct loads in flight; the waits that order a tile's loads before its
// reads are explicit. Everything after the load issue is one basic block, so
// the scheduler can interleave the statistics with the MFMAs.
template <int NW, bool CLOSE>
__device__ __attribute__((always_inline)) inline void scoring_step(
    uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd, const float4* __restrict__ xr,
    float4* __restrict__ xw, float* __restrict__ tslot, const TileSrc<NW>& src, int next_first, int wave, int lane,
    int dh, int tprev, bool prev_valid, bool fine, const bf16x8 (&A)[HSTEPS], float hs, float (&own)[8],
    float (&m)[8], float (&l)[8], float (&sprev)[8], float* __restrict__ dkp, int H) {
  const int col = lane & 31, kh = lane >> 5;
  if (wr) issue_tile<NW>(wr, src, next_first, wave);
  float cur[8], send[8], s[8];
  score_half(rd, A, hs, col, kh, dh, cur, send);
  finish_scores(own, xr, prev_valid, s);
  if (dkp && tprev >= 0) store_scores(dkp, tprev, col, H, s);
  if constexpr (CLOSE) {
    tile_stats(tprev >> 1, sprev, s, tslot, fine, col, m, l);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) sprev[e] = s[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) own[e] = cur[e];
  hand_over(send, xw);
  // Schedule: the LDS reads first, then every MFMA followed by a few vector
  // instructions (conversions for the next MFMA, statistics of the previous
  // tile), so the vector work issues while the MFMA runs.
  __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
  for (int i = 0; i < 2 * HPAIRS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, CLOSE ? 9 : 5, 0);
  }
}

__device__ inline void stamp_mla(const MlaArgs& a, int k) {
  if (a.times && threadIdx.x == 0) a.times[int64_t(blockIdx.x) * 16 + k] = wall_clock64();
}

// s_waitcnt lgkmcnt(0) (this wave's LDS accesses are complete) then s_barrier
__device__ inline void bar_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

}  // namespace mla

using namespace mla;

// ----------------------------------------------------------------------------- scores
// NW waves = 2 per 32-head block: wave w takes head block w mod NB and latent
// half w / NB; the two waves of a block exchange partial scores through LDS.
template <int NW>
__global__ __launch_bounds__(64 * NW) void mla_scores(MlaArgs a) {
  constexpr int NT = 64 * NW;         // threads
  constexpr int NB = NW / 2;          // 32-head blocks
  constexpr int H = 32 * NB;          // heads
  extern __shared__ __align__(16) unsigned char smem[];
  const int P = a.P;
  const bool fine = a.tpe == 1;       // tile-maximum entries per 32-position tile (else per pair)
  const int NLT = P / (TILE * a.tpe); // tile-maximum entries per split
  uint8_t* ring = smem;                                                  // [NBUF][BUF_BYTES]
  float4* xbuf = reinterpret_cast<float4*>(ring + NBUF * BUF_BYTES);     // [2][NW][2][64] handed-over halves
  float* tmax = reinterpret_cast<float*>(xbuf + 2 * NW * 128);           // [H][NLT]
  float* lse = tmax + H * NLT;                                           // [H]
  int* live = reinterpret_cast<int*>(lse + H);                           // [NLT (+pad)]
  unsigned* keepmask = reinterpret_cast<unsigned*>(live + ((NLT + 3) & ~3));  // [2][TILE]
  int* misc = reinterpret_cast<int*>(keepmask + 2 * TILE);               // [8]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hb = wave % NB;           // head block
  const int dh = wave / NB;           // latent half
  const int partner = hb + NB * (1 - dh);
  const int b = blockIdx.x / a.S;
  const int split = blockIdx.x - b * a.S;
  const int pos0 = split * P;
  const int ctx = a.ctx;
  const int64_t row0 = int64_t(b) * a.cap;
  const uint32_t epoch = __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const int col = lane & 31;          // MFMA column / A row
  const int kh = lane >> 5;           // k half (0: dims 0..7 of a k-step, 1: 8..15)
  const int head_a = 32 * hb + (col ^ (16 * dh));  // head of this lane's A operand row (half 1: h ^ 16)
  const int hrow = 32 * hb + 16 * dh + 4 * kh;   // first head of this lane's finished rows (+8i + j)

  stamp_mla(a, 0);
  if (blockIdx.x == 0 && tid == 0) {
    a.hdr->batch = a.B; a.hdr->q_heads = H; a.hdr->kv_heads = 1; a.hdr->ctx = ctx;
    a.hdr->splits = a.S; a.hdr->positions_per_split = P; a.hdr->fmt = KVQ_FP8_B128; a.hdr->v_dim = DV;
    a.hdr->nwg = int(gridDim.x);
    a.hdr->k_row_bytes = D + 4 * NGROUPS;               // a whole latent row
    a.hdr->v_row_bytes = DV + 4 * (DV / 128);           // its value part
    a.hdr->live_off = a.live_off;
    a.hdr->launches = 2;                             // the scores kernel, then one output kernel
  }

  const TileSrc<NW> src(a.kc + row0 * D, reinterpret_cast<const float*>(a.ks) + row0 * NGROUPS, ctx, wave, lane);
  const int T = P / TILE;
  // the first three tiles start loading before the query is set up
  for (int t = 0; t < 3 && t < T; ++t) issue_tile<NW>(ring + t * BUF_BYTES, src, pos0 + t * TILE, wave);

  // ---------------------------------------------------------------- q operands
  // The bf16 query is the A operand as it is, in the k order of score_half:
  // local step pair j < 8 is pair 8 dh + j of the latent, pair 8 is 16 + dh.
  bf16x8 A[HSTEPS];
  {
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + (int64_t(b) * H + head_a) * D + 16 * kh;
#pragma unroll
    for (int ks = 0; ks < HSTEPS; ++ks) {
      const int gp = (ks >> 1) < 8 ? 8 * dh + (ks >> 1) : 16 + dh;
      A[ks] = *reinterpret_cast<const bf16x8*>(qh + 32 * gp + 8 * (ks & 1));
    }
  }
  const float hs = a.sigma_log2e;     // score scale: softmax scale * log2 e

  // ---------------------------------------------------------------- phase 1
  stamp_mla(a, 1);
  float m[8], l[8], sprev[8], own[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { m[e] = -INFINITY; l[e] = 0.f; sprev[e] = -INFINITY; own[e] = 0.f; }
  // the tile-maximum entry this lane writes: head 8 (col & 1) + ((col >> 1) & 3) of its rows
  float* tslot = tmax + (hrow + 8 * (col & 1) + ((col >> 1) & 3)) * NLT;
  auto xr_of = [&](int t) { return xbuf + ((t & 1) * NW + partner) * 128 + lane; };
  auto xw_of = [&](int t) { return xbuf + ((t & 1) * NW + wave) * 128 + lane; };
  auto wr_of = [&](int t) { return t + 3 < T ? ring + ((t + 3) % NBUF) * BUF_BYTES : nullptr; };
  // Step t scores tile t and finishes tile t - 1; a pair of tiles closes at
  // even t >= 2. Step 0 finishes nothing (its "previous" scores are dropped).
  // Before each step: this wave's loads of tile t have landed (wait_tiles),
  // then everyone's have and tile t - 1's halves are handed over (barrier),
  // and buffer (t + 3) mod NBUF is free.
  // threshold 0 with the dense output kernel: every finished tile's scores go to kp
  float* dkp = a.scores_out ? a.kp + (int64_t(b) * a.S + split) * P * H + hrow : nullptr;
  wait_tiles<NW>(min(2, T - 1), wave);
  bar_lds();
  scoring_step<NW, false>(wr_of(0), ring, xr_of(1), xw_of(0), tslot, src, pos0 + 3 * TILE, wave, lane, dh, -1, false,
                          fine, A, hs, own, m, l, sprev, dkp, H);
  for (int t = 1; t < T; t += 2) {
    wait_tiles<NW>(min(2, T - 1 - t), wave);
    bar_lds();
    scoring_step<NW, false>(wr_of(t), ring + (t % NBUF) * BUF_BYTES, xr_of(t - 1), xw_of(t), tslot, src,
                            pos0 + (t + 3) * TILE, wave, lane, dh, t - 1, pos0 + (t - 1) * TILE + col < ctx, fine,
                            A, hs, own, m, l, sprev, dkp, H);
    if (t + 1 < T) {
      wait_tiles<NW>(min(2, T - 2 - t), wave);
      bar_lds();
      scoring_step<NW, true>(wr_of(t + 1), ring + ((t + 1) % NBUF) * BUF_BYTES, xr_of(t), xw_of(t + 1), tslot, src,
                             pos0 + (t + 4) * TILE, wave, lane, dh, t, pos0 + t * TILE + col < ctx, fine, A, hs,
                             own, m, l, sprev, dkp, H);
    }
  }
  bar_lds();
  {
    float s[8];
    finish_scores(own, xr_of(T - 1), pos0 + (T - 1) * TILE + col < ctx, s);
    if (dkp) store_scores(dkp, T - 1, col, H, s);
    tile_stats((T - 1) >> 1, sprev, s, tslot, fine, col, m, l);
  }
  __syncthreads();
  stamp_mla(a, 2);
  // split statistics per head: the lanes' running maxima differ; take the
  // maximum over the 32 columns and rescale each lane's sum to it
  {
    float mm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mm[e] = m[e];
    reduce32<true, 8>(mm);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      l[e] = mm[e] == -INFINITY ? 0.f : l[e] * ex2(m[e] - mm[e]);
      m[e] = mm[e];
    }
  }
  reduce32<false, 8>(l);
  // (test aid: split 0 of the first sequence withholds its statistics, so
  // every workgroup of that sequence waits in vain)
  if (col == 0 && !(a.withhold && b == 0 && split == 0)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = hrow + 8 * (e >> 2) + (e & 3);
      u64* dst = a.split_ml + ((int64_t(b) * a.S + split) * H + h) * 2;
      put_tagged_f(dst, epoch, m[e]);
      put_tagged_f(dst + 1, epoch, l[e]);
    }
  }

  // ---------------------------------------------------------------- phase 2: LSE
  // Two hand-offs of epoch-tagged words. Stage 1: workgroup `split` merges
  // the split statistics of its share of the heads (hp = ceil(H / S) heads
  // from split * hp), one wave per head: lane l merges splits l, l + 64, ...
  // in order, then a fixed butterfly over the lanes; the head's log-sum-exp
  // is published. Stage 2: every workgroup reads the published log-sum-exps
  // of all heads, so all of them use the same bits. A workgroup reads
  // S * hp + H words instead of the S * H pairs of every split (64 KB per
  // workgroup, 16 MB per call at 32 splits and 128 heads).
  bool sbad;                                          // a wait of this workgroup gave up
  {
    bool gave_up = false;
    const int hp = (H + a.S - 1) / a.S;
    const int h0 = split * hp;
    const int nh = max(0, min(hp, H - h0));
    constexpr int SB = 4;                             // pairs per lane in flight
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(a.split_ml + int64_t(b) * a.S * H * 2, 0, a.S * H * 16, 0x00020000);
    for (int hh = wave; hh < nh; hh += NW) {          // uniform across the wave
      const int h = h0 + hh;
      float2 acc = make_float2(-INFINITY, 0.f);
      bool gone = false;
      for (int s0 = 0; s0 < a.S; s0 += 64 * SB) {
        u32x4 v[SB];
        int off[SB];
        bool use[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int sp = s0 + lane + 64 * u;
          use[u] = sp < a.S;
          off[u] = ((use[u] ? sp : 0) * H + h) * 16;
          v[u] = use[u] ? __builtin_amdgcn_raw_buffer_load_b128(r, off[u], 0, kCoherentLoad) : u32x4{0u, epoch, 0u, epoch};
        }
        for (uint32_t spins = 0;; ++spins) {
          bool stale = false;
#pragma unroll
          for (int u = 0; u < SB; ++u) stale |= use[u] && (v[u][1] != epoch || v[u][3] != epoch);
          if (!stale || gone) break;
          if (spins > a.spin_limit) {
            __hip_atomic_fetch_or(&a.hdr->status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            gone = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int u = 0; u < SB; ++u)
            if (use[u] && (v[u][1] != epoch || v[u][3] != epoch))
              v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off[u], 0, kCoherentLoad);
        }
#pragma unroll
        for (int u = 0; u < SB; ++u)
          if (use[u]) acc = lse_merge(acc, make_float2(__uint_as_float(v[u][0]), __uint_as_float(v[u][2])));
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) acc = lse_merge(acc, make_float2(__shfl_xor(acc.x, o), __shfl_xor(acc.y, o)));
      gone = __ballot(gone) != 0ull;
      if (lane == 0) put_tagged_f(a.lsep + int64_t(b) * H + h, epoch, poison_if(gone, acc.x + log2f(acc.y)));
      gave_up = gave_up || gone;
    }
    if (tid < H) {
      const u64* p = a.lsep + int64_t(b) * H + tid;
      bool late = false;
      const float x = settle_f(peek(p), p, epoch, a.hdr, a.spin_limit, late);
      // a head whose publisher gave up carries NaN (tested on the bits: the
      // kernel is compiled without NaN semantics)
      const uint32_t xb = __float_as_uint(x);
      gave_up = gave_up || late || ((xb & 0x7F800000u) == 0x7F800000u && (xb & 0x007FFFFFu) != 0u);
      lse[tid] = x;
    }
    sbad = __syncthreads_or(gave_up) != 0;
    if (tid < H) {
      lse[tid] = poison_if(sbad, lse[tid]);
      if (a.scores_out && split == 0) a.lseo[int64_t(b) * H + tid] = lse[tid];
    }
    __syncthreads();
  }
  stamp_mla(a, 3);
  if (a.scores_out) {
    // every row is kept and its scores are stored: publish the positions only
    const int nv = min(P, ctx - pos0);
    const int64_t kb = int64_t(b) * a.S + split;
    for (int i = tid; i < nv; i += NT) a.kpos[kb * P + i] = pos0 + i;
    if (a.mask_out) {                                  // every valid position is kept by every head
      const int nt = (nv + TILE - 1) / TILE;
      for (int i = tid; i < H * nt; i += NT) {
        const int h = i / nt, u = i - h * nt;
        const int left = nv - u * TILE;
        a.mask_out[(int64_t(b) * H + h) * a.mask_words + pos0 / TILE + u] = left >= TILE ? ~0u : (1u << left) - 1u;
      }
    }
    if (tid == 0) {
      a.kcount[kb] = nv;
      a.kpairs[kb] = nv * H;
      a.live[kb] = (nv + TILE - 1) / TILE;             // every tile holds kept rows
    }
    stamp_mla(a, 4);
    return;
  }

  // ---------------------------------------------------------------- phase 3: live tiles
  // A table entry (a 32-position tile, or a pair of them when the finer table
  // does not fit) is live when some head's maximum can reach the threshold
  // (a small margin keeps the test conservative); only the tiles of live
  // entries are re-read and re-scored, with the same code and so the same bits.
  const float log2tau = a.tau > 0.f ? log2f(a.tau) : -INFINITY;
  // every (tile, head) pair is tested by its own thread and marks its tile
  // (all marks store the same 1); wave 0 then compacts the marked tile ids in
  // position order, 64 at a time, in place (a chunk's marks are read before
  // any id lands at or below them)
  for (int u = tid; u < NLT; u += NT) live[u] = 0;
  if (tid < 2 * TILE) keepmask[tid] = 0u;
  if (tid == 0) misc[2] = 0;                           // kept pairs
  __syncthreads();
  for (int i = tid; i < NLT * H; i += NT) {
    const int u = i % NLT, h = i / NLT;
    if (pos0 + u * a.tpe * TILE < ctx && tmax[h * NLT + u] >= lse[h] + log2tau - 0.01f) live[u] = 1;
  }
  __syncthreads();
  if (a.mask_out) {
    // tiles that are not re-scored keep no position: their words are zero
    // (the re-scored tiles' words are written as their weights are formed)
    const int nt = min(P, ctx - pos0 + TILE - 1) / TILE;   // tiles holding a valid position
    for (int i = tid; i < H * nt; i += NT) {
      const int h = i / nt, u = i - h * nt;
      if (!live[u / a.tpe]) a.mask_out[(int64_t(b) * H + h) * a.mask_words + pos0 / TILE + u] = 0u;
    }
    __syncthreads();                                   // live[] is compacted in place below
  }
  if (wave == 0) {
    int nl = 0;
    for (int u0 = 0; u0 < NLT; u0 += 64) {
      const bool mk = u0 + lane < NLT && live[u0 + lane] != 0;
      const unsigned long long bal = __ballot(mk);
      if (mk) live[nl + __popcll(bal & ((1ull << lane) - 1ull))] = u0 + lane;
      nl += __popcll(bal);
    }
    if (lane == 0) misc[0] = nl;
  }
  __syncthreads();
  const int nlive = misc[0];

  // Register staging of 32-position tiles into ring buffers 0 and 1, two
  // register sets, so two tiles are in flight while one is scored.
  constexpr int CHUNKS = TILE * (D / 16);
  constexpr int PER = (CHUNKS + NT - 1) / NT;
  constexpr int NSC = TILE * NGROUPS;
  constexpr int PERS = (NSC + NT - 1) / NT;
  struct Stage {
    uint4 v[PER];
    float s[PERS];
  };
  Stage st0, st1;
  auto fetch = [&](Stage& st, int t) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      const int r = i / (D / 16), c = i - r * (D / 16);
      const int pos = pos0 + t * TILE + r;
      st.v[k] = (i < CHUNKS && pos < ctx) ? *reinterpret_cast<const uint4*>(a.kc + (row0 + pos) * D + c * 16)
                                          : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < PERS; ++k) {
      const int i = tid + k * NT;
      const int r = i / NGROUPS, gi = i - r * NGROUPS;
      const int pos = pos0 + t * TILE + r;
      st.s[k] = (i < NSC && pos < ctx) ? reinterpret_cast<const float*>(a.ks + (row0 + pos) * (4 * NGROUPS))[gi]
                                       : 0.f;
    }
  };
  auto put = [&](const Stage& st, uint8_t* buf) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      if (i < CHUNKS) {
        const int r = i / (D / 16), c = i - r * (D / 16);
        *reinterpret_cast<uint4*>(buf + r * ROW_LDS + c * 16) = st.v[k];
      }
    }
#pragma unroll
    for (int k = 0; k < PERS; ++k)
      if (tid + k * NT < NSC) reinterpret_cast<float*>(buf + SC_OFF)[tid + k * NT] = st.s[k];
  };
  // normalized weights of a finished tile and its keep bits (OR-ed per column)
  int kept_pairs = 0;
  auto weigh = [&](int k, int t, float (&p)[8]) {     // k: place in the list (slots), t: tile in the split
    float s[8];
    finish_scores(own, xbuf + ((k & 1) * NW + partner) * 128 + lane, pos0 + t * TILE + col < ctx, s);
    bool any = false;
    uint32_t word = 0u;                               // keep bits of this lane's mask word (lanes 8i + j, j < 8)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = exp2f(s[e] - lse[hrow + 8 * (e >> 2) + (e & 3)]);   // denormal-exact
      const bool keep = (s[e] != -INFINITY) && pe >= a.tau;
      p[e] = keep ? pe : 0.f;
      any |= keep;
      kept_pairs += keep ? 1 : 0;
      if (a.mask_out) {
        // columns 0..31 of head hrow + 8(e >> 2) + (e & 3) in the low half of
        // the ballot, those of the head 4 above (kh = 1) in the high half
        const unsigned long long bal = __ballot(keep);
        if ((lane & 31) == e) word = kh ? uint32_t(bal >> 32) : uint32_t(bal);
      }
    }
    // (the second tile of a 64-position entry can lie past the context: no word)
    const int widx = (pos0 + t * TILE) / TILE;
    if (a.mask_out && (lane & 31) < 8 && widx < a.mask_words) {
      const int e = lane & 31;
      const int h = hrow + 8 * (e >> 2) + (e & 3);
      a.mask_out[(int64_t(b) * H + h) * a.mask_words + widx] = word;
    }
    if (any) atomicOr(&keepmask[(k & 1) * TILE + col], 1u);
  };
  // row index of each kept column: the running count plus the kept columns
  // before it (every wave derives the same numbers from the same bits)
  const int64_t kbase = int64_t(b) * a.S + split;
  int nkept = 0;
  auto publish = [&](int k, int t, const float (&p)[8]) {
    const unsigned km = lane < TILE ? keepmask[(k & 1) * TILE + lane] : 0u;
    const unsigned cm = unsigned(__ballot(km != 0u));
    if ((cm >> col) & 1u) {
      const int idx = nkept + __popc(cm & ((1u << col) - 1u));
      if (wave == 0 && kh == 0) a.kpos[kbase * P + idx] = pos0 + t * TILE + col;
      float* dst = a.kp + (kbase * P + idx) * H + hrow;
      *reinterpret_cast<float4*>(dst) = make_float4(p[0], p[1], p[2], p[3]);
      *reinterpret_cast<float4*>(dst + 8) = make_float4(p[4], p[5], p[6], p[7]);
    }
    nkept += __popc(cm);
  };
  const int n3 = a.tpe * nlive;                       // 32-position tiles to re-score
  auto tile_at = [&](int k) { return fine ? live[k] : 2 * live[k >> 1] + (k & 1); };
  // tile k is scored from buffer k % 2; even tiles are staged through st0,
  // odd ones through st1. Step k first stages tile k + 1 (loaded two steps
  // earlier) into the buffer tile k - 1 used and starts loading tile k + 3
  // into the set it came from.
  if (n3 > 0) fetch(st0, tile_at(0));
  if (n3 > 1) fetch(st1, tile_at(1));
  if (n3 > 0) put(st0, ring);
  if (n3 > 2) fetch(st0, tile_at(2));
  auto step = [&](int k, Stage& nx) {
    bar_lds();                                         // tile k staged; tile k - 1's halves handed over
    if (k + 1 < n3) {
      put(nx, ring + ((k + 1) & 1) * BUF_BYTES);
      if (k + 3 < n3) fetch(nx, tile_at(k + 3));
    }
    if (k >= 2 && wave == 0 && lane < TILE) keepmask[(k & 1) * TILE + lane] = 0u;   // read two tiles ago
    float cur[8], send[8];
    score_half(ring + (k & 1) * BUF_BYTES, A, hs, col, kh, dh, cur, send);
    float p[8];
    if (k > 0) weigh(k - 1, tile_at(k - 1), p);
#pragma unroll
    for (int e = 0; e < 8; ++e) own[e] = cur[e];
    hand_over(send, xbuf + ((k & 1) * NW + wave) * 128 + lane);
    bar_lds();                                         // keep bits of tile k - 1 complete
    if (k > 0) publish(k - 1, tile_at(k - 1), p);
  };
  for (int k = 0; k < n3; k += 2) {
    step(k, st1);
    if (k + 1 < n3) step(k + 1, st0);
  }
  if (n3 > 0) {
    bar_lds();
    float p[8];
    weigh(n3 - 1, tile_at(n3 - 1), p);
    bar_lds();
    publish(n3 - 1, tile_at(n3 - 1), p);
  }
  // kept pairs of the split
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kept_pairs += __shfl_xor(kept_pairs, o);
  if (lane == 0) atomicAdd(&misc[2], kept_pairs);
  __syncthreads();
  if (tid == 0) {
    a.kcount[kbase] = int32_t(uint32_t(nkept) | (sbad ? kCountPoison : 0u));
    a.kpairs[kbase] = misc[2];
    a.live[kbase] = n3;                                // tiles re-scored (those that could keep a row)
  }
  stamp_mla(a, 4);
}

// ----------------------------------------------------------------------------- out
// Output block (sequence b, 32 heads hb, 128-dim value group g): out[h][d] =
// sum over the sequence's kept rows r of p[h][r] * v[r][d], a contraction over
// rows on v_mfma_f32_32x32x16_bf16 (M = heads, N = dims, K = rows; wave w owns
// dims 32w..32w+31 of the group). Exact operands: v is the e4m3 code converted
// to bf16 (exact) and the row's fp32 group scale goes to the weight side,
// p * scale (one fp32 rounding) split into three bf16 terms that add up to it
// exactly (8 + 8 + 8 significant bits); each term is a separate MFMA into the
// same fp32 accumulator. Rows are taken in split order and, within a split, in
// position order, 64 at a time; both operands are staged transposed in LDS
// (rows contiguous per head / dim), and the next 64 rows are loaded while the
// current ones are multiplied.
//
// R workgroups share a block, each taking one range of the kept rows; with N
// kept rows, min(R, ceil(N / kOutMinRows)) ranges are used. One range writes
// the block directly. Several write their partial sums to the workspace and
// count themselves done; the last to finish (after a device-scope fence)
// adds the partials in range order, so the result does not depend on timing.
constexpr int OUT_CHUNK = 64;                   // rows per LDS stage (4 MFMA k-steps)
constexpr int OUT_PITCH = OUT_CHUNK + 8;        // bf16 per staged head / dim line (bank spread)
constexpr int OUT_MAX_S = 1024;                 // splits per sequence the prefix table holds

__device__ inline uint16_t bf16_bits_rne(float x) {  // exact-to-nearest-even fp32 -> bf16
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline float bf16_value(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// One staged row of an output chunk: 32 value dims of the group (quarter sq
// of the group's 128), the group scale, and the weights of 8 heads.
struct OutRow {
  uint4 v0, v1;
  float sc;
  float pw[8];
};

__global__ __launch_bounds__(256) void mla_out(MlaArgs a) {
  __shared__ __align__(16) uint16_t vt[128 * OUT_PITCH];            // [dim][row] bf16 values
  __shared__ __align__(16) uint16_t pt[3 * 32 * OUT_PITCH];         // [term][head][row] bf16 weight terms
  __shared__ int pre[OUT_MAX_S + 1];                                // exclusive prefix of kept rows per split
  __shared__ float mpart[256][8];                                   // kept-mass partials [thread][head slot]
  __shared__ long long cnt[4];
  __shared__ int last;

  const int H = a.Hq;
  const int nhb = H / 32;
  const int R = a.R;
  int blk = blockIdx.x;
  const int rg = blk % R;
  blk /= R;
  const int g = blk & 3;
  blk >>= 2;
  const int hb = blk % nhb, b = blk / nhb;
  const int obk = (b * nhb + hb) * 4 + g;          // output block index
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S;
  const int64_t row0 = int64_t(b) * a.cap;
  const uint32_t epoch_next =
      __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // kept rows per split: one batch of loads, then an exclusive prefix sum
  long long pairs_part = 0;
  bool obad = false;                                  // a split of the sequence gave up a wait: NaN out
  {
    int c[OUT_MAX_S / 256];
#pragma unroll
    for (int k = 0; k < OUT_MAX_S / 256; ++k) {
      const int sp = tid * (OUT_MAX_S / 256) + k;
      c[k] = sp < S ? a.kcount[int64_t(b) * S + sp] : 0;
      obad |= (uint32_t(c[k]) & kCountPoison) != 0u;
      c[k] &= int(~kCountPoison);
      if (sp < S) pairs_part += a.kpairs[int64_t(b) * S + sp];
    }
    int local = 0;
#pragma unroll
    for (int k = 0; k < OUT_MAX_S / 256; ++k) local += c[k];
    // block-wide exclusive scan of the per-thread sums (wave scan, then waves)
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) pre[OUT_MAX_S - 4 + wave] = incl;   // wave totals parked at the table's end
    obad = __syncthreads_or(obad) != 0;
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += pre[OUT_MAX_S - 4 + w];
    const int total = pre[OUT_MAX_S - 4] + pre[OUT_MAX_S - 3] + pre[OUT_MAX_S - 2] + pre[OUT_MAX_S - 1];
    __syncthreads();
    int run = wbase + incl - local;
#pragma unroll
    for (int k = 0; k < OUT_MAX_S / 256; ++k) {
      pre[tid * (OUT_MAX_S / 256) + k] = run;
      run += c[k];
    }
    if (tid == 0) pre[OUT_MAX_S] = total;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pairs_part += __shfl_xor(pairs_part, o);
    if (lane == 0) cnt[wave] = pairs_part;
    __syncthreads();
  }
  const int N = pre[OUT_MAX_S];
  int nr = (N + kOutMinRows - 1) / kOutMinRows;    // row ranges in use (uniform over the block's workgroups)
  nr = nr < 1 ? 1 : nr > R ? R : nr;
  const bool active = rg < nr;
  const int rbeg = active ? int(int64_t(N) * rg / nr) : 0;
  const int rend = active ? int(int64_t(N) * (rg + 1) / nr) : 0;

  floatx16 acc = {};
  float mass[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mass[j] = 0.f;
  const int col = lane & 31, kh = lane >> 5;
  // staging roles: row sr of the chunk, quarter sq of the group's dims and
  // heads 8sq..8sq+7; a thread's rows advance in order, so its split index
  // only moves forward
  const int sr = tid >> 2, sq = tid & 3;
  int sp = 0;
  {
    const int r = rbeg + sr;                       // last split whose prefix is <= r (binary search)
    if (r < rend) {
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= r) lo = mid; else hi = mid - 1;
      }
      sp = lo;
    }
  }
  auto fetch = [&](int r, OutRow& o) {
    o.v0 = make_uint4(0u, 0u, 0u, 0u);
    o.v1 = o.v0;
    o.sc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o.pw[j] = 0.f;
    if (r < rend) {
      while (sp + 1 < S && pre[sp + 1] <= r) ++sp;
      const int64_t kb = int64_t(b) * S + sp;
      const int64_t idx = kb * a.P + (r - pre[sp]);
      const int pos = a.kpos[idx];
      const uint8_t* vrow = a.kc + (row0 + pos) * D + 128 * g + 32 * sq;
      o.v0 = *reinterpret_cast<const uint4*>(vrow);
      o.v1 = *reinterpret_cast<const uint4*>(vrow + 16);
      o.sc = reinterpret_cast<const float*>(a.ks + (row0 + pos) * (4 * NGROUPS))[g];
      const float4 p0 = *reinterpret_cast<const float4*>(a.kp + idx * H + 32 * hb + 8 * sq);
      const float4 p1 = *reinterpret_cast<const float4*>(a.kp + idx * H + 32 * hb + 8 * sq + 4);
      o.pw[0] = p0.x; o.pw[1] = p0.y; o.pw[2] = p0.z; o.pw[3] = p0.w;
      o.pw[4] = p1.x; o.pw[5] = p1.y; o.pw[6] = p1.z; o.pw[7] = p1.w;
    }
  };
  OutRow cur, nxt;
  fetch(rbeg + sr, cur);
  for (int c0 = rbeg; c0 < rend; c0 += OUT_CHUNK) {
    // values: 32 dims of row sr -> bf16, transposed into vt[dim][row]
    {
      const uint32_t w[8] = {cur.v0.x, cur.v0.y, cur.v0.z, cur.v0.w, cur.v1.x, cur.v1.y, cur.v1.z, cur.v1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t lo2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.0f, false));
        const uint32_t hi2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[k], 1.0f, true));
        const int d = 32 * sq + 4 * k;
        vt[(d + 0) * OUT_PITCH + sr] = uint16_t(lo2);
        vt[(d + 1) * OUT_PITCH + sr] = uint16_t(lo2 >> 16);
        vt[(d + 2) * OUT_PITCH + sr] = uint16_t(hi2);
        vt[(d + 3) * OUT_PITCH + sr] = uint16_t(hi2 >> 16);
      }
    }
    // weights: p * scale as three bf16 terms, transposed into pt[term][head][row]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mass[j] += cur.pw[j];
      const float x = cur.pw[j] * cur.sc;
      const uint16_t t0 = bf16_bits_rne(x);
      const float r1 = x - bf16_value(t0);
      const uint16_t t1 = bf16_bits_rne(r1);
      const uint16_t t2 = bf16_bits_rne(r1 - bf16_value(t1));
      const int h = 8 * sq + j;
      pt[(0 * 32 + h) * OUT_PITCH + sr] = t0;
      pt[(1 * 32 + h) * OUT_PITCH + sr] = t1;
      pt[(2 * 32 + h) * OUT_PITCH + sr] = t2;
    }
    fetch(c0 + OUT_CHUNK + sr, nxt);                 // the next rows load during the products
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < OUT_CHUNK / 16; ++ks) {
      const int k0 = 16 * ks + 8 * kh;
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&vt[(32 * wave + col) * OUT_PITCH + k0]);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&pt[(t * 32 + col) * OUT_PITCH + k0]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
    }
    __syncthreads();                                 // the next chunk reuses vt / pt
    cur = nxt;
  }
  // accumulator 4i+j of the lane: head 8i + 4kh + j, dim 32*wave + col of the group
  const int64_t ob_off = (int64_t(b) * H + 32 * hb) * DV + 128 * g + 32 * wave + col;
  float* part = a.opart + (int64_t(obk) * R + rg) * 32 * 128 + 32 * wave + col;   // [32 heads][128 dims]
  if (active) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 8 * i + 4 * kh + j;
        if (nr == 1) a.out[ob_off + int64_t(h) * DV] = poison_if(obad, acc[4 * i + j]);
        else part[h * 128] = poison_if(obad, acc[4 * i + j]);
      }
  }
  // kept mass of the 32 heads (g == 0): thread t summed the rows t/4 (mod 64)
  // of heads 8*(t%4)..+7; the 64 threads of a head are added in thread order
  if (g == 0 && active) {
#pragma unroll
    for (int j = 0; j < 8; ++j) mpart[tid][j] = mass[j];
    __syncthreads();
    if (tid < 32) {
      const int q = tid >> 3, j = tid & 7;
      float m = 0.f;
      for (int t = q; t < 256; t += 4) m += mpart[t][j];
      m = poison_if(obad, m);
      if (nr == 1) a.kept_mass[int64_t(b) * H + 32 * hb + 8 * q + j] = m;
      else a.mpart[(int64_t(b * nhb + hb) * R + rg) * 32 + 8 * q + j] = m;
    }
  }
  if (nr > 1 && active) {
    // the last range of the block to finish adds the partials in range order
    __threadfence();
    __syncthreads();
    if (tid == 0) last = atomicAdd(&a.ocnt[obk], 1u) == uint32_t(nr - 1);
    __syncthreads();
    if (last) {
      __threadfence();
      const float* p0 = a.opart + int64_t(obk) * R * 32 * 128;
      for (int e = tid; e < 32 * 128; e += 256) {
        float v = 0.f;
        for (int k = 0; k < nr; ++k) v += p0[int64_t(k) * 32 * 128 + e];
        a.out[(int64_t(b) * H + 32 * hb + (e >> 7)) * DV + 128 * g + (e & 127)] = v;
      }
      if (g == 0 && tid < 32) {
        float m = 0.f;
        for (int k = 0; k < nr; ++k) m += a.mpart[(int64_t(b * nhb + hb) * R + k) * 32 + tid];
        a.kept_mass[int64_t(b) * H + 32 * hb + tid] = m;
      }
      if (tid == 0) a.ocnt[obk] = 0u;                // ready for the next call
    }
  }
  if (hb == 0 && g == 0 && rg == 0 && tid == 0) {
    a.bgstat[2 * b] = (unsigned long long)(cnt[0] + cnt[1] + cnt[2] + cnt[3]);
    a.bgstat[2 * b + 1] = (unsigned long long)N;
  }
  // the last workgroup advances the epoch for the next call
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.hdr->groups_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(&a.hdr->groups_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.hdr->epoch, epoch_next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ----------------------------------------------------------------------------- out, every row kept
// Threshold 0 keeps every row, and the blocks of mla_out would each convert
// the same value rows and split the same weights. Here one workgroup takes a
// range of rows of a sequence for 64 of its heads and all 512 value dims:
// eight waves, two per SIMD (one's vector work and waits overlap the other's
// MFMAs); wave w owns heads 32(w/4)..+31 of the 64 and value group w%4 (four
// MFMA column tiles of 32 dims). A 64-row chunk is staged once: values
// converted to bf16 (exact) and transposed [dim][slot], weights transposed
// [head][slot] in fp32 (the scores kernel stored every row's log2-domain
// scores; the weight exp2(score - LSE) is formed here, as that kernel forms
// kept weights), group scales [group][slot]. Loads are coalesced (32 lanes
// read one 512-byte value row, 16 lanes one row's 64 scores). The
// chunk's rows take the MFMA k order slot 8b + m <- row b + 8m: a thread
// loads rows b + 8m, m = 4s..4s+3, of 16 dims, so each of its LDS writes is
// 8 bytes (4 slots of one dim). Unit (dim d, block b) of 16 bytes sits at
// 8 * (d ^ ((d >> 4) & 1)) + ((b + (d >> 1) + (d >> 5)) & 7): the 16 lanes of
// an operand read (consecutive dims, one block) fall in 16 different bank
// groups, and so do dims 16 apart (the writes). Each wave forms its A
// operand from its heads' weights times its group's scale, split into two
// bf16 terms: the product rounded to nearest, then its remainder (exact in
// fp32) rounded to nearest, so the pair carries it within 2^-17 relative
// (mla_out keeps a third term; here the conversions bound the chunk time).
// The R ranges of a sequence write fp32 partial sums, mark themselves done
// with a tagged word (after a device-scope fence), wait for the other ranges
// and then each adds, in range order, one slice of the sequence's outputs
// (all R workgroups of a sequence are resident: the plan launches at most one
// per CU).
constexpr int DN_CHUNK = 64;                     // rows per stage
constexpr int DN_SEG = 2048;                     // rows whose (slot, position) are looked up at once
constexpr int DN_PP = DN_CHUNK + 4;              // floats per staged head line (16-byte rows)
constexpr int DN_NT = kDenseOutThreads;          // threads per workgroup

size_t mla_out_dense_lds(int) {
  return size_t(DV) * DN_CHUNK * 2 + size_t(64) * DN_PP * 4 + size_t(DN_CHUNK) * 4 * 4 + size_t(OUT_MAX_S + 4) * 4 +
         size_t(DN_SEG) * 8;
}

constexpr int DN_HW = 64;                        // heads per workgroup

__device__ inline int dn_unit(int d, int b) {    // 16-byte unit of (value dim d, block b)
  return 8 * (d ^ ((d >> 4) & 1)) + ((b + (d >> 1) + (d >> 5)) & 7);
}
__device__ inline int dn_slot(int r) { return 8 * (r & 7) + (r >> 3); }   // chunk row -> MFMA k slot

__global__ __launch_bounds__(DN_NT) void mla_out_dense(MlaArgs a) {
  constexpr int HW = DN_HW, NT = DN_NT;
  constexpr int NPV = DN_CHUNK * 32 / NT;          // 16-byte value pieces per thread and chunk
  constexpr int NPW = DN_CHUNK * (HW / 4) / NT;    // 4-head weight pieces per thread and chunk
  static_assert(NPV == 4 && NPW * NT == DN_CHUNK * (HW / 4), "staging roles");
  extern __shared__ __align__(16) unsigned char dsm[];
  uint4* vt = reinterpret_cast<uint4*>(dsm);                                         // [512 x 8] units of 8 bf16
  float* pf = reinterpret_cast<float*>(dsm + size_t(DV) * DN_CHUNK * 2);            // [HW][DN_PP] weights
  float* gsc = pf + HW * DN_PP;                                                      // [4][DN_CHUNK] group scales
  int* pre = reinterpret_cast<int*>(gsc + DN_CHUNK * 4);                             // [OUT_MAX_S + 4]
  int2* rowtab = reinterpret_cast<int2*>(pre + OUT_MAX_S + 4);                       // [DN_SEG] (slot, position)

  const int R = a.R, H = a.Hq, NHH = H / HW;      // head halves (or the one 64-head set) per sequence
  const int rg = blockIdx.x % R, bh = blockIdx.x / R, hh = bh % NHH, b = bh / NHH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = wave >> 2, g = wave & 3;
  const int S = a.S;
  const int64_t row0 = int64_t(b) * a.cap;
  const uint32_t epoch = __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // kept rows per split (every row here, counted the same way) -> exclusive prefix
  {
    int c[4] = {0, 0, 0, 0};
    if (tid < OUT_MAX_S / 4)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int sp = 4 * tid + k;
        c[k] = sp < S ? a.kcount[int64_t(b) * S + sp] : 0;
      }
    const int local = c[0] + c[1] + c[2] + c[3];
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63 && wave < 4) pre[OUT_MAX_S + wave] = incl;    // totals of the four counting waves
    __syncthreads();
    if (tid < OUT_MAX_S / 4) {
      int run = incl - local;
      for (int w = 0; w < wave; ++w) run += pre[OUT_MAX_S + w];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pre[4 * tid + k] = run;
        run += c[k];
      }
    }
    __syncthreads();
  }
  const int N = pre[OUT_MAX_S] + pre[OUT_MAX_S + 1] + pre[OUT_MAX_S + 2] + pre[OUT_MAX_S + 3];
  const int rbeg = int(int64_t(N) * rg / R), rend = int(int64_t(N) * (rg + 1) / R);

  floatx16 acc[4] = {};
  float msum = 0.f;                                   // weights of head 32hb + (lane & 31), this lane's slots
  const int col = lane & 31, kh = lane >> 5;
  // staged data of one chunk, loaded a chunk ahead: value pieces (rows
  // vb + 8(4vs + i), bytes 16vq..), 4-head weight pieces (row (tid + 512i) / 16,
  // heads 4 * (tid % 16)..) and, for the first 64 threads, the four value-group
  // scales of row tid
  struct Stage { uint4 v[NPV]; float4 w[NPW]; float4 sc; };
  const int vq = tid & 31, vb = (tid >> 5) & 7, vs = tid >> 8;
  // kp holds the scores (log2 domain) of every row; this thread's weight
  // pieces are always heads HW*hh + 4 (tid % 16) .. + 3, whose weight is
  // exp2(score - LSE), as the scores kernel computes kept weights
  float lsv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) lsv[j] = a.lseo[int64_t(b) * H + HW * hh + 4 * (tid & 15) + j];
  auto load_stage = [&](int c0, int seg0, int segn, Stage& st) {
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int rs = c0 + vb + 8 * (4 * vs + i) - seg0;      // row within the segment
      st.v[i] = make_uint4(0u, 0u, 0u, 0u);
      if (rs < segn) st.v[i] = *reinterpret_cast<const uint4*>(a.kc + (row0 + rowtab[rs].y) * D + 16 * vq);
    }
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int pw = tid + i * NT, rs = c0 + (pw >> 4) - seg0;
      st.w[i] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);   // weight 0
      if (rs < segn)
        st.w[i] = *reinterpret_cast<const float4*>(a.kp + int64_t(rowtab[rs].x) * H + HW * hh + 4 * (pw & 15));
    }
    const int rs = c0 + tid - seg0;
    st.sc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < DN_CHUNK && rs < segn)
      st.sc = *reinterpret_cast<const float4*>(a.ks + (row0 + rowtab[rs].y) * (4 * NGROUPS));
  };
  auto write_stage = [&](const Stage& st) {
    // slots 8vb + 4vs .. + 3 of dims 16vq + 2j, + 1: pack the two dims' bf16 over the 4 rows
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = j < 2 ? st.v[i].x : j < 4 ? st.v[i].y : j < 6 ? st.v[i].z : st.v[i].w;
        pr[i] = __builtin_bit_cast(uint32_t, (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
      }
      uint2 lo, hi;                                   // dim 16vq + 2j (low halves), + 1 (high halves)
      lo.x = __builtin_amdgcn_perm(pr[1], pr[0], 0x05040100u);
      lo.y = __builtin_amdgcn_perm(pr[3], pr[2], 0x05040100u);
      hi.x = __builtin_amdgcn_perm(pr[1], pr[0], 0x07060302u);
      hi.y = __builtin_amdgcn_perm(pr[3], pr[2], 0x07060302u);
      const int d = 16 * vq + 2 * j;
      reinterpret_cast<uint2*>(vt + dn_unit(d, vb))[vs] = lo;
      reinterpret_cast<uint2*>(vt + dn_unit(d + 1, vb))[vs] = hi;
    }
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int pw = tid + i * NT, sl = dn_slot(pw >> 4), h4 = pw & 15;
      pf[(4 * h4 + 0) * DN_PP + sl] = exp2f(st.w[i].x - lsv[0]);
      pf[(4 * h4 + 1) * DN_PP + sl] = exp2f(st.w[i].y - lsv[1]);
      pf[(4 * h4 + 2) * DN_PP + sl] = exp2f(st.w[i].z - lsv[2]);
      pf[(4 * h4 + 3) * DN_PP + sl] = exp2f(st.w[i].w - lsv[3]);
    }
    if (tid < DN_CHUNK) {
      const int sl = dn_slot(tid);
      gsc[0 * DN_CHUNK + sl] = st.sc.x;
      gsc[1 * DN_CHUNK + sl] = st.sc.y;
      gsc[2 * DN_CHUNK + sl] = st.sc.z;
      gsc[3 * DN_CHUNK + sl] = st.sc.w;
    }
  };

  for (int seg0 = rbeg; seg0 < rend; seg0 += DN_SEG) {
    const int segn = min(DN_SEG, rend - seg0);
    // (slot in the split's published rows, position) of every row of the segment
    __syncthreads();                                   // the previous segment's table is no longer read
    {
      int idx[DN_SEG / NT], pos[DN_SEG / NT];
#pragma unroll
      for (int i = 0; i < DN_SEG / NT; ++i) {
        const int r = seg0 + min(tid + i * NT, segn - 1);
        int lo = 0, hi = S - 1;                        // the last split whose prefix is <= r
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= r) lo = mid; else hi = mid - 1;
        }
        idx[i] = (b * S + lo) * a.P + (r - pre[lo]);
      }
#pragma unroll
      for (int i = 0; i < DN_SEG / NT; ++i) pos[i] = a.kpos[idx[i]];     // one batch of loads
#pragma unroll
      for (int i = 0; i < DN_SEG / NT; ++i)
        if (tid + i * NT < segn) rowtab[tid + i * NT] = make_int2(idx[i], pos[i]);
    }
    __syncthreads();
    Stage st;                                          // one set of registers: written to LDS, then refilled
    load_stage(seg0, seg0, segn, st);
    for (int c0 = seg0; c0 < seg0 + segn; c0 += DN_CHUNK) {
      write_stage(st);
      if (c0 + DN_CHUNK < seg0 + segn) load_stage(c0 + DN_CHUNK, seg0, segn, st);
      __syncthreads();
      // products: 4 k-steps of 16 slots; lane (col, kh) takes head 32hb + col
      // and slots 16ks + 8kh .. + 7 of the chunk; the LDS operands of step
      // ks + 1 are read while the MFMAs of step ks run
      float pw[2][8], gs[2][8];
      bf16x8 bv[2][4], ah[2], al[2];
      auto read_ops = [&](int ks, float (&w)[8], float (&s8)[8], bf16x8 (&bq)[4]) {
        const int k0 = 16 * ks + 8 * kh;
        const float* ph = pf + (32 * hb + col) * DN_PP + k0;
        const float4 pa = *reinterpret_cast<const float4*>(ph), pb = *reinterpret_cast<const float4*>(ph + 4);
        const float4 sa = *reinterpret_cast<const float4*>(gsc + g * DN_CHUNK + k0);
        const float4 sb = *reinterpret_cast<const float4*>(gsc + g * DN_CHUNK + k0 + 4);
        w[0] = pa.x; w[1] = pa.y; w[2] = pa.z; w[3] = pa.w; w[4] = pb.x; w[5] = pb.y; w[6] = pb.z; w[7] = pb.w;
        s8[0] = sa.x; s8[1] = sa.y; s8[2] = sa.z; s8[3] = sa.w; s8[4] = sb.x; s8[5] = sb.y; s8[6] = sb.z; s8[7] = sb.w;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bq[t] = __builtin_bit_cast(bf16x8, vt[dn_unit(128 * g + 32 * t + col, 2 * ks + kh)]);
      };
      auto make_a = [&](const float (&w)[8], const float (&s8)[8], bf16x8& hv, bf16x8& lv) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          msum += w[i];
          const float x = w[i] * s8[i];
          const __bf16 h = __bf16(x);                  // v_cvt_pk_bf16_f32: round to nearest even
          hv[i] = h;
          lv[i] = __bf16(x - float(h));
        }
      };
      read_ops(0, pw[0], gs[0], bv[0]);
      make_a(pw[0], gs[0], ah[0], al[0]);
#pragma unroll
      for (int ks = 0; ks < DN_CHUNK / 16; ++ks) {
        const int c = ks & 1, n = c ^ 1;
        if (ks + 1 < DN_CHUNK / 16) read_ops(ks + 1, pw[n], gs[n], bv[n]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[c], bv[c][t], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[c], bv[c][t], acc[t], 0, 0, 0);
        if (ks + 1 < DN_CHUNK / 16) make_a(pw[n], gs[n], ah[n], al[n]);
      }
      __syncthreads();                                 // the next chunk reuses the staging
    }
  }
  // partial of this range: accumulator 4i+j of tile t -> head HW*hh + 32hb + 8i + 4kh + j, dim 128g + 32t + col
  float* part = a.opart + (int64_t(b) * R + rg) * H * DV + int64_t(HW * hh) * DV;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        part[(32 * hb + 8 * i + 4 * kh + j) * DV + 128 * g + 32 * t + col] = acc[t][4 * i + j];
  if (g == 0) {                                        // head 32hb + col: the two lane halves' slots
    const float other = __shfl_xor(msum, 32);
    if (kh == 0) a.mpart[(int64_t(b) * R + rg) * H + HW * hh + 32 * hb + col] = msum + other;
  }
  __threadfence();
  __syncthreads();
  u64* done = a.done + int64_t(bh) * R;
  if (tid == 0) put_tagged_f(done + rg, epoch, 1.f);
  // wait for the other ranges of these heads, then add one slice of their outputs
  bool gave_up = false;
  for (int k = tid; k < R; k += NT) settle_f(peek(done + k), done + k, epoch, a.hdr, a.spin_limit, gave_up);
  const bool dbad = __syncthreads_or(gave_up) != 0;   // another range's partials are not this call's: NaN
  __threadfence();
  // slices in float4 units; the R partials of an element are loaded eight at
  // a time and added in range order (the loads of a batch are in flight together)
  const float4* p0 = reinterpret_cast<const float4*>(a.opart + int64_t(b) * R * H * DV + int64_t(HW * hh) * DV);
  const int64_t pstride = int64_t(H) * DV / 4;
  const int e0 = int(int64_t(HW) * DV / 4 * rg / R), e1 = int(int64_t(HW) * DV / 4 * (rg + 1) / R);
  for (int e = e0 + tid; e < e1; e += NT) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    int k = 0;
    for (; k + 8 <= R; k += 8) {
      float4 t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = p0[(k + u) * pstride + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) { v.x += t[u].x; v.y += t[u].y; v.z += t[u].z; v.w += t[u].w; }
    }
    for (; k < R; ++k) {
      const float4 t = p0[k * pstride + e];
      v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
    }
    v.x = poison_if(dbad, v.x); v.y = poison_if(dbad, v.y); v.z = poison_if(dbad, v.z); v.w = poison_if(dbad, v.w);
    reinterpret_cast<float4*>(a.out + (int64_t(b) * H + HW * hh) * DV)[e] = v;
  }
  if (rg == 0 && tid < HW) {                          // kept mass of head HW*hh + tid, ranges in order
    const float* mp = a.mpart + int64_t(b) * R * H + HW * hh + tid;
    float m = 0.f;
    int k = 0;
    for (; k + 8 <= R; k += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = mp[int64_t(k + u) * H];
#pragma unroll
      for (int u = 0; u < 8; ++u) m += t[u];
    }
    for (; k < R; ++k) m += mp[int64_t(k) * H];
    a.kept_mass[int64_t(b) * H + HW * hh + tid] = poison_if(dbad, m);
  }
  if (rg == 0 && hh == 0 && wave == 0) {              // kept pairs of the sequence (integer sum: any order)
    long long pairs = 0;
    for (int sp = lane; sp < S; sp += 64) pairs += a.kpairs[int64_t(b) * S + sp];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pairs += __shfl_xor(pairs, o);
    if (lane == 0) {
      a.bgstat[2 * b] = (unsigned long long)pairs;
      a.bgstat[2 * b + 1] = (unsigned long long)N;
    }
  }
  // the last workgroup advances the epoch for the next call
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.hdr->groups_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(&a.hdr->groups_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.hdr->epoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// 32 heads have no dense variant; they use mla_out's ranges.
const void* mla_out_dense_kernel(int H) {
  return (H == 64 || H == 128) ? reinterpret_cast<const void*>(&mla_out_dense) : nullptr;
}

// LDS bytes of mla_scores (every region is a multiple of 16 bytes).
size_t mla_lds_bytes(int H, int P, int S, int tpe) {
  const int NLT = P / (TILE * tpe);
  const int NW = 2 * (H / 32);
  (void)S;
  return size_t(NBUF) * BUF_BYTES + size_t(2) * NW * 128 * 16 + size_t(H) * NLT * 4 + size_t(H) * 4 +
         size_t((NLT + 3) & ~3) * 4 + 2 * TILE * 4 + 8 * 4 + 64;
}

const void* mla_scores_kernel(int H) {
  if (H == 32) return reinterpret_cast<const void*>(&mla_scores<2>);
  if (H == 64) return reinterpret_cast<const void*>(&mla_scores<4>);
  if (H == 128) return reinterpret_cast<const void*>(&mla_scores<8>);
  return nullptr;
}
const void* mla_out_kernel() { return reinterpret_cast<const void*>(&mla_out); }

}  // namespace kvq
