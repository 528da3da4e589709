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
//  mla_scores  (one workgroup per (sequence, split); wave w owns heads
//              32w..32w+31 with q resident in registers as bf16 MFMA operands)
//    1. streams 32-row latent tiles into a 4-deep LDS ring with direct
//       global->LDS loads (three tiles in flight), scores them with
//       v_mfma_f32_32x32x16_bf16 (fp8 -> bf16 with the hardware converter,
//       exact), applies the per-group fp32 scale to the fp32 accumulators,
//       keeps per-head (max, sum exp2) and a per-(head, 64-position tile)
//       maximum;
//    2. the group's split statistics are merged into per-head log-sum-exps
//       (head h by split h mod S) and exchanged as epoch-tagged words;
//    3. re-scores only the 64-position tiles whose maximum can reach the
//       threshold (identical code, identical bits), computes the normalized
//       weights and publishes, per kept row, its position and the weights of
//       all heads (0 where a head skips it).
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

constexpr int D = 576;          // latent width (scores)
constexpr int DV = 512;         // value width
constexpr int KSTEPS = D / 16;  // 36 MFMA k-steps of 16 dims
constexpr int NGROUPS = 5;      // scale groups: 4 x 128 + 1 x 64
constexpr int ROW_LDS = 592;    // LDS pitch of a staged latent row: 37 x 16 bytes (odd), so the 16-byte
                                // reads of 8 consecutive rows hit distinct bank groups
constexpr int TILE = 32;        // positions per MFMA tile
constexpr int LTILE = 64;       // positions per liveness tile
constexpr uint32_t kSpinLimit = 1u << 23;

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
__device__ inline float settle_f(u64 w, const u64* p, uint32_t epoch, WsHeader* h) {
  uint32_t spins = 0;
  while (uint32_t(w >> 32) != epoch) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit) {
      __hip_atomic_fetch_or(&h->status, kStatusWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    w = peek(p);
  }
  return __uint_as_float(uint32_t(w));
}

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
// lane j <- lane j ^ 16 within each half of the wave (swizzle, bit-mask mode)
__device__ inline float swz16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// Reduce 16 independent values over the 32 lanes of each wave half (max or
// sum), every lane getting the result. Steps: neighbour in quad, other pair
// in quad, mirrored quad in the 8-lane half row, mirrored half row, other row.
template <bool MAX>
__device__ inline void reduce32x16(float (&v)[16]) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  float t[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = dpp<0xB1>(v[e]);     // quad_perm [1,0,3,2]
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = dpp<0x4E>(v[e]);     // quad_perm [2,3,0,1]
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = dpp<0x141>(v[e]);    // row_half_mirror
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = dpp<0x140>(v[e]);    // row_mirror
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = op(v[e], t[e]);
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = swz16(v[e]);
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = op(v[e], t[e]);
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

// Barrier between the waves of the workgroup without a memory fence (a fence
// would wait for every load in flight, including the tiles being prefetched);
// the empty asm keeps the compiler from moving memory accesses across it.
__device__ inline void bar_nofence() {
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

struct TileSrc {
  const uint8_t* kc;
  const float* ks;
  int64_t row0;
  int ctx;
};

// Issue this wave's direct loads of the tile starting at position `first`
// into buffer `dst`. Rows at or past ctx (and padding slots) repeat a real
// chunk of row ctx-1, so every instruction runs with all lanes and the
// per-wave instruction count is the same for every tile.
template <int NW>
__device__ __attribute__((always_inline)) inline void issue_tile(uint8_t* __restrict__ dst, const TileSrc& src,
                                                                 int first, int wave, int lane) {
  for (int j = wave; j < NDMA; j += NW) {
    if (j < NCHUNK_I) {
      const int sl = 64 * j + lane;
      int r = sl / PITCH16, c = sl - r * PITCH16;
      r = min(r, TILE - 1);
      c = min(c, D / 16 - 1);
      const int pos = min(first + r, src.ctx - 1);
      __builtin_amdgcn_global_load_lds(src.kc + (src.row0 + pos) * D + c * 16, dst + j * 1024, 16, 0, 0);
    } else {
      const int i = 64 * (j - NCHUNK_I) + lane;
      int64_t gi = (src.row0 + first) * NGROUPS + min(i, TILE * NGROUPS - 1);
      gi = min(gi, (src.row0 + src.ctx) * NGROUPS - 1);
      __builtin_amdgcn_global_load_lds(src.ks + gi, dst + SC_OFF + (j - NCHUNK_I) * 256, 4, 0, 0);
    }
  }
}

// Scores of one staged tile (log2 domain): 16 heads of this lane x its
// column. MFMA k order: step ks = 2p + e takes, in k-half kh, the latent dims
// 32p + 16kh + 8e .. +7, so one 16-byte LDS read of chunk 2p + kh of a row
// feeds steps 2p and 2p + 1, and every step stays inside one scale group
// (group g = steps 8g .. 8g + 7, the last group has 4). The groups accumulate
// separately (their fp32 scales differ per row); the operands of the next
// group are read while the current group's MFMAs run.
__device__ __attribute__((always_inline)) inline void score_tile(const uint8_t* __restrict__ buf,
                                                                 const bf16x8 (&A)[KSTEPS], float hs, int col, int kh,
                                                                 bool valid, float (&s2)[16]) {
  const uint8_t* src = buf + col * ROW_LDS + 16 * kh;
  const float* sc = reinterpret_cast<const float*>(buf + SC_OFF) + col * NGROUPS;
  constexpr int NP = KSTEPS / 2;                     // 18 step pairs
  uint4 cur[4], nxt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cur[j] = *reinterpret_cast<const uint4*>(src + 32 * j);
  floatx16 cg[NGROUPS];
#pragma unroll
  for (int g = 0; g < NGROUPS; ++g) {
    const int np = g < 4 ? 4 : 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * (g + 1) + j < NP) nxt[j] = *reinterpret_cast<const uint4*>(src + 32 * (4 * (g + 1) + j));
    floatx16 c = {};
#pragma unroll
    for (int j = 0; j < np; ++j) {
      const int p = 4 * g + j;
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * p], fp8x8_to_bf16(cur[j].x, cur[j].y), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[2 * p + 1], fp8x8_to_bf16(cur[j].z, cur[j].w), c, 0, 0, 0);
    }
    cg[g] = c;
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
  }
  const float g0 = sc[0] * hs, g1 = sc[1] * hs, g2 = sc[2] * hs, g3 = sc[3] * hs, g4 = sc[4] * hs;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float v = g0 * cg[0][e];
    v = fmaf(g1, cg[1][e], v);
    v = fmaf(g2, cg[2][e], v);
    v = fmaf(g3, cg[3][e], v);
    v = fmaf(g4, cg[4][e], v);
    s2[e] = valid ? v : -INFINITY;
  }
}

// One tile of the scoring pass: start the direct loads of a later tile into
// `wr` (when given), score the tile staged in `rd`, and fold it into the
// split statistics. The restrict qualifiers state that the buffer being
// filled, the buffer being read and the tile-maximum table are disjoint, so
// the compiler adds no wait for the loads in flight; the waits that order a
// tile's loads before its reads are explicit (wait_tiles + bar_nofence).
template <int NW>
__device__ __attribute__((always_inline)) inline void scoring_step(
    uint8_t* __restrict__ wr, const uint8_t* __restrict__ rd, float* __restrict__ tmax, const TileSrc& src,
    int next_first, int wave, int lane, int t, int pos, int nlt, const bf16x8 (&A)[KSTEPS], float hs,
    float (&m)[16], float (&l)[16], float (&sprev)[16]) {
  const int col = lane & 31, kh = lane >> 5;
  if (wr) issue_tile<NW>(wr, src, next_first, wave, lane);
  float s2[16];
  score_tile(rd, A, hs, col, kh, pos < src.ctx, s2);
  if ((t & 1) == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sprev[e] = s2[e];
    return;
  }
  // end of a 64-position liveness tile: its maximum per head becomes the
  // running reference of the lane-local sums
  float tm[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) tm[e] = fmaxf(sprev[e], s2[e]);
  reduce32x16<true>(tm);
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) tmax[(32 * wave + 8 * i + 4 * kh + j) * nlt + (t >> 1)] = tm[4 * i + j];
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float mn = fmaxf(m[e], tm[e]);
    const float ms = mn == -INFINITY ? 0.f : mn;  // nothing valid yet: every term is 0
    l[e] = l[e] * ex2(m[e] - ms) + ex2(sprev[e] - ms) + ex2(s2[e] - ms);
    m[e] = mn;
  }
}

__device__ inline void stamp_mla(const MlaArgs& a, int k) {
  if (a.times && threadIdx.x == 0) a.times[int64_t(blockIdx.x) * 16 + k] = wall_clock64();
}

}  // namespace mla

using namespace mla;

// ----------------------------------------------------------------------------- scores
template <int NW>
__global__ __launch_bounds__(64 * NW) void mla_scores(MlaArgs a) {
  constexpr int NT = 64 * NW;         // threads
  constexpr int H = 32 * NW;          // heads
  extern __shared__ __align__(16) unsigned char smem[];
  const int P = a.P;
  const int NLT = P / LTILE;          // liveness tiles per split
  uint8_t* ring = smem;                                                  // [NBUF][BUF_BYTES]
  float* tmax = reinterpret_cast<float*>(ring + NBUF * BUF_BYTES);       // [H][NLT]
  float* lse = tmax + H * NLT;                                           // [H]
  int* live = reinterpret_cast<int*>(lse + H);                           // [NLT (+pad)]
  unsigned* keepmask = reinterpret_cast<unsigned*>(live + ((NLT + 3) & ~3));  // [TILE]
  int* misc = reinterpret_cast<int*>(keepmask + TILE);                   // [8]
  float2* mlbuf = reinterpret_cast<float2*>(misc + 8);                   // [H + S] scratch (16-B aligned)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x / a.S;
  const int split = blockIdx.x - b * a.S;
  const int pos0 = split * P;
  const int ctx = a.ctx;
  const int64_t row0 = int64_t(b) * a.cap;
  const uint32_t epoch = __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  const int col = lane & 31;          // MFMA column / A row
  const int kh = lane >> 5;           // k half (0: dims 0..7 of a k-step, 1: 8..15)
  const int head_a = 32 * wave + col; // head of this lane's A operand row

  stamp_mla(a, 0);
  if (blockIdx.x == 0 && tid == 0) {
    a.hdr->batch = a.B; a.hdr->q_heads = H; a.hdr->kv_heads = 1; a.hdr->ctx = ctx;
    a.hdr->splits = a.S; a.hdr->positions_per_split = P; a.hdr->fmt = KVQ_FP8_B128; a.hdr->v_dim = DV;
    a.hdr->nwg = int(gridDim.x);
    a.hdr->k_row_bytes = D + 4 * NGROUPS;               // a whole latent row
    a.hdr->v_row_bytes = DV + 4 * (DV / 128);           // its value part
  }

  // ---------------------------------------------------------------- tile staging
  // Register staging of one tile into buffer 0 (the re-scoring pass).
  constexpr int CHUNKS = TILE * (D / 16);
  constexpr int PER = (CHUNKS + NT - 1) / NT;
  constexpr int NSC = TILE * NGROUPS;
  constexpr int PERS = (NSC + NT - 1) / NT;
  auto stage = [&](int t) {
    uint4 v[PER];
    float sv[PERS];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      const int r = i / (D / 16), c = i - r * (D / 16);
      const int pos = pos0 + t * TILE + r;
      v[k] = (i < CHUNKS && pos < ctx) ? *reinterpret_cast<const uint4*>(a.kc + (row0 + pos) * D + c * 16)
                                       : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < PERS; ++k) {
      const int i = tid + k * NT;
      const int r = i / NGROUPS, gi = i - r * NGROUPS;
      const int pos = pos0 + t * TILE + r;
      sv[k] = (i < NSC && pos < ctx) ? reinterpret_cast<const float*>(a.ks + (row0 + pos) * (4 * NGROUPS))[gi] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      if (i < CHUNKS) {
        const int r = i / (D / 16), c = i - r * (D / 16);
        *reinterpret_cast<uint4*>(ring + r * ROW_LDS + c * 16) = v[k];
      }
    }
#pragma unroll
    for (int k = 0; k < PERS; ++k)
      if (tid + k * NT < NSC) reinterpret_cast<float*>(ring + SC_OFF)[tid + k * NT] = sv[k];
  };
  const TileSrc src{a.kc, reinterpret_cast<const float*>(a.ks), row0, ctx};
  const int T = P / TILE;
  // the first three tiles start loading before the query is set up
  for (int t = 0; t < 3 && t < T; ++t) issue_tile<NW>(ring + t * BUF_BYTES, src, pos0 + t * TILE, wave, lane);

  // ---------------------------------------------------------------- q operands
  // The bf16 query is the A operand as it is, in the k order of score_tile.
  bf16x8 A[KSTEPS];
  {
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + (int64_t(b) * H + head_a) * D + 16 * kh;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      A[ks] = *reinterpret_cast<const bf16x8*>(qh + 32 * (ks >> 1) + 8 * (ks & 1));
  }
  const float hs = a.sigma_log2e;     // score scale: softmax scale * log2 e

  // ---------------------------------------------------------------- phase 1
  // Per 64-position tile: the tile maximum per head (reduced over the 32
  // columns) becomes the running reference m, every lane adds exp2(s - m) of
  // its own two scores to a lane-local sum l (rescaled when m grows).
  stamp_mla(a, 1);
  float m[16], l[16], sprev[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) { m[e] = -INFINITY; l[e] = 0.f; sprev[e] = -INFINITY; }
  for (int t = 0; t < T; ++t) {
    wait_tiles<NW>(min(2, T - 1 - t), wave);       // this wave's loads of tile t have landed
    bar_nofence();                                  // everyone's have; buffer (t+3) % NBUF is free
    uint8_t* wr = t + 3 < T ? ring + ((t + 3) % NBUF) * BUF_BYTES : nullptr;
    scoring_step<NW>(wr, ring + (t % NBUF) * BUF_BYTES, tmax, src, pos0 + (t + 3) * TILE, wave, lane, t,
                     pos0 + t * TILE + col, NLT, A, hs, m, l, sprev);
  }
  __syncthreads();
  stamp_mla(a, 2);
  // split statistics per head: m is already common to the 32 columns; sum l
  reduce32x16<false>(l);
  if (col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 32 * wave + 8 * i + 4 * kh + j;
        u64* dst = a.split_ml + ((int64_t(b) * a.S + split) * H + h) * 2;
        put_tagged_f(dst, epoch, m[4 * i + j]);
        put_tagged_f(dst + 1, epoch, l[4 * i + j]);
      }
  }

  // ---------------------------------------------------------------- phase 2: LSE
  // head h is merged by split (h mod S) over all splits, in split order
  {
    const int nh = (H - split + a.S - 1) / a.S;      // heads this split merges: split, split + S, ...
    for (int it = tid; it < nh * a.S; it += NT) {
      const int hl = it / a.S, sp = it - hl * a.S;
      const int h = split + hl * a.S;
      const u64* src = a.split_ml + ((int64_t(b) * a.S + sp) * H + h) * 2;
      const u64 w0 = peek(src), w1 = peek(src + 1);
      float2 v;
      v.x = settle_f(w0, src, epoch, a.hdr);
      v.y = settle_f(w1, src + 1, epoch, a.hdr);
      // scratch: [hl][sp], fits because nh * S <= H + S - 1 <= mlbuf size checked by the host
      mlbuf[it] = v;
    }
    __syncthreads();
    if (tid < nh) {
      float2 acc = make_float2(-INFINITY, 0.f);
      for (int sp = 0; sp < a.S; ++sp) acc = lse_merge(acc, mlbuf[tid * a.S + sp]);
      put_tagged_f(a.lse + int64_t(b) * H + split + tid * a.S, epoch, acc.x + log2f(acc.y));
    }
    if (tid < H) {
      const u64* src = a.lse + int64_t(b) * H + tid;
      lse[tid] = settle_f(peek(src), src, epoch, a.hdr);
    }
    __syncthreads();
  }
  stamp_mla(a, 3);

  // ---------------------------------------------------------------- phase 3: live tiles
  // A 64-position tile is live when some head's tile maximum can reach the
  // threshold (a small margin keeps the test conservative); only live tiles
  // are re-read and re-scored.
  const float log2tau = a.tau > 0.f ? log2f(a.tau) : -INFINITY;
  if (tid == 0) misc[0] = 0;
  __syncthreads();
  for (int u = tid; u < NLT; u += NT) {
    bool lv = false;
    if (pos0 + u * LTILE < ctx)
      for (int h = 0; h < H && !lv; ++h) lv = tmax[h * NLT + u] >= lse[h] + log2tau - 0.01f;
    if (lv) live[atomicAdd(&misc[0], 1)] = u;
  }
  __syncthreads();
  const int nlive = misc[0];
  // sort the (few) live tile ids so the published rows come out in position order
  if (tid == 0)
    for (int i = 1; i < nlive; ++i)
      for (int j = i; j > 0 && live[j - 1] > live[j]; --j) { const int x = live[j]; live[j] = live[j - 1]; live[j - 1] = x; }
  if (tid == 1) { misc[1] = 0; misc[2] = 0; }        // kept rows, kept pairs
  __syncthreads();
  int kept_pairs = 0;
  const int64_t kbase = int64_t(b) * a.S + split;
  for (int li = 0; li < nlive; ++li) {
    const int u = live[li];
    for (int half = 0; half < 2; ++half) {
      const int t = 2 * u + half;
      stage(t);
      if (tid < TILE) keepmask[tid] = 0u;
      __syncthreads();
      float s2[16];
      score_tile(ring, A, hs, col, kh, pos0 + t * TILE + col < ctx, s2);
      // normalized weights and keep bits
      unsigned bits = 0u;
      float p[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * i + j;
          const float pe = exp2f(s2[e] - lse[32 * wave + 8 * i + 4 * kh + j]);   // denormal-exact
          const bool keep = (s2[e] != -INFINITY) && pe >= a.tau;
          p[e] = keep ? pe : 0.f;
          bits |= keep ? 1u : 0u;
          kept_pairs += keep ? 1 : 0;
        }
      if (bits) atomicOr(&keepmask[col], 1u);
      __syncthreads();
      // compaction: row index of each kept column within this split's list
      if (tid == 0) {
        int n = misc[1];
        for (int c = 0; c < TILE; ++c) {
          if (keepmask[c]) { keepmask[c] = 0x80000000u | unsigned(n); a.kpos[kbase * P + n] = pos0 + t * TILE + c; ++n; }
        }
        misc[1] = n;
      }
      __syncthreads();
      const unsigned km = keepmask[col];
      if (km & 0x80000000u) {
        float* dst = a.kp + (kbase * P + (km & 0x7FFFFFFFu)) * H;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[32 * wave + 8 * i + 4 * kh + j] = p[4 * i + j];
      }
      __syncthreads();
    }
  }
  // kept pairs of the split
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kept_pairs += __shfl_xor(kept_pairs, o);
  if (lane == 0) atomicAdd(&misc[2], kept_pairs);
  __syncthreads();
  if (tid == 0) {
    a.kcount[kbase] = misc[1];
    a.kpairs[kbase] = misc[2];
  }
  stamp_mla(a, 4);
}

// ----------------------------------------------------------------------------- out
// One workgroup per (sequence, 32 heads, 128-dim value group g): the output
// block out[h][d] = sum over the sequence's kept rows r of p[h][r] * v[r][d],
// a contraction over rows on v_mfma_f32_32x32x16_bf16 (M = heads, N = dims,
// K = rows; wave w owns dims 32w..32w+31 of the group). Exact operands: v is
// the e4m3 code converted to bf16 (exact) and the row's fp32 group scale
// goes to the weight side, p * scale (one fp32 rounding) split into three
// bf16 terms that add up to it exactly (8 + 8 + 8 significant bits); each
// term is a separate MFMA into the same fp32 accumulator. Rows are taken in
// split order and, within a split, in position order, 64 at a time; both
// operands are staged transposed in LDS (rows contiguous per head / dim).
constexpr int OUT_CHUNK = 64;                   // rows per LDS stage (4 MFMA k-steps)
constexpr int OUT_PITCH = OUT_CHUNK + 8;        // bf16 per staged head / dim line (bank spread)
constexpr int OUT_MAX_S = 1024;                 // splits per sequence the prefix table holds

__device__ inline uint16_t bf16_bits_rne(float x) {  // exact-to-nearest-even fp32 -> bf16
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline float bf16_value(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__global__ __launch_bounds__(256) void mla_out(MlaArgs a) {
  __shared__ __align__(16) uint16_t vt[128 * OUT_PITCH];            // [dim][row] bf16 values
  __shared__ __align__(16) uint16_t pt[3 * 32 * OUT_PITCH];         // [term][head][row] bf16 weight terms
  __shared__ int pre[OUT_MAX_S + 1];                                // exclusive prefix of kept rows per split
  __shared__ float mpart[256][8];                                   // kept-mass partials [thread][head slot]
  __shared__ long long cnt[4];

  const int H = a.Hq;
  const int nhb = H / 32;
  const int b = blockIdx.x / (nhb * 4);
  const int rem = blockIdx.x - b * nhb * 4;
  const int hb = rem >> 2, g = rem & 3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S;
  const int64_t row0 = int64_t(b) * a.cap;
  const uint32_t epoch_next =
      __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // kept rows per split: one batch of loads, then an exclusive prefix sum
  long long pairs_part = 0;
  {
    int c[OUT_MAX_S / 256];
#pragma unroll
    for (int k = 0; k < OUT_MAX_S / 256; ++k) {
      const int sp = tid * (OUT_MAX_S / 256) + k;
      c[k] = sp < S ? a.kcount[int64_t(b) * S + sp] : 0;
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
    __syncthreads();
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

  floatx16 acc = {};
  float mass[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mass[j] = 0.f;
  const int col = lane & 31, kh = lane >> 5;
  // staging roles: row r = tid / 4 of the chunk, quarter q = tid % 4
  const int sr = tid >> 2, sq = tid & 3;
  for (int c0 = 0; c0 < N; c0 += OUT_CHUNK) {
    const int r = c0 + sr;
    uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
    float pw[8], sc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) pw[j] = 0.f;
    if (r < N) {
      // split of global row r: the last split whose prefix is <= r (binary search)
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= r) lo = mid; else hi = mid - 1;
      }
      const int64_t kb = int64_t(b) * S + lo;
      const int64_t idx = kb * a.P + (r - pre[lo]);
      const int pos = a.kpos[idx];
      const uint8_t* vrow = a.kc + (row0 + pos) * D + 128 * g + 32 * sq;
      v0 = *reinterpret_cast<const uint4*>(vrow);
      v1 = *reinterpret_cast<const uint4*>(vrow + 16);
      sc = reinterpret_cast<const float*>(a.ks + (row0 + pos) * (4 * NGROUPS))[g];
      const float4 p0 = *reinterpret_cast<const float4*>(a.kp + idx * H + 32 * hb + 8 * sq);
      const float4 p1 = *reinterpret_cast<const float4*>(a.kp + idx * H + 32 * hb + 8 * sq + 4);
      pw[0] = p0.x; pw[1] = p0.y; pw[2] = p0.z; pw[3] = p0.w;
      pw[4] = p1.x; pw[5] = p1.y; pw[6] = p1.z; pw[7] = p1.w;
    }
    // values: 32 dims of row sr -> bf16, transposed into vt[dim][row]
    {
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
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
      mass[j] += pw[j];
      const float x = pw[j] * sc;
      const uint16_t t0 = bf16_bits_rne(x);
      const float r1 = x - bf16_value(t0);
      const uint16_t t1 = bf16_bits_rne(r1);
      const uint16_t t2 = bf16_bits_rne(r1 - bf16_value(t1));
      const int h = 8 * sq + j;
      pt[(0 * 32 + h) * OUT_PITCH + sr] = t0;
      pt[(1 * 32 + h) * OUT_PITCH + sr] = t1;
      pt[(2 * 32 + h) * OUT_PITCH + sr] = t2;
    }
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
  }
  // accumulator 4i+j of the lane: head 8i + 4kh + j, dim 32*wave + col of the group
  float* ob = a.out + (int64_t(b) * H + 32 * hb) * DV + 128 * g + 32 * wave + col;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) ob[int64_t(8 * i + 4 * kh + j) * DV] = acc[4 * i + j];
  if (g == 0) {
    // kept mass of the 32 heads: thread t summed the rows t/4 (mod 64) of
    // heads 8*(t%4)..+7; the 64 threads of a head are added in thread order
#pragma unroll
    for (int j = 0; j < 8; ++j) mpart[tid][j] = mass[j];
    __syncthreads();
    if (tid < 32) {
      const int q = tid >> 3, j = tid & 7;
      float m = 0.f;
      for (int t = q; t < 256; t += 4) m += mpart[t][j];
      a.kept_mass[int64_t(b) * H + 32 * hb + 8 * q + j] = m;
    }
  }
  if (hb == 0 && g == 0 && tid == 0) {
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

// LDS bytes of mla_scores; the float2 scratch must start 8-byte aligned, which
// the sizes below guarantee (every earlier region is a multiple of 16 bytes).
size_t mla_lds_bytes(int H, int P, int S) {
  const int NLT = P / LTILE;
  return size_t(NBUF) * BUF_BYTES + size_t(H) * NLT * 4 + size_t(H) * 4 +
         size_t((NLT + 3) & ~3) * 4 + TILE * 4 + 8 * 4 + size_t(H + S) * 8 + 64;
}

const void* mla_scores_kernel(int H) {
  if (H == 32) return reinterpret_cast<const void*>(&mla_scores<1>);
  if (H == 64) return reinterpret_cast<const void*>(&mla_scores<2>);
  if (H == 128) return reinterpret_cast<const void*>(&mla_scores<4>);
  return nullptr;
}
const void* mla_out_kernel() { return reinterpret_cast<const void*>(&mla_out); }

}  // namespace kvq
