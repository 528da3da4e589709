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
//              32w..32w+31 with q resident in registers as f16 MFMA operands)
//    1. streams 32-row latent tiles through LDS (double-buffered), scores
//       them with v_mfma_f32_32x32x16_f16 (fp8 -> f16 with the hardware
//       converter, exact), applies the per-group fp32 scale to the fp32
//       accumulator, keeps per-head (max, sum exp2) and a per-(head,
//       64-position tile) maximum;
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

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned long long u64;

constexpr int D = 576;          // latent width (scores)
constexpr int DV = 512;         // value width
constexpr int KSTEPS = D / 16;  // 36 MFMA k-steps of 16 dims
constexpr int NGROUPS = 5;      // scale groups: 4 x 128 + 1 x 64
constexpr int ROW_LDS = 584;    // LDS pitch of a staged latent row (576 + 8; keeps b64 reads conflict-free)
constexpr int TILE = 32;        // positions per MFMA tile
constexpr int LTILE = 64;       // positions per liveness tile
constexpr uint32_t kSpinLimit = 1u << 23;

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

__device__ inline void online_add(float& m, float& l, float s) {
  if (s == -INFINITY) return;
  if (s > m) { l = l * exp2f(m - s) + 1.f; m = s; }
  else l += exp2f(s - m);
}

// 8 fp8 e4m3 bytes -> 8 f16 (exact: every e4m3 value is an f16 value)
__device__ inline half8 fp8x8_to_f16(uint2 w) {
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false));
  u.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true));
  u.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false));
  u.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true));
  return __builtin_bit_cast(half8, u);
}

__device__ inline int group_of_kstep(int ks) { return ks < 32 ? ks >> 3 : 4; }

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
  uint8_t* tiles = smem;                                                 // [2][32][ROW_LDS]
  float* tscale = reinterpret_cast<float*>(tiles + 2 * TILE * ROW_LDS);  // [2][32][5]
  float* tmax = tscale + 2 * TILE * NGROUPS;                             // [H][NLT]
  float* lse = tmax + H * NLT;                                           // [H]
  float* hsl = lse + H;                                                  // [H] per-head score scale
  int* live = reinterpret_cast<int*>(hsl + H);                           // [NLT (+pad)]
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

  if (blockIdx.x == 0 && tid == 0) {
    a.hdr->batch = a.B; a.hdr->q_heads = H; a.hdr->kv_heads = 1; a.hdr->ctx = ctx;
    a.hdr->splits = a.S; a.hdr->positions_per_split = P; a.hdr->fmt = KVQ_FP8_B128; a.hdr->v_dim = DV;
    a.hdr->nwg = int(gridDim.x);
    a.hdr->k_row_bytes = D + 4 * NGROUPS;               // a whole latent row
    a.hdr->v_row_bytes = DV + 4 * (DV / 128);           // its value part
  }

  // ---------------------------------------------------------------- tile staging
  // a 32-row tile = 32 x 36 chunks of 16 bytes + 32 x 5 scales; loads go to
  // registers first so they can be in flight while the previous tile computes
  constexpr int CHUNKS = TILE * (D / 16);
  constexpr int PER = (CHUNKS + NT - 1) / NT;
  constexpr int NSC = TILE * NGROUPS;
  constexpr int PERS = (NSC + NT - 1) / NT;
  struct Staged { uint4 v[PER]; float s[PERS]; };
  auto stage_load = [&](int t) {
    Staged st;
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
    return st;
  };
  auto stage_store = [&](const Staged& st, int buf) {
    uint8_t* dst = tiles + buf * TILE * ROW_LDS;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      if (i < CHUNKS) {
        const int r = i / (D / 16), c = i - r * (D / 16);
        uint2* d2 = reinterpret_cast<uint2*>(dst + r * ROW_LDS + c * 16);
        d2[0] = make_uint2(st.v[k].x, st.v[k].y);
        d2[1] = make_uint2(st.v[k].z, st.v[k].w);
      }
    }
#pragma unroll
    for (int k = 0; k < PERS; ++k)
      if (tid + k * NT < NSC) tscale[buf * NSC + tid + k * NT] = st.s[k];
  };
  auto stage = [&](int t, int buf) { stage_store(stage_load(t), buf); };

  // ---------------------------------------------------------------- q operands
  // per-head power-of-two prescale so the bf16 query fits f16 without loss
  half8 A[KSTEPS];
  {
    float mx = 0.f;
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + (int64_t(b) * H + head_a) * D + 8 * kh;
    uint4 raw[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) raw[ks] = *reinterpret_cast<const uint4*>(qh + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint32_t w[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mx = fmaxf(mx, fabsf(__uint_as_float(w[e] << 16)));
        mx = fmaxf(mx, fabsf(__uint_as_float(w[e] & 0xFFFF0000u)));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int ex = (mx > 0.f) ? ilogbf(mx) + 1 : 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint32_t w[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
      half8 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[2 * e] = _Float16(ldexpf(__uint_as_float(w[e] << 16), -ex));
        h[2 * e + 1] = _Float16(ldexpf(__uint_as_float(w[e] & 0xFFFF0000u), -ex));
      }
      A[ks] = h;
    }
    if (kh == 0) hsl[head_a] = ldexpf(a.sigma_log2e, ex);
  }
  stage(0, 0);
  __syncthreads();
  // per-accumulator head scale: accumulator 4i+j of lane holds head 8i + 4kh + j (of this wave)
  float hsc[16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) hsc[4 * i + j] = hsl[32 * wave + 8 * i + 4 * kh + j];

  // scores of staged tile `buf` (log2 domain), 16 heads of this lane x its column
  auto score_tile = [&](int buf, int t, floatx16& s2) {
    const uint8_t* src = tiles + buf * TILE * ROW_LDS + col * ROW_LDS + 8 * kh;
    const float* sc = tscale + buf * TILE * NGROUPS + col * NGROUPS;
    floatx16 acc = {};
#pragma unroll
    for (int g = 0; g < NGROUPS; ++g) {
      floatx16 cg = {};
      const int k0 = 8 * g, k1 = (g < 4) ? 8 * g + 8 : KSTEPS;
#pragma unroll
      for (int ks = k0; ks < k1; ++ks) {
        const uint2 w = *reinterpret_cast<const uint2*>(src + 16 * ks);
        cg = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[ks], fp8x8_to_f16(w), cg, 0, 0, 0);
      }
      const float s = sc[g];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = fmaf(s, cg[e], acc[e]);
    }
    const bool valid = pos0 + t * TILE + col < ctx;
#pragma unroll
    for (int e = 0; e < 16; ++e) s2[e] = valid ? acc[e] * hsc[e] : -INFINITY;
  };

  // ---------------------------------------------------------------- phase 1
  float m[16], l[16], tm[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) { m[e] = -INFINITY; l[e] = 0.f; tm[e] = -INFINITY; }
  const int T = P / TILE;
  for (int t = 0; t < T; ++t) {
    Staged nxt;
    if (t + 1 < T) nxt = stage_load(t + 1);         // next tile's loads overlap this tile's MFMAs
    floatx16 s2;
    score_tile(t & 1, t, s2);
#pragma unroll
    for (int e = 0; e < 16; ++e) { online_add(m[e], l[e], s2[e]); tm[e] = fmaxf(tm[e], s2[e]); }
    if (t & 1) {                                    // end of a 64-position liveness tile
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = tm[e];
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 32));
        tm[e] = v;
      }
      if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) tmax[(32 * wave + 8 * i + 4 * kh + j) * NLT + (t >> 1)] = tm[4 * i + j];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) tm[e] = -INFINITY;
    }
    if (t + 1 < T) stage_store(nxt, (t + 1) & 1);
    __syncthreads();                                // buffer (t & 1) free; buffer (t+1)&1 staged
  }
  // split statistics per head: merge over the 32 columns, publish
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float2 x = make_float2(m[e], l[e]);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      float2 y;
      y.x = __shfl_xor(x.x, o, 32);
      y.y = __shfl_xor(x.y, o, 32);
      x = lse_merge(x, y);
    }
    m[e] = x.x; l[e] = x.y;
  }
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
      stage(t, 0);
      if (tid < TILE) keepmask[tid] = 0u;
      __syncthreads();
      floatx16 s2;
      score_tile(0, t, s2);
      // normalized weights and keep bits
      unsigned bits = 0u;
      float p[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * i + j;
          const float pe = (s2[e] == -INFINITY) ? 0.f : exp2f(s2[e] - lse[32 * wave + 8 * i + 4 * kh + j]);
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
}

// ----------------------------------------------------------------------------- out
// One workgroup per (sequence, 32 heads, 128 value dims): thread t owns head
// 32*hb + t/8 and dims 128*db + 16*(t%8) .. +15.
__global__ __launch_bounds__(256) void mla_out(MlaArgs a) {
  const int H = a.Hq;
  const int nhb = H / 32, ndb = DV / 128;
  const int b = blockIdx.x / (nhb * ndb);
  const int rem = blockIdx.x - b * nhb * ndb;
  const int hb = rem / ndb, db = rem - hb * ndb;
  const int tid = threadIdx.x;
  const int h = 32 * hb + (tid >> 3);
  const int d0 = 128 * db + 16 * (tid & 7);
  const int64_t row0 = int64_t(b) * a.cap;
  const uint32_t epoch_next =
      __hip_atomic_load(&a.hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  float mass = 0.f;
  int rows = 0;
  long long pairs = 0;
  for (int sp = 0; sp < a.S; ++sp) {
    const int64_t kbase = int64_t(b) * a.S + sp;
    const int n = a.kcount[kbase];
    rows += n;
    pairs += a.kpairs[kbase];
    for (int k0 = 0; k0 < n; k0 += 8) {
      int pos[8];
      float p[8];
      uint4 v[8];
      float s[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = k0 + u < n;
        pos[u] = in ? a.kpos[kbase * a.P + k0 + u] : 0;
        p[u] = in ? a.kp[(kbase * a.P + k0 + u) * H + h] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = k0 + u < n;
        v[u] = in ? *reinterpret_cast<const uint4*>(a.kc + (row0 + pos[u]) * D + d0) : make_uint4(0u, 0u, 0u, 0u);
        s[u] = in ? reinterpret_cast<const float*>(a.ks + (row0 + pos[u]) * (4 * NGROUPS))[db] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u >= n) break;
        mass += p[u];
        const float ps = p[u] * s[u];
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[q], 1.0f, false);
          const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[q], 1.0f, true);
          o[4 * q + 0] = fmaf(ps, float(lo[0]), o[4 * q + 0]);
          o[4 * q + 1] = fmaf(ps, float(lo[1]), o[4 * q + 1]);
          o[4 * q + 2] = fmaf(ps, float(hi[0]), o[4 * q + 2]);
          o[4 * q + 3] = fmaf(ps, float(hi[1]), o[4 * q + 3]);
        }
      }
    }
  }
  float* dst = a.out + (int64_t(b) * H + h) * DV + d0;
#pragma unroll
  for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
  if (db == 0 && (tid & 7) == 0) a.kept_mass[int64_t(b) * H + h] = mass;
  if (hb == 0 && db == 0 && tid == 0) {
    a.bgstat[2 * b] = (unsigned long long)pairs;
    a.bgstat[2 * b + 1] = (unsigned long long)rows;
  }
  // the last sequence's output workgroup advances the epoch for the next call
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
  return size_t(2) * TILE * ROW_LDS + 2 * TILE * NGROUPS * 4 + size_t(H) * NLT * 4 + 2 * size_t(H) * 4 +
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
