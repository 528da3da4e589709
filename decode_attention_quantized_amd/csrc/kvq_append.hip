// Device append packer: quantizes float32 rows that are already in device
// memory (the new token's key and value rows of a decode step, or a whole
// prefill) straight into a packed device cache, byte for byte as the host
// packer kvq_pack does. The per-element and per-scale steps are the shared
// ones of kvq_formats.h; what differs from the host loop is only the order of
// the order-free parts: block maxima (exact in any order), the first-index
// argmax of q4_0 (a reduction with the lower index winning ties) and the LUT3
// sum of squared magnitudes (a sum of 128 values with at most 36 significant
// bits, exact in any order). The LUT3 sum of squares of the input, whose
// rounding depends on the order, is added sequentially in element order as in
// the host packer.
//
// One wave per row, element i of a row on lane i mod 64. Must be compiled
// with -ffp-contract=off (as the host packer) so no multiply-add is fused.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kvq.h"
#include "kvq_formats.h"

namespace kvq {
namespace {

using namespace kvq::fmt;

constexpr int kWavesPerBlock = 4;
constexpr int kMaxBlocks = 65535;

// status bits a skipped row reports
constexpr int kBadInput = 1;      // a NaN or infinity in the row
constexpr int kBadScale = 2;      // a scale overflows fp16
constexpr int kBadDest = 4;       // destination row outside the cache

__device__ inline double max_over(double v, int width) {
  for (int o = width / 2; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

// orders this wave's LDS writes before its later LDS reads (a wave executes
// its LDS instructions in order; this keeps the compiler from moving them)
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ inline double sum_over(double v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

struct Row {
  const float* x;
  int dim;
  uint8_t* codes;
  uint8_t* scales;
  int lane;
};

// q8_0 and q4_0: blocks of 32; chunk c of a row (elements 64c..64c+63) has
// one block on lanes 0-31 and the next on lanes 32-63. NC chunks are handled
// together (independent chains the compiler interleaves): first the block
// scales, then, if no scale overflows anywhere in the row (a wave-wide
// decision), the codes. Returns the error bits.
template <int FMT, int NC>
__device__ int q_row(const Row& r) {
  float x[NC];
  uint16_t dbits[NC];
  bool bad = false;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 64 * c + r.lane;
    x[c] = i < r.dim ? r.x[i] : 0.f;                           // dim % 32 == 0: whole blocks
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (FMT == KVQ_Q8_0) {
      const double amax = max_over(fabs(static_cast<double>(x[c])), 32);
      dbits[c] = f64_to_f16(amax / 127.0);
    } else {
      // the element of largest magnitude, the first one on ties (the
      // reduction keeps the lower index when magnitudes are equal, which is
      // the host's forward scan with a strict comparison); its sign is kept
      float bv = fabsf(x[c]), bx = x[c];
      int bi = r.lane;
      for (int o = 16; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o), ox = __shfl_xor(bx, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bx = ox; bi = oi; }
      }
      dbits[c] = f64_to_f16(static_cast<double>(bx) / -8.0);
    }
    bad = bad || (dbits[c] & 0x7C00u) == 0x7C00u;
  }
  if (__ballot(bad)) return kBadScale;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 64 * c + r.lane;
    const bool in = i < r.dim;
    const double d = f16_to_f64(dbits[c]);
    if (FMT == KVQ_Q8_0) {
      if (in) r.codes[i] = d != 0.0 ? q8_code(x[c], d) : 0;
    } else {
      const uint8_t code = d != 0.0 ? q4_code(x[c], d) : 8;
      const uint8_t up = static_cast<uint8_t>(__shfl_down(static_cast<int>(code), 1));   // element i + 1
      if (in && (i & 1) == 0) r.codes[(i / 32) * 16 + (i & 31) / 2] = static_cast<uint8_t>(code | (up << 4));
    }
    if (in && (i & 31) == 0) reinterpret_cast<uint16_t*>(r.scales)[i / 32] = dbits[c];
  }
  return 0;
}

// Rows longer than 8 chunks: the same steps, 8 chunks at a time, with the
// scale check over the whole row before any write.
template <int FMT>
__device__ int q_row_long(const Row& r) {
  bool bad = false;
  for (int c0 = 0; c0 < r.dim; c0 += 64) {
    const int i = c0 + r.lane;
    const float x = i < r.dim ? r.x[i] : 0.f;
    uint16_t dbits;
    if (FMT == KVQ_Q8_0) {
      dbits = f64_to_f16(max_over(fabs(static_cast<double>(x)), 32) / 127.0);
    } else {
      float bv = fabsf(x), bx = x;
      int bi = r.lane;
      for (int o = 16; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o), ox = __shfl_xor(bx, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bx = ox; bi = oi; }
      }
      dbits = f64_to_f16(static_cast<double>(bx) / -8.0);
    }
    bad = bad || (dbits & 0x7C00u) == 0x7C00u;
  }
  if (__ballot(bad)) return kBadScale;
  for (int c0 = 0; c0 < r.dim; c0 += 8 * 64) {
    const Row part{r.x + c0, min(r.dim - c0, 8 * 64), r.codes + (FMT == KVQ_Q8_0 ? c0 : c0 / 2), r.scales + c0 / 16,
                   r.lane};
    q_row<FMT, 8>(part);
  }
  return 0;
}

template <int FMT>
__device__ int q_row_any(const Row& r) {
  switch ((r.dim + 63) / 64) {
    case 1: return q_row<FMT, 1>(r);
    case 2: return q_row<FMT, 2>(r);
    case 3: return q_row<FMT, 3>(r);
    case 4: return q_row<FMT, 4>(r);
    case 5: case 6: return q_row<FMT, 6>(r);
    case 7: case 8: return q_row<FMT, 8>(r);
    default: return q_row_long<FMT>(r);
  }
}

// fp8 with BlockWise1x128 scaling: groups of 128 (the last may be shorter),
// each spanning two 64-element chunks; NG groups handled together. No scale
// can overflow (fp32 scales of finite inputs), so one pass writes.
template <int NG>
__device__ void fp8_groups(const Row& r, int g0) {
  float x0[NG], x1[NG];
  float s32[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int b = g0 + 128 * g, e = min(b + 128, r.dim);
    x0[g] = b + r.lane < e ? r.x[b + r.lane] : 0.f;
    x1[g] = b + 64 + r.lane < e ? r.x[b + 64 + r.lane] : 0.f;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const double amax = max_over(fmax(fabs(static_cast<double>(x0[g])), fabs(static_cast<double>(x1[g]))), 64);
    s32[g] = static_cast<float>(amax / 448.0);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int b = g0 + 128 * g, e = min(b + 128, r.dim);
    if (b >= r.dim) continue;
    const double s = s32[g];
    if (b + r.lane < e) r.codes[b + r.lane] = s != 0.0 ? fp8_code(x0[g], s) : 0;
    if (b + 64 + r.lane < e) r.codes[b + 64 + r.lane] = s != 0.0 ? fp8_code(x1[g], s) : 0;
    if (r.lane == 0) reinterpret_cast<float*>(r.scales)[b / 128] = s32[g];
  }
}

__device__ void fp8_row(const Row& r) {
  const int ng = (r.dim + 127) / 128;
  if (ng == 1) fp8_groups<1>(r, 0);
  else if (ng == 2) fp8_groups<2>(r, 0);
  else if (ng <= 5) fp8_groups<5>(r, 0);
  else
    for (int g0 = 0; g0 < r.dim; g0 += 8 * 128) fp8_groups<8>(r, g0);
}

// The Walsh-Hadamard rotation of kvq_formats.h's wht128 on a row held as
// elements (lane, lane + 64): the same butterflies in the same stage order
// (stages h < 64 pair lanes l and l ^ h, stage 64 the two elements of a
// lane), each one float64 addition, then the one multiply.
__device__ inline void wht_lanes(int lane, double& v0, double& v1) {
  for (int h = 1; h < 64; h *= 2) {
    const double p0 = __shfl_xor(v0, h), p1 = __shfl_xor(v1, h);
    const bool upper = lane & h;
    v0 = upper ? p0 - v0 : v0 + p0;
    v1 = upper ? p1 - v1 : v1 + p1;
  }
  const double a = v0, b = v1;
  v0 = a + b;
  v1 = a - b;
  v0 = v0 * kWhtScale;
  v1 = v1 * kWhtScale;
}

// LUT3 (128-wide rows): norm from the sequential float64 sum of squares,
// magnitude indices against the level midpoints, and the row scalar that
// keeps the decoded norm; one pass, written only when the scalar fits fp16.
// ROTATE: LUT3_WHT, the row is rotated first (and stays float64).
// `sq` is this wave's 128 doubles of LDS, `cb` its 128 bytes.
template <bool ROTATE>
__device__ int lut3_row(const Row& r, double* sq, uint8_t* cb) {
  double v0 = r.x[r.lane], v1 = r.x[r.lane + 64];
  if (ROTATE) wht_lanes(r.lane, v0, v1);
  sq[r.lane] = v0 * v0;
  sq[r.lane + 64] = v1 * v1;
  wave_lds_order();
  double ss = 0.0;
  if (r.lane == 0)
    for (int i = 0; i < 128; ++i) ss = ss + sq[i];
  ss = __shfl(ss, 0);
  const double norm = sqrt(ss);
  if (norm == 0.0) {
    if (r.lane < 48) r.codes[r.lane] = 0;
    if (r.lane == 0) reinterpret_cast<uint16_t*>(r.scales)[0] = 0;
    return 0;
  }
  const double rr = sqrt(128.0) / norm;
  const int k0 = lut3_index(v0, rr), k1 = lut3_index(v1, rr);
  const double m0 = f16_to_f64(kLut3Bits[k0]), m1 = f16_to_f64(kLut3Bits[k1]);
  const double lsq = sum_over(m0 * m0 + m1 * m1);              // exact, so order-free
  const uint16_t nu = f64_to_f16((norm * sqrt(128.0)) / sqrt(lsq));
  if ((nu & 0x7C00u) == 0x7C00u) return kBadScale;
  cb[r.lane] = static_cast<uint8_t>(k0 | (v0 < 0.0 ? 4 : 0));
  cb[r.lane + 64] = static_cast<uint8_t>(k1 | (v1 < 0.0 ? 4 : 0));
  wave_lds_order();
  if (r.lane < 48) {
    // byte b holds bits 8b..8b+7 of the little-endian string, element e at bits 3e..3e+2
    unsigned byte = 0;
    for (int k = 0; k < 8; ++k) {
      const int bit = 8 * r.lane + k;
      byte |= ((cb[bit / 3] >> (bit % 3)) & 1u) << k;
    }
    r.codes[r.lane] = static_cast<uint8_t>(byte);
  }
  if (r.lane == 0) reinterpret_cast<uint16_t*>(r.scales)[0] = nu;
  return 0;
}

// One set of rows to pack: sources and the planes they go to.
struct Job {
  const float* src;
  uint8_t* codes;
  uint8_t* scales;
};

// Waves walk the rows of job 0 then job 1 (n_rows each); both jobs use the
// same destination rows (a key and a value cache share their layout).
__global__ __launch_bounds__(64 * kWavesPerBlock) void append_rows(int32_t fmt, Job j0, Job j1, int32_t njobs,
                                                                   int64_t n_rows, int32_t dim,
                                                                   const int64_t* __restrict__ dst_rows, int64_t cb,
                                                                   int64_t sb, int64_t cache_rows, int32_t* status) {
  __shared__ double sq[kWavesPerBlock][128];
  __shared__ uint8_t cbuf[kWavesPerBlock][128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t t = int64_t(blockIdx.x) * kWavesPerBlock + wave; t < njobs * n_rows;
       t += int64_t(gridDim.x) * kWavesPerBlock) {
    const bool second = t >= n_rows;
    const int64_t row = second ? t - n_rows : t;
    const Job& jb = second ? j1 : j0;
    const float* x = jb.src + row * dim;
    const int64_t dst = dst_rows ? dst_rows[row] : row;
    int err = (dst < 0 || dst >= cache_rows) ? kBadDest : 0;
    bool finite = true;
    for (int i = lane; i < dim; i += 64) finite = finite && __builtin_isfinite(x[i]);
    if (__ballot(!finite)) err |= kBadInput;
    if (err == 0) {
      const Row r{x, dim, jb.codes + dst * cb, jb.scales + dst * sb, lane};
      int e = 0;
      switch (fmt) {
        case KVQ_Q8_0: e = q_row_any<KVQ_Q8_0>(r); break;
        case KVQ_Q4_0: e = q_row_any<KVQ_Q4_0>(r); break;
        case KVQ_LUT3: e = lut3_row<false>(r, sq[wave], cbuf[wave]); break;
        case KVQ_LUT3_WHT: e = lut3_row<true>(r, sq[wave], cbuf[wave]); break;
        case KVQ_FP8_B128: fp8_row(r); break;
      }
      err |= e;
    }
    if (err && lane == 0 && status) atomicOr(status, err);
  }
}

int32_t launch_append(int32_t fmt, const Job* jobs, int njobs, int64_t n_rows, int32_t dim, const int64_t* dst_rows,
                      int64_t cache_rows, int32_t* status, void* stream) {
  int64_t cb = 0, sb = 0;
  const int32_t rc = kvq_row_bytes(fmt, dim, &cb, &sb);
  if (rc) return rc;
  if (n_rows < 0 || cache_rows < 0) return KVQ_ERR_ARG;
  if (n_rows == 0) return KVQ_OK;
  for (int j = 0; j < njobs; ++j) {
    if (!jobs[j].src || !jobs[j].codes || !jobs[j].scales) return KVQ_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(jobs[j].src) & 3) || (reinterpret_cast<uintptr_t>(jobs[j].codes) & 15) ||
        (reinterpret_cast<uintptr_t>(jobs[j].scales) & 15))
      return KVQ_ERR_ALIGN;
  }
  if (reinterpret_cast<uintptr_t>(dst_rows) & 7) return KVQ_ERR_ALIGN;
  if (!dst_rows && n_rows > cache_rows) return KVQ_ERR_RANGE;
  const int64_t blocks = (njobs * n_rows + kWavesPerBlock - 1) / kWavesPerBlock;
  const unsigned grid = static_cast<unsigned>(blocks < kMaxBlocks ? blocks : kMaxBlocks);
  hipLaunchKernelGGL(append_rows, dim3(grid), dim3(64 * kWavesPerBlock), 0, static_cast<hipStream_t>(stream), fmt,
                     jobs[0], jobs[njobs - 1], njobs, n_rows, dim, dst_rows, cb, sb, cache_rows, status);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

// Largest dequantized row norm of 64-row blocks (the summaries the decode
// kernel's key skipping reads): one wave per block, lane r takes row 64k + r
// of its sequence-head and computes the row's float64 norm with the host
// packer's function (sum of squares in element order), the wave takes the
// maximum and lane 0 stores it rounded up to float32. Blocks come from a
// list of flat ids (sequence-head * blocks per capacity + block) or, with
// no list, are all blocks.
__global__ __launch_bounds__(64 * kWavesPerBlock) void key_norms_rows(int32_t fmt, const uint8_t* codes,
                                                                      const uint8_t* scales, int64_t cb, int64_t sb,
                                                                      int64_t n_seqs, int32_t capacity, int32_t dim,
                                                                      const int64_t* blocks, int64_t n_blocks,
                                                                      float* norms, int32_t* status) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nbc = (int64_t(capacity) + 63) / 64;
  for (int64_t i = int64_t(blockIdx.x) * kWavesPerBlock + wave; i < n_blocks; i += int64_t(gridDim.x) * kWavesPerBlock) {
    const int64_t fb = blocks ? blocks[i] : i;
    if (fb < 0 || fb >= n_seqs * nbc) {                  // uniform across the wave
      if (lane == 0 && status) atomicOr(status, 8);
      continue;
    }
    const int64_t q = fb / nbc, r = (fb - q * nbc) * 64 + lane;
    double n = 0.0;
    if (r < capacity) {
      const int64_t row = q * capacity + r;
      n = fmt::row_norm_f64(fmt, codes + row * cb, scales + row * sb, dim);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n = fmax(n, __shfl_xor(n, o));
    if (lane == 0) norms[fb] = fmt::f64_to_f32_up(n);
  }
}

}  // namespace
}  // namespace kvq

extern "C" int32_t kvq_key_norms_device(int32_t fmt, const void* codes, const void* scales, int64_t n_seqs,
                                        int32_t capacity, int32_t dim, const int64_t* blocks, int64_t n_blocks,
                                        float* norms, int32_t* status, void* stream) {
  int64_t cb = 0, sb = 0;
  const int32_t rc = kvq_row_bytes(fmt, dim, &cb, &sb);
  if (rc) return rc;
  if (n_seqs < 0 || capacity < 1 || n_blocks < 0) return KVQ_ERR_ARG;
  const int64_t total = n_seqs * ((int64_t(capacity) + 63) / 64);
  if (!blocks) n_blocks = total;
  if (n_blocks == 0) return KVQ_OK;
  if (!codes || !scales || !norms) return KVQ_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(norms) & 3) || (reinterpret_cast<uintptr_t>(blocks) & 7)) return KVQ_ERR_ALIGN;
  const int64_t grid = std::min<int64_t>((n_blocks + kvq::kWavesPerBlock - 1) / kvq::kWavesPerBlock, kvq::kMaxBlocks);
  hipLaunchKernelGGL(kvq::key_norms_rows, dim3(unsigned(grid)), dim3(64 * kvq::kWavesPerBlock), 0,
                     static_cast<hipStream_t>(stream), fmt, static_cast<const uint8_t*>(codes),
                     static_cast<const uint8_t*>(scales), cb, sb, n_seqs, capacity, dim, blocks, n_blocks, norms,
                     status);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

extern "C" int32_t kvq_append(int32_t fmt, const float* src, int64_t n_rows, int32_t dim, const int64_t* dst_rows,
                              void* codes, void* scales, int64_t cache_rows, int32_t* status, void* stream) {
  const kvq::Job job{src, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales)};
  return kvq::launch_append(fmt, &job, 1, n_rows, dim, dst_rows, cache_rows, status, stream);
}

extern "C" int32_t kvq_append_kv(int32_t fmt, const float* k_src, const float* v_src, int64_t n_rows, int32_t dim,
                                 const int64_t* dst_rows, void* k_codes, void* k_scales, void* v_codes,
                                 void* v_scales, int64_t cache_rows, int32_t* status, void* stream) {
  const kvq::Job jobs[2] = {{k_src, static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(k_scales)},
                            {v_src, static_cast<uint8_t*>(v_codes), static_cast<uint8_t*>(v_scales)}};
  return kvq::launch_append(fmt, jobs, 2, n_rows, dim, dst_rows, cache_rows, status, stream);
}
