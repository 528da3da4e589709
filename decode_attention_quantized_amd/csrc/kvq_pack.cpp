// Host-side packer for the KV-cache formats (see include/kvq.h for the format
// rules). Pure C++17 with float64 arithmetic; no HIP dependency, so the same
// file also builds with plain g++. Must be compiled with -ffp-contract=off so
// that no multiply-add is fused (every rounding step is the one written). The
// scalar steps live in kvq_formats.h, which the device append packer shares.
//
// Formats: q8_0, q4_0 and a turbo3-style LUT codebook are the ones the sparse
// V page ("Пропуск 90% работы по деквантизации…", tproger.ru, section "Почему
// это работает для любой квантизации") validated; the fp8 latent with
// BlockWise1x128 scaling is from "FP8 MLA KV compression projection"
// (kernelindex.com).

#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kvq.h"
#include "kvq_formats.h"

namespace {

using namespace kvq::fmt;

void put_u16(uint8_t* p, uint16_t v) { p[0] = v & 0xFF; p[1] = v >> 8; }
uint16_t get_u16(const uint8_t* p) { return static_cast<uint16_t>(p[0] | (p[1] << 8)); }
void put_f32(uint8_t* p, float f) { uint32_t u; std::memcpy(&u, &f, 4); for (int i = 0; i < 4; ++i) p[i] = (u >> (8 * i)) & 0xFF; }
float get_f32(const uint8_t* p) { uint32_t u = p[0] | (p[1] << 8) | (p[2] << 16) | (static_cast<uint32_t>(p[3]) << 24); float f; std::memcpy(&f, &u, 4); return f; }

bool all_finite(const float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(x[i])) return false;
  return true;
}

int32_t pack_q8_0(const float* x, int32_t dim, uint8_t* codes, uint8_t* scales) {
  for (int b = 0; b < dim / 32; ++b) {
    const float* xb = x + 32 * b;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = std::fmax(amax, std::fabs(static_cast<double>(xb[i])));
    const uint16_t dbits = f64_to_f16(amax / 127.0);
    if ((dbits & 0x7C00u) == 0x7C00u) return KVQ_ERR_RANGE;
    const double d = f16_to_f64(dbits);
    for (int i = 0; i < 32; ++i) codes[32 * b + i] = d != 0.0 ? q8_code(xb[i], d) : 0;
    put_u16(scales + 2 * b, dbits);
  }
  return KVQ_OK;
}

int32_t pack_q4_0(const float* x, int32_t dim, uint8_t* codes, uint8_t* scales) {
  for (int b = 0; b < dim / 32; ++b) {
    const float* xb = x + 32 * b;
    int best = 0;
    for (int i = 1; i < 32; ++i)
      if (std::fabs(xb[i]) > std::fabs(xb[best])) best = i;     // first index on ties
    const uint16_t dbits = f64_to_f16(static_cast<double>(xb[best]) / -8.0);
    if ((dbits & 0x7C00u) == 0x7C00u) return KVQ_ERR_RANGE;
    const double d = f16_to_f64(dbits);
    uint8_t c[32];
    for (int i = 0; i < 32; ++i) c[i] = d != 0.0 ? q4_code(xb[i], d) : 8;
    for (int j = 0; j < 16; ++j) codes[16 * b + j] = static_cast<uint8_t>(c[2 * j] | (c[2 * j + 1] << 4));
    put_u16(scales + 2 * b, dbits);
  }
  return KVQ_OK;
}

// LUT3 of a float64 row (the input row widened, or the rotated row of
// LUT3-WHT, which stays float64)
int32_t pack_lut3_f64(const double* x, uint8_t* codes, uint8_t* scales) {
  double M[4];
  for (int k = 0; k < 4; ++k) M[k] = f16_to_f64(kLut3Bits[k]);
  double ss = 0.0;
  for (int i = 0; i < 128; ++i) { const double v = x[i]; ss = ss + v * v; }
  std::memset(codes, 0, 48);
  const double norm = std::sqrt(ss);
  if (norm == 0.0) { put_u16(scales, 0); return KVQ_OK; }
  const double r = std::sqrt(128.0) / norm;
  double lsq = 0.0;
  for (int i = 0; i < 128; ++i) {
    const double v = x[i];
    const int idx = lut3_index(v, r);
    const unsigned code = static_cast<unsigned>(idx) | (v < 0.0 ? 4u : 0u);
    // code i occupies bits 3i..3i+2 of the little-endian 384-bit row
    for (int k = 0; k < 3; ++k)
      if ((code >> k) & 1u) codes[(3 * i + k) / 8] |= static_cast<uint8_t>(1u << ((3 * i + k) % 8));
    lsq = lsq + M[idx] * M[idx];
  }
  const uint16_t nu = f64_to_f16((norm * std::sqrt(128.0)) / std::sqrt(lsq));
  if ((nu & 0x7C00u) == 0x7C00u) return KVQ_ERR_RANGE;
  put_u16(scales, nu);
  return KVQ_OK;
}

int32_t pack_lut3(const float* x, uint8_t* codes, uint8_t* scales, bool rotate) {
  double y[128];
  for (int i = 0; i < 128; ++i) y[i] = x[i];
  if (rotate) wht128(y);
  return pack_lut3_f64(y, codes, scales);
}

int32_t pack_fp8(const float* x, int32_t dim, uint8_t* codes, uint8_t* scales) {
  for (int g0 = 0, gi = 0; g0 < dim; g0 += 128, ++gi) {
    const int g1 = (g0 + 128 < dim) ? g0 + 128 : dim;
    double amax = 0.0;
    for (int i = g0; i < g1; ++i) amax = std::fmax(amax, std::fabs(static_cast<double>(x[i])));
    const float s32 = static_cast<float>(amax / 448.0);
    const double s = s32;
    for (int i = g0; i < g1; ++i) codes[i] = s != 0.0 ? fp8_code(x[i], s) : 0;   // zero scale: code 0x00
    put_f32(scales + 4 * gi, s32);
  }
  return KVQ_OK;
}

}  // namespace

extern "C" int32_t kvq_row_bytes(int32_t fmt, int32_t dim, int64_t* code_bytes, int64_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return KVQ_ERR_ARG;
  switch (fmt) {
    case KVQ_Q8_0:
      if (dim <= 0 || dim % 32) return KVQ_ERR_UNSUPPORTED;
      *code_bytes = dim; *scale_bytes = 2 * (dim / 32); return KVQ_OK;
    case KVQ_Q4_0:
      if (dim <= 0 || dim % 32) return KVQ_ERR_UNSUPPORTED;
      *code_bytes = dim / 2; *scale_bytes = 2 * (dim / 32); return KVQ_OK;
    case KVQ_LUT3:
    case KVQ_LUT3_WHT:
      if (dim != 128) return KVQ_ERR_UNSUPPORTED;
      *code_bytes = 48; *scale_bytes = 2; return KVQ_OK;
    case KVQ_FP8_B128:
      if (dim <= 0) return KVQ_ERR_UNSUPPORTED;
      *code_bytes = dim; *scale_bytes = 4 * ((dim + 127) / 128); return KVQ_OK;
    default:
      return KVQ_ERR_ARG;
  }
}

extern "C" int32_t kvq_pack(int32_t fmt, const float* src, int64_t n_rows, int32_t dim,
                            uint8_t* codes, uint8_t* scales) {
  int64_t cb = 0, sb = 0;
  const int32_t rc = kvq_row_bytes(fmt, dim, &cb, &sb);
  if (rc) return rc;
  if (n_rows < 0) return KVQ_ERR_ARG;
  if (n_rows == 0) return KVQ_OK;
  if (!src || !codes || !scales) return KVQ_ERR_ARG;
  if (!all_finite(src, n_rows * dim)) return KVQ_ERR_NONFINITE;
  if (std::fegetround() != FE_TONEAREST) return KVQ_ERR_ARG;
  for (int64_t r = 0; r < n_rows; ++r) {
    const float* x = src + r * dim;
    uint8_t* c = codes + r * cb;
    uint8_t* s = scales + r * sb;
    int32_t e = KVQ_OK;
    switch (fmt) {
      case KVQ_Q8_0: e = pack_q8_0(x, dim, c, s); break;
      case KVQ_Q4_0: e = pack_q4_0(x, dim, c, s); break;
      case KVQ_LUT3: e = pack_lut3(x, c, s, false); break;
      case KVQ_LUT3_WHT: e = pack_lut3(x, c, s, true); break;
      case KVQ_FP8_B128: e = pack_fp8(x, dim, c, s); break;
    }
    if (e) return e;
  }
  return KVQ_OK;
}

extern "C" int32_t kvq_unpack(int32_t fmt, const uint8_t* codes, const uint8_t* scales,
                              int64_t n_rows, int32_t dim, float* dst) {
  int64_t cb = 0, sb = 0;
  const int32_t rc = kvq_row_bytes(fmt, dim, &cb, &sb);
  if (rc) return rc;
  if (n_rows < 0) return KVQ_ERR_ARG;
  if (n_rows == 0) return KVQ_OK;
  if (!codes || !scales || !dst) return KVQ_ERR_ARG;
  for (int64_t r = 0; r < n_rows; ++r) {
    const uint8_t* c = codes + r * cb;
    const uint8_t* s = scales + r * sb;
    float* y = dst + r * dim;
    switch (fmt) {
      case KVQ_Q8_0:
        for (int i = 0; i < dim; ++i)
          y[i] = static_cast<float>(static_cast<int8_t>(c[i]) * f16_to_f64(get_u16(s + 2 * (i / 32))));
        break;
      case KVQ_Q4_0:
        for (int i = 0; i < dim; ++i) {
          const uint8_t byte = c[16 * (i / 32) + (i % 32) / 2];
          const int code = (i & 1) ? (byte >> 4) : (byte & 15);
          y[i] = static_cast<float>((code - 8) * f16_to_f64(get_u16(s + 2 * (i / 32))));
        }
        break;
      case KVQ_LUT3:
      case KVQ_LUT3_WHT: {
        const double nu = f16_to_f64(get_u16(s));
        double t[128];
        for (int i = 0; i < 128; ++i) {
          unsigned code = 0;
          for (int k = 0; k < 3; ++k) code |= ((c[(3 * i + k) / 8] >> ((3 * i + k) % 8)) & 1u) << k;
          const int idx = code & 3;
          const bool neg = (code >> 2) & 1;
          const double m = f16_to_f64(kLut3Bits[idx]);
          t[i] = (nu * (neg ? -m : m)) / std::sqrt(128.0);
        }
        if (fmt == KVQ_LUT3_WHT) wht128(t);           // the rotation is its own inverse
        for (int i = 0; i < 128; ++i) y[i] = static_cast<float>(t[i]);
        break;
      }
      case KVQ_FP8_B128:
        for (int i = 0; i < dim; ++i)
          y[i] = static_cast<float>(e4m3_to_f64(c[i]) * static_cast<double>(get_f32(s + 4 * (i / 128))));
        break;
    }
  }
  return KVQ_OK;
}

extern "C" int32_t kvq_key_norms(int32_t fmt, const void* codes, const void* scales, int64_t n_seqs,
                                 int32_t capacity, int32_t dim, float* out) {
  int64_t cb = 0, sb = 0;
  const int32_t rc = kvq_row_bytes(fmt, dim, &cb, &sb);
  if (rc) return rc;
  if (n_seqs < 0 || capacity < 1) return KVQ_ERR_ARG;
  if (n_seqs == 0) return KVQ_OK;
  if (!codes || !scales || !out) return KVQ_ERR_ARG;
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const uint8_t* s = static_cast<const uint8_t*>(scales);
  const int64_t nbc = (int64_t(capacity) + 63) / 64;
  for (int64_t q = 0; q < n_seqs; ++q)
    for (int64_t k = 0; k < nbc; ++k) {
      double m = 0.0;
      for (int64_t r = 64 * k; r < std::min<int64_t>(64 * k + 64, capacity); ++r) {
        const int64_t row = q * capacity + r;
        const double n = kvq::fmt::row_norm_f64(fmt, c + row * cb, s + row * sb, dim);
        if (n > m) m = n;
      }
      out[q * nbc + k] = kvq::fmt::f64_to_f32_up(m);
    }
  return KVQ_OK;
}

extern "C" int32_t kvq_lut3_levels(uint16_t* out4) {
  if (!out4) return KVQ_ERR_ARG;
  for (int k = 0; k < 4; ++k) out4[k] = kLut3Bits[k];
  return KVQ_OK;
}
