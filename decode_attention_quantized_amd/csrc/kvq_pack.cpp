// Host-side packer for the KV-cache formats (see include/kvq.h for the format
// rules). Pure C++17 with float64 arithmetic; no HIP dependency, so the same
// file also builds with plain g++. Must be compiled with -ffp-contract=off so
// that no multiply-add is fused (every rounding step is the one written).
//
// Formats: q8_0, q4_0 and a turbo3-style LUT codebook are the ones the sparse
// V page ("Пропуск 90% работы по деквантизации…", tproger.ru, section "Почему
// это работает для любой квантизации") validated; the fp8 latent with
// BlockWise1x128 scaling is from "FP8 MLA KV compression projection"
// (kernelindex.com). Narrowing conversions here are written from the IEEE 754
// / OCP FP8 definitions (exponent from frexp, significand rounded with rint in
// the default round-to-nearest-even mode).

#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kvq.h"

namespace {

// float64 -> IEEE binary16 bits, round to nearest even, overflow -> inf.
uint16_t f64_to_f16(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  const double a = std::fabs(x);
  if (std::isnan(a)) return sign | 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u;           // >= max + half ulp rounds to inf
  if (a < 0x1p-14) {                                 // subnormal: multiples of 2^-24
    const double m = std::rint(a * 0x1p24);          // exact scaling, then RNE
    return sign | static_cast<uint16_t>(m);          // m == 1024 is the min normal
  }
  int e;
  std::frexp(a, &e);                                 // a = f * 2^e, f in [0.5, 1)
  double m = std::rint(std::ldexp(a, 11 - e));       // 11-bit significand in [1024, 2048]
  int E = e - 1 + 15;
  if (m == 2048.0) { m = 1024.0; E += 1; }
  if (E >= 31) return sign | 0x7C00u;
  return sign | static_cast<uint16_t>(E << 10) | static_cast<uint16_t>(m - 1024.0);
}

double f16_to_f64(uint16_t h) {
  const double s = (h & 0x8000u) ? -1.0 : 1.0;
  const int E = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  if (E == 0) return s * std::ldexp(static_cast<double>(m), -24);
  if (E == 31) return m ? NAN : s * INFINITY;
  return s * std::ldexp(static_cast<double>(1024 + m), E - 25);
}

// float64 in [-448, 448] -> OCP E4M3 (e4m3fn) byte, round to nearest even.
uint8_t f64_to_e4m3(double t) {
  const uint8_t sign = std::signbit(t) ? 0x80u : 0u;
  const double a = std::fabs(t);
  if (a < 0x1p-6) {                                  // subnormal: multiples of 2^-9
    const double m = std::rint(a * 0x1p9);           // m == 8 is the min normal 0x08
    return sign | static_cast<uint8_t>(m);
  }
  int e;
  std::frexp(a, &e);
  double m = std::rint(std::ldexp(a, 4 - e));        // 4-bit significand in [8, 16]
  int E = e - 1 + 7;
  if (m == 16.0) { m = 8.0; E += 1; }
  return sign | static_cast<uint8_t>(E << 3) | static_cast<uint8_t>(m - 8.0);
}

double e4m3_to_f64(uint8_t c) {
  const double s = (c & 0x80u) ? -1.0 : 1.0;
  const int E = (c >> 3) & 0xF;
  const int m = c & 7;
  if (E == 15 && m == 7) return NAN;
  if (E == 0) return s * std::ldexp(static_cast<double>(m), -9);
  return s * std::ldexp(static_cast<double>(8 + m), E - 10);
}

void put_u16(uint8_t* p, uint16_t v) { p[0] = v & 0xFF; p[1] = v >> 8; }
uint16_t get_u16(const uint8_t* p) { return static_cast<uint16_t>(p[0] | (p[1] << 8)); }
void put_f32(uint8_t* p, float f) { uint32_t u; std::memcpy(&u, &f, 4); for (int i = 0; i < 4; ++i) p[i] = (u >> (8 * i)) & 0xFF; }
float get_f32(const uint8_t* p) { uint32_t u = p[0] | (p[1] << 8) | (p[2] << 16) | (static_cast<uint32_t>(p[3]) << 24); float f; std::memcpy(&f, &u, 4); return f; }

// integer part of |t| plus one when the exact fraction reaches one half
double round_half_away(double t) {
  const double a = std::fabs(t);
  const double f = std::floor(a);
  const double r = (a - f >= 0.5) ? f + 1.0 : f;
  return std::copysign(r, t);
}

// floor(t + 1/2) computed without the rounding of t + 0.5
double round_half_up(double t) {
  const double f = std::floor(t);
  return (t - f >= 0.5) ? f + 1.0 : f;
}

// The four LUT3 magnitudes: the positive levels of the 8-level minimum-MSE
// (Lloyd-Max) quantizer of the standard normal, 0.2451 0.7560 1.3439 2.1519,
// each rounded to binary16.
constexpr uint16_t kLut3Bits[4] = {0x33D8, 0x3A0C, 0x3D60, 0x404E};

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
    for (int i = 0; i < 32; ++i) {
      double q = 0.0;
      if (d != 0.0) {
        q = round_half_away(static_cast<double>(xb[i]) / d);
        if (q > 127.0) q = 127.0;
        if (q < -127.0) q = -127.0;
      }
      codes[32 * b + i] = static_cast<uint8_t>(static_cast<int8_t>(q));
    }
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
    for (int i = 0; i < 32; ++i) {
      double v = 8.0;
      if (d != 0.0) {
        v = 8.0 + round_half_up(static_cast<double>(xb[i]) / d);
        if (v < 0.0) v = 0.0;
        if (v > 15.0) v = 15.0;
      }
      c[i] = static_cast<uint8_t>(v);
    }
    for (int j = 0; j < 16; ++j) codes[16 * b + j] = static_cast<uint8_t>(c[2 * j] | (c[2 * j + 1] << 4));
    put_u16(scales + 2 * b, dbits);
  }
  return KVQ_OK;
}

int32_t pack_lut3(const float* x, uint8_t* codes, uint8_t* scales) {
  double M[4], thr[3];
  for (int k = 0; k < 4; ++k) M[k] = f16_to_f64(kLut3Bits[k]);
  for (int k = 0; k < 3; ++k) thr[k] = (M[k] + M[k + 1]) / 2.0;
  double ss = 0.0;
  for (int i = 0; i < 128; ++i) { const double v = x[i]; ss = ss + v * v; }
  std::memset(codes, 0, 48);
  const double norm = std::sqrt(ss);
  if (norm == 0.0) { put_u16(scales, 0); return KVQ_OK; }
  const double r = std::sqrt(128.0) / norm;
  double lsq = 0.0;
  for (int i = 0; i < 128; ++i) {
    const double v = x[i];
    const double a = std::fabs(v * r);
    int idx = 0;
    for (int k = 0; k < 3; ++k) if (a > thr[k]) idx = k + 1;
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

int32_t pack_fp8(const float* x, int32_t dim, uint8_t* codes, uint8_t* scales) {
  for (int g0 = 0, gi = 0; g0 < dim; g0 += 128, ++gi) {
    const int g1 = (g0 + 128 < dim) ? g0 + 128 : dim;
    double amax = 0.0;
    for (int i = g0; i < g1; ++i) amax = std::fmax(amax, std::fabs(static_cast<double>(x[i])));
    const float s32 = static_cast<float>(amax / 448.0);
    const double s = s32;
    for (int i = g0; i < g1; ++i) {
      double t = 0.0;                                // a zero scale gives code 0x00
      if (s != 0.0) {
        t = static_cast<double>(x[i]) / s;
        if (t > 448.0) t = 448.0;
        if (t < -448.0) t = -448.0;
      }
      codes[i] = f64_to_e4m3(t);
    }
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
      case KVQ_LUT3: e = pack_lut3(x, c, s); break;
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
      case KVQ_LUT3: {
        const double nu = f16_to_f64(get_u16(s));
        for (int i = 0; i < 128; ++i) {
          unsigned code = 0;
          for (int k = 0; k < 3; ++k) code |= ((c[(3 * i + k) / 8] >> ((3 * i + k) % 8)) & 1u) << k;
          const int idx = code & 3;
          const bool neg = (code >> 2) & 1;
          const double m = f16_to_f64(kLut3Bits[idx]);
          y[i] = static_cast<float>((nu * (neg ? -m : m)) / std::sqrt(128.0));
        }
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

extern "C" int32_t kvq_lut3_levels(uint16_t* out4) {
  if (!out4) return KVQ_ERR_ARG;
  for (int k = 0; k < 4; ++k) out4[k] = kLut3Bits[k];
  return KVQ_OK;
}
