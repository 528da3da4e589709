// Scalar steps of the packed formats (the format rules are in include/kvq.h),
// shared by the host packer (kvq_pack.cpp, plain C++) and the device append
// packer (kvq_append.hip), so both quantize with one definition. float64
// throughout; narrowing conversions are written from the IEEE 754 binary16
// and OCP FP8 E4M3 definitions (exponent from frexp, significand rounded
// with rint in the default round-to-nearest-even mode). Every translation
// unit that includes this must be compiled without multiply-add contraction
// (-ffp-contract=off) so each rounding step is the one written.
#ifndef KVQ_FORMATS_H
#define KVQ_FORMATS_H

#include <math.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define KVQ_HD __host__ __device__
#else
#define KVQ_HD
#endif

namespace kvq {
namespace fmt {

// float64 -> IEEE binary16 bits, round to nearest even, overflow -> inf.
KVQ_HD inline uint16_t f64_to_f16(double x) {
  const uint16_t sign = __builtin_signbit(x) ? 0x8000u : 0u;
  const double a = fabs(x);
  if (__builtin_isnan(a)) return sign | 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u;           // >= max + half ulp rounds to inf
  if (a < 0x1p-14) {                                 // subnormal: multiples of 2^-24
    const double m = rint(a * 0x1p24);               // exact scaling, then RNE
    return sign | static_cast<uint16_t>(m);          // m == 1024 is the min normal
  }
  int e;
  frexp(a, &e);                                      // a = f * 2^e, f in [0.5, 1)
  double m = rint(ldexp(a, 11 - e));                 // 11-bit significand in [1024, 2048]
  int E = e - 1 + 15;
  if (m == 2048.0) { m = 1024.0; E += 1; }
  if (E >= 31) return sign | 0x7C00u;
  return sign | static_cast<uint16_t>(E << 10) | static_cast<uint16_t>(m - 1024.0);
}

KVQ_HD inline double f16_to_f64(uint16_t h) {
  const double s = (h & 0x8000u) ? -1.0 : 1.0;
  const int E = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  if (E == 0) return s * ldexp(static_cast<double>(m), -24);
  if (E == 31) return m ? __builtin_nan("") : s * __builtin_inf();
  return s * ldexp(static_cast<double>(1024 + m), E - 25);
}

// float64 in [-448, 448] -> OCP E4M3 (e4m3fn) byte, round to nearest even.
KVQ_HD inline uint8_t f64_to_e4m3(double t) {
  const uint8_t sign = __builtin_signbit(t) ? 0x80u : 0u;
  const double a = fabs(t);
  if (a < 0x1p-6) {                                  // subnormal: multiples of 2^-9
    const double m = rint(a * 0x1p9);                // m == 8 is the min normal 0x08
    return sign | static_cast<uint8_t>(m);
  }
  int e;
  frexp(a, &e);
  double m = rint(ldexp(a, 4 - e));                  // 4-bit significand in [8, 16]
  int E = e - 1 + 7;
  if (m == 16.0) { m = 8.0; E += 1; }
  return sign | static_cast<uint8_t>(E << 3) | static_cast<uint8_t>(m - 8.0);
}

KVQ_HD inline double e4m3_to_f64(uint8_t c) {
  const double s = (c & 0x80u) ? -1.0 : 1.0;
  const int E = (c >> 3) & 0xF;
  const int m = c & 7;
  if (E == 15 && m == 7) return __builtin_nan("");
  if (E == 0) return s * ldexp(static_cast<double>(m), -9);
  return s * ldexp(static_cast<double>(8 + m), E - 10);
}

// integer part of |t| plus one when the exact fraction reaches one half
KVQ_HD inline double round_half_away(double t) {
  const double a = fabs(t);
  const double f = floor(a);
  const double r = (a - f >= 0.5) ? f + 1.0 : f;
  return copysign(r, t);
}

// floor(t + 1/2) computed without the rounding of t + 0.5
KVQ_HD inline double round_half_up(double t) {
  const double f = floor(t);
  return (t - f >= 0.5) ? f + 1.0 : f;
}

// q8_0 code of x for block scale d (d != 0): x/d rounded half away, clamped
KVQ_HD inline uint8_t q8_code(float x, double d) {
  double q = round_half_away(static_cast<double>(x) / d);
  if (q > 127.0) q = 127.0;
  if (q < -127.0) q = -127.0;
  return static_cast<uint8_t>(static_cast<int8_t>(q));
}

// q4_0 code of x for block scale d (d != 0): floor(x/d + 1/2) + 8, clamped
KVQ_HD inline uint8_t q4_code(float x, double d) {
  double v = 8.0 + round_half_up(static_cast<double>(x) / d);
  if (v < 0.0) v = 0.0;
  if (v > 15.0) v = 15.0;
  return static_cast<uint8_t>(v);
}

// fp8 code of x for group scale s (s != 0): e4m3(clamp(x/s, -448, 448))
KVQ_HD inline uint8_t fp8_code(float x, double s) {
  double t = static_cast<double>(x) / s;
  if (t > 448.0) t = 448.0;
  if (t < -448.0) t = -448.0;
  return f64_to_e4m3(t);
}

// The four LUT3 magnitudes: the positive levels of the 8-level minimum-MSE
// (Lloyd-Max) quantizer of the standard normal, 0.2451 0.7560 1.3439 2.1519,
// each rounded to binary16.
constexpr uint16_t kLut3Bits[4] = {0x33D8, 0x3A0C, 0x3D60, 0x404E};

// LUT3 magnitude index of |v * r| against the midpoints of the magnitudes
// (ties to the smaller magnitude)
KVQ_HD inline int lut3_index(double v, double r) {
  const double a = fabs(v * r);
  int idx = 0;
  for (int k = 0; k < 3; ++k) {
    const double thr = (f16_to_f64(kLut3Bits[k]) + f16_to_f64(kLut3Bits[k + 1])) / 2.0;
    if (a > thr) idx = k + 1;
  }
  return idx;
}

// y = H x / sqrt(128) for a 128-wide row, H the Sylvester Hadamard matrix
// (H[i][j] = (-1)^popcount(i & j)): butterflies (a, b) -> (a + b, a - b) for
// h = 1, 2, ..., 64 over pairs (j, j + h) with j mod 2h < h, each one float64
// addition, then one multiply by the float64 value of 1/sqrt(128). The
// transform is its own inverse.
constexpr double kWhtScale = 0.088388347648318440550;      // 1/sqrt(128), correctly rounded

KVQ_HD inline void wht128(double* y) {
  for (int h = 1; h < 128; h *= 2)
    for (int j0 = 0; j0 < 128; j0 += 2 * h)
      for (int j = j0; j < j0 + h; ++j) {
        const double a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
  for (int i = 0; i < 128; ++i) y[i] = y[i] * kWhtScale;
}

// Little-endian loads from byte planes.
KVQ_HD inline uint16_t ld_u16(const uint8_t* p) { return uint16_t(p[0] | (p[1] << 8)); }
KVQ_HD inline float ld_f32(const uint8_t* p) {
  const uint32_t u = uint32_t(p[0]) | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16) | (uint32_t(p[3]) << 24);
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

// Element i of a dequantized row in float64 for the formats whose elements
// stand alone (q8_0, q4_0: code times the block's fp16 scale; FP8-B128: the
// e4m3 value times its group's fp32 scale). fmt: 0 = q8_0, 1 = q4_0, 3 = fp8.
KVQ_HD inline double dequant_elem_f64(int fmt, const uint8_t* c, const uint8_t* s, int i) {
  if (fmt == 0) return static_cast<int8_t>(c[i]) * f16_to_f64(ld_u16(s + 2 * (i / 32)));
  if (fmt == 1) {
    const uint8_t byte = c[16 * (i / 32) + (i % 32) / 2];
    const int code = (i & 1) ? (byte >> 4) : (byte & 15);
    return (code - 8) * f16_to_f64(ld_u16(s + 2 * (i / 32)));
  }
  return e4m3_to_f64(c[i]) * static_cast<double>(ld_f32(s + 4 * (i / 128)));
}

// A LUT3 row (128 elements) dequantized in float64: element i is the norm
// scalar times the signed table magnitude of its 3-bit code, over sqrt(128);
// the rotated variant then applies the (self-inverse) transform.
KVQ_HD inline void dequant_lut3_f64(bool rotated, const uint8_t* c, const uint8_t* s, double* t) {
  const double nu = f16_to_f64(ld_u16(s));
  for (int i = 0; i < 128; ++i) {
    unsigned code = 0;
    for (int k = 0; k < 3; ++k) code |= ((c[(3 * i + k) / 8] >> ((3 * i + k) % 8)) & 1u) << k;
    const double m = f16_to_f64(kLut3Bits[code & 3]);
    t[i] = (nu * ((code >> 2) & 1 ? -m : m)) / sqrt(128.0);
  }
  if (rotated) wht128(t);
}

// Norm of a dequantized row: the square root of the float64 sum of squares
// added in element order. fmt as in include/kvq.h (LUT3 rows are 128 wide).
KVQ_HD inline double row_norm_f64(int fmt, const uint8_t* c, const uint8_t* s, int dim) {
  double acc = 0.0;
  if (fmt == 2 || fmt == 4) {
    double t[128];
    dequant_lut3_f64(fmt == 4, c, s, t);
    for (int i = 0; i < 128; ++i) acc += t[i] * t[i];
  } else {
    for (int i = 0; i < dim; ++i) {
      const double y = dequant_elem_f64(fmt, c, s, i);
      acc += y * y;
    }
  }
  return sqrt(acc);
}

// float64 -> float32 rounded toward +infinity (never below x; x >= 0 finite).
KVQ_HD inline float f64_to_f32_up(double x) {
  float f = static_cast<float>(x);
  if (static_cast<double>(f) < x) f = nextafterf(f, INFINITY);
  return f;
}

}  // namespace fmt
}  // namespace kvq

#endif  // KVQ_FORMATS_H
