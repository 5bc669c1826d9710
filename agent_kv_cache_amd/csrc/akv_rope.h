// bf16 helpers and the fp64 rotation of NeoX pairs shared by the move kernel
// (re-rotation by R(q - p), [CE] sec. 3.3 eq. 5) and the RoPE-fused append
// (rotation by R(p) of a new key, eq. 3).
#pragma once

#include "akv_internal.h"

namespace akv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r.x = (__bf16)a;
  r.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// fp64 -> fp32 such that a following fp32 -> bf16 round-to-nearest-even gives
// the correctly rounded bf16 of x (one rounding).  A double rounding error can
// only occur when the fp32 value sits exactly on a bf16 halfway point
// (low 16 bits 0x8000) while x is not that value; then the fp32 value is
// nudged one fp32 step towards x, which breaks the tie the right way.
__device__ __forceinline__ float f64_to_f32_for_bf16(double x) {
  float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if (__builtin_expect((u & 0xFFFFu) == 0x8000u, 0)) {
    double back = (double)f;
    if (back != x) u += (fabs(x) > fabs(back)) ? 1u : 0xFFFFFFFFu;
  }
  return __uint_as_float(u);
}

// Rotate 8 NeoX pairs: lo holds x_i (8 bf16), hi holds y_i = k[i + d/2].
// x' = x cos - y sin, y' = y cos + x sin in fp64, one rounding to bf16.
__device__ __forceinline__ void rotate8(u32x4 &lo, u32x4 &hi, const double2 *cs) {
  uint32_t a[4] = {lo.x, lo.y, lo.z, lo.w};
  uint32_t bb[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float xo[2], yo[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const double x = (double)bf16_to_f32((a[q] >> (16 * e)) & 0xFFFFu);
      const double y = (double)bf16_to_f32((bb[q] >> (16 * e)) & 0xFFFFu);
      const double2 v = cs[2 * q + e];
      const double cc = v.x, ss = v.y;
      xo[e] = f64_to_f32_for_bf16(fma(x, cc, -(y * ss)));
      yo[e] = f64_to_f32_for_bf16(fma(y, cc, x * ss));
    }
    a[q] = f32x2_to_bf16x2(xo[0], xo[1]);
    bb[q] = f32x2_to_bf16x2(yo[0], yo[1]);
  }
  lo = u32x4{a[0], a[1], a[2], a[3]};
  hi = u32x4{bb[0], bb[1], bb[2], bb[3]};
}


// One side of 8 NeoX pairs: `own` holds 8 values of one side (x_i when is_x,
// else y_i = k[i + d/2]) and `other` the partner side.  x' = x cos - y sin,
// y' = y cos + x sin: the same fp64 operations and single rounding as
// rotate8, so both mappings give identical bits.
__device__ __forceinline__ u32x4 rotate8_side(u32x4 own, u32x4 other, bool is_x,
                                              const double2 *cs) {
  const uint32_t a[4] = {own.x, own.y, own.z, own.w};
  const uint32_t bb[4] = {other.x, other.y, other.z, other.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const double x = (double)bf16_to_f32((a[q] >> (16 * e)) & 0xFFFFu);
      const double y = (double)bf16_to_f32((bb[q] >> (16 * e)) & 0xFFFFu);
      const double2 v = cs[2 * q + e];
      const double p = y * v.y;
      r[e] = f64_to_f32_for_bf16(fma(x, v.x, is_x ? -p : p));
    }
    o[q] = f32x2_to_bf16x2(r[0], r[1]);
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// sin and cos of x = delta * theta_i in fp64, for |x| < 2^31 (|delta| < 2^31,
// 0 <= theta_i <= 1).  Cody-Waite reduction by pi/2, with pi/2 split into
// three 22-bit parts and a double tail so that k * part is exact for
// |k| < 2^31, then the Taylor series of sin and cos on [-pi/4, pi/4] (terms
// through r^19 and r^20; the first omitted term is below 1e-21) in Horner
// form.  Short and free of table loads: the move computes it per page.
__host__ __device__ inline void sincos_rope(double x, double *sn, double *cs) {
  const double kTwoOverPi = 0x1.45f306dc9c883p-1;
  const double kP1 = 0x1.921fb8p+0, kP2 = -0x1.5dde98p-23, kP3 = 0x1.846988p-48,
               kP4 = 0x1.8cc51701b839ap-72;
  const double k = rint(x * kTwoOverPi);
  double r = fma(-k, kP1, x);
  r = fma(-k, kP2, r);
  r = fma(-k, kP3, r);
  r = fma(-k, kP4, r);
  const double z = r * r;
  // 1/n! for odd n = 3..19 (sin) and even n = 2..20 (cos)
  double ps = -0x1.2f49b46814157p-57;              // -1/19!
  ps = fma(ps, z, 0x1.952c77030ad4ap-49);          //  1/17!
  ps = fma(ps, z, -0x1.ae7f3e733b81fp-41);         // -1/15!
  ps = fma(ps, z, 0x1.6124613a86d09p-33);          //  1/13!
  ps = fma(ps, z, -0x1.ae64567f544e4p-26);         // -1/11!
  ps = fma(ps, z, 0x1.71de3a556c734p-19);          //  1/9!
  ps = fma(ps, z, -0x1.a01a01a01a01ap-13);         // -1/7!
  ps = fma(ps, z, 0x1.1111111111111p-7);           //  1/5!
  ps = fma(ps, z, -0x1.5555555555555p-3);          // -1/3!
  const double s = fma(ps * z, r, r);
  double pc = 0x1.e542ba4020225p-62;               //  1/20!
  pc = fma(pc, z, -0x1.6827863b97d97p-53);         // -1/18!
  pc = fma(pc, z, 0x1.ae7f3e733b81fp-45);          //  1/16!
  pc = fma(pc, z, -0x1.93974a8c07c9dp-37);         // -1/14!
  pc = fma(pc, z, 0x1.1eed8eff8d898p-29);          //  1/12!
  pc = fma(pc, z, -0x1.27e4fb7789f5cp-22);         // -1/10!
  pc = fma(pc, z, 0x1.a01a01a01a01ap-16);          //  1/8!
  pc = fma(pc, z, -0x1.6c16c16c16c17p-10);         // -1/6!
  pc = fma(pc, z, 0x1.5555555555555p-5);           //  1/4!
  pc = fma(pc, z, -0x1.0p-1);                      // -1/2!
  const double c = fma(pc, z, 1.0);
  const int q = (int)((long long)k & 3);
  *sn = (q == 0) ? s : (q == 1) ? c : (q == 2) ? -s : -c;
  *cs = (q == 0) ? c : (q == 1) ? -s : (q == 2) ? -c : s;
}

}  // namespace akv
