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

}  // namespace akv
