// Division of many values by one per-row divisor, correctly rounded.
//
// The output step of the Falcon-Edge blog's BitLinear.post_quant_process
// divides every accumulator of a token row by the same fp32 value
// d = x_scale * w_scale.  A correctly rounded fp32 division is about a dozen
// instructions; with the reciprocal y = RN(1/d) computed once per row, one
// multiply and two fused multiply-adds give the same correctly rounded
// quotient (Markstein's correction step):
//     q0 = RN(a * y),  r = a - q0 * d (exact, one FMA),  q = RN(q0 + r * y).
// The identity needs no underflow or overflow in these steps; rows whose
// divisor is outside [2^-100, 2^100] (never the case for activation scales
// of finite bf16 rows and weight scales of finite weights in practice) use
// the plain division.  Plain C++ so host-side checks run the same code.
#pragma once

#include <math.h>

#if defined(__HIPCC__)
#define BL_RD_HD __host__ __device__
#else
#define BL_RD_HD
#endif

namespace bl {

struct RowDiv {
  float d;     // divisor
  float y;     // RN(1 / d)
  int fast;    // d in [2^-100, 2^100]
};

BL_RD_HD inline RowDiv row_div_setup(float d) {
  RowDiv r;
  r.d = d;
  r.y = 1.0f / d;
  r.fast = (d >= 7.888609052210118e-31f && d <= 1.2676506002282294e30f) ? 1 : 0;
  return r;
}

// a / d for d in the fast range: one multiply, two fused multiply-adds.
BL_RD_HD inline float row_div_fast(float a, float d, float y) {
  const float q0 = a * y;
  const float rem = fmaf(-q0, d, a);
  return fmaf(rem, y, q0);
}

BL_RD_HD inline float row_div(float a, const RowDiv& r) {
  if (!r.fast) return a / r.d;
  return row_div_fast(a, r.d, r.y);
}

}  // namespace bl
