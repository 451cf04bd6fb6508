// Activation quantisation rule shared by the quantise kernel and the GEMM
// epilogue that quantises h: s = f32(amax / 448) with a correctly rounded FP32
// division; code = E4M3 round-to-nearest-even of f32(v / s), saturated at
// +-448, sign bit kept (Transformers PR #47844, implementation list: E4M3 with
// dynamically quantised activations).
#pragma once

#include "dmoe_device.h"

namespace dmoe {

__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }

// Division by a slice scale for the E4M3 decision, cheaper than one correctly
// rounded division per element. Both operands are first scaled by the same
// power of two so that the divisor lies in [1, 2); with the correctly rounded
// reciprocal r of the divisor, q = v' r corrected once by the exact residual
// v' - q s' (a fused multiply-add) is the quotient, and the sign of zero is
// restored. This is the FMA correction step of Markstein's division
// (P. Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", IBM J. Res. Develop. 34(1), 1990): with r the
// correctly rounded reciprocal, one step q + (v' - q s') r yields the
// correctly rounded quotient except in rare cases that need a second step.
// The code chosen from it equals the code of the correctly rounded
// f32(v / s) for every BF16 v and every scale s = f32(amax / 448) with
// |v| <= amax (checked exhaustively on gfx950 for all BF16 amax); quotients
// that differ in the last f32 bit are far below the smallest E4M3 subnormal.
struct ScaleDiv {
  float sn, r;
  int k;
};
__device__ __forceinline__ ScaleDiv make_scale_div(float s) {
  ScaleDiv d;
  int e;
  (void)frexpf(s, &e);  // s = m * 2^e, m in [0.5, 1)
  d.k = 1 - e;
  d.sn = ldexpf(s, d.k);
  d.r = __fdiv_rn(1.0f, d.sn);
  return d;
}
__device__ __forceinline__ float scale_div(const ScaleDiv& d, float v) {
  const float vn = ldexpf(v, d.k);
  const float q0 = vn * d.r;
  const float res = fmaf(-q0, d.sn, vn);
  return copysignf(fmaf(res, d.r, q0), v);
}

// Four |q| < 464 values to E4M3 codes (byte i = code of q[i]) with the hardware
// conversion, which rounds to nearest even exactly like e4m3_encode on that
// range (checked on gfx950 for every binary32 pattern with |q| < 464).
__device__ __forceinline__ uint32_t e4m3x4_hw(float q0, float q1, float q2, float q3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return (uint32_t)w;
}

}  // namespace dmoe
