// Per-element arithmetic of the bf16 epilogues, shared by the fused GEMM's
// epilogue and the K-split reduction so that both produce the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace w8a8 {

// y = fl32(fl32(fl32(acc) * sa) * sw) + b), each step rounded on its own
// (the int32 accumulator is converted to fp32 with round to nearest even).
__device__ __forceinline__ float dequant(float acc, float sa, float sw, float b) {
  return __fadd_rn(__fmul_rn(__fmul_rn(acc, sa), sw), b);
}

// GELU with the exact (erf) definition, gelu(v) = v * Phi(v), where the
// normal CDF is Phi(v) = 1 - erfc(v/sqrt2)/2 for v >= 0 and erfc(|v|/sqrt2)/2
// below.  erfc(z), z >= 0, takes the form of the "erfcc" routine of Numerical
// Recipes (2nd ed., section 6.2): t = 1/(1 + z/2), erfc = t * exp(-z^2 + P(t)),
// with our own degree-5 P (gelu_fit.py beside this file: a near-minimax fit of
// ln(erfc(z)/t) + z^2 on z in [0, 10]; |P - that| < 7.9e-6 evaluated in fp32,
// so erfc's relative error is below 8e-6).  With the exp argument's rounding
// (about z^2 * 2^-24) and the hardware reciprocal's 1-ulp error the GELU's
// relative error stays near 1e-5 -- far below the bf16 rounding of the stored
// result.  Branch-free: one reciprocal, one exp.
__device__ __forceinline__ float gelu(float v) {
  const float z = fabsf(v) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));   // v_rcp_f32 (1 ulp)
  float p = 0.22880949f;
  p = fmaf(p, t, -0.7092441f);
  p = fmaf(p, t, 0.47454774f);
  p = fmaf(p, t, 0.25441802f);
  p = fmaf(p, t, 1.0180185f);
  p = fmaf(p, t, -1.2665421f);
  const float half_erfc = 0.5f * t * __expf(fmaf(-z, z, p));
  return v * (v >= 0.0f ? 1.0f - half_erfc : half_erfc);
}

}  // namespace w8a8
