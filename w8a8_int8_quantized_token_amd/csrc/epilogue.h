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
// so erfc's relative error is below 8e-6).  Evaluated as
//   h = erfc(z)/2 = t * 2^(-log2(e) v^2/2 + Q(t)),  Q = log2(e) P - 1,
// (z = |v|/sqrt2 folded into the constants, the exponential taken base 2 by
// the hardware's v_exp_f32, the halving folded into Q's constant term), and
//   gelu(v) = max(v, 0) - |v h|,
// which is v - v h for v >= 0 and v h below.  With the exponent's rounding
// (about v^2 2^-25) and the 1-ulp hardware reciprocal and exp2 the relative
// error stays near 1e-5 -- far below the bf16 rounding of the stored result.
// Branch-free: one reciprocal, one exp2, fourteen other operations.
__device__ __forceinline__ float gelu(float v) {
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(v), 0.35355339059327373f, 1.0f));   // v_rcp_f32 (1 ulp)
  float q = 0.33010232f;
  q = fmaf(q, t, -1.0232229f);
  q = fmaf(q, t, 0.6846277f);
  q = fmaf(q, t, 0.3670476f);
  q = fmaf(q, t, 1.4686903f);
  q = fmaf(q, t, -2.827234f);
  const float h = t * __builtin_amdgcn_exp2f(fmaf(v * -0.72134752044448170f, v, q));   // v_exp_f32
  return fmaxf(v, 0.0f) - fabsf(v * h);
}

}  // namespace w8a8
