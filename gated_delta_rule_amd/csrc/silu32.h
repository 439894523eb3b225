// The conv front's exact fp32 SiLU and the layer's gates, shared by every
// kernel that evaluates them so that they give the same bits everywhere
// (deepmagic page, architecture section: kernel-4 causal conv + SiLU in front
// of the recurrence; yfxerp page, section 1.2: beta = sigmoid(b),
// g = -exp(A_log) * softplus(a + dt_bias) in fp32).
//
// SiLU contract: y = v / (1 + exp32(-v)), where exp32 is Cody and Waite's
// reduction x = n ln2 + r with ln2 = C1 + C2, then the degree-7 Taylor
// polynomial of exp(r) in Horner form and a scale by 2^n, every step one IEEE
// fp32 operation (FMA contraction off inside these functions).
#pragma once

#include <hip/hip_runtime.h>

namespace gdr {

// Cody-Waite reduction and the Taylor polynomial scaled by 2^n, with no
// special cases (exp32 for x in [kExpLo, kExpHi]).
__device__ __forceinline__ float exp_poly(float x) {
#pragma clang fp contract(off)
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  const float r = (x - n * 0x1.630000p-1f) - n * -0x1.bd0106p-13f;
  float p = 0x1.a01a02p-13f;
  p = p * r + 0x1.6c16c2p-10f;
  p = p * r + 0x1.111112p-7f;
  p = p * r + 0x1.555556p-5f;
  p = p * r + 0x1.555556p-3f;
  p = p * r + 0x1.0p-1f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return __builtin_ldexpf(p, static_cast<int>(n));
}

// exp32 is +inf above kExpHi = 0x1.62e430p+6 (about 88.72) and 0 below kExpLo.
constexpr float kExpLo = -0x1.9fe368p+6f;

// SiLU by the contract for every v.  exp32(-v) is taken as exp_poly on -v
// clamped into [kExpLo, 128], which gives the same quotient: above kExpHi the
// scale by 2^n overflows to +inf for every x up to 128, as exp32 does; below
// kExpLo the clamped value is at most 2^-149, so 1 + e rounds to 1, as it does
// for exp32's 0; a NaN v stays NaN through the division.
__device__ __forceinline__ float silu32(float v) {
#pragma clang fp contract(off)
  return v / (1.0f + exp_poly(fminf(fmaxf(-v, kExpLo), 128.f)));
}

// SiLU for |v| <= 80, where no clamp is needed and the IEEE division can be
// replaced by one residual correction of v * rcp(d): q0 = v y0, r = d q0 - v
// (exact by the fused multiply-add), q = q0 - r y0.  The residual is taken
// as d q0 - v rather than v - d q0 so that v = -0 keeps its sign.  Checked
// equal, bit for bit, to silu32 for every fp32 v in [-80, 80].
__device__ __forceinline__ float silu32_mid(float v) {
#pragma clang fp contract(off)
  const float d = 1.0f + exp_poly(-v);
  const float y0 = __builtin_amdgcn_rcpf(d);
  const float q0 = v * y0;
  const float rn = __builtin_fmaf(d, q0, -v);
  return __builtin_fmaf(-rn, y0, q0);
}

// The conv taps in the contract's order, ((p0 + p1) + p2) + p3 with
// p_j = w_j x_j (oldest first; exact in fp32 for bf16 operands).
__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float x0, float x1, float x2,
                                       float x3) {
#pragma clang fp contract(off)
  return ((w0 * x0 + w1 * x1) + w2 * x2) + w3 * x3;
}

// beta = 1 / (1 + e^-b), g = -e^{A_log} softplus(a + dt_bias) with
// softplus(x) = max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ void gates(float a, float b, float A_log, float dt_bias, float& g, float& beta) {
#pragma clang fp contract(off)
  const float x = a + dt_bias;
  const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
  g = -expf(A_log) * sp;
  beta = 1.f / (1.f + expf(-b));
}

}  // namespace gdr
