// Back of the delta-rule layer: gated RMS norm per (token, value head) over
// d_v, y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z) (deepmagic page,
// architecture section: a gated RMS norm after the recurrence; yfxerp page,
// parameter ledger: the gate z is Hv * d_v = 6144 wide).
//
// HBM-bound streaming kernel: d_v/4 lanes per row, 16-byte o loads, one
// reduction per row, bf16 output; four rows per thread in flight.
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

// Each thread takes kNormUnroll rows per pass and issues all their loads
// before the first reduction, so several rows of o and z are in flight.  o, z
// and y are touched once and are far larger than the last-level cache: they
// stream past it (non-temporal), which measured 8% faster.
constexpr int kNormUnroll = 4;

__device__ __forceinline__ void load4_nt(const float* p, float* o) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  for (int j = 0; j < 4; ++j) o[j] = t[j];
}
__device__ __forceinline__ void load4_nt(const uint16_t* p, float* o) {
  const u16x4 t = __builtin_nontemporal_load(reinterpret_cast<const u16x4*>(p));
  for (int j = 0; j < 4; ++j) o[j] = bf16_to_f32(t[j]);
}

template <int D, typename TO>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const TO* __restrict__ o,
                                                            const uint16_t* __restrict__ z,
                                                            const float* __restrict__ w,
                                                            uint16_t* __restrict__ y, int rows, float eps) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;  // rows per workgroup per unrolled step
  const int sub = threadIdx.x / LPR, c4 = threadIdx.x % LPR;
  float wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wv[j] = w[4 * c4 + j];
  for (int base = blockIdx.x * RPB * kNormUnroll; base < rows; base += gridDim.x * RPB * kNormUnroll) {
    float ov[kNormUnroll][4], zv[kNormUnroll][4];
#pragma unroll
    for (int u = 0; u < kNormUnroll; ++u) {
      const int row = base + u * RPB + sub;
      if (row < rows) {
        const TO* op = o + (size_t)row * D + 4 * c4;
        load4_nt(op, ov[u]);
        const u16x4 zr = __builtin_nontemporal_load(reinterpret_cast<const u16x4*>(z + (size_t)row * D + 4 * c4));
#pragma unroll
        for (int j = 0; j < 4; ++j) zv[u][j] = bf16_to_f32(zr[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[u][j] = zv[u][j] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kNormUnroll; ++u) {
      const int row = base + u * RPB + sub;
      float ss = ov[u][0] * ov[u][0] + ov[u][1] * ov[u][1] + ov[u][2] * ov[u][2] + ov[u][3] * ov[u][3];
      ss = group_sum<LPR>(ss);
      const float rstd = 1.f / sqrtf(ss / D + eps);
      float yv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // z sigmoid(z) with the hardware exp2 and reciprocal (about 1e-7
        // relative, far inside a bf16 ulp): z = -inf gives NaN, z = +inf
        // gives +inf, as z / (1 + e^-z) does.
        const float e = __builtin_amdgcn_exp2f(zv[u][j] * -1.44269504f);
        const float gate = zv[u][j] * __builtin_amdgcn_rcpf(1.f + e);
        yv[j] = ov[u][j] * rstd * wv[j] * gate;
      }
      if (row < rows)
        __builtin_nontemporal_store(u32x2{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])},
                                    reinterpret_cast<u32x2*>(y + (size_t)row * D + 4 * c4));
    }
  }
}

template <int D>
hipError_t launch_norm_d(const NormArgs& a, hipStream_t st) {
  const int rows = a.T * a.H;
  constexpr int RPB = 256 / (D / 4);
  int blocks = (rows + RPB * kNormUnroll - 1) / (RPB * kNormUnroll);
  if (blocks > 8192) blocks = 8192;
  if (a.o_bf16)
    hipLaunchKernelGGL((gated_rmsnorm_kernel<D, uint16_t>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.z), a.w,
                       static_cast<uint16_t*>(a.y), rows, a.eps);
  else
    hipLaunchKernelGGL((gated_rmsnorm_kernel<D, float>), dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(a.o), static_cast<const uint16_t*>(a.z), a.w,
                       static_cast<uint16_t*>(a.y), rows, a.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  switch (a.D) {
    case 32: return launch_norm_d<32>(a, st);
    case 64: return launch_norm_d<64>(a, st);
    case 128: return launch_norm_d<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdr
