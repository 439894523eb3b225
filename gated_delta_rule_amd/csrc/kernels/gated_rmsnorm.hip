// Back of the delta-rule layer: gated RMS norm per (token, value head) over
// d_v, y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z) (deepmagic page,
// architecture section: a gated RMS norm after the recurrence; yfxerp page,
// parameter ledger: the gate z is Hv * d_v = 6144 wide).
//
// HBM-bound streaming kernel: d_v/4 lanes per row, 16-byte o loads, one
// reduction per row, bf16 output.
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

template <int D, typename TO>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const TO* __restrict__ o,
                                                            const uint16_t* __restrict__ z,
                                                            const float* __restrict__ w,
                                                            uint16_t* __restrict__ y, int rows, float eps) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;  // rows per workgroup per iteration
  const int sub = threadIdx.x / LPR, c4 = threadIdx.x % LPR;
  float wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wv[j] = w[4 * c4 + j];
  for (int row = blockIdx.x * RPB + sub; row < rows; row += gridDim.x * RPB) {
    float ov[4], zv[4];
    const TO* op = o + (size_t)row * D + 4 * c4;
#pragma unroll
    for (int j = 0; j < 4; ++j) ov[j] = load_as_f32(op + j);
    const u16x4 zr = *reinterpret_cast<const u16x4*>(z + (size_t)row * D + 4 * c4);
#pragma unroll
    for (int j = 0; j < 4; ++j) zv[j] = bf16_to_f32(zr[j]);
    float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
    ss = group_sum<LPR>(ss);
    const float rstd = 1.f / sqrtf(ss / D + eps);
    u16x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float gate = zv[j] / (1.f + expf(-zv[j]));
      out[j] = f32_to_bf16(ov[j] * rstd * wv[j] * gate);
    }
    *reinterpret_cast<u16x4*>(y + (size_t)row * D + 4 * c4) = out;
  }
}

template <int D>
hipError_t launch_norm_d(const NormArgs& a, hipStream_t st) {
  const int rows = a.T * a.H;
  constexpr int RPB = 256 / (D / 4);
  int blocks = (rows + RPB - 1) / RPB;
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
