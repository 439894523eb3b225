// One-token decode of the gated delta rule (yfxerp page, section 1.2: decode
// takes a single-step fused recurrence), for N independent sequences.
//
// Per (sequence n, value head h) the state S (d_v x d_k fp32, row = one value
// channel, d_k contiguous) is streamed through registers exactly once:
//
//   u = S k^, w = S q^              (row reductions over d_k)
//   delta = beta (v - alpha u)
//   S'   = alpha S + delta k^T       (written back in place)
//   o    = scale (alpha w + delta (k^ . q^))
//
// which is S_t = alpha S (I - beta k k^T) + beta v k^T, o = S_t q multiplied
// out.  The whole update is HBM-bound (0.875 FLOP per state byte), so the
// kernel is organised for streaming: one workgroup per state, every lane
// issues all of its 16-byte state loads before reducing, rows are read as
// contiguous 512-byte runs by 32 lanes, and the state is written back from the
// same registers.
#include "../common.h"
#include "../internal.h"

namespace gdr {

template <int D, typename TQ, typename TO>
__global__ __launch_bounds__(256) void decode_kernel(const TQ* __restrict__ q, const TQ* __restrict__ k,
                                                     const TQ* __restrict__ v, const float* __restrict__ g,
                                                     const float* __restrict__ beta, float* __restrict__ state,
                                                     TO* __restrict__ o, int Hk, int Hv, int use_l2,
                                                     float scale, float eps) {
  constexpr int LPR = D / 4;         // lanes per state row (4 floats each)
  constexpr int RPS = 64 / LPR;      // rows per wave per step
  constexpr int NS = (D / 4) / RPS;  // steps per wave (each wave owns D/4 rows)
  const int nh = blockIdx.x;
  const int n = nh / Hv, h = nh - n * Hv;
  const int kh = h / (Hv / Hk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, c4 = lane % LPR;

  float* S = state + (size_t)nh * D * D;
  const int row0 = wave * (D / 4) + sub;

  // Issue every state load first: 16 x 16 B per lane in flight for D = 128.
  f32x4 s[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    s[i] = *reinterpret_cast<const f32x4*>(S + (size_t)(row0 + i * RPS) * D + 4 * c4);

  float kv[4], qv[4];
  const TQ* kp = k + ((size_t)n * Hk + kh) * D + 4 * c4;
  const TQ* qp = q + ((size_t)n * Hk + kh) * D + 4 * c4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kv[j] = load_as_f32(kp + j);
    qv[j] = load_as_f32(qp + j);
  }
  float kk = 0.f, qq = 0.f, kq = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kk += kv[j] * kv[j];
    qq += qv[j] * qv[j];
    kq += kv[j] * qv[j];
  }
  kk = group_sum<LPR>(kk);
  qq = group_sum<LPR>(qq);
  kq = group_sum<LPR>(kq);
  float rk = 1.f, rq = 1.f;
  if (use_l2) {
    rk = 1.f / sqrtf(kk + eps);
    rq = 1.f / sqrtf(qq + eps);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kv[j] *= rk;
    qv[j] *= rq;
  }
  kq *= rk * rq;

  const float alpha = expf(g[nh]);
  const float b = beta[nh];
  const TQ* vp = v + (size_t)nh * D;
  TO* op = o + (size_t)nh * D;

#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = row0 + i * RPS;
    float pu = s[i].x * kv[0] + s[i].y * kv[1] + s[i].z * kv[2] + s[i].w * kv[3];
    float pw = s[i].x * qv[0] + s[i].y * qv[1] + s[i].z * qv[2] + s[i].w * qv[3];
    pu = group_sum<LPR>(pu);
    pw = group_sum<LPR>(pw);
    const float delta = b * (load_as_f32(vp + r) - alpha * pu);
    if (c4 == 0) store_from_f32(op + r, scale * (alpha * pw + delta * kq));
    f32x4 ns;
    ns.x = alpha * s[i].x + delta * kv[0];
    ns.y = alpha * s[i].y + delta * kv[1];
    ns.z = alpha * s[i].z + delta * kv[2];
    ns.w = alpha * s[i].w + delta * kv[3];
    *reinterpret_cast<f32x4*>(S + (size_t)r * D + 4 * c4) = ns;
  }
}

template <int D, typename TQ, typename TO>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, TQ, TO>), dim3(a.N * a.Hv), dim3(256), 0, st,
                     static_cast<const TQ*>(a.q), static_cast<const TQ*>(a.k), static_cast<const TQ*>(a.v),
                     a.g, a.beta, a.state, static_cast<TO*>(a.o), a.Hk, a.Hv, a.use_l2, a.scale, a.eps);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  if (a.qkv_bf16) {
    return a.out_bf16 ? launch_decode_t<D, uint16_t, uint16_t>(a, st) : launch_decode_t<D, uint16_t, float>(a, st);
  }
  return a.out_bf16 ? launch_decode_t<D, float, uint16_t>(a, st) : launch_decode_t<D, float, float>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.D) {
    case 32: return launch_decode_d<32>(a, st);
    case 64: return launch_decode_d<64>(a, st);
    case 128: return launch_decode_d<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdr
