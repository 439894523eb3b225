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
// kernel is organised for streaming: one or two workgroups per state, every
// lane issues all of its 16-byte state loads before reducing, and the state
// is written back from the same registers.  State loads and stores are
// non-temporal: a pool of states is read once and written once per token and
// in a real model (dozens of layers) never fits the 256 MB last-level cache,
// so they stream past it; measured, this gives the same rate whether or not
// the state would have fit there.  Eight lanes share a state row: lane
// e (0..7) holds columns 32 j + 4 e .. +3 for j < D/32, so every load
// instruction reads 128 contiguous bytes of each of its 8 rows, and a row's
// dot products finish with three cross-lane adds inside the 8-lane group
// (data-parallel-primitive moves, no LDS traffic).
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

// Workgroups per state: at d = 128 two, each streaming 64 of the 128 rows,
// so that a lane holds 32 state registers and more workgroups share a
// compute unit (every state row is independent given k, q, v and the gates).
template <int D>
constexpr int kDecodeSplit = D == 128 ? 2 : 1;

}  // namespace

template <int D, typename TQ, typename TO>
__global__ __launch_bounds__(256) void decode_kernel(const TQ* __restrict__ q, const TQ* __restrict__ k,
                                                     const TQ* __restrict__ v, const float* __restrict__ g,
                                                     const float* __restrict__ beta, float* __restrict__ state,
                                                     const int32_t* __restrict__ state_indices, int pool_size,
                                                     TO* __restrict__ o, int Hk, int Hv, int use_l2,
                                                     float scale, float eps) {
  constexpr int F4 = D / 32;                 // 16-byte pieces per lane per row
  constexpr int SPLIT = kDecodeSplit<D>;     // workgroups per state
  constexpr int NS = D / (32 * SPLIT);       // row steps per wave, 8 rows each
  const int nh = blockIdx.x / SPLIT, part = blockIdx.x % SPLIT;
  const int n = nh / Hv, h = nh - n * Hv;
  const int kh = h / (Hv / Hk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> 3, e8 = lane & 7;

  const int row0 = part * (D / SPLIT) + wave * (D / (4 * SPLIT)) + sub;
  // State slot of sequence n: n itself, or its pool index.  A padding row
  // (index outside [0, pool_size)) writes zeros for its outputs and touches
  // no state.
  const int slot = state_indices ? state_indices[n] : n;
  if (state_indices && (slot < 0 || slot >= pool_size)) {
    TO* op = o + (size_t)nh * D;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (e8 == 0) store_from_f32(op + row0 + 8 * i, 0.f);
    return;
  }
  float* S = state + ((size_t)slot * Hv + h) * D * D;

  // Issue every state load first: NS * F4 x 16 B per lane in flight.
  f32x4 s[NS][F4];
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int j = 0; j < F4; ++j)
      s[i][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(row0 + 8 * i) * D + 32 * j + 4 * e8));

  float kv[F4][4], qv[F4][4];
  const TQ* kp = k + ((size_t)n * Hk + kh) * D + 4 * e8;
  const TQ* qp = q + ((size_t)n * Hk + kh) * D + 4 * e8;
#pragma unroll
  for (int j = 0; j < F4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[j][e] = load_as_f32(kp + 32 * j + e);
      qv[j][e] = load_as_f32(qp + 32 * j + e);
    }
  // Every multiply-add below is an explicit fma, so that the fused
  // decode-layer kernel, which spells out the same operations, gives the same
  // bits whatever the compiler would contract on its own.
  float kk = 0.f, qq = 0.f, kq = 0.f;
#pragma unroll
  for (int j = 0; j < F4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kk = __builtin_fmaf(kv[j][e], kv[j][e], kk);
      qq = __builtin_fmaf(qv[j][e], qv[j][e], qq);
      kq = __builtin_fmaf(kv[j][e], qv[j][e], kq);
    }
  kk = sum8(kk);
  qq = sum8(qq);
  kq = sum8(kq);
  float rk = 1.f, rq = 1.f;
  if (use_l2) {
    rk = 1.f / sqrtf(kk + eps);
    rq = 1.f / sqrtf(qq + eps);
  }
#pragma unroll
  for (int j = 0; j < F4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[j][e] *= rk;
      qv[j][e] *= rq;
    }
  kq *= rk * rq;

  const float alpha = expf(g[nh]);
  const float b = beta[nh];
  const TQ* vp = v + (size_t)nh * D;
  TO* op = o + (size_t)nh * D;

#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = row0 + 8 * i;
    float pu = 0.f, pw = 0.f;
#pragma unroll
    for (int j = 0; j < F4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pu = __builtin_fmaf(s[i][j][e], kv[j][e], pu);
        pw = __builtin_fmaf(s[i][j][e], qv[j][e], pw);
      }
    pu = sum8(pu);
    pw = sum8(pw);
    const float delta = b * __builtin_fmaf(-alpha, pu, load_as_f32(vp + r));
    if (e8 == 0) store_from_f32(op + r, scale * __builtin_fmaf(delta, kq, alpha * pw));
#pragma unroll
    for (int j = 0; j < F4; ++j) {
      f32x4 ns;
#pragma unroll
      for (int e = 0; e < 4; ++e) ns[e] = __builtin_fmaf(delta, kv[j][e], alpha * s[i][j][e]);
      __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + (size_t)r * D + 32 * j + 4 * e8));
    }
  }
}

template <int D, typename TQ, typename TO>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<D, TQ, TO>), dim3(a.N * a.Hv * kDecodeSplit<D>), dim3(256), 0, st,
                     static_cast<const TQ*>(a.q), static_cast<const TQ*>(a.k), static_cast<const TQ*>(a.v),
                     a.g, a.beta, a.state, a.state_indices, a.pool_size, static_cast<TO*>(a.o), a.Hk, a.Hv,
                     a.use_l2, a.scale, a.eps);
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
