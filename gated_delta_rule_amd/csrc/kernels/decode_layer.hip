// One decode token of the whole delta-rule layer path in one launch: the
// conv front for the token (kernel-4 causal conv + SiLU against a rolling
// conv state), the gates, the recurrent state update and the gated RMS norm
// (deepmagic page, architecture section: conv in front, gated RMS norm
// behind; yfxerp page, section 1.2: the decode path takes a single-step
// recurrence and carries the conv state alongside the recurrent state).
//
// One workgroup per (sequence n, key head kh), 256 threads per value head of
// that key head (G = Hv/Hk of them).  The workgroup owns every channel it
// reads -- the key head's q and k channels and its value heads' v channels --
// so it updates their conv state in place without racing another workgroup.
//
//   phase 0  each thread loads its conv channel's inputs and (threads
//            0 .. G-1) the gate inputs, then every lane issues the state
//            loads of its first two row steps (non-temporal): waves
//            4g .. 4g+3 stream value head kh*G + g, 32 rows each, 8 lanes
//            per row
//   phase 1  conv + SiLU of the (2 + G) * 128 channels under the front's
//            bit-exact contract (same code as the prefill front), the
//            conv state rolled by one token, the gates; results to LDS
//   phase 2  the state update and o, with the decode kernel's arithmetic,
//            fma for fma, and reduction order (so o and S match
//            gdr_recurrent_step bit for bit),
//            in two passes of two row steps: as the first pass writes a row
//            back, the registers it held load the matching second-pass row,
//            so those loads stream under the first pass's arithmetic and
//            stores
//   phase 3  the gated RMS norm of each value head's 128 outputs
//
// Bound by the state traffic like the decode step; the front and back add
// (2 + G) * 128 * 8 + G * 128 * 4 bytes per workgroup to its 3 x 64 KiB.
#include "../common.h"
#include "../internal.h"
#include "../silu32.h"

namespace gdr {

namespace {

constexpr int kLD = 128;  // head dim of this kernel

// Workgroup barrier for LDS traffic only (the state loads stay in flight).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int G>
__global__ __launch_bounds__(256 * G) void decode_layer_kernel(LayerStepArgs a) {
  constexpr int D = kLD, F4 = D / 32, NS = D / 32;
  const int n = blockIdx.x / a.Hk, kh = blockIdx.x % a.Hk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gh = wv >> 2, wh = wv & 3;  // value head within the group, wave within the head
  const int h = kh * G + gh;
  const int sub = lane >> 3, e8 = lane & 7;
  const int C = (2 * a.Hk + a.Hv) * D;
  const int HvD = a.Hv * D;

  __shared__ float xs[(2 + G) * D];  // q | k | v of the group's value heads (bf16 values)
  __shared__ float gl[G], bl[G];
  __shared__ float os[G][D];
  __shared__ float rs[G];

  // channel index of the group's local channel cl: q, then k, then the v
  // channels of value heads kh*G .. kh*G+G-1 (contiguous)
  auto channel = [&](int cl) {
    return cl < D ? kh * D + cl : cl < 2 * D ? a.Hk * D + kh * D + (cl - D) : 2 * a.Hk * D + kh * G * D + (cl - 2 * D);
  };

  const int slot = a.state_indices ? a.state_indices[n] : n;
  if (a.state_indices && (slot < 0 || slot >= a.pool_size)) {
    // padding row: zeros out, no state read or written
    uint16_t* y = static_cast<uint16_t*>(a.y) + (size_t)n * HvD + kh * G * D;
    for (int t = tid; t < G * D; t += 256 * G) {
      y[t] = 0;
      if (a.o) a.o[(size_t)n * HvD + kh * G * D + t] = 0.f;
    }
    if (a.qkv_out)
      for (int cl = tid; cl < (2 + G) * D; cl += 256 * G) static_cast<uint16_t*>(a.qkv_out)[(size_t)n * C + channel(cl)] = 0;
    return;
  }

  // ---- phase 0: this thread's conv channel inputs, then the state loads.
  // Loads complete in issue order, so the small conv loads go first: the
  // conv, its LDS writes and the barrier then run while the state streams in.
  constexpr int NCH = (2 + G) * D, CPT = (NCH + 256 * G - 1) / (256 * G);  // conv channels per thread
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + (size_t)n * C;
  const uint16_t* w = static_cast<const uint16_t*>(a.conv_w);
  uint16_t* cst = static_cast<uint16_t*>(a.conv_state) + (size_t)slot * C * 3;
  uint16_t xr[CPT], h0[CPT], h1[CPT], h2[CPT];
  u16x4 wr[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    // unconditional (clamped) loads: a branch here would let the compiler
    // consume them, and so wait for them, before the state loads issue
    const int c = channel(min(tid + 256 * G * i, NCH - 1));
    const uint16_t* cs = cst + (size_t)c * 3;
    xr[i] = x[c];
    wr[i] = *reinterpret_cast<const u16x4*>(w + (size_t)c * 4);
    h0[i] = cs[0];
    h1[i] = cs[1];
    h2[i] = cs[2];
  }
  const int gh_ld = kh * G + min(tid, G - 1);
  const float ga = a.a[(size_t)n * a.Hv + gh_ld], gb = a.b[(size_t)n * a.Hv + gh_ld];
  const float gA = a.A_log[gh_ld], gdt = a.dt_bias[gh_ld];
  const int row0 = wh * (D / 4) + sub;
  float* S = a.state + ((size_t)slot * a.Hv + h) * D * D;
  constexpr int NH = NS / 2;  // rows per pass
  f32x4 s[NH][F4];
#pragma unroll
  for (int i = 0; i < NH; ++i)
#pragma unroll
    for (int j = 0; j < F4; ++j)
      s[i][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(row0 + 8 * i) * D + 32 * j + 4 * e8));
  __builtin_amdgcn_sched_barrier(0);  // every load above issues before any use

  // ---- phase 1: conv + SiLU, rolling conv state, gates
  {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cl = tid + 256 * G * i;
      if (cl >= NCH) continue;
      const int c = channel(cl);
      const float acc = conv4(bf16_to_f32(wr[i][0]), bf16_to_f32(wr[i][1]), bf16_to_f32(wr[i][2]),
                              bf16_to_f32(wr[i][3]), bf16_to_f32(h0[i]), bf16_to_f32(h1[i]), bf16_to_f32(h2[i]),
                              bf16_to_f32(xr[i]));
      // same bits on either path; the wave takes the short one when it can
      const float yv = __all(fabsf(acc) <= 80.f) ? silu32_mid(acc) : silu32(acc);
      const uint16_t yb = f32_to_bf16(yv);
      xs[cl] = bf16_to_f32(yb);
      if (a.qkv_out) static_cast<uint16_t*>(a.qkv_out)[(size_t)n * C + c] = yb;
      uint16_t* cs = cst + (size_t)c * 3;
      cs[0] = h1[i];
      cs[1] = h2[i];
      cs[2] = xr[i];
    }
    if (tid < G) gates(ga, gb, gA, gdt, gl[tid], bl[tid]);
  }
  lds_sync();

  // ---- phase 2: the state update (the decode kernel's arithmetic)
  float kv[F4][4], qv[F4][4];
#pragma unroll
  for (int j = 0; j < F4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[j][e] = xs[D + 32 * j + 4 * e8 + e];
      qv[j][e] = xs[32 * j + 4 * e8 + e];
    }
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
  if (a.use_l2) {
    rk = 1.f / sqrtf(kk + a.eps);
    rq = 1.f / sqrtf(qq + a.eps);
  }
#pragma unroll
  for (int j = 0; j < F4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[j][e] *= rk;
      qv[j][e] *= rq;
    }
  kq *= rk * rq;
  const float alpha = expf(gl[gh]);
  const float b = bl[gh];
  // two passes of NH row steps; as pass 0 frees a row's registers, the
  // matching pass-1 row is loaded into them
#pragma unroll
  for (int pass = 0; pass < 2; ++pass)
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const int r = row0 + 8 * (i + NH * pass);
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
    const float delta = b * __builtin_fmaf(-alpha, pu, xs[2 * D + gh * D + r]);
    if (e8 == 0) {
      const float ov = a.scale * __builtin_fmaf(delta, kq, alpha * pw);
      os[gh][r] = ov;
      if (a.o) a.o[(size_t)n * HvD + h * D + r] = ov;
    }
#pragma unroll
    for (int j = 0; j < F4; ++j) {
      f32x4 ns;
#pragma unroll
      for (int e = 0; e < 4; ++e) ns[e] = __builtin_fmaf(delta, kv[j][e], alpha * s[i][j][e]);
      __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + (size_t)r * D + 32 * j + 4 * e8));
    }
    if (pass == 0) {
#pragma unroll
      for (int j = 0; j < F4; ++j)
        s[i][j] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(S + (size_t)(r + 8 * NH) * D + 32 * j + 4 * e8));
    }
  }
  lds_sync();

  // ---- phase 3: gated RMS norm of each value head's outputs
  if (wh == 0) {
    const float o0 = os[gh][lane], o1 = os[gh][lane + 64];
    const float ss = group_sum<64>(o0 * o0 + o1 * o1);
    if (lane == 0) rs[gh] = 1.f / sqrtf(ss / D + a.norm_eps);
  }
  lds_sync();
  {
    const uint16_t* z = static_cast<const uint16_t*>(a.z) + (size_t)n * HvD + kh * G * D;
    uint16_t* y = static_cast<uint16_t*>(a.y) + (size_t)n * HvD + kh * G * D;
    for (int t = tid; t < G * D; t += 256 * G) {
      const int g2 = t / D, r = t % D;
      const float zv = bf16_to_f32(z[t]);
      // z sigmoid(z) as in the gated RMS norm kernel (hardware exp2 and reciprocal)
      const float gate = zv * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(zv * -1.44269504f));
      y[t] = f32_to_bf16(os[g2][r] * rs[g2] * a.norm_w[r] * gate);
    }
  }
}

}  // namespace

hipError_t launch_decode_layer(const LayerStepArgs& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const dim3 grid((unsigned)(a.N * a.Hk));
  switch (a.Hv / a.Hk) {
    case 1: hipLaunchKernelGGL(decode_layer_kernel<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_layer_kernel<2>, grid, dim3(512), 0, st, a); break;
    case 3: hipLaunchKernelGGL(decode_layer_kernel<3>, grid, dim3(768), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_layer_kernel<4>, grid, dim3(1024), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdr
