// Front of the delta-rule layer: depthwise causal conv (kernel 4) + SiLU over
// every q|k|v channel, and the gates beta = sigmoid(b),
// g = -exp(A_log) * softplus(a + dt_bias) (deepmagic page, architecture
// section: kernel-4 causal conv in front of the recurrence; yfxerp page,
// section 1.2: the gate formulas, evaluated in fp32).
//
// Bit-exact contract: with p_j = w_j * x_j in fp32 (exact for bf16 operands),
// acc = ((p0 + p1) + p2) + p3, y = acc / (1 + exp32(-acc)), rounded to nearest
// even bf16, where exp32 is Cody and Waite's reduction x = n ln2 + r with
// ln2 = C1 + C2, followed by the degree-7 Taylor polynomial of exp(r) in
// Horner form and a scale by 2^n.  Every step is one IEEE fp32 operation; FMA
// contraction is disabled below so that no two of them are fused.
//
// HBM-bound: each thread owns 8 channels (16-byte loads) of a run of tokens
// and slides a 3-token window through registers, so each input is read once.
#include "../common.h"
#include "../internal.h"

#pragma clang fp contract(off)

namespace gdr {

namespace {

constexpr int kConvThreads = 256;
constexpr int kConvRun = 16;  // tokens per thread

__device__ __forceinline__ float exp32(float x) {
  if (x != x) return x;
  if (x > 0x1.62e430p+6f) return __builtin_inff();
  if (x < -0x1.9fe368p+6f) return 0.f;
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

__device__ __forceinline__ float silu32(float v) { return v / (1.0f + exp32(-v)); }

__device__ __forceinline__ void load8(const uint16_t* p, float* out) {
  const u16x8 raw = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = bf16_to_f32(raw[j]);
}

// Sequence index n with cu[n] <= t < cu[n+1] (empty sequences skipped).
__device__ __forceinline__ int seq_of(const int32_t* cu, int N, int t) {
  int lo = 0, hi = N;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kConvThreads) void conv_front_kernel(ConvArgs a) {
  const int C = (2 * a.Hk + a.Hv) * a.D;
  const int Cq = a.Hk * a.D;
  const int t0 = blockIdx.y * kConvRun;
  const int t_end = min(t0 + kConvRun, a.T);

  // Gates for this token run, one workgroup column per run.
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < kConvRun * a.Hv; e += kConvThreads) {
      const int t = t0 + e / a.Hv, hh = e % a.Hv;
      if (t < a.T) {
        const size_t i = (size_t)t * a.Hv + hh;
        const float x = a.a[i] + a.dt_bias[hh];
        const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
        a.g[i] = -expf(a.A_log[hh]) * sp;
        a.beta[i] = 1.f / (1.f + expf(-a.b[i]));
      }
    }
  }

  const int cg = blockIdx.x * kConvThreads + threadIdx.x;
  if (cg * 8 >= C || t0 >= a.T) return;
  const int c0 = cg * 8;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* sin = static_cast<const uint16_t*>(a.state_in);

  float w[4][8];
  {
    const u16x8* wp = reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(a.w) + (size_t)c0 * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u16x8 raw = wp[q];  // channels c0 + 2q, c0 + 2q + 1, taps 0..3 each
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j][2 * q] = bf16_to_f32(raw[j]);
        w[j][2 * q + 1] = bf16_to_f32(raw[4 + j]);
      }
    }
  }

  uint16_t* out;
  int ld, col;
  if (c0 < Cq) {
    out = static_cast<uint16_t*>(a.q_out); ld = Cq; col = c0;
  } else if (c0 < 2 * Cq) {
    out = static_cast<uint16_t*>(a.k_out); ld = Cq; col = c0 - Cq;
  } else {
    out = static_cast<uint16_t*>(a.v_out); ld = a.Hv * a.D; col = c0 - 2 * Cq;
  }

  int n = seq_of(a.cu_seqlens, a.N, t0);
  int bos = a.cu_seqlens[n], eos = a.cu_seqlens[n + 1];
  float h[3][8];
  // History of the token before t0: inputs of the same sequence, else the
  // carried conv state (oldest first), else zero.
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int p = t0 - 3 + j;
    if (p >= bos) {
      load8(x + (size_t)p * C + c0, h[j]);
    } else if (sin) {
#pragma unroll
      for (int c = 0; c < 8; ++c) h[j][c] = bf16_to_f32(sin[((size_t)n * C + c0 + c) * 3 + (p - bos + 3)]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) h[j][c] = 0.f;
    }
  }

  for (int t = t0; t < t_end; ++t) {
    if (t >= eos) {  // a new sequence starts at t
      while (a.cu_seqlens[n + 1] <= t) ++n;
      bos = a.cu_seqlens[n];
      eos = a.cu_seqlens[n + 1];
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          h[j][c] = sin ? bf16_to_f32(sin[((size_t)n * C + c0 + c) * 3 + j]) : 0.f;
    }
    float xt[8];
    load8(x + (size_t)t * C + c0, xt);
    u16x8 y;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float acc = w[0][c] * h[0][c];
      acc = acc + w[1][c] * h[1][c];
      acc = acc + w[2][c] * h[2][c];
      acc = acc + w[3][c] * xt[c];
      y[c] = f32_to_bf16(silu32(acc));
      h[0][c] = h[1][c];
      h[1][c] = h[2][c];
      h[2][c] = xt[c];
    }
    *reinterpret_cast<u16x8*>(out + (size_t)t * ld + col) = y;
  }
}

// conv_state_out[n, c, j] = extended input (history + tokens) at position
// len + j, i.e. the last three inputs of sequence n.
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
  const int C = (2 * a.Hk + a.Hv) * a.D;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)a.N * C) return;
  const int n = idx / C, c = idx % C;
  const int bos = a.cu_seqlens[n], eos = a.cu_seqlens[n + 1];
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* sin = static_cast<const uint16_t*>(a.state_in);
  uint16_t* sout = static_cast<uint16_t*>(a.state_out);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int p = eos - 3 + j;
    uint16_t val;
    if (p >= bos) val = x[(size_t)p * C + c];
    else if (sin) val = sin[((size_t)n * C + c) * 3 + (p - bos + 3)];
    else val = 0;
    sout[((size_t)n * C + c) * 3 + j] = val;
  }
}

}  // namespace

hipError_t launch_conv_front(const ConvArgs& a, hipStream_t st) {
  const int C = (2 * a.Hk + a.Hv) * a.D;
  if (a.T > 0) {
    const dim3 grid((C / 8 + kConvThreads - 1) / kConvThreads, (a.T + kConvRun - 1) / kConvRun);
    hipLaunchKernelGGL(conv_front_kernel, grid, dim3(kConvThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.state_out && a.N > 0) {
    const size_t total = (size_t)a.N * C;
    hipLaunchKernelGGL(conv_state_kernel, dim3((total + 255) / 256), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdr
