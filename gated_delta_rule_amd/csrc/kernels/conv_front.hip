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
// Horner form and a scale by 2^n.  Every step of exp32 is one IEEE fp32
// operation; FMA contraction is disabled below so that no two of them are
// fused.
//
// Bound by the vector ALU, not by HBM: the contract costs about 40 fp32
// instructions per element (the unfused Horner steps alone are 14), and
// gfx950 retires 64 lanes of them per clock per compute unit.  Everything
// else is cut to the bone: the division is replaced where that is exact
// (silu32_mid), rounding uses the hardware conversion, and the special cases
// cost no per-element compare.  Each thread owns 8 channels (16-byte loads) of
// a run of 8 tokens and reads each of the run's 11 input rows (3 of history)
// once; a run of 8 keeps the fully unrolled body in the instruction cache.
#include "../common.h"
#include "../internal.h"
#include "../silu32.h"

#pragma clang fp contract(off)

namespace gdr {

namespace {

constexpr int kConvThreads = 256;
constexpr int kConvRun = 8;  // tokens per thread

// Sequence index n with cu[n] <= t < cu[n+1] (empty sequences skipped).
__device__ __forceinline__ int seq_of(const int32_t* cu, int N, int t) {
  int lo = 0, hi = N;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Conv + SiLU of channels cg*8 .. +7 over tokens t0 .. t0+7.  The run's 11
// input rows (3 of history; indexes clamped into [0, T), the clamped ones
// never used) are loaded before anything else, the sequence lookup included.
__device__ __forceinline__ void conv_run(const ConvArgs& a, int cg, int t0) {
  const int C = (2 * a.Hk + a.Hv) * a.D;
  const int Cq = a.Hk * a.D;
  if (cg * 8 >= C || t0 >= a.T) return;
  const int c0 = cg * 8;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* sin = static_cast<const uint16_t*>(a.state_in);

  u16x8 raw[kConvRun + 3];  // raw[i]: input row t0 - 3 + i
#pragma unroll
  for (int i = 0; i < kConvRun + 3; ++i) {
    const int r = min(max(t0 - 3 + i, 0), a.T - 1);
    raw[i] = *reinterpret_cast<const u16x8*>(x + (size_t)r * C + c0);
  }

  float w[4][8];
  {
    const u16x8* wp = reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(a.w) + (size_t)c0 * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u16x8 rw = wp[q];  // channels c0 + 2q, c0 + 2q + 1, taps 0..3 each
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j][2 * q] = bf16_to_f32(rw[j]);
        w[j][2 * q + 1] = bf16_to_f32(rw[4 + j]);
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
  // History of token t0: inputs of the same sequence, else the carried conv
  // state (oldest first), else zero.
  float h[3][8];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int p = t0 - 3 + j;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      h[j][c] = p >= bos ? bf16_to_f32(raw[j][c])
              : sin      ? bf16_to_f32(sin[((size_t)n * C + c0 + c) * 3 + (p - bos + 3)])
                         : 0.f;
  }

#pragma unroll
  for (int i = 0; i < kConvRun; ++i) {
    const int t = t0 + i;
    if (t >= a.T) break;
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
    float acc[8];
    bool mid = true;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float xt = bf16_to_f32(raw[i + 3][c]);
      float s = w[0][c] * h[0][c];
      s = s + w[1][c] * h[1][c];
      s = s + w[2][c] * h[2][c];
      s = s + w[3][c] * xt;
      acc[c] = s;
      mid = mid && fabsf(s) <= 80.f;
      h[0][c] = h[1][c];
      h[1][c] = h[2][c];
      h[2][c] = xt;
    }
    // One wave-wide test per token: the general path runs only when some
    // lane's pre-activation leaves [-80, 80] (or is NaN).
    if (__all(mid)) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = silu32_mid(acc[c]);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = silu32(acc[c]);
    }
    u32x4 y;
#pragma unroll
    for (int c = 0; c < 8; c += 2) y[c / 2] = pack_bf16x2(acc[c], acc[c + 1]);
    *reinterpret_cast<u32x4*>(out + (size_t)t * ld + col) = y;
  }
}

__global__ __launch_bounds__(kConvThreads) void conv_front_kernel(ConvArgs a) {
  const int t0 = blockIdx.y * kConvRun;
  conv_run(a, blockIdx.x * kConvThreads + threadIdx.x, t0);
  // Gates of this token run, spread over the run's workgroups, after the
  // conv so that its row loads go out first.
  for (int e = blockIdx.x * kConvThreads + threadIdx.x; e < kConvRun * a.Hv; e += gridDim.x * kConvThreads) {
    const int t = t0 + e / a.Hv, hh = e % a.Hv;
    if (t < a.T) {
      const size_t i = (size_t)t * a.Hv + hh;
      gates(a.a[i], a.b[i], a.A_log[hh], a.dt_bias[hh], a.g[i], a.beta[i]);
    }
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
