// Chunked prefill of the gated delta rule in fp32 on the vector ALUs.
//
// The pages (yfxerp page, section 1.2) say prefill runs a chunk_size=64
// block-parallel path that is numerically interchangeable with the token
// recurrence.  For a chunk of L tokens with start state S0 (d_v x d_k), local
// cumulative log-decay G_i = sum_{m<=i} g_m and Gamma_ij = exp(G_i - G_j)
// (j <= i), the recurrence unrolls exactly into
//
//   (I + A) Delta = diag(beta) V - diag(beta e^G) K^ S0^T,
//                   A_ij = beta_i Gamma_ij k^_i . k^_j  (j < i)
//   O   = scale [diag(e^G) Q^ S0^T + (Gamma * Q^ K^^T) Delta]
//   S_L = e^{G_L} S0 + (diag(Gamma_{L,:}) Delta)^T K^
//
// This kernel evaluates those equations literally in fp32 (Delta by forward
// substitution), one workgroup per (sequence, value head, d_v slice).  It is
// the path for fp32 q/k/v (where operands are not bf16-exact and the required
// accuracy is 1e-5 of the output RMS) and for shapes the MFMA kernel does not
// take; speed is secondary here.  The chunk-local cumulative decay is summed in
// fp64 so exp(G_i - G_j) keeps full fp32 accuracy even when |G| reaches
// hundreds within a chunk.
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

template <int D, int C, int DVS>
struct F32Smem {
  float K[C][D + 1];
  float Q[C][D + 1];
  float V[C][DVS];
  float Dl[C][DVS];  // R, then Delta
  float A[C][C + 1];
  float P[C][C + 1];
  float S[DVS][D + 1];
  double G[C];
  float beta[C], eG[C], cL[C], r[2][C];
  float eGL;
};

template <int D, int C, int DVS, typename TQ, typename TO>
__global__ __launch_bounds__(256) void chunk_f32_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  F32Smem<D, C, DVS>& sm = *reinterpret_cast<F32Smem<D, C, DVS>*>(smem_raw);
  const int tid = threadIdx.x;
  const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int Hk = a.Hk, Hv = a.Hv;
  const int kh = h / (Hv / Hk);
  const int v0 = slice * DVS;
  int bos, eos;
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  const TQ* q = static_cast<const TQ*>(a.q);
  const TQ* k = static_cast<const TQ*>(a.k);
  const TQ* v = static_cast<const TQ*>(a.v);
  TO* o = static_cast<TO*>(a.o);

  const size_t sbase = ((size_t)n * Hv + h) * D * D + (size_t)v0 * D;
  for (int e = tid; e < DVS * D; e += 256) {
    const int c = e / D, j = e % D;
    sm.S[c][j] = a.initial_state ? a.initial_state[sbase + (size_t)c * D + j] : 0.f;
  }

  for (int c0 = bos; c0 < eos; c0 += C) {
    const int L = min(C, eos - c0);
    __syncthreads();
    for (int e = tid; e < C * D; e += 256) {
      const int i = e / D, j = e % D;
      float kv = 0.f, qv = 0.f;
      if (i < L) {
        const size_t off = ((size_t)(c0 + i) * Hk + kh) * D + j;
        kv = load_as_f32(k + off);
        qv = load_as_f32(q + off);
      }
      sm.K[i][j] = kv;
      sm.Q[i][j] = qv;
    }
    for (int e = tid; e < C * DVS; e += 256) {
      const int i = e / DVS, j = e % DVS;
      sm.V[i][j] = i < L ? load_as_f32(v + ((size_t)(c0 + i) * Hv + h) * D + v0 + j) : 0.f;
    }
    if (tid < C) sm.beta[tid] = tid < L ? a.beta[(size_t)(c0 + tid) * Hv + h] : 0.f;
    if (tid == 0) {
      double G = 0.0;
      for (int i = 0; i < C; ++i) {
        if (i < L) {
          const float gi = a.g[(size_t)(c0 + i) * Hv + h];
          G += (double)(gi < kMinLogDecay ? kMinLogDecay : gi);  // (a NaN stays NaN)
        }
        sm.G[i] = G;
      }
    }
    __syncthreads();
    // L2 norms (thread i: key row i, thread C + i: query row i).
    if (tid < 2 * C) {
      const int i = tid % C;
      float (*X)[D + 1] = tid < C ? sm.K : sm.Q;
      float ss = 0.f;
      for (int j = 0; j < D; ++j) ss += X[i][j] * X[i][j];
      sm.r[tid / C][i] = a.use_l2 ? 1.f / sqrtf(ss + a.eps) : 1.f;
    }
    if (tid < C) {
      sm.eG[tid] = expf((float)sm.G[tid]);
      sm.cL[tid] = expf((float)(sm.G[C - 1] - sm.G[tid]));
    }
    if (tid == 0) sm.eGL = expf((float)sm.G[C - 1]);
    __syncthreads();
    for (int e = tid; e < C * D; e += 256) {
      const int i = e / D, j = e % D;
      sm.K[i][j] *= sm.r[0][i];
      sm.Q[i][j] *= sm.r[1][i];
    }
    __syncthreads();
    // A (strictly lower) and P (lower incl. diagonal).
    for (int e = tid; e < C * C; e += 256) {
      const int i = e / C, j = e % C;
      float av = 0.f, pv = 0.f;
      if (j <= i) {
        const float gam = expf((float)(sm.G[i] - sm.G[j]));
        float kk = 0.f, qk = 0.f;
        for (int d = 0; d < D; ++d) {
          kk += sm.K[i][d] * sm.K[j][d];
          qk += sm.Q[i][d] * sm.K[j][d];
        }
        if (j < i) av = sm.beta[i] * gam * kk;
        pv = a.scale * gam * qk;
      }
      sm.A[i][j] = av;
      sm.P[i][j] = pv;
    }
    // R = diag(beta) V - diag(beta e^G) K^ S0^T
    for (int e = tid; e < C * DVS; e += 256) {
      const int i = e / DVS, c = e % DVS;
      float x = 0.f;
      for (int d = 0; d < D; ++d) x += sm.K[i][d] * sm.S[c][d];
      sm.Dl[i][c] = sm.beta[i] * (sm.V[i][c] - sm.eG[i] * x);
    }
    __syncthreads();
    // Forward substitution (I + A) Delta = R, one lane per value column.
    if (tid < DVS) {
      for (int i = 1; i < L; ++i) {
        float x = sm.Dl[i][tid];
        for (int j = 0; j < i; ++j) x -= sm.A[i][j] * sm.Dl[j][tid];
        sm.Dl[i][tid] = x;
      }
    }
    __syncthreads();
    // O = scale e^G Q^ S0^T + P Delta
    for (int e = tid; e < L * DVS; e += 256) {
      const int i = e / DVS, c = e % DVS;
      float y = 0.f;
      for (int d = 0; d < D; ++d) y += sm.Q[i][d] * sm.S[c][d];
      float pd = 0.f;
      for (int j = 0; j <= i; ++j) pd += sm.P[i][j] * sm.Dl[j][c];
      store_from_f32(o + ((size_t)(c0 + i) * Hv + h) * D + v0 + c, a.scale * sm.eG[i] * y + pd);
    }
    __syncthreads();
    // S <- e^{G_L} S0 + (diag(Gamma_L) Delta)^T K^
    for (int e = tid; e < DVS * D; e += 256) {
      const int c = e / D, d = e % D;
      float x = 0.f;
      for (int j = 0; j < L; ++j) x += sm.cL[j] * sm.Dl[j][c] * sm.K[j][d];
      sm.S[c][d] = sm.eGL * sm.S[c][d] + x;
    }
  }
  __syncthreads();
  if (a.final_state) {
    for (int e = tid; e < DVS * D; e += 256) {
      const int c = e / D, j = e % D;
      a.final_state[sbase + (size_t)c * D + j] = sm.S[c][j];
    }
  }
}

template <int D, int C, typename TQ, typename TO>
hipError_t launch_f32_t(const ChunkArgs& a, hipStream_t st) {
  constexpr int DVS = D < 32 ? D : 32;
  auto kern = chunk_f32_kernel<D, C, DVS, TQ, TO>;
  const size_t smem = sizeof(F32Smem<D, C, DVS>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(D / DVS, a.Hv, a.N), dim3(256), smem, st, a);
  return hipGetLastError();
}

template <int D, int C>
hipError_t launch_f32_dc(const ChunkArgs& a, hipStream_t st) {
  if (a.qkv_bf16)
    return a.out_bf16 ? launch_f32_t<D, C, uint16_t, uint16_t>(a, st) : launch_f32_t<D, C, uint16_t, float>(a, st);
  return a.out_bf16 ? launch_f32_t<D, C, float, uint16_t>(a, st) : launch_f32_t<D, C, float, float>(a, st);
}

template <int D>
hipError_t launch_f32_d(const ChunkArgs& a, hipStream_t st) {
  return a.C == 64 ? launch_f32_dc<D, 64>(a, st) : launch_f32_dc<D, 32>(a, st);
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a, hipStream_t st) {
  switch (a.D) {
    case 32: return launch_f32_d<32>(a, st);
    case 64: return launch_f32_d<64>(a, st);
    case 128: return launch_f32_d<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdr
