// Chunked prefill of the gated delta rule on CDNA4 bf16 matrix cores.
//
// The pages (yfxerp page, section 1.2) say prefill runs a chunk_size=64
// block-parallel path numerically interchangeable with the token recurrence
// S_t = S_{t-1} e^{g_t} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t.
// For a chunk of L <= 64 tokens with start state S0 (d_v x d_k), cumulative
// log-decay G_i = sum_{m<=i} g_m and Gamma_ij = e^{G_i - G_j} (j <= i):
//
//   T     = (I + A)^{-1},   A_ij = beta_i Gamma_ij k^_i . k^_j   (j < i)
//   R     = diag(beta) V - diag(beta e^G) K^ S0^T
//   Delta = T R
//   O     = scale diag(e^G) Q^ S0^T + P Delta,  P_ij = scale Gamma_ij q^_i . k^_j (j <= i)
//   S_L   = e^{G_L} S0 + (diag(Gamma_{L,:}) Delta)^T K^
//
// Work split: one workgroup per (sequence, value head, d_v slice of 16*NW);
// wave w owns a 16-wide column block of the state for the whole sequence and
// runs its chain (X = K S0^T, R, Delta, O, S update) without exchanging data
// with other waves.  The trick that makes this possible: the matrix-core
// output layout (lane holds rows 4*(l/16)+i of column l%16) is fed back as the
// B operand of the next contraction by permuting the contraction index in the
// same way on both operands, so R, Delta and the state never leave registers.
// The shared A operands (K, Q, K^T, T, P) live in LDS with their contraction
// columns stored in that permuted order, so each fragment is one 16-byte read.
//
// Precision: q, k, v are exact bf16 MFMA operands; the L2-norm factors and
// gates are applied as fp32 scales after the products.  Every computed operand
// (state, T, R, Delta, P) is split into bf16 hi + lo and multiplied with 2 or 3
// MFMAs (lo x lo dropped), which keeps ~16 significant bits; accumulation is
// fp32 and the state carry is fp32.  The chunk-local cumulative decay is summed
// in fp64, and only exponents e^{G_i - G_j} with j <= i are ever formed.
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

constexpr int kD = 128;  // head dim (d_k = d_v)
constexpr int kC = 64;   // chunk

// Position of contraction index x inside its 32-block: logical
// x = 16*hi + 4*q + e is stored at 8*q + 4*hi + e, so the 8 values lane group
// q needs for one 16x16x32 step (rows 4q..4q+3 of two consecutive 16-row
// output tiles) are contiguous.
__device__ __forceinline__ int perm32(int x) {
  const int y = x & 31;
  return (x & ~31) + ((y >> 2) & 3) * 8 + (y >> 4) * 4 + (y & 3);
}

template <int DVS>
struct __align__(16) MfmaSmem {
  uint16_t Kr[kC][kD + 8];  // k rows, columns permuted
  uint16_t Qr[kC][kD + 8];  // q rows, columns permuted
  uint16_t Kt[kD][kC + 8];  // k transposed, tokens permuted
  uint16_t Vt[DVS][kC + 4]; // v slice transposed (token-contiguous)
  uint16_t Th[kC][kC + 8], Tl[kC][kC + 8];  // T hi/lo, columns permuted
  uint16_t Ph[kC][kC + 8], Pl[kC][kC + 8];  // P hi/lo, columns permuted
  float A[kC][kC + 1];
  float Tf[kC][kC + 1];
  float Ys[32][33];
  double G[kC];
  float gin[kC], bt[kC], rk[kC], rq[kC], xr[kC], yq[kC], cL[kC];
  float eGL;
};

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u16x8*>(p));
}

// bf16 hi/lo fragments of 8 fp32 values: first four from x0, last four from x1.
__device__ __forceinline__ void split8(const f32x4& x0, const f32x4& x1, bf16x8& hi, bf16x8& lo) {
  u16x8 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint16_t a, b, c, d;
    split_bf16(x0[j], a, b);
    split_bf16(x1[j], c, d);
    h[j] = a;
    l[j] = b;
    h[4 + j] = c;
    l[4 + j] = d;
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

// 8 fp32 values from LDS (stride-1 or strided) split to hi/lo; zero if !on.
__device__ __forceinline__ void split8_lds(const float* p, int stride, bool on, bf16x8& hi, bf16x8& lo) {
  u16x8 h, l;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = on ? p[j * stride] : 0.f;
    uint16_t a, b;
    split_bf16(x, a, b);
    h[j] = a;
    l[j] = b;
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 acc) {
  acc = mfma16x16x32(ah, bh, acc);
  acc = mfma16x16x32(ah, bl, acc);
  acc = mfma16x16x32(al, bh, acc);
  return acc;
}

// 16x16 tile of M1 * M2 with fp32 operands in LDS split to bf16 hi/lo.
// M1 rows r0.., columns k0..k0+K-1; M2 rows k0'.., columns c0'..  (K = 16 or 32)
template <int K>
__device__ __forceinline__ f32x4 tile_mm_f32(const float* m1, int ld1, const float* m2, int ld2, int lane) {
  const int c = lane & 15, q4 = lane >> 4;
  const bool on = (q4 * 8) < K;
  bf16x8 ah, al, bh, bl;
  split8_lds(m1 + c * ld1 + q4 * 8, 1, on, ah, al);
  split8_lds(m2 + (q4 * 8) * ld2 + c, ld2, on, bh, bl);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  return mfma3(ah, al, bh, bl, acc);
}

template <int NW, typename TO>
__global__ __launch_bounds__(64 * NW) void chunk_bf16_kernel(ChunkArgs a) {
  constexpr int DVS = 16 * NW;
  constexpr int NT = 64 * NW;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  MfmaSmem<DVS>& sm = *reinterpret_cast<MfmaSmem<DVS>*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q4 = lane >> 4;
  const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int Hk = a.Hk, Hv = a.Hv;
  const int kh = h / (Hv / Hk);
  const int v0 = slice * DVS;      // first value channel of this workgroup
  const int vw = 16 * wave;        // this wave's column block inside the slice
  int bos, eos;
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* vg = static_cast<const uint16_t*>(a.v);
  TO* og = static_cast<TO*>(a.o);

  // State S^T tiles (kd-tile kt): lane holds S[v0 + vw + c][16 kt + 4 q4 + i].
  f32x4 s[8];
  const size_t sbase = ((size_t)n * Hv + h) * kD * kD + (size_t)(v0 + vw + c) * kD + 4 * q4;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    if (a.initial_state) s[kt] = *reinterpret_cast<const f32x4*>(a.initial_state + sbase + 16 * kt);
    else s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int c0 = bos; c0 < eos; c0 += kC) {
    const int L = min(kC, eos - c0);

    // ---- load k, q (8x8 blocks: row-major permuted copy + transposed copy of k), v, g, beta
    for (int blk = tid; blk < 256; blk += NT) {
      const int isq = blk >> 7, b = blk & 127, rb = b >> 4, cb = b & 15;
      const uint16_t* src = isq ? qg : kg;
      u16x8 val[8];
      float ss[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int row = 8 * rb + r;
        if (row < L) val[r] = *reinterpret_cast<const u16x8*>(src + ((size_t)(c0 + row) * Hk + kh) * kD + 8 * cb);
        else val[r] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = bf16_to_f32(val[r][e]);
          acc += x * x;
        }
        ss[r] = acc;
      }
      uint16_t(*X)[kD + 8] = isq ? sm.Qr : sm.Kr;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int row = 8 * rb + r;
        *reinterpret_cast<u16x4*>(&X[row][perm32(8 * cb)]) = u16x4{val[r][0], val[r][1], val[r][2], val[r][3]};
        *reinterpret_cast<u16x4*>(&X[row][perm32(8 * cb + 4)]) = u16x4{val[r][4], val[r][5], val[r][6], val[r][7]};
      }
      if (!isq) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          *reinterpret_cast<u16x4*>(&sm.Kt[8 * cb + e][perm32(8 * rb)]) =
              u16x4{val[0][e], val[1][e], val[2][e], val[3][e]};
          *reinterpret_cast<u16x4*>(&sm.Kt[8 * cb + e][perm32(8 * rb + 4)]) =
              u16x4{val[4][e], val[5][e], val[6][e], val[7][e]};
        }
      }
      // squared norms: reduce over the 16 column blocks (16 consecutive lanes)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float tot = group_sum<16>(ss[r]);
        if (cb == 0) {
          const float rr = a.use_l2 ? 1.f / sqrtf(tot + a.eps) : 1.f;
          (isq ? sm.rq : sm.rk)[8 * rb + r] = rr;
        }
      }
    }
    for (int id = tid; id < kC * (DVS / 8); id += NT) {
      const int tok = id / (DVS / 8), vc = (id % (DVS / 8)) * 8;
      u16x8 val = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (tok < L) val = *reinterpret_cast<const u16x8*>(vg + ((size_t)(c0 + tok) * Hv + h) * kD + v0 + vc);
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.Vt[vc + e][tok] = val[e];
    }
    for (int i = tid; i < 2 * kC; i += NT) {
      const int tok = i & (kC - 1);
      const float x = tok < L ? (i < kC ? a.g : a.beta)[(size_t)(c0 + tok) * Hv + h] : 0.f;
      (i < kC ? sm.gin : sm.bt)[tok] = x;
    }
    __syncthreads();

    // ---- chunk-local cumulative decay (fp64) and per-token factors
    if (wave == 0) {
      double G = (double)sm.gin[lane];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(G, off, 64);
        if (lane >= off) G += o;
      }
      const double GL = __shfl(G, 63, 64);
      sm.G[lane] = G;
      const float eG = expf((float)G);
      const float rkv = sm.rk[lane];
      sm.xr[lane] = sm.bt[lane] * eG * rkv;
      sm.yq[lane] = a.scale * sm.rq[lane] * eG;
      sm.cL[lane] = rkv * expf((float)(GL - G));
      if (lane == 0) sm.eGL = expf((float)GL);
    }
    __syncthreads();

    // ---- Gram tiles: A (fp32, strictly lower) from K K^T, P (hi/lo) from Q K^T
    for (int job = wave; job < 20; job += NW) {
      const bool isq = job >= 10;
      const int idx = job % 10;  // lower-triangular tile (ti, tj), row-major order
      const int ti = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
      const int tj = idx - ti * (ti + 1) / 2;
      const uint16_t(*X)[kD + 8] = isq ? sm.Qr : sm.Kr;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(lds8(&X[16 * ti + c][32 * ks + 8 * q4]), lds8(&sm.Kr[16 * tj + c][32 * ks + 8 * q4]), acc);
      const int j = 16 * tj + c;
      const double Gj = sm.G[j];
      const float rkj = sm.rk[j];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int i = 16 * ti + 4 * q4 + i4;
        const float gam = j <= i ? expf((float)(sm.G[i] - Gj)) : 0.f;
        if (!isq) {
          sm.A[i][j] = j < i ? sm.bt[i] * gam * sm.rk[i] * rkj * acc[i4] : 0.f;
        } else {
          uint16_t hi, lo;
          split_bf16(a.scale * gam * sm.rq[i] * rkj * acc[i4], hi, lo);
          sm.Ph[i][perm32(j)] = hi;
          sm.Pl[i][perm32(j)] = lo;
        }
      }
    }
    // zero the above-diagonal tiles that the 32-wide contraction steps touch
    for (int e = tid; e < 2 * 256; e += NT) {
      const int t = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int i = 32 * t + r, j = 32 * t + 16 + cc;
      sm.Ph[i][perm32(j)] = 0;
      sm.Pl[i][perm32(j)] = 0;
      sm.Th[i][perm32(j)] = 0;
      sm.Tl[i][perm32(j)] = 0;
      sm.Tf[i][j] = 0.f;
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution
    if (wave == 0) {
      const int b = q4;  // block
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) {
          const float am = sm.A[16 * b + r][16 * b + m];
          if (m & 1) s1 += am * x[m]; else s0 += am * x[m];
        }
        if (r > c) x[r] = -(s0 + s1);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Tf[16 * b + r][16 * b + c] = x[r];
    }
    __syncthreads();
    // level 1: T_{p+1,p} = -T_{p+1,p+1} (A_{p+1,p} T_{p,p}), p = 0, 2
    for (int m = wave; m < 2; m += NW) {
      const int p = 16 * (2 * m);
      const f32x4 y = tile_mm_f32<16>(&sm.A[p + 16][p], kC + 1, &sm.Tf[p][p], kC + 1, lane);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Ys[16 * m + 4 * q4 + i4][c] = y[i4];
    }
    __syncthreads();
    for (int m = wave; m < 2; m += NW) {
      const int p = 16 * (2 * m);
      const f32x4 t = tile_mm_f32<16>(&sm.Tf[p + 16][p + 16], kC + 1, &sm.Ys[16 * m][0], 33, lane);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Tf[p + 16 + 4 * q4 + i4][p + c] = -t[i4];
    }
    __syncthreads();
    // level 2: T_{2:4,0:2} = -T_{2:4,2:4} (A_{2:4,0:2} T_{0:2,0:2})  (32x32 blocks)
    for (int jb = wave; jb < 4; jb += NW) {
      const int yi = jb >> 1, yj = jb & 1;
      const f32x4 y = tile_mm_f32<32>(&sm.A[32 + 16 * yi][0], kC + 1, &sm.Tf[0][16 * yj], kC + 1, lane);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Ys[16 * yi + 4 * q4 + i4][16 * yj + c] = y[i4];
    }
    __syncthreads();
    for (int jb = wave; jb < 4; jb += NW) {
      const int xi = jb >> 1, xj = jb & 1;
      const f32x4 t = tile_mm_f32<32>(&sm.Tf[32 + 16 * xi][32], kC + 1, &sm.Ys[0][16 * xj], 33, lane);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Tf[32 + 16 * xi + 4 * q4 + i4][16 * xj + c] = -t[i4];
    }
    __syncthreads();
    // the lower 32x32-block triangle, including the zero upper parts of the
    // diagonal blocks that the 32-wide contraction steps read
    for (int e = tid; e < kC * kC; e += NT) {
      const int i = e >> 6, j = e & 63;
      if (j < 32 * (i / 32 + 1)) {
        uint16_t hi, lo;
        split_bf16(sm.Tf[i][j], hi, lo);
        sm.Th[i][perm32(j)] = hi;
        sm.Tl[i][perm32(j)] = lo;
      }
    }
    __syncthreads();

    // ---- per-wave chain on this wave's 16 value channels
    bf16x8 sbh[4], sbl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) split8(s[2 * ks], s[2 * ks + 1], sbh[ks], sbl[ks]);

    f32x4 R[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ak = lds8(&sm.Kr[16 * ti + c][32 * ks + 8 * q4]);
        acc = mfma16x16x32(ak, sbh[ks], acc);
        acc = mfma16x16x32(ak, sbl[ks], acc);
      }
      const u16x4 vv = *reinterpret_cast<const u16x4*>(&sm.Vt[vw + c][16 * ti + 4 * q4]);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int t = 16 * ti + 4 * q4 + i4;
        R[ti][i4] = sm.bt[t] * bf16_to_f32(vv[i4]) - sm.xr[t] * acc[i4];
      }
    }
    bf16x8 rbh[2], rbl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) split8(R[2 * ks], R[2 * ks + 1], rbh[ks], rbl[ks]);

    f32x4 Dl[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks * 2 > ti) continue;
        acc = mfma3(lds8(&sm.Th[16 * ti + c][32 * ks + 8 * q4]), lds8(&sm.Tl[16 * ti + c][32 * ks + 8 * q4]),
                    rbh[ks], rbl[ks], acc);
      }
      Dl[ti] = acc;
    }
    bf16x8 dbh[2], dbl[2], dph[2], dpl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      split8(Dl[2 * ks], Dl[2 * ks + 1], dbh[ks], dbl[ks]);
      f32x4 d0, d1;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        d0[i4] = Dl[2 * ks][i4] * sm.cL[32 * ks + 4 * q4 + i4];
        d1[i4] = Dl[2 * ks + 1][i4] * sm.cL[32 * ks + 16 + 4 * q4 + i4];
      }
      split8(d0, d1, dph[ks], dpl[ks]);
    }

    // outputs
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 aq = lds8(&sm.Qr[16 * ti + c][32 * ks + 8 * q4]);
        y = mfma16x16x32(aq, sbh[ks], y);
        y = mfma16x16x32(aq, sbl[ks], y);
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) y[i4] *= sm.yq[16 * ti + 4 * q4 + i4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks * 2 > ti) continue;
        y = mfma3(lds8(&sm.Ph[16 * ti + c][32 * ks + 8 * q4]), lds8(&sm.Pl[16 * ti + c][32 * ks + 8 * q4]),
                  dbh[ks], dbl[ks], y);
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int t = 16 * ti + 4 * q4 + i4;
        if (t < L) store_from_f32(og + ((size_t)(c0 + t) * Hv + h) * kD + v0 + vw + c, y[i4]);
      }
    }

    // state update S^T <- e^{G_L} S^T + K^T Delta'
    const float eGL = sm.eGL;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 acc = s[kt] * eGL;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 akt = lds8(&sm.Kt[16 * kt + c][32 * ks + 8 * q4]);
        acc = mfma16x16x32(akt, dph[ks], acc);
        acc = mfma16x16x32(akt, dpl[ks], acc);
      }
      s[kt] = acc;
    }
    __syncthreads();
  }

  if (a.final_state) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) *reinterpret_cast<f32x4*>(a.final_state + sbase + 16 * kt) = s[kt];
  }
}

template <int NW, typename TO>
hipError_t launch_bf16_t(const ChunkArgs& a, hipStream_t st) {
  auto kern = chunk_bf16_kernel<NW, TO>;
  const size_t smem = sizeof(MfmaSmem<16 * NW>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(kD / (16 * NW), a.Hv, a.N), dim3(64 * NW), smem, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t st) {
  return a.out_bf16 ? launch_bf16_t<4, uint16_t>(a, st) : launch_bf16_t<4, float>(a, st);
}

}  // namespace gdr
