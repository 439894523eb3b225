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
// Work split: one workgroup of 4 waves per (sequence, value head, 64 value
// channels); wave w owns 16 value channels of the state for the whole
// sequence and runs their chain (X = K S0^T, R, Delta, O, S update) without
// exchanging data with other waves.  The matrix-core output layout (lane l
// holds rows 4*(l/16)+i of column l%16) is fed back as the B operand of the
// next contraction by permuting the contraction index identically on both
// operands, so R, Delta and the state stay in registers.  The shared A
// operands (K, Q, K^T, T, P) live in LDS with their contraction index stored
// in that permuted order, so each fragment is one 16-byte read.  The chunk's
// setup (Gram matrices, norms, decays, T) is shared by the 4 waves; the next
// chunk's global loads are issued before the state phase of the current one.
//
// Precision: q, k, v are exact bf16 MFMA operands; L2-norm factors and gates
// are fp32 scales applied after the products.  Every computed operand (state,
// T, R, Delta, P) is split into bf16 hi + lo and multiplied with 2 or 3 MFMAs
// (lo x lo dropped), keeping ~16 significant bits; accumulation and the state
// carry are fp32.  The chunk-local cumulative decay is summed in fp64; only
// exponents exp2(G_i - G_j) with j <= i are formed (never overflow).
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

constexpr int kD = 128;  // head dim (d_k = d_v)
constexpr int kC = 64;   // chunk
constexpr int kNW = 4;   // waves per workgroup
constexpr int kNT = 64 * kNW;
constexpr int kDVS = 16 * kNW;  // value channels per workgroup

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Physical position of contraction index x in a 32-block: logical
// x = 16*hi + 4*q + e lives at 8*q + 4*hi + e, so the 8 values lane group q
// needs for one 16x16x32 step (rows 4q..4q+3 of two consecutive 16-row output
// tiles) are contiguous.  Groups of 4 stay contiguous.
__device__ __forceinline__ int perm32(int x) {
  const int y = x & 31;
  return (x & ~31) + ((y >> 2) & 3) * 8 + (y >> 4) * 4 + (y & 3);
}
// perm32(8*b) for a block of 8 consecutive logical indices (second half at +8)
__device__ __forceinline__ int perm8(int b) {
  return 32 * (b >> 2) + ((0x14041000u >> (8 * (b & 3))) & 0xff);
}

struct __align__(16) Smem {
  uint16_t Kr[kC][kD + 8];   // k rows, columns permuted
  uint16_t Qr[kC][kD + 8];   // q rows, columns permuted
  uint16_t Kt[kD][kC + 8];   // k transposed, tokens permuted
  uint16_t Th[kC][kC + 8], Tl[kC][kC + 8];  // T hi/lo, columns permuted
  uint16_t Ph[kC][kC + 8], Pl[kC][kC + 8];  // P hi/lo, columns permuted
  float A[kC][kC + 4];
  float Tf[kC][kC + 4];
  float Ys[32][36];
  float ssk[kC], ssq[kC];            // squared norms
  float G2[kC];                      // cumulative log2-decay
  float rk[kC], ar[kC], pr[kC];      // column / row factors of A and P
  float bt[kC], xr[kC], yq[kC], cL[kC];  // token factors of the state phase
  float gin[kC], bin[kC];
  float eGL;
};

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// bf16 hi/lo of two fp32 values, packed: hi = rne(x), lo = rne(x - hi).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  bf16x2 h;
  h[0] = (__bf16)x0;
  h[1] = (__bf16)x1;
  hi = __builtin_bit_cast(uint32_t, h);
  const float r0 = x0 - __uint_as_float(hi << 16);
  const float r1 = x1 - __uint_as_float(hi & 0xffff0000u);
  bf16x2 l;
  l[0] = (__bf16)r0;
  l[1] = (__bf16)r1;
  lo = __builtin_bit_cast(uint32_t, l);
}

// Fragments of 8 values: first four from x0, last four from x1.
__device__ __forceinline__ void split8(const f32x4& x0, const f32x4& x1, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
  uint32_t t0, t1;
  split2(x0[0], x0[1], t0, t1); h[0] = t0; l[0] = t1;
  split2(x0[2], x0[3], t0, t1); h[1] = t0; l[1] = t1;
  split2(x1[0], x1[1], t0, t1); h[2] = t0; l[2] = t1;
  split2(x1[2], x1[3], t0, t1); h[3] = t0; l[3] = t1;
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ void split4(const f32x4& x, u32x2& hi, u32x2& lo) {
  uint32_t t0, t1;
  split2(x[0], x[1], t0, t1); hi[0] = t0; lo[0] = t1;
  split2(x[2], x[3], t0, t1); hi[1] = t0; lo[1] = t1;
}

__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 acc) {
  acc = mfma16x16x32(ah, bh, acc);
  acc = mfma16x16x32(ah, bl, acc);
  acc = mfma16x16x32(al, bh, acc);
  return acc;
}

// 16x16 tile of M1 * M2, fp32 operands in LDS (leading dims ld1, ld2), split
// to bf16 hi/lo.  K = 16 or 32 contraction length.
template <int K>
__device__ __forceinline__ f32x4 tile_mm_f32(const float* m1, int ld1, const float* m2, int ld2, int c, int q4) {
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
  if (8 * q4 < K) {
    a0 = *reinterpret_cast<const f32x4*>(m1 + c * ld1 + 8 * q4);
    a1 = *reinterpret_cast<const f32x4*>(m1 + c * ld1 + 8 * q4 + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0[j] = m2[(8 * q4 + j) * ld2 + c];
      b1[j] = m2[(8 * q4 + 4 + j) * ld2 + c];
    }
  }
  bf16x8 ah, al, bh, bl;
  split8(a0, a1, ah, al);
  split8(b0, b1, bh, bl);
  return mfma3(ah, al, bh, bl, f32x4{0.f, 0.f, 0.f, 0.f});
}

// Registers holding one chunk's global inputs between issue and LDS store.
struct ChunkRegs {
  u16x8 kq[8];      // 8 rows x 8 columns of k (threads 0..127) or q (128..255)
  uint16_t vv[16];  // this lane's v values in accumulator layout
  float gb;         // g (wave 0) or beta (wave 1) of token `lane`
};

template <bool kFull>
__device__ __forceinline__ void issue_loads(ChunkRegs& r, const ChunkArgs& a, int c0, int L, int kh, int h,
                                            int vcol, int tid, int lane, int wave, int q4) {
  const uint16_t* src = static_cast<const uint16_t*>(tid < 128 ? a.k : a.q);
  const int b = tid & 127, rb = b >> 4, cb = b & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * rb + i;
    if (kFull || row < L)
      r.kq[i] = *reinterpret_cast<const u16x8*>(src + ((size_t)(c0 + row) * a.Hk + kh) * kD + 8 * cb);
    else
      r.kq[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  const uint16_t* vg = static_cast<const uint16_t*>(a.v);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int t = 16 * ti + 4 * q4 + i4;
      r.vv[4 * ti + i4] = (kFull || t < L) ? vg[((size_t)(c0 + t) * a.Hv + h) * kD + vcol] : uint16_t(0);
    }
  r.gb = 0.f;
  if (wave < 2) {
    const float* p = wave == 0 ? a.g : a.beta;
    r.gb = (kFull || lane < L) ? p[(size_t)(c0 + lane) * a.Hv + h] : 0.f;
  }
}

template <typename TO>
__global__ __launch_bounds__(kNT) void chunk_bf16_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q4 = lane >> 4;
  const int slice = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int kh = h / (a.Hv / a.Hk);
  const int v0 = slice * kDVS;
  const int vcol = v0 + 16 * wave + c;  // this lane's value channel
  int bos, eos;
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  TO* og = static_cast<TO*>(a.o);

  // State S^T tiles (kd-tile kt): lane holds S[vcol][16 kt + 4 q4 + i].
  f32x4 s[8];
  const size_t sbase = ((size_t)n * a.Hv + h) * kD * kD + (size_t)vcol * kD + 4 * q4;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
    s[kt] = a.initial_state ? *reinterpret_cast<const f32x4*>(a.initial_state + sbase + 16 * kt)
                            : f32x4{0.f, 0.f, 0.f, 0.f};

  ChunkRegs cur;
  if (bos < eos) {
    const int L0 = min(kC, eos - bos);
    if (L0 == kC) issue_loads<true>(cur, a, bos, L0, kh, h, vcol, tid, lane, wave, q4);
    else issue_loads<false>(cur, a, bos, L0, kh, h, vcol, tid, lane, wave, q4);
  }

  for (int c0 = bos; c0 < eos; c0 += kC) {
    const int L = min(kC, eos - c0);

    // ---- store this chunk's k/q blocks to LDS (k also transposed)
    {
      const int b = tid & 127, rb = b >> 4, cb = b & 15;
      uint16_t(*X)[kD + 8] = tid < 128 ? sm.Kr : sm.Qr;
      const int pc = perm8(cb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 w = __builtin_bit_cast(u32x4, cur.kq[i]);
        *reinterpret_cast<u32x2*>(&X[8 * rb + i][pc]) = u32x2{w[0], w[1]};
        *reinterpret_cast<u32x2*>(&X[8 * rb + i][pc + 8]) = u32x2{w[2], w[3]};
      }
      if (tid < 128) {
        const int pr8 = perm8(rb);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {  // columns 2*e2, 2*e2+1 of the 8x8 block
          uint32_t lo01[4], hi01[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const uint32_t w0 = __builtin_bit_cast(u32x4, cur.kq[i])[e2];
            const uint32_t w1 = __builtin_bit_cast(u32x4, cur.kq[i + 1])[e2];
            lo01[i / 2] = (w0 & 0xffffu) | (w1 << 16);
            hi01[i / 2] = (w0 >> 16) | (w1 & 0xffff0000u);
          }
          *reinterpret_cast<u32x2*>(&sm.Kt[8 * cb + 2 * e2][pr8]) = u32x2{lo01[0], lo01[1]};
          *reinterpret_cast<u32x2*>(&sm.Kt[8 * cb + 2 * e2][pr8 + 8]) = u32x2{lo01[2], lo01[3]};
          *reinterpret_cast<u32x2*>(&sm.Kt[8 * cb + 2 * e2 + 1][pr8]) = u32x2{hi01[0], hi01[1]};
          *reinterpret_cast<u32x2*>(&sm.Kt[8 * cb + 2 * e2 + 1][pr8 + 8]) = u32x2{hi01[2], hi01[3]};
        }
      }
      if (wave == 0) sm.gin[lane] = cur.gb;
      if (wave == 1) sm.bin[lane] = cur.gb;
    }
    uint16_t vv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) vv[i] = cur.vv[i];
    __syncthreads();

    // ---- Gram tiles (raw bf16 products): job 0..9 K_j K_i^T, 10..19 K_j Q_i^T,
    // 20..23 Q_i Q_i^T (diagonal only, for the q norms).  Lane holds
    // G[row i = 16 ti + c][cols j = 16 tj + 4 q4 .. +3].
    f32x4 gacc[5];
    int gti[5], gtj[5];
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int job = wave + kNW * u;
      int ti, tj;
      const uint16_t(*XA)[kD + 8];
      const uint16_t(*XB)[kD + 8];
      if (job < 20) {
        const int idx = job % 10;
        ti = idx >= 6 ? 3 : (idx >= 3 ? 2 : (idx >= 1 ? 1 : 0));
        tj = idx - ti * (ti + 1) / 2;
        XA = sm.Kr;
        XB = job < 10 ? sm.Kr : sm.Qr;
      } else {
        ti = tj = job - 20;
        XA = sm.Qr;
        XB = sm.Qr;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(lds8(&XA[16 * tj + c][32 * ks + 8 * q4]), lds8(&XB[16 * ti + c][32 * ks + 8 * q4]), acc);
      if (u < 5) {
        gacc[u] = acc;
        gti[u] = ti;
        gtj[u] = tj;
      }
      if (ti == tj && (job < 10 || job >= 20) && (c >> 2) == q4) {
        (job < 10 ? sm.ssk : sm.ssq)[16 * ti + c] = acc[c & 3];
      }
    }
    __syncthreads();

    // ---- per-token factors (wave 0): norms, fp64 cumulative decay, scales
    if (wave == 0) {
      const float rkv = a.use_l2 ? 1.f / sqrtf(sm.ssk[lane] + a.eps) : 1.f;
      const float rqv = a.use_l2 ? 1.f / sqrtf(sm.ssq[lane] + a.eps) : 1.f;
      double G = (double)sm.gin[lane];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(G, off, 64);
        if (lane >= off) G += o;
      }
      const float g2 = (float)(G * 1.4426950408889634);
      const float g2L = __shfl(g2, 63, 64);
      const float eG = exp2f(g2);
      const float bv = sm.bin[lane];
      sm.G2[lane] = g2;
      sm.rk[lane] = rkv;
      sm.ar[lane] = bv * rkv;
      sm.pr[lane] = a.scale * rqv;
      sm.bt[lane] = bv;
      sm.xr[lane] = bv * eG * rkv;
      sm.yq[lane] = a.scale * rqv * eG;
      sm.cL[lane] = rkv * exp2f(g2L - g2);
      if (lane == 0) sm.eGL = exp2f(g2L);
    }
    __syncthreads();

    // ---- scale Gram tiles into A (fp32) and P (hi/lo bf16)
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int job = wave + kNW * u;
      if (job >= 20) break;
      const int ti = gti[u], tj = gtj[u];
      const int i = 16 * ti + c, j0 = 16 * tj + 4 * q4;
      const float g2i = sm.G2[i];
      const f32x4 g2j = *reinterpret_cast<const f32x4*>(&sm.G2[j0]);
      const f32x4 rkj = *reinterpret_cast<const f32x4*>(&sm.rk[j0]);
      const float rowf = job < 10 ? sm.ar[i] : sm.pr[i];
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + e;
        const bool keep = job < 10 ? (j < i) : (j <= i);
        val[e] = keep ? rowf * rkj[e] * exp2f(g2i - g2j[e]) * gacc[u][e] : 0.f;
      }
      if (job < 10) {
        *reinterpret_cast<f32x4*>(&sm.A[i][j0]) = val;
      } else {
        u32x2 hi, lo;
        split4(val, hi, lo);
        const int pj = perm32(j0);
        *reinterpret_cast<u32x2*>(&sm.Ph[i][pj]) = hi;
        *reinterpret_cast<u32x2*>(&sm.Pl[i][pj]) = lo;
      }
    }
    // zero the above-diagonal tiles (0,1) and (2,3) that 32-wide steps read
    if (wave < 2) {
      const int i = 32 * wave + c, pj = perm32(32 * wave + 16 + 4 * q4);
      *reinterpret_cast<u32x2*>(&sm.Ph[i][pj]) = u32x2{0u, 0u};
      *reinterpret_cast<u32x2*>(&sm.Pl[i][pj]) = u32x2{0u, 0u};
      *reinterpret_cast<f32x4*>(&sm.Tf[i][32 * wave + 16 + 4 * q4]) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution
    // (wave w inverts block w; lane c < 16 computes column c)
    if (lane < 16) {
      const int b = wave;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        const float* arow = &sm.A[16 * b + r][16 * b];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int m4 = 0; m4 < r; m4 += 4) {
          const f32x4 av = *reinterpret_cast<const f32x4*>(arow + m4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (m4 + e < r) {
              if (e & 1) s1 += av[e] * x[m4 + e];
              else s0 += av[e] * x[m4 + e];
            }
        }
        x[r] = (r > c) ? -(s0 + s1) : x[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Tf[16 * b + r][16 * b + c] = x[r];
    }
    __syncthreads();
    // level 1: T_{p+1,p} = -T_{p+1,p+1} (A_{p+1,p} T_{p,p}), p = 0, 32 (waves 0, 1)
    if (wave < 2) {
      const int p = 32 * wave;
      const f32x4 y = tile_mm_f32<16>(&sm.A[p + 16][p], kC + 4, &sm.Tf[p][p], kC + 4, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Ys[16 * wave + 4 * q4 + i4][c] = y[i4];
    }
    __syncthreads();
    if (wave < 2) {
      const int p = 32 * wave;
      const f32x4 t = tile_mm_f32<16>(&sm.Tf[p + 16][p + 16], kC + 4, &sm.Ys[16 * wave][0], 36, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Tf[p + 16 + 4 * q4 + i4][p + c] = -t[i4];
    }
    __syncthreads();
    // level 2: T_{2:4,0:2} = -T_{2:4,2:4} (A_{2:4,0:2} T_{0:2,0:2}), one 16x16 tile per wave
    {
      const int yi = wave >> 1, yj = wave & 1;
      const f32x4 y = tile_mm_f32<32>(&sm.A[32 + 16 * yi][0], kC + 4, &sm.Tf[0][16 * yj], kC + 4, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Ys[16 * yi + 4 * q4 + i4][16 * yj + c] = y[i4];
    }
    __syncthreads();
    {
      const int xi = wave >> 1, xj = wave & 1;
      const f32x4 t = tile_mm_f32<32>(&sm.Tf[32 + 16 * xi][32], kC + 4, &sm.Ys[0][16 * xj], 36, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Tf[32 + 16 * xi + 4 * q4 + i4][16 * xj + c] = -t[i4];
    }
    __syncthreads();
    // T to hi/lo bf16 over the lower 32x32-block triangle (the upper parts of
    // the diagonal blocks are zero and are read by 32-wide steps)
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int gidx = tid + kNT * k;  // 768 groups of 4: rows 0..31 x 8, rows 32..63 x 16
      int i, j0;
      if (gidx < 256) {
        i = gidx >> 3;
        j0 = 4 * (gidx & 7);
      } else {
        i = 32 + ((gidx - 256) >> 4);
        j0 = 4 * ((gidx - 256) & 15);
      }
      u32x2 hi, lo;
      split4(*reinterpret_cast<const f32x4*>(&sm.Tf[i][j0]), hi, lo);
      const int pj = perm32(j0);
      *reinterpret_cast<u32x2*>(&sm.Th[i][pj]) = hi;
      *reinterpret_cast<u32x2*>(&sm.Tl[i][pj]) = lo;
    }

    // ---- prefetch the next chunk's inputs while this one finishes
    ChunkRegs nxt;
    const int c1 = c0 + kC;
    if (c1 < eos) {
      const int L1 = min(kC, eos - c1);
      if (L1 == kC) issue_loads<true>(nxt, a, c1, L1, kh, h, vcol, tid, lane, wave, q4);
      else issue_loads<false>(nxt, a, c1, L1, kh, h, vcol, tid, lane, wave, q4);
    }
    __syncthreads();

    // ---- state phase: this wave's 16 value channels
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
      const f32x4 btv = *reinterpret_cast<const f32x4*>(&sm.bt[16 * ti + 4 * q4]);
      const f32x4 xrv = *reinterpret_cast<const f32x4*>(&sm.xr[16 * ti + 4 * q4]);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) R[ti][i4] = btv[i4] * bf16_to_f32(vv[4 * ti + i4]) - xrv[i4] * acc[i4];
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
        if (2 * ks > ti) continue;
        acc = mfma3(lds8(&sm.Th[16 * ti + c][32 * ks + 8 * q4]), lds8(&sm.Tl[16 * ti + c][32 * ks + 8 * q4]),
                    rbh[ks], rbl[ks], acc);
      }
      Dl[ti] = acc;
    }
    bf16x8 dbh[2], dbl[2], dph[2], dpl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      split8(Dl[2 * ks], Dl[2 * ks + 1], dbh[ks], dbl[ks]);
      const f32x4 cl0 = *reinterpret_cast<const f32x4*>(&sm.cL[32 * ks + 4 * q4]);
      const f32x4 cl1 = *reinterpret_cast<const f32x4*>(&sm.cL[32 * ks + 16 + 4 * q4]);
      split8(Dl[2 * ks] * cl0, Dl[2 * ks + 1] * cl1, dph[ks], dpl[ks]);
    }

    // outputs O = yq * (Q S0^T) + P Delta
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 aq = lds8(&sm.Qr[16 * ti + c][32 * ks + 8 * q4]);
        y = mfma16x16x32(aq, sbh[ks], y);
        y = mfma16x16x32(aq, sbl[ks], y);
      }
      y = y * *reinterpret_cast<const f32x4*>(&sm.yq[16 * ti + 4 * q4]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (2 * ks > ti) continue;
        y = mfma3(lds8(&sm.Ph[16 * ti + c][32 * ks + 8 * q4]), lds8(&sm.Pl[16 * ti + c][32 * ks + 8 * q4]),
                  dbh[ks], dbl[ks], y);
      }
      TO* op = og + ((size_t)(c0 + 16 * ti + 4 * q4) * a.Hv + h) * kD + vcol;
      const size_t ts = (size_t)a.Hv * kD;
      if (L == kC) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) store_from_f32(op + i4 * ts, y[i4]);
      } else {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          if (16 * ti + 4 * q4 + i4 < L) store_from_f32(op + i4 * ts, y[i4]);
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
    cur = nxt;
    __syncthreads();
  }

  if (a.final_state) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) *reinterpret_cast<f32x4*>(a.final_state + sbase + 16 * kt) = s[kt];
  }
}

template <typename TO>
hipError_t launch_bf16_t(const ChunkArgs& a, hipStream_t st) {
  auto kern = chunk_bf16_kernel<TO>;
  const size_t smem = sizeof(Smem);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(kD / kDVS, a.Hv, a.N), dim3(kNT), smem, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t st) {
  return a.out_bf16 ? launch_bf16_t<uint16_t>(a, st) : launch_bf16_t<float>(a, st);
}

}  // namespace gdr
