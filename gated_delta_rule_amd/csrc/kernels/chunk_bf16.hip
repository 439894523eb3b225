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
// Two kernels.  The part that does not depend on the state -- Gram matrices,
// q/k norms, decays, T and P -- is computed by chunk_prep_kernel, one
// workgroup per (chunk, key head) serving the key head's value heads in
// turn, all chunks of all sequences in parallel, into a caller-provided
// workspace.  chunk_rec_kernel then carries the state: one workgroup per
// (sequence, value head, 32 value channels), two state waves owning 16
// value channels each for the whole sequence, chunk after chunk:
// X = K S0^T, R, Delta = T R, S update; two output waves form O and two load
// waves stage the inputs (see chunk_rec_kernel).  The matrix-core output layout
// (lane l holds rows 4*(l/16)+i of column l%16) is fed back as the B operand
// of the next contraction by permuting the contraction index identically on
// both operands, so R, Delta and the state stay in registers; the shared A
// operands (K, Q, K^T, T, P) sit in LDS with their contraction index stored in
// that permuted order, so each fragment is one 16-byte read.  The next
// chunk's inputs are loaded while the current chunk's state phase runs.
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
constexpr int kNT = 256;  // threads per workgroup (4 waves)
constexpr int kDVS = 32;  // value channels per recurrence workgroup
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// Workspace record of one (chunk, value head), in bytes: T hi, T lo, P hi,
// P lo (each: rows 0..31 x 32 columns, then rows 32..63 x 64 columns, bf16,
// columns permuted), then token factors bt, xr, yq, cL (fp32 x 64 each) and
// e^{G_L}.
constexpr int kMatBytes = 6144;
constexpr int kFacOff = 4 * kMatBytes;
constexpr size_t kRecBytes = 25728;
// Workspace head: table[0..N] (chunk offsets of the sequences), then
// order[0..N-1] (sequences by falling chunk count, the recurrence's launch
// order).
constexpr size_t kTableBytes(int N) { return (((size_t)N * 2 + 1) * 4 + 255) / 256 * 256; }
constexpr int kOrderBins = 1024;  // chunk-count classes of the launch order

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
// Index of the first f32x4 piece of row r (1..15) of a 16x16 lower
// triangle read row by row, pieces m4 = 0, 4, .. < r.
__host__ __device__ constexpr int piece_base(int r) {
  int n = 0;
  for (int i = 1; i < r; ++i) n += (i + 3) / 4;
  return n;
}
// Element offset of (row i, physical column p) in a compact T/P matrix: rows
// 0..31 hold 32 columns (four 16-byte slots), rows 32..63 all 64 (eight);
// slot s of row i is stored at s ^ ((i >> 1) & 3), resp. s ^ (i & 7), so
// that the recurrence's fragment reads (lanes on 16 consecutive rows, one
// slot each) hit distinct LDS banks when the record is copied to LDS as is.
__device__ __forceinline__ int compact_idx(int i, int p) {
  return i < 32 ? i * 32 + 8 * ((p >> 3) ^ ((i >> 1) & 3)) + (p & 7)
                : 1024 + (i - 32) * 64 + 8 * ((p >> 3) ^ (i & 7)) + (p & 7);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads and stores (which __syncthreads() would also wait
// for), so loads and stores can stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// bf16 hi/lo of two fp32 values, packed: hi = rne(x), lo = rne(x - hi).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  bf16x2 h;
  h[0] = (__bf16)x0;
  h[1] = (__bf16)x1;
  hi = __builtin_bit_cast(uint32_t, h);
  // keep the packed conversion: the halves below come from it (one
  // instruction each) instead of a second conversion of x0
  asm("" : "+v"(hi));
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

// Sequence of chunk j and its token range [c0, c0 + L).
struct ChunkPos {
  int n, c0, L;
  bool valid;
};

__device__ __forceinline__ ChunkPos locate_chunk(const ChunkArgs& a, const int32_t* table, int j) {
  ChunkPos p;
  if (a.cu_seqlens) {
    if (j >= table[a.N]) { p.valid = false; return p; }
    int lo = 0, hi = a.N;  // table[lo] <= j < table[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (table[mid] <= j) lo = mid; else hi = mid;
    }
    p.n = lo;
    p.c0 = a.cu_seqlens[lo] + (j - table[lo]) * kC;
    p.L = min(kC, a.cu_seqlens[lo + 1] - p.c0);
  } else {
    const int per = (a.T + kC - 1) / kC;
    p.n = j / per;
    const int i = j - p.n * per;
    p.c0 = p.n * a.T + i * kC;
    p.L = min(kC, a.T - i * kC);
  }
  p.valid = true;
  return p;
}

// ---------------------------------------------------------------------------
// Chunk table: table[n] = number of chunks of sequences 0..n-1, and
// order[] = the sequences by falling chunk count (counts above
// kOrderBins - 1 share one class; order inside a class is whatever the LDS
// atomics give, which moves only the launch schedule, never a result).

__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* cu, int N, int32_t* table) {
  __shared__ int part[1024];
  __shared__ int hist[kOrderBins];
  const int t = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int n0 = min(N, t * per), n1 = min(N, n0 + per);
  auto nchunks = [&](int n) { return (cu[n + 1] - cu[n] + kC - 1) / kC; };
  auto bin = [&](int n) { return min(nchunks(n), kOrderBins - 1); };
  hist[t] = 0;
  int sum = 0;
  for (int n = n0; n < n1; ++n) sum += nchunks(n);
  part[t] = sum;
  __syncthreads();
  for (int n = n0; n < n1; ++n) atomicAdd(&hist[bin(n)], 1);
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  for (int n = n0; n < n1; ++n) {
    table[n] = run;
    run += nchunks(n);
  }
  if (t == 1023) table[N] = part[1023];
  // Start of class b in the order: sequences in classes above b.  Inclusive
  // scan of the classes taken from the top: part[i] = sum of hist[1023 - i'],
  // i' <= i.
  __syncthreads();
  part[t] = hist[kOrderBins - 1 - t];
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  hist[kOrderBins - 1 - t] = part[t] - hist[kOrderBins - 1 - t];  // exclusive start
  __syncthreads();
  int32_t* order = table + N + 1;
  for (int n = n0; n < n1; ++n) order[atomicAdd(&hist[bin(n)], 1)] = n;
}

// ---------------------------------------------------------------------------
// Chunk preparation: T = (I + A)^{-1}, P and token factors of every value
// head of one (chunk, key head).

// LDS of chunk_prep_kernel (35 KiB plus 512 B per value head of the key
// head, so four workgroups share a compute unit up to 8 value heads per key
// head): k and q rows are dead once the Gram tiles are in registers, so A and
// T reuse their space; the 16x16 and 32x32 products of the merges are staged
// in A's never-used upper right 32x32 block (rows 0..31, columns 32..63).
struct __align__(16) PrepSmem {
  union {
    uint16_t Kr[kC][kD + 8];  // k rows, columns permuted
    float A[kC][kC + 4];
  };
  union {
    uint16_t Qr[kC][kD + 8];  // q rows, columns permuted
    float Tf[kC][kC + 4];
  };
  float ssk[kC], ssq[kC];
  float rk[kC], pr[kC];
};  // followed in LDS by the per-head log2 decays and beta r_k, [G][64] each
static_assert(sizeof(PrepSmem) <= 40 * 1024, "four prepare workgroups per compute unit");
static_assert(sizeof(PrepSmem) + 2 * kChunkMaxHeadRatio * kC * sizeof(float) <= 160 * 1024,
              "the largest value-head ratio must fit the LDS of one compute unit");

__global__ __launch_bounds__(kNT, 4) void chunk_prep_kernel(ChunkArgs a, unsigned char* ws) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrepSmem& sm = *reinterpret_cast<PrepSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int c = lane & 15, q4 = lane >> 4;
  // Workgroup -> (chunk j, key head kh), spread over the XCDs in contiguous
  // runs.  The Gram tiles depend only on k and q, so they are formed once
  // and serve the G = Hv / Hk value heads of the key head in turn.
  const int total = (int)gridDim.x;
  int lin = blockIdx.x;
  if (total % kXcds == 0) lin = (lin % kXcds) * (total / kXcds) + lin / kXcds;
  const int j = lin / a.Hk, kh = lin % a.Hk;
  const int G = a.Hv / a.Hk;
  const int32_t* table = reinterpret_cast<const int32_t*>(ws);
  const ChunkPos pos = locate_chunk(a, table, j);
  if (!pos.valid) return;
  const int c0 = pos.c0, L = pos.L;
  // g and beta of token `lane` of value head kh*G + hh (zero past L)
  auto load_g = [&](int hh) { return lane < L ? a.g[(size_t)(c0 + lane) * a.Hv + kh * G + hh] : 0.f; };
  auto load_b = [&](int hh) { return lane < L ? a.beta[(size_t)(c0 + lane) * a.Hv + kh * G + hh] : 0.f; };
  // wave w's first head (w) now, so the loads run under the k/q loads and the Gram tiles
  const float g_first = wave < G ? load_g(wave) : 0.f, b_first = wave < G ? load_b(wave) : 0.f;
  float* G2h = reinterpret_cast<float*>(smem_raw + sizeof(PrepSmem));  // [G][64] log2 decays
  float* arh = G2h + G * kC;                                             // [G][64] beta r_k

  // ---- k, q rows to LDS with permuted columns
  {
    const uint16_t* src = static_cast<const uint16_t*>(tid < 128 ? a.k : a.q);
    uint16_t(*X)[kD + 8] = tid < 128 ? sm.Kr : sm.Qr;
    const int b = tid & 127, rb = b >> 4, cb = b & 15;
    const int pc = perm8(cb);
    // all eight k/q loads in flight before the LDS stores; rows past L read
    // row L-1 (in bounds) and are zeroed
    u32x4 w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(8 * rb + i, L - 1);
      w[i] = *reinterpret_cast<const u32x4*>(src + ((size_t)(c0 + row) * a.Hk + kh) * kD + 8 * cb);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * rb + i;
      const u32x4 v = row < L ? w[i] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x2*>(&X[row][pc]) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(&X[row][pc + 8]) = u32x2{v[2], v[3]};
    }
  }
  lds_barrier();

  // ---- Gram tiles (raw bf16 products): job 0..9 K_j K_i^T, 10..19 K_j Q_i^T,
  // 20..23 Q_i Q_i^T (diagonal only, for the q norms).  Lane holds
  // G[row i = 16 ti + c][cols j = 16 tj + 4 q4 .. +3].
  f32x4 gacc[5];
  int gti[5], gtj[5];
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int job = wave + 4 * u;
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
    if (ti == tj && (job < 10 || job >= 20) && (c >> 2) == q4) (job < 10 ? sm.ssk : sm.ssq)[16 * ti + c] = acc[c & 3];
  }
  lds_barrier();

  // ---- decays and factors of every value head, wave w taking heads w, w + 4, ...
  {
    const float rkv = a.use_l2 ? 1.f / sqrtf(sm.ssk[lane] + a.eps) : 1.f;
    const float rqv = a.use_l2 ? 1.f / sqrtf(sm.ssq[lane] + a.eps) : 1.f;
    if (wave == 0) {
      sm.rk[lane] = rkv;
      sm.pr[lane] = a.scale * rqv;
    }
    for (int hh = wave; hh < G; hh += kNT / 64) {
      float gv = hh == wave ? g_first : load_g(hh);
      const float bv = hh == wave ? b_first : load_b(hh);
      gv = gv < kMinLogDecay ? kMinLogDecay : gv;  // (a NaN stays NaN)
      // chunk-local cumulative log-decay, summed in fp64; kept as log2 (G * log2 e)
      double Gs = (double)gv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(Gs, off, 64);
        if (lane >= off) Gs += o;
      }
      const float g2 = (float)(Gs * 1.4426950408889634);
      const float g2L = __shfl(g2, 63, 64);
      const float eG = exp2f(g2);
      G2h[hh * kC + lane] = g2;
      arh[hh * kC + lane] = bv * rkv;
      float* facg = reinterpret_cast<float*>(ws + kTableBytes(a.N) + ((size_t)j * a.Hv + kh * G + hh) * kRecBytes +
                                             kFacOff);
      facg[lane] = bv;                           // bt
      facg[64 + lane] = bv * eG * rkv;           // xr
      facg[128 + lane] = a.scale * rqv * eG;     // yq
      facg[192 + lane] = rkv * exp2f(g2L - g2);  // cL
      if (lane == 0) facg[256] = exp2f(g2L);     // e^{G_L}
    }
  }
  lds_barrier();

  for (int hh = 0; hh < G; ++hh) {
    const int h = kh * G + hh;
    const float* G2 = G2h + hh * kC;
    const float* ar = arh + hh * kC;
    // every wave is done with the previous head's T (split below) before
    // this head rewrites A and T
    if (hh > 0) lds_barrier();
    unsigned char* rec = ws + kTableBytes(a.N) + ((size_t)j * a.Hv + h) * kRecBytes;
    uint16_t* Thg = reinterpret_cast<uint16_t*>(rec);
    uint16_t* Tlg = reinterpret_cast<uint16_t*>(rec + kMatBytes);
    uint16_t* Phg = reinterpret_cast<uint16_t*>(rec + 2 * kMatBytes);
    uint16_t* Plg = reinterpret_cast<uint16_t*>(rec + 3 * kMatBytes);
    // ---- scale Gram tiles into A (fp32, LDS) and P (hi/lo bf16, workspace)
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int job = wave + 4 * u;
      if (job >= 20) break;
      const int ti = gti[u], tj = gtj[u];
      const int i = 16 * ti + c, j0 = 16 * tj + 4 * q4;
      const float g2i = G2[i];
      const f32x4 g2j = *reinterpret_cast<const f32x4*>(&G2[j0]);
      const f32x4 rkj = *reinterpret_cast<const f32x4*>(&sm.rk[j0]);
      const float rowf = job < 10 ? ar[i] : sm.pr[i];
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = j0 + e;
        const bool keep = job < 10 ? (jj < i) : (jj <= i);
        // exponent <= 0 where kept; the hardware exp2 may flush results below
        // 2^-126 to zero, far under the precision these entries carry
        const float x = rowf * rkj[e] * __builtin_amdgcn_exp2f(g2i - g2j[e]) * gacc[u][e];
        val[e] = keep ? x : 0.f;
      }
      if (job < 10) {
        *reinterpret_cast<f32x4*>(&sm.A[i][j0]) = val;
      } else {
        u32x2 hi, lo;
        split4(val, hi, lo);
        const int off = compact_idx(i, perm32(j0));
        *reinterpret_cast<u32x2*>(Phg + off) = hi;
        *reinterpret_cast<u32x2*>(Plg + off) = lo;
      }
    }
    // zero the above-diagonal tiles (0,1) and (2,3) that 32-wide steps read
    if (wave < 2) {
      const int i = 32 * wave + c;
      const int off = compact_idx(i, perm32(32 * wave + 16 + 4 * q4));
      *reinterpret_cast<u32x2*>(Phg + off) = u32x2{0u, 0u};
      *reinterpret_cast<u32x2*>(Plg + off) = u32x2{0u, 0u};
      *reinterpret_cast<f32x4*>(&sm.Tf[i][32 * wave + 16 + 4 * q4]) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    lds_barrier();

    // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution
    // (wave w inverts block w; lane c < 16 computes column c)
    if (lane < 16) {
      const int b = wave;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
      // the 36 f32x4 pieces of the block's lower triangle (row r: m4 < r),
      // in order, each read one piece before its use (two or more ahead
      // spill under this kernel's 128-register budget)
      constexpr int kAhead = 1;
      constexpr int kPr[36] = {1, 2, 3, 4, 5, 5, 6, 6, 7, 7, 8, 8, 9, 9, 9, 10, 10, 10, 11, 11, 11, 12, 12, 12, 13, 13, 13, 13, 14, 14, 14, 14, 15, 15, 15, 15};
      constexpr int kPm[36] = {0, 0, 0, 0, 0, 4, 0, 4, 0, 4, 0, 4, 0, 4, 8, 0, 4, 8, 0, 4, 8, 0, 4, 8, 0, 4, 8, 12, 0, 4, 8, 12, 0, 4, 8, 12};
      f32x4 ring[kAhead + 1];
#pragma unroll
      for (int q = 0; q < kAhead; ++q) ring[q] = *reinterpret_cast<const f32x4*>(&sm.A[16 * b + kPr[q]][16 * b + kPm[q]]);
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int m4 = 0; m4 < r; m4 += 4) {
          const int q = piece_base(r) + m4 / 4;
          if (q + kAhead < 36)
            ring[(q + kAhead) % (kAhead + 1)] =
                *reinterpret_cast<const f32x4*>(&sm.A[16 * b + kPr[q + kAhead]][16 * b + kPm[q + kAhead]]);
          const f32x4 av = ring[q % (kAhead + 1)];
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
    lds_barrier();
    // level 1: T_{p+1,p} = -T_{p+1,p+1} (A_{p+1,p} T_{p,p}), p = 0, 32 (waves 0, 1)
    if (wave < 2) {
      const int p = 32 * wave;
      const f32x4 y = tile_mm_f32<16>(&sm.A[p + 16][p], kC + 4, &sm.Tf[p][p], kC + 4, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.A[16 * wave + 4 * q4 + i4][32 + c] = y[i4];
    }
    lds_barrier();
    if (wave < 2) {
      const int p = 32 * wave;
      const f32x4 t = tile_mm_f32<16>(&sm.Tf[p + 16][p + 16], kC + 4, &sm.A[16 * wave][32], kC + 4, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Tf[p + 16 + 4 * q4 + i4][p + c] = -t[i4];
    }
    lds_barrier();
    // level 2: T_{2:4,0:2} = -T_{2:4,2:4} (A_{2:4,0:2} T_{0:2,0:2}), one 16x16 tile per wave
    {
      const int yi = wave >> 1, yj = wave & 1;
      const f32x4 y = tile_mm_f32<32>(&sm.A[32 + 16 * yi][0], kC + 4, &sm.Tf[0][16 * yj], kC + 4, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.A[16 * yi + 4 * q4 + i4][32 + 16 * yj + c] = y[i4];
    }
    lds_barrier();
    {
      const int xi = wave >> 1, xj = wave & 1;
      const f32x4 t = tile_mm_f32<32>(&sm.Tf[32 + 16 * xi][32], kC + 4, &sm.A[0][32 + 16 * xj], kC + 4, c, q4);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) sm.Tf[32 + 16 * xi + 4 * q4 + i4][16 * xj + c] = -t[i4];
    }
    lds_barrier();
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
      const int off = compact_idx(i, perm32(j0));
      *reinterpret_cast<u32x2*>(Thg + off) = hi;
      *reinterpret_cast<u32x2*>(Tlg + off) = lo;
    }
  }  // value heads
}

// ---------------------------------------------------------------------------
// Recurrence: carries the state of 32 value channels of one (sequence,
// value head) through its chunks, with three kinds of wave per workgroup:
//   state waves 0, 1  own 16 channels each and run only the serial chain:
//                     X = K S0^T, R, Delta = T R, the state update;
//   output waves 2, 3 get S0 and Delta (bf16 hi/lo) from the state wave of
//                     the same channels through LDS and form and store
//                     O = yq * (Q S0^T) + P Delta off the chain;
//   load waves 4, 5   fetch each chunk's inputs into registers two chunks
//                     ahead and write them to LDS one chunk ahead.
// So the state waves never issue a global load or store.  Waves go to the
// four SIMDs in turn, so each state wave shares its SIMD with a load wave,
// which waits at barriers most of the time, rather than with a busy output
// wave.

constexpr int kRecNT = 384;  // threads per recurrence workgroup: 2 state + 2 output + 2 load waves

// One chunk's shared inputs in LDS (62 KiB; two buffers).  Every region is a
// whole number of 1 KiB blocks, so one 64-lane load of 16 bytes per lane
// fills one block:
//   K, Q (16 blocks each): 64 rows x 256 bytes; 16-byte slot s of row r is
//        kept at slot s ^ kqswz(r), which makes the row-strided fragment reads
//        and the transposing reads of the state phase conflict-free
//   M (24): the record's T hi, T lo, P hi, P lo, byte for byte (the record
//        itself is laid out for these reads, see compact_idx)
//   fac (2): bt, xr, yq, cL (fp32 x 64), then e^{G_L}
//   V (4): 64 token rows of this workgroup's 32 value channels
struct __align__(16) RecBuf {
  uint16_t K[kC][kD];
  uint16_t Q[kC][kD];
  unsigned char M[4 * kMatBytes];
  float fac[4][kC];
  float eGL[4];
  float pad_[252];
  uint16_t V[kC][kDVS];
};
static_assert(sizeof(RecBuf) == 62 * 1024, "RecBuf must be 62 KiB");
// State-to-output exchange, one per state wave: S0 hi/lo (8 fragments) and
// Delta hi/lo (4 fragments), 16 bytes per lane each, stored lane-major.
struct __align__(16) Xchg {
  u32x4 S[8][64];
  u32x4 D[4][64];
};
static_assert(sizeof(Xchg) == 12 * 1024, "Xchg must be 12 KiB");
constexpr int kRecLoads = 62;      // 1 KiB blocks per buffer
constexpr int kLoadsPerWave = 31;  // block i = lw + 2 jj, lw = load wave 0 or 1
constexpr int kBlkQ = 16, kBlkM = 32, kBlkF = 56, kBlkV = 58;  // region starts
static_assert(kBlkQ % 2 == 0 && kBlkM % 2 == 0 && kBlkF % 2 == 0 && kBlkV % 2 == 0,
              "a pair of blocks never straddles two regions");

// Slot swizzle of k / q row r.
__device__ __forceinline__ int kqswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// Per-lane parts of the load source offsets (bytes) of load wave lw.
struct RecLane {
  uint32_t slot0;   // (lane%16) ^ 4 (lane/16): k/q block b reads slot slot0 ^ (b%4) of row 4b + lane/16
  uint32_t lane16;  // 16 lane
  uint32_t fac;     // factor blocks: 16 lane (lw 0), 16 min(lane, 7) (lw 1: e^{G_L} only)
};

// Source of load wave lw's block jj of one chunk (block i = lw + 2 jj, lane
// `lane`).  kb, qb, vb point at row 0 of the chunk (k, q of the key head;
// this workgroup's v channels), rb at the chunk record.  Rows at or past L
// (a partial last chunk) repeat row L-1: they are never used, but must be
// finite.  Whole and partial chunks take the same code, so the load waves'
// loop has no branch around its loads.
__device__ __forceinline__ const unsigned char* rec_src(int jj, const unsigned char* kb, const unsigned char* qb,
                                                        const unsigned char* rb, const unsigned char* vb,
                                                        const RecLane& ln, int lw, int lane, int row_bytes,
                                                        int vrow_bytes, int L) {
  const int i = lw + 2 * jj;
  if (2 * jj < kBlkM) {  // k or q: block b covers rows 4b .. 4b+3
    const int b = 2 * jj < kBlkQ ? i : i - kBlkQ;
    const unsigned char* base = 2 * jj < kBlkQ ? kb : qb;
    const int row = min(4 * b + (lane >> 4), L - 1);
    return base + (size_t)row * row_bytes + 16 * (ln.slot0 ^ (uint32_t)(b & 3));
  }
  if (2 * jj < kBlkF) return rb + 1024 * (i - kBlkM) + ln.lane16;
  if (2 * jj < kBlkV) return rb + kFacOff + 1024 * lw + ln.fac;
  const int b = i - kBlkV;
  const int row = min(16 * b + (lane >> 2), L - 1);
  return vb + (size_t)row * vrow_bytes + 16 * (lane & 3);
}

// Load wave lw's blocks jj0..jj1-1 of one chunk into registers (each lane's 16
// bytes of block i go to LDS at 1024 i + 16 lane later, see rec_put).
__device__ __forceinline__ void rec_fetch(u32x4* stage, const unsigned char* kb, const unsigned char* qb,
                                          const unsigned char* rb, const unsigned char* vb, const RecLane& ln,
                                          int lw, int lane, int row_bytes, int vrow_bytes, int L, int jj0, int jj1) {
#pragma unroll
  for (int jj = 0; jj < kLoadsPerWave; ++jj)
    if (jj >= jj0 && jj < jj1)
      stage[jj] = *reinterpret_cast<const u32x4*>(rec_src(jj, kb, qb, rb, vb, ln, lw, lane, row_bytes, vrow_bytes, L));
}
__device__ __forceinline__ void rec_put(RecBuf* buf, const u32x4* stage, int lw, int lane, int jj0 = 0,
                                        int jj1 = kLoadsPerWave) {
#pragma unroll
  for (int jj = 0; jj < kLoadsPerWave; ++jj)
    if (jj >= jj0 && jj < jj1)
      *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(buf) + 1024 * (lw + 2 * jj) + 16 * lane) = stage[jj];
}

// Output stores of tiles ti0..ti1-1 of one chunk: Ot[ti][i] is the output of
// token 16 ti + c at value channel 4 q4 + i of this wave's 16, so each lane
// stores 4 adjacent channels; `op` points at token c, channel 4 q4 of the
// chunk, `ts` is the token stride in elements; tokens at or past L are skipped.
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(uint16_t* p, const f32x4& v) {
  *reinterpret_cast<u16x4*>(p) = u16x4{f32_to_bf16(v[0]), f32_to_bf16(v[1]), f32_to_bf16(v[2]), f32_to_bf16(v[3])};
}
template <typename TO>
__device__ __forceinline__ void store_out(TO* op, size_t ts, const f32x4* Ot, int L, int c, int ti0, int ti1) {
#pragma unroll
  for (int ti = ti0; ti < ti1; ++ti)
    if (L == kC || 16 * ti + c < L) store4(op + (size_t)(16 * ti) * ts, Ot[ti]);
}

// bf16x8 fragment from two transposing LDS reads at byte offsets o0, o1 of
// the buffer (see ds_read_b64_tr_b16).
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* base, int o0, int o1) {
  const v4i16 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + o0));
  const v4i16 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(base + o1));
  const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
  return __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
}

// State update of one chunk for this wave's 16 value channels:
// S^T <- e^{G_L} S^T + K^T Delta'.  Output tile kt = 2 ks + hh holds key
// channels 32 ks + 8 q4 + 4 hh + i, so that two tiles side by side give each
// lane 8 adjacent key channels (one 16-byte k fragment read in the next
// chunk).  The K^T fragments come from transposing reads of the k tile:
// lane (c, q4) of the 16-lane group reads row 4 q4 + c/4 (+16, +32 ks2) at
// key channels 32 ks + 8 (c%4) + 4 hh .. +3; tro[ks] holds the swizzled byte
// offset of that piece without the row terms common to all lanes.
__device__ __forceinline__ void state_update(f32x4* s, const RecBuf& B, const bf16x8* dph, const bf16x8* dpl,
                                             const int* tro) {
  const float eGL = B.eGL[0];
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(&B.K[0][0]);
  // fragments of tile kt + 1 are read while tile kt multiplies
  auto frag = [&](int kt, int ks2) {
    const int o = tro[kt >> 1] + 8 * (kt & 1) + 256 * 32 * ks2;
    return tr_frag(kbase, o, o + 256 * 16);
  };
  bf16x8 f[2][2];
  f[0][0] = frag(0, 0);
  f[0][1] = frag(0, 1);
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    if (kt < 7) {
      f[(kt + 1) & 1][0] = frag(kt + 1, 0);
      f[(kt + 1) & 1][1] = frag(kt + 1, 1);
    }
    f32x4 acc = s[kt] * eGL;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      acc = mfma16x16x32(f[kt & 1][ks2], dph[ks2], acc);
      acc = mfma16x16x32(f[kt & 1][ks2], dpl[ks2], acc);
    }
    s[kt] = acc;
  }
}

template <typename TO>
__global__ __launch_bounds__(kRecNT) void chunk_rec_kernel(ChunkArgs a, const unsigned char* ws) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  RecBuf* bufs = reinterpret_cast<RecBuf*>(smem_raw);

  Xchg* xch = reinterpret_cast<Xchg*>(smem_raw + 2 * sizeof(RecBuf));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int role = wv >> 1;  // 0 state, 1 output, 2 load
  const int wave = wv & 1;   // channel group of a state/output wave, or load wave index lw
  const int c = lane & 15, q4 = lane >> 4;
  // Workgroup -> (sequence, value head, slice).  A unit is the G workgroups
  // of one (sequence, key head): every value head of the key head and every
  // slice, all reading the same k and q.  Workgroup ids go round-robin to the
  // 8 XCDs (each with its own L2), so id = 8 * (G * w + m) + x runs member m
  // of the x-th unit of dispatch wave w on XCD x, and a unit never straddles
  // two L2s.  Units go out longest sequence first (the table's order), which
  // spreads a long sequence over every XCD and lets the short ones fill in
  // behind it.
  const int nslice = kD / kDVS, G = (a.Hv / a.Hk) * nslice;
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int u = (loc / G) * kXcds + xcd;
  if (u >= a.N * a.Hk) return;
  const int kh = u % a.Hk, m = loc % G;
  const int n = a.cu_seqlens ? reinterpret_cast<const int32_t*>(ws)[a.N + 1 + u / a.Hk] : u / a.Hk;
  const int h = kh * (a.Hv / a.Hk) + m / nslice, slice = m % nslice;
  const int vcol = slice * kDVS + 16 * wave + c;  // this lane's value channel
  int bos, eos, jb;
  if (a.cu_seqlens) {
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
    jb = reinterpret_cast<const int32_t*>(ws)[n];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
    jb = n * ((a.T + kC - 1) / kC);
  }
  const unsigned char* recs = ws + kTableBytes(a.N) + (size_t)h * kRecBytes;
  const size_t rstride = (size_t)a.Hv * kRecBytes;
  const size_t kqts = (size_t)a.Hk * kD;  // token stride of k and q (elements)
  const size_t vts = (size_t)a.Hv * kD;   // token stride of v and o
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (size_t)kh * kD;
  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + (size_t)kh * kD;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (size_t)h * kD + slice * kDVS;
  TO* og = static_cast<TO*>(a.o) + ((size_t)(bos + c) * a.Hv + h) * kD + slice * kDVS + 16 * wave + 4 * q4;
  const int row_bytes = (int)(kqts * 2), vrow_bytes = (int)(vts * 2);

  RecLane ln;
  ln.slot0 = (uint32_t)((lane & 15) ^ (4 * (lane >> 4)));
  ln.lane16 = 16 * lane;
  ln.fac = wave ? 16 * min(lane, 7) : 16 * lane;
  // LDS byte offsets of this lane's fragment reads (see RecBuf and the
  // record layout).  xo[ks]: k/q row 16 ti + c (ti added as 4096 ti), key
  // channels 32 ks + 8 q4 .. +7.  mA: T/P rows 16 ti + c < 32, columns
  // 8 q4 .. +7; mB[ks]: rows >= 32, columns 32 ks + 8 q4 .. +7.
  int xo[4], tro[4];
  const int fx = kqswz(c);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    xo[ks] = 256 * c + 16 * ((4 * ks + q4) ^ fx);
    tro[ks] = 256 * (4 * q4 + (c >> 2)) + 16 * (4 * (ks ^ (c >> 2)) + ((c & 3) ^ q4));
  }
  const int mA = 64 * c + 16 * (q4 ^ ((c >> 1) & 3));
  const int mB0 = 2048 + 128 * c + 16 * (q4 ^ (c & 7));
  const int mB1 = 2048 + 128 * c + 16 * ((4 + q4) ^ (c & 7));
  const int vto = 64 * (4 * q4 + (c >> 2)) + 2 * (16 * wave + 4 * (c & 3));

  // State S^T tiles: tile 2 ks + hh, lane holds S[vcol][32 ks + 8 q4 + 4 hh + i].
  f32x4 s[8];
  const size_t sbase = ((size_t)n * a.Hv + h) * kD * kD + (size_t)vcol * kD + 8 * q4;
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
    s[kt] = a.initial_state
                ? *reinterpret_cast<const f32x4*>(a.initial_state + sbase + 32 * (kt >> 1) + 4 * (kt & 1))
                : f32x4{0.f, 0.f, 0.f, 0.f};

  if (role == 2) {
    // Load waves.  Chunk j+1 goes into the buffer of chunk j-1, in two parts:
    //   after the first barrier of iteration j (the other waves are then done
    //   with that buffer): its k, q and v, which the state waves read right
    //   after the second barrier;
    //   after the second barrier: its record and factors, first read after
    //   the first barrier of iteration j+1 (T and factors, state waves) and
    //   after its second (P, output waves).
    // Each part's global loads for chunk j+2 are issued right after its put,
    // so their latency is hidden behind a whole iteration.
    u32x4 stage[kLoadsPerWave];
    auto fetch = [&](int cc, int jc, int jj0, int jj1) {
      const int Lc = min(kC, eos - cc);
      const unsigned char* nk = reinterpret_cast<const unsigned char*>(kg + (size_t)cc * kqts);
      const unsigned char* nq = reinterpret_cast<const unsigned char*>(qg + (size_t)cc * kqts);
      const unsigned char* nv = reinterpret_cast<const unsigned char*>(vg + (size_t)cc * vts);
      const unsigned char* nr = recs + (size_t)jc * rstride;
      rec_fetch(stage, nk, nq, nr, nv, ln, wave, lane, row_bytes, vrow_bytes, Lc, jj0, jj1);
      __builtin_amdgcn_sched_barrier(0);  // keep the groups in issue order
    };
    // jj ranges: k, q [0, kKQV); record [kKQV, kVj); factors kVj - 1; v [kVj, end)
    constexpr int kKQV = kBlkM / 2, kVj = kBlkV / 2;
    // Every iteration issues the same loads in the same order -- v, k and q,
    // then record and factors -- with chunks past the last one clamped to it
    // (loaded, put into the dead buffer, never read).  With no branch around
    // the loads the compiler counts the loads in flight exactly across
    // iterations, so no put waits for a load issued after it (with branches,
    // the put after the second barrier waited for the k, q and v loads
    // issued just before that barrier).
    const int last_c = bos + ((eos - bos - 1) / kC) * kC, last_j = jb + (eos - bos - 1) / kC;
    if (bos < eos) {
      fetch(bos, jb, 0, kLoadsPerWave);
      rec_put(bufs, stage, wave, lane);
      const int c1 = min(bos + kC, last_c), j1 = min(jb + 1, last_j);
      fetch(c1, j1, kVj, kLoadsPerWave);
      fetch(c1, j1, 0, kKQV);
      fetch(c1, j1, kKQV, kVj);
    }
    lds_barrier();
    int it = 0;
    for (int c0 = bos, j = jb; c0 < eos; c0 += kC, ++j, ++it) {
      lds_barrier();
      RecBuf* nb = bufs + ((it & 1) ^ 1);
      const int c2 = min(c0 + 2 * kC, last_c), j2 = min(j + 2, last_j);
      rec_put(nb, stage, wave, lane, 0, kKQV);
      rec_put(nb, stage, wave, lane, kVj, kLoadsPerWave);
      fetch(c2, j2, kVj, kLoadsPerWave);
      fetch(c2, j2, 0, kKQV);
      lds_barrier();
      rec_put(nb, stage, wave, lane, kKQV, kVj);
      fetch(c2, j2, kKQV, kVj);
    }
    return;
  }
  if (role == 0) {
    u32x4* k1 = reinterpret_cast<u32x4*>(&bufs[1].K[0][0]);
#pragma unroll
    for (int r = 0; r < 8; ++r) k1[(8 * wave + r) * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
  }
  lds_barrier();

  // Delta = T R and P Delta need the six nonzero 32-wide steps of the block
  // lower triangle, (ti, ks) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
  auto mrd = [&](const unsigned char* bb, int m, int ti, int ks) {
    const int o = ti < 2 ? mA + 1024 * ti : (ks ? mB1 : mB0) + 2048 * (ti - 2);
    return lds8(reinterpret_cast<const uint16_t*>(bb + offsetof(RecBuf, M) + m * kMatBytes + o));
  };
  Xchg& X = xch[wave];

  if (role == 1) {
    // Output waves: O^T = yq * (S0 Q^T) + Delta^T P^T for the channels of
    // state wave `wave`, transposed so each lane stores 4 adjacent channels.
    int it = 0;
    for (int c0 = bos; c0 < eos; c0 += kC, ++it) {
      const int L = min(kC, eos - c0);
      const unsigned char* bb = reinterpret_cast<const unsigned char*>(&bufs[it & 1]);
      const RecBuf& B = bufs[it & 1];
      lds_barrier();  // S0 of this chunk is in the exchange
      bf16x8 sbh[4], sbl[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sbh[ks] = __builtin_bit_cast(bf16x8, X.S[ks][lane]);
        sbl[ks] = __builtin_bit_cast(bf16x8, X.S[4 + ks][lane]);
      }
      lds_barrier();  // Delta of this chunk is in the exchange
      // Y^T (token 16 ti + c) and the outputs, after the second barrier: the
      // chunk's q, P and factors stay in LDS until the next first barrier
      f32x4 Y[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 aq = lds8(reinterpret_cast<const uint16_t*>(bb + offsetof(RecBuf, Q) + xo[ks] + 4096 * ti));
          y = mfma16x16x32(sbh[ks], aq, y);
          y = mfma16x16x32(sbl[ks], aq, y);
        }
        Y[ti] = y * B.fac[2][16 * ti + c];
      }
      bf16x8 ph[6], pl[6];
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int ti = u < 2 ? u : 2 + (u - 2) / 2, ks = u < 2 ? 0 : (u - 2) % 2;
        ph[u] = mrd(bb, 2, ti, ks);
        pl[u] = mrd(bb, 3, ti, ks);
      }
      bf16x8 dbh[2], dbl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dbh[ks] = __builtin_bit_cast(bf16x8, X.D[ks][lane]);
        dbl[ks] = __builtin_bit_cast(bf16x8, X.D[2 + ks][lane]);
      }
      f32x4 O[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 y = Y[ti];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (2 * ks > ti) continue;
          const int u = ti < 2 ? ti : 2 + 2 * (ti - 2) + ks;
          y = mfma3(dbh[ks], dbl[ks], ph[u], pl[u], y);
        }
        O[ti] = y;
      }
      store_out(og + (size_t)(c0 - bos) * vts, vts, O, L, c, 0, 4);
    }
    return;
  }

  // State waves.  The transposing LDS reads (state update, v) are safe from
  // the compiler's wait for outstanding vector memory operations: these waves
  // issue none.  Iteration j runs the state update of chunk j-1 (k^T from
  // chunk j-1's buffer) fused with chunk j's X = K S0^T, one 32-wide key step
  // at a time: update state tiles 2 ks and 2 ks + 1, split them to bf16
  // hi/lo (also for the output waves), multiply them into X.  So the matrix
  // core has independent work while each step's split runs.
  // Before the first chunk there is no previous one: its state update must
  // leave S as it is, so Delta' starts at zero and the k tile of the unused
  // second buffer is zero-filled (the load waves first write that buffer
  // after the first barrier).
  bf16x8 dph[2], dpl[2];  // Delta' of the previous chunk, for its state update
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    dph[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    dpl[ks] = dph[ks];
  }
  int it = 0;
  for (int c0 = bos; c0 < eos; c0 += kC, ++it) {
    RecBuf& B = bufs[it & 1];
    RecBuf* NB = bufs + ((it & 1) ^ 1);  // chunk j-1's inputs, then chunk j+1's
    const unsigned char* bb = reinterpret_cast<const unsigned char*>(&B);
    const unsigned char* nkb = reinterpret_cast<const unsigned char*>(&NB->K[0][0]);
    // v[16 ti + 4 q4 + e][vcol], e = 0..3, one transposing read per tile
    v4i16 vt[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
      vt[ti] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_ptr)(reinterpret_cast<const unsigned char*>(&B.V[0][0]) + vto + 1024 * ti));
    // fragments of key step ks: k rows of the 4 token tiles (X), and k^T of
    // state tiles 2 ks, 2 ks + 1 for both 32-token halves (state update)
    auto rd_k = [&](int ks, bf16x8* fk) {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        fk[ti] = lds8(reinterpret_cast<const uint16_t*>(bb + offsetof(RecBuf, K) + xo[ks] + 4096 * ti));
    };
    auto rd_kt = [&](int ks, bf16x8* ft) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // u = 2 hh + ks2
        const int o = tro[ks] + 8 * (u >> 1) + 256 * 32 * (u & 1);
        ft[u] = tr_frag(nkb, o, o + 256 * 16);
      }
    };
    const float eGL = it > 0 ? NB->eGL[0] : 1.f;
    bf16x8 fk[2][4], ft[2][4];
    rd_k(0, fk[0]);
    rd_kt(0, ft[0]);
    f32x4 Xa[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
        rd_k(ks + 1, fk[(ks + 1) & 1]);
        rd_kt(ks + 1, ft[(ks + 1) & 1]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 acc = s[2 * ks + hh] * eGL;
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          acc = mfma16x16x32(ft[ks & 1][2 * hh + ks2], dph[ks2], acc);
          acc = mfma16x16x32(ft[ks & 1][2 * hh + ks2], dpl[ks2], acc);
        }
        s[2 * ks + hh] = acc;
      }
      bf16x8 sbh, sbl;
      split8(s[2 * ks], s[2 * ks + 1], sbh, sbl);
      X.S[ks][lane] = __builtin_bit_cast(u32x4, sbh);
      X.S[4 + ks][lane] = __builtin_bit_cast(u32x4, sbl);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        Xa[ti] = mfma16x16x32(fk[ks & 1][ti], sbh, Xa[ti]);
        Xa[ti] = mfma16x16x32(fk[ks & 1][ti], sbl, Xa[ti]);
      }
    }
    lds_barrier();  // done with chunk j-1's buffer; S0 is in the exchange

    bf16x8 th[6], tl[6];
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int ti = u < 2 ? u : 2 + (u - 2) / 2, ks = u < 2 ? 0 : (u - 2) % 2;
      th[u] = mrd(bb, 0, ti, ks);
      tl[u] = mrd(bb, 1, ti, ks);
    }
    f32x4 R[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const f32x4 btv = *reinterpret_cast<const f32x4*>(&B.fac[0][16 * ti + 4 * q4]);
      const f32x4 xrv = *reinterpret_cast<const f32x4*>(&B.fac[1][16 * ti + 4 * q4]);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        R[ti][i4] = btv[i4] * __uint_as_float((uint32_t)(uint16_t)vt[ti][i4] << 16) - xrv[i4] * Xa[ti][i4];
    }
    bf16x8 rbh[2], rbl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) split8(R[2 * ks], R[2 * ks + 1], rbh[ks], rbl[ks]);

    // Delta = T R (block lower triangular: steps above the diagonal skipped)
    f32x4 Dl[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (2 * ks > ti) continue;
        const int u = ti < 2 ? ti : 2 + 2 * (ti - 2) + ks;
        acc = mfma3(th[u], tl[u], rbh[ks], rbl[ks], acc);
      }
      Dl[ti] = acc;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 dbh, dbl;
      split8(Dl[2 * ks], Dl[2 * ks + 1], dbh, dbl);
      X.D[ks][lane] = __builtin_bit_cast(u32x4, dbh);
      X.D[2 + ks][lane] = __builtin_bit_cast(u32x4, dbl);
      const f32x4 cl0 = *reinterpret_cast<const f32x4*>(&B.fac[3][32 * ks + 4 * q4]);
      const f32x4 cl1 = *reinterpret_cast<const f32x4*>(&B.fac[3][32 * ks + 16 + 4 * q4]);
      split8(Dl[2 * ks] * cl0, Dl[2 * ks + 1] * cl1, dph[ks], dpl[ks]);
    }
    lds_barrier();  // Delta is in the exchange; the next chunk's inputs are in LDS
  }
  if (it > 0) state_update(s, bufs[(it - 1) & 1], dph, dpl, tro);

  if (a.final_state) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      *reinterpret_cast<f32x4*>(a.final_state + sbase + 32 * (kt >> 1) + 4 * (kt & 1)) = s[kt];
  }
}

template <typename TO>
hipError_t launch_rec_t(const ChunkArgs& a, const unsigned char* ws, hipStream_t st) {
  auto kern = chunk_rec_kernel<TO>;
  const size_t smem = 2 * sizeof(RecBuf) + 2 * sizeof(Xchg);  // 148 KiB: double-buffered inputs + exchange
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int units = a.N * a.Hk, G = (a.Hv / a.Hk) * (kD / kDVS);
  const unsigned grid = (unsigned)((units + kXcds - 1) / kXcds * kXcds * G);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kRecNT), smem, st, a, ws);
  return hipGetLastError();
}

size_t max_chunks(const ChunkArgs& a) {
  const size_t per = ((size_t)a.T + kC - 1) / kC;
  return a.cu_seqlens ? per + (size_t)a.N : per * (size_t)a.N;
}

}  // namespace

size_t chunk_bf16_workspace_bytes(const ChunkArgs& a) {
  return kTableBytes(a.N) + max_chunks(a) * (size_t)a.Hv * kRecBytes;
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, void* workspace, hipStream_t st, int stages) {
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (!(stages & kStagePrepare)) return a.out_bf16 ? launch_rec_t<uint16_t>(a, ws, st) : launch_rec_t<float>(a, ws, st);
  if (a.cu_seqlens) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.N,
                       reinterpret_cast<int32_t*>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t nch = max_chunks(a);
  if (nch > 0) {
    const size_t smem = sizeof(PrepSmem) + 2 * (size_t)(a.Hv / a.Hk) * kC * sizeof(float);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_prep_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)(nch * a.Hk)), dim3(kNT), smem, st, a, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & kStageRecur)) return hipSuccess;
  return a.out_bf16 ? launch_rec_t<uint16_t>(a, ws, st) : launch_rec_t<float>(a, ws, st);
}

}  // namespace gdr
