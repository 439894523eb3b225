// The global attention layer of the hybrid decoder: grouped-query attention
// with an RMS norm on q and k, rotary encoding on the first 64 dims of each
// head and a sigmoid gate on the output (deepmagic page, architecture
// section: 24 query / 4 key-value heads, head dim 256, q/k RMS norm, sigmoid
// output gate, rotary encoding on the first quarter of each head with base
// 1e7; kongchang page, attention details).
//
// Prefill, three launches:
//   attn_table_kernel  per-sequence offsets of 64-key chunks and 128-query
//                      blocks (prefix sums over cu_seqlens)
//   attn_prep_kernel   per token: RMS norm of every q and k head, rotation
//                      of dims (j, j + 32), j < 32; q to a bf16 buffer, k to a
//                      key buffer padded per sequence to whole 64-key chunks
//                      (and to the caller's KV cache)
//   attn_vt_kernel     V transposed per 64-key chunk (dims x keys)
//   attn_fwd_kernel    causal attention, one workgroup per (query head,
//                      128-query block), 32-key blocks through LDS
// The keys and V^T go to per-head buffers in the order the matrix cores
// read them (32-key tiles of 16 KiB, each made of 1 KiB fragments), so
// that both the copies into LDS and the reads out of it are contiguous.
// Decode: attn_prep_kernel (one row per sequence, at its cache position,
// appending k and v to the cache), attn_decode_kernel (split over the cached
// keys) and attn_combine_kernel (merges the splits, applies the gate).
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

constexpr int kAD = 256;      // head dim
constexpr int kRot = 64;      // rotated dims
constexpr int kQB = 128;      // queries per workgroup (4 waves x 32)
constexpr int kKB = 64;       // keys per block
constexpr int kXcds = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One 16-byte direct-to-LDS load per lane from the wave-uniform address
// base + voff (voff a per-lane byte offset): lane l's bytes land at LDS byte
// address lds_addr + 16 l.  No register receives data; waits are explicit.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
// A pointer every lane of the wave holds, moved to scalar registers.
__device__ __forceinline__ const void* wave_uniform(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Index of the sequence holding item i, given offsets off[0..N] (off[0] = 0,
// non-decreasing): the largest n < N with off[n] <= i.
__device__ __forceinline__ int find_seq(const int32_t* off, int N, int i) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Per-sequence offsets: table[n] = sum over m < n of ceil(L_m / 64) (key
// chunks), table[N + 1 + n] = sum of ceil(L_m / 128) (query blocks), n = 0..N.
__global__ __launch_bounds__(256) void attn_table_kernel(const int32_t* cu, int N, int32_t* table) {
  __shared__ int32_t s_c[256], s_q[256];
  const int tid = threadIdx.x;
  const int per = (N + 255) / 256, a = tid * per, b = min(a + per, N);
  int c = 0, q = 0;
  for (int n = a; n < b; ++n) {
    const int L = cu[n + 1] - cu[n];
    c += (L + kKB - 1) / kKB;
    q += (L + kQB - 1) / kQB;
  }
  s_c[tid] = c;
  s_q[tid] = q;
  __syncthreads();
  if (tid == 0) {
    int rc = 0, rq = 0;
    for (int i = 0; i < 256; ++i) {
      const int tc = s_c[i], tq = s_q[i];
      s_c[i] = rc;
      s_q[i] = rq;
      rc += tc;
      rq += tq;
    }
    table[N] = rc;
    table[N + 1 + N] = rq;
  }
  __syncthreads();
  c = s_c[tid];
  q = s_q[tid];
  for (int n = a; n < b; ++n) {
    table[n] = c;
    table[N + 1 + n] = q;
    const int L = cu[n + 1] - cu[n];
    c += (L + kKB - 1) / kKB;
    q += (L + kQB - 1) / kQB;
  }
}

// ---------------------------------------------------------------------------
// RMS norm + rotation of one token's heads.  One workgroup per token (prefill)
// or per sequence (decode, one new token at its cache position).  Waves take
// heads round-robin; lane l holds dims 4l .. 4l+3.
// Fragment order of the prefill's key and V^T buffers.  Each head holds
// kblocks tiles of 32 keys (16 KiB); 1 KiB fragment f of a tile is what
// lane l of the attention kernel's matrix-core operand holds, at byte 16 l:
//   keys: f = dims 16 f .. 16 f + 15; lane l = key l % 32, dims 16 f + 8 (l / 32) .. +7
//   V^T:  f = 2 dt + g; lane l = dim 32 dt + l % 32, slots 16 g + 8 (l / 32) .. +7
// (slots: the keys of a tile in the order the probabilities leave the score
// registers, kperm below).  key and slot count from the head's first padded key.
__host__ __device__ inline size_t kfrag_index(int h, int64_t kblocks, int64_t key, int d) {
  return (((size_t)h * kblocks + key / 32) * 16 + d / 16) * 512 + (((d >> 3) & 1) * 32 + key % 32) * 8 + (d & 7);
}
__host__ __device__ inline size_t vfrag_index(int h, int64_t kblocks, int64_t slot, int d) {
  const int s = (int)(slot % 32);
  return ((size_t)h * kblocks + slot / 32) * (32 * 256) +
         ((2 * (d >> 5) + (s >> 4)) * 64 + ((s >> 3) & 1) * 32 + (d & 31)) * 8 + (s & 7);
}

struct PrepArgs {
  const uint16_t *q, *k, *v;     // [rows, Hq | Hk, D] bf16
  const float *q_w, *k_w;        // [D]
  const int32_t* cu;             // prefill: cu_seqlens [N+1]; decode: NULL
  const int32_t* table;          // prefill: key-chunk offsets [N+1]
  const int32_t* cache_lens;     // decode: [N] position of the new token
  uint16_t* q_rot;               // [rows, Hq, D]
  uint16_t* k_pad;               // prefill: keys in fragment order (kfrag_index) or NULL
  uint16_t* k_rot;               // [rows, Hk, D] or NULL (the rotated k, unpadded)
  uint16_t *k_cache, *v_cache;   // [N, cache_len, Hk, D] and the blocked layout below, or NULL
  int rows, N, Hq, Hk, cache_len;
  int64_t kblocks;               // prefill: 32-key tiles per head in k_pad
  float eps;
  double base;
};

// Decode V cache [N, Hk, cache_len / 32, 256, 32]: key 32 b + k of dim d
// sits in block b, row d, at position vc_pos(k), so that the 8 keys one lane
// of the decode's value product needs -- {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}
// for lane group g -- are one 16-byte read, and a 16-row read is 1 KiB.
__host__ __device__ constexpr int vc_pos(int k) { return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3); }
__device__ __forceinline__ size_t vc_index(int n, int h, int Hk, int cache_len, int d, int key) {
  return ((((size_t)n * Hk + h) * (cache_len / 32) + (key >> 5)) * kAD + d) * 32 + vc_pos(key & 31);
}

__global__ __launch_bounds__(256) void attn_prep_kernel(PrepArgs a) {
  __shared__ float s_cos[kRot / 2], s_sin[kRot / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x;
  int n, pos;
  if (a.cu) {
    n = find_seq(a.cu, a.N, t);
    pos = t - a.cu[n];
  } else {
    n = t;
    pos = a.cache_lens[t];
  }
  // rows hh = wave + 4 k of this token (q heads, then k heads), up to 8 per
  // wave and pass; a pass loads all of its rows before it uses any, and the
  // first pass's loads go out before the rotary angles are formed
  const int rows = a.Hq + a.Hk;
  auto row_src = [&](int hh) {
    return hh < a.Hq ? a.q + ((size_t)t * a.Hq + hh) * kAD : a.k + ((size_t)t * a.Hk + (hh - a.Hq)) * kAD;
  };
  constexpr int kRowsPerPass = 8;
  // (rows past the last are clamped to it: loaded, never used)
  u16x4 raw[kRowsPerPass];
#pragma unroll
  for (int k = 0; k < kRowsPerPass; ++k)
    raw[k] = *reinterpret_cast<const u16x4*>(row_src(min(wave + 4 * k, rows - 1)) + 4 * lane);
  if (tid < kRot / 2) {
    // angle pos * base^(-2j/64) in fp64, reduced to [-pi, pi] before the
    // fp32 sine and cosine, so large positions keep their accuracy
    const double inv = pow(a.base, -2.0 * tid / kRot);
    const double ang = (double)pos * inv;
    const double two_pi = 6.283185307179586476925287;
    const float r = (float)(ang - two_pi * rint(ang / two_pi));
    s_cos[tid] = cosf(r);
    s_sin[tid] = sinf(r);
  }
  __syncthreads();
  // a decode row whose position lies outside the cache is a padding row: no cache write
  const bool to_cache = a.k_cache && pos >= 0 && pos < a.cache_len;
  for (int h0 = wave; h0 < rows; h0 += 4 * kRowsPerPass) {
    if (h0 != wave) {
#pragma unroll
      for (int k = 0; k < kRowsPerPass; ++k)
        raw[k] = *reinterpret_cast<const u16x4*>(row_src(min(h0 + 4 * k, rows - 1)) + 4 * lane);
    }
#pragma unroll
    for (int k = 0; k < kRowsPerPass; ++k) {
      const int hh = h0 + 4 * k;
      if (hh >= rows) break;
      const bool is_q = hh < a.Hq;
      const int h = is_q ? hh : hh - a.Hq;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = bf16_to_f32(raw[k][e]);
      float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      ss = group_sum<64>(ss);
      const float rn = 1.f / sqrtf(ss / kAD + a.eps);
      const float* w = is_q ? a.q_w : a.k_w;
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w + 4 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = x[e] * rn * wv[e];
      // rotation: lanes 0..7 hold dims 0..31 (first of each pair), lanes
      // 8..15 dims 32..63 (second); partner lane l ^ 8
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float o = __shfl_xor(x[e], 8, 64);
        y[e] = x[e];
        if (lane < 8) {
          const int j = 4 * lane + e;
          y[e] = x[e] * s_cos[j] - o * s_sin[j];
        } else if (lane < 16) {
          const int j = 4 * (lane - 8) + e;
          y[e] = x[e] * s_cos[j] + o * s_sin[j];
        }
      }
      const u32x2 out = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      if (is_q) {
        *reinterpret_cast<u32x2*>(a.q_rot + ((size_t)t * a.Hq + h) * kAD + 4 * lane) = out;
      } else {
        if (a.k_pad) {
          const size_t tp = (size_t)kKB * a.table[n] + pos;
          *reinterpret_cast<u32x2*>(a.k_pad + kfrag_index(h, a.kblocks, (int64_t)tp, 4 * lane)) = out;
        }
        if (a.k_rot) *reinterpret_cast<u32x2*>(a.k_rot + ((size_t)t * a.Hk + h) * kAD + 4 * lane) = out;
        if (to_cache) {
          const size_t c = ((size_t)n * a.cache_len + pos) * a.Hk + h;
          *reinterpret_cast<u32x2*>(a.k_cache + c * kAD + 4 * lane) = out;
          if (!a.cu) {
            // decode: the token's v into the blocked cache, one key column
            const u16x4 vv = *reinterpret_cast<const u16x4*>(a.v + ((size_t)t * a.Hk + h) * kAD + 4 * lane);
            uint16_t* vc = a.v_cache + vc_index(n, h, a.Hk, a.cache_len, 4 * lane, pos);
#pragma unroll
            for (int e = 0; e < 4; ++e) vc[32 * e] = vv[e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// V transposed per 64-key chunk into two 32-key tiles in fragment order
// (vfrag_index), keys in slot order kperm (within each group of 16 keys the
// middle two quarters swap), the order in which the attention kernel's
// probabilities come out of its score registers.  Keys past the sequence
// end are zero.
__device__ __forceinline__ int kperm(int i) {
  const int q = (i >> 2) & 3;
  return (i & ~12) | ((q == 1 ? 2 : q == 2 ? 1 : q) << 2);
}

__global__ __launch_bounds__(256) void attn_vt_kernel(const uint16_t* v, const int32_t* cu, const int32_t* table,
                                                      int N, int Hk, int64_t tpad, uint16_t* vt, uint16_t* v_cache,
                                                      int cache_len) {
  __shared__ uint16_t tile[kKB][kAD + 2];
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (c >= table[N]) return;
  const int n = find_seq(table, N, c);
  const int L = cu[n + 1] - cu[n], k0 = kKB * (c - table[n]);
  for (int i = tid; i < kKB * kAD / 4; i += 256) {
    const int key = i / (kAD / 4), d4 = i % (kAD / 4);
    u16x4 val = {0, 0, 0, 0};
    if (k0 + key < L) val = *reinterpret_cast<const u16x4*>(v + ((size_t)(cu[n] + k0 + key) * Hk + h) * kAD + 4 * d4);
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[key][4 * d4 + e] = val[e];
  }
  __syncthreads();
  const int d = tid;  // one dim (row of vt) per thread: 64 keys, 128 bytes
  uint16_t row[kKB];
#pragma unroll
  for (int s = 0; s < kKB; ++s) row[s] = tile[(s & ~15) | kperm(s & 15)][d];
#pragma unroll
  for (int s = 0; s < kKB; s += 8) {
    u16x8 pk;
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[e] = row[s + e];
    // slots s .. s + 7 of row d
    uint16_t* dst = vt + vfrag_index(h, tpad / 32, (int64_t)kKB * c + s, d);
    *reinterpret_cast<u16x8*>(dst) = pk;
  }
  if (v_cache) {
    // the blocked decode cache: this chunk's keys k0 .. k0+63 of row d (two
    // 32-key blocks), only positions inside the sequence and the cache
    const int kend = min(L, cache_len) - k0;
    if (kend >= kKB) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint16_t* vc = v_cache + vc_index(n, h, Hk, cache_len, d, k0 + 32 * b);  // position 0 of the block
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u16x8 pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) pk[e] = tile[32 * b + 4 * g + (e & 3) + 16 * (e >> 2)][d];
          *reinterpret_cast<u16x8*>(vc + 8 * g) = pk;
        }
      }
    } else {
      for (int s = 0; s < kend; ++s) v_cache[vc_index(n, h, Hk, cache_len, d, k0 + s)] = tile[s][d];
    }
  }
}

// ---------------------------------------------------------------------------
// Causal attention.  Workgroup: one query head, 128 queries of one sequence,
// 4 waves of 32 queries.  Keys go in blocks of 32 through four LDS stages
// (a K tile and a V^T tile of 16 KiB each, in fragment order), copied by
// direct-to-LDS loads, 1 KiB per instruction, three blocks ahead of their
// use.  A wave's operand reads are 1 KiB contiguous runs at fixed offsets.
// Per block j, one wave does
//   S^T(j+1) = K Q^T   16 MFMAs (32x32x16): lane l holds query l % 32 and 16
//                      of the block's keys (the other 16 are in lane l ^ 32),
//                      beside the exponentials of block j (VALU)
//   O^T += V^T P^T(j)  8 dim tiles x 2 key steps, P straight from the score
//                      registers (bf16), beside the mask and maximum of
//                      block j+1
// Softmax is online and in base 2: the running maximum is kept in scaled
// units, each probability is exp2(s * log2(e)/sqrt(d) - max) with the
// argument one fma, and the accumulator is rescaled only when the maximum
// grows by more than 8.
struct FwdArgs {
  const uint16_t *q_rot, *k_pad, *vt, *gate;
  const int32_t *cu, *table;
  uint16_t* out;
  int N, Hq, Hk;
  int64_t tpad;
  float scale_log2;  // log2(e) / sqrt(D)
};

constexpr float kRescale = 8.f;
constexpr int kFB = 32;    // keys per block
constexpr int kStg = 4;    // LDS stages

__device__ __forceinline__ void wait_vm8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }
__device__ __forceinline__ void wait_vm16() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }

__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(FwdArgs a) {
  __shared__ __align__(16) uint16_t sK[kStg][kFB * kAD], sV[kStg][kAD * kFB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.Hq / a.Hk;
  // workgroup -> (kv head, query block, member head); the G query heads of
  // one kv head and block run on one XCD; heaviest blocks (latest in their
  // sequence) first
  const int nqb = a.table[a.N + 1 + a.N];
  const int units = nqb * a.Hk;
  const int x = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int u = (loc / G) * kXcds + x, m = loc % G;
  if (u >= units) return;
  const int kvh = u % a.Hk, qb = nqb - 1 - u / a.Hk;
  const int h = kvh * G + m;
  const int32_t* qoff = a.table + a.N + 1;
  const int n = find_seq(qoff, a.N, qb);
  const int s0 = a.cu[n], L = a.cu[n + 1] - s0;
  const int q0 = kQB * (qb - qoff[n]);                 // first query of the block (in the sequence)
  const int qw = q0 + 32 * wave;                       // first query of this wave
  const int my_q = min(qw + (lane & 31), L - 1);       // this lane's query (rows past L repeat the last)
  const int last_q = min(q0 + kQB - 1, L - 1);
  const int nkb = last_q / kFB + 1;
  // first tile of the sequence in this kv head's key and V^T buffers
  const int64_t tile0 = (int64_t)kvh * (a.tpad / kFB) + (int64_t)kKB / kFB * a.table[n];

  // Q^T fragments (B operand): query my_q, dims 16 ks + 8 (l / 32) .. +7
  bf16x8 qf[16];
  {
    const uint16_t* qrow = a.q_rot + ((size_t)(s0 + my_q) * a.Hq + h) * kAD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
  }

  f32x16 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float mrun = -INFINITY, lsum = 0.f;

  const uint32_t ldsK = (uint32_t)(uintptr_t)(lds_ptr)(&sK[0][0]), ldsV = (uint32_t)(uintptr_t)(lds_ptr)(&sV[0][0]);
  // piece i (0..7) of the copy of key block jb (clamped to the last block,
  // so every iteration issues eight) into stage jb % 4: pieces 0..3 are the
  // K fragments 4 wave + i, pieces 4..7 the V^T fragments 4 wave + i - 4
  auto copy_piece = [&](int jb, int i) {
    const int st = jb % kStg;
    jb = min(jb, nkb - 1);
    const int f = 4 * wave + (i & 3);
    const uint16_t* g = (i < 4 ? a.k_pad : a.vt) + (tile0 + jb) * (kFB * kAD) + 512 * f;
    dma16(wave_uniform(g), 16 * lane, (i < 4 ? ldsK : ldsV) + (uint32_t)(st * kFB * kAD + 512 * f) * 2);
  };
  auto scores = [&](int jb, f32x16& s) {
    const uint16_t* K = sK[jb % kStg] + 8 * lane;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(K + 512 * ks), qf[ks], s, 0, 0, 0);
  };
  // mask block jb's (unscaled) scores in place and update the running
  // maximum; any_grow and alpha say whether and by how much O and lsum are
  // rescaled (lsum here, O before the block's value product)
  bool any_grow = false;
  float alpha = 1.f;
  auto mask_max = [&](int jb, f32x16& s) {
    const int lim = my_q - kFB * jb - 4 * (lane >> 5);  // largest key offset 8 (r / 4) + r % 4 this lane sees
    float bmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = 8 * (r >> 2) + (r & 3) <= lim ? s[r] : -INFINITY;
      s[r] = v;
      bmax = fmaxf(bmax, v);
    }
    // lanes l and l ^ 32 hold the two halves of the query's keys
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
    bmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
    const bool grow = bmax > mrun + kRescale;
    any_grow = __builtin_amdgcn_ballot_w64(grow) != 0;
    const float mnew = grow ? bmax : mrun;
    alpha = __builtin_amdgcn_exp2f(mrun - mnew);  // 1 where the maximum stays; 0 at the first block
    if (any_grow) lsum *= alpha;
    mrun = mnew;
  };

#pragma unroll
  for (int jb = 0; jb < kStg - 1; ++jb)
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_piece(jb, i);
  wait_vm16();
  __syncthreads();
  f32x16 sc;
  scores(0, sc);
  mask_max(0, sc);

  for (int j = 0; j < nkb; ++j) {
    wait_vm8();      // this wave's copy of block j+1 has landed (j+2 may be in flight)
    __syncthreads(); // ... and every wave's; every wave is done with block j-1's stage
    // (unconditional, so that these MFMAs share a basic block with the
    // exponentials below; after the last block it scores a clamped block
    // that is never used)
    f32x16 sn;
    scores(min(j + 1, nkb - 1), sn);
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_piece(j + kStg - 1, i);
    bf16x8 pf[2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      u16x8 pk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * uu + e], a.scale_log2, -mrun));
        lsum += p;
        pk[e] = f32_to_bf16(p);
      }
      pf[uu] = __builtin_bit_cast(bf16x8, pk);
    }
    // keep the exponentials in this basic block, beside the score MFMAs (the
    // compiler would otherwise sink them past the rescale branch)
    asm volatile("" : "+v"(pf[0]), "+v"(pf[1]), "+v"(lsum));
    if (any_grow) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
    }
    // O^T += V^T P^T: 8 dim tiles, 2 steps of 16 keys; the other half of
    // the copy goes out between them
    const uint16_t* V = sV[j % kStg] + 8 * lane;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(V + 512 * (2 * dt + g)), pf[g],
                                                        o[dt], 0, 0, 0);
      if (dt & 1) copy_piece(j + kStg - 1, 4 + (dt >> 1));
    }
    // the next block's mask and maximum (a block past the last is wholly
    // masked, so the final call changes nothing)
    mask_max(j + 1, sn);
    sc = sn;
  }
  wait_vm0();

  // out = O / l * sigmoid(gate): lane holds query my_q, dims 32 dt + 8 (r/4) + 4 (l/32) + r%4
  lsum += __shfl_xor(lsum, 32, 64);
  const float inv = 1.f / lsum;
  const int qi = qw + (lane & 31);
  if (qi < L) {
    const size_t base = ((size_t)(s0 + qi) * a.Hq + h) * kAD + 4 * (lane >> 5);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const size_t at = base + 32 * dt + 8 * g4;
        const u16x4 gr = *reinterpret_cast<const u16x4*>(a.gate + at);
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = bf16_to_f32(gr[e]);
          y[e] = o[dt][4 * g4 + e] * inv * (1.f / (1.f + __expf(-z)));
        }
        *reinterpret_cast<u32x2*>(a.out + at) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      }
  }
}

// ---------------------------------------------------------------------------
// Decode: one query token per sequence against its cache.  Each wave takes
// one split (256 .. 2048 keys) of one (sequence, kv head) and the G query
// heads that read it, with no LDS: its MFMA operands come straight from the
// caches (K [N, L, Hk, D] rows, V^T [N, Hk, D, L] rows).  16x16x32 MFMAs keep
// the heads in 16 columns (the other columns' queries are zero), so a wave
// needs about half the registers of 32-wide tiles and two waves share a
// SIMD.  Per 32-key block:
//   S^T = K Q^T   2 key tiles x 8 dim steps; lane l holds head l % 16 and
//                 keys 16 t + 4 (l / 16) + i of tile t
//   softmax as in the prefill, over the 4 lane groups of each head
//   O^T += V^T P^T  16 dim tiles, one 32-key step; lane group g supplies
//                 the keys it holds, {4 g .. 4 g + 3, 16 + 4 g .. +3}, and reads
//                 the same keys of V^T (two 8-byte loads)
// All of a block's K loads go out before its MFMAs and all of its V loads
// before the softmax (scheduling barriers keep them from being sunk next to
// their uses).  The split's running maximum, sum and unnormalised output go
// to a workspace; attn_combine_kernel merges the splits and applies the gate.
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Keys per split: 256 .. 2048 (a multiple of 64), chosen on the host so that
// a step has about 8192 waves.
__host__ __device__ inline int dec_split_keys(int N, int Hk, int cache_len) {
  int s = 256;
  while (s < 2048 && (int64_t)N * Hk * ((cache_len + 2 * s - 1) / (2 * s)) >= 8192) s *= 2;
  return s;
}

struct DecArgs {
  const uint16_t* q_rot;        // [N, Hq, D]
  const uint16_t *k_cache, *v_cache;
  const int32_t* cache_lens;    // [N]; this step's token sits at cache_lens[n]
  float* part;                  // [N, Hk, nsplit, G, D + 2]
  int N, Hq, Hk, cache_len, nsplit, split_keys;
  float scale_log2;
};

__global__ __launch_bounds__(256, 2) void attn_decode_kernel(DecArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = gw % a.nsplit, nk = gw / a.nsplit;
  const int kvh = nk % a.Hk, n = nk / a.Hk;
  if (n >= a.N) return;
  const int G = a.Hq / a.Hk;
  // a row whose position lies outside [0, cache_len) is a padding row: every
  // split reports an empty part (and attn_combine_kernel writes zeros)
  const int pos = a.cache_lens[n];
  const int len = (pos >= 0 && pos < a.cache_len) ? pos + 1 : 0;
  const int kb = split * a.split_keys;
  const int col = lane & 15, grp = lane >> 4;
  float* part = a.part + ((((size_t)n * a.Hk + kvh) * a.nsplit + split) * G) * (kAD + 2);
  if (kb >= len) {
    if (col < G && grp == 0) {
      part[col * (kAD + 2) + kAD] = -INFINITY;
      part[col * (kAD + 2) + kAD + 1] = 0.f;
    }
    return;
  }
  // Q^T fragments (B operand): head col, dims 32 ks + 8 grp .. +7
  bf16x8 qf[8];
  {
    const uint16_t* qrow = a.q_rot + ((size_t)n * a.Hq + kvh * G + min(col, G - 1)) * kAD + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
      if (col >= G) qf[ks] = bf16x8{};
    }
  }
  f32x4v o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lsum = 0.f;
  const uint16_t* kbase = a.k_cache + ((size_t)n * a.cache_len * a.Hk + kvh) * kAD + 8 * grp;
  const uint16_t* vbase = a.v_cache + ((size_t)n * a.Hk + kvh) * kAD * a.cache_len + 8 * grp;
  const int kend = min(kb + a.split_keys, len);
  for (int k0 = kb; k0 < kend; k0 += 32) {
    bf16x8 kf[16];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* krow = kbase + (size_t)(k0 + 16 * t + col) * a.Hk * kAD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[8 * t + ks] = *reinterpret_cast<const bf16x8*>(krow + 32 * ks);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4v s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[8 * t + ks], qf[ks], s[t], 0, 0, 0);
    }
    // V^T fragments: dim row 16 dt + col, keys 4 grp .. +3 and 16 + 4 grp .. +3,
    // one 16-byte read from the blocked cache (16 rows: 1 KiB contiguous)
    u32x4 vf[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      vf[dt] = *reinterpret_cast<const u32x4*>(vbase + ((size_t)(k0 >> 5) * kAD + 16 * dt + col) * 32);
    __builtin_amdgcn_sched_barrier(0);
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 16 * t + 4 * grp + i;
        const float v = key < len ? s[t][i] * a.scale_log2 : -INFINITY;
        s[t][i] = v;
        bmax = fmaxf(bmax, v);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const bool grow = bmax > mrun + kRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float mnew = grow ? bmax : mrun;
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] *= alpha;
      mrun = mnew;
    }
    uint32_t pk[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(s[t][2 * e] - mrun);
        const float p1 = __builtin_amdgcn_exp2f(s[t][2 * e + 1] - mrun);
        lsum += p0 + p1;
        pk[2 * t + e] = pack_bf16x2(p0, p1);
      }
    const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, vf[dt]);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf, o[dt], 0, 0, 0);
    }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (col < G) {
    float* pr = part + col * (kAD + 2);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<f32x4*>(pr + 16 * dt + 4 * grp) = o[dt];
    if (grp == 0) {
      pr[kAD] = mrun;
      pr[kAD + 1] = lsum;
    }
  }
}

// Merge of the splits of one (sequence, query head), one thread per dim:
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s * sigmoid(gate).
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* part, const uint16_t* gate,
                                                           const int32_t* cache_lens, uint16_t* out, int Hq, int Hk,
                                                           int nsplit, int split_keys, int cache_len) {
  const int n = blockIdx.x / Hq, h = blockIdx.x % Hq, d = threadIdx.x;
  const int G = Hq / Hk, kvh = h / G, c = h % G;
  const size_t at = ((size_t)n * Hq + h) * kAD + d;
  const int pos = cache_lens[n];
  if (pos < 0 || pos >= cache_len) {  // padding row
    out[at] = 0;
    return;
  }
  const int used = (pos + 1 + split_keys - 1) / split_keys;
  const float* p = part + (((size_t)n * Hk + kvh) * nsplit * G + c) * (kAD + 2);
  const size_t stride = (size_t)G * (kAD + 2);
  float M = -INFINITY;
  for (int s = 0; s < used; ++s) M = fmaxf(M, p[s * stride + kAD]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < used; ++s) {
    const float w = __builtin_amdgcn_exp2f(p[s * stride + kAD] - M);
    num += w * p[s * stride + d];
    den += w * p[s * stride + kAD + 1];
  }
  const float z = bf16_to_f32(gate[at]);
  out[at] = f32_to_bf16(num / den * (1.f / (1.f + __expf(-z))));
}

}  // namespace

size_t attn_decode_workspace_bytes(const AttnArgs& a) {
  const int sk = dec_split_keys(a.N, a.Hk, a.cache_len);
  const size_t nsplit = (a.cache_len + sk - 1) / sk;
  const size_t q = ((size_t)a.N * a.Hq * kAD * 2 + 255) / 256 * 256;
  return q + (size_t)a.N * a.Hk * nsplit * (a.Hq / a.Hk) * (kAD + 2) * 4;
}

hipError_t launch_attn_decode(const AttnArgs& a, void* ws, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const int sk = dec_split_keys(a.N, a.Hk, a.cache_len);
  const int nsplit = (a.cache_len + sk - 1) / sk;
  unsigned char* p = static_cast<unsigned char*>(ws);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(p);
  float* part = reinterpret_cast<float*>(p + ((size_t)a.N * a.Hq * kAD * 2 + 255) / 256 * 256);
  PrepArgs pa{};
  pa.q = static_cast<const uint16_t*>(a.q);
  pa.k = static_cast<const uint16_t*>(a.k);
  pa.v = static_cast<const uint16_t*>(a.v);
  pa.q_w = a.q_norm_w;
  pa.k_w = a.k_norm_w;
  pa.cache_lens = a.cache_lens;
  pa.q_rot = q_rot;
  pa.k_cache = static_cast<uint16_t*>(a.k_cache);
  pa.v_cache = static_cast<uint16_t*>(a.v_cache);
  pa.rows = a.N;
  pa.N = a.N;
  pa.Hq = a.Hq;
  pa.Hk = a.Hk;
  pa.cache_len = a.cache_len;
  pa.eps = a.eps;
  pa.base = a.rope_base;
  hipLaunchKernelGGL(attn_prep_kernel, dim3((unsigned)a.N), dim3(256), 0, st, pa);
  DecArgs d{};
  d.q_rot = q_rot;
  d.k_cache = static_cast<const uint16_t*>(a.k_cache);
  d.v_cache = static_cast<const uint16_t*>(a.v_cache);
  d.cache_lens = a.cache_lens;
  d.part = part;
  d.N = a.N;
  d.Hq = a.Hq;
  d.Hk = a.Hk;
  d.cache_len = a.cache_len;
  d.nsplit = nsplit;
  d.split_keys = sk;
  d.scale_log2 = 1.4426950408889634f / 16.f;
  const int64_t waves = (int64_t)a.N * a.Hk * nsplit;
  hipLaunchKernelGGL(attn_decode_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, d);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.N * a.Hq)), dim3(256), 0, st, part,
                     static_cast<const uint16_t*>(a.gate), a.cache_lens, static_cast<uint16_t*>(a.out), a.Hq, a.Hk,
                     nsplit, sk, a.cache_len);
  return hipGetLastError();
}

hipError_t launch_attn_qk_prep(const AttnArgs& a, void* q_out, void* k_out, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  PrepArgs pa{};
  pa.q = static_cast<const uint16_t*>(a.q);
  pa.k = static_cast<const uint16_t*>(a.k);
  pa.q_w = a.q_norm_w;
  pa.k_w = a.k_norm_w;
  pa.cu = a.cu_seqlens;
  pa.q_rot = static_cast<uint16_t*>(q_out);
  pa.k_rot = static_cast<uint16_t*>(k_out);
  pa.rows = a.T;
  pa.N = a.N;
  pa.Hq = a.Hq;
  pa.Hk = a.Hk;
  pa.eps = a.eps;
  pa.base = a.rope_base;
  hipLaunchKernelGGL(attn_prep_kernel, dim3((unsigned)a.T), dim3(256), 0, st, pa);
  return hipGetLastError();
}

size_t attn_prefill_workspace_bytes(const AttnArgs& a) {
  const size_t T = a.T, N = a.N;
  const size_t tpad = (size_t)kKB * ((T + kKB - 1) / kKB + N);
  size_t b = ((2 * (N + 1)) * 4 + 255) / 256 * 256;
  b += (T * a.Hq * kAD * 2 + 255) / 256 * 256;       // q_rot
  b += (tpad * a.Hk * kAD * 2 + 255) / 256 * 256;    // k_pad
  b += (tpad * a.Hk * kAD * 2 + 255) / 256 * 256;    // vt
  return b;
}

hipError_t launch_attn_prefill(const AttnArgs& a, void* ws, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const size_t T = a.T, N = a.N;
  const int64_t chunks = (int64_t)((T + kKB - 1) / kKB + N);
  const int64_t tpad = kKB * chunks;
  unsigned char* p = static_cast<unsigned char*>(ws);
  int32_t* table = reinterpret_cast<int32_t*>(p);
  p += ((2 * (N + 1)) * 4 + 255) / 256 * 256;
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(p);
  p += (T * a.Hq * kAD * 2 + 255) / 256 * 256;
  uint16_t* k_pad = reinterpret_cast<uint16_t*>(p);
  p += (tpad * a.Hk * kAD * 2 + 255) / 256 * 256;
  uint16_t* vt = reinterpret_cast<uint16_t*>(p);

  hipLaunchKernelGGL(attn_table_kernel, dim3(1), dim3(256), 0, st, a.cu_seqlens, a.N, table);
  PrepArgs pa{};
  pa.q = static_cast<const uint16_t*>(a.q);
  pa.k = static_cast<const uint16_t*>(a.k);
  pa.v = static_cast<const uint16_t*>(a.v);
  pa.q_w = a.q_norm_w;
  pa.k_w = a.k_norm_w;
  pa.cu = a.cu_seqlens;
  pa.table = table;
  pa.q_rot = q_rot;
  pa.k_pad = k_pad;
  pa.k_cache = static_cast<uint16_t*>(a.k_cache);
  pa.v_cache = static_cast<uint16_t*>(a.v_cache);
  pa.rows = a.T;
  pa.N = a.N;
  pa.Hq = a.Hq;
  pa.Hk = a.Hk;
  pa.cache_len = a.cache_len;
  pa.kblocks = tpad / kFB;
  pa.eps = a.eps;
  pa.base = a.rope_base;
  hipLaunchKernelGGL(attn_prep_kernel, dim3((unsigned)T), dim3(256), 0, st, pa);
  hipLaunchKernelGGL(attn_vt_kernel, dim3((unsigned)chunks, (unsigned)a.Hk), dim3(256), 0, st,
                     static_cast<const uint16_t*>(a.v), a.cu_seqlens, table, a.N, a.Hk, tpad, vt,
                     static_cast<uint16_t*>(a.v_cache), a.cache_len);
  FwdArgs f{};
  f.q_rot = q_rot;
  f.k_pad = k_pad;
  f.vt = vt;
  f.gate = static_cast<const uint16_t*>(a.gate);
  f.cu = a.cu_seqlens;
  f.table = table;
  f.out = static_cast<uint16_t*>(a.out);
  f.N = a.N;
  f.Hq = a.Hq;
  f.Hk = a.Hk;
  f.tpad = tpad;
  f.scale_log2 = 1.4426950408889634f / 16.f;
  const int G = a.Hq / a.Hk;
  const int64_t units = (int64_t)a.Hk * ((T + kQB - 1) / kQB + N);
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds * G;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace gdr
