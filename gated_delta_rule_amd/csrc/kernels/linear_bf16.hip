// Dense projection y = x W^T on the bf16 matrix cores, fp32 accumulation:
// the delta layer's in-projection (hidden -> q|k|v, z, b, a) and its
// out-projection (normed output -> hidden) (deepmagic page, parameter table:
// the delta-rule layer's projection widths; architecture section: the
// hidden width 5120).
//
//   x [M, K] bf16 (row stride ldx), W [N, K] bf16 (row stride ldw): both
//   operands run along K, so each 16-byte piece of a row is one MFMA operand
//   slice and neither needs a transpose.
//
// Tiling: one workgroup of 4 waves per 256 x 256 output tile.
//   - K runs in steps of 32 through four LDS stages (4 x 2 x 16 KiB); the x
//     and W tiles of a step go straight from global memory into LDS with
//     16-byte direct-to-LDS loads, issued three steps ahead of their use;
//   - wave (wr, wc) owns the 128 x 128 sub-tile at rows 128 wr, columns
//     128 wc: 4 x 4 tiles of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators
//     per lane in the accumulation registers;
//   - the copy instructions sit between the MFMAs, one after every four: a
//     copy can hold up issue while the memory pipeline drains, and the matrix
//     core keeps running meanwhile (issued in a burst, the copies kept it idle
//     for a third of each step);
//   - W is the MFMA's A operand and x its B operand, so each lane ends up
//     holding 4 consecutive output columns of one row: 8-byte (bf16) or
//     16-byte (fp32) stores.
// LDS rows are 32 bf16 = 64 bytes = four 16-byte slots; slot s of row r holds
// K piece s ^ ((r >> 2) & 3).  A 16-byte-per-lane LDS read serves 16 lanes
// per cycle from 64 banks; a fragment read's 16 lanes are 16 consecutive rows
// at one piece, and the swizzle puts them on 16 different 16-byte bank groups
// (rows with the same r & 3 differ in r >> 2).
//
// Launch order: 256 consecutive workgroups cover a 16 x 16 window of tiles
// (grouped raster: 16 tile rows, then along the columns), and the hardware
// deals consecutive workgroup ids round-robin to the 8 XCDs, so the window is
// split into eight 4 x 8 blocks, one per XCD: the 32 workgroups an XCD runs
// together share 4 row panels of x and 8 of W in its L2.
#include "../common.h"
#include "../internal.h"

namespace gdr {

namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32, kStages = 4;
constexpr int kWin = 16;
constexpr int kXcds = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// M0 is named as clobbered; nothing else in this file uses it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// One 1-KiB piece of the direct-to-LDS copy of the 64 rows [r0 + 64 wave,
// +64) x [k0, k0 + 32) of a row-major bf16 matrix into its swizzled LDS tile:
// piece i writes LDS rows 64 wave + 16 i .. +16 (lane l fills slot l % 4 of
// row l / 4).  Rows past rmax read row rmax (in bounds); their products land
// in output rows or columns that are never stored.
__device__ __forceinline__ void dma_piece(const uint16_t* g, int64_t ld, int r0, int rmax, int k0, uint16_t* s,
                                          int wave, int lane, int i) {
  const int rr = lane >> 2;
  const int row = 64 * wave + 16 * i;
  const int piece = (lane & 3) ^ ((rr >> 2) & 3);  // row & 15 = rr
  const int gr = min(r0 + row + rr, rmax);
  const uint32_t base = (uint32_t)(uintptr_t)(lds_ptr)s;
  dma16(g + gr * ld + k0 + 8 * piece, __builtin_amdgcn_readfirstlane(base + row * kBK * 2));
}

__device__ __forceinline__ void dma_rows(const uint16_t* g, int64_t ld, int r0, int rmax, int k0,
                                         uint16_t* s, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dma_piece(g, ld, r0, rmax, k0, s, wave, lane, i);
}

// A later step's copy: x and W tiles, 8 pieces per wave.
struct NextCopy {
  const uint16_t *X, *W;
  int64_t ldx, ldw;
  int m0, n0, mmax, nmax, k0;
  uint16_t *sX, *sW;
  __device__ __forceinline__ void piece(int j, int wave, int lane) const {
    if (j < 4)
      dma_piece(X, ldx, m0, mmax, k0, sX, wave, lane, j);
    else
      dma_piece(W, ldw, n0, nmax, k0, sW, wave, lane, j - 4);
  }
};

// MFMA operand fragment of 32 rows [r0, r0 + 32) for K sub-step ks (16 wide):
// lane l reads 8 consecutive K of row r0 + l % 32, piece 2 ks + l / 32.
__device__ __forceinline__ bf16x8 frag(const uint16_t* s, int r0, int ks, int lane) {
  const int row = r0 + (lane & 31), piece = 2 * ks + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(s + row * kBK + 8 * (piece ^ ((row >> 2) & 3)));
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm16() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }

// One K step (two sub-steps of 16) on a staged pair of tiles, with a later
// step's copy issued between its MFMAs: per sub-step, four groups of 4 MFMAs,
// each followed by one 1-KiB copy piece; sub-step 1's fragment reads follow
// the first group of sub-step 0.  Scheduling barriers keep that order.
__device__ __forceinline__ void mma_step(const uint16_t* sX, const uint16_t* sW, f32x16 (&acc)[4][4], int wr,
                                         int wc, int lane, int wave, const NextCopy& nc) {
  bf16x8 fw[2][4], fx[2][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    fw[0][t] = frag(sW, 128 * wc + 32 * t, 0, lane);
    fx[0][t] = frag(sX, 128 * wr + 32 * t, 0, lane);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[ks][tn], fx[ks][tm], acc[tn][tm], 0, 0, 0);
      nc.piece(4 * ks + tn, wave, lane);
      if (tn == 0 && ks == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          fw[1][t] = frag(sW, 128 * wc + 32 * t, 1, lane);
          fx[1][t] = frag(sX, 128 * wr + 32 * t, 1, lane);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The column block holding output column n.
__device__ __forceinline__ LinearOut block_of(const LinearArgs& a, int n) {
  LinearOut o = a.out[0];
  if (a.nout > 1 && n >= a.out[1].n0) o = a.out[1];
  if (a.nout > 2 && n >= a.out[2].n0) o = a.out[2];
  if (a.nout > 3 && n >= a.out[3].n0) o = a.out[3];
  return o;
}

__device__ __forceinline__ float out_value(int kind, float v) {
  return kind == kLinearF32Bf16 ? bf16_to_f32(f32_to_bf16(v)) : v;
}

// Four consecutive output columns n .. n+3 of row m.  One 8- or 16-byte store
// when all four lie inside one block laid out for it (vec), else one store
// per column, each routed to its own block.  kAllVec: every block is vec and
// starts at a multiple of 4, so the first case always holds.
template <bool kAllVec>
__device__ __forceinline__ void store4(const LinearArgs& a, int m, int n, float v0, float v1, float v2, float v3) {
  const LinearOut o = block_of(a, n);
  if (kAllVec || (o.vec && n + 3 < o.n1)) {
    const int64_t off = (int64_t)m * o.ld + (n - o.n0);
    if (o.kind == kLinearBf16) {
      const u32x2 p = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o.ptr) + off) = p;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(o.ptr) + off) =
          f32x4{out_value(o.kind, v0), out_value(o.kind, v1), out_value(o.kind, v2), out_value(o.kind, v3)};
    }
    return;
  }
  if (kAllVec) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ve = e == 0 ? v0 : e == 1 ? v1 : e == 2 ? v2 : v3;
    if (n + e < a.N) {
      const LinearOut b = block_of(a, n + e);
      const int64_t off = (int64_t)m * b.ld + (n + e - b.n0);
      if (b.kind == kLinearBf16)
        static_cast<uint16_t*>(b.ptr)[off] = f32_to_bf16(ve);
      else
        static_cast<float*>(b.ptr)[off] = out_value(b.kind, ve);
    }
  }
}

template <bool kAllVec>
__global__ __launch_bounds__(256, 1) void linear_kernel(LinearArgs a) {
  __shared__ __align__(16) uint16_t sX[kStages][kBM * kBK], sW[kStages][kBN * kBK];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;

  // workgroup -> tile
  const int Mt = (a.M + kBM - 1) / kBM, Nt = (a.N + kBN - 1) / kBN;
  const int b = blockIdx.x, x = b % kXcds, loc = (b % 256) / kXcds;
  const int t = 256 * (b / 256) + (8 * (x & 1) + loc / 4) * kWin + 4 * (x >> 1) + (loc & 3);
  if (t >= Mt * Nt) return;
  const int per_group = kWin * Nt, first = (t / per_group) * kWin;
  const int gsz = min(Mt - first, kWin), r = t % per_group;
  const int m0 = (first + r % gsz) * kBM, n0 = (r / gsz) * kBN;

  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Four stages, K = 32 each: step kt sits in stage kt % 4, and the copy of
  // step kt + 3 is issued while step kt is multiplied, three steps (about
  // 3000 cycles) ahead of its use.  One barrier per step: once every wave's
  // copy of step kt has landed and every wave has finished step kt - 1, the
  // stage of step kt - 1 is refilled.  Copies past the last step are clamped
  // to it (so the count of loads in flight is always the same) and never read.
  const int nk = a.K / kBK;
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) {
    const int kj = min(j, nk - 1) * kBK;
    dma_rows(X, a.ldx, m0, a.M - 1, kj, sX[j], wave, lane);
    dma_rows(W, a.ldw, n0, a.N - 1, kj, sW[j], wave, lane);
  }
  NextCopy nc{X, W, a.ldx, a.ldw, m0, n0, a.M - 1, a.N - 1, 0, nullptr, nullptr};
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm16();  // this wave's copy of step kt has landed (kt + 1, kt + 2 may be in flight)
    __syncthreads();
    const int sn = (kt + kStages - 1) % kStages;
    nc.k0 = min(kt + kStages - 1, nk - 1) * kBK;
    nc.sX = sX[sn];
    nc.sW = sW[sn];
    mma_step(sX[kt % kStages], sW[kt % kStages], acc, wr, wc, lane, wave, nc);
  }
  wait_vm0();

  // Output tile (tn, tm) of this wave: lane l holds row m = .. + l % 32 and,
  // in accumulator group q, columns 8 q + 4 (l / 32) .. +3.
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int m = m0 + 128 * wr + 32 * tm + (lane & 31);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 128 * wc + 32 * tn + 8 * q + 4 * (lane >> 5);
        if (m < a.M && n < a.N)
          store4<kAllVec>(a, m, n, acc[tn][tm][4 * q], acc[tn][tm][4 * q + 1], acc[tn][tm][4 * q + 2],
                 acc[tn][tm][4 * q + 3]);
      }
  }
}

}  // namespace

hipError_t launch_linear(const LinearArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const int64_t tiles = (int64_t)((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  const int64_t grid = (tiles + 255) / 256 * 256;
  bool all_vec = a.N % 4 == 0;
  for (int i = 0; i < a.nout; ++i) all_vec = all_vec && a.out[i].vec;
  if (all_vec)
    hipLaunchKernelGGL(linear_kernel<true>, dim3((unsigned)grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(linear_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdr
