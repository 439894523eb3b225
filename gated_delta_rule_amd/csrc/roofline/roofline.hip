// Roofline probes (include/gdr_roofline.h): achievable HBM streaming rates
// and the bf16 matrix-core issue rate of the GPU they run on, and two
// exhaustive checks of the numeric behaviour the conv front's bit-exact
// contract relies on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "gdr_roofline.h"
#include "silu32.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr size_t kSlab = 65536;  // bytes per workgroup

// Lane (wave w, lane l) of a slab reads rows 32 w + l/32 + 2 i (i < 16) of
// 512 bytes, at byte 16 (l % 32): each load instruction covers two whole rows.
__device__ __forceinline__ size_t slab_offset(int i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (size_t)(wave * 32 + (lane >> 5) + 2 * i) * 128 + 4 * (lane & 31);
}

template <bool kNT>
__global__ __launch_bounds__(256) void rmw_kernel(float* p, float scale) {
  float* base = p + (size_t)blockIdx.x * (kSlab / 4);
  f32x4 s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const f32x4* src = reinterpret_cast<const f32x4*>(base + slab_offset(i));
    s[i] = kNT ? __builtin_nontemporal_load(src) : *src;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f32x4* dst = reinterpret_cast<f32x4*>(base + slab_offset(i));
    const f32x4 v = s[i] * scale;
    if (kNT) __builtin_nontemporal_store(v, dst);
    else *dst = v;
  }
}

__global__ __launch_bounds__(256) void read_kernel(const float* p, float* sums) {
  const float* base = p + (size_t)blockIdx.x * (kSlab / 4);
  f32x4 s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = *reinterpret_cast<const f32x4*>(base + slab_offset(i));
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += (s[i][0] + s[i][1]) + (s[i][2] + s[i][3]);
  __shared__ float part[256];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) sums[blockIdx.x] = part[0];
}

__global__ __launch_bounds__(256) void mfma_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  // operands from the lane index, so that nothing is constant-folded
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[u], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) r += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = r;
}

// Vector-ALU issue: 8 independent chains of a = a * m + c per thread, the
// multiply and the add issued as two fp32 instructions (no contraction), so
// every wave issues 16 VALU instructions per round with no dependency stall.
__global__ __launch_bounds__(256) void valu_kernel(float* out, int iters) {
#pragma clang fp contract(off)
  const float m = 0.999f + 1e-7f * (float)(threadIdx.x & 63), c = 1e-3f * (float)(threadIdx.x & 7);
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = (float)(u + 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = acc[u] * m + c;
  }
  float r = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) r += acc[u];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = r;
}

// Sum of the wave's mismatch counts and minimum of its first mismatching
// patterns, added to the totals by lane 0 (vector atomics).
__device__ __forceinline__ void report(unsigned long long nbad, uint32_t first, unsigned long long* bad,
                                       uint32_t* first_bad) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    nbad += __shfl_xor(nbad, m, 64);
    first = min(first, (uint32_t)__shfl_xor((int)first, m, 64));
  }
  if ((threadIdx.x & 63) == 0 && nbad) {
    atomicAdd(bad, nbad);
    atomicMin(first_bad, first);
  }
}

// silu32_mid against silu32 for the fp32 patterns lo .. lo + count - 1 whose
// value lies in [-80, 80] (others, NaN included, are skipped).
__global__ __launch_bounds__(256) void silu_mid_probe(uint32_t lo, unsigned long long count,
                                                      unsigned long long* bad, uint32_t* first_bad) {
  unsigned long long nbad = 0;
  uint32_t first = 0xffffffffu;
  const unsigned long long stride = (unsigned long long)gridDim.x * blockDim.x;
  for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint32_t bits = lo + (uint32_t)i;
    const float v = __uint_as_float(bits);
    if (!(fabsf(v) <= 80.f)) continue;
    if (__float_as_uint(gdr::silu32_mid(v)) != __float_as_uint(gdr::silu32(v))) {
      ++nbad;
      first = min(first, bits);
    }
  }
  report(nbad, first, bad, first_bad);
}

// The hardware fp32 -> bf16 conversion against round to nearest even on the
// bit pattern (u + 0x7fff + bit 16 of u) >> 16; a NaN must give a quiet NaN
// of the same sign.
__global__ __launch_bounds__(256) void bf16_rne_probe(uint32_t lo, unsigned long long count,
                                                      unsigned long long* bad, uint32_t* first_bad) {
  unsigned long long nbad = 0;
  uint32_t first = 0xffffffffu;
  const unsigned long long stride = (unsigned long long)gridDim.x * blockDim.x;
  for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint32_t bits = lo + (uint32_t)i;
    const uint32_t hw = gdr::f32_to_bf16(__uint_as_float(bits));
    bool ok;
    if ((bits & 0x7fffffffu) > 0x7f800000u)
      ok = (hw & 0x7fc0u) == 0x7fc0u && (hw >> 15) == (bits >> 31);
    else
      ok = hw == ((bits + 0x7fffu + ((bits >> 16) & 1u)) >> 16);
    if (!ok) {
      ++nbad;
      first = min(first, bits);
    }
  }
  report(nbad, first, bad, first_bad);
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -3; }

}  // namespace

extern "C" int gdr_roofline_rmw(float* buf, size_t bytes, float scale, int nontemporal, void* stream) {
  if (!buf || bytes == 0 || bytes % kSlab || (uintptr_t)buf % 16) return -1;
  const dim3 grid((unsigned)(bytes / kSlab));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal) hipLaunchKernelGGL(rmw_kernel<true>, grid, dim3(256), 0, st, buf, scale);
  else hipLaunchKernelGGL(rmw_kernel<false>, grid, dim3(256), 0, st, buf, scale);
  return launched();
}

extern "C" int gdr_roofline_read(const float* buf, size_t bytes, float* sums, void* stream) {
  if (!buf || !sums || bytes == 0 || bytes % kSlab || (uintptr_t)buf % 16) return -1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)(bytes / kSlab)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     buf, sums);
  return launched();
}

extern "C" int gdr_roofline_mfma(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return launched();
}

extern "C" int gdr_roofline_valu(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(valu_kernel, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return launched();
}

extern "C" int gdr_probe_silu_mid(uint32_t first_bits, unsigned long long count, unsigned long long* mismatches,
                                  uint32_t* first_mismatch, void* stream) {
  if (!mismatches || !first_mismatch || count == 0 || count > (1ull << 32)) return -1;
  hipLaunchKernelGGL(silu_mid_probe, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), first_bits, count,
                     mismatches, first_mismatch);
  return launched();
}

extern "C" int gdr_probe_bf16_rne(uint32_t first_bits, unsigned long long count, unsigned long long* mismatches,
                                  uint32_t* first_mismatch, void* stream) {
  if (!mismatches || !first_mismatch || count == 0 || count > (1ull << 32)) return -1;
  hipLaunchKernelGGL(bf16_rne_probe, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), first_bits, count,
                     mismatches, first_mismatch);
  return launched();
}
