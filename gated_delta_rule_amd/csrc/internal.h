// Launch interface between the C ABI (gdr_api.cpp) and the kernels.  Every
// launcher assumes its arguments were validated by the ABI layer and only
// enqueues work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

struct DecodeArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  float* state;
  const int32_t* state_indices;  // NULL: sequence n uses state n; else a pool slot
  int pool_size;                 // slots of the pool (with state_indices)
  void* o;
  int N, Hk, Hv, D;
  int qkv_bf16, out_bf16, use_l2;
  float scale, eps;
};

struct ChunkArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  const float* initial_state;
  float* final_state;
  const int32_t* cu_seqlens;  // NULL: N rows of T tokens
  void* o;
  int N, T, Hk, Hv, D, C;     // T: tokens per row (or packed total)
  int qkv_bf16, out_bf16, use_l2;
  float scale, eps;
};

struct ConvArgs {
  const void *x, *w;
  const int32_t* cu_seqlens;
  const void* state_in;
  void* state_out;
  const float *a, *b, *A_log, *dt_bias;
  void *q_out, *k_out, *v_out;
  float *g, *beta;
  int T, N, Hk, Hv, D;
};

struct LayerStepArgs {
  const void* x;           // [N, C] bf16 token projections (q | k | v)
  const void* conv_w;      // [C, 4] bf16
  void* conv_state;        // [P, C, 3] bf16, rolled in place
  const float *a, *b;      // [N, Hv]
  const float *A_log, *dt_bias;  // [Hv]
  float* state;            // [P, Hv, d, d] fp32, in place
  const int32_t* state_indices;  // NULL: row n uses slot n
  int pool_size;
  const void* z;           // [N, Hv*d] bf16
  const float* norm_w;     // [d]
  void* y;                 // [N, Hv*d] bf16
  float* o;                // [N, Hv, d] fp32 or NULL
  void* qkv_out;           // [N, C] bf16 or NULL
  int N, Hk, Hv, use_l2;
  float scale, eps, norm_eps;
};

struct NormArgs {
  const void* o;
  const void* z;
  const float* w;
  void* y;
  int T, H, D, o_bf16;
  float eps;
};

// y = x W^T (bf16 operands, fp32 accumulation); output columns are split into
// up to four blocks, each written to its own buffer.
constexpr int kLinearBf16 = 0;     // bf16, round to nearest even
constexpr int kLinearF32 = 1;      // fp32 accumulator
constexpr int kLinearF32Bf16 = 2;  // fp32 holding the bf16-rounded value
struct LinearOut {
  void* ptr;
  int64_t ld;  // row stride in elements
  int n0, n1;  // output columns [n0, n1) of the block
  int kind;    // kLinear*
  int vec;     // n0 and ld multiples of 4 and ptr 8 (bf16) / 16 (fp32) byte aligned
};
struct LinearArgs {
  const void* x;  // [M, K] bf16, row stride ldx
  const void* w;  // [N, K] bf16, row stride ldw
  int64_t ldx, ldw;
  int M, N, K;    // K a multiple of 32
  int nout;       // 1..4 blocks, contiguous, out[0].n0 = 0, empty ones allowed
  LinearOut out[4];
};

// Global attention (GQA, head dim 256): prefill over a packed batch, and one
// decode token per sequence against a KV cache.
struct AttnArgs {
  const void *q, *k, *v, *gate;    // bf16: q, gate [rows, Hq, 256]; k, v [rows, Hk, 256]
  const float *q_norm_w, *k_norm_w;  // [256]
  const int32_t* cu_seqlens;       // prefill [N+1]
  const int32_t* cache_lens;       // decode [N]: cached tokens before this one
  void* out;                       // [rows, Hq, 256] bf16
  void *k_cache, *v_cache;         // [N, cache_len, Hk, 256] and [N, Hk, cache_len/32, 256, 32] bf16, or NULL (prefill)
  int cache_len;
  int T, N, Hq, Hk;                // T: packed tokens (prefill) or N (decode)
  float eps;
  double rope_base;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_linear(const LinearArgs& a, hipStream_t st);
size_t attn_prefill_workspace_bytes(const AttnArgs& a);
hipError_t launch_attn_qk_prep(const AttnArgs& a, void* q_out, void* k_out, hipStream_t st);
size_t attn_decode_workspace_bytes(const AttnArgs& a);
hipError_t launch_attn_decode(const AttnArgs& a, void* workspace, hipStream_t st);
hipError_t launch_attn_prefill(const AttnArgs& a, void* workspace, hipStream_t st);
hipError_t launch_decode_layer(const LayerStepArgs& a, hipStream_t st);
hipError_t launch_chunk_f32(const ChunkArgs& a, hipStream_t st);
// The bf16-MFMA prefill needs a device workspace of
// chunk_bf16_workspace_bytes(a) bytes (chunk table + per-chunk records).  It
// runs in two stages: kStagePrepare fills the workspace (state-independent
// per-chunk factors), kStageRecur carries the state through the chunks.
constexpr int kStagePrepare = 1, kStageRecur = 2;
// Value heads per key head the bf16-MFMA prefill takes: its prepare kernel
// keeps 512 bytes of LDS per value head of a key head (four workgroups per
// compute unit up to 8).
constexpr int kChunkMaxHeadRatio = 64;
size_t chunk_bf16_workspace_bytes(const ChunkArgs& a);
hipError_t launch_chunk_bf16(const ChunkArgs& a, void* workspace, hipStream_t st, int stages);
hipError_t launch_conv_front(const ConvArgs& a, hipStream_t st);
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t st);

}  // namespace gdr
