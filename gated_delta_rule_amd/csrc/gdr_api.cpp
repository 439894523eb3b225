// C ABI of libgdr: argument validation and kernel dispatch.  Every check runs
// on the host before anything is enqueued; no entry point allocates, frees or
// synchronises.  See include/gdr.h for the contract of each call.
#include "gdr.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

gdr_status fail(gdr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gdr_status ok() {
  g_last_error.clear();
  return GDR_OK;
}

gdr_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t t) { return t == GDR_F32 || t == GDR_BF16; }

bool supported_dim(int32_t d) { return d == 32 || d == 64 || d == 128; }

// Shape/option checks shared by gdr_chunk_fwd and gdr_recurrent_step.
gdr_status check_desc(const gdr_desc* d, bool decode, bool has_cu) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size < sizeof(gdr_desc))
    return fail(GDR_ERR_INVALID_ARG, "descriptor struct_size %u < %zu", d->struct_size, sizeof(gdr_desc));
  if (d->batch < 0 || d->seq_len < 0 || d->num_seqs < 0)
    return fail(GDR_ERR_INVALID_ARG, "negative batch/seq_len/num_seqs");
  if (d->num_k_heads <= 0 || d->num_v_heads <= 0)
    return fail(GDR_ERR_INVALID_ARG, "head counts must be positive");
  if (d->num_v_heads % d->num_k_heads)
    return fail(GDR_ERR_INVALID_ARG, "num_v_heads (%d) must be a multiple of num_k_heads (%d)", d->num_v_heads,
                d->num_k_heads);
  if (!valid_dtype(d->qkv_dtype) || !valid_dtype(d->out_dtype))
    return fail(GDR_ERR_INVALID_ARG, "unknown dtype code");
  if (!(d->l2norm_eps >= 0.f) || !std::isfinite(d->scale))
    return fail(GDR_ERR_INVALID_ARG, "l2norm_eps must be >= 0 and scale finite");
  if (d->head_dim_k != d->head_dim_v || !supported_dim(d->head_dim_k))
    return fail(GDR_ERR_UNSUPPORTED, "head dims %d/%d: need d_k == d_v in {32, 64, 128}", d->head_dim_k,
                d->head_dim_v);
  if (decode) {
    if (d->seq_len != 1) return fail(GDR_ERR_INVALID_ARG, "decode needs seq_len == 1");
    if (d->num_seqs != d->batch) return fail(GDR_ERR_INVALID_ARG, "decode needs num_seqs == batch");
  } else {
    if (d->chunk_size != 64 && d->chunk_size != 32)
      return fail(GDR_ERR_UNSUPPORTED, "chunk_size %d: need 32 or 64", d->chunk_size);
    if (has_cu) {
      if (d->batch != 1) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens needs batch == 1");
    } else if (d->num_seqs != d->batch) {
      return fail(GDR_ERR_INVALID_ARG, "without cu_seqlens num_seqs must equal batch");
    }
  }
  const double tokens = (double)d->batch * d->seq_len;
  if (tokens * d->num_v_heads * d->head_dim_v >= 9.0e18)
    return fail(GDR_ERR_INVALID_ARG, "problem too large");
  return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char* gdr_status_string(int status) {
  switch (status) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
    default: return "GDR_UNKNOWN_STATUS";
  }
}

const char* gdr_last_error(void) { return g_last_error.c_str(); }

// The MFMA path (bf16 q/k/v, d = 128, chunk 64) keeps per-chunk records in a
// workspace; every other combination needs none.
static bool mfma_path(const gdr_desc* d) {
  return d->qkv_dtype == GDR_BF16 && d->head_dim_k == 128 && d->chunk_size == 64;
}

static size_t workspace_bytes_for(const gdr_desc* d) {
  if (!mfma_path(d)) return 0;
  gdr::ChunkArgs a{};
  a.N = d->num_seqs;
  a.T = d->seq_len;
  a.Hv = d->num_v_heads;
  // With batch == 1 the same descriptor may describe a packed batch, whose
  // chunk count is bounded by ceil(T/64) + N; size for that bound.
  static const int32_t any_cu = 0;
  a.cu_seqlens = d->batch == 1 ? &any_cu : nullptr;
  return gdr::chunk_bf16_workspace_bytes(a);
}

gdr_status gdr_chunk_fwd_workspace_size(const gdr_desc* d, size_t* bytes) {
  if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
  // a packed batch (cu_seqlens) is the only way num_seqs can differ from batch
  gdr_status st = check_desc(d, false, d && d->num_seqs != d->batch);
  if (st != GDR_OK) return st;
  *bytes = workspace_bytes_for(d);
  return ok();
}

// gdr_chunk_fwd and its two stages: checks, then the stages asked for.
static gdr_status chunk_fwd(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* initial_state, float* final_state,
                            const int32_t* cu_seqlens, void* o, void* workspace, size_t workspace_bytes,
                            void* stream, int stages, const char* name) {
  gdr_status st = check_desc(d, false, cu_seqlens != nullptr);
  if (st != GDR_OK) return st;
  const long long tokens = (long long)d->batch * d->seq_len;
  if (tokens > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, g, beta and o are required");
  if (cu_seqlens == nullptr && d->num_seqs > 0 && d->seq_len == 0 && !final_state) return ok();
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(initial_state) ||
      !aligned16(final_state))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, o and state pointers must be 16-byte aligned");
  if (d->num_seqs == 0) return ok();
  const size_t need = workspace_bytes_for(d);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GDR_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace)) return fail(GDR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  gdr::ChunkArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.initial_state = initial_state;
  a.final_state = final_state;
  a.cu_seqlens = cu_seqlens;
  a.o = o;
  a.N = d->num_seqs;
  a.T = d->seq_len;
  a.Hk = d->num_k_heads;
  a.Hv = d->num_v_heads;
  a.D = d->head_dim_k;
  a.C = d->chunk_size;
  a.qkv_bf16 = d->qkv_dtype == GDR_BF16;
  a.out_bf16 = d->out_dtype == GDR_BF16;
  a.use_l2 = d->use_qk_l2norm != 0;
  a.scale = d->scale;
  a.eps = d->l2norm_eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma_path(d)) return hip_status(gdr::launch_chunk_bf16(a, workspace, s, stages), name);
  // the fp32 path has no prepare stage: the recurrence stage does all the work
  if (!(stages & gdr::kStageRecur)) return ok();
  return hip_status(gdr::launch_chunk_f32(a, s), name);
}

gdr_status gdr_chunk_fwd(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, float* final_state,
                         const int32_t* cu_seqlens, void* o, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return chunk_fwd(d, q, k, v, g, beta, initial_state, final_state, cu_seqlens, o, workspace, workspace_bytes,
                   stream, gdr::kStagePrepare | gdr::kStageRecur, "gdr_chunk_fwd launch");
}

gdr_status gdr_chunk_fwd_prepare(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state, float* final_state,
                                 const int32_t* cu_seqlens, void* o, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return chunk_fwd(d, q, k, v, g, beta, initial_state, final_state, cu_seqlens, o, workspace, workspace_bytes,
                   stream, gdr::kStagePrepare, "gdr_chunk_fwd_prepare launch");
}

gdr_status gdr_chunk_fwd_recurrence(const gdr_desc* d, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const float* initial_state,
                                    float* final_state, const int32_t* cu_seqlens, void* o, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return chunk_fwd(d, q, k, v, g, beta, initial_state, final_state, cu_seqlens, o, workspace, workspace_bytes,
                   stream, gdr::kStageRecur, "gdr_chunk_fwd_recurrence launch");
}

static gdr_status recurrent_step(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, float* state, int32_t pool_size, const int32_t* state_indices,
                                 void* o, void* stream, const char* name) {
  gdr_status st = check_desc(d, true, false);
  if (st != GDR_OK) return st;
  if (d->batch == 0) return ok();
  // an empty pool (every row padding) may be NULL
  const bool empty_pool = state_indices && pool_size == 0;
  if (!q || !k || !v || !g || !beta || (!state && !empty_pool) || !o)
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, g, beta, state and o are required");
  if (!aligned16(state)) return fail(GDR_ERR_INVALID_ARG, "state must be 16-byte aligned");
  gdr::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state = state;
  a.state_indices = state_indices;
  a.pool_size = pool_size;
  a.o = o;
  a.N = d->batch;
  a.Hk = d->num_k_heads;
  a.Hv = d->num_v_heads;
  a.D = d->head_dim_k;
  a.qkv_bf16 = d->qkv_dtype == GDR_BF16;
  a.out_bf16 = d->out_dtype == GDR_BF16;
  a.use_l2 = d->use_qk_l2norm != 0;
  a.scale = d->scale;
  a.eps = d->l2norm_eps;
  return hip_status(gdr::launch_decode(a, static_cast<hipStream_t>(stream)), name);
}

gdr_status gdr_recurrent_step(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                              const float* beta, float* state, void* o, void* stream) {
  return recurrent_step(d, q, k, v, g, beta, state, 0, nullptr, o, stream, "gdr_recurrent_step launch");
}

gdr_status gdr_recurrent_step_indexed(const gdr_desc* d, const void* q, const void* k, const void* v,
                                      const float* g, const float* beta, float* state_pool, int32_t pool_size,
                                      const int32_t* state_indices, void* o, void* stream) {
  if (pool_size < 0) return fail(GDR_ERR_INVALID_ARG, "pool_size must be >= 0 (got %d)", pool_size);
  if (!state_indices) return fail(GDR_ERR_INVALID_ARG, "state_indices is required");
  return recurrent_step(d, q, k, v, g, beta, state_pool, pool_size, state_indices, o, stream,
                        "gdr_recurrent_step_indexed launch");
}

gdr_status gdr_decode_layer_step(const gdr_desc* d, const void* x, const void* conv_w, void* conv_state,
                                 const float* a, const float* b, const float* A_log, const float* dt_bias,
                                 float* state, int32_t pool_size, const int32_t* state_indices, const void* z,
                                 const float* norm_w, float norm_eps, void* y, float* o, void* qkv_out,
                                 void* stream) {
  gdr_status st = check_desc(d, true, false);
  if (st != GDR_OK) return st;
  if (d->head_dim_k != 128 || d->head_dim_v != 128)
    return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_layer_step supports d = 128 (got %d)", d->head_dim_k);
  const int G = d->num_v_heads / d->num_k_heads;
  if (G < 1 || G > 4)
    return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_layer_step supports Hv/Hk in 1..4 (got %d)", G);
  if (d->qkv_dtype != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "gdr_decode_layer_step takes bf16 x");
  if (pool_size < 0) return fail(GDR_ERR_INVALID_ARG, "pool_size must be >= 0 (got %d)", pool_size);
  if (d->batch == 0) return ok();
  const bool empty_pool = state_indices && pool_size == 0;
  if (!x || !conv_w || !a || !b || !A_log || !dt_bias || !z || !norm_w || !y ||
      ((!state || !conv_state) && !empty_pool))
    return fail(GDR_ERR_INVALID_ARG, "x, conv_w, conv_state, a, b, A_log, dt_bias, state, z, norm_w and y are required");
  if (!aligned16(state) || reinterpret_cast<uintptr_t>(conv_w) % 8)
    return fail(GDR_ERR_INVALID_ARG, "state must be 16-byte and conv_w 8-byte aligned");
  gdr::LayerStepArgs la{};
  la.x = x;
  la.conv_w = conv_w;
  la.conv_state = conv_state;
  la.a = a;
  la.b = b;
  la.A_log = A_log;
  la.dt_bias = dt_bias;
  la.state = state;
  la.state_indices = state_indices;
  la.pool_size = pool_size;
  la.z = z;
  la.norm_w = norm_w;
  la.y = y;
  la.o = o;
  la.qkv_out = qkv_out;
  la.N = d->batch;
  la.Hk = d->num_k_heads;
  la.Hv = d->num_v_heads;
  la.use_l2 = d->use_qk_l2norm != 0;
  la.scale = d->scale;
  la.eps = d->l2norm_eps;
  la.norm_eps = norm_eps;
  return hip_status(gdr::launch_decode_layer(la, static_cast<hipStream_t>(stream)), "gdr_decode_layer_step launch");
}

gdr_status gdr_conv_gate_fused(const gdr_conv_desc* d, const void* x, const void* conv_w,
                               const int32_t* cu_seqlens, const void* conv_state_in, void* conv_state_out,
                               const float* a, const float* b, const float* A_log, const float* dt_bias,
                               void* q_out, void* k_out, void* v_out, float* g, float* beta, void* stream) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size < sizeof(gdr_conv_desc))
    return fail(GDR_ERR_INVALID_ARG, "descriptor struct_size %u < %zu", d->struct_size, sizeof(gdr_conv_desc));
  if (d->num_tokens < 0 || d->num_seqs < 1 || d->num_k_heads <= 0 || d->num_v_heads <= 0)
    return fail(GDR_ERR_INVALID_ARG, "need num_tokens >= 0, num_seqs >= 1, positive head counts");
  if (!supported_dim(d->head_dim)) return fail(GDR_ERR_UNSUPPORTED, "head_dim %d: need 32, 64 or 128", d->head_dim);
  if (!cu_seqlens) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is required");
  if (d->num_tokens > 0 &&
      (!x || !conv_w || !a || !b || !A_log || !dt_bias || !q_out || !k_out || !v_out || !g || !beta))
    return fail(GDR_ERR_INVALID_ARG, "x, conv_w, a, b, A_log, dt_bias and all outputs are required");
  if (conv_state_out && conv_state_out == conv_state_in)
    return fail(GDR_ERR_INVALID_ARG, "conv_state_out must not alias conv_state_in");
  if (!aligned16(x) || !aligned16(conv_w) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out))
    return fail(GDR_ERR_INVALID_ARG, "x, conv_w and q/k/v outputs must be 16-byte aligned");
  gdr::ConvArgs c{};
  c.x = x;
  c.w = conv_w;
  c.cu_seqlens = cu_seqlens;
  c.state_in = conv_state_in;
  c.state_out = conv_state_out;
  c.a = a;
  c.b = b;
  c.A_log = A_log;
  c.dt_bias = dt_bias;
  c.q_out = q_out;
  c.k_out = k_out;
  c.v_out = v_out;
  c.g = g;
  c.beta = beta;
  c.T = d->num_tokens;
  c.N = d->num_seqs;
  c.Hk = d->num_k_heads;
  c.Hv = d->num_v_heads;
  c.D = d->head_dim;
  return hip_status(gdr::launch_conv_front(c, static_cast<hipStream_t>(stream)), "gdr_conv_gate_fused launch");
}

gdr_status gdr_gated_rmsnorm(const gdr_norm_desc* d, const void* o, const void* z, const float* w, void* y,
                             void* stream) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size < sizeof(gdr_norm_desc))
    return fail(GDR_ERR_INVALID_ARG, "descriptor struct_size %u < %zu", d->struct_size, sizeof(gdr_norm_desc));
  if (d->num_tokens < 0 || d->num_heads <= 0) return fail(GDR_ERR_INVALID_ARG, "bad num_tokens/num_heads");
  if (!valid_dtype(d->o_dtype)) return fail(GDR_ERR_INVALID_ARG, "unknown dtype code");
  if (!(d->eps >= 0.f)) return fail(GDR_ERR_INVALID_ARG, "eps must be >= 0");
  if (!supported_dim(d->head_dim)) return fail(GDR_ERR_UNSUPPORTED, "head_dim %d: need 32, 64 or 128", d->head_dim);
  if (d->num_tokens > 0 && (!o || !z || !w || !y)) return fail(GDR_ERR_INVALID_ARG, "o, z, w and y are required");
  if (!aligned16(o) || !aligned16(z) || !aligned16(y) || !aligned16(w))
    return fail(GDR_ERR_INVALID_ARG, "o, z, w and y must be 16-byte aligned");
  gdr::NormArgs n{};
  n.o = o;
  n.z = z;
  n.w = w;
  n.y = y;
  n.T = d->num_tokens;
  n.H = d->num_heads;
  n.D = d->head_dim;
  n.o_bf16 = d->o_dtype == GDR_BF16;
  n.eps = d->eps;
  return hip_status(gdr::launch_gated_rmsnorm(n, static_cast<hipStream_t>(stream)), "gdr_gated_rmsnorm launch");
}

}  // extern "C"
