// C ABI of libgdr: argument validation and kernel dispatch.  Every check runs
// on the host before anything is enqueued; no entry point allocates, frees or
// synchronises.  See include/gdr.h for the contract of each call.
#include "gdr.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "host_checks.h"
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
    // the bf16-MFMA path (bf16, d = 128, chunk 64) bounds the value heads per key head
    if (d->qkv_dtype == GDR_BF16 && d->head_dim_k == 128 && d->chunk_size == 64 &&
        d->num_v_heads / d->num_k_heads > gdr::kChunkMaxHeadRatio)
      return fail(GDR_ERR_UNSUPPORTED, "bf16 prefill supports up to %d value heads per key head (got %d)",
                  gdr::kChunkMaxHeadRatio, d->num_v_heads / d->num_k_heads);
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


// GDR_DEBUG_CHECKS (read at every call; unset, empty or "0" = off): the index
// arrays the kernels trust are copied to the host and checked, and workspaces
// are filled with NaN bytes before the kernels run, so a read of a workspace
// entry that no kernel wrote shows up in the results.  The copies wait for
// the stream; the mode is for debugging, not for graph capture.
bool debug_checks() {
  const char* e = std::getenv("GDR_DEBUG_CHECKS");
  return e && *e && std::strcmp(e, "0") != 0;
}

gdr_status debug_read_i32(const int32_t* p, size_t n, hipStream_t s, std::vector<int32_t>* out, const char* what) {
  out->assign(n, 0);
  if (n == 0) return GDR_OK;
  hipError_t e = hipMemcpyAsync(out->data(), p, n * sizeof(int32_t), hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "GDR_DEBUG_CHECKS: reading %s: %s", what, hipGetErrorString(e));
  return GDR_OK;
}

gdr_status debug_check_cu(const int32_t* cu, int N, long long tokens, void* stream, const char* what) {
  if (!cu || !debug_checks()) return GDR_OK;
  std::vector<int32_t> h;
  gdr_status st = debug_read_i32(cu, (size_t)N + 1, static_cast<hipStream_t>(stream), &h, what);
  if (st != GDR_OK) return st;
  char msg[256];
  if (!gdr::check_cu_seqlens(h.data(), N, tokens, what, msg, sizeof msg))
    return fail(GDR_ERR_INVALID_ARG, "GDR_DEBUG_CHECKS: %s", msg);
  return GDR_OK;
}

gdr_status debug_check_indices(const int32_t* idx, int N, int pool, void* stream) {
  if (!idx || !debug_checks()) return GDR_OK;
  std::vector<int32_t> h;
  gdr_status st = debug_read_i32(idx, (size_t)N, static_cast<hipStream_t>(stream), &h, "state_indices");
  if (st != GDR_OK) return st;
  char msg[256];
  if (!gdr::check_state_indices(h.data(), N, pool, msg, sizeof msg))
    return fail(GDR_ERR_INVALID_ARG, "GDR_DEBUG_CHECKS: %s", msg);
  return GDR_OK;
}

gdr_status debug_poison(void* ws, size_t bytes, void* stream) {
  if (!ws || !bytes || !debug_checks()) return GDR_OK;
  hipError_t e = hipMemsetAsync(ws, 0xFF, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "GDR_DEBUG_CHECKS: filling the workspace: %s", hipGetErrorString(e));
  return GDR_OK;
}

}  // namespace

// Static device scratch of gdr_chunk_fwd_noalloc: the workspace of callers
// that cannot allocate.  Every GPU the library runs on holds its own copy
// for the life of the process.  In host code `scratch` names a host-side
// stand-in, so kernels only ever get the device address that
// hipGetSymbolAddress returns for the current device.
namespace {
__device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

gdr_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDR_ERR_UNSUPPORTED, "device %d: the scratch table covers devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(GDR_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
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
  a.Hk = d->num_k_heads;
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
  if ((st = debug_check_cu(cu_seqlens, d->num_seqs, d->seq_len, stream, "cu_seqlens")) != GDR_OK) return st;
  // the recurrence stage alone reads what prepare left in the workspace
  if ((stages & gdr::kStagePrepare) && (st = debug_poison(workspace, need, stream)) != GDR_OK) return st;
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


gdr_status gdr_chunk_fwd_noalloc(const gdr_desc* d, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* initial_state, float* final_state,
                                 const int32_t* cu_seqlens, void* o, void* stream) {
  gdr_status st = check_desc(d, false, cu_seqlens != nullptr);
  if (st != GDR_OK) return st;
  const size_t need = workspace_bytes_for(d);
  if (need > (size_t)GDR_NOALLOC_SCRATCH_BYTES)
    return fail(GDR_ERR_INVALID_ARG,
                "gdr_chunk_fwd_noalloc: this call needs %zu bytes of workspace, the static scratch holds %zu "
                "(use gdr_chunk_fwd with a caller workspace)",
                need, (size_t)GDR_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_of_current_device(&ws);
    if (st != GDR_OK) return st;
  }
  return chunk_fwd(d, q, k, v, g, beta, initial_state, final_state, cu_seqlens, o, ws,
                   need > 0 ? (size_t)GDR_NOALLOC_SCRATCH_BYTES : 0, stream, gdr::kStagePrepare | gdr::kStageRecur,
                   "gdr_chunk_fwd_noalloc launch");
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
  if ((st = debug_check_indices(state_indices, d->batch, pool_size, stream)) != GDR_OK) return st;
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
  if ((st = debug_check_indices(state_indices, d->batch, pool_size, stream)) != GDR_OK) return st;
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
  const gdr_status st = debug_check_cu(cu_seqlens, d->num_seqs, d->num_tokens, stream, "cu_seqlens");
  if (st != GDR_OK) return st;
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

gdr_status gdr_linear(int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w, int64_t ldw,
                      const gdr_linear_out* outs, int32_t num_outs, void* stream) {
  if (M < 0 || N < 0 || K <= 0) return fail(GDR_ERR_INVALID_ARG, "need M, N >= 0 and K > 0 (got %d, %d, %d)", M, N, K);
  if (K % 32) return fail(GDR_ERR_INVALID_ARG, "K (%d) must be a multiple of 32", K);
  if (ldx < K || ldw < K || ldx % 8 || ldw % 8)
    return fail(GDR_ERR_INVALID_ARG, "ldx and ldw must be >= K and multiples of 8");
  if (!outs || num_outs < 1 || num_outs > 4) return fail(GDR_ERR_INVALID_ARG, "need 1..4 output blocks");
  const bool work = M > 0 && N > 0;
  if (work && (!x || !w)) return fail(GDR_ERR_INVALID_ARG, "x and w are required");
  if (!aligned16(x) || !aligned16(w)) return fail(GDR_ERR_INVALID_ARG, "x and w must be 16-byte aligned");
  gdr::LinearArgs a{};
  a.x = x;
  a.w = w;
  a.ldx = ldx;
  a.ldw = ldw;
  a.M = M;
  a.N = N;
  a.K = K;
  a.nout = num_outs;
  int64_t col = 0;
  for (int i = 0; i < num_outs; ++i) {
    const gdr_linear_out& o = outs[i];
    if (o.cols < 0 || o.ld < o.cols) return fail(GDR_ERR_INVALID_ARG, "output block %d: need 0 <= width <= ld", i);
    if (o.dtype != GDR_BF16 && o.dtype != GDR_F32) return fail(GDR_ERR_INVALID_ARG, "output block %d: bad dtype", i);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(o.ptr);
    const unsigned elem = o.dtype == GDR_BF16 ? 2u : 4u;
    if (M > 0 && o.cols > 0 && !o.ptr) return fail(GDR_ERR_INVALID_ARG, "output block %d is NULL", i);
    if (addr % elem) return fail(GDR_ERR_INVALID_ARG, "output block %d must be %u-byte aligned", i, elem);
    a.out[i].ptr = o.ptr;
    a.out[i].ld = o.ld;
    a.out[i].n0 = (int)col;
    a.out[i].n1 = (int)(col + o.cols);
    a.out[i].kind = o.dtype == GDR_BF16 ? gdr::kLinearBf16 : o.round_bf16 ? gdr::kLinearF32Bf16 : gdr::kLinearF32;
    a.out[i].vec = col % 4 == 0 && o.ld % 4 == 0 && addr % (4u * elem) == 0;
    col += o.cols;
  }
  if (col != N) return fail(GDR_ERR_INVALID_ARG, "output block widths sum to %lld, N is %d", (long long)col, N);
  // An empty block starts where the next one does, so routing by first column
  // never picks it.
  return hip_status(gdr::launch_linear(a, static_cast<hipStream_t>(stream)), "gdr_linear launch");
}

namespace {

// Intermediates of gdr_delta_layer_fwd, 256-byte aligned pieces of the workspace.
struct LayerBufs {
  size_t qkv, z, b, a, q, k, v, g, beta, o, chunk, total, chunk_bytes;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

gdr_desc layer_chunk_desc(const gdr_layer_desc* d) {
  gdr_desc c{};
  c.struct_size = sizeof(gdr_desc);
  c.batch = 1;
  c.seq_len = d->num_tokens;
  c.num_seqs = d->num_seqs;
  c.num_k_heads = d->num_k_heads;
  c.num_v_heads = d->num_v_heads;
  c.head_dim_k = c.head_dim_v = d->head_dim;
  c.chunk_size = 64;
  c.qkv_dtype = GDR_BF16;
  c.out_dtype = GDR_F32;
  c.use_qk_l2norm = 1;
  c.scale = 1.f;
  c.l2norm_eps = d->l2norm_eps;
  return c;
}

gdr_status layer_plan(const gdr_layer_desc* d, LayerBufs* p) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size < sizeof(gdr_layer_desc))
    return fail(GDR_ERR_INVALID_ARG, "descriptor struct_size %u < %zu", d->struct_size, sizeof(gdr_layer_desc));
  if (d->num_tokens < 0 || d->num_seqs < 1 || d->num_k_heads <= 0 || d->num_v_heads <= 0 || d->hidden <= 0)
    return fail(GDR_ERR_INVALID_ARG, "need num_tokens >= 0, num_seqs >= 1, positive heads and hidden");
  if (d->num_v_heads % d->num_k_heads)
    return fail(GDR_ERR_INVALID_ARG, "num_v_heads must be a multiple of num_k_heads");
  if (d->head_dim != 128) return fail(GDR_ERR_UNSUPPORTED, "the delta layer takes head_dim 128 (got %d)", d->head_dim);
  if (d->hidden % 32) return fail(GDR_ERR_INVALID_ARG, "hidden (%d) must be a multiple of 32", d->hidden);
  if (!(d->l2norm_eps >= 0.f) || !(d->norm_eps >= 0.f)) return fail(GDR_ERR_INVALID_ARG, "eps must be >= 0");
  const size_t T = (size_t)d->num_tokens, Hk = d->num_k_heads, Hv = d->num_v_heads, D = d->head_dim;
  const size_t C = (2 * Hk + Hv) * D, V = Hv * D;
  const gdr_desc cd = layer_chunk_desc(d);
  size_t cb = 0;
  const gdr_status st = gdr_chunk_fwd_workspace_size(&cd, &cb);
  if (st != GDR_OK) return st;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  p->qkv = take(T * C * 2);  // reused for y once the front has read it
  p->z = take(T * V * 2);
  p->b = take(T * Hv * 4);
  p->a = take(T * Hv * 4);
  p->q = take(T * Hk * D * 2);
  p->k = take(T * Hk * D * 2);
  p->v = take(T * V * 2);
  p->g = take(T * Hv * 4);
  p->beta = take(T * Hv * 4);
  p->o = take(T * V * 4);
  p->chunk = take(cb);
  p->chunk_bytes = cb;
  p->total = off;
  return ok();
}

}  // namespace

gdr_status gdr_delta_layer_workspace_size(const gdr_layer_desc* d, size_t* bytes) {
  if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
  LayerBufs p;
  const gdr_status st = layer_plan(d, &p);
  if (st != GDR_OK) return st;
  *bytes = p.total;
  return ok();
}

gdr_status gdr_delta_layer_fwd(const gdr_layer_desc* d, const void* hidden, const void* w_in, const void* conv_w,
                               const float* A_log, const float* dt_bias, const float* norm_w, const void* w_out,
                               const int32_t* cu_seqlens, const void* conv_state_in, void* conv_state_out,
                               const float* initial_state, float* final_state, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  LayerBufs p;
  gdr_status st = layer_plan(d, &p);
  if (st != GDR_OK) return st;
  if (!hidden || !w_in || !conv_w || !A_log || !dt_bias || !norm_w || !w_out || !cu_seqlens || !out)
    return fail(GDR_ERR_INVALID_ARG, "hidden, w_in, conv_w, A_log, dt_bias, norm_w, w_out, cu_seqlens and out are required");
  if (!workspace || workspace_bytes < p.total)
    return fail(GDR_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", p.total, workspace ? workspace_bytes : 0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GDR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if ((st = debug_check_cu(cu_seqlens, d->num_seqs, d->num_tokens, stream, "cu_seqlens")) != GDR_OK) return st;
  if ((st = debug_poison(workspace, p.total, stream)) != GDR_OK) return st;
  const int T = d->num_tokens, H = d->hidden, Hk = d->num_k_heads, Hv = d->num_v_heads, D = d->head_dim;
  const int C = (2 * Hk + Hv) * D, V = Hv * D;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  void* qkv = ws + p.qkv;
  void* z = ws + p.z;
  float* bb = reinterpret_cast<float*>(ws + p.b);
  float* aa = reinterpret_cast<float*>(ws + p.a);
  void* q = ws + p.q;
  void* k = ws + p.k;
  void* v = ws + p.v;
  float* g = reinterpret_cast<float*>(ws + p.g);
  float* beta = reinterpret_cast<float*>(ws + p.beta);
  float* o = reinterpret_cast<float*>(ws + p.o);
  void* y = qkv;

  gdr_linear_out in_outs[4] = {
      {qkv, C, C, GDR_BF16, 0, 0}, {z, V, V, GDR_BF16, 0, 0}, {bb, Hv, Hv, GDR_F32, 1, 0}, {aa, Hv, Hv, GDR_F32, 1, 0}};
  if ((st = gdr_linear(T, C + V + 2 * Hv, H, hidden, H, w_in, H, in_outs, 4, stream)) != GDR_OK) return st;

  gdr_conv_desc cd{};
  cd.struct_size = sizeof(cd);
  cd.num_tokens = T;
  cd.num_seqs = d->num_seqs;
  cd.num_k_heads = Hk;
  cd.num_v_heads = Hv;
  cd.head_dim = D;
  if ((st = gdr_conv_gate_fused(&cd, qkv, conv_w, cu_seqlens, conv_state_in, conv_state_out, aa, bb, A_log, dt_bias,
                                q, k, v, g, beta, stream)) != GDR_OK)
    return st;

  const gdr_desc rd = layer_chunk_desc(d);
  if ((st = gdr_chunk_fwd(&rd, q, k, v, g, beta, initial_state, final_state, cu_seqlens, o, ws + p.chunk,
                          p.chunk_bytes, stream)) != GDR_OK)
    return st;

  gdr_norm_desc nd{};
  nd.struct_size = sizeof(nd);
  nd.num_tokens = T;
  nd.num_heads = Hv;
  nd.head_dim = D;
  nd.o_dtype = GDR_F32;
  nd.eps = d->norm_eps;
  if ((st = gdr_gated_rmsnorm(&nd, o, z, norm_w, y, stream)) != GDR_OK) return st;

  gdr_linear_out out_blk = {out, H, H, GDR_BF16, 0, 0};
  return gdr_linear(T, H, V, y, V, w_out, V, &out_blk, 1, stream);
}

namespace {

gdr_status check_attn(const gdr_attn_desc* d, bool decode) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size < sizeof(gdr_attn_desc))
    return fail(GDR_ERR_INVALID_ARG, "descriptor struct_size %u < %zu", d->struct_size, sizeof(gdr_attn_desc));
  if (d->num_tokens < 0 || d->num_seqs < 1 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->cache_len < 0)
    return fail(GDR_ERR_INVALID_ARG, "need num_tokens >= 0, num_seqs >= 1, positive heads, cache_len >= 0");
  if (d->head_dim != 256) return fail(GDR_ERR_UNSUPPORTED, "attention takes head_dim 256 (got %d)", d->head_dim);
  if (d->num_q_heads % d->num_kv_heads)
    return fail(GDR_ERR_UNSUPPORTED, "num_q_heads must be a multiple of num_kv_heads");
  if (!(d->norm_eps >= 0.f) || !(d->rope_base > 1.0)) return fail(GDR_ERR_INVALID_ARG, "need eps >= 0, rope_base > 1");
  if (decode && d->num_tokens != d->num_seqs) return fail(GDR_ERR_INVALID_ARG, "decode needs num_tokens == num_seqs");
  return ok();
}

gdr::AttnArgs attn_args(const gdr_attn_desc* d) {
  gdr::AttnArgs a{};
  a.T = d->num_tokens;
  a.N = d->num_seqs;
  a.Hq = d->num_q_heads;
  a.Hk = d->num_kv_heads;
  a.cache_len = d->cache_len;
  a.eps = d->norm_eps;
  a.rope_base = d->rope_base;
  return a;
}

}  // namespace

gdr_status gdr_attn_qk_norm_rope(const gdr_attn_desc* d, const void* q, const void* k, const float* q_norm_w,
                                 const float* k_norm_w, const int32_t* cu_seqlens, void* q_out, void* k_out,
                                 void* stream) {
  gdr_status st = check_attn(d, false);
  if (st != GDR_OK) return st;
  if (!cu_seqlens || !q_norm_w || !k_norm_w) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens and the norm weights are required");
  if (d->num_tokens > 0 && (!q || !k || !q_out || !k_out)) return fail(GDR_ERR_INVALID_ARG, "q, k, q_out and k_out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(q_norm_w) ||
      !aligned16(k_norm_w))
    return fail(GDR_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if ((st = debug_check_cu(cu_seqlens, d->num_seqs, d->num_tokens, stream, "cu_seqlens")) != GDR_OK) return st;
  gdr::AttnArgs a = attn_args(d);
  a.q = q;
  a.k = k;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.cu_seqlens = cu_seqlens;
  return hip_status(gdr::launch_attn_qk_prep(a, q_out, k_out, static_cast<hipStream_t>(stream)),
                    "gdr_attn_qk_norm_rope launch");
}

gdr_status gdr_attn_prefill_workspace_size(const gdr_attn_desc* d, size_t* bytes) {
  if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
  const gdr_status st = check_attn(d, false);
  if (st != GDR_OK) return st;
  *bytes = gdr::attn_prefill_workspace_bytes(attn_args(d));
  return ok();
}

gdr_status gdr_attn_prefill(const gdr_attn_desc* d, const void* q, const void* k, const void* v, const void* gate,
                            const float* q_norm_w, const float* k_norm_w, const int32_t* cu_seqlens, void* out,
                            void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes, void* stream) {
  gdr_status st = check_attn(d, false);
  if (st != GDR_OK) return st;
  if (!cu_seqlens || !q_norm_w || !k_norm_w) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens and the norm weights are required");
  if (d->num_tokens > 0 && (!q || !k || !v || !gate || !out))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, gate and out are required");
  if (!k_cache != !v_cache) return fail(GDR_ERR_INVALID_ARG, "give both k_cache and v_cache or neither");
  if (k_cache && (d->cache_len <= 0 || d->cache_len % 64))
    return fail(GDR_ERR_INVALID_ARG, "a cache needs cache_len > 0, a multiple of 64 (got %d)", d->cache_len);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(q_norm_w) || !aligned16(k_norm_w))
    return fail(GDR_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  gdr::AttnArgs a = attn_args(d);
  const size_t need = gdr::attn_prefill_workspace_bytes(a);
  if (!workspace || workspace_bytes < need)
    return fail(GDR_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace ? workspace_bytes : 0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GDR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if ((st = debug_check_cu(cu_seqlens, d->num_seqs, d->num_tokens, stream, "cu_seqlens")) != GDR_OK) return st;
  if ((st = debug_poison(workspace, need, stream)) != GDR_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.cu_seqlens = cu_seqlens;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return hip_status(gdr::launch_attn_prefill(a, workspace, static_cast<hipStream_t>(stream)), "gdr_attn_prefill launch");
}

gdr_status gdr_attn_decode_workspace_size(const gdr_attn_desc* d, size_t* bytes) {
  if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
  const gdr_status st = check_attn(d, true);
  if (st != GDR_OK) return st;
  if (d->cache_len <= 0 || d->cache_len % 64)
    return fail(GDR_ERR_INVALID_ARG, "decode needs cache_len > 0, a multiple of 64 (got %d)", d->cache_len);
  *bytes = gdr::attn_decode_workspace_bytes(attn_args(d));
  return ok();
}

gdr_status gdr_attn_decode(const gdr_attn_desc* d, const void* q, const void* k, const void* v, const void* gate,
                           const float* q_norm_w, const float* k_norm_w, void* k_cache, void* v_cache,
                           const int32_t* cache_lens, void* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  gdr_status st = check_attn(d, true);
  if (st != GDR_OK) return st;
  if (d->cache_len <= 0 || d->cache_len % 64)
    return fail(GDR_ERR_INVALID_ARG, "decode needs cache_len > 0, a multiple of 64 (got %d)", d->cache_len);
  if (!q || !k || !v || !gate || !q_norm_w || !k_norm_w || !k_cache || !v_cache || !cache_lens || !out)
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, gate, norm weights, caches, cache_lens and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(q_norm_w) || !aligned16(k_norm_w))
    return fail(GDR_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  gdr::AttnArgs a = attn_args(d);
  const size_t need = gdr::attn_decode_workspace_bytes(a);
  if (!workspace || workspace_bytes < need)
    return fail(GDR_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace ? workspace_bytes : 0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GDR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if ((st = debug_poison(workspace, need, stream)) != GDR_OK) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_lens = cache_lens;
  a.out = out;
  return hip_status(gdr::launch_attn_decode(a, workspace, static_cast<hipStream_t>(stream)), "gdr_attn_decode launch");
}

}  // extern "C"
