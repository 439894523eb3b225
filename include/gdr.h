/*
 * gdr.h -- C ABI of the gated delta rule library (libgdr.so) for AMD MI355X (gfx950).
 *
 * The library computes the hot path of a gated delta rule layer as the
 * Agnes-3.0-Flash pages describe it: per (sequence, value head) an fp32 state
 * S in R^{d_v x d_k} updated token by token as
 *
 *     S_t = S_{t-1} * exp(g_t) * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t
 *
 * (gpts24 page: the delta-rule update in words and the gated variant's forget
 * gate; yfxerp page, section 1.2: the recurrent call with g, beta, an initial
 * state, an optional final state and q/k L2 normalisation inside the kernel,
 * a chunk_size=64 block-parallel prefill and a single-step decode; deepmagic
 * page, architecture section: 16 key heads / 48 value heads of dim 128, a
 * kernel-4 causal conv in front, a gated RMS norm behind, an fp32 state).
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers, owned by the caller, contiguous
 *     in the layout documented per argument and 16-byte aligned.  Descriptor
 *     and size arguments are HOST pointers.
 *   - The library allocates nothing, frees nothing and never synchronises
 *     (apart from the debug mode below and gdr_chunk_fwd_noalloc's static
 *     scratch):
 *     every kernel is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns immediately.
 *   - Argument errors are reported synchronously, before anything is
 *     enqueued, as a negative gdr_status; gdr_last_error() then returns a
 *     thread-local message.  Device-side faults surface at the caller's next
 *     synchronisation.  Device array CONTENTS (e.g. cu_seqlens) are trusted.
 *   - Debug mode: with the environment variable GDR_DEBUG_CHECKS set (and not
 *     "0"), read at every call, each entry point first copies the index
 *     arrays it would trust to the host and checks them -- cu_seqlens
 *     (cu[0] == 0, non-decreasing, cu[N] == the token count) and
 *     state_indices (no pool slot named twice) -- and returns
 *     GDR_ERR_INVALID_ARG naming the first bad entry; then it fills
 *     its workspace with 0xFF bytes (NaN in fp32 and bf16) before the
 *     kernels run, so that a read of a workspace entry no kernel wrote shows
 *     up as NaN in the results.  The copies wait for `stream` to drain; a
 *     failed copy returns GDR_ERR_HIP.  The mode is for debugging, not for
 *     HIP graph capture.  Results are bit-identical with and without it.
 *   - Value head h reads key head h / (Hv / Hk) (contiguous groups).
 *   - Thread safety: calls from several host threads are safe; kernels that
 *     write the same output buffers concurrently race, as usual.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 1

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = -1, /* NULL where required, bad shape, misalignment, short workspace */
  GDR_ERR_UNSUPPORTED = -2, /* valid but not implemented: head dim, chunk size, dtype combination */
  GDR_ERR_HIP = -3          /* a HIP runtime error while enqueueing (launch failure) */
} gdr_status;

typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* Shape and options of the recurrence (gdr_chunk_fwd, gdr_recurrent_step). */
typedef struct gdr_desc {
  uint32_t struct_size; /* sizeof(gdr_desc) */
  int32_t batch;        /* B rows; must be 1 when cu_seqlens is given */
  int32_t seq_len;      /* T tokens per row (packed total with cu_seqlens); 1 for decode */
  int32_t num_seqs;     /* N sequences: B without cu_seqlens, else length of cu_seqlens - 1 */
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv, a multiple of Hk */
  int32_t head_dim_k;   /* d_k */
  int32_t head_dim_v;   /* d_v */
  int32_t chunk_size;   /* C: 64 or 32 (prefill only) */
  int32_t qkv_dtype;    /* gdr_dtype of q, k, v */
  int32_t out_dtype;    /* gdr_dtype of o */
  int32_t use_qk_l2norm; /* nonzero: q, k <- x / sqrt(sum(x^2) + l2norm_eps) per token and key head */
  float scale;          /* output scale (1.0 reproduces o_t = S_t q_t) */
  float l2norm_eps;     /* 1e-6 by convention */
} gdr_desc;

/* Shape of the conv + gate front (gdr_conv_gate_fused). */
typedef struct gdr_conv_desc {
  uint32_t struct_size; /* sizeof(gdr_conv_desc) */
  int32_t num_tokens;   /* T, packed over all sequences */
  int32_t num_seqs;     /* N = length of cu_seqlens - 1 */
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv */
  int32_t head_dim;     /* d (= d_k = d_v); channels C = 2*Hk*d + Hv*d */
} gdr_conv_desc;

/* Shape of the gated RMSNorm back (gdr_gated_rmsnorm). */
typedef struct gdr_norm_desc {
  uint32_t struct_size; /* sizeof(gdr_norm_desc) */
  int32_t num_tokens;   /* T */
  int32_t num_heads;    /* Hv */
  int32_t head_dim;     /* d_v: the normalised group */
  int32_t o_dtype;      /* gdr_dtype of o */
  float eps;            /* 1e-6 by convention */
} gdr_norm_desc;

/* Version of this ABI (GDR_ABI_VERSION of the built library). */
int gdr_abi_version(void);

/* Static name of a status code. */
const char* gdr_status_string(int status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* gdr_last_error(void);

/*
 * Device workspace that gdr_chunk_fwd needs for descriptor *d, in bytes.
 * The bf16-MFMA path (bf16 q/k/v, d = 128, chunk 64) stores a chunk table
 * and launch order (2N+1 int32, padded to 256 bytes) and one 25728-byte
 * record per (chunk,
 * value head) -- the chunk's T = (I+A)^{-1} and P as bf16 hi/lo pairs and its
 * per-token factors -- for an upper bound of ceil(T/64) + N chunks when
 * batch == 1 (packed or single sequence) and B * ceil(T/64) otherwise.  Every
 * other combination needs 0 bytes (workspace may then be NULL).  The
 * contents need no initialisation and are dead after the call returns.
 * Errors: INVALID_ARG / UNSUPPORTED as gdr_chunk_fwd would report them.
 */
gdr_status gdr_chunk_fwd_workspace_size(const gdr_desc* d, size_t* bytes);

/*
 * Chunked prefill (the pages' chunk_size=64 block-parallel path; the chunk
 * form is an exact rewrite of the token recurrence above).
 *
 *   q, k          [B, T, Hk, d_k]  qkv_dtype
 *   v             [B, T, Hv, d_v]  qkv_dtype
 *   g             [B, T, Hv] fp32  log-decay (exp(g) multiplies the state)
 *   beta          [B, T, Hv] fp32  write strength
 *   initial_state [N, Hv, d_v, d_k] fp32, d_k contiguous; NULL = zero state
 *   final_state   [N, Hv, d_v, d_k] fp32 output; NULL = not written.  May be
 *                 the same pointer as initial_state (updated in place).
 *   cu_seqlens    [N+1] int32 device array, cu[0] = 0, non-decreasing,
 *                 cu[N] = T; sequence n is tokens [cu[n], cu[n+1]) of the
 *                 single packed row.  NULL = B independent rows of T tokens.
 *   o             [B, T, Hv, d_v]  out_dtype output (never aliases inputs)
 *   workspace     device buffer of at least gdr_chunk_fwd_workspace_size()
 *                 bytes, 16-byte aligned (INVALID_ARG if missing or short);
 *                 used by the kernels of this call only
 *
 * Supported: d_k = d_v in {32, 64, 128}; chunk_size 64 or 32; qkv bf16 with
 * d = 128 and chunk 64 takes the bf16-MFMA path, every other supported
 * combination the fp32 path.  Chunks restart at every sequence start, so a
 * packed batch gives results bit-identical to separate calls; a zero-length
 * sequence copies its initial state to final_state.
 */
gdr_status gdr_chunk_fwd(const gdr_desc* d, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* initial_state,
                         float* final_state, const int32_t* cu_seqlens, void* o,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_chunk_fwd without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of gdr_chunk_fwd; the kernels are the same, so the outputs are bit for bit
 * those of gdr_chunk_fwd.  The workspace is a static device array of
 * GDR_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until the
 * process ends; its address is looked up (hipGetSymbolAddress) on the first
 * call made with that device current.  The call allocates and frees
 * nothing.
 *   INVALID_ARG  the call needs more workspace than the scratch holds
 *                (gdr_chunk_fwd_workspace_size(d) > GDR_NOALLOC_SCRATCH_BYTES;
 *                about 2 700 tokens at 48 value heads) -- nothing is enqueued
 *   UNSUPPORTED  the current device index is 64 or more
 * The calling thread's current device must be the device of `stream`.  All
 * calls on one GPU share its scratch and it keeps the last call's contents:
 * two calls that can run at the same time on one GPU (different streams, or
 * different threads) race and give undefined results.  Nothing in the
 * scratch needs to start at zero.
 */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_desc* d, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* initial_state,
                                 float* final_state, const int32_t* cu_seqlens, void* o, void* stream);

/*
 * The two stages of gdr_chunk_fwd, for callers that time or schedule them
 * apart.  Arguments, checks and errors are those of gdr_chunk_fwd, and
 * gdr_chunk_fwd_prepare followed by gdr_chunk_fwd_recurrence on one stream
 * with the same arguments and workspace is gdr_chunk_fwd, bit for bit.
 *   prepare:    fills the workspace with everything that does not depend on
 *               the state (per-chunk decays, q/k norms, (I+A)^{-1} and the
 *               causal decayed q.k products); writes nothing else
 *   recurrence: carries the state through the chunks using that workspace;
 *               writes o and final_state.  The workspace must not change
 *               between the two calls.
 * On a combination whose workspace size is 0, prepare enqueues nothing and
 * recurrence does all the work.
 */
gdr_status gdr_chunk_fwd_prepare(const gdr_desc* d, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* initial_state,
                                 float* final_state, const int32_t* cu_seqlens, void* o,
                                 void* workspace, size_t workspace_bytes, void* stream);
gdr_status gdr_chunk_fwd_recurrence(const gdr_desc* d, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const float* initial_state,
                                    float* final_state, const int32_t* cu_seqlens, void* o,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode token for N independent sequences (the pages' single-step
 * fused recurrent path).  d->batch = N, d->seq_len = 1, cu_seqlens unused.
 *
 *   q, k   [N, Hk, d_k] qkv_dtype;  v [N, Hv, d_v] qkv_dtype
 *   g, beta [N, Hv] fp32
 *   state  [N, Hv, d_v, d_k] fp32, read and overwritten IN PLACE with S_t
 *   o      [N, Hv, d_v] out_dtype
 *
 * Supported: d_k = d_v in {32, 64, 128}.
 */
gdr_status gdr_recurrent_step(const gdr_desc* d, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, float* state, void* o,
                              void* stream);

/*
 * gdr_recurrent_step on states kept in a persistent pool, as a serving
 * cache does (yfxerp page, section 1.2: the delta-rule layers keep their
 * recurrent state in a cache layer of their own, apart from the attention
 * layers' key/value cache).  Sequence n updates pool slot state_indices[n].
 *
 *   state_pool    [pool_size, Hv, d_v, d_k] fp32, slots read and overwritten
 *                 IN PLACE
 *   state_indices [N] int32 device array; an entry < 0 or >= pool_size marks
 *                 a padding row: its o is written as zeros and no slot is
 *                 read or written.  The other entries must be distinct (two
 *                 rows updating one slot would race).
 *   everything else as gdr_recurrent_step.
 *
 * Errors: as gdr_recurrent_step; INVALID_ARG also for pool_size < 0 or a NULL
 * state_indices.  state_pool may be NULL only when pool_size is 0 (every row
 * padding).  With state_indices[n] = n and pool_size = N the result is
 * bit-identical to gdr_recurrent_step.
 */
gdr_status gdr_recurrent_step_indexed(const gdr_desc* d, const void* q, const void* k, const void* v,
                                      const float* g, const float* beta, float* state_pool,
                                      int32_t pool_size, const int32_t* state_indices, void* o,
                                      void* stream);

/*
 * One decode token of the whole layer path in one launch: the conv front for
 * the token against a rolling conv state, the gates, the recurrent step and
 * the gated RMS norm (deepmagic page, architecture section: conv in front,
 * gated RMS norm behind; yfxerp page, section 1.2: the decode path takes a
 * single-step recurrence and keeps the conv state beside the recurrent
 * state).  d->batch = N rows, d->seq_len = 1, d_k = d_v = 128, bf16 x,
 * Hv/Hk in {1, 2, 3, 4}; d->scale, use_qk_l2norm and l2norm_eps as for
 * gdr_recurrent_step.  C = (2*Hk + Hv) * 128.
 *
 *   x             [N, C] bf16: the token's projections, channel blocks q | k | v
 *   conv_w        [C, 4] bf16 (8-byte aligned); tap 3 multiplies this token
 *   conv_state    [P, C, 3] bf16, the three previous inputs of each channel,
 *                 oldest first; rolled IN PLACE to end with this token
 *   a, b          [N, Hv] fp32;  A_log, dt_bias [Hv] fp32 (the gates)
 *   state         [P, Hv, 128, 128] fp32, updated IN PLACE
 *   state_indices NULL: row n uses slot n of both pools (P = N); else [N]
 *                 int32 device array naming each row's slot of both pools,
 *                 pool_size slots each; an entry outside [0, pool_size) marks
 *                 a padding row: its outputs are zeros and no slot is read or
 *                 written.  The other entries must be distinct.
 *   z             [N, Hv*128] bf16, the norm's gate input;  norm_w [128] fp32
 *   y             [N, Hv*128] bf16 = o / sqrt(mean(o^2) + norm_eps) * norm_w
 *                 * z * sigmoid(z) per (row, value head)
 *   o             [N, Hv, 128] fp32 pre-norm outputs, or NULL (not written)
 *   qkv_out       [N, C] bf16 conv + SiLU outputs, or NULL (not written)
 *
 * The conv output is bit-identical to gdr_conv_gate_fused on the same token
 * and state; o and the new state are bit-identical to gdr_recurrent_step on
 * that front's q, k, v, g and beta.  Errors: INVALID_ARG for a NULL required
 * pointer, misalignment, pool_size < 0, seq_len != 1; UNSUPPORTED for other
 * head sizes or ratios or a non-bf16 x.
 */
gdr_status gdr_decode_layer_step(const gdr_desc* d, const void* x, const void* conv_w, void* conv_state,
                                 const float* a, const float* b, const float* A_log, const float* dt_bias,
                                 float* state, int32_t pool_size, const int32_t* state_indices,
                                 const void* z, const float* norm_w, float norm_eps, void* y, float* o,
                                 void* qkv_out, void* stream);

/*
 * Front of the layer: depthwise causal conv (kernel 4, no bias) + SiLU over
 * all C = 2*Hk*d + Hv*d channels, plus the gates (deepmagic page: kernel-4
 * causal conv in front; yfxerp page, section 1.2: beta = sigmoid(b),
 * g = -exp(A_log) * softplus(a + dt_bias) in fp32).
 *
 *   x             [T, C] bf16, channel blocks q | k | v, each head-major
 *   conv_w        [C, 4] bf16; tap 3 multiplies the current token, taps
 *                 0..2 the three previous tokens of the same sequence
 *   cu_seqlens    [N+1] int32 device array (required; N = 1 for one sequence)
 *   conv_state_in [N, C, 3] bf16 history before each sequence, oldest first;
 *                 NULL = zeros
 *   conv_state_out[N, C, 3] bf16: the last three inputs of every sequence
 *                 (history included); NULL = not written; must not alias
 *                 conv_state_in
 *   a, b          [T, Hv] fp32 raw projections;  A_log, dt_bias [Hv] fp32
 *   q_out, k_out  [T, Hk, d] bf16;  v_out [T, Hv, d] bf16
 *   g, beta       [T, Hv] fp32 outputs
 *
 * The bf16 outputs are bit-exact with this fixed evaluation: p_j = w_j*x_j in
 * fp32 (exact for bf16 operands), acc = ((p0 + p1) + p2) + p3 with each add
 * rounded to fp32, y = acc / (1 + exp32(-acc)) with exp32 the Cody-Waite /
 * degree-7 Taylor exponential evaluated one IEEE fp32 operation at a time,
 * then round to nearest-even bf16.  g and beta are fp32 (not bit-exact).
 */
gdr_status gdr_conv_gate_fused(const gdr_conv_desc* d, const void* x, const void* conv_w,
                               const int32_t* cu_seqlens, const void* conv_state_in,
                               void* conv_state_out, const float* a, const float* b,
                               const float* A_log, const float* dt_bias, void* q_out,
                               void* k_out, void* v_out, float* g, float* beta, void* stream);

/*
 * Back of the layer: gated RMS norm per (token, head) over d_v (deepmagic
 * page: gated RMS norm after the recurrence; yfxerp page: z is Hv*d_v wide):
 *
 *   y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z)
 *
 *   o  [T, Hv, d_v] o_dtype;  z [T, Hv*d_v] bf16;  w [d_v] fp32
 *   y  [T, Hv*d_v] bf16
 *
 * Supported: d_v in {32, 64, 128}.
 */
gdr_status gdr_gated_rmsnorm(const gdr_norm_desc* d, const void* o, const void* z,
                             const float* w, void* y, void* stream);

/* ------------------------------------------------------------------------
 * The delta layer around the path: its dense projections and the whole layer
 * prefill (deepmagic page, parameter table: per delta-rule layer a q|k|v
 * projection, a z projection 6144 wide, b and a projections 48 wide each
 * and an output projection from 6144; architecture section: hidden width
 * 5120).  The weights are the caller's; nothing here depends on trained
 * values.
 * ------------------------------------------------------------------------ */

/* One block of output columns of gdr_linear. */
typedef struct gdr_linear_out {
  void* ptr;          /* device [M, cols] with row stride ld, aligned to its element */
  int64_t ld;         /* row stride in elements, >= cols */
  int32_t cols;       /* block width (0 allowed) */
  int32_t dtype;      /* GDR_BF16 (round to nearest even) or GDR_F32 */
  int32_t round_bf16; /* GDR_F32 only: nonzero stores the value rounded to bf16 */
  int32_t reserved;   /* 0 */
} gdr_linear_out;

/*
 * y = x W^T, bf16 operands, fp32 accumulation on the matrix cores:
 *
 *   x     [M, K] bf16, row stride ldx (elements)
 *   w     [N, K] bf16, row stride ldw (the out x in layout of a linear layer)
 *   outs  HOST array of num_outs (1..4) blocks: block i receives output
 *         columns [c_i, c_i + outs[i].cols) with c_0 = 0, c_{i+1} = c_i +
 *         outs[i].cols, and N = the sum of the widths
 *
 * Each output element is the fp32 sum of the K products, accumulated in an
 * unspecified order; |y - exact| <= K * 2^-24 * sum_k |x_k w_k| (per element,
 * before the bf16 rounding of a bf16 or round_bf16 block).
 * A block whose first column and ld are multiples of 4 and whose pointer is 8-
 * (bf16) or 16-byte (fp32) aligned is written 4 columns per store; any other
 * block one element per store.
 * Errors: INVALID_ARG for M, N < 0, K <= 0, K not a multiple of 32, ldx or
 * ldw < K or not a multiple of 8, x or w not 16-byte aligned, a bad block
 * (NULL with M > 0 and cols > 0, cols < 0, ld < cols, bad dtype, pointer not
 * aligned to its element), widths not summing to N.
 */
gdr_status gdr_linear(int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w, int64_t ldw,
                      const gdr_linear_out* outs, int32_t num_outs, void* stream);

/* Shape of the delta layer (gdr_delta_layer_fwd). */
typedef struct gdr_layer_desc {
  uint32_t struct_size; /* sizeof(gdr_layer_desc) */
  int32_t num_tokens;   /* T, packed over all sequences */
  int32_t num_seqs;     /* N = length of cu_seqlens - 1 */
  int32_t hidden;       /* H: model width, a multiple of 32 (5120 in the pages' model) */
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv, a multiple of Hk */
  int32_t head_dim;     /* d = d_k = d_v: 128 */
  float l2norm_eps;     /* q/k L2 norm epsilon (1e-6) */
  float norm_eps;       /* gated RMS norm epsilon (1e-6) */
} gdr_layer_desc;

/* Device workspace gdr_delta_layer_fwd needs for *d, in bytes. */
gdr_status gdr_delta_layer_workspace_size(const gdr_layer_desc* d, size_t* bytes);

/*
 * Prefill of one whole delta layer over a packed batch:
 *
 *   [qkv | z | b | a] = hidden W_in^T        (bf16 results; b, a widened to fp32)
 *   q, k, v, g, beta  = front(qkv, a, b)      (gdr_conv_gate_fused)
 *   o, S              = chunk recurrence      (gdr_chunk_fwd: chunk 64, q/k L2
 *                                              norm in the kernel, scale 1, fp32 o)
 *   y                 = gated RMS norm(o, z)  (gdr_gated_rmsnorm)
 *   out               = y W_out^T             (bf16)
 *
 * With C = (2*Hk + Hv)*d and V = Hv*d:
 *   hidden         [T, H] bf16
 *   w_in           [C + V + 2*Hv, H] bf16: rows for the C conv channels (q | k
 *                  | v blocks), then the V z channels, then b, then a
 *   conv_w         [C, 4] bf16;  A_log, dt_bias [Hv] fp32;  norm_w [d] fp32
 *   w_out          [H, V] bf16
 *   cu_seqlens     [N+1] int32 device array (required)
 *   conv_state_in / conv_state_out [N, C, 3] bf16 (NULL = zeros / not written)
 *   initial_state / final_state    [N, Hv, d, d] fp32 (NULL = zeros / not
 *                  written; may be the same pointer)
 *   out            [T, H] bf16
 *   workspace      >= gdr_delta_layer_workspace_size bytes, 256-byte aligned;
 *                  holds the intermediates of this call only
 *
 * Bit for bit the same as calling gdr_linear, gdr_conv_gate_fused,
 * gdr_chunk_fwd, gdr_gated_rmsnorm and gdr_linear in turn.  Errors: those of
 * the five steps; UNSUPPORTED unless d = 128.
 */
gdr_status gdr_delta_layer_fwd(const gdr_layer_desc* d, const void* hidden, const void* w_in, const void* conv_w,
                               const float* A_log, const float* dt_bias, const float* norm_w, const void* w_out,
                               const int32_t* cu_seqlens, const void* conv_state_in, void* conv_state_out,
                               const float* initial_state, float* final_state, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The global attention layer, every fourth layer of the hybrid decoder
 * (deepmagic page, architecture section; kongchang page, attention details):
 * grouped-query attention, 24 query / 4 key-value heads of dim 256, an RMS
 * norm on q and on k, rotary encoding on the first 64 dims of each head
 * (base 1e7), a sigmoid gate on the output.  For every query head h (key /
 * value head h / (Hq / Hk)) and token t at position p inside its sequence:
 *
 *   q' = rot_p(rmsnorm(q_t,h) * q_norm_w),  k'_s = rot_s(rmsnorm(k_s) * k_norm_w)
 *   out_t,h = softmax_s<=t(q' . k'_s / 16) v_s * sigmoid(gate_t,h)
 *
 * rmsnorm(x) = x / sqrt(mean(x^2) + eps) over the head's 256 dims; rot_p turns
 * the pairs (j, j + 32), j < 32, of the first 64 dims by p * base^(-j/32) and
 * leaves dims 64..255 alone.  q, k, v, gate and out are bf16; the norms and
 * rotation run in fp32 (angles reduced in fp64) and round q', k' to bf16;
 * scores and softmax are fp32; probabilities enter the value product as bf16.
 * ------------------------------------------------------------------------ */

typedef struct gdr_attn_desc {
  uint32_t struct_size; /* sizeof(gdr_attn_desc) */
  int32_t num_tokens;   /* prefill: T packed tokens; decode: N */
  int32_t num_seqs;     /* N */
  int32_t num_q_heads;  /* Hq (24) */
  int32_t num_kv_heads; /* Hk (4), Hq a multiple of it */
  int32_t head_dim;     /* 256 */
  int32_t cache_len;    /* slots per sequence in k_cache / v_cache (0 without a cache) */
  float norm_eps;       /* RMS norm epsilon (1e-6) */
  double rope_base;     /* 1e7 */
} gdr_attn_desc;

/*
 * The first step alone: q' and k' of every token of a packed batch
 * (positions restart at 0 in each sequence).
 *   q [T, Hq, 256], k [T, Hk, 256] bf16;  q_norm_w, k_norm_w [256] fp32
 *   cu_seqlens [N+1] int32 device array;  q_out [T, Hq, 256], k_out [T, Hk, 256] bf16
 * gdr_attn_prefill computes q' and k' with this same code.  Errors as
 * gdr_attn_prefill.
 */
gdr_status gdr_attn_qk_norm_rope(const gdr_attn_desc* d, const void* q, const void* k, const float* q_norm_w,
                                 const float* k_norm_w, const int32_t* cu_seqlens, void* q_out, void* k_out,
                                 void* stream);

/* Device workspace gdr_attn_prefill needs for *d, in bytes. */
gdr_status gdr_attn_prefill_workspace_size(const gdr_attn_desc* d, size_t* bytes);

/*
 * Causal prefill over a packed batch:
 *   q, gate      [T, Hq, 256] bf16;  k, v [T, Hk, 256] bf16
 *   q_norm_w, k_norm_w [256] fp32
 *   cu_seqlens   [N+1] int32 device array (positions restart at 0 in each sequence)
 *   out          [T, Hq, 256] bf16
 *   k_cache      [N, cache_len, Hk, 256] bf16 and
 *   v_cache      [N, Hk, cache_len / 32, 256, 32] bf16, or both NULL: when
 *                given, position p of sequence n receives its token p's k'
 *                and v, for every p < cache_len (ready for gdr_attn_decode);
 *                other positions are not written.  cache_len must be a
 *                multiple of 64.
 *                v_cache is blocked by 32 positions: position 32 b + i of
 *                dim d is element [n][h][b][d][8 ((i mod 16) / 4) +
 *                4 (i / 16) + i mod 4], the order in which the decode's value
 *                product takes the keys, so it reads each block as one
 *                contiguous 16 KiB run.
 *   workspace    >= gdr_attn_prefill_workspace_size bytes, 256-byte aligned
 * Errors: INVALID_ARG for NULL required pointers, misalignment (16 bytes),
 * a short workspace, one cache pointer without the other, cache_len not a
 * multiple of 64; UNSUPPORTED unless head_dim = 256 and Hq is a multiple of Hk.
 */
gdr_status gdr_attn_prefill(const gdr_attn_desc* d, const void* q, const void* k, const void* v, const void* gate,
                            const float* q_norm_w, const float* k_norm_w, const int32_t* cu_seqlens, void* out,
                            void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace gdr_attn_decode needs for *d (num_seqs, heads, cache_len), in bytes. */
gdr_status gdr_attn_decode_workspace_size(const gdr_attn_desc* d, size_t* bytes);

/*
 * One decode token per sequence (d->num_tokens = d->num_seqs = N):
 *   q, gate      [N, Hq, 256] bf16;  k, v [N, Hk, 256] bf16 (the new token)
 *   k_cache      [N, cache_len, Hk, 256] bf16, v_cache [N, Hk, cache_len / 32,
 *                256, 32] bf16 (the layouts gdr_attn_prefill fills), updated IN
 *                PLACE: the token's k' and v are written at position
 *                cache_lens[n]
 *   cache_lens   [N] int32 device array: tokens already cached; the token sits
 *                at that position and attends to positions 0 .. cache_lens[n].
 *                A value outside [0, cache_len) marks a padding row: its out
 *                is zero and neither cache is written.  Not modified: the
 *                caller advances it.
 *   out          [N, Hq, 256] bf16
 *   workspace    >= gdr_attn_decode_workspace_size bytes, 256-byte aligned
 * The keys are split into pieces of 256 to 2048 positions (chosen from N, Hk
 * and cache_len), each attended on its own and merged: exactly the softmax
 * over all of them, up to rounding.
 * Errors: as gdr_attn_prefill; INVALID_ARG also for cache_len <= 0.
 */
gdr_status gdr_attn_decode(const gdr_attn_desc* d, const void* q, const void* k, const void* v, const void* gate,
                           const float* q_norm_w, const float* k_norm_w, void* k_cache, void* v_cache,
                           const int32_t* cache_lens, void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
