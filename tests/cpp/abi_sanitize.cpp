// The C ABI's host-side argument checks under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; no GPU needed: every call
// below fails validation before any HIP call, or, in debug mode, at the
// first HIP call).  Built and run by tests/test_sanitized_abi.py.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdr.h"
#include "host_checks.h"

static int failures = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      fprintf(stderr, "FAILED line %d: %s (%s)\n", __LINE__, #cond, gdr_last_error()); \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

static void* const FAKE = (void*)0x7F0000000000ull;

static gdr_desc desc() {
  gdr_desc d;
  memset(&d, 0, sizeof d);
  d.struct_size = sizeof d;
  d.batch = 1;
  d.seq_len = 128;
  d.num_seqs = 1;
  d.num_k_heads = 16;
  d.num_v_heads = 48;
  d.head_dim_k = d.head_dim_v = 128;
  d.chunk_size = 64;
  d.qkv_dtype = GDR_BF16;
  d.out_dtype = GDR_F32;
  d.use_qk_l2norm = 1;
  d.scale = 1.f;
  d.l2norm_eps = 1e-6f;
  return d;
}

static void index_checks() {
  char msg[256];
  const int32_t good[] = {0, 3, 3, 10};
  EXPECT(gdr::check_cu_seqlens(good, 3, 10, "cu", msg, sizeof msg));
  const int32_t start[] = {1, 3, 10};
  EXPECT(!gdr::check_cu_seqlens(start, 2, 10, "cu", msg, sizeof msg) && strstr(msg, "must be 0"));
  const int32_t down[] = {0, 5, 4, 10};
  EXPECT(!gdr::check_cu_seqlens(down, 3, 10, "cu", msg, sizeof msg) && strstr(msg, "decreases"));
  EXPECT(!gdr::check_cu_seqlens(good, 3, 11, "cu", msg, sizeof msg) && strstr(msg, "token count"));
  const int32_t idx_ok[] = {3, -1, 0, 7, 1};  // -1 and 7 are padding rows of a 4-slot pool
  EXPECT(gdr::check_state_indices(idx_ok, 5, 4, msg, sizeof msg));
  const int32_t idx_dup[] = {2, 0, 2};
  EXPECT(!gdr::check_state_indices(idx_dup, 3, 4, msg, sizeof msg) && strstr(msg, "twice"));
  EXPECT(gdr::check_state_indices(idx_dup, 3, 0, msg, sizeof msg));  // empty pool: all padding
}

static void abi_checks() {
  gdr_desc d = desc();
  size_t n = 0;
  EXPECT(gdr_chunk_fwd_workspace_size(&d, &n) == GDR_OK && n > 0);
  EXPECT(gdr_chunk_fwd_workspace_size(NULL, &n) == GDR_ERR_INVALID_ARG);
  EXPECT(gdr_chunk_fwd_workspace_size(&d, NULL) == GDR_ERR_INVALID_ARG);
  gdr_desc bad = d;
  bad.num_v_heads = 40;
  EXPECT(gdr_chunk_fwd(&bad, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, NULL, 0, NULL) ==
         GDR_ERR_INVALID_ARG);
  bad = d;
  bad.head_dim_k = bad.head_dim_v = 96;
  EXPECT(gdr_chunk_fwd(&bad, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, NULL, 0, NULL) ==
         GDR_ERR_UNSUPPORTED);
  bad = d;
  bad.struct_size = 8;
  EXPECT(gdr_chunk_fwd_prepare(&bad, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, NULL, 0,
                               NULL) == GDR_ERR_INVALID_ARG);
  // short workspace, missing tensors, misaligned pointers
  EXPECT(gdr_chunk_fwd(&d, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, FAKE, 10, NULL) ==
         GDR_ERR_INVALID_ARG);
  EXPECT(strstr(gdr_last_error(), "workspace") != NULL);
  EXPECT(gdr_chunk_fwd(&d, NULL, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, NULL, 0, NULL) ==
         GDR_ERR_INVALID_ARG);
  EXPECT(gdr_chunk_fwd(&d, (char*)FAKE + 2, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, FAKE,
                       n, NULL) == GDR_ERR_INVALID_ARG);
  // beyond the no-alloc scratch
  gdr_desc big = d;
  big.seq_len = 1 << 20;
  EXPECT(gdr_chunk_fwd_noalloc(&big, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, NULL, FAKE, NULL) ==
         GDR_ERR_INVALID_ARG);
  // decode
  gdr_desc dd = d;
  dd.seq_len = 1;
  dd.batch = dd.num_seqs = 4;
  EXPECT(gdr_recurrent_step(&dd, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, FAKE, NULL) ==
         GDR_ERR_INVALID_ARG);
  EXPECT(gdr_recurrent_step_indexed(&dd, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, (float*)FAKE, -1,
                                    (int32_t*)FAKE, FAKE, NULL) == GDR_ERR_INVALID_ARG);
  // conv front and norm back
  gdr_conv_desc cd;
  memset(&cd, 0, sizeof cd);
  cd.struct_size = sizeof cd;
  cd.num_tokens = 10;
  cd.num_seqs = 1;
  cd.num_k_heads = 16;
  cd.num_v_heads = 48;
  cd.head_dim = 128;
  EXPECT(gdr_conv_gate_fused(&cd, FAKE, FAKE, NULL, NULL, NULL, (float*)FAKE, (float*)FAKE, (float*)FAKE,
                             (float*)FAKE, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL) ==
         GDR_ERR_INVALID_ARG);
  gdr_norm_desc nd;
  memset(&nd, 0, sizeof nd);
  nd.struct_size = sizeof nd;
  nd.num_tokens = 4;
  nd.num_heads = 48;
  nd.head_dim = 96;
  EXPECT(gdr_gated_rmsnorm(&nd, FAKE, FAKE, (float*)FAKE, FAKE, NULL) == GDR_ERR_UNSUPPORTED);
  EXPECT(strcmp(gdr_status_string(-3), "GDR_ERR_HIP") == 0);
  EXPECT(gdr_abi_version() == GDR_ABI_VERSION);
}

// Debug mode: a call that passes the host checks first reads cu_seqlens
// back.  On a host without a GPU that read fails and the call returns
// GDR_ERR_HIP naming the debug mode -- before any kernel launch.
static void debug_mode(bool have_gpu) {
  setenv("GDR_DEBUG_CHECKS", "1", 1);
  gdr_desc d = desc();
  d.num_seqs = 2;
  size_t n = 0;
  EXPECT(gdr_chunk_fwd_workspace_size(&d, &n) == GDR_OK);
  const int32_t cu[3] = {0, 100, 128};  // host memory
  const gdr_status st = gdr_chunk_fwd(&d, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, cu, FAKE, FAKE,
                                      n, NULL);
  if (!have_gpu) {
    EXPECT(st == GDR_ERR_HIP);
    EXPECT(strstr(gdr_last_error(), "GDR_DEBUG_CHECKS") != NULL);
  }
  // argument errors still come first
  gdr_desc bad = d;
  bad.num_v_heads = 40;
  EXPECT(gdr_chunk_fwd(&bad, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, NULL, NULL, cu, FAKE, FAKE, n, NULL) ==
         GDR_ERR_INVALID_ARG);
  unsetenv("GDR_DEBUG_CHECKS");
}

int main(int argc, char** argv) {
  const bool have_gpu = argc > 1 && strcmp(argv[1], "--gpu") == 0;
  index_checks();
  abi_checks();
  if (!have_gpu) debug_mode(false);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_sanitize: all checks passed\n");
  return 0;
}
