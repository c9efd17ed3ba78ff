/* Host-side checks of the C-ABI (include/seer.h) for a sanitizer build: every
 * call here must return before anything reaches the GPU (argument, size,
 * capacity and workspace checks, size functions, status helpers).  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host code by
 * tests/test_host_sanitize.py; exits non-zero on the first wrong status. */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "seer.h"

static int g_checks = 0;

#define CHECK(expr, want)                                                                 \
  do {                                                                                    \
    const long long got_ = (long long)(expr);                                             \
    ++g_checks;                                                                           \
    if (got_ != (long long)(want)) {                                                      \
      fprintf(stderr, "FAIL line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_,      \
              (long long)(want));                                                         \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

/* Never dereferenced on these paths: only checked for NULL and alignment. */
static _Alignas(256) char buf[4096];
#define P ((void*)buf)
#define F ((float*)buf)
#define I ((int32_t*)buf)
#define MIS16 ((void*)(buf + 8))   /* 8-byte aligned, not 16 */
#define MIS256 ((void*)(buf + 16)) /* 16-byte aligned, not 256 */

int main(void) {
  const float nanf_ = NAN, inff_ = INFINITY;

  /* Status helpers. */
  CHECK(strcmp(seer_status_string(SEER_OK), "SEER_OK"), 0);
  CHECK(strcmp(seer_status_string(99), "SEER_ERR_UNKNOWN"), 0);
  CHECK(seer_version() > 0, 1);
  CHECK(seer_topk_budget(-1, 0.1, 1), -1);
  CHECK(seer_topk_budget(10, 0.0, 1), -1);
  CHECK(seer_topk_budget(10, 1.5, 1), -1);
  CHECK(seer_topk_budget(10, nanf_, 1), -1);
  CHECK(seer_topk_budget(0, 0.5, 1), 0);
  CHECK(seer_topk_budget(1, 0.1, 1), 1);
  CHECK(seer_topk_budget(512, 0.1, 1), 52);
  CHECK(seer_topk_budget(100, 0.001, 1), 2);
  CHECK(seer_topk_budget(INT_MAX, 1.0, 1), INT_MAX);
  CHECK(seer_list_flags_status(0), SEER_OK);
  CHECK(seer_list_flags_status(SEER_LIST_CAPACITY | SEER_LIST_REPEAT), SEER_ERR_CAPACITY);
  CHECK(seer_list_flags_status(SEER_LIST_REPEAT), SEER_ERR_INVALID_ARG);
  CHECK(seer_list_flags_status(SEER_LIST_UNSORTED | SEER_LIST_BAD_ENTRY | SEER_LIST_BAD_COUNT),
        SEER_OK);

  /* Mask build. */
  CHECK(seer_build_mask(F, -1, 1, 4, 4, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, 1, 1, 4, 3, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, 1, 1, 4097, 4097, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, 4097, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_build_mask(F, 1, 1, 4, 4, 7, 0.f, 0.5, 1, I, I, 4, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, INT_MAX, INT_MAX, 2, 2, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, 2, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_build_mask(F, 1, 1, 4, 4, SEER_MASK_TOPK, 0.f, 0.0, 1, I, I, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, 1, 1, 4, 4, SEER_MASK_TOPK, 0.f, 1.5, 1, I, I, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, 1, 1, 4, 4, SEER_MASK_THRESHOLD, nanf_, 0.5, 1, I, I, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, 1, 1, 4, 4, SEER_MASK_THRESHOLD, 0.1f, 0.5, 1, I, I, 0, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_build_mask(NULL, 0, 1, 4, 4, SEER_MASK_TOPK, 0.f, 0.5, 1, NULL, NULL, 4, 0),
        SEER_OK);
  CHECK(seer_build_mask(NULL, 1, 1, 4, 4, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask(F, 1, 1, 512, 512, SEER_MASK_TOPK, 0.f, 0.1, 1, I, I, 51, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_build_mask(F, 1, 1, 8, 8, SEER_MASK_THRESHOLD, 0.1f, 0.5, 1, I, I, 1, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_build_mask_need(F, 1, 1, 4, 4, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, NULL, 4, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_build_mask_need(F, 0, 1, 4, 4, SEER_MASK_TOPK, 0.f, 0.5, 1, I, I, NULL, 4, 0),
        SEER_OK);

  /* List validation (host checks only: a valid call launches). */
  CHECK(seer_validate_lists(I, I, NULL, -1, 1, 4, 4, NULL, I, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_validate_lists(I, I, NULL, 1, 1, 4, 0, NULL, I, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_validate_lists(I, I, NULL, 1, 1, 4, 4, NULL, NULL, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_validate_lists(NULL, I, NULL, 1, 1, 4, 4, NULL, I, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_validate_lists(I, I, NULL, INT_MAX, INT_MAX, 2, 4, NULL, I, 0),
        SEER_ERR_UNSUPPORTED);

  /* Sparse prefill. */
  CHECK(seer_sparse_prefill_workspace_size(-1, 1, 1, 64), 0);
  CHECK(seer_sparse_prefill_workspace_size(1, 3, 2, 64), 0);
  CHECK(seer_sparse_prefill_workspace_size(1, 32, 8, 32768), 262400);
  CHECK(seer_sparse_prefill_workspace_size(1, 1, 1, INT_MAX) > 0, 1);
  CHECK(seer_sparse_prefill_workspace_size(INT_MAX, 1, 1, INT_MAX), 0);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, -1, 128, 1.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 0, 1, 64, 128, 1.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 3, 2, 64, 128, 1.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, 0.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, nanf_, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 96, 1.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_sparse_prefill(NULL, NULL, NULL, 0, 1, 1, 64, 128, 1.f, NULL, NULL, 4, NULL, NULL,
                            0, 0),
        SEER_OK);
  CHECK(seer_sparse_prefill(NULL, P, P, 1, 1, 1, 64, 128, 1.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(MIS16, P, P, 1, 1, 1, 64, 128, 1.f, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, 1.f, I, I, 0, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, 1.f, NULL, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, 1.f, I, I, 4, P, NULL, 1 << 20, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, 1.f, I, I, 4, P, P, 16, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, 64, 128, 1.f, I, I, 4, P, MIS256, 1 << 20, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_sparse_prefill(P, P, P, 1, 1, 1, INT_MAX, 128, 1.f, I, I, 4, P, P, 16, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_sparse_prefill(P, P, P, INT_MAX, 1, 1, INT_MAX, 128, 1.f, I, I, 4, P, P, 16, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_sparse_prefill_block(P, P, P, 1, 1, 1, 64, 128, 1.f, 32, I, I, 4, P, P, 1 << 20, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_sparse_prefill_noalloc(P, P, P, 1, 1024, 1, 32768, 128, 1.f, I, I, 52, P, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_sparse_prefill_noalloc(P, P, P, 1, 1, 1, 64, 128, 1.f, NULL, I, 4, P, 0),
        SEER_ERR_INVALID_ARG);

  /* Pooled map and target. */
  CHECK(seer_pooled_attn_map_workspace_size(-1, 1, 64), 0);
  CHECK(seer_pooled_attn_map_workspace_size(1, 1, 128), 3 * 64 * 4 + 256);
  CHECK(seer_pooled_attn_map(P, P, P, 1, 1, 1, 64, 128, 1.f, P, NULL, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_pooled_attn_map(P, P, P, 1, 1, 1, 64, 128, 1.f, P, F, P, 16, 0), SEER_ERR_WORKSPACE);
  CHECK(seer_pooled_target_mse(F, F, -1, 1, 4, F, F, F, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_pooled_target_mse(NULL, NULL, 0, 1, 4, NULL, NULL, NULL, 0), SEER_OK);
  CHECK(seer_pooled_target_mse(NULL, F, 1, 1, 4, F, F, F, 0), SEER_ERR_INVALID_ARG);
  CHECK(seer_pooled_target_mse(F, NULL, 1, 1, 4, F, F, F, 0), SEER_ERR_INVALID_ARG);

  /* AttnGate (prefill). */
  CHECK(seer_attn_gate_workspace_size(1, 3, 2, 64, 128), 0);
  CHECK(seer_attn_gate_workspace_size(1, 2, 1, 64, 128) > 0, 1);
  CHECK(seer_attn_gate_mask_workspace_size(1, 2, 1, 640, 64, 0) >
            seer_attn_gate_mask_workspace_size(1, 2, 1, 640, 64, 1),
        1);
  CHECK(seer_attn_gate_mask_pass_workspace_size(1, 2, 1, 640, 64, 0), 0);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 96, F, F, 64, 1.f, 1e4f, F, P, 1 << 20, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 128, F, F, 48, 1.f, 1e4f, F, P, 1 << 20, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 128, F, F, 64, inff_, 1e4f, F, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 128, F, F, 64, 1.f, 1.f, F, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_scores(NULL, NULL, 0, 2, 1, 64, 128, NULL, NULL, 64, 1.f, 1e4f, NULL,
                              NULL, 0, 0),
        SEER_OK);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 128, F, F, 64, 1.f, 1e4f, NULL, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 128, (float*)MIS16, F, 64, 1.f, 1e4f, F, P,
                              1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_scores(P, P, 1, 2, 1, 64, 128, F, F, 64, 1.f, 1e4f, F, P, 16, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_attn_gate_mask(P, P, 1, 1, 1, 4097 * 64, 128, F, F, 64, 1.f, 1e4f, SEER_MASK_TOPK,
                            0.f, 0.5, 1, I, I, 4097, F, P, 1 << 20, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_attn_gate_mask(P, P, 1, 1, 1, 640, 128, F, F, 64, 1.f, 1e4f, 9, 0.f, 0.5, 1, I, I,
                            10, F, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_mask(P, P, 1, 1, 1, 640, 128, F, F, 64, 1.f, 1e4f, SEER_MASK_TOPK, 0.f,
                            0.5, 1, I, I, 0, F, P, 1 << 20, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_attn_gate_mask(P, P, 1, 1, 1, 640, 128, F, F, 64, 1.f, 1e4f, SEER_MASK_TOPK, 0.f,
                            0.5, 1, I, I, 4, F, P, 1 << 20, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_attn_gate_mask(P, P, 1, 1, 1, 640, 128, F, F, 64, 1.f, 1e4f, SEER_MASK_THRESHOLD,
                            0.1f, 0.5, 1, I, I, 1, F, P, 1 << 20, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_attn_gate_mask(P, P, 1, 1, 1, 640, 128, F, F, 64, 1.f, 1e4f, SEER_MASK_THRESHOLD,
                            0.1f, 0.5, 1, I, I, 10, F, P, 16, 0),
        SEER_ERR_WORKSPACE);

  /* Decode. */
  CHECK(seer_attn_gate_decode_keys_workspace_size(1, 1, 4096, 128, 96), 0);
  CHECK(seer_attn_gate_decode_keys_workspace_size(1, 1, 0, 128, 64), 0);
  CHECK(seer_attn_gate_decode_keys(P, I, 1, 1, 4096, 128, F, 64, 1e4f, 64, 0, F, P, 16, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_attn_gate_decode_keys(P, I, 1, 1, 4096, 128, F, 64, nanf_, 64, 0, F, P, 1 << 20, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_decode_scores(P, F, I, 1, 2, 1, 4096, 128, F, 64, 0.f, 1e4f, 64, F, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_decode_mask(P, F, I, 1, 2, 1, 4096, 128, F, 64, 1.f, 1e4f, 64, 9, 0.f,
                                   8, 1, I, I, 8, F, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_decode_mask(P, F, I, 1, 2, 1, 4096, 128, F, 64, 1.f, 1e4f, 64,
                                   SEER_MASK_TOPK, 0.f, 0, 1, I, I, 8, F, 0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_attn_gate_decode_mask(P, F, I, 1, 2, 1, 4096, 128, F, 64, 1.f, 1e4f, 64,
                                   SEER_MASK_TOPK, 0.f, 8, 1, I, I, 0, F, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_attn_gate_decode_mask(P, F, I, INT_MAX, 2, 1, 4096, 128, F, 64, 1.f, 1e4f, 64,
                                   SEER_MASK_TOPK, 0.f, 8, 1, I, I, 8, F, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_build_mask_decode(F, I, 1, 1, 64, 96, SEER_MASK_TOPK, 0.f, 8, 1, I, I, 8, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_build_mask_decode(F, I, 1, 1, 4097, 64, SEER_MASK_TOPK, 0.f, 8, 1, I, I, 8, 0),
        SEER_ERR_UNSUPPORTED);
  CHECK(seer_build_mask_decode(F, I, 1, 1, 640, 64, SEER_MASK_TOPK, 0.f, 64, 1, I, I, 63, 0),
        SEER_ERR_CAPACITY);
  CHECK(seer_sparse_decode_workspace_size(1, 4, 2, 4096, 128, 3, 8, 64), 0);
  CHECK(seer_sparse_decode_workspace_size(1, 18, 2, 4096, 128, 18, 8, 64), 0);
  CHECK(seer_sparse_decode_workspace_size(1, 4, 2, 4096, 128, 4, 8, 64) > 0, 1);
  CHECK(seer_sparse_decode(P, P, P, I, 1, 4, 2, 4096, 128, nanf_, 64, I, I, 4, 8, P, P, 1 << 20,
                           0),
        SEER_ERR_INVALID_ARG);
  CHECK(seer_sparse_decode(P, P, P, I, 1, 4, 2, 4096, 128, 1.f, 64, I, I, 4, 8, P, P, 16, 0),
        SEER_ERR_WORKSPACE);
  CHECK(seer_sparse_decode(P, P, P, I, 1, 4, 2, 4096, 128, 1.f, 64, I, I, 4, 8, MIS16, P,
                           1 << 20, 0),
        SEER_ERR_INVALID_ARG);

  printf("host checks: %d passed\n", g_checks);
  return 0;
}
