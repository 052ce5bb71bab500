/* A plain C99 caller of libs3r: include/s3r.h must compile as C, and the
 * library must be callable without C++ or torch. Only calls that fail host
 * validation, and the host-only queries, are made, so no GPU is needed.
 * Prints "ok" and returns 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "s3r.h"

#define CHECK(c)                                                \
  do {                                                          \
    if (!(c)) {                                                 \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                 \
    }                                                           \
  } while (0)

int main(void) {
  s3r_paged_kv kv;
  void* fake = (void*)(uintptr_t)0x1000; /* never dereferenced */
  memset(&kv, 0, sizeof kv);
  kv.num_seqs = 2;
  kv.num_q_heads = 8;
  kv.num_kv_heads = 2;
  kv.head_dim = 128;
  kv.page_size = 16;
  kv.max_pages_per_seq = 64;
  kv.kv_dtype = S3R_BF16;
  kv.k_pool = fake;
  kv.v_pool = fake;
  kv.page_table = (const int32_t*)fake;
  kv.seq_lens = (const int32_t*)fake;

  CHECK(s3r_version() >= 200);
  CHECK(strcmp(s3r_status_string(S3R_OK), "S3R_OK") == 0);
  CHECK(strcmp(s3r_status_string(S3R_ERR_UNSUPPORTED), "S3R_ERR_UNSUPPORTED") == 0);

  /* host-only workspace queries */
  CHECK(s3r_spec_sample_workspace(2, 4, 1000) > 0);
  CHECK(s3r_spec_sample_workspace(2, 17, 1000) == 0); /* gamma out of range */
  CHECK(s3r_page_select_workspace(&kv, 256) > 0);
  CHECK(s3r_page_select_workspace(NULL, 256) == 0);

  /* validation failures, before any HIP call */
  CHECK(s3r_page_select(NULL, fake, fake, 256, 0.1f, fake, fake, fake, 1u << 20, NULL) ==
        S3R_ERR_INVALID_ARGUMENT);
  CHECK(s3r_page_select(&kv, fake, fake, 8, 0.1f, fake, fake, fake, 1u << 20, NULL) ==
        S3R_ERR_INVALID_ARGUMENT); /* budget below one page */
  CHECK(s3r_dense_verify_attn(&kv, fake, 0, 0.1f, S3R_F32, fake, fake, 1u << 20, NULL) ==
        S3R_ERR_INVALID_ARGUMENT); /* no queries */
  CHECK(s3r_dense_verify_attn(&kv, fake, 17, 0.1f, S3R_F32, fake, fake, 1u << 20, NULL) ==
        S3R_ERR_UNSUPPORTED); /* G * n_q = 4 * 17 = 68 rows, past the 64 supported */
  kv.head_dim = 96;
  CHECK(s3r_sparse_draft_attn(&kv, fake, (const int32_t*)fake, 4, 0.1f, S3R_F32, fake, fake, 1u << 20,
                              NULL) == S3R_ERR_UNSUPPORTED);
  kv.head_dim = 128;
  CHECK(s3r_spec_sample(2, 4, 1000, (const float*)fake, (const float*)fake, (const int32_t*)fake, 0.0f,
                        0, 0, (int32_t*)fake, (int32_t*)fake, fake, 1u << 20, NULL) ==
        S3R_ERR_INVALID_ARGUMENT); /* temperature 0 */
  CHECK(s3r_kv_commit(&kv, fake, fake, NULL, 1, NULL, NULL) == S3R_ERR_INVALID_ARGUMENT);

  /* the drafter's draws, the acceptance rate and the allocation-free sampler */
  CHECK(s3r_draft_sample_workspace(2, 4, 151936) > 0);
  CHECK(s3r_draft_sample(2, 4, 1000, (const float*)fake, 1.0f, 0, 0, -1, (int32_t*)fake, fake, 1u << 20,
                         NULL) == S3R_ERR_INVALID_ARGUMENT); /* first_slot < 0 */
  CHECK(s3r_draft_sample(1 << 20, 1 << 10, 1 << 20, (const float*)fake, 1.0f, 0, 0, 0, (int32_t*)fake,
                         fake, (size_t)-1, NULL) == S3R_ERR_UNSUPPORTED); /* grid past 2^31 blocks */
  CHECK(s3r_acceptance_rate_workspace(2, 4, 151936) > 0);
  CHECK(s3r_acceptance_rate(2, 4, 1000, (const float*)fake, (const float*)fake, 1.0f,
                            (double*)((uintptr_t)fake + 4), fake, 1u << 20, NULL) ==
        S3R_ERR_INVALID_ARGUMENT); /* misaligned alpha */
  CHECK(s3r_spec_sample_noalloc_max_workspace() == ((size_t)4 << 20));
  CHECK(s3r_spec_sample_noalloc(4096, 16, 151936, (const float*)fake, (const float*)fake,
                                (const int32_t*)fake, 1.0f, 0, 0, (int32_t*)fake, (int32_t*)fake, NULL) ==
        S3R_ERR_WORKSPACE_TOO_SMALL);

  /* workspace queries on large shapes: sizes, not overflow */
  kv.num_seqs = 4096;
  kv.max_pages_per_seq = 32768;
  kv.total_pages_hint = 1 << 30;
  CHECK(s3r_attn_workspace(&kv, 5, 32768) > 0);
  CHECK(s3r_sparse_draft_step_workspace(&kv, 1 << 20) > 0);
  CHECK(s3r_page_select_workspace(&kv, 2048) == (size_t)4096 * 2 * 32768 * 4);
  kv.total_pages_hint = 4096 * 100; /* ragged: the order is reserved too */
  CHECK(s3r_attn_workspace(&kv, 1, 128) > 0);
  puts("ok");
  return 0;
}
