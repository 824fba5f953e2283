/* abi_from_c.c -- include/lsa.h used from plain C99: the header compiles as
 * C, every call below links against liblsa.so, and the host-side calls that
 * need no GPU (version, status names, keep counts, schedule, workspace sizes,
 * the attention plan, argument checks) behave as the header states.  Prints
 * "abi_from_c ok" and exits 0, or names the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "../../include/lsa.h"

static int failed = 0;
#define CHECK(cond)                                             \
  do {                                                          \
    if (!(cond)) {                                              \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      failed = 1;                                               \
    }                                                           \
  } while (0)

static lsa_shape headline(void) {
  lsa_shape s;
  memset(&s, 0, sizeof s);
  s.batch = 16;
  s.chunk_size = 64;
  s.index_dim = 128;
  s.num_q_heads = 16;
  s.head_dim_qk = 128;
  s.head_dim_v = 128;
  s.v_aliases_k = 0;
  s.dtype = LSA_DTYPE_BF16;
  s.softmax_scale = 0.08838834764831845f;
  s.max_chunks = 2048;
  s.max_k = 276;
  s.total_chunks = 16 * 2048;
  s.total_k = 16 * 276;
  s.attn_tiles_per_block = 0;
  s.flags = LSA_SHAPE_UNIFORM;
  return s;
}

int main(void) {
  CHECK(lsa_abi_version() >= 4);
  CHECK(strcmp(lsa_status_string(LSA_OK), "LSA_OK") == 0);
  CHECK(strcmp(lsa_status_string(LSA_ERR_WORKSPACE_TOO_SMALL), "LSA_ERR_WORKSPACE_TOO_SMALL") == 0);
  /* the keep counts of the workloads: 13.5 % of 2048, 10 % of 8192, 8 % of 8192 */
  CHECK(lsa_keep_count(2048, 135, 1000, 0) == 276);
  CHECK(lsa_keep_count(8192, 10, 100, 0) == 819);
  CHECK(lsa_keep_count(8192, 8, 100, 0) == 655);
  CHECK(lsa_keep_count(0, 1, 2, 0) == 0);
  CHECK(lsa_reindex_due(128, 64) == 1 && lsa_reindex_due(129, 64) == 0);
  CHECK(lsa_reindex_due(5, 0) == -1);

  lsa_shape s = headline();
  const size_t ws = lsa_workspace_bytes(&s);
  CHECK(ws > 0);
  lsa_attn_plan_info info;
  CHECK(lsa_attention_plan(&s, &info) == LSA_OK);
  CHECK(info.kernel == LSA_ATTN_KERNEL_MQA && info.tiles_per_chunk == 2);
  CHECK(info.grid > 0 && info.partial_rows >= info.grid);
  CHECK(lsa_attention_plan(&s, NULL) == LSA_ERR_INVALID_ARGUMENT);

  /* argument checks run on the host before anything is enqueued */
  lsa_shape bad = s;
  bad.num_q_heads = 100;
  CHECK(lsa_workspace_bytes(&bad) == 0);
  CHECK(lsa_attention_plan(&bad, &info) != LSA_OK);
  CHECK(lsa_score(&s, NULL, NULL, NULL, NULL, NULL) == LSA_ERR_INVALID_ARGUMENT);
  CHECK(lsa_select_topk(NULL, NULL, NULL, NULL, NULL, NULL) == LSA_ERR_INVALID_ARGUMENT);
  CHECK(lsa_decode_step(&s, NULL, NULL, 0, NULL) == LSA_ERR_INVALID_ARGUMENT);

  if (failed) return 1;
  printf("abi_from_c ok\n");
  return 0;
}
