/* A plain C caller of libpagedattn: the host-side calls (block manager, the
 * engine in plan-only mode, size queries and argument checks) through the
 * headers alone, no C++ and no Python.  Exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pagedattn.h"
#include "pagedattn_blocks.h"
#include "pagedattn_engine.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main(void) {
  /* block manager: the pool picture of a 10-block pool, 16-token blocks */
  pa_block_manager *bm = pa_bm_create(10, 16);
  CHECK(bm != NULL);
  int32_t slots[40];
  CHECK(pa_bm_add_sequence(bm, 1, 40, slots) == PA_OK);  /* 3 blocks, LIFO: 9, 8, 7 */
  int32_t table[8];
  CHECK(pa_bm_block_table(bm, 1, table, 8) == 3);
  CHECK(table[0] == 9 && table[1] == 8 && table[2] == 7);
  CHECK(slots[0] == 9 * 16 && slots[17] == 8 * 16 + 1 && slots[39] == 7 * 16 + 7);
  CHECK(pa_bm_fork(bm, 1, 2) == PA_OK);
  int32_t slot, src, dst;
  CHECK(pa_bm_append_slot(bm, 2, &slot, &src, &dst) == PA_OK);  /* shared partial block: copy */
  CHECK(src == 7 && dst == 6 && slot == 6 * 16 + 8);
  pa_block_stats st;
  CHECK(pa_bm_stats(bm, &st) == PA_OK);
  CHECK(st.free_blocks == 6 && st.shared_blocks == 2 && st.num_sequences == 2);
  CHECK(pa_bm_free_sequence(bm, 1) == PA_OK && pa_bm_free_sequence(bm, 2) == PA_OK);
  CHECK(pa_bm_num_free_blocks(bm) == 10);
  CHECK(pa_bm_free_sequence(bm, 2) == PA_ERR_NO_SEQ);
  pa_bm_destroy(bm);

  /* engine, plan only: two requests, one with two samples */
  pa_engine_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.num_blocks = 64; cfg.block_size = 16; cfg.num_q_heads = 8; cfg.num_kv_heads = 2;
  cfg.head_dim = 128; cfg.dtype = PA_BF16; cfg.max_batch = 8; cfg.max_context_len = 256;
  cfg.max_prompt_rows = 256; cfg.partition_size = 0; cfg.device = 0;
  cfg.k_scale = 1.f; cfg.v_scale = 1.f; cfg.host_plan = 1;
  pa_engine *e = NULL;
  CHECK(pa_engine_create(&cfg, NULL, NULL, &e) == PA_OK && e != NULL);
  CHECK(pa_engine_submit(e, 5, 20, 3, 2) == PA_OK);
  CHECK(pa_engine_submit(e, 6, 16, 2, 1) == PA_OK);
  CHECK(pa_engine_submit(e, 6, 16, 2, 1) == PA_ERR_SEQ_EXISTS);
  pa_step_info info;
  CHECK(pa_engine_step(e, NULL, NULL, NULL, NULL, NULL, 0.1f, NULL, NULL, &info) == PA_OK);
  CHECK(info.batch == 3 && info.admitted == 2 && info.prompt_rows == 36);
  CHECK(info.context_lens[0] == 21 && info.context_lens[2] == 17);
  CHECK(info.num_copies == 1);  /* the fork copies the shared partial block */
  int steps = 1;
  while (pa_engine_num_running(e) > 0 || pa_engine_num_waiting(e) > 0) {
    CHECK(pa_engine_step(e, NULL, NULL, NULL, NULL, NULL, 0.1f, NULL, NULL, &info) == PA_OK);
    CHECK(++steps < 10);
  }
  CHECK(steps == 3);
  pa_engine_destroy(e);

  /* size queries and argument checks of the device calls (nothing launched) */
  CHECK(paged_attention_num_partitions(256, 8, 8192, 0) == 2);
  CHECK(paged_attention_workspace_size(256, 32, 8, 128, 8192, 0) ==
        (size_t)256 * 32 * 2 * 130 * 4 + (size_t)256 * 2 * 4); /* partials + dispatch list */
  CHECK(paged_attention_multi_query_partitions(256, 32, 8, 5, 8192, 0) == 2);
  /* shared prefixes: one more partial slot per row, four list entries per group */
  CHECK(paged_attention_prefix_workspace_size(256, 32, 8, 128, 8192, 0, 16, PA_BF16) ==
        (size_t)256 * 32 * 3 * 130 * 4 + (size_t)(256 * 2 + 4 * 16) * 4);
  CHECK(paged_attention_prefix_workspace_size(256, 32, 8, 128, 8192, 0, 16, PA_F32) ==
        paged_attention_workspace_size(256, 32, 8, 128, 8192, 0));
  CHECK(paged_attention_decode_prefix(NULL, NULL, NULL, NULL, NULL, NULL, 3, NULL, NULL, 0.1f, 1.f,
                                      1.f, NULL, 2, 8, 2, 128, 16, 8, 4, 64, PA_BF16, 0, NULL, 0,
                                      NULL) == PA_ERR_SHAPE); /* more groups than sequences */
  CHECK(paged_attention_decode(NULL, NULL, NULL, NULL, NULL, 0.1f, NULL, 1, 4, 2, 96, 16, 8, 4,
                               64, PA_BF16, 0, NULL, 0, NULL) == PA_ERR_UNSUPPORTED);
  CHECK(kv_cache_write_fp8(NULL, NULL, NULL, 1, NULL, NULL, 8, 16, 2, 128, PA_BF16, 0.f, 1.f,
                           NULL) == PA_ERR_SHAPE); /* a zero scale */
  CHECK(kv_cache_append(NULL, 0, NULL, NULL, NULL, 0, NULL, NULL, 8, 16, 2, 128, PA_BF16, PA_BF16,
                        1.f, 1.f, NULL, NULL) == PA_OK); /* nothing to do */
  CHECK(kv_cache_append(NULL, 2, NULL, NULL, NULL, 0, NULL, NULL, 8, 16, 2, 128, PA_BF16, PA_BF16,
                        1.f, 1.f, NULL, NULL) == PA_ERR_NULL);
  CHECK(kv_cache_append(NULL, 0, NULL, NULL, NULL, 1, NULL, NULL, 8, 16, 2, 128, PA_INT8,
                        PA_FP8_E4M3, 1.f, 1.f, NULL, NULL) == PA_ERR_DTYPE);
  CHECK(strncmp(pagedattn_version(), "libpagedattn", 12) == 0);
  /* the index-checking switch (a debug mode; no call here reaches a check) */
  pagedattn_set_index_check(1);
  CHECK(pagedattn_index_check() == 1);
  CHECK(kv_cache_write(NULL, NULL, NULL, 1, NULL, NULL, 8, 16, 2, 128, PA_BF16, NULL) ==
        PA_ERR_NULL);
  pagedattn_set_index_check(0);
  CHECK(pagedattn_index_check() == 0);
  CHECK(strcmp(pagedattn_status_string(PA_ERR_INDEX), "unknown status") != 0);
  printf("ok\n");
  return 0;
}
