/* A plain C99 consumer of include/pagedkv.h: the boundary compiles as C and its host-side
 * calls work without a GPU.  Exit status 0 when every check holds; each failure names its
 * check on stderr. */
#include <stdio.h>
#include <string.h>

#include "pagedkv.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  const char* v = pkv_version();
  CHECK(v != NULL && strncmp(v, "pagedkv", 7) == 0);

  /* optiverse "Block table and non-contiguous allocation": 825 tokens in 16-token blocks
   * take 52 blocks (832 slots, 7 unused) */
  pkv_bm* bm = pkv_bm_create(64, 16, NULL, 0);
  CHECK(bm != NULL);
  pkv_bm_stats_t st;
  CHECK(pkv_bm_add_seq(bm, 0, 825) == PKV_OK);
  CHECK(pkv_bm_stats(bm, &st) == PKV_OK);
  CHECK(st.used_blocks == 52 && st.free_blocks == 12 && st.tokens == 825);
  CHECK(st.slots_allocated == 832);

  /* fork shares the blocks; an append to the fork's partly filled shared last block copies
   * it first (ithome section 4, copy-on-write) */
  CHECK(pkv_bm_add_seq(bm, 1, 20) == PKV_OK);          /* blocks 52, 53: 16 + 4 tokens */
  CHECK(pkv_bm_fork(bm, 1, 2) == PKV_OK);
  CHECK(pkv_bm_refcount(bm, 53) == 2);
  int64_t slot = -1, src = -1, dst = -1;
  CHECK(pkv_bm_append(bm, 2, &slot, &src, &dst) == PKV_OK);
  CHECK(src == 53 && dst == 54 && slot == 54 * 16 + 4);
  CHECK(pkv_bm_refcount(bm, 53) == 1 && pkv_bm_refcount(bm, 54) == 1);
  CHECK(pkv_bm_refcount(bm, 52) == 2);                 /* the full block stays shared */

  int64_t seqs[2] = {1, 2};
  int32_t tables[2][4], lens[2];
  CHECK(pkv_bm_block_tables(bm, seqs, 2, &tables[0][0], 4, lens) == PKV_OK);
  CHECK(lens[0] == 20 && lens[1] == 21);
  CHECK(tables[0][0] == 52 && tables[0][1] == 53 && tables[0][2] == -1);
  CHECK(tables[1][0] == 52 && tables[1][1] == 54 && tables[1][2] == -1);

  /* not enough free blocks: refused, nothing changes */
  pkv_bm_stats_t before, after;
  CHECK(pkv_bm_stats(bm, &before) == PKV_OK);
  CHECK(pkv_bm_add_seq(bm, 3, 16 * 64) == PKV_E_NOMEM);
  CHECK(pkv_bm_stats(bm, &after) == PKV_OK);
  CHECK(memcmp(&before, &after, sizeof before) == 0);
  CHECK(strlen(pkv_last_error()) > 0);
  pkv_bm_destroy(bm);

  /* shared-prefix units: two sequences with the same two leading blocks form one unit */
  int32_t t2[2][3] = {{5, 6, 1}, {5, 6, 2}};
  int32_t l2[2] = {40, 41};
  int32_t rows[2][4], seq_rows[2][4];
  CHECK(pkv_prefix_rows(&t2[0][0], l2, 2, 3, 16, 4, 1, &rows[0][0], &seq_rows[0][0]) == 1);
  CHECK(rows[0][0] == 0 && rows[0][1] == 32 && rows[0][2] == 2 && rows[0][3] == 0);
  CHECK(seq_rows[1][0] == 0 && seq_rows[1][1] == 1);

  /* sizes and argument checks that need no device */
  CHECK(pkv_decode_workspace_bytes(4, 8, 128, 1000, 0) > 0);
  CHECK(pkv_paged_attn_decode(NULL, PKV_BF16, NULL, NULL, NULL, NULL, 1, NULL, 1, 8, 0.1f,
                              NULL, 16, 0, NULL, 0, NULL) == PKV_E_INVAL);
  CHECK(strlen(pkv_last_error()) > 0);

  if (failures == 0) printf("abi smoke ok\n");
  return failures == 0 ? 0 : 1;
}
