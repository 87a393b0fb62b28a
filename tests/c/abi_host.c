/* Host-only use of libpkv from plain C11: the header compiles as C, and the
 * table verbs (fork, append planning with copy-on-write, truncation, prompt
 * cache, free) behave as documented. Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>

#include "pkv.h"

#define CHECK(x)                                                            \
  do {                                                                      \
    if (!(x)) {                                                             \
      fprintf(stderr, "%s:%d: %s (%s)\n", __FILE__, __LINE__, #x,          \
              pkv_last_error());                                            \
      return 1;                                                             \
    }                                                                       \
  } while (0)

int main(void) {
  pkv_pool_desc d = {0};
  d.num_blocks = 64;
  d.block_size = 4;
  d.num_layers = 1;
  d.num_kv_heads = 1;
  d.num_q_heads = 2;
  d.head_dim = 64;
  d.kv_dtype = PKV_F32;
  pkv_pool* p = NULL;
  CHECK(pkv_pool_create(&d, &p) == PKV_OK);

  pkv_seq a, b;
  int64_t slots[32];
  pkv_cow_op op;
  int32_t n_cow = -1, len = 0, nb = 0, rc = 0;
  CHECK(pkv_seq_create(p, &a) == PKV_OK);
  CHECK(pkv_seq_append_plan(p, a, 6, slots, &op, &n_cow) == PKV_OK);  /* blocks 0, 1 */
  CHECK(n_cow == 0 && slots[0] == 0 && slots[5] == 4 * 1 + 1);
  CHECK(pkv_seq_fork(p, a, &b) == PKV_OK);
  CHECK(pkv_block_refcount(p, 1, &rc) == PKV_OK && rc == 2);
  /* b writes into the shared, partly filled block 1: it copies it first */
  CHECK(pkv_seq_append_plan(p, b, 1, slots, &op, &n_cow) == PKV_OK);
  CHECK(n_cow == 1 && op.src == 1 && op.dst == 2 && op.n_valid == 2 && slots[0] == 2 * 4 + 2);
  CHECK(pkv_block_refcount(p, 1, &rc) == PKV_OK && rc == 1);
  int32_t t[8];
  CHECK(pkv_seq_blocks(p, b, t, 8) == PKV_OK && t[0] == 0 && t[1] == 2);
  CHECK(pkv_seq_info(p, b, &len, &nb) == PKV_OK && len == 7 && nb == 2);

  /* truncation and the prompt cache */
  CHECK(pkv_seq_truncate(p, b, 4) == PKV_OK);
  CHECK(pkv_seq_info(p, b, &len, &nb) == PKV_OK && len == 4 && nb == 1);
  int32_t toks[6] = {7, 8, 9, 10, 11, 12}, added = -1, matched = -1, entries = -1, evict = -1;
  CHECK(pkv_prefix_insert(p, a, toks, 6, &added) == PKV_OK && added == 1);
  pkv_seq m;
  CHECK(pkv_prefix_match(p, toks, 6, &m, &matched) == PKV_OK && matched == 4);
  CHECK(pkv_seq_blocks(p, m, t, 8) == PKV_OK && t[0] == 0);
  CHECK(pkv_block_refcount(p, 0, &rc) == PKV_OK && rc == 4);  /* a, b, m, the entry */
  CHECK(pkv_prefix_info(p, &entries, &evict) == PKV_OK && entries == 1 && evict == 0);

  /* errors: stale handle, bad length */
  CHECK(pkv_seq_free(p, b) == PKV_OK);
  CHECK(pkv_seq_free(p, b) == PKV_E_INVALID);
  CHECK(pkv_seq_truncate(p, a, 99) == PKV_E_INVALID);

  pkv_stats st;
  CHECK(pkv_seq_free(p, a) == PKV_OK && pkv_seq_free(p, m) == PKV_OK);
  CHECK(pkv_pool_stats(p, &st) == PKV_OK && st.total_refs == 1 && st.free_blocks == 63);
  CHECK(pkv_prefix_clear(p) == PKV_OK);
  CHECK(pkv_pool_stats(p, &st) == PKV_OK && st.total_refs == 0 && st.free_blocks == 64);
  CHECK(pkv_pool_destroy(p) == PKV_OK);
  printf("ok\n");
  return 0;
}
