/* A plain C99 caller of the library's boundary: it includes the header, links
 * libpagedkv.so and calls entry points that run on the host only (no GPU is touched).
 * Prints one line per check and exits non-zero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pagedkv.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  pkv_pool_desc pool;
  pkv_pool_desc bad;
  int32_t tables[2 * 4];
  int32_t lens[2];
  int64_t slots[3];
  uint32_t sink_word = 0;
  int i;

  check(pkv_abi_version() == PKV_ABI_VERSION, "ABI version matches the header");
  check(strcmp(pkv_status_str(PKV_OK), "OK") == 0, "status string of OK");
  check(strcmp(pkv_status_str(PKV_ERR_WORKSPACE), "WORKSPACE") == 0,
        "status string of WORKSPACE");

  /* 64 blocks of 16 slots, 4 KV heads of 128, bfloat16, HND */
  pool.num_blocks = 64;
  pool.block_size = 16;
  pool.num_kv_heads = 4;
  pool.head_dim = 128;
  pool.dtype = PKV_BF16;
  pool.layout = PKV_LAYOUT_HND;
  check(pkv_check_pool(&pool) == PKV_OK, "a valid descriptor");
  check(pkv_sink_slot(&pool) == 64 * 16, "sink slot = num_blocks * block_size");
  check(pkv_pool_elements(&pool) == (int64_t)65 * 16 * 4 * 128,
        "pool elements = (num_blocks + 1) * block_size * kv_heads * head_dim");
  check(pkv_workspace_bytes(&pool, 2, 8, 4) > 0, "a workspace size for 2 rows");

  bad = pool;
  bad.head_dim = 96;
  check(pkv_check_pool(&bad) == PKV_ERR_UNSUPPORTED, "head_dim 96 is unsupported");
  check(pkv_sink_slot(&bad) == -1, "no sink slot for an unsupported descriptor");

  /* host refusal checks: a slot past the sink, a block id past the pool */
  slots[0] = 0;
  slots[1] = 64 * 16;          /* the sink: legal */
  slots[2] = 64 * 16 + 1;      /* past it */
  check(pkv_check_write_host(&pool, slots, 2) == PKV_OK, "slots up to the sink pass");
  check(pkv_check_write_host(&pool, slots, 3) == PKV_ERR_SLOT, "a slot past the sink");
  check(strlen(pkv_last_error_detail()) > 0, "the refusal has a detail string");

  for (i = 0; i < 8; ++i) tables[i] = -1;
  tables[0] = 3;
  tables[1] = 7;
  tables[4] = 64;              /* row 1's first block: outside [0, 64) */
  lens[0] = 17;                /* two blocks */
  lens[1] = 0;                 /* an empty row reads nothing: its table is not checked */
  check(pkv_check_attention_host(&pool, tables, 4, lens, 2, 8) == PKV_OK,
        "live prefixes in range pass");
  lens[1] = 1;
  check(pkv_check_attention_host(&pool, tables, 4, lens, 2, 8) == PKV_ERR_BLOCK_ID,
        "a live block id past the pool");
  check(pkv_check_attention_host(&pool, tables, 4, lens, 2, 6) == PKV_ERR_SHAPE,
        "6 query heads over 4 KV heads");

  /* the benchmark reads refuse bad shapes before touching the device */
  check(pkv_gather_read(&sink_word, &sink_word, (const int64_t*)slots, 1, 4096, &sink_word,
                        1, 3, 2, NULL) == PKV_ERR_SHAPE,
        "a gather read of 3 waves per workgroup");
  check(pkv_stream_read(&sink_word, 24, &sink_word, 1, NULL) == PKV_ERR_SHAPE,
        "a streaming read of 24 bytes");

  printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
