/* A plain C caller of the library's C ABI (include/bi_logprob.h), built by
 * tests/test_abi.py with gcc as C99.  It calls only entry points that do their
 * work on the host: the launch geometry, the lm_head tile counts, and argument
 * validation, which rejects a call before any device memory is touched.
 * Exit status 0 when every check holds; the first failed check's number
 * otherwise. */
#include <stdio.h>
#include <string.h>

#include "bi_logprob.h"

int main(void) {
  int threads = 0, vec = 0, group = 0;
  if (bi_row_geometry(BI_BF16, 151936, &threads, &vec, &group) != BI_OK) return 1;
  if (threads != 1024 || vec != 8) return 2;
  printf("bf16 rows of 151936: %d threads, %d elements per load, %d loads per group\n", threads,
         vec, group);
  if (bi_lmhead_tile_rows() != 256) return 3;
  if (bi_lmhead_tiles(151936) != 594 || bi_lmhead_tiles(0) != 0) return 4;

  /* negative row count: rejected on the host, with a message for this thread */
  int rc = bi_logprob_fwd(NULL, BI_BF16, -1, 10, 10, NULL, -100, NULL, NULL, NULL, NULL, NULL);
  if (rc != BI_ERR_SHAPE) return 5;
  if (strlen(bi_last_error()) == 0 || strlen(bi_status_string(rc)) == 0) return 6;
  printf("bi_logprob_fwd(n_rows = -1): %s (%s)\n", bi_status_string(rc), bi_last_error());

  /* an unknown dtype */
  rc = bi_logprob_fwd(NULL, 7, 1, 10, 10, NULL, -100, NULL, NULL, NULL, NULL, NULL);
  if (rc != BI_ERR_DTYPE) return 7;

  /* zero rows is a valid empty call: nothing to read or write */
  rc = bi_logprob_fwd(NULL, BI_F32, 0, 10, 10, NULL, -100, NULL, NULL, NULL, NULL, NULL);
  if (rc != BI_OK) return 8;
  return 0;
}
