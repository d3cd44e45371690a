/* Plain C99 client of the library's C ABI: compiles against include/cpattn.h
 * alone and calls the host-only entry points (no device is touched).  Built
 * and run by tests/test_c_abi.py; exits non-zero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cpattn.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  /* one 256-token sequence, cp = 4: chunks of 32, rank 0 keeps chunks 0 and 7 */
  const int32_t cu[2] = {0, 256};
  int32_t cu_l[2] = {-1, -1};
  int64_t l2g[64];
  int i, r, s;
  CHECK(strlen(cpattn_version()) > 0);
  CHECK(strcmp(cpattn_status_string(CPATTN_OK), "ok") == 0);
  CHECK(cpattn_partition_index(cu, 1, 4, 0, cu_l, l2g) == CPATTN_OK);
  CHECK(cu_l[0] == 0 && cu_l[1] == 64);
  for (i = 0; i < 32; ++i) CHECK(l2g[i] == i && l2g[32 + i] == 224 + i);
  /* rejected arguments come back as status codes */
  CHECK(cpattn_partition_index(cu, 1, 4, 4, cu_l, l2g) == CPATTN_ERR_INVALID_ARG);
  CHECK(cpattn_partition_index(NULL, 1, 4, 0, cu_l, l2g) == CPATTN_ERR_INVALID_ARG);
  /* causal pairs per ring step: 2C^2 + C at step 0, 2C^2 after (C = 32), on every rank */
  for (r = 0; r < 4; ++r)
    for (s = 0; s < 4; ++s) {
      cpattn_step st;
      st.cp = 4;
      st.rank = r;
      st.step = s;
      st.tf_chunk_tokens = 0;
      st.tf_num_chunks = 0;
      CHECK(cpattn_count_pairs(cu, 1, CPATTN_MASK_CAUSAL, &st) == (s == 0 ? 2 * 32 * 32 + 32 : 2 * 32 * 32));
    }
  /* ring source rule: (rank - step) mod cp, -1 for an invalid step */
  for (r = 0; r < 4; ++r)
    for (s = 0; s < 4; ++s) {
      cpattn_step st;
      st.cp = 4;
      st.rank = r;
      st.step = s;
      st.tf_chunk_tokens = 0;
      st.tf_num_chunks = 0;
      CHECK(cpattn_step_source(&st) == (r - s + 4) % 4);
    }
  CHECK(cpattn_step_source(NULL) == -1);
  {
    int32_t sh = 0, sw = 0;
    CHECK(cpattn_split_hw(30, 52, 8, &sh, &sw) == CPATTN_OK);
    CHECK(sh * sw == 8 && 30 % sh == 0 && 52 % sw == 0);
  }
  CHECK(cpattn_workspace_size(64, 64, 1) > 0);
  CHECK(cpattn_fill_f32(NULL, 0, 0.0f, NULL) == CPATTN_OK);
  CHECK(cpattn_fill_f32(NULL, 4, 0.0f, NULL) == CPATTN_ERR_INVALID_ARG);
  printf("c abi ok\n");
  return 0;
}
