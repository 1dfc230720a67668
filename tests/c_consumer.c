/* A plain C99 caller of libbsga: includes the header, links the library and
 * exercises the host-only entry points (no GPU work).  Prints "ok" and
 * returns 0 when every check holds. */
#include <math.h>
#include <stdio.h>

#include "bsga.h"

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      printf("check failed, line %d: %s\n", __LINE__, #c);    \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  /* 32 frames of 37 x 37 patches, 5 special tokens, 16 heads, b = 128 */
  bsga_shape s = {32, 1369, 5, 16, 64, 128};
  int32_t B = 0, k = 0;
  int64_t cap = 0;
  size_t ws = 0;
  double w[4] = {1.0, 2.0, 3.0, 4.0}, rho[4];
  double mean_keep = 0.0;
  int h;

  CHECK(bsga_version() == BSGA_VERSION);
  CHECK(bsga_status_string(BSGA_ERR_WORKSPACE) != NULL);
  CHECK(bsga_num_blocks(&s, &B) == BSGA_OK && B == 343); /* ceil(43808 / 128) */
  CHECK(bsga_keep_count(2140, 0.9, &k) == BSGA_OK && k == 214);
  CHECK(bsga_keep_count(B, 1.5, &k) == BSGA_ERR_INVALID_ARG);
  CHECK(bsga_csr_capacity(&s, &cap) == BSGA_OK && cap == (int64_t)16 * 343 * 343);
  CHECK(bsga_workspace_bytes(&s, BSGA_OP_LAYER, &ws) == BSGA_OK && ws > 0 && ws % 256 == 0);
  s.head_dim = 128;
  CHECK(bsga_num_blocks(&s, &B) == BSGA_ERR_UNSUPPORTED);
  s.head_dim = 64;
  /* validation happens before any launch: null tensors are rejected */
  CHECK(bsga_predict_mask(&s, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
        BSGA_ERR_INVALID_ARG);
  /* budgets: keep fractions proportional to the weights, mean 1 - 0.75 */
  CHECK(bsga_redistribute(4, w, 0.75, 0.0, 1.0, rho) == BSGA_OK);
  for (h = 0; h < 4; ++h) mean_keep += (1.0 - rho[h]) / 4.0;
  CHECK(fabs(mean_keep - 0.25) < 1e-12);
  CHECK(fabs((1.0 - rho[3]) / (1.0 - rho[0]) - 4.0) < 1e-9);
  printf("ok\n");
  return 0;
}
