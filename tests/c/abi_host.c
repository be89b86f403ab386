/* Plain-C user of include/moonep.h: validation, workspace sizing, status text and
 * argument checks, all answered on the host before any device work. Exit 0 when
 * every check passes; prints the first failing check otherwise. */
#include <stdio.h>
#include <string.h>

#include "moonep.h"

static int fails = 0;
#define CHECK(cond)                                               \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

int main(void) {
  moonep_shape s = {8, 8192, 384, 8, 48, 7168, 2048, MOONEP_TRAIN, MOONEP_BF16};
  CHECK(moonep_version() >= 100);
  CHECK(moonep_validate_shape(&s) == MOONEP_OK);
  CHECK(moonep_workspace_bytes(&s) > 0 && moonep_workspace_bytes(&s) % 256 == 0);
  CHECK(strlen(moonep_strerror(MOONEP_ELIMIT)) > 0);

  moonep_shape bad = s;
  bad.B = 47; /* training needs B = E/R */
  CHECK(moonep_validate_shape(&bad) == MOONEP_EINVAL);
  CHECK(moonep_workspace_bytes(&bad) == 0);
  bad = s;
  bad.mode = MOONEP_INFER;
  bad.B = 0; /* inference may run without slots */
  CHECK(moonep_validate_shape(&bad) == MOONEP_OK);

  /* argument errors come back before any launch */
  CHECK(moonep_plan(&s, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOONEP_EINVAL);
  CHECK(moonep_grouped_gemm(&s, 7, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
        MOONEP_EINVAL);
  moonep_shape inf = s;
  inf.mode = MOONEP_INFER;
  inf.B = 4;
  void* p = (void*)0x1000;
  CHECK(moonep_grouped_gemm(&inf, MOONEP_DGRAD, p, p, p, p, NULL, NULL, p, (size_t)1 << 30,
                            NULL) == MOONEP_EMODE);
  CHECK(moonep_reduce_grad(&inf, p, p, p, NULL) == MOONEP_EMODE);
  /* the no-alloc GEMM: the same argument checks, and shapes whose tile lists exceed its
   * scratch array refused before any device call */
  CHECK(moonep_grouped_gemm_noalloc(&s, 7, p, p, p, p, NULL, NULL, NULL) == MOONEP_EINVAL);
  CHECK(moonep_grouped_gemm_noalloc(&inf, MOONEP_DGRAD, p, p, p, p, NULL, NULL, NULL) ==
        MOONEP_EMODE);
  moonep_shape big = s;
  big.S = 131072; /* R*ceil(S*K/64) = 131072 list entries: 2 MiB of tiles alone */
  CHECK(moonep_validate_shape(&big) == MOONEP_OK);
  CHECK(moonep_grouped_gemm_noalloc(&big, MOONEP_FWD, p, p, p, p, NULL, NULL, NULL) ==
        MOONEP_ELIMIT);
  CHECK(MOONEP_NOALLOC_SCRATCH_BYTES == (size_t)2 << 20);
  moonep_pool* pool = NULL;
  CHECK(moonep_pool_create(&bad, 1, &pool) == MOONEP_EINVAL && pool == NULL);
  CHECK(moonep_view_destroy(NULL) == MOONEP_EINVAL);
  CHECK(MOONEP_SWIGLU_BLOCK == 32);

  if (fails == 0) printf("abi_host: all checks passed\n");
  return fails ? 1 : 0;
}
