/* A plain C99 client of include/sparcml.h and include/sparcml_bench.h, built and run by test_abi.py with
 * no GPU: it checks that the header compiles as C and that the library links
 * and answers the calls that need no device (status names, the host-side
 * estimate, and argument checks that return before any launch). Prints "ok"
 * and exits 0 on success. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "sparcml.h"
#include "sparcml_bench.h"

static int fails = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      printf("FAIL line %d: %s\n", __LINE__, #c);             \
      ++fails;                                                \
    }                                                         \
  } while (0)

int main(void) {
  CHECK(strcmp(sparcml_status_string(SPARCML_OK), "SPARCML_OK") == 0);
  CHECK(strncmp(sparcml_status_string(SPARCML_ERR_WORKSPACE), "SPARCML_ERR_WORKSPACE", 21) == 0);

  /* two nodes of 100 disjoint-or-not indices out of 1000: 1000 (1 - 0.9^2) = 190 */
  const uint64_t off[3] = {0, 100, 200};
  CHECK(fabs(sparcml_estimate_nnz(2, 1000, off) - 190.0) < 1e-9);

  /* argument errors are reported before anything is launched */
  CHECK(sparcml_topk_ef(0, 1000, 10, NULL, NULL, NULL, NULL, NULL, 0, NULL) == SPARCML_ERR_INVALID_ARG);
  CHECK(sparcml_topk_ef(4, 1000, 1001, NULL, NULL, NULL, NULL, NULL, 0, NULL) == SPARCML_ERR_INVALID_ARG);
  CHECK(sparcml_q4(0, 100, 512, 1, 0, NULL, NULL, NULL, NULL) == SPARCML_ERR_INVALID_ARG);
  CHECK(sparcml_qsgd(3, 1, 100, 512, 1, 0, 0, NULL, NULL, NULL, NULL) == SPARCML_ERR_INVALID_ARG);
  CHECK(sparcml_topk_ef_workspace(0, 1000, 10) == 0);
  CHECK(sparcml_topk_ef_workspace(4, 1000, 10) > 0);
  CHECK(sparcml_sparse_reduce_workspace(4, 1000, 400) > 0);

  /* the measurement variants take the same checks before touching any event */
  sparcml_bench_events ev = {NULL, NULL, NULL, NULL};
  CHECK(sparcml_bench_topk_ef(0, 1000, 10, NULL, NULL, NULL, NULL, NULL, 0, &ev, NULL) == SPARCML_ERR_INVALID_ARG);
  CHECK(sparcml_bench_qsgd(3, 1, 100, 512, 1, 0, 0, NULL, NULL, NULL, &ev, NULL) == SPARCML_ERR_INVALID_ARG);

  if (fails == 0) printf("ok\n");
  return fails == 0 ? 0 : 1;
}
