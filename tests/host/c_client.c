/* A plain C99 client of the library's C ABI: plans a small group on the host
 * (no device call), reads its layout back, checks a refused plan's status and
 * message, and frees the plan.  Built with gcc -std=c99 by
 * tests/test_c_client.py; prints "c client ok" and exits 0 when every check
 * holds. */
#include <stdio.h>
#include <string.h>

#include "muon.h"

static int fails = 0;
#define CHECK(cond, what)                             \
  do {                                                \
    if (!(cond)) {                                    \
      fprintf(stderr, "c client: %s\n", (what));      \
      ++fails;                                        \
    }                                                 \
  } while (0)

int main(void) {
  muon_options o;
  CHECK(muon_default_options(&o) == MUON_OK, "default options");
  CHECK(o.ns_steps == 5 && o.method == MUON_NS_STANDARD, "default values");
  o.method = MUON_NS_GRAM;

  /* two matrices, the second split into 2 heads, over 2 partitions */
  muon_matrix mats[2];
  memset(mats, 0, sizeof(mats));
  mats[0].rows = 17; mats[0].cols = 13; mats[0].flat_offset = 0;
  mats[1].rows = 256; mats[1].cols = 96; mats[1].num_heads = 2; mats[1].flat_offset = 17 * 13;
  muon_layout lay;
  lay.num_partitions = 2;
  lay.partition_numel = (17 * 13 + 256 * 96 + 1) / 2;
  lay.reserved = 0;

  muon_plan *p = NULL;
  CHECK(muon_plan_create(&p, mats, 2, &o, &lay) == MUON_OK && p != NULL, "plan create");
  if (p) {
    size_t ws = 0;
    CHECK(muon_plan_workspace_bytes(p, &ws) == MUON_OK && ws > 0, "workspace bytes");
    int32_t count = 0;
    muon_problem_info probs[4];
    CHECK(muon_plan_problems(p, probs, 4, &count) == MUON_OK && count == 3, "three problems");
    /* the head blocks of matrix 1 are 128 x 96: transposed to 96 x 128 */
    CHECK(count == 3 && probs[1].m == 96 && probs[1].n == 128 && probs[1].transposed == 1, "head orientation");
    muon_run runs[4];
    CHECK(muon_plan_runs(p, 1, runs, 4, &count) == MUON_OK && count >= 1, "runs of matrix 1");
    int64_t total = 0;
    for (int32_t i = 0; i < count && i < 4; ++i) total += runs[i].length;
    CHECK(total == 256 * 96, "runs cover the matrix");
    muon_stats st;
    CHECK(muon_plan_stats(p, &st) == MUON_OK && st.steps == 0 && st.waves >= 1, "stats");
    muon_plan_destroy(p);
  }

  /* a refused group: num_heads does not divide rows */
  mats[1].num_heads = 3;
  muon_plan *q = NULL;
  muon_status s = muon_plan_create(&q, mats, 2, &o, &lay);
  CHECK(s == MUON_ERR_UNSUPPORTED && q == NULL, "refused group");
  CHECK(strcmp(muon_status_string(s), "MUON_ERR_UNSUPPORTED") == 0, "status string");
  CHECK(strlen(muon_last_error()) > 0, "error message");

  if (fails) return 1;
  printf("c client ok\n");
  return 0;
}
