/* The library's boundary used from plain C (C11): include/moe.h compiled as
 * C, libmoe.so linked and called without any Python or torch.  Only calls
 * that make no HIP call run here (status strings, table sizes, the
 * byte-budget planner, the popularity ranking of moe_build_tiers with host
 * outputs, argument validation), so no GPU is needed.  Prints "ok" and
 * exits 0, or names the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "moe.h"

#define CHECK(cond)                                                 \
  do {                                                              \
    if (!(cond)) {                                                  \
      printf("failed: %s (line %d)\n", #cond, __LINE__);            \
      return 1;                                                     \
    }                                                               \
  } while (0)

int main(void) {
  const moe_dims full = {2048, 512, 512, 10, 1, MOE_BF16};
  const int32_t bits[3] = {4, 3, 2};
  const int32_t slots[3] = {128, 256, 128};

  CHECK(strcmp(moe_status_string(MOE_OK), "MOE_OK") == 0);
  CHECK(strncmp(moe_status_string(MOE_EINVAL), "MOE_", 4) == 0);

  /* all tier tables of the full-size layer: 768 MiB (codes + scales) */
  size_t total = 0;
  for (int t = 0; t < 3; t++)
    for (int m = 0; m < 3; m++)
      total += moe_tier_table_bytes(&full, bits[t], slots[t], m, MOE_CODES) +
               moe_tier_table_bytes(&full, bits[t], slots[t], m, MOE_DM);
  CHECK(total == (size_t)768 << 20);

  /* popularity: expert e used (e * 7919) % 1000 + 1 times */
  uint64_t pop[512];
  for (int e = 0; e < 512; e++) pop[e] = (uint64_t)((e * 7919) % 1000 + 1);

  /* the planner: every expert gets a tier, and a budget of every expert at
     4 bits keeps them all in tier 0 */
  int32_t plan[3] = {0, 0, 0};
  CHECK(moe_plan_tiers(&full, pop, bits, (uint64_t)512 * 1966080u, plan) == MOE_OK);
  CHECK(plan[0] == 512 && plan[1] == 0 && plan[2] == 0);
  CHECK(moe_plan_tiers(&full, pop, bits, (uint64_t)768 << 20, plan) == MOE_OK);
  CHECK(plan[0] + plan[1] + plan[2] == 512);

  /* the ranking alone (no weights, no tables): hottest first, ties to the
     lower id; the map is a bijection onto the slots */
  int32_t tmap[512], order[512];
  CHECK(moe_build_tiers(&full, pop, slots, bits, NULL, tmap, order, NULL, 0, NULL) == MOE_OK);
  int seen[512];
  memset(seen, 0, sizeof seen);
  for (int r = 0; r < 512; r++) {
    const int e = order[r];
    CHECK(e >= 0 && e < 512 && !seen[e]);
    seen[e] = 1;
    if (r > 0) {
      const int prev = order[r - 1];
      CHECK(pop[prev] > pop[e] || (pop[prev] == pop[e] && prev < e));
    }
    const int tier = r < 128 ? 0 : (r < 384 ? 1 : 2);
    const int slot = r - (tier == 0 ? 0 : (tier == 1 ? 128 : 384));
    CHECK(tmap[e] == (tier << 16 | slot));
  }

  /* argument validation happens before any HIP call */
  CHECK(moe_forward_decode(NULL, NULL, NULL, 1, NULL, MOE_F32, NULL, NULL, NULL, NULL, NULL) ==
        MOE_EINVAL);
  const moe_dims bad = {2048, 512, 512, 600, 1, MOE_BF16};   /* top_k > n_experts */
  size_t ws = 0;
  CHECK(moe_forward_prefill(&bad, NULL, NULL, 1, NULL, MOE_F32, NULL, NULL, NULL, NULL, NULL, &ws,
                            NULL) == MOE_EINVAL);

  printf("ok\n");
  return 0;
}
