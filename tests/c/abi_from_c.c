/* Plain C use of include/tmoe.h: host-only calls (plan, sizes, validation) and the fail-closed
 * checks of the forward entry points with fake device pointers, which are never dereferenced.
 * Prints one line per check and exits non-zero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tmoe.h"

static int fails = 0;
#define CHECK(cond, what)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      printf("FAIL %s\n", what);                            \
      fails++;                                              \
    } else {                                                \
      printf("ok %s\n", what);                              \
    }                                                       \
  } while (0)

int main(void) {
  uint8_t bits[96];
  memset(bits, 4, sizeof bits);
  tmoe_config cfg = {1024, 512, 96, 8, 16, bits, TMOE_ROT_HADAMARD, TMOE_IDS_I64, 0};
  tmoe_plan_t plan = NULL;
  size_t scratch = 0, words = 0;
  CHECK(tmoe_plan(&cfg, &plan, &scratch, &words) == TMOE_OK, "plan decode geometry");
  CHECK(words == (size_t)96 * 3 * 1024 * 512 * 4 / 16, "payload words = E * 3HI * bits / 16");
  CHECK(scratch > 0 && scratch % 256 == 0, "scratch size planned");
  tmoe_plan_info info;
  CHECK(tmoe_plan_get_info(plan, &info) == TMOE_OK && info.scratch_bytes == scratch, "plan info");
  size_t off = 0;
  CHECK(tmoe_plan_expert_offset(plan, 3, &off) == TMOE_OK && off == (size_t)3 * 3 * 1024 * 512 * 4 / 16,
        "expert offset");

  /* fail closed: every argument error returns before any launch */
  void *fake = (void *)(uintptr_t)(1u << 20);
  tmoe_weights w = {fake, fake, fake, fake, fake, fake, fake};
  CHECK(tmoe_forward_w4a16(plan, fake, fake, fake, 17, &w, fake, fake, scratch, NULL) == TMOE_ERR_CAPACITY,
        "T above capacity");
  CHECK(tmoe_forward_w4a16(plan, fake, fake, fake, 4, &w, fake, fake, scratch - 1, NULL) == TMOE_ERR_SCRATCH,
        "short arena");
  CHECK(tmoe_forward_w4a16(plan, fake, fake, fake, 4, &w, fake, (char *)fake + 8, scratch, NULL) ==
            TMOE_ERR_SCRATCH,
        "misaligned arena");
  CHECK(tmoe_forward_w4a16(plan, fake, fake, fake, 0, &w, fake, fake, scratch, NULL) == TMOE_OK,
        "T = 0 launches nothing");
  CHECK(strlen(tmoe_status_str(TMOE_ERR_UNSUPPORTED)) > 0, "status strings");
  CHECK(tmoe_plan_destroy(plan) == TMOE_OK, "destroy");

  cfg.hidden = 1000;
  CHECK(tmoe_plan(&cfg, &plan, NULL, NULL) == TMOE_ERR_UNSUPPORTED, "unsupported hidden size");

  tmoe_linear_config lc = {2560, 320, 3, 64, TMOE_ROT_HADAMARD};
  tmoe_linear_plan_t lp = NULL;
  CHECK(tmoe_linear_plan(&lc, &lp, &scratch, &words) == TMOE_OK, "linear plan");
  CHECK(words == (size_t)(2560 / 16) * (320 / 16) * 16 * 3, "linear payload words");
  tmoe_linear_weights lw = {fake, fake, fake, fake};
  CHECK(tmoe_linear_w4a16(lp, fake, 65, &lw, fake, fake, scratch, NULL) == TMOE_ERR_CAPACITY, "linear capacity");
  CHECK(tmoe_linear_plan_destroy(lp) == TMOE_OK, "linear destroy");
  printf("%s\n", fails ? "FAILED" : "PASSED");
  return fails ? 1 : 0;
}
