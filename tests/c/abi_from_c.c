/* A C99 program against include/attn.h and libattn.so: the boundary is plain C.  It calls
 * only entry points that need no GPU (validation, planning, error text, split ranges,
 * workspace sizes, a call with no query rows), prints what it checked and returns 0 when
 * every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  /* fake, far-apart device addresses: validation only compares them */
  const void* q = (const void*)(uintptr_t)(1ull << 40);
  const void* k = (const void*)(uintptr_t)(2ull << 40);
  const void* v = (const void*)(uintptr_t)(3ull << 40);
  void* o = (void*)(uintptr_t)(4ull << 40);
  float* lse = (float*)(uintptr_t)(5ull << 40);

  CHECK(attn_validate(q, k, v, o, lse, 1, 32, 2, 16384, 16384, 256, 0.0625f, ATTN_F16) ==
        ATTN_OK);
  CHECK(attn_validate(q, k, v, o, lse, 1, 32, 2, 16384, 16384, 64, 0.0625f, ATTN_F16) ==
        ATTN_E_HEADDIM);
  CHECK(attn_validate(q, k, v, o, lse, 1, 32, 3, 64, 64, 128, 0.1f, ATTN_BF16) == ATTN_E_GQA);
  CHECK(attn_validate(q, k, v, q, lse, 1, 32, 2, 64, 64, 128, 0.1f, ATTN_BF16) == ATTN_E_ALIAS);
  CHECK(attn_validate_ex(q, k, v, o, lse, 1, 32, 2, 64, 64, 128, 0.1f, ATTN_F16, 4u, 1) ==
        ATTN_E_FLAGS);
  CHECK(strlen(attn_strerror(ATTN_E_SHAPE)) > 0 && strlen(attn_strerror(12345)) > 0);
  CHECK(strlen(attn_version()) >= 5);

  attn_plan_t plan;
  CHECK(attn_plan_ex(1, 32, 2, 16, 16384, 256, ATTN_F16, ATTN_CAUSAL, &plan) == ATTN_OK);
  CHECK(plan.nsplit > 1 && plan.block_n == 32 && plan.grid > 0 && plan.kernel[0] != '\0');
  CHECK(plan.workspace_bytes == attn_workspace_bytes(1, 32, 16, 256, plan.nsplit));

  int64_t b = -1, e = -1, covered = 0;
  for (int64_t s = 0; s < 7; ++s) {
    CHECK(attn_split_range(1000, 7, s, &b, &e) == ATTN_OK);
    CHECK(b == covered || (b == e && e == 1000));
    covered = e;
  }
  CHECK(covered == 1000);

  /* no query rows: valid, nothing launched, NULL tensors allowed */
  CHECK(attn_fwd(NULL, NULL, NULL, NULL, NULL, 0, 32, 2, 128, 0, 256, 0.0625f, ATTN_F16) ==
        ATTN_OK);
  CHECK(attn_merge(NULL, NULL, 3, 0, 256, NULL, NULL, ATTN_F32, NULL) == ATTN_OK);

  printf("abi_from_c: %s (%d failed)\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
