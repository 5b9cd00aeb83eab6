/* A plain C99 caller of the library: include/moe.h must compile as C with
 * every warning an error, and the host-only entry points must answer without
 * a GPU.  Exit status 0 when every check holds; each failed check prints one
 * line. */
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

static void check(int ok, const char* what) {
  if (!ok) {
    printf("FAIL: %s\n", what);
    ++failures;
  }
}

int main(void) {
  size_t bytes = 0;
  const char* v = moe_version();
  check(v != NULL && strncmp(v, "moe-gfx950", 10) == 0, "moe_version");

  check(moe_permute_workspace_size(64, 256, 8, &bytes) == MOE_OK && bytes > 0,
        "moe_permute_workspace_size, R1 decode");
  check(moe_grouped_swiglu_workspace_size(512, 256, 7168, 2048, MOE_BF16, &bytes) == MOE_OK &&
            bytes > 0,
        "moe_grouped_swiglu_workspace_size, R1 decode");

  /* argument errors come back as codes with a message, before any device work */
  check(moe_permute_workspace_size(64, 0, 8, &bytes) == MOE_ERR_ARG, "E = 0 rejected");
  check(strlen(moe_last_error()) > 0, "moe_last_error after a rejected call");
  check(moe_grouped_swiglu_workspace_size(512, 256, 7168, 2048, (moe_dtype)7, &bytes) ==
            MOE_ERR_ARG,
        "unknown dtype rejected");
  check(moe_route(NULL, 4, 8, 9, NULL, NULL, NULL, NULL) == MOE_ERR_ARG, "k > E rejected");

  if (failures == 0) printf("ok %s\n", v);
  return failures == 0 ? 0 : 1;
}
