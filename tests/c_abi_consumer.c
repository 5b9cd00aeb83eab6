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
  check(moe_route(NULL, 4, 2048, 2, NULL, NULL, NULL, NULL) == MOE_ERR_UNSUPPORTED,
        "E above the kernel limit rejected");
  check(moe_permute_noalloc(NULL, 2, 2048, 2, NULL, 8, MOE_BF16, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL) == MOE_ERR_UNSUPPORTED,
        "moe_permute_noalloc: E above the limit rejected");
  check(moe_grouped_swiglu_combine(NULL, NULL, NULL, 4, 2, NULL, 8, 64, 32, MOE_F32, NULL, NULL,
                                   0, NULL, NULL, NULL) == MOE_ERR_UNSUPPORTED,
        "moe_grouped_swiglu_combine: f32 rejected");
  check(moe_combine(NULL, NULL, NULL, 4, 65, 8, NULL, NULL) == MOE_ERR_UNSUPPORTED,
        "moe_combine: k above the limit rejected");

  /* the merge's id checks read the host id array: unsorted, out of range, too many ids */
  {
    moe_pool pool;
    moe_wbuf buf;
    int32_t slots[8];
    static char fake_base[1];
    const int32_t unsorted[2] = {3, 1};
    const int32_t out_of_range[2] = {0, 8};
    const int32_t too_many[5] = {0, 1, 2, 3, 4};
    pool.base = fake_base;
    pool.expert_bytes = 96;
    pool.first_expert = 0;
    pool.n_experts = 4;
    buf.base = fake_base;
    buf.expert_bytes = 96;
    buf.n_slots = 4;
    buf.n_experts = 8;
    buf.slot_of = slots;
    check(moe_merge_weights(&pool, unsorted, 2, &buf, NULL, NULL, NULL, MOE_COPY_SDMA) ==
              MOE_ERR_ARG, "merge: unsorted ids rejected");
    check(moe_merge_weights(&pool, out_of_range, 2, &buf, NULL, NULL, NULL, MOE_COPY_SDMA) ==
              MOE_ERR_ARG, "merge: id out of range rejected");
    check(moe_prefetch_layer(&pool, too_many, 5, &buf, NULL, NULL, NULL, MOE_COPY_SDMA) ==
              MOE_ERR_ARG, "prefetch: more ids than slots rejected");
    check(moe_prefetch_layer(&pool, unsorted, 2, &buf, NULL, NULL, NULL, 3) == MOE_ERR_ARG,
          "prefetch: unknown copy mode rejected");
    check(strstr(moe_last_error(), "moe_prefetch_layer") != NULL, "error text names the call");
    /* the routed pull on the device: its argument checks run before any HIP call */
    {
      int32_t counts[8] = {0};
      moe_pool remote = pool;
      remote.first_expert = 4;
      check(moe_prefetch_routed(&remote, NULL, &buf, NULL, NULL, NULL, NULL, 0) == MOE_ERR_ARG,
            "routed prefetch: null counts rejected");
      check(moe_prefetch_routed(&remote, counts, &buf, NULL, NULL, NULL, NULL, -1) ==
                MOE_ERR_ARG, "routed prefetch: negative workgroup bound rejected");
      /* experts 4..7 need slots up to 7; the buffer has 4 */
      check(moe_prefetch_routed(&remote, counts, &buf, NULL, NULL, NULL, NULL, 0) ==
                MOE_ERR_ARG, "routed prefetch: slot = expert id past the slots rejected");
      check(strstr(moe_last_error(), "moe_prefetch_routed") != NULL,
            "routed prefetch: error text names the call");
      remote.expert_bytes = 48;
      check(moe_prefetch_routed(&remote, counts, &buf, NULL, NULL, NULL, NULL, 0) ==
                MOE_ERR_ARG, "routed prefetch: pool block size differing from the buffer's rejected");
    }
  }
  {
    moe_phys_t ph = NULL;
    size_t zero = 0;
    void* va = NULL;
    check(moe_vmm_create(0, 0, &ph) == MOE_ERR_ARG, "vmm: empty block rejected");
    check(moe_vmm_map(0, NULL, &zero, 1, &va) == MOE_ERR_ARG, "vmm: map without blocks rejected");
  }

  if (failures == 0) printf("ok %s\n", v);
  return failures == 0 ? 0 : 1;
}
