/* A plain C99 caller of the C ABI (host-only queries, no device needed): the header
 * must compile as C, and the library must answer its size and plan queries and
 * reject out-of-contract calls with a message. */
#include <stdio.h>
#include <string.h>

#include "drafter_attn.h"

int main(void) {
  int32_t splits = 0, pages = 0;
  size_t ws = drafter_attn_workspace_bytes(8, 8, 24, 4, 64, 512);
  if (ws == 0 || ws % 256) { printf("bad workspace size %zu\n", ws); return 1; }
  if (drafter_attn_plan(8, 4, 512, &splits, &pages) != DA_OK) { printf("plan failed\n"); return 1; }
  if (splits < 1 || (size_t)splits * (size_t)pages < 512u) { printf("plan does not cover the row\n"); return 1; }
  if (drafter_attn_workspace_bytes(9, 8, 6, 1, 64, 4) != 0) { printf("R = 9 accepted\n"); return 1; }
  /* an attention call that fails validation before any launch (head_dim 128) */
  int rc = drafter_attn((const void*)0x10000, 512, (const void*)0x200000, (const void*)0x202000, 16384, 4,
                        (const int32_t*)0x900000, 1, (const int32_t*)0x900100, NULL, 1, 8, 6, 1, 128, 64,
                        0.125f, (void*)0xA00000, (size_t)1 << 20, (void*)0xB00000, 384, NULL, NULL);
  if (rc != DA_EUNSUPPORTED || strlen(drafter_attn_last_error()) == 0) { printf("rc %d\n", rc); return 1; }
  rc = drafter_qk_norm_rope((void*)0x10000, 512, 0, 6, 1, 64, (const void*)0x900000, DA_POS_INT32,
                            (const void*)0x900100, (const void*)0x900200, 1e-5f, 10000.0f, NULL);
  if (rc != DA_EINVAL) { printf("rc %d\n", rc); return 1; }
  /* YaRN parameters travel as a host struct; a factor below 1 is refused before any launch */
  const da_yarn bad = {.factor = 0.5f, .original_max_position = 4096, .alpha = 1.0f, .beta = 32.0f};
  rc = drafter_qk_norm_rope_yarn((void*)0x10000, 512, 8, 6, 1, 64, (const void*)0x900000, DA_POS_INT32,
                                 (const void*)0x900100, (const void*)0x900200, 1e-5f, 10000.0f, &bad, NULL);
  if (rc != DA_EINVAL || strstr(drafter_attn_last_error(), "yarn") == NULL) { printf("yarn rc %d\n", rc); return 1; }
  /* so is a ramp outside DA_YARN_RAMP_* */
  const da_yarn bad_ramp = {.factor = 4.0f, .original_max_position = 4096, .alpha = 1.0f, .beta = 32.0f,
                           .ramp = DA_YARN_RAMP_INDEX_UNROUNDED + 1};
  rc = drafter_qk_norm_rope_yarn((void*)0x10000, 512, 8, 6, 1, 64, (const void*)0x900000, DA_POS_INT32,
                                 (const void*)0x900100, (const void*)0x900200, 1e-5f, 10000.0f, &bad_ramp, NULL);
  if (rc != DA_EINVAL || strstr(drafter_attn_last_error(), "ramp") == NULL) { printf("ramp rc %d\n", rc); return 1; }
  /* the no-allocation variant refuses a head_dim of 128 before it touches any device */
  rc = drafter_attn_qknorm_noalloc((const void*)0x10000, 512, (const void*)0x200000, (const void*)0x202000, 16384, 4,
                                   (const int32_t*)0x900000, 1, (const int32_t*)0x900100, NULL, 1, 8, 6, 1, 128, 64,
                                   0.125f, (const void*)0x900200, DA_POS_INT32, (const void*)0x900300,
                                   (const void*)0x900400, 1e-5f, 10000.0f, (void*)0xB00000, 384, NULL, NULL);
  if (rc != DA_EUNSUPPORTED) { printf("noalloc rc %d\n", rc); return 1; }
  printf("ok splits=%d pages=%d workspace=%zu flags=%d,%d,%d\n", splits, pages, ws, DA_FLAG_CONTEXT_LEN,
         DA_FLAG_PAGE_ID, DA_FLAG_BLOCK_LEN);
  return 0;
}
