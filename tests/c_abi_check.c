/* Plain-C client of libsprms: compiled with gcc against include/sprms.h only
 * (no HIP or C++ headers), linked against the built library, and run on the
 * CPU.  It calls the host-only entry points; no kernel is launched. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sprms.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  int64_t S = 0, start = 0, v = 0;
  /* 3500 tokens padded to 3504 over TP=16: 219 rows per rank, 4 padding rows on rank 15 */
  CHECK(sp_shard_geometry(3500, 3504, 16, 15, &S, &start, &v) == SP_OK);
  CHECK(S == 219 && start == 3285 && v == 215);
  CHECK(sp_shard_geometry(3500, 3503, 16, 0, &S, &start, &v) == SP_ERR_SHAPE);
  CHECK(strlen(sp_last_error()) > 0);

  sp_problem p;
  memset(&p, 0, sizeof p);
  p.tp = 8;
  p.tp_rank = 7;
  p.shard_rows = 128;
  p.hidden = 4096;
  p.num_tokens = 1000;
  p.partial_dtype = SP_BF16;
  p.act_dtype = SP_BF16;
  p.out_dtype = SP_FP8_E4M3;
  p.residual_rows = 128;
  p.deepstack_rows = 0;
  p.residual_out = NULL;
  /* fake, aligned, non-overlapping device addresses: validation only */
  const void* partials = (const void*)(uintptr_t)0x10000000000ull;
  void* residual = (void*)(uintptr_t)0x20000000000ull;
  const void* weight = (const void*)(uintptr_t)0x30000000000ull;
  void* out = (void*)(uintptr_t)0x40000000000ull;
  float* scale = (float*)(uintptr_t)0x50000000000ull;
  CHECK(sp_validate(&p, partials, residual, weight, NULL, 1e-6f, SP_QUANT_DYNAMIC_TOKEN, NULL, out,
                    scale) == SP_OK);
  CHECK(sp_validate(&p, partials, residual, weight, NULL, 1e-6f, 3, NULL, out, scale) ==
        SP_ERR_UNSUPPORTED);
  CHECK(sp_validate(&p, partials, residual, weight, NULL, 1e-6f, SP_QUANT_NONE, NULL, out, NULL) ==
        SP_ERR_DTYPE);
  /* the layout calls through their C descriptors: empty problems are no-ops,
   * invalid ones are refused before anything is enqueued */
  sp_gather_problem g = {4, SP_BF16, 0, 4096, 0, 0};
  CHECK(sp_all_gather_unpad(&g, NULL, NULL, NULL, NULL, NULL) == SP_OK);
  sp_fc2_problem f = {4, 2, SP_BF16, -1, 0, 1024};
  CHECK(sp_fc2_regroup(&f, NULL, NULL, NULL) == SP_OK);
  f.otp = 3;
  CHECK(sp_fc2_regroup(&f, NULL, NULL, NULL) == SP_ERR_SHAPE);
  sp_dsacp_problem d = {16, SP_BF16, -1, 0, 0, 1024};
  CHECK(sp_dsacp_heads_to_tokens(&d, NULL, NULL, NULL) == SP_OK);
  d.rank = 16;
  CHECK(sp_dsacp_heads_to_tokens(&d, NULL, NULL, NULL) == SP_ERR_SHAPE);
  CHECK(strcmp(sp_error_string(SP_OK), "success") == 0);
  printf("c abi ok\n");
  return 0;
}
