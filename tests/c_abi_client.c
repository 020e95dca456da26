/* A C99 caller of the MLA library: the header compiles as C and the library links and runs from C.
 * Only host-side calls are made (planning, sizes, status strings, and argument errors, which every
 * entry point returns before its first HIP call), so no GPU is needed. Exit status 0 = all checks
 * passed; otherwise the number of the failed check. */
#include <stdio.h>
#include <string.h>

#include "mla.h"

#define CHECK(n, cond)                                 \
  do {                                                 \
    if (!(cond)) {                                     \
      fprintf(stderr, "check %d failed: %s\n", n, #cond); \
      return n;                                        \
    }                                                  \
  } while (0)

int main(void) {
  mla_dims d = {128, 512, 64, 128, 128, 64, 0.07216878f, 10000.0f};
  int32_t st = 0, ns = 0, use_x = -1;
  int32_t lens[2] = {9216, 9216}, q[2] = {1024, 1024};
  float est_a = 0.f, est_x = 0.f;
  uint16_t fake[8];
  mla_cache cache;

  CHECK(1, strcmp(mla_status_string(MLA_OK), mla_status_string(MLA_ERR_NULL)) != 0);
  CHECK(2, mla_decode_plan(&d, 32, 4096, 256, &st, &ns) == MLA_OK && st == 512 && ns == 8);
  CHECK(3, mla_decode_workspace_size(&d, 32) == (size_t)32 * 128 * 576 * 2);
  CHECK(4, mla_chunked_prefill_plan(&d, 2, lens, q, 256, &use_x, &est_a, &est_x) == MLA_OK && use_x == 1 &&
               est_x < est_a);
  /* argument errors come back before any HIP call */
  CHECK(5, mla_decode(NULL, NULL, 1, NULL, NULL, NULL, NULL, 512, 1, NULL, 0, NULL, NULL, NULL) == MLA_ERR_NULL);
  memset(&cache, 0, sizeof(cache));
  cache.data = fake;
  cache.num_blocks = 1;
  cache.max_blocks_per_seq = 1;
  CHECK(6, mla_decode(&d, &cache, 1, (const int32_t*)fake, fake, fake, fake, 100, 1, fake, 1 << 20, fake,
                      (float*)fake, NULL) == MLA_ERR_BAD_ARG); /* split_tokens not a block multiple */
  d.n_heads = 120;
  CHECK(7, mla_decode_plan(&d, 32, 4096, 256, &st, &ns) == MLA_ERR_UNSUPPORTED);
  printf("c abi client: 7 checks passed\n");
  return 0;
}
