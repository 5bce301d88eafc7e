/* A plain C99 consumer of the library's C ABI (include/hq.h): plan creation,
 * description, sizes, tuning read-back and rejection paths, with no device
 * work, so that the header is checked as C (not C++) and the library as a
 * C-linkable shared object.  Exit status 0 and "ok" on success. */
#include <stdio.h>
#include <string.h>

#include "hq.h"

#define CHECK(c)                                                                            \
  do {                                                                                      \
    if (!(c)) {                                                                             \
      fprintf(stderr, "failed: %s (line %d): %s\n", #c, __LINE__, hq_last_error());         \
      return 1;                                                                             \
    }                                                                                       \
  } while (0)

static hq_layer_desc w4a16_layer(int64_t n, int64_t k) {
  hq_layer_desc l;
  memset(&l, 0, sizeof l);
  l.n = n;
  l.k = k;
  l.num_experts = 1;
  l.q.w_elem = HQ_U4;
  l.q.w_bits = 4;
  l.q.group_size = 128;
  l.q.scale = HQ_BF16;
  l.q.zp = HQ_ZP_PER_GROUP_U4;
  l.q.act = HQ_BF16;
  l.q.act_scale = HQ_ASCALE_NONE;
  l.q.out = HQ_BF16;
  return l;
}

int main(void) {
  hq_layer_desc l = w4a16_layer(4096, 4096);
  hq_compute c;
  hq_plan* p = NULL;
  char buf[512];
  size_t wb = 0, mb = 0, ws = 1;
  hq_tuning t;
  int tuned = -1;

  CHECK(hq_abi_version() == HQ_ABI_VERSION);
  CHECK(strcmp(hq_status_str(HQ_ERR_WORKSPACE), "") != 0);
  c.kind = HQ_GEMM_DENSE;
  c.epi = HQ_EPI_NONE;
  c.mfma_in = HQ_MFMA_AUTO;
  CHECK(hq_plan_create(&l, &c, 64, NULL, &p) == HQ_OK && p != NULL);
  CHECK(hq_plan_describe(p, 1, buf, sizeof buf) == HQ_OK && strstr(buf, "kernel=skinny") != NULL);
  CHECK(hq_repacked_bytes(p, &wb, &mb) == HQ_OK && wb == (size_t)4096 * 4096 / 2 && mb > 0);
  CHECK(hq_plan_workspace_bytes(p, 1, &ws) == HQ_OK && ws == 0);
  memset(&t, 0, sizeof t);
  CHECK(hq_plan_get_tuning(p, 1, &t, &tuned) == HQ_OK && tuned == 0 && t.kernel == 1);
  /* rejections happen before any launch */
  CHECK(hq_gemm(p, 65, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == HQ_ERR_INVALID_ARG);
  CHECK(strlen(hq_last_error()) > 0);
  CHECK(hq_moe_gemm_by_slot(p, 1, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
        HQ_ERR_INVALID_ARG); /* a dense plan */
  CHECK(hq_plan_destroy(p) == HQ_OK);

  /* INT4 with per-group zero points and int8 activations has no kernel */
  l.q.act = HQ_INT8;
  l.q.act_scale = HQ_ASCALE_PER_TOKEN_F32;
  p = NULL;
  CHECK(hq_plan_create(&l, &c, 64, NULL, &p) == HQ_ERR_UNSUPPORTED && p == NULL);

  /* a grouped gate_up plan: 256 experts of [512, 7168] */
  l = w4a16_layer(512, 7168);
  l.num_experts = 256;
  l.q.zp = HQ_ZP_FIXED;
  l.q.zp_value = 8;
  c.kind = HQ_GEMM_GROUPED;
  c.epi = HQ_EPI_SILU_MUL;
  CHECK(hq_plan_create(&l, &c, 4096, NULL, &p) == HQ_OK);
  {
    int bm = 0;
    int64_t mp = 0;
    CHECK(hq_moe_block_m(p, 1, 8, &bm) == HQ_OK && bm == 16);
    CHECK(hq_moe_max_padded(1, 8, 256, bm, &mp) == HQ_OK && mp == 8 + 257 * 15 + 9);
  }
  CHECK(hq_repacked_bytes(p, &wb, &mb) == HQ_OK && wb == (size_t)256 * 512 * 7168 / 2);
  CHECK(hq_plan_destroy(p) == HQ_OK);
  puts("ok");
  return 0;
}
