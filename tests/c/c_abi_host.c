/* Calls the library through its C header from plain C (no HIP types, no torch): the host
 * building blocks, the status strings and argument validation.  Prints one line per check
 * and exits non-zero on the first failure.  Device calls are only validated, never run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tq.h"

#define CHECK(cond, what)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      printf("FAIL %s\n", what);                           \
      return 1;                                            \
    }                                                      \
    printf("ok %s\n", what);                               \
  } while (0)

int main(void) {
  /* codebook: mirror-symmetric, sorted, thresholds between neighbouring levels */
  double lev[8], thr[7];
  CHECK(tq_codebook(128, 3, lev, thr) == TQ_OK, "tq_codebook(128, 3)");
  int sym = 1, sorted = 1;
  for (int i = 0; i < 8; ++i) sym &= lev[i] == -lev[7 - i];
  for (int i = 0; i < 7; ++i) sorted &= lev[i] < thr[i] && thr[i] < lev[i + 1];
  CHECK(sym && sorted && thr[3] == 0.0, "codebook symmetric and ordered");
  CHECK(tq_codebook(128, 0, lev, thr) == TQ_EINVAL, "tq_codebook rejects R = 0");

  /* rotation signs: +-1 only, deterministic, and seeds differ */
  int8_t s1[3 * 128], s2[3 * 128], s3[3 * 128];
  CHECK(tq_rotation_signs(7, 0, 128, s1) == TQ_OK && tq_rotation_signs(7, 0, 128, s2) == TQ_OK &&
            tq_rotation_signs(8, 0, 128, s3) == TQ_OK,
        "tq_rotation_signs");
  int pm = 1;
  for (int i = 0; i < 3 * 128; ++i) pm &= s1[i] == 1 || s1[i] == -1;
  CHECK(pm && memcmp(s1, s2, sizeof s1) == 0 && memcmp(s1, s3, sizeof s1) != 0,
        "signs are +-1, repeatable, seed-dependent");

  /* projection matrix: bf16 bit patterns of a roughly unit-variance Gaussian */
  uint16_t* S = (uint16_t*)malloc(128 * 128 * sizeof(uint16_t));
  CHECK(S && tq_qjl_matrix(3, 0, 128, 128, S) == TQ_OK, "tq_qjl_matrix");
  double m2 = 0.0;
  for (int i = 0; i < 128 * 128; ++i) {
    uint32_t u = (uint32_t)S[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    m2 += (double)f * f;
  }
  m2 /= 128 * 128;
  CHECK(fabs(m2 - 1.0) < 0.05, "S second moment near 1");
  free(S);

  /* status strings and validation before any device work */
  CHECK(strlen(tq_status_string(TQ_OK)) > 0 && strlen(tq_status_string(TQ_EINVAL)) > 0,
        "tq_status_string");
  tq_plan* plan = NULL;
  CHECK(tq_plan_create(0, 3, 0, NULL, 0, &plan) == TQ_EINVAL && plan == NULL, "plan d = 0 rejected");
  CHECK(tq_plan_create(128, 9, 0, NULL, 0, &plan) == TQ_EINVAL, "plan bits = 9 rejected");
  CHECK(tq_encode(NULL, NULL, TQ_BF16, 1, 128, NULL, NULL) == TQ_EINVAL, "encode without plan");
  CHECK(tq_topk(NULL, 1, 10, 3, NULL, NULL, NULL) == TQ_EINVAL, "topk with null buffers");
  CHECK(tq_score_noalloc(NULL, NULL, TQ_BF16, 4, 1, 128, NULL, 16, NULL, NULL) == TQ_EINVAL,
        "score_noalloc without plan");
  CHECK(tq_score_noalloc(NULL, NULL, TQ_BF16, 0, 0, 128, NULL, 0, NULL, NULL) == TQ_EINVAL,
        "score_noalloc without plan, empty sizes");
  CHECK(tq_score_topk(NULL, NULL, TQ_F32, 8, 1, 128, NULL, 100, 10, NULL, NULL, NULL) == TQ_EINVAL,
        "score_topk without plan");
  CHECK(tq_score_topk(NULL, NULL, TQ_F32, 8, 1, 128, NULL, 5, 10, NULL, NULL, NULL) == TQ_EINVAL,
        "score_topk with k > n");
  {
    uint8_t masks[2 * 64];
    memset(masks, 0, sizeof(masks));
    masks[3] = masks[64 + 5] = masks[64 + 6] = 1;          /* 1 and 2 outlier channels */
    CHECK(tq_plan_create_heads(64, 3, 0, 2, masks, 5, &plan) == TQ_EINVAL && plan == NULL,
          "layer plan with unequal outlier counts rejected");
    CHECK(tq_plan_create_heads(256, 3, 0, 2, masks, 5, &plan) == TQ_EINVAL, "layer plan d > 128 rejected");
    CHECK(tq_plan_create_heads(64, 3, 0, 2, NULL, 5, &plan) == TQ_EINVAL, "layer plan without masks rejected");
    CHECK(tq_plan_create_heads(64, 3, 0, 0, masks, 5, &plan) == TQ_EINVAL, "layer plan without heads rejected");
    CHECK(tq_encode_groups(NULL, NULL, TQ_BF16, 2, 4, 64, NULL, NULL) == TQ_EINVAL, "grouped encode without plan");
  }
  CHECK(tq_plan_create_mse(128, 0, 0, &plan) == TQ_EINVAL && plan == NULL, "mse plan bits = 0 rejected");
  CHECK(tq_plan_create_mse(128, 5, 0, &plan) == TQ_EINVAL, "mse plan bits = 5 rejected");
  CHECK(tq_plan_create_mse(128, 3, 0, NULL) == TQ_EINVAL, "mse plan without output");
  CHECK(tq_dequantize(NULL, NULL, 1, NULL, TQ_F32, 128, NULL) == TQ_EINVAL, "dequantize without plan");
  CHECK(tq_attend(NULL, NULL, 4, 1, 10, 1.0f, NULL, NULL, TQ_F32, 128, NULL) == TQ_EINVAL,
        "attend without plan");
  {
    tq_plan* vp = NULL;
    if (tq_plan_create_mse(128, 3, 1, &vp) == TQ_OK) {
      /* host-side limits fail before any device use */
      CHECK(tq_attend(vp, (const float*)16, 262140, 65535, 10, 1.0f, (const void*)16, (void*)16,
                      TQ_F32, 128, NULL) == TQ_EINVAL,
            "attend with 2^34 rows");
      CHECK(tq_attend(vp, (const float*)16, 4, 1, 1, 1.0f / 0.0f, (const void*)16, (void*)16,
                      TQ_F32, 128, NULL) == TQ_EINVAL,
            "attend with an infinite scale");
      tq_plan_destroy(vp);
    }
  }
  CHECK(tq_rerank(NULL, TQ_F32, 1, 64, NULL, TQ_F32, 10, 64, 64, NULL, 8, 9, NULL, NULL, NULL) ==
            TQ_EINVAL,
        "rerank with k > kc");
  CHECK(tq_rerank(NULL, TQ_F32, 1, 64, NULL, TQ_F32, 10, 64, 64, NULL, 300, 10, NULL, NULL, NULL) ==
            TQ_EINVAL,
        "rerank with kc > 256");
  CHECK(tq_rerank(NULL, TQ_F32, 0, 64, NULL, TQ_F32, 10, 64, 64, NULL, 8, 4, NULL, NULL, NULL) == TQ_OK,
        "rerank with no queries is a no-op");
  CHECK(tq_calibrate_outliers(NULL, TQ_F32, 0, 128, 128, 8, NULL, NULL, NULL) == TQ_EINVAL,
        "calibrate with no rows");
  CHECK(tq_calibrate_outliers(NULL, TQ_F32, 10, 128, 128, 129, NULL, NULL, NULL) == TQ_EINVAL,
        "calibrate with n_out > d");
  CHECK(tq_encode_scatter(NULL, NULL, TQ_BF16, 1, 128, NULL, 10, NULL, NULL) == TQ_EINVAL,
        "scatter without plan");
  tq_plan_destroy(NULL);
  printf("all passed\n");
  return 0;
}
