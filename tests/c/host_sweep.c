/* Runs the library's host code over many shapes from plain C: the Lloyd-Max solver for
 * every padded length and index width, the Philox sign and projection generators, and plan
 * creation (which builds every host table before it allocates device memory) for inner-
 * product, split, TurboQuant-MSE and layer plans, each then described.  Meant for
 * a build of the host code under the address and undefined-behaviour sanitizers (with the
 * HIP calls standing in on host memory, plan creation succeeds; kernel launches report that
 * there is no device).  Prints "all passed". */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tq.h"

static int plan_ok(tq_status st, tq_plan* p, const char* what, int d, int bits) {
  if (st == TQ_OK || st == TQ_EDEVICE) {
    if (p != NULL) {
      tq_plan_desc desc;
      if (tq_plan_info(p, &desc) != TQ_OK || desc.d != d || desc.record_bytes <= 0) {
        printf("FAIL %s d=%d bits=%d: plan description\n", what, d, bits);
        return 0;
      }
    }
    tq_plan_destroy(p);
    return 1;
  }
  printf("FAIL %s d=%d bits=%d: %s\n", what, d, bits, tq_status_string(st));
  return 0;
}

int main(void) {
  static const int Ds[] = {32, 64, 128, 256, 512, 1024, 2048};
  double lev[16], thr[15];
  for (int i = 0; i < 7; ++i)
    for (int R = 1; R <= 4; ++R)
      if (tq_codebook(Ds[i], R, lev, thr) != TQ_OK) {
        printf("FAIL tq_codebook(%d, %d)\n", Ds[i], R);
        return 1;
      }
  printf("ok codebooks\n");

  int8_t* sg = (int8_t*)malloc(3 * 2048);
  uint16_t* S = (uint16_t*)malloc((size_t)2048 * 2048 * 2);
  if (!sg || !S) return 1;
  for (int i = 0; i < 7; ++i) {
    if (tq_rotation_signs(11, i & 1, Ds[i], sg) != TQ_OK ||
        tq_qjl_matrix(11, i & 1, Ds[i], Ds[i], S) != TQ_OK) {
      printf("FAIL generators D=%d\n", Ds[i]);
      return 1;
    }
  }
  free(sg);
  free(S);
  printf("ok generators\n");

  static const int ds[] = {2, 17, 32, 63, 96, 100, 128, 129, 200, 512, 1000, 1536, 2048};
  uint8_t* mask = (uint8_t*)malloc(2048);
  if (!mask) return 1;
  for (size_t i = 0; i < sizeof ds / sizeof ds[0]; ++i) {
    const int d = ds[i];
    for (int bits = 2; bits <= 5; ++bits) {
      tq_plan* p = NULL;
      tq_status st = tq_plan_create(d, bits, 5, NULL, 0, &p);
      if (!plan_ok(st, p, "plan", d, bits)) return 1;
      memset(mask, 0, (size_t)d);
      for (int c = 0; c < d; c += 4) mask[c] = 1;   /* a quarter of the channels */
      if (d >= 4) {
        p = NULL;
        st = tq_plan_create(d, bits, 5, mask, bits + 1 > 5 ? 5 : bits + 1, &p);
        if (!plan_ok(st, p, "split plan", d, bits)) return 1;
      }
      if (bits <= 4) {
        p = NULL;
        st = tq_plan_create_mse(d, bits, 5, &p);
        if (!plan_ok(st, p, "mse plan", d, bits)) return 1;
      }
    }
  }
  printf("ok plans\n");

  /* layer plans: 8 heads, a quarter of the channels each, rotated from head to head */
  static const int dl[] = {8, 64, 100, 128};
  for (size_t i = 0; i < sizeof dl / sizeof dl[0]; ++i) {
    const int d = dl[i], H = 8;
    uint8_t* m = (uint8_t*)calloc((size_t)H * d, 1);
    if (!m) return 1;
    for (int h = 0; h < H; ++h)
      for (int c = 0; c < d / 4; ++c) m[h * d + (c * 4 + h) % d] = 1;
    for (int bits = 2; bits <= 5; ++bits) {
      tq_plan* p = NULL;
      const tq_status st = tq_plan_create_heads(d, bits, 9, H, m, 5, &p);
      if (!plan_ok(st, p, "layer plan", d, bits)) return 1;
    }
    free(m);
  }
  free(mask);
  printf("ok layer plans\n");
  printf("all passed\n");
  return 0;
}
