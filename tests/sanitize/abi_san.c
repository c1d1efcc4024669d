/* abi_san.c -- the host validation path of libzq, built host-only with
 * AddressSanitizer and UndefinedBehaviorSanitizer: every call below must be
 * refused (or accepted as empty) before any HIP call, with bogus pointers
 * that would fault if anything touched them. Returns nonzero on a wrong
 * status. Test infrastructure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "zq.h"

static int fails = 0;
static void expect(zq_status got, zq_status want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, want %d (%s)\n", what, (int)got, (int)want, zq_last_error());
    ++fails;
  }
}

static zq_weight W(int bits, int group, int64_t n, int64_t k) {
  zq_weight w;
  memset(&w, 0, sizeof w);
  w.bits = bits;
  w.group = group;
  w.n = n;
  w.k = k;
  w.packed = (const void*)0x100000;
  w.scales = (const uint16_t*)0x200000;
  return w;
}

int main(void) {
  void* X = (void*)0x300000;
  void* Y = (void*)0x400000;
  zq_weight w = W(4, 128, 16, 256);
  expect(zq_packed_bytes(4, 16, 256) == 2048 ? ZQ_OK : ZQ_ERR_HIP, ZQ_OK, "packed bytes");
  expect(zq_num_scales(128, 16, 256) == 32 ? ZQ_OK : ZQ_ERR_HIP, ZQ_OK, "num scales");
  for (int s = 0; s < 8; ++s)
    if (!zq_status_string((zq_status)s)) ++fails;
  /* zq_gemm */
  zq_weight b3 = W(3, 128, 16, 256), g64 = W(4, 64, 16, 256), k200 = W(4, 128, 16, 200), neg = W(4, 128, -1, 256);
  expect(zq_gemm(&b3, X, ZQ_F16, 1, 256, Y, ZQ_F32, 16, NULL), ZQ_ERR_UNSUPPORTED, "bits 3");
  expect(zq_gemm(&g64, X, ZQ_F16, 1, 256, Y, ZQ_F32, 16, NULL), ZQ_ERR_UNSUPPORTED, "group 64");
  expect(zq_gemm(&k200, X, ZQ_F16, 1, 200, Y, ZQ_F32, 16, NULL), ZQ_ERR_UNSUPPORTED, "k 200");
  expect(zq_gemm(&neg, X, ZQ_F16, 1, 256, Y, ZQ_F32, 16, NULL), ZQ_ERR_INVALID_ARG, "n -1");
  expect(zq_gemm(&w, X, ZQ_F32, 1, 256, Y, ZQ_F32, 16, NULL), ZQ_ERR_INVALID_ARG, "x dtype");
  expect(zq_gemm(&w, X, ZQ_F16, 2, 100, Y, ZQ_F32, 16, NULL), ZQ_ERR_INVALID_ARG, "ldx");
  expect(zq_gemm(&w, X, ZQ_F16, 1, 256, Y, ZQ_F32, 3, NULL), ZQ_ERR_INVALID_ARG, "ldy");
  expect(zq_gemm(&w, NULL, ZQ_F16, 1, 256, Y, ZQ_F32, 16, NULL), ZQ_ERR_INVALID_ARG, "null x");
  expect(zq_gemm(NULL, X, ZQ_F16, 1, 256, Y, ZQ_F32, 16, NULL), ZQ_ERR_INVALID_ARG, "null W");
  expect(zq_gemm(&w, X, ZQ_F16, 0, 256, Y, ZQ_F32, 16, NULL), ZQ_OK, "m = 0");
  expect(zq_gemv(&b3, X, ZQ_F16, Y, ZQ_F32, NULL), ZQ_ERR_UNSUPPORTED, "gemv bits");
  expect(zq_unpack(&w, Y, (zq_dtype)9, NULL), ZQ_ERR_INVALID_ARG, "unpack dtype");
  /* zq_pack / zq_pack_noalloc / zq_pack_asym */
  expect(zq_pack(X, ZQ_F32, 4, 256, 3, 128, NULL, Y, (uint16_t*)0x500000, NULL), ZQ_ERR_UNSUPPORTED, "pack bits");
  expect(zq_pack(X, ZQ_F32, 4, 100, 4, 128, NULL, Y, (uint16_t*)0x500000, NULL), ZQ_ERR_UNSUPPORTED, "pack k");
  expect(zq_pack(NULL, ZQ_F32, 4, 256, 4, 128, NULL, Y, (uint16_t*)0x500000, NULL), ZQ_ERR_INVALID_ARG, "pack w");
  expect(zq_pack_noalloc(X, ZQ_F32, 4, 256, 3, 128, NULL, Y, (uint16_t*)0x500000, NULL), ZQ_ERR_UNSUPPORTED,
         "noalloc bits");
  expect(zq_pack_asym(X, ZQ_F32, 4, 256, 8, NULL, NULL, Y, (uint16_t*)0x500000, (uint16_t*)0x600000, NULL),
         ZQ_ERR_UNSUPPORTED, "asym INT8");
  /* plans: lists refused before any allocation */
  zq_problem pr[2];
  memset(pr, 0, sizeof pr);
  for (int i = 0; i < 2; ++i) {
    pr[i].w = W(4, 0, 64, 512);
    pr[i].x = X;
    pr[i].x_dtype = ZQ_BF16;
    pr[i].ldx = 512;
    pr[i].y = Y;
    pr[i].y_dtype = ZQ_F32;
    pr[i].ldy = 64;
    pr[i].phase = i;
  }
  zq_plan plan = NULL;
  expect(zq_plan_create(pr, 2, 128, &plan), ZQ_ERR_UNSUPPORTED, "prefill plan, two phases");
  expect(zq_plan_create(pr, 2, 0, &plan), ZQ_ERR_UNSUPPORTED, "plan m = 0");
  pr[1].phase = 0;
  pr[1].x_dtype = ZQ_F16;
  expect(zq_plan_create(pr, 2, 128, &plan), ZQ_ERR_UNSUPPORTED, "prefill plan, two x types");
  pr[0].w = W(8, 128, 64, 512);
  pr[1].w = W(8, 128, 64, 512);
  pr[1].x_dtype = ZQ_BF16;
  pr[1].phase = 1;
  expect(zq_plan_create(pr, 2, 48, &plan), ZQ_ERR_UNSUPPORTED, "mid-batch INT8 in two phases");
  expect(zq_plan_create(NULL, 0, 1, &plan), ZQ_ERR_INVALID_ARG, "empty list");
  if (plan) ++fails;
  expect(zq_plan_destroy(NULL), ZQ_OK, "destroy null");
  printf("abi sanitizer run: %d failures\n", fails);
  return fails != 0;
}
