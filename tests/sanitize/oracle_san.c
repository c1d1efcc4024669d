/* oracle_san.c -- drives every function of the fp64 oracle on small seeded
 * inputs, built with AddressSanitizer and UndefinedBehaviorSanitizer (host
 * code only). Returns nonzero on a failed round trip; the sanitizers abort on
 * any out-of-bounds access or undefined operation. Test infrastructure. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zq_oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return (uint32_t)(st >> 11);
}
static double uni(void) { return (rnd() & 0xFFFFFF) / 16777216.0 * 2.0 - 1.0; }

static int fails = 0;
#define CHECK(c, ...)              \
  do {                             \
    if (!(c)) {                    \
      fprintf(stderr, __VA_ARGS__); \
      fputc('\n', stderr);         \
      ++fails;                     \
    }                              \
  } while (0)

/* float weights of dtype dt (0 i8 is not a float type here) */
static void* make_w(int dt, int64_t cnt) {
  const size_t es = dt == 3 ? 4 : 2;
  uint8_t* p = malloc((size_t)cnt * es);
  for (int64_t i = 0; i < cnt; ++i) {
    const double v = uni() * 0.05;
    if (dt == 3) ((float*)p)[i] = (float)v;
    else if (dt == 1) ((uint16_t*)p)[i] = zqo_f64_to_f16(v);
    else ((uint16_t*)p)[i] = zqo_f64_to_bf16(v);
  }
  return p;
}

static void symmetric(int bits, int group, int dt) {
  const int64_t n = 5, k = 256, m = 3, ldx = k + 8, ldy = n + 1;
  const int64_t ns = group ? n * (k / group) : 1;
  void* w = make_w(dt, n * k);
  uint16_t* s = malloc(ns * 2);
  int8_t* q = malloc(n * k);
  int8_t* q2 = malloc(n * k);
  uint8_t* p = malloc(n * k * bits / 8);
  double* dq = malloc(n * k * sizeof(double));
  uint16_t* x = malloc(m * ldx * 2);
  double* y = malloc(m * ldy * sizeof(double));
  for (int64_t i = 0; i < m * ldx; ++i) x[i] = zqo_f64_to_bf16(uni());
  CHECK(zqo_compute_scales(w, dt, n, k, bits, group, s) == 0, "scales b%d g%d dt%d", bits, group, dt);
  CHECK(zqo_quantize(w, dt, n, k, bits, group, s, q) == 0, "quantize");
  CHECK(zqo_pack(q, n, k, bits, p) == 0, "pack");
  zqo_unpack(p, n, k, bits, q2);
  CHECK(memcmp(q, q2, n * k) == 0, "round trip b%d", bits);
  zqo_dequant(q, n, k, group, s, dq);
  CHECK(zqo_gemm(p, bits, s, group, n, k, x, 2, m, ldx, y, ldy) == 0, "gemm bf16");
  for (int64_t i = 0; i < m * ldx; ++i) x[i] = zqo_f64_to_f16(uni());
  CHECK(zqo_gemm(p, bits, s, group, n, k, x, 1, m, ldx, y, ldy) == 0, "gemm f16");
  /* one output recomputed from the dequantized weights */
  double r = 0;
  for (int64_t j = 0; j < k; ++j) r += zqo_f16_to_f64(x[ldx + j]) * dq[2 * k + j];
  CHECK(r == y[ldy + 2], "gemm vs dequant");
  free(w), free(s), free(q), free(q2), free(p), free(dq), free(x), free(y);
}

static void asymmetric(int bits, int dt) {
  const int64_t n = 3, k = 384, m = 2;
  const int64_t ns = n * (k / 128);
  void* w = make_w(dt, n * k);
  uint16_t *s = malloc(ns * 2), *z = malloc(ns * 2);
  uint8_t *q = malloc(n * k), *q2 = malloc(n * k), *p = malloc(n * k * bits / 8);
  double* dq = malloc(n * k * sizeof(double));
  uint16_t* x = malloc(m * k * 2);
  double* y = malloc(m * n * sizeof(double));
  for (int64_t i = 0; i < m * k; ++i) x[i] = zqo_f64_to_f16(uni());
  CHECK(zqo_compute_scales_zeros(w, dt, n, k, bits, s, z) == 0, "asym scales");
  CHECK(zqo_quantize_asym(w, dt, n, k, bits, s, z, q) == 0, "asym quantize");
  CHECK(zqo_pack_u(q, n, k, bits, p) == 0, "pack_u");
  zqo_unpack_u(p, n, k, bits, q2);
  CHECK(memcmp(q, q2, n * k) == 0, "asym round trip");
  zqo_dequant_asym(q, n, k, s, z, dq);
  CHECK(zqo_gemm_asym(p, bits, s, z, n, k, x, 1, m, k, y, n) == 0, "gemm asym");
  free(w), free(s), free(z), free(q), free(q2), free(p), free(dq), free(x), free(y);
}

int main(void) {
  const int bits[3] = {2, 4, 8};
  for (int b = 0; b < 3; ++b)
    for (int g = 0; g <= 128; g += 128)
      for (int dt = 1; dt <= 3; ++dt) symmetric(bits[b], g, dt);
  for (int b = 0; b < 2; ++b)
    for (int dt = 1; dt <= 3; ++dt) asymmetric(bits[b], dt);
  /* conversions: every fp16 pattern through double and back */
  for (uint32_t h = 0; h < 65536; ++h) {
    const double v = zqo_f16_to_f64((uint16_t)h);
    if (v == v) CHECK(zqo_f64_to_f16(v) == (uint16_t)h, "f16 round trip %u", h);
    const double vb = zqo_bf16_to_f64((uint16_t)h);
    if (vb == vb) CHECK(zqo_f64_to_bf16(vb) == (uint16_t)h, "bf16 round trip %u", h);
  }
  /* refused inputs */
  int8_t bad[8] = {9, 0, 0, 0, 0, 0, 0, 0};
  uint8_t pb[4];
  CHECK(zqo_pack(bad, 1, 8, 4, pb) != 0, "out-of-range code accepted");
  printf("oracle sanitizer run: %d failures\n", fails);
  return fails != 0;
}
