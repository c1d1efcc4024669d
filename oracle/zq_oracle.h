/*
 * zq_oracle.h -- plain, slow, fp64 CPU oracle for the weight-only quantized
 * linear layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this code. The product library never links
 * it, and this code includes nothing from the product library: the two share no
 * headers, helpers, tables or constants.
 *
 * What it computes (sources are web pages about the ZSE inference engine):
 *   - "ZSE wiki" = the wiki.iphoster.net article "ZSE - open-source движок для
 *     запуска LLM локально на GPU - 2026".
 *   - "openclawradar" = the openclawradar.com articles (pt and de) on ZSE,
 *     section "Componentes da arquitetura" / "Architekturkomponenten".
 *   - "lavx" = the news.lavx.hu article "ZSE: A Memory-Efficient LLM Inference
 *     Engine with Smart Resource Orchestration", section "Technical Architecture".
 *
 * Format (the ZSE wiki, section ".zse model format", gives groups of 128
 * weights, two 4-bit values per byte with the low nibble first, and fp16 scales;
 * its quantizer is asymmetric with a zero point. This library fixes the
 * symmetric signed variant; the per-tensor INT2..INT8 choice is zQuantize from
 * openclawradar and lavx):
 *   - codes q are two's-complement integers in [-2^(b-1), 2^(b-1)-1], b in {2,4,8};
 *   - packed along K, rows dense, no padding; 8/b codes per byte, code i of a
 *     byte in bits [b*i + b-1 : b*i] (so for INT4 the even k is the low nibble);
 *   - scales are IEEE binary16 bit patterns, one per tensor (group = 0) or one
 *     per 128 consecutive k of each output row (group = 128), layout [N][K/128];
 *   - dequantized weight w_deq[n][k] = q[n][k] * s(n,k), exact in double.
 *
 * Readings where the pages are silent are listed with each function.
 *
 * Parity pins: every function here is pinned by a CPU test against something
 * other than itself (library conversions, exhaustive round trips, closed forms,
 * brute force with exact rational arithmetic, hand-worked golden examples).
 */
#ifndef ZQ_ORACLE_H
#define ZQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes of the oracle (its own numbering). */
enum {
  ZQO_OK = 0,
  ZQO_ERR_INVALID_ARG = 1,
  ZQO_ERR_UNSUPPORTED = 2,
  ZQO_ERR_RANGE = 3
};

/* Element types of oracle inputs. */
enum { ZQO_I8 = 0, ZQO_F16 = 1, ZQO_BF16 = 2, ZQO_F32 = 3 };

/* IEEE 754 binary16 and bfloat16 conversions, written from the format
 * definitions. Narrowing rounds to nearest, ties to even; overflow gives inf. */
double   zqo_f16_to_f64(uint16_t h);
uint16_t zqo_f64_to_f16(double v);
double   zqo_bf16_to_f64(uint16_t h);
uint16_t zqo_f64_to_bf16(double v);

/* Exact widening of element i of a typed array to double. */
double zqo_widen(const void* p, int dtype, int64_t i);

/* Scales computed from float weights w[n][k] (step "a1"):
 *   a = max |w| over the unit; a == 0 -> scale +0;
 *   otherwise s16 = RNE_fp16(a / qmax), qmax = 2^(b-1)-1, bumped to the next
 *   fp16 if s16 * qmax < a (so no code clips);
 * non-finite w or a scale beyond the fp16 range -> ZQO_ERR_RANGE. */
int zqo_compute_scales(const void* w, int w_dtype, int64_t n, int64_t k,
                       int bits, int group, uint16_t* scales);

/* Codes: q = clamp(rne(w / s), -2^(b-1), 2^(b-1)-1), division in double;
 * s == 0 gives q = 0; a non-finite w or s -> ZQO_ERR_RANGE. */
int zqo_quantize(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                 int group, const uint16_t* scales, int8_t* codes);

/* Bit packing of codes [n][k] into [n][k*b/8] bytes, and its inverse
 * (sign-extending). k must be a multiple of 8/b. Codes outside the b-bit
 * signed range make zqo_pack return ZQO_ERR_RANGE. */
int  zqo_pack(const int8_t* codes, int64_t n, int64_t k, int bits, uint8_t* packed);
void zqo_unpack(const uint8_t* packed, int64_t n, int64_t k, int bits, int8_t* codes);

/* w_deq[n][k] = q * s in double (exact). */
void zqo_dequant(const int8_t* codes, int64_t n, int64_t k, int group,
                 const uint16_t* scales, double* out);

/* y[m][n] = sum over k ascending of double(x[m][k]) * (q[n][k] * s(n,k)),
 * reading q straight from the packed bytes. x has row stride ldx elements,
 * y has row stride ldy. Any row range of the weight can be passed by offsetting
 * `packed` and `scales` (rows are dense). */
int zqo_gemm(const uint8_t* packed, int bits, const uint16_t* scales, int group,
             int64_t n, int64_t k, const void* x, int x_dtype, int64_t m,
             int64_t ldx, double* y, int64_t ldy);

/* ---------------------------------------------------------------------------
 * Asymmetric variant: the quantizer the ZSE wiki prints in its section on the
 * .zse model format (unsigned codes, one fp16 scale and one fp16 zero point per
 * group of 128 weights, two 4-bit values per byte with the low nibble first).
 * For b bits, qmax = 2^b - 1 (the wiki's formula is the b = 4 case, qmax = 15);
 * b in {2, 4}, groups of 128 along K only.
 *
 * Readings where the page is silent:
 *   - max and min are taken over the group's weights widened exactly to double;
 *   - scale s16 = RNE_fp16((max - min) / qmax) and zero z16 = RNE_fp16(min),
 *     both computed in double, stored as fp16 bit patterns;
 *   - codes are computed from the stored s16 and z16:
 *     q = clamp(rne((w - z16) / s16), 0, qmax) in double, ties to even;
 *     s16 == 0 (max == min, or a span below the fp16 range) gives q = 0;
 *   - w_deq = q * s16 + z16, exact in double;
 *   - non-finite w, or a scale or zero beyond the fp16 range -> ZQO_ERR_RANGE.
 * Scales and zeros share the layout of the symmetric group scales: [N][K/128].
 */
int zqo_compute_scales_zeros(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                             uint16_t* scales, uint16_t* zeros);
int zqo_quantize_asym(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                      const uint16_t* scales, const uint16_t* zeros, uint8_t* codes);
/* Packing of unsigned codes in [0, 2^b - 1] (same bit positions as zqo_pack;
 * codes out of range -> ZQO_ERR_RANGE), and its inverse (no sign extension). */
int  zqo_pack_u(const uint8_t* codes, int64_t n, int64_t k, int bits, uint8_t* packed);
void zqo_unpack_u(const uint8_t* packed, int64_t n, int64_t k, int bits, uint8_t* codes);
void zqo_dequant_asym(const uint8_t* codes, int64_t n, int64_t k, const uint16_t* scales,
                      const uint16_t* zeros, double* out);
/* y[m][n] = sum over k ascending of double(x[m][k]) * (q[n][k] * s + z). */
int zqo_gemm_asym(const uint8_t* packed, int bits, const uint16_t* scales, const uint16_t* zeros,
                  int64_t n, int64_t k, const void* x, int x_dtype, int64_t m, int64_t ldx,
                  double* y, int64_t ldy);

#ifdef __cplusplus
}
#endif
#endif /* ZQ_ORACLE_H */
