/*
 * zq_oracle.c -- plain fp64 CPU oracle for the weight-only quantized linear
 * layer. TEST INFRASTRUCTURE: see zq_oracle.h for who may use it, the page
 * citations and the format definition.
 *
 * Everything here is deliberately written as the definition reads: no blocking,
 * no vectorisation, no reordering of sums.
 */
#include "zq_oracle.h"

#include <math.h>
#include <stddef.h>

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction bits)
 * and bfloat16 (1 sign, 8 exponent bits with bias 127, 7 fraction bits).      */

double zqo_f16_to_f64(uint16_t h) {
  int neg = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 15 - 10); /* (1 + f/2^10) * 2^(e-15) */
  return neg ? -v : v;
}

double zqo_bf16_to_f64(uint16_t h) {
  int neg = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  int f = h & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 127 - 7);  /* (1 + f/2^7) * 2^(e-127) */
  return neg ? -v : v;
}

/* Round |v| to the binary format with `fbits` fraction bits, exponent bias
 * `bias` and all-ones exponent reserved for inf/nan; ties to even. */
static uint16_t narrow(double v, int fbits, int ebits) {
  const int bias = (1 << (ebits - 1)) - 1;
  const uint16_t sign = signbit(v) ? (uint16_t)(1u << (fbits + ebits)) : 0;
  const uint16_t inf = (uint16_t)(((1u << ebits) - 1) << fbits);
  if (isnan(v)) return (uint16_t)(sign | inf | (1u << (fbits - 1)));
  double a = fabs(v);
  if (isinf(a)) return (uint16_t)(sign | inf);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);            /* a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;           /* unbiased exponent of a */
  const int Emin = 1 - bias;
  if (E > bias) return (uint16_t)(sign | inf);
  /* spacing of representable values around a */
  int qexp = (E < Emin) ? (Emin - fbits) : (E - fbits);
  double r = nearbyint(ldexp(a, -qexp)); /* exact scaling, then RNE to integer */
  uint32_t bits;
  if (E < Emin) {
    bits = (uint32_t)r;     /* subnormal count; r == 2^fbits is the min normal */
  } else {
    /* r in [2^fbits, 2^(fbits+1)]; the top value carries into the exponent */
    bits = ((uint32_t)(E + bias) << fbits) + ((uint32_t)r - (1u << fbits));
  }
  if (bits >= inf) return (uint16_t)(sign | inf);
  return (uint16_t)(sign | bits);
}

uint16_t zqo_f64_to_f16(double v) { return narrow(v, 10, 5); }
uint16_t zqo_f64_to_bf16(double v) { return narrow(v, 7, 8); }

double zqo_widen(const void* p, int dtype, int64_t i) {
  switch (dtype) {
    case ZQO_I8: return (double)((const int8_t*)p)[i];
    case ZQO_F16: return zqo_f16_to_f64(((const uint16_t*)p)[i]);
    case ZQO_BF16: return zqo_bf16_to_f64(((const uint16_t*)p)[i]);
    case ZQO_F32: return (double)((const float*)p)[i];
    default: return NAN;
  }
}

/* ------------------------------------------------------------------------- */

static int bits_ok(int bits) { return bits == 2 || bits == 4 || bits == 8; }

static int shape_ok(int64_t n, int64_t k, int bits, int group) {
  if (!bits_ok(bits)) return ZQO_ERR_UNSUPPORTED;
  if (group != 0 && group != 128) return ZQO_ERR_UNSUPPORTED;
  if (n < 0 || k < 0) return ZQO_ERR_INVALID_ARG;
  if (group == 128 && k % 128 != 0) return ZQO_ERR_UNSUPPORTED;
  if (k % (8 / bits) != 0) return ZQO_ERR_UNSUPPORTED;
  return ZQO_OK;
}

/* index of the scale that covers element (r, c) */
static int64_t scale_index(int64_t r, int64_t c, int64_t k, int group) {
  if (group == 0) return 0;
  return r * (k / group) + c / group;
}

int zqo_compute_scales(const void* w, int w_dtype, int64_t n, int64_t k,
                       int bits, int group, uint16_t* scales) {
  int st = shape_ok(n, k, bits, group);
  if (st) return st;
  if (w_dtype != ZQO_F16 && w_dtype != ZQO_BF16 && w_dtype != ZQO_F32)
    return ZQO_ERR_INVALID_ARG;
  const double qmax = (double)((1 << (bits - 1)) - 1);
  const int64_t unit_len = group == 0 ? n * k : group;
  const int64_t units = group == 0 ? 1 : n * (k / group);
  for (int64_t u = 0; u < units; ++u) {
    double a = 0.0;
    for (int64_t j = 0; j < unit_len; ++j) {
      int64_t idx;
      if (group == 0) {
        idx = j;
      } else {
        int64_t r = u / (k / group), g = u % (k / group);
        idx = r * k + g * group + j;
      }
      double v = zqo_widen(w, w_dtype, idx);
      if (!isfinite(v)) return ZQO_ERR_RANGE;
      if (fabs(v) > a) a = fabs(v);
    }
    uint16_t s16 = 0;
    if (a > 0.0) {
      s16 = zqo_f64_to_f16(a / qmax);
      if (zqo_f16_to_f64(s16) * qmax < a) s16 = (uint16_t)(s16 + 1); /* next fp16 up */
      if (!isfinite(zqo_f16_to_f64(s16))) return ZQO_ERR_RANGE;
    }
    scales[u] = s16;
  }
  return ZQO_OK;
}

int zqo_quantize(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                 int group, const uint16_t* scales, int8_t* codes) {
  int st = shape_ok(n, k, bits, group);
  if (st) return st;
  if (w_dtype != ZQO_F16 && w_dtype != ZQO_BF16 && w_dtype != ZQO_F32)
    return ZQO_ERR_INVALID_ARG;
  const double qmin = -(double)(1 << (bits - 1));
  const double qmax = (double)((1 << (bits - 1)) - 1);
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      double s = zqo_f16_to_f64(scales[scale_index(r, c, k, group)]);
      double v = zqo_widen(w, w_dtype, r * k + c);
      if (!isfinite(s) || !isfinite(v)) return ZQO_ERR_RANGE;
      double q = 0.0;
      if (s != 0.0) {
        q = nearbyint(v / s); /* double division, round half to even */
        if (q < qmin) q = qmin;
        if (q > qmax) q = qmax;
      }
      codes[r * k + c] = (int8_t)q;
    }
  }
  return ZQO_OK;
}

int zqo_pack(const int8_t* codes, int64_t n, int64_t k, int bits, uint8_t* packed) {
  int st = shape_ok(n, k, bits, 0);
  if (st) return st;
  const int per = 8 / bits;
  const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
  const unsigned mask = (1u << bits) - 1u;
  const int64_t row_bytes = k / per;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < row_bytes; ++j) {
      unsigned byte = 0;
      for (int i = 0; i < per; ++i) {
        int q = codes[r * k + j * per + i];
        if (q < lo || q > hi) return ZQO_ERR_RANGE;
        byte |= ((unsigned)q & mask) << (i * bits);
      }
      packed[r * row_bytes + j] = (uint8_t)byte;
    }
  }
  return ZQO_OK;
}

/* code of element (r, c) read from the packed rows */
static int code_at(const uint8_t* packed, int bits, int64_t k, int64_t r, int64_t c) {
  const int per = 8 / bits;
  const int64_t row_bytes = k / per;
  unsigned byte = packed[r * row_bytes + c / per];
  int i = (int)(c % per);
  int f = (int)((byte >> (i * bits)) & ((1u << bits) - 1u));
  if (f >= (1 << (bits - 1))) f -= (1 << bits); /* sign-extend */
  return f;
}

void zqo_unpack(const uint8_t* packed, int64_t n, int64_t k, int bits, int8_t* codes) {
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c)
      codes[r * k + c] = (int8_t)code_at(packed, bits, k, r, c);
}

void zqo_dequant(const int8_t* codes, int64_t n, int64_t k, int group,
                 const uint16_t* scales, double* out) {
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c)
      out[r * k + c] = (double)codes[r * k + c] *
                       zqo_f16_to_f64(scales[scale_index(r, c, k, group)]);
}

int zqo_gemm(const uint8_t* packed, int bits, const uint16_t* scales, int group,
             int64_t n, int64_t k, const void* x, int x_dtype, int64_t m,
             int64_t ldx, double* y, int64_t ldy) {
  int st = shape_ok(n, k, bits, group);
  if (st) return st;
  if (x_dtype != ZQO_F16 && x_dtype != ZQO_BF16 && x_dtype != ZQO_F32)
    return ZQO_ERR_INVALID_ARG;
  if (m < 0 || ldx < k || ldy < n) return ZQO_ERR_INVALID_ARG;
  for (int64_t mi = 0; mi < m; ++mi) {
    for (int64_t r = 0; r < n; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        double s = zqo_f16_to_f64(scales[scale_index(r, c, k, group)]);
        double wdeq = (double)code_at(packed, bits, k, r, c) * s;
        acc += zqo_widen(x, x_dtype, mi * ldx + c) * wdeq;
      }
      y[mi * ldy + r] = acc;
    }
  }
  return ZQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Asymmetric variant (ZSE wiki, section on the .zse model format). */

static int asym_shape_ok(int64_t n, int64_t k, int bits) {
  if (bits != 2 && bits != 4) return ZQO_ERR_UNSUPPORTED;
  if (n < 0 || k < 0) return ZQO_ERR_INVALID_ARG;
  if (k % 128 != 0) return ZQO_ERR_UNSUPPORTED;
  return ZQO_OK;
}

int zqo_compute_scales_zeros(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                             uint16_t* scales, uint16_t* zeros) {
  int st = asym_shape_ok(n, k, bits);
  if (st) return st;
  if (w_dtype != ZQO_F16 && w_dtype != ZQO_BF16 && w_dtype != ZQO_F32)
    return ZQO_ERR_INVALID_ARG;
  const double qmax = (double)((1 << bits) - 1);
  const int64_t gpr = k / 128;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t g = 0; g < gpr; ++g) {
      double lo = INFINITY, hi = -INFINITY;
      for (int64_t j = 0; j < 128; ++j) {
        double v = zqo_widen(w, w_dtype, r * k + g * 128 + j);
        if (!isfinite(v)) return ZQO_ERR_RANGE;
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      uint16_t s16 = zqo_f64_to_f16((hi - lo) / qmax);
      uint16_t z16 = zqo_f64_to_f16(lo);
      if (!isfinite(zqo_f16_to_f64(s16)) || !isfinite(zqo_f16_to_f64(z16))) return ZQO_ERR_RANGE;
      scales[r * gpr + g] = s16;
      zeros[r * gpr + g] = z16;
    }
  }
  return ZQO_OK;
}

int zqo_quantize_asym(const void* w, int w_dtype, int64_t n, int64_t k, int bits,
                      const uint16_t* scales, const uint16_t* zeros, uint8_t* codes) {
  int st = asym_shape_ok(n, k, bits);
  if (st) return st;
  if (w_dtype != ZQO_F16 && w_dtype != ZQO_BF16 && w_dtype != ZQO_F32)
    return ZQO_ERR_INVALID_ARG;
  const double qmax = (double)((1 << bits) - 1);
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      const int64_t si = r * (k / 128) + c / 128;
      double s = zqo_f16_to_f64(scales[si]);
      double z = zqo_f16_to_f64(zeros[si]);
      double v = zqo_widen(w, w_dtype, r * k + c);
      if (!isfinite(s) || !isfinite(z) || !isfinite(v)) return ZQO_ERR_RANGE;
      double q = 0.0;
      if (s != 0.0) {
        q = nearbyint((v - z) / s); /* double arithmetic, round half to even */
        if (q < 0.0) q = 0.0;
        if (q > qmax) q = qmax;
      }
      codes[r * k + c] = (uint8_t)q;
    }
  }
  return ZQO_OK;
}

int zqo_pack_u(const uint8_t* codes, int64_t n, int64_t k, int bits, uint8_t* packed) {
  int st = shape_ok(n, k, bits, 0);
  if (st) return st;
  const int per = 8 / bits;
  const unsigned qmax = (1u << bits) - 1u;
  const int64_t row_bytes = k / per;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < row_bytes; ++j) {
      unsigned byte = 0;
      for (int i = 0; i < per; ++i) {
        unsigned q = codes[r * k + j * per + i];
        if (q > qmax) return ZQO_ERR_RANGE;
        byte |= q << (i * bits);
      }
      packed[r * row_bytes + j] = (uint8_t)byte;
    }
  }
  return ZQO_OK;
}

/* unsigned code of element (r, c) read from the packed rows */
static unsigned ucode_at(const uint8_t* packed, int bits, int64_t k, int64_t r, int64_t c) {
  const int per = 8 / bits;
  const int64_t row_bytes = k / per;
  unsigned byte = packed[r * row_bytes + c / per];
  return (byte >> ((c % per) * bits)) & ((1u << bits) - 1u);
}

void zqo_unpack_u(const uint8_t* packed, int64_t n, int64_t k, int bits, uint8_t* codes) {
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c)
      codes[r * k + c] = (uint8_t)ucode_at(packed, bits, k, r, c);
}

void zqo_dequant_asym(const uint8_t* codes, int64_t n, int64_t k, const uint16_t* scales,
                      const uint16_t* zeros, double* out) {
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      const int64_t si = r * (k / 128) + c / 128;
      out[r * k + c] = (double)codes[r * k + c] * zqo_f16_to_f64(scales[si]) + zqo_f16_to_f64(zeros[si]);
    }
}

int zqo_gemm_asym(const uint8_t* packed, int bits, const uint16_t* scales, const uint16_t* zeros,
                  int64_t n, int64_t k, const void* x, int x_dtype, int64_t m, int64_t ldx,
                  double* y, int64_t ldy) {
  int st = asym_shape_ok(n, k, bits);
  if (st) return st;
  if (x_dtype != ZQO_F16 && x_dtype != ZQO_BF16 && x_dtype != ZQO_F32)
    return ZQO_ERR_INVALID_ARG;
  if (m < 0 || ldx < k || ldy < n) return ZQO_ERR_INVALID_ARG;
  for (int64_t mi = 0; mi < m; ++mi) {
    for (int64_t r = 0; r < n; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        const int64_t si = r * (k / 128) + c / 128;
        double wdeq = (double)ucode_at(packed, bits, k, r, c) * zqo_f16_to_f64(scales[si]) +
                      zqo_f16_to_f64(zeros[si]);
        acc += zqo_widen(x, x_dtype, mi * ldx + c) * wdeq;
      }
      y[mi * ldy + r] = acc;
    }
  }
  return ZQO_OK;
}
