// zq_pack.hip -- quantize-and-pack and unpack kernels.
//
// The ZSE wiki article ("ZSE - open-source движок для запуска LLM локально на
// GPU - 2026", section "Формат модели .zse") quantizes groups of 128 weights
// once, at conversion time, stores fp16 scales and packs two 4-bit values per
// byte with the low nibble first. The pages' quantizer is asymmetric; this
// library's format is symmetric and signed (per tensor or per 128-group,
// INT2/INT4/INT8 -- the zQuantize widths of the openclawradar and lavx pages):
//   scale  a = max|w| over the unit; a == 0 -> +0; else
//          s16 = fp16_rne(a / qmax) (double division), raised by one fp16 step
//          when s16 * qmax < a, so the symmetric grid never clips;
//   code   q = clamp(rne(w / s16), -2^(b-1), 2^(b-1)-1), double division;
//   pack   code i of a byte in bits [b*i + b-1 : b*i], codes along K.
// Pack runs offline; it favours obviously exact arithmetic (fp64) over speed.
#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace zq {

// Exact widening of one input weight to float (f16, bf16 and f32 all fit).
__device__ __forceinline__ float load_w(const void* w, int wt, int64_t i) {
  if (wt == 1) return f16_bits_to_float(((const uint16_t*)w)[i]);
  if (wt == 2) return bf16_bits_to_float(((const uint16_t*)w)[i]);
  return ((const float*)w)[i];
}

// double -> IEEE binary16 bit pattern, round to nearest even, by integer
// manipulation of the double's significand. Overflow -> inf pattern.
__device__ uint16_t double_to_f16_rne(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7ff);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (ex == 0x7ff) return sign | (frac ? 0x7e00 : 0x7c00);
  if (ex == 0) return sign;  // double subnormals are far below half of fp16's smallest step
  const int e = ex - 1023;
  if (e > 15) return sign | 0x7c00;
  const uint64_t sig = (1ull << 52) | frac;  // value = sig * 2^(e-52)
  // fp16 step is 2^(e-10) for normal results, 2^-24 below 2^-14
  const int shift = (e >= -14) ? 42 : (28 - e);
  if (shift > 54) return sign;  // below a quarter of the smallest step
  const uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
  uint32_t bits = (e >= -14) ? (uint32_t)(((e + 15) << 10) + (int64_t)r - 1024) : (uint32_t)r;
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | (uint16_t)bits;
}

__device__ __forceinline__ double f16_bits_to_double(uint16_t h) {
  return (double)f16_bits_to_float(h);
}

// scale from an exact absmax (a >= 0, finite); sets FLAG_SCALE_RANGE on overflow
__device__ uint16_t scale_from_absmax(float a, int bits, uint32_t* flags) {
  if (a == 0.f) return 0;
  const double qmax = (double)((1 << (bits - 1)) - 1);
  const double ad = (double)a;
  uint16_t s = double_to_f16_rne(ad / qmax);
  if (f16_bits_to_double(s) * qmax < ad) s = (uint16_t)(s + 1);
  if ((s & 0x7c00u) == 0x7c00u) atomicOr(flags, FLAG_SCALE_RANGE);
  return s;
}

// One thread per (row, 128-group) unit.
__global__ void scales_group_kernel(const void* __restrict__ w, int wt, int64_t n, int64_t k,
                                    int bits, uint16_t* __restrict__ scales, uint32_t* flags) {
  const int64_t G = k / 128;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n * G) return;
  const int64_t r = u / G, g = u - r * G;
  float a = 0.f;
  bool finite = true;
  for (int i = 0; i < 128; ++i) {
    const float v = load_w(w, wt, r * k + g * 128 + i);
    finite = finite && __builtin_isfinite(v);
    a = fmaxf(a, fabsf(v));
  }
  if (!finite) {
    atomicOr(flags, FLAG_NONFINITE);
    scales[u] = 0;
    return;
  }
  scales[u] = scale_from_absmax(a, bits, flags);
}

// Whole-tensor absmax: per-thread max, block max in LDS, one atomicMax on the
// float's bit pattern (monotone for non-negative floats).
__global__ void absmax_kernel(const void* __restrict__ w, int wt, int64_t total, uint32_t* flags) {
  __shared__ float red[256];
  float a = 0.f;
  bool finite = true;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float v = load_w(w, wt, i);
    finite = finite && __builtin_isfinite(v);
    a = fmaxf(a, fabsf(v));
  }
  if (!finite) atomicOr(flags, FLAG_NONFINITE);
  red[threadIdx.x] = a;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(flags + 1, __float_as_uint(red[0]));
}

__global__ void tensor_scale_kernel(int bits, uint16_t* scales, uint32_t* flags) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const float a = __uint_as_float(flags[1]);
    scales[0] = (flags[0] & FLAG_NONFINITE) ? 0 : scale_from_absmax(a, bits, flags);
  }
}

// One thread per output byte: quantize (or range-check codes) and pack.
__global__ void quantize_pack_kernel(const void* __restrict__ w, int wt, int64_t n, int64_t k,
                                     int bits, int group, const uint16_t* __restrict__ scales,
                                     uint8_t* __restrict__ packed, uint32_t* flags) {
  const int per = 8 / bits;
  const int64_t rowbytes = k / per;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * rowbytes) return;
  const int64_t r = idx / rowbytes, jb = idx - r * rowbytes;
  const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
  uint32_t byte = 0, err = 0;
  for (int i = 0; i < per; ++i) {
    const int64_t c = jb * per + i;
    int q;
    if (wt == 0) {
      q = ((const int8_t*)w)[r * k + c];
      if (q < lo || q > hi) err |= FLAG_CODE_RANGE;
    } else {
      const uint16_t sb = group ? scales[r * (k / group) + c / group] : scales[0];
      const double s = f16_bits_to_double(sb);
      const double v = (double)load_w(w, wt, r * k + c);
      if (!__builtin_isfinite(v) || !__builtin_isfinite(s)) err |= FLAG_NONFINITE;
      double qd = 0.0;
      if (s != 0.0 && __builtin_isfinite(v) && __builtin_isfinite(s)) {
        qd = __builtin_rint(v / s);
        qd = qd < (double)lo ? (double)lo : qd;
        qd = qd > (double)hi ? (double)hi : qd;
      }
      q = (int)qd;
    }
    byte |= ((uint32_t)q & ((1u << bits) - 1u)) << (i * bits);
  }
  packed[idx] = (uint8_t)byte;
  if (err) atomicOr(flags, err);
}

// ---------------------------------------------------------------------------
// Asymmetric weights: the quantizer of the ZSE wiki's section on the .zse
// model format (unsigned codes, per 128-group fp16 scale (max - min) / qmax
// and zero point min, qmax = 2^b - 1). Codes come from the stored fp16 scale
// and zero: q = clamp(rne((w - z) / s), 0, qmax), double arithmetic.

// One thread per (row, 128-group) unit.
__global__ void scales_zeros_kernel(const void* __restrict__ w, int wt, int64_t n, int64_t k, int bits,
                                    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros,
                                    uint32_t* flags) {
  const int64_t G = k / 128;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= n * G) return;
  const int64_t r = u / G, g = u - r * G;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  bool finite = true;
  for (int i = 0; i < 128; ++i) {
    const float v = load_w(w, wt, r * k + g * 128 + i);
    finite = finite && __builtin_isfinite(v);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  if (!finite) {
    atomicOr(flags, FLAG_NONFINITE);
    scales[u] = 0;
    zeros[u] = 0;
    return;
  }
  const double qmax = (double)((1 << bits) - 1);
  const uint16_t s = double_to_f16_rne(((double)hi - (double)lo) / qmax);
  const uint16_t z = double_to_f16_rne((double)lo);
  if ((s & 0x7c00u) == 0x7c00u || (z & 0x7c00u) == 0x7c00u) atomicOr(flags, FLAG_SCALE_RANGE);
  scales[u] = s;
  zeros[u] = z;
}

// One thread per output byte: quantize (or range-check unsigned codes) and pack.
__global__ void quantize_pack_asym_kernel(const void* __restrict__ w, int wt, int64_t n, int64_t k, int bits,
                                          const uint16_t* __restrict__ scales,
                                          const uint16_t* __restrict__ zeros, uint8_t* __restrict__ packed,
                                          uint32_t* flags) {
  const int per = 8 / bits;
  const int64_t rowbytes = k / per;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * rowbytes) return;
  const int64_t r = idx / rowbytes, jb = idx - r * rowbytes;
  const int qmax = (1 << bits) - 1;
  uint32_t byte = 0, err = 0;
  for (int i = 0; i < per; ++i) {
    const int64_t c = jb * per + i;
    int q;
    if (wt == 0) {
      q = ((const int8_t*)w)[r * k + c];
      if (q < 0 || q > qmax) err |= FLAG_CODE_RANGE;
    } else {
      const int64_t si = r * (k / 128) + c / 128;
      const double s = f16_bits_to_double(scales[si]);
      const double z = f16_bits_to_double(zeros[si]);
      const double v = (double)load_w(w, wt, r * k + c);
      if (!__builtin_isfinite(v) || !__builtin_isfinite(s) || !__builtin_isfinite(z)) err |= FLAG_NONFINITE;
      double qd = 0.0;
      if (s != 0.0 && __builtin_isfinite(v) && __builtin_isfinite(s) && __builtin_isfinite(z)) {
        qd = __builtin_rint((v - z) / s);
        qd = qd < 0.0 ? 0.0 : qd;
        qd = qd > (double)qmax ? (double)qmax : qd;
      }
      q = (int)qd;
    }
    byte |= ((uint32_t)q & ((1u << bits) - 1u)) << (i * bits);
  }
  packed[idx] = (uint8_t)byte;
  if (err) atomicOr(flags, err);
}

// double -> bfloat16 bit pattern, round to nearest even: round to odd into
// float (24 bits, enough guard bits), then round float to bf16 (8 bits).
__device__ uint16_t double_to_bf16_rne(double d) {
  float f = __double2float_rz(d);
  uint32_t b = __float_as_uint(f);
  if ((double)f != d && __builtin_isfinite(f)) b |= 1u;  // sticky
  return float_to_bf16_bits(__uint_as_float(b));
}

// One thread per packed byte: decode its codes into the requested output.
// Asymmetric weights (zeros != nullptr) have unsigned codes and dequantize to
// q * s + z, computed exactly in double and rounded once to the output type.
__global__ void unpack_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                              const uint16_t* __restrict__ zeros, int bits, int group, int64_t n, int64_t k,
                              void* __restrict__ out, int out_dtype) {
  const int per = 8 / bits;
  const int64_t rowbytes = k / per;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * rowbytes) return;
  const int64_t r = idx / rowbytes, jb = idx - r * rowbytes;
  const uint32_t byte = packed[idx];
  for (int i = 0; i < per; ++i) {
    const int64_t c = jb * per + i;
    int q = (int)((byte >> (i * bits)) & ((1u << bits) - 1u));
    const int64_t o = r * k + c;
    if (zeros) {
      if (out_dtype == 0) {
        ((int8_t*)out)[o] = (int8_t)q;
      } else {
        const int64_t si = r * (k / 128) + c / 128;
        const double v = (double)q * f16_bits_to_double(scales[si]) + f16_bits_to_double(zeros[si]);
        if (out_dtype == 3) ((float*)out)[o] = (float)v;
        else if (out_dtype == 1) ((uint16_t*)out)[o] = double_to_f16_rne(v);
        else ((uint16_t*)out)[o] = double_to_bf16_rne(v);
      }
      continue;
    }
    if (q >= (1 << (bits - 1))) q -= (1 << bits);
    if (out_dtype == 0) {
      ((int8_t*)out)[o] = (int8_t)q;
    } else {
      const uint16_t sb = group ? scales[r * (k / group) + c / group] : scales[0];
      const float v = (float)q * f16_bits_to_float(sb);  // exact: <= 19 significant bits
      if (out_dtype == 3) ((float*)out)[o] = v;
      else if (out_dtype == 1) ((uint16_t*)out)[o] = float_to_f16_bits(v);
      else ((uint16_t*)out)[o] = float_to_bf16_bits(v);
    }
  }
}

static unsigned blocks_for(int64_t items, int threads) {
  return (unsigned)((items + threads - 1) / threads);
}

hipError_t launch_compute_scales(const PackArgs& a, uint16_t* scales_out) {
  if (a.group) {
    const int64_t units = a.n * (a.k / 128);
    if (units > 0)
      hipLaunchKernelGGL(scales_group_kernel, dim3(blocks_for(units, 256)), dim3(256), 0, a.stream,
                         a.w, a.wt, a.n, a.k, a.bits, scales_out, a.flags);
  } else {
    const int64_t total = a.n * a.k;
    const DeviceInfo& di = device_info();
    int64_t blocks = blocks_for(total, 256);
    if (blocks > (int64_t)di.num_cus * 8) blocks = (int64_t)di.num_cus * 8;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, a.stream, a.w, a.wt,
                       total, a.flags);
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(64), 0, a.stream, a.bits, scales_out,
                       a.flags);
  }
  return hipGetLastError();
}

hipError_t launch_compute_scales_zeros(const PackArgs& a, uint16_t* scales_out, uint16_t* zeros_out) {
  const int64_t units = a.n * (a.k / 128);
  if (units > 0)
    hipLaunchKernelGGL(scales_zeros_kernel, dim3(blocks_for(units, 256)), dim3(256), 0, a.stream, a.w, a.wt,
                       a.n, a.k, a.bits, scales_out, zeros_out, a.flags);
  return hipGetLastError();
}

hipError_t launch_quantize_pack_asym(const PackArgs& a) {
  const int64_t bytes = a.n * (a.k * a.bits / 8);
  if (bytes > 0)
    hipLaunchKernelGGL(quantize_pack_asym_kernel, dim3(blocks_for(bytes, 256)), dim3(256), 0, a.stream, a.w,
                       a.wt, a.n, a.k, a.bits, a.scales, a.zeros, a.packed, a.flags);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const PackArgs& a) {
  const int64_t bytes = a.n * (a.k * a.bits / 8);
  if (bytes > 0)
    hipLaunchKernelGGL(quantize_pack_kernel, dim3(blocks_for(bytes, 256)), dim3(256), 0, a.stream,
                       a.w, a.wt, a.n, a.k, a.bits, a.group, a.scales, a.packed, a.flags);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros, int bits,
                         int group, int64_t n, int64_t k, void* out, int out_dtype, hipStream_t stream) {
  const int64_t bytes = n * (k * bits / 8);
  if (bytes > 0)
    hipLaunchKernelGGL(unpack_kernel, dim3(blocks_for(bytes, 256)), dim3(256), 0, stream, packed,
                       scales, zeros, bits, group, n, k, out, out_dtype);
  return hipGetLastError();
}

}  // namespace zq
