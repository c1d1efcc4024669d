// zq_device.hpp -- device-side helpers shared by the HIP kernels of libzq:
// storage types, fp16/bf16 conversions, the code-to-half "magic" decode and
// wave64 cross-lane reductions. gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// Global-address-space views of pointers that come out of structs: loads and
// stores through generic pointers compile to FLAT instructions, which count
// against both the vector-memory and the LDS counters and make the compiler
// wait for every load in flight before any LDS access.
template <class T>
using gptr = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ gptr<T> to_global(T* p) {
  return (gptr<T>)(p);
}

enum XType { XF16 = 1, XBF16 = 2 };
enum YType { YF32 = 3, YF16 = 1, YBF16 = 2 };

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float f16_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}
template <int XT>
__device__ __forceinline__ float x_bits_to_float(uint16_t h) {
  if constexpr (XT == XF16) return f16_bits_to_float(h);
  else return bf16_bits_to_float(h);
}
// float -> fp16 / bf16, round to nearest even (hardware conversions).
__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Store one fp32 result in the requested output type.
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v, int yt) {
  if (yt == YF32) ((float*)y)[idx] = v;
  else if (yt == YF16) ((uint16_t*)y)[idx] = float_to_f16_bits(v);
  else ((uint16_t*)y)[idx] = float_to_bf16_bits(v);
}

// ---------------------------------------------------------- code extraction
// A packed dword holds E = 32/BITS codes. The decoder turns the pair of fields
// (i, i + E/2) -- which sit 16 bits apart -- into two 16-bit floats.
//  * Magic path (fp16 for every width, bf16 for INT2/INT4): one shift and one
//    and-or move each field to the top of the half's fraction and OR in the
//    exponent of 2^BITS, giving the exact value 2^BITS + u, where
//    u = q + 2^(BITS-1) once the field's sign bit has been flipped. Each decoded
//    half is q + BIAS, BIAS = 2^BITS + 2^(BITS-1).
//  * bf16 with INT8 (8-bit fields do not fit the 7-bit bf16 fraction): the
//    sign-flipped byte u = q + 128 is converted to float exactly
//    (v_cvt_f32_ubyte), and its upper 16 bits are the exact bf16; BIAS = 128.
// The kernels subtract BIAS * sum(x) once per 16-byte chunk instead of
// correcting every weight.
template <int BITS>
struct Codes {
  static constexpr int E = 32 / BITS;                 // codes per dword
  static constexpr int PAIRS = E / 2;                 // 16-bit pairs per dword
  static constexpr uint32_t SIGNS = BITS == 4 ? 0x88888888u : BITS == 8 ? 0x80808080u : 0xAAAAAAAAu;
};

template <int XT, int BITS>
struct Decoder {
  static constexpr int FB = XT == XF16 ? 10 : 7;      // fraction bits
  static constexpr int EB = XT == XF16 ? 15 : 127;    // exponent bias
  static constexpr bool MAGIC = BITS < FB;
  static constexpr int POS = FB - BITS;
  static constexpr uint32_t FIELD = ((1u << BITS) - 1u) << (POS > 0 ? POS : 0);
  static constexpr uint32_t MASK = FIELD | (FIELD << 16);
  static constexpr uint32_t EXP1 = (uint32_t)(EB + BITS) << FB;  // 2^BITS
  static constexpr uint32_t OR = EXP1 | (EXP1 << 16);
  static constexpr float BIAS = MAGIC ? (float)((1 << BITS) + (1 << (BITS - 1))) : 128.0f;

  // pair I of the sign-flipped dword v, as packed 16-bit values q + BIAS
  template <int I>
  static __device__ __forceinline__ uint32_t pair(uint32_t v) {
    if constexpr (MAGIC) {
      constexpr int SH = POS - I * BITS;
      uint32_t t;
      if constexpr (SH >= 0) t = v << SH;
      else t = v >> (-SH);
      return (t & MASK) | OR;
    } else {
      // INT8 into bf16: bytes I and I+2
      float lo = (float)((v >> (8 * I)) & 0xFFu);
      float hi = (float)((v >> (8 * (I + 2))) & 0xFFu);
      return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
  }
};

// dot of two packed 16-bit pairs, accumulated in fp32.
template <int XT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (XT == XF16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
}

// ---------------------------------------------------------- cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over each row of 16 lanes; every lane of the row receives the sum.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return v;
}

}  // namespace zq
