// zq_prefill_impl.hpp -- the prefill MFMA tile (m > 64; one scale per tensor
// or one per row and 128 k) and its kernels; host launchers in
// zq_prefill.hip, instantiations per bit width in zq_prefill_b2/b4/b8.hip.
//
// The ZSE wiki article ("ZSE - open-source движок для запуска LLM локально на
// GPU - 2026", sections "Компилятор GPU-ядер (zse-compiler)" and "Оркестратор и
// GPU-ядра") lists a dequantizing matmul and a shared-memory tiled matmul;
// zQuantize (openclawradar articles, section "Componentes da arquitetura";
// lavx article, section "Technical Architecture") picks INT2..INT8 per
// tensor, and the .zse format (wiki, section "Формат модели .zse") scales
// each group of 128 weights of a row by its own fp16 value. Prefill is
// compute-bound (2 * 2048 flop per weight byte at m = 2048); the design is a
// bf16/fp16 MFMA GEMM for gfx950 with the dequantization in the registers
// that feed the matrix cores:
//   * a workgroup of 4 waves computes a 128 x 256 tile of Y; each wave owns
//     64 columns and all 128 rows as 4 x 2 MFMA 32x32x16 tiles (128 fp32
//     accumulators per lane, in vector registers), so each decoded weight
//     fragment feeds 4 MFMAs. Two workgroups share a CU (2 waves per SIMD):
//     while one wave decodes, the other keeps the matrix core busy;
//   * activations and weight codes move from memory straight into LDS
//     (buffer loads with the LDS destination, 16 bytes per lane): no
//     registers, no permutation and no address arithmetic per step;
//   * codes decode to exact bf16 / fp16 values with no offset: bf16 through
//     sign-extended byte conversions (the code moved to the top of its byte,
//     which multiplies it by 16 for INT4 and by 64 for INT2 -- folded into the
//     scale), fp16 through a magic-number decode (a code placed in a binary16
//     fraction is an exact q + offset) and one packed fp16 subtraction of the
//     offset;
//   * scales are applied in fp32, never to the bf16 weights (rounding q * s to
//     bf16 would cost each weight up to 2^-8 of its value, the order of the
//     error bound itself). Each output column keeps its accumulators in units
//     of the scale of the group it is in: at a group boundary they are
//     multiplied by s_old / s_new (one multiply per accumulator and group) and
//     the MFMAs of the new group add X * q in the new units; the epilogue
//     multiplies by the last scale. A zero scale keeps the old units and
//     zeroes the decoded codes of its group (the decode masks come from the
//     scale), so a zero group adds nothing. With one scale per tensor the
//     accumulators are in its units from the start;
//   * each k-step's vector ALU, LDS and load instructions are interleaved
//     between its MFMAs (sched_group_barrier), and each wave runs a copy of
//     the tile specialised for its index.
#pragma once
#include <algorithm>
#include <utility>

#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace zq {

constexpr int PF_BN = 256, PF_BK = 64, PF_GROUP = 128;
constexpr int PF_NS = 3;  // activation stages
// Tile heights: FI row tiles of 32 (FI = 4 for m > 64; 1 and 2 for the
// batched-decode range 17..64, where the weights stream once and the matrix
// cores have time to spare).
__host__ __device__ constexpr int pf_bm(int fi) { return 32 * fi; }
__host__ __device__ constexpr int pf_stage(int fi) { return pf_bm(fi) * PF_BK * 2; }  // bytes of one activation stage
__host__ __device__ constexpr int pf_fi(int64_t m) { return m <= 32 ? 1 : m <= 64 ? 2 : 4; }

template <int XT>
__device__ __forceinline__ f16v pf_mfma(u4 a, u4 b, f16v c) {
  if constexpr (XT == XF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

// byte offset of 16-byte piece kc (k/8 within a 64-k step) of tile row r in
// a stage: pieces XOR-swizzled by row, so that 8 lanes reading one piece
// column of 8 consecutive rows hit 8 different bank groups
// Rows r and r' of one group of 16 (or 8) lanes must land in different
// 16-byte bank groups: with 64 banks a 128-byte row covers half of them, so
// even and odd rows of 16 consecutive ones each need 8 distinct positions;
// with 32 banks, 8 consecutive rows do. sw(r) = (r & 7) ^ ((r >> 3) & 1) does
// both.
__device__ __forceinline__ int pf_sw(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int pf_off(int r, int kc) { return r * 128 + ((kc ^ pf_sw(r)) << 4); }

// buffer resource of a raw byte range (gfx9 descriptor: stride 0, data
// format of a plain 32-bit buffer)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Waits until at most N vector memory instructions of this wave are in
// flight. The loads here go straight to LDS, which the compiler's own wait
// counting does not follow: these explicit waits are the only ones that
// order them, and the memory clobber keeps LDS accesses on their side.
template <int N>
__device__ __forceinline__ void pf_wait() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// the same, then a workgroup barrier (__syncthreads would wait for all loads)
template <int N>
__device__ __forceinline__ void pf_barrier() {
  __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One k-step's instructions interleaved: each of its NM MFMAs followed by
// an even share of the vector ALU (NVALU), LDS read (NDS) and vector memory
// (NVM) instructions of the same scheduling region, so that they issue while
// the matrix core is busy (with one wave per SIMD, no other wave fills the
// gaps). Masks: 0x008 MFMA, 0x002 VALU, 0x100 DS read, 0x020 VMEM read.
template <int MASK, int N>
__device__ __forceinline__ void pf_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
template <int NM, int NVALU, int NDS, int NVM, int... T>
__device__ __forceinline__ void pf_interleave_seq(std::integer_sequence<int, T...>) {
  ((pf_group<0x008, 1>(), pf_group<0x100, (T + 1) * NDS / NM - T * NDS / NM>(),
    pf_group<0x002, (T + 1) * NVALU / NM - T * NVALU / NM>(), pf_group<0x020, (T + 1) * NVM / NM - T * NVM / NM>()),
   ...);
}
template <int NM, int NVALU, int NDS, int NVM>
__device__ __forceinline__ void pf_interleave() {
  pf_interleave_seq<NM, NVALU, NDS, NVM>(std::make_integer_sequence<int, NM>{});
}

// LDS of one workgroup, two per CU (80 KB at most): 3 activation stages and
// the code stages -- 2 for INT4 and INT8 (a wave's codes of a step are in its
// registers before the stage is loaded again), 3 for INT2 (a stage holds a
// pair of steps); per stage 4 waves x 64 rows x (INT2 32, INT4 32, INT8 64)
// bytes
__host__ __device__ constexpr int pf_cstage(int bits) { return bits == 8 ? 16384 : 8192; }
__host__ __device__ constexpr int pf_cr(int bits) { return bits == 2 ? 3 : 2; }
__host__ __device__ constexpr int pf_lds(int bits, int fi) {
  return PF_NS * pf_stage(fi) + pf_cr(bits) * pf_cstage(bits);
}
// workgroups per CU: 2 (4 with one row tile; 3 for INT8, whose code stages
// are twice as large)
__host__ __device__ constexpr int pf_wpc(int bits, int fi) { return fi != 1 ? 2 : bits == 8 ? 3 : 4; }
static_assert(pf_wpc(2, 4) * pf_lds(2, 4) <= 163840 && pf_wpc(4, 4) * pf_lds(4, 4) <= 163840 &&
                  pf_wpc(8, 4) * pf_lds(8, 4) <= 163840 && pf_wpc(4, 1) * pf_lds(4, 1) <= 163840 &&
                  pf_wpc(2, 1) * pf_lds(2, 1) <= 163840 && pf_wpc(8, 1) * pf_lds(8, 1) <= 163840,
              "the workgroups of a CU share its 160 KB of LDS");

__device__ __forceinline__ float pf_sx(uint32_t w, int b) { return (float)(int)(int8_t)(w >> (8 * b)); }
__device__ __forceinline__ uint32_t pf_bf(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, b2{(__bf16)lo, (__bf16)hi});
}
__device__ __forceinline__ uint32_t pf_hadd(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) + __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pf_h2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, h2{(_Float16)lo, (_Float16)hi});
}

// Magic-number decode (one scale per tensor): the 8 codes k0..k7 of one MFMA
// step become 4 dwords of 16-bit pairs (k 2j, 2j+1) = (q + BE, q + BO),
// exact; the offsets times the activations' row sums are removed in the
// epilogue. Pairs are built by
// one v_perm_b32 (the code byte copied to bytes 0 and 2, zeros elsewhere)
// and one and-xor (v_bitop3): the field mask, the sign flip and the magic
// exponent. The two halves may use different magic numbers.
template <int XT, int BITS>
struct PfMagic;

// INT4. bf16: both nibbles at fraction bits 3:0 under 128 (v >> 4 brings
// the odd nibble down): 136 + q. fp16: even nibble at bits 3:0 under 1024,
// odd nibble left at bits 7:4 under 64: 1032 + q, 72 + q; no shift.
template <int XT>
struct PfMagic<XT, 4> {
  static constexpr float BE = XT == XBF16 ? 136.f : 1032.f, BO = XT == XBF16 ? 136.f : 72.f;
  static constexpr uint32_t BW = XT == XBF16 ? 0x43084308u : 0x54806408u;  // (BE, BO) as a 16-bit pair
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk) {
    const uint32_t v = c[0][kk];
    if constexpr (XT == XBF16) {
      const uint32_t s = v >> 4;
      return u4{(__builtin_amdgcn_perm(s, v, 0x0C040C00u) & 0x000F000Fu) ^ 0x43084308u,
                (__builtin_amdgcn_perm(s, v, 0x0C050C01u) & 0x000F000Fu) ^ 0x43084308u,
                (__builtin_amdgcn_perm(s, v, 0x0C060C02u) & 0x000F000Fu) ^ 0x43084308u,
                (__builtin_amdgcn_perm(s, v, 0x0C070C03u) & 0x000F000Fu) ^ 0x43084308u};
    } else {
      return u4{(__builtin_amdgcn_perm(v, v, 0x0C000C00u) & 0x00F0000Fu) ^ 0x54806408u,
                (__builtin_amdgcn_perm(v, v, 0x0C010C01u) & 0x00F0000Fu) ^ 0x54806408u,
                (__builtin_amdgcn_perm(v, v, 0x0C020C02u) & 0x00F0000Fu) ^ 0x54806408u,
                (__builtin_amdgcn_perm(v, v, 0x0C030C03u) & 0x00F0000Fu) ^ 0x54806408u};
    }
  }
};

// INT2: a byte holds codes 4j..4j+3 at bits 1:0, 3:2, 5:4, 7:6.
// bf16: even codes at fraction bits 1:0 under 128, odd codes at bits 3:2 of
// the upper half under 32 (v >> 4 serves the upper two codes of each byte):
// 130 + q, 34 + q. fp16: every code at fraction bits 9:8 under 4 (the byte
// moved to the upper byte of its half, the sources shifted by 0, 2, 4, 6):
// 6 + q for both halves -- a small offset, so that the fp32 sums of long rows
// carry little of it.
template <int XT>
struct PfMagic<XT, 2> {
  static constexpr float BE = XT == XBF16 ? 130.f : 6.f, BO = XT == XBF16 ? 34.f : 6.f;
  static constexpr uint32_t BW = XT == XBF16 ? 0x42084302u : 0x46004600u;
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk) {
    const uint32_t v = c[0][kk >> 1];
    // bytes 2(kk&1) and 2(kk&1)+1 of the dword hold this step's 8 codes
    const uint32_t j0 = 2 * (kk & 1), j1 = j0 + 1;
    if constexpr (XT == XBF16) {
      constexpr uint32_t M = 0x000C0003u, K = 0x42084302u;  // field masks; exponents | sign flips
      const uint32_t s = v >> 4;
      auto pr = [&](uint32_t src, uint32_t j) __attribute__((always_inline)) {
        return (__builtin_amdgcn_perm(src, src, 0x0C000C00u | (j << 16) | j) & M) ^ K;
      };
      return u4{pr(v, j0), pr(s, j0), pr(v, j1), pr(s, j1)};
    } else {
      constexpr uint32_t M = 0x03000300u, K = 0x46004600u;
      auto pr = [&](uint32_t lo, uint32_t hi, uint32_t j) __attribute__((always_inline)) {
        return (__builtin_amdgcn_perm(hi, lo, 0x000C000Cu | ((4 + j) << 24) | (j << 8)) & M) ^ K;
      };
      const uint32_t v2 = v >> 2, v4 = v >> 4, v6 = v >> 6;
      return u4{pr(v, v2, j0), pr(v4, v6, j0), pr(v, v2, j1), pr(v4, v6, j1)};
    }
  }
};

// INT8. bf16: u = q + 128 (sign flip) converted to float exactly, upper
// halves joined: 128 + q. fp16: the flipped byte in fraction bits 7:0 under
// 1024: 1152 + q, one v_perm and one xor per pair.
template <int XT>
struct PfMagic<XT, 8> {
  static constexpr float BE = XT == XBF16 ? 128.f : 1152.f, BO = BE;
  static constexpr uint32_t BW = XT == XBF16 ? 0x43004300u : 0x64806480u;
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk) {
    const uint32_t v0 = c[kk >> 1][2 * (kk & 1)], v1 = c[kk >> 1][2 * (kk & 1) + 1];
    if constexpr (XT == XBF16) {
      auto pr = [](uint32_t v, int i) __attribute__((always_inline)) {
        const uint32_t f = v ^ 0x80808080u;
        const float lo = (float)((f >> (16 * i)) & 0xFFu), hi = (float)((f >> (16 * i + 8)) & 0xFFu);
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
      };
      return u4{pr(v0, 0), pr(v0, 1), pr(v1, 0), pr(v1, 1)};
    } else {
      return u4{__builtin_amdgcn_perm(v0, v0, 0x0C010C00u) ^ 0x64806480u,
                __builtin_amdgcn_perm(v0, v0, 0x0C030C02u) ^ 0x64806480u,
                __builtin_amdgcn_perm(v1, v1, 0x0C010C00u) ^ 0x64806480u,
                __builtin_amdgcn_perm(v1, v1, 0x0C030C02u) ^ 0x64806480u};
    }
  }
};

// Exact decoders: frag(c, kk, key) gives the 8 codes of MFMA k-step kk as 4
// dwords of 16-bit pairs (k 2d, 2d + 1) = F^-1 * (q, q'), all zero where the
// key was made from a zero mask. Code layout as in PfDec.
template <int XT, int BITS>
struct PfDec;

// bf16, INT4: nibble k 2d moved to the top of byte d (16 q), nibble 2d + 1
// already there
template <>
struct PfDec<XBF16, 4> {
  static constexpr float F = 1.f / 16;
  struct Key {
    uint32_t m;
  };
  static __device__ __forceinline__ Key key(uint32_t z) { return Key{0xF0F0F0F0u & z}; }
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk, Key kc) {
    const uint32_t v = c[0][kk];
    const uint32_t lo = (v << 4) & kc.m, hi = v & kc.m;
    return u4{pf_bf(pf_sx(lo, 0), pf_sx(hi, 0)), pf_bf(pf_sx(lo, 1), pf_sx(hi, 1)),
              pf_bf(pf_sx(lo, 2), pf_sx(hi, 2)), pf_bf(pf_sx(lo, 3), pf_sx(hi, 3))};
  }
};
// bf16, INT2: code j of byte d (bits 2j+1:2j) moved to the top of its byte
// by a shift of 6 - 2j (64 q)
template <>
struct PfDec<XBF16, 2> {
  static constexpr float F = 1.f / 64;
  struct Key {
    uint32_t m;
  };
  static __device__ __forceinline__ Key key(uint32_t z) { return Key{0xC0C0C0C0u & z}; }
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk, Key kc) {
    const uint32_t v = c[0][kk >> 1];
    const int j0 = 2 * (kk & 1), j1 = j0 + 1;
    const uint32_t c0 = (v << 6) & kc.m, c1 = (v << 4) & kc.m, c2 = (v << 2) & kc.m, c3 = v & kc.m;
    return u4{pf_bf(pf_sx(c0, j0), pf_sx(c1, j0)), pf_bf(pf_sx(c2, j0), pf_sx(c3, j0)),
              pf_bf(pf_sx(c0, j1), pf_sx(c1, j1)), pf_bf(pf_sx(c2, j1), pf_sx(c3, j1))};
  }
};
// bf16, INT8: the signed bytes converted as they are
template <>
struct PfDec<XBF16, 8> {
  static constexpr float F = 1.f;
  struct Key {
    uint32_t m;
  };
  static __device__ __forceinline__ Key key(uint32_t z) { return Key{z}; }
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk, Key kc) {
    const uint32_t v0 = c[kk >> 1][2 * (kk & 1)] & kc.m, v1 = c[kk >> 1][2 * (kk & 1) + 1] & kc.m;
    return u4{pf_bf(pf_sx(v0, 0), pf_sx(v0, 1)), pf_bf(pf_sx(v0, 2), pf_sx(v0, 3)), pf_bf(pf_sx(v1, 0), pf_sx(v1, 1)),
              pf_bf(pf_sx(v1, 2), pf_sx(v1, 3))};
  }
};
// fp16: the magic-number values of PfDec (field mask and exponent masked by
// the key, so a zero key gives +0), then the offset pair subtracted exactly
// by one packed fp16 add (also masked)
template <int BITS>
struct PfDec<XF16, BITS> {
  static constexpr float F = 1.f;
  struct Key {
    uint32_t m, k, nb;
  };
  static __device__ __forceinline__ Key key(uint32_t z) {
    if constexpr (BITS == 4) return Key{0x00F0000Fu & z, 0x54806408u & z, pf_h2(-1032.f, -72.f) & z};
    else if constexpr (BITS == 2) return Key{0x03000300u & z, 0x46004600u & z, pf_h2(-6.f, -6.f) & z};
    else return Key{z, 0x64806480u & z, pf_h2(-1152.f, -1152.f) & z};
  }
  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk, Key kc) {
    auto fin = [&](uint32_t p) __attribute__((always_inline)) { return pf_hadd((p & kc.m) ^ kc.k, kc.nb); };
    if constexpr (BITS == 4) {
      const uint32_t v = c[0][kk];
      return u4{fin(__builtin_amdgcn_perm(v, v, 0x0C000C00u)), fin(__builtin_amdgcn_perm(v, v, 0x0C010C01u)),
                fin(__builtin_amdgcn_perm(v, v, 0x0C020C02u)), fin(__builtin_amdgcn_perm(v, v, 0x0C030C03u))};
    } else if constexpr (BITS == 2) {
      const uint32_t v = c[0][kk >> 1];
      const uint32_t j0 = 2 * (kk & 1), j1 = j0 + 1;
      auto pr = [&](uint32_t lo, uint32_t hi, uint32_t j) __attribute__((always_inline)) {
        return fin(__builtin_amdgcn_perm(hi, lo, 0x000C000Cu | ((4 + j) << 24) | (j << 8)));
      };
      const uint32_t v2 = v >> 2, v4 = v >> 4, v6 = v >> 6;
      return u4{pr(v, v2, j0), pr(v4, v6, j0), pr(v, v2, j1), pr(v4, v6, j1)};
    } else {
      const uint32_t v0 = c[kk >> 1][2 * (kk & 1)], v1 = c[kk >> 1][2 * (kk & 1) + 1];
      return u4{fin(__builtin_amdgcn_perm(v0, v0, 0x0C010C00u)), fin(__builtin_amdgcn_perm(v0, v0, 0x0C030C02u)),
                fin(__builtin_amdgcn_perm(v1, v1, 0x0C010C00u)), fin(__builtin_amdgcn_perm(v1, v1, 0x0C030C02u))};
    }
  }
};

// One 128 x 256 tile of Y = X * dequant(Q)^T. GS: one scale per row and 128
// k (k a multiple of 128); else one scale for the tensor (k a multiple of
// 64), the accumulators in its units from the start. Four waves; wave w owns
// columns 64w..64w+63 and all 128 rows (4 x 2 tiles of MFMA 32x32x16).
//
// The k-steps of 64 run as in the per-tensor tile (activations and codes
// moved straight into LDS, two steps ahead; a barrier in the middle of each
// step), two steps per scale group. The first step of group g issues the
// scale loads of group g + 1; the second reads them (they arrived by its
// middle barrier), makes the decode keys for group g + 1 and the ratio of
// old to new units, which the first step of group g + 1 applies to the
// accumulators before its MFMAs.
template <int XT, int BITS, int W, bool GS, int FI>
__device__ __forceinline__ void pf_tile_w(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                                        int64_t n, int64_t k, const uint16_t* __restrict__ x, int64_t m,
                                        int64_t ldx, void* __restrict__ y, int64_t ldy, int yt, int64_t m0,
                                        int64_t n0, uint8_t* smem) {
  using D = PfDec<XT, BITS>;
  using Key = typename D::Key;
  // one scale per tensor: the magic-number decode, its offsets removed in the
  // epilogue with the activations' row sums (bf16 INT8 decodes exactly at
  // the same cost); group scales: the exact decode
  constexpr bool MAGIC = !GS && !(XT == XBF16 && BITS == 8);
  using MG = PfMagic<XT, BITS>;
  constexpr int FJ = 2, NS = PF_NS, CR = pf_cr(BITS), CST = pf_cstage(BITS);
  constexpr int BM = pf_bm(FI), STAGE = pf_stage(FI);
  constexpr int CB = 8 * BITS;  // code bytes of one row per 64-k step
  constexpr int NCL = BITS == 8 ? 2 : 1;
  constexpr int CDMA = BITS == 2 ? 1 : FJ * NCL;  // code loads issued per step
  constexpr int XDMA = FI;                        // activation loads per wave and step
  // vector memory instructions issued before the middle barrier of a step:
  // the codes two steps ahead and, in the first step of a group, the two
  // scale loads of the next group
  constexpr int VM_ODD = CDMA, VM_EVEN = VM_ODD + (GS ? 2 : 0);
  int tid_ = threadIdx.x;
  __asm__ volatile("" : "+v"(tid_));
  const int tid = tid_, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  constexpr int w = W;
  const int KT = (int)(k / PF_BK), G = (int)(k / PF_GROUP);
  const int64_t rowbytes = k * BITS / 8;

  // ---- activations: wave w moves tile rows 8FI w .. 8FI w + 8FI - 1 of
  // each step into LDS with FI direct loads of 8 rows x 128 bytes; lane l of
  // load c lands at slot l of its 1 KB (row 8FI w + 8c + l/8, position l%8),
  // so it reads piece (l%8) ^ sw(row) of that row. Rows past m re-read row
  // m - 1.
  const int64_t mrows = m - m0 < BM ? m - m0 : BM;
  const __amdgpu_buffer_rsrc_t xr = pf_rsrc(x + m0 * ldx, (uint32_t)(mrows * ldx * 2));
  uint32_t aoff[XDMA];
#pragma unroll
  for (int c = 0; c < XDMA; ++c) {
    const int r = 8 * FI * w + 8 * c + (lane >> 3);
    aoff[c] = (uint32_t)((r < mrows ? r : mrows - 1) * ldx * 2 + (((lane & 7) ^ pf_sw(r)) << 4));
  }
  auto dma_x = [&](int ks, int kt) __attribute__((always_inline)) {
    uint8_t* dst = smem + (kt % NS) * STAGE + 8 * FI * w * 128;
#pragma unroll
    for (int c = 0; c < XDMA; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(dst + c * 1024), 16,
                                               aoff[c], ks * (PF_BK * 2), 0, 0);
  };
  // ---- weight codes: as in the per-tensor tile, a ring of CR stages per wave
  const int64_t nrows = n - n0 < PF_BN ? n - n0 : PF_BN;
  const __amdgpu_buffer_rsrc_t wr = pf_rsrc(packed + n0 * rowbytes, (uint32_t)(nrows * rowbytes));
  uint32_t boff[FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int r = 64 * w + 32 * j + l32;
    boff[j] = (uint32_t)((r < nrows ? r : nrows - 1) * rowbytes + (BITS == 2 ? 16 : CB / 2) * g);
  }
  uint8_t* cwave = smem + NS * STAGE + w * (CST / 4);
  auto dma_codes = [&](int ks, int kt) __attribute__((always_inline)) {
    uint8_t* dst = cwave + (kt % CR) * CST;
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int i = 0; i < NCL; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(dst + (j * NCL + i) * 1024), 16, boff[j] + i * 16,
            ks * CB, 0, 0);
  };
  auto dma_codes2 = [&](int ps, int pt, int j) __attribute__((always_inline)) {
    uint8_t* dst = cwave + (pt % 3) * CST + j * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)dst, 16, boff[j], ps * 32,
                                             0, 0);
  };
  auto read_codes = [&](int kt, u4 (&cb)[FJ][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      if constexpr (BITS == 2) {
        const uint8_t* src = cwave + ((kt >> 1) % 3) * CST + j * 1024 + (l32 + 32 * (kt & 1)) * 16 + 8 * g;
        const u2 d = *reinterpret_cast<const u2*>(src);
        cb[j][0] = u4{d[0], d[1], 0u, 0u};
      } else {
        const uint8_t* src = cwave + (kt % CR) * CST;
#pragma unroll
        for (int i = 0; i < NCL; ++i) cb[j][i] = *reinterpret_cast<const u4*>(src + (j * NCL + i) * 1024 + lane * 16);
      }
    }
  };

  // ---- scales: the lane's two columns (rows of Q), one fp16 per group
  const gptr<const uint16_t> sp = to_global(scales);
  int64_t srow[FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int r = 64 * w + 32 * j + l32;
    srow[j] = GS ? (n0 + (r < nrows ? r : nrows - 1)) * G : 0;
  }
  float u[FJ], rat[FJ];  // units of each column; their ratio at the next boundary
  Key kc[FJ], kn[FJ];    // decode keys of this group and the next
  auto next_units = [&](const uint16_t (&s16)[FJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const float s = f16_bits_to_float(s16[j]) * (MAGIC ? 1.f : D::F);
      // one scale per tensor: y = s * acc, whatever s is
      const bool nz = !GS || s != 0.f;
      // ratio through the hardware reciprocal (1 ulp; exact for powers of 2)
      rat[j] = nz ? u[j] * __builtin_amdgcn_rcpf(s) : 1.f;
      u[j] = nz ? s : u[j];
      kn[j] = D::key(nz ? 0xFFFFFFFFu : 0u);
    }
  };

  f16v acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f16v{};

  auto read_a = [&](const uint8_t* st, int kk, u4 (&a)[FI]) __attribute__((always_inline)) {
    const int off = pf_off(l32, 4 * g + kk);
#pragma unroll
    for (int i = 0; i < FI; ++i) a[i] = *reinterpret_cast<const u4*>(st + off + i * 32 * 128);
  };
  auto mfmas = [&](const u4 (&a)[FI], const u4 (&b)[FJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = pf_mfma<XT>(a[i], b[j], acc[i][j]);
  };
  auto decode = [&](const u4 (&cb)[FJ][2], int kk, const Key (&key)[FJ], u4 (&b)[FJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      if constexpr (MAGIC) b[j] = MG::frag(cb[j], kk);
      else b[j] = D::frag(cb[j], kk, key[j]);
    }
  };
  // ---- row sums for the magic decode's offsets: in k-step kk the wave sums
  // the fragment of row tile (kk + W) & 3, if there is one, that it has in
  // registers for its MFMAs (every row tile and k-step once over the four
  // waves); bs[r]: rows 32r + l32, k-half g. The four waves' partials are
  // added at the end.
  float bs[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) bs[i] = 0.f;
  auto bias_sum = [&](const u4 (&a)[FI], int kk) __attribute__((always_inline)) {
    if constexpr (MAGIC) {
      const int r = (kk + W) & 3;
      if (r < FI) {
#pragma unroll
        for (int d = 0; d < 4; ++d) bs[r] = dot2<XT>(a[r][d], MG::BW, bs[r]);
      }
    }
  };
  auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] *= rat[j];
  };
  // decode of one k-step (both fragments) and its row sums
  constexpr int DEC_VALU = MAGIC ? 22 : XT == XF16 ? 26 : BITS == 2 ? 38 : 30;
  static_assert(FI == 1 || FI == 2 || FI == 4, "row tiles");

  u4 a0[FI], a1[FI], b0[FJ], b1[FJ];
  u4 cb[FJ][2], ncb[FJ][2];
  uint16_t s16[FJ];
  // prologue: codes and activations of steps 0 and 1, scales of group 0
  if constexpr (BITS == 2) {
    const int npair = (KT + 1) >> 1;
    dma_codes2(0, 0, 0);
    dma_codes2(0, 0, 1);
    dma_codes2(npair > 1 ? 1 : 0, 1, 0);
    dma_codes2(npair > 1 ? 1 : 0, 1, 1);
  } else {
    dma_codes(0, 0);
    dma_codes(1, 1);
  }
  dma_x(0, 0);
  dma_x(1, 1);
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    s16[j] = sp[srow[j]];
    u[j] = 1.f;
  }
  pf_barrier<0>();
  next_units(s16);
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    kc[j] = kn[j];
    rat[j] = 1.f;  // the accumulators start at zero
  }
  read_codes(0, cb);
  decode(cb, 0, kc, b0);
  read_a(smem, 0, a0);

  // one k-step of 64; ODD: the second step of its group
  auto step = [&]<int ODD>(int kt) __attribute__((always_inline)) {
    const uint8_t* cur = smem + (kt % NS) * STAGE;
    const uint8_t* nxt = smem + ((kt + 1) % NS) * STAGE;
    const int ks = kt + 2 < KT ? kt + 2 : KT - 1;  // past the end: reload the last step
    if constexpr (BITS == 2) {
      const int pt = (kt >> 1) + 2, npair = (KT + 1) >> 1;
      dma_codes2(pt < npair ? pt : npair - 1, pt, kt & 1);
    } else {
      dma_codes(ks, kt + 2);
    }
    if constexpr (GS && !ODD) {
      const int gs = (kt >> 1) + 1 < G ? (kt >> 1) + 1 : G - 1;
#pragma unroll
      for (int j = 0; j < FJ; ++j) s16[j] = sp[srow[j] + gs];
    }
    constexpr int VM_EARLY = ODD ? VM_ODD : VM_EVEN;
    // k-step 0 (the first step of a group first moves the accumulators to
    // the group's units)
    if constexpr (GS && !ODD) rescale();
    read_a(cur, 1, a1);
    decode(cb, 1, kc, b1);
    bias_sum(a0, 0);
    mfmas(a0, b0);
    pf_interleave<FI * FJ, DEC_VALU + (GS && !ODD ? FI * FJ * 16 : 0), FI, VM_EARLY>();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 1
    read_a(cur, 2, a0);
    decode(cb, 2, kc, b0);
    bias_sum(a1, 1);
    mfmas(a1, b1);
    pf_interleave<FI * FJ, DEC_VALU, FI, 0>();
    __builtin_amdgcn_sched_barrier(0);
    pf_barrier<VM_EARLY>();
    // the activations two steps ahead: their stage was read until step kt - 1,
    // which every wave has finished
    dma_x(ks, kt + 2);
    // k-step 2: the next step's codes; the second step of a group also
    // turns the next group's scales into keys and a ratio
    read_a(cur, 3, a1);
    decode(cb, 3, kc, b1);
    read_codes(kt + 1, ncb);
    if constexpr (GS && ODD) next_units(s16);
    bias_sum(a0, 2);
    mfmas(a0, b0);
    pf_interleave<FI * FJ, DEC_VALU + (GS && ODD ? 24 : 0), FI + (BITS == 2 ? FJ : FJ * NCL), XDMA>();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 3: the next step's first fragments
    read_a(nxt, 0, a0);
    if constexpr (GS && ODD) decode(ncb, 0, kn, b0);
    else decode(ncb, 0, kc, b0);
    bias_sum(a1, 3);
    mfmas(a1, b1);
    pf_interleave<FI * FJ, DEC_VALU, FI, 0>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      cb[j][0] = ncb[j][0];
      cb[j][1] = ncb[j][1];
      if constexpr (GS && ODD) kc[j] = kn[j];
    }
  };
  for (int gi = 0; gi < KT >> 1; ++gi) {
    step.template operator()<0>(2 * gi);
    step.template operator()<1>(2 * gi + 1);
  }
  if (!GS && (KT & 1)) step.template operator()<0>(KT - 1);  // one scale: k a multiple of 64 only

  // ---- epilogue: every load done and every wave past the loop; y = units *
  // acc (less the scaled offset sums of the row with the magic decode:
  // partials of the two k-halves added, then those of the four waves, in
  // LDS: [wave][row], then the total of row t by thread t)
  pf_barrier<0>();
  const float* sb = reinterpret_cast<const float*>(smem + 4 * BM * 4);
  if constexpr (MAGIC) {
    float* sbw = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const float v = bs[i] + __shfl_xor(bs[i], 32, 64);
      if (g == 0) sbw[w * BM + 32 * i + l32] = v;
    }
    __syncthreads();
    if (tid < BM)
      reinterpret_cast<float*>(smem + 4 * BM * 4)[tid] =
          u[0] * (sbw[tid] + sbw[BM + tid] + sbw[2 * BM + tid] + sbw[3 * BM + tid]);
    __syncthreads();
  }
  auto epi = [&]<int YT, bool EDGE>() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // D layout of 32x32: value r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
        // column l%32
        const int rl = 32 * i + 8 * q + 4 * g;
        f4 c4 = f4{};
        if constexpr (MAGIC) c4 = *reinterpret_cast<const f4*>(sb + rl);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int64_t row = m0 + rl + rr;
#pragma unroll
          for (int j = 0; j < FJ; ++j) {
            const int64_t col = n0 + 64 * w + 32 * j + l32;
            float v;
            if constexpr (MAGIC) v = __builtin_fmaf(u[j], acc[i][j][4 * q + rr], -c4[rr]);
            else v = u[j] * acc[i][j][4 * q + rr];
            if (!EDGE || (row < m && col < n)) store_y(y, row * ldy + col, v, YT);
          }
        }
      }
    }
  };
  const bool edge = m0 + BM > m || n0 + PF_BN > n;
  if (yt == YF32) {
    if (edge) epi.template operator()<YF32, true>();
    else epi.template operator()<YF32, false>();
  } else if (yt == YF16) {
    if (edge) epi.template operator()<YF16, true>();
    else epi.template operator()<YF16, false>();
  } else {
    if (edge) epi.template operator()<YBF16, true>();
    else epi.template operator()<YBF16, false>();
  }
  __syncthreads();  // every wave is done with the LDS: the next tile may reuse it
}

template <int XT, int BITS, bool GS, int FI>
__device__ __forceinline__ void pf_tile(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                                        int64_t n, int64_t k, const uint16_t* __restrict__ x, int64_t m,
                                        int64_t ldx, void* __restrict__ y, int64_t ldy, int yt, int64_t m0,
                                        int64_t n0, uint8_t* smem) {
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: pf_tile_w<XT, BITS, 0, GS, FI>(packed, scales, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
    case 1: pf_tile_w<XT, BITS, 1, GS, FI>(packed, scales, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
    case 2: pf_tile_w<XT, BITS, 2, GS, FI>(packed, scales, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
    default: pf_tile_w<XT, BITS, 3, GS, FI>(packed, scales, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
  }
}

// Single call: one tile per workgroup, grid (row blocks, column blocks). The
// hardware dispatches workgroups x-fastest and deals them out to the 8 XCDs
// in turn, so consecutive row blocks of one column block keep their
// activation rows within one XCD's L2 when there are 8k row blocks.
template <int XT, int BITS, bool GS, int FI>
__global__ __launch_bounds__(256, pf_wpc(BITS, FI)) void prefill_kernel(const uint8_t* __restrict__ packed,
                                                                  const uint16_t* __restrict__ scales, int64_t n,
                                                                  int64_t k, const uint16_t* __restrict__ x, int64_t m,
                                                                  int64_t ldx, void* __restrict__ y, int64_t ldy,
                                                                  int yt) {
  extern __shared__ __align__(16) uint8_t smem[];
  pf_tile<XT, BITS, GS, FI>(packed, scales, n, k, x, m, ldx, y, ldy, yt, (int64_t)blockIdx.x * pf_bm(FI),
                            (int64_t)blockIdx.y * PF_BN, smem);
}

// Prefill plan: the tiles of many products of one bit width and scale kind
// in one persistent launch (pf_wpc workgroups per CU). Plan order lists
// products by decreasing k, each product's tiles with the row block fastest
// (a product's tile count is a multiple of 8 when its row blocks are). Tile
// t belongs to queue t % 8, one queue per XCD: with 16 row blocks (m = 2048)
// an XCD then runs two row blocks of every product, so its activation rows
// stay in its own L2, and the last round of each queue is made of short
// tiles. A workgroup takes tiles from its XCD's queue (a device counter),
// then from the others' until all are empty, so every tile is computed
// whatever the grid. The last workgroup to finish leaves the counters at
// zero for the next run.
constexpr int PP_QUEUES = 8;

template <int XT, int BITS, bool GS, int FI>
__global__ __launch_bounds__(256, pf_wpc(BITS, FI)) void prefill_plan_kernel(const PrefillProblem* __restrict__ probs, int nprob,
                                                              int64_t total, uint32_t* __restrict__ sync) {
  extern __shared__ __align__(16) uint8_t smem[];
  // the tile, its product and its row and column blocks pass through the
  // first 16 bytes of the LDS, which no tile uses before the barrier that
  // follows their reading (loads from LDS read into scalar registers keep
  // the tile's addressing scalar)
  int* s_tile = reinterpret_cast<int*>(smem);  // tiles of one plan stay below 2^31
  int* s_prob = s_tile + 1;
  int* s_mb = s_tile + 2;
  int* s_nb = s_tile + 3;
  const int xcc = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & (PP_QUEUES - 1));  // HW_REG_XCC_ID
  int q = 0;  // queues tried so far, starting with this XCD's
  for (;;) {
    if (threadIdx.x == 0) {
      int64_t t = total;
      while (q < PP_QUEUES) {
        const int qi = (xcc + q) & (PP_QUEUES - 1);
        const int64_t j = (int64_t)__hip_atomic_fetch_add(sync + qi, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = qi + PP_QUEUES * j;
        if (t < total) break;
        ++q;  // this queue is empty
      }
      int p = 0, mb = 0, nb = 0;
      if (t < total) {
        int lo = 0, hi = nprob - 1;  // last product whose first tile is <= t
        while (lo < hi) {
          const int mid = (lo + hi + 1) / 2;
          if (probs[mid].tile0 <= t) lo = mid;
          else hi = mid - 1;
        }
        p = lo;
        const int local = (int)(t - probs[p].tile0), mt = (int)probs[p].mtiles;
        nb = local / mt;
        mb = local - nb * mt;
      }
      *s_tile = (int)(t < total ? t : total);
      *s_prob = p;
      *s_mb = mb;
      *s_nb = nb;
    }
    __syncthreads();
    // uniform values: read into scalar registers, so the tile's addressing
    // stays scalar
    const int64_t t = (int64_t)__builtin_amdgcn_readfirstlane(*s_tile);
    const int pi = __builtin_amdgcn_readfirstlane(*s_prob);
    const int mb = __builtin_amdgcn_readfirstlane(*s_mb), nb = __builtin_amdgcn_readfirstlane(*s_nb);
    __syncthreads();  // read before the tile's loads and thread 0's next tile
    if (t >= total) break;
    const PrefillProblem& pr = probs[pi];
    pf_tile<XT, BITS, GS, FI>(pr.packed, pr.scales, pr.n, pr.k, pr.x, pr.m, pr.ldx, pr.y, pr.ldy, pr.yt,
                              (int64_t)mb * pf_bm(FI), (int64_t)nb * PF_BN, smem);
  }
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(sync + PP_QUEUES, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
    for (int i = 0; i <= PP_QUEUES; ++i) __hip_atomic_store(sync + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// kernels of one bit width (instantiated in zq_prefill_b<BITS>.hip): plan ?
// prefill_plan_kernel : prefill_kernel, for activations of type xt, one scale
// per 128 k (gs) or per tensor, and fi row tiles
template <int BITS>
const void* prefill_fn(int xt, bool plan, bool gs, int fi) {
  auto pick = [&]<int XT, bool G, int FI>() -> const void* {
    return plan ? reinterpret_cast<const void*>(&prefill_plan_kernel<XT, BITS, G, FI>)
                : reinterpret_cast<const void*>(&prefill_kernel<XT, BITS, G, FI>);
  };
  auto by_fi = [&]<int XT, bool G>() -> const void* {
    return fi == 1 ? pick.template operator()<XT, G, 1>()
                   : fi == 2 ? pick.template operator()<XT, G, 2>() : pick.template operator()<XT, G, 4>();
  };
  auto by_gs = [&]<int XT>() -> const void* {
    return gs ? by_fi.template operator()<XT, true>() : by_fi.template operator()<XT, false>();
  };
  return xt == XF16 ? by_gs.template operator()<XF16>() : by_gs.template operator()<XBF16>();
}
const void* prefill_fn_b2(int xt, bool plan, bool gs, int fi);
const void* prefill_fn_b4(int xt, bool plan, bool gs, int fi);
const void* prefill_fn_b8(int xt, bool plan, bool gs, int fi);

}  // namespace zq
