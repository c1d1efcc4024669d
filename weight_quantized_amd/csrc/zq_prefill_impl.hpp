// zq_prefill_impl.hpp -- the prefill MFMA tile (m > 64, one scale per tensor)
// and its kernels; host launchers in zq_prefill.hip, instantiations per bit
// width in zq_prefill_b2/b4/b8.hip.
//
// The ZSE wiki article ("ZSE - open-source движок для запуска LLM локально на
// GPU - 2026", sections "Компилятор GPU-ядер (zse-compiler)" and "Оркестратор и
// GPU-ядра") lists a dequantizing matmul and a shared-memory tiled matmul, and
// zQuantize (openclawradar articles, section "Componentes da arquitetura";
// lavx article, section "Technical Architecture") picks INT2..INT8 per tensor.
// Prefill is compute-bound (2 * 2048 flop per weight byte at m = 2048); the
// design is a bf16/fp16 MFMA GEMM for gfx950 with the dequantization in the
// registers that feed the matrix cores:
//   * a workgroup of 4 waves (one per SIMD) computes a 256 x 256 tile of Y;
//     each wave owns 64 columns and all 256 rows as 8 x 2 MFMA 32x32x16
//     tiles (256 fp32 accumulators per lane, in the accumulation registers),
//     so each decoded weight fragment feeds 8 MFMAs;
//   * activations and weight codes move from memory straight into LDS
//     (buffer loads with the LDS destination, 16 bytes per lane): no
//     registers, no permutation and no address arithmetic per step;
//     activations fill a ring of stages shared by the workgroup, each wave's
//     codes three stages of its own;
//   * codes are decoded in their natural k order by magic numbers (a code
//     placed in a binary16 / bfloat16 fraction is an exact value q + bias),
//     one v_perm_b32 and one v_bitop3 per pair of k; the bias times each
//     activation row's sum is removed in the epilogue, the row sums taken
//     from the activation fragments the MFMAs read anyway;
//   * with one wave per SIMD, each k-step's vector ALU, LDS and load
//     instructions are interleaved between its MFMAs (sched_group_barrier),
//     and each wave runs a copy of the tile specialised for its index, so
//     its share of the row sums has static register indices.
#pragma once
#include <algorithm>
#include <utility>

#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace zq {

constexpr int PF_BM = 256, PF_BN = 256, PF_BK = 64;
constexpr int PF_STAGE = PF_BM * PF_BK * 2;  // bytes of one activation stage (32 KB)

template <int XT>
__device__ __forceinline__ f16v pf_mfma(u4 a, u4 b, f16v c) {
  if constexpr (XT == XF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

// Natural-order decode: the 8 codes k0..k7 of one MFMA step become 4 dwords
// of 16-bit pairs (k 2j, 2j+1) = (q + BE, q + BO), exact. Pairs are built by
// one v_perm_b32 (the code byte copied to bytes 0 and 2, zeros elsewhere)
// and one and-xor (v_bitop3): the field mask, the sign flip and the magic
// exponent. The two halves may use different magic numbers.
template <int XT, int BITS>
struct PfDec;

// INT4. bf16: both nibbles at fraction bits 3:0 under 128 (v >> 4 brings
// the odd nibble down): 136 + q. fp16: even nibble at bits 3:0 under 1024,
// odd nibble left at bits 7:4 under 64: 1032 + q, 72 + q; no shift.
template <int XT>
struct PfDec<XT, 4> {
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
struct PfDec<XT, 2> {
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
struct PfDec<XT, 8> {
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

// s_waitcnt with only vmcnt bounded (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

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

// LDS per bit width: activation stages (4, or 3 for INT8) and 3 weight-code
// stages of 4 waves x (INT2 1 KB, INT4 2 KB, INT8 4 KB)
__host__ __device__ constexpr int pf_ns(int bits) { return bits == 8 ? 3 : 4; }
__host__ __device__ constexpr int pf_cstage(int bits) { return bits == 8 ? 16384 : 8192; }
__host__ __device__ constexpr int pf_lds(int bits) { return pf_ns(bits) * PF_STAGE + 3 * pf_cstage(bits); }

// One 256 x 256 tile of Y = s * (X * (Q + bias)^T - bias sums), one scale per
// tensor. Four waves; wave w owns columns 64w..64w+63 of the tile and all 256
// rows (8 x 2 tiles of MFMA 32x32x16). k a multiple of 64.
//
// K runs in steps of 64. Activations and weight codes both move from memory
// straight into LDS: activations into a ring of 4 stages shared by the
// workgroup, each wave's codes into two stages of its own. Step kt decodes
// its weight fragments (from the codes that arrived during step kt - 1),
// issues the codes of step kt + 1 and the activations of step kt + 2, and
// computes its 4 MFMA k-steps; in its middle (after k-step 1) it waits until
// the activations of step kt + 1 are in LDS for every wave, so k-step 3
// already reads step kt + 1's first fragments. The activation stage written
// at step kt was last read in step kt - 2, which every wave finished before
// the middle barrier of step kt - 1.
template <int XT, int BITS, int W>
__device__ __forceinline__ void pf_tile_w(const uint8_t* __restrict__ packed, float scale, int64_t n, int64_t k,
                                        const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
                                        void* __restrict__ y, int64_t ldy, int yt, int64_t m0, int64_t n0,
                                        uint8_t* smem) {
  using D = PfDec<XT, BITS>;
  constexpr int FI = 8, FJ = 2, NS = pf_ns(BITS), CST = pf_cstage(BITS);
  constexpr int CB = 8 * BITS;  // code bytes of one row per 64-k step
  // 16-byte code loads per fragment and step: INT4 1, INT8 2; INT2 one per
  // pair of steps (issued one fragment per step)
  constexpr int NCL = BITS == 8 ? 2 : 1;
  constexpr int CDMA = BITS == 2 ? 1 : FJ * NCL;  // code loads issued per step
  // vector memory instructions issued before the middle barrier of a step
  // (the codes two steps ahead, and with 4 stages the activations too)
  constexpr int VM_EARLY = CDMA + (pf_ns(BITS) == 4 ? 8 : 0);
  int tid_ = threadIdx.x;
  __asm__ volatile("" : "+v"(tid_));
  const int tid = tid_, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  constexpr int w = W;
  const int KT = (int)(k / PF_BK);
  const int64_t rowbytes = k * BITS / 8;

  // ---- activations: wave w moves tile rows 64w..64w+63 of each step into LDS
  // with 8 direct loads of 8 rows x 128 bytes; lane l of load c lands at
  // slot l of its 1 KB (row 64w + 8c + l/8, position l%8), so it reads piece
  // (l%8) ^ (row & 7) of that row. Rows past m re-read row m - 1.
  const int64_t mrows = m - m0 < PF_BM ? m - m0 : PF_BM;
  const __amdgpu_buffer_rsrc_t xr = pf_rsrc(x + m0 * ldx, (uint32_t)(mrows * ldx * 2));
  uint32_t aoff[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int r = 64 * w + 8 * c + (lane >> 3);
    aoff[c] = (uint32_t)((r < mrows ? r : mrows - 1) * ldx * 2 + (((lane & 7) ^ pf_sw(r)) << 4));
  }
  // activations of step ks into the stage of step kt
  auto dma_x = [&](int ks, int kt) __attribute__((always_inline)) {
    uint8_t* dst = smem + (kt % NS) * PF_STAGE + 64 * w * 128;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(dst + c * 1024), 16,
                                               aoff[c], ks * (PF_BK * 2), 0, 0);
  };
  // ---- weight codes: lane (j, l32, g) takes the CB/2 bytes of row
  // n0 + 64w + 32j + l32 at byte CB/2 * g of each step (k 32g..32g+31); its
  // load i of fragment j lands at slot `lane` of 64 * CL_BYTES bytes
  const int64_t nrows = n - n0 < PF_BN ? n - n0 : PF_BN;
  const __amdgpu_buffer_rsrc_t wr = pf_rsrc(packed + n0 * rowbytes, (uint32_t)(nrows * rowbytes));
  uint32_t boff[FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    if constexpr (BITS == 2) {
      // INT2: lane l of fragment j's load takes bytes 16 (l / 32) .. + 15 of
      // row 64w + 32j + l%32 in each 128-k pair of steps (32 bytes per row)
      const int r = 64 * w + 32 * j + l32;
      boff[j] = (uint32_t)((r < nrows ? r : nrows - 1) * rowbytes + 16 * g);
    } else {
      const int r = 64 * w + 32 * j + l32;
      boff[j] = (uint32_t)((r < nrows ? r : nrows - 1) * rowbytes + (CB / 2) * g);
    }
  }
  uint8_t* cwave = smem + NS * PF_STAGE + w * (CST / 4);
  // codes of step ks into code stage of step kt (INT4/INT8)
  auto dma_codes = [&](int ks, int kt) __attribute__((always_inline)) {
    uint8_t* dst = cwave + (kt % 3) * CST;
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int i = 0; i < NCL; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(dst + (j * NCL + i) * 1024), 16, boff[j] + i * 16,
            ks * CB, 0, 0);
  };
  // INT2: fragment j of the step pair ps into the stage of pair pt
  auto dma_codes2 = [&](int ps, int pt, int j) __attribute__((always_inline)) {
    uint8_t* dst = cwave + (pt % 3) * CST + j * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)dst, 16,
                                             j == 0 ? boff[0] : boff[1], ps * 32, 0, 0);
  };
  auto read_codes = [&](int kt, u4 (&cb)[FJ][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      if constexpr (BITS == 2) {
        // step kt: pair kt / 2, half kt % 2 -> slot l32 + 32 (kt % 2), bytes 8g..
        const uint8_t* src = cwave + ((kt >> 1) % 3) * CST + j * 1024 + (l32 + 32 * (kt & 1)) * 16 + 8 * g;
        const u2 d = *reinterpret_cast<const u2*>(src);
        cb[j][0] = u4{d[0], d[1], 0u, 0u};
      } else {
        const uint8_t* src = cwave + (kt % 3) * CST;
#pragma unroll
        for (int i = 0; i < NCL; ++i) cb[j][i] = *reinterpret_cast<const u4*>(src + (j * NCL + i) * 1024 + lane * 16);
      }
    }
  };

  // ---- bias sums: from the fragments it has in registers for its MFMAs
  // anyway, the wave sums a[2kk], a[2kk+1] in k-step kk: bs[i] is the partial
  // of rows 32 rt(i) + l32 over k-half g and k-step i / 2 of every step. The
  // four waves' partials are added at the end.
  float bs[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) bs[i] = 0.f;
  auto bias_frags = [&](const u4 (&a)[FI], int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 2 * kk; i < 2 * kk + 2; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) bs[i] = dot2<XT>(a[i][d], D::BW, bs[i]);
  };

  f16v acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f16v{};

  // A fragment of row tile i, k-step kk: row 32i + l32, piece 4g + kk
  // this wave's row tiles in rotated order: a[i] and acc[i][.] belong to row
  // tile rt(i) = (i + 2W) & 7, so that the bias share of k-step kk is always
  // a[2kk], a[2kk+1] (row tiles 2(kk + W), +1 mod 8: every (row tile,
  // k-step) pair once over the four waves)
  auto rt = [](int i) { return (i + 2 * W) & 7; };
  auto read_a = [&](const uint8_t* st, int kk, u4 (&a)[FI]) __attribute__((always_inline)) {
    const int off = pf_off(l32, 4 * g + kk);
#pragma unroll
    for (int i = 0; i < FI; ++i) a[i] = *reinterpret_cast<const u4*>(st + off + rt(i) * 32 * 128);
  };
  auto mfmas = [&](const u4 (&a)[FI], const u4 (&b)[FJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = pf_mfma<XT>(a[i], b[j], acc[i][j]);
  };
  auto decode = [&](const u4 (&cb)[FJ][2], int kk, u4 (&b)[FJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) b[j] = D::frag(cb[j], kk);
  };
  constexpr int DEC_VALU = BITS == 8 && XT == XBF16 ? 28 : 18;  // decode of one k-step (both fragments)

  u4 a0[FI], a1[FI], b0[FJ], b1[FJ];
  u4 cb[FJ][2], ncb[FJ][2];
  // prologue: codes of steps 0 and 1, activations of steps 0 and 1
  if constexpr (BITS == 2) {
    const int npair = (KT + 1) >> 1;
    dma_codes2(0, 0, 0);
    dma_codes2(0, 0, 1);
    dma_codes2(npair > 1 ? 1 : 0, 1, 0);
    dma_codes2(npair > 1 ? 1 : 0, 1, 1);
  } else {
    dma_codes(0, 0);
    dma_codes(KT > 1 ? 1 : 0, 1);
  }
  dma_x(0, 0);
  dma_x(KT > 1 ? 1 : 0, 1);
  pf_barrier<0>();
  read_codes(0, cb);
  decode(cb, 0, b0);
  read_a(smem, 0, a0);
  // Every step issues the same loads and barriers (past the end they reload
  // the last step's data into stages nobody reads any more), so the loop
  // body has no branch and every wait count is exact.
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* cur = smem + (kt % NS) * PF_STAGE;
    const uint8_t* nxt = smem + ((kt + 1) % NS) * PF_STAGE;
    if constexpr (BITS == 2) {
      // load slot kt: pair kt/2 + 2, fragment kt % 2 (pair p is first read
      // in step 2p - 1, after the middle barriers of steps 2p - 3 and 2p - 2)
      const int pt = (kt >> 1) + 2, npair = (KT + 1) >> 1;
      dma_codes2(pt < npair ? pt : npair - 1, pt, kt & 1);
    } else {
      dma_codes(kt + 2 < KT ? kt + 2 : KT - 1, kt + 2);
    }
    if constexpr (NS == 4) dma_x(kt + 2 < KT ? kt + 2 : KT - 1, kt + 2);
    // k-step 0: MFMAs on (a0, b0); fetch a1, decode b1, the loads above. The
    // wave whose index is the k-step then sums the fragments' activations
    read_a(cur, 1, a1);
    decode(cb, 1, b1);
    bias_frags(a0, 0);
    mfmas(a0, b0);
    pf_interleave<FI * FJ, DEC_VALU + 8, FI, VM_EARLY>();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 1
    read_a(cur, 2, a0);
    decode(cb, 2, b0);
    bias_frags(a1, 1);
    mfmas(a1, b1);
    pf_interleave<FI * FJ, DEC_VALU + 8, FI, 0>();
    __builtin_amdgcn_sched_barrier(0);
    // middle of the step: every load issued before this step is done (the
    // activations of step kt + 1, the codes of step kt + 1), and every wave
    // has passed step kt - 1, whose stage this step's loads overwrite
    pf_barrier<VM_EARLY>();
    // with 3 stages the activations two steps ahead go out only now: their
    // stage was read until step kt - 1, which every wave has finished
    if constexpr (NS == 3) dma_x(kt + 2 < KT ? kt + 2 : KT - 1, kt + 2);
    // k-step 2: also read the next step's codes
    read_a(cur, 3, a1);
    decode(cb, 3, b1);
    read_codes(kt + 1, ncb);
    bias_frags(a0, 2);
    mfmas(a0, b0);
    pf_interleave<FI * FJ, DEC_VALU + 8, FI + (BITS == 2 ? FJ : FJ * NCL), NS == 3 ? 8 : 0>();
    __builtin_amdgcn_sched_barrier(0);
    // k-step 3: the next step's first fragments
    read_a(nxt, 0, a0);
    decode(ncb, 0, b0);
    bias_frags(a1, 3);
    mfmas(a1, b1);
    pf_interleave<FI * FJ, DEC_VALU + 8, FI, 0>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      cb[j][0] = ncb[j][0];
      cb[j][1] = ncb[j][1];
    }
  }

  // ---- epilogue: every load done and every wave past the loop; bias sums
  // to LDS (stage 0), then y = s * acc - s * (bias sum of the row)
  pf_barrier<0>();
  // partials of rows 32i + l32: add the two k-halves, then the four waves'
  // k-steps (LDS: [wave][row], then the total of row t by thread t)
  float* sbw = reinterpret_cast<float*>(smem + 4096);
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const float v = bs[i] + __shfl_xor(bs[i], 32, 64);
    if (g == 0) sbw[w * PF_BM + 32 * rt(i) + l32] = v;
  }
  __syncthreads();
  float* sb = reinterpret_cast<float*>(smem);
  sb[tid] = scale * (sbw[tid] + sbw[PF_BM + tid] + sbw[2 * PF_BM + tid] + sbw[3 * PF_BM + tid]);
  __syncthreads();
  // D layout of 32x32: value r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32. The output type and the edge checks are decided once per
  // tile, outside the element loops.
  auto epi = [&]<int YT, bool EDGE>() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rl = 32 * rt(i) + 8 * q + 4 * g;
        const f4 c4 = *reinterpret_cast<const f4*>(sb + rl);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int64_t row = m0 + rl + rr;
#pragma unroll
          for (int j = 0; j < FJ; ++j) {
            const int64_t col = n0 + 64 * w + 32 * j + l32;
            const float v = __builtin_fmaf(scale, acc[i][j][4 * q + rr], -c4[rr]);
            if (!EDGE || (row < m && col < n)) store_y(y, row * ldy + col, v, YT);
          }
        }
      }
    }
  };
  const bool edge = m0 + PF_BM > m || n0 + PF_BN > n;
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
  __syncthreads();  // the bias sums are read: the next tile may reuse the LDS
}

// the tile, specialised for the wave index (uniform, so each wave runs its
// own copy of the code with static register indices)
template <int XT, int BITS>
__device__ __forceinline__ void pf_tile(const uint8_t* __restrict__ packed, float scale, int64_t n, int64_t k,
                                        const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
                                        void* __restrict__ y, int64_t ldy, int yt, int64_t m0, int64_t n0,
                                        uint8_t* smem) {
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: pf_tile_w<XT, BITS, 0>(packed, scale, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
    case 1: pf_tile_w<XT, BITS, 1>(packed, scale, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
    case 2: pf_tile_w<XT, BITS, 2>(packed, scale, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
    default: pf_tile_w<XT, BITS, 3>(packed, scale, n, k, x, m, ldx, y, ldy, yt, m0, n0, smem); break;
  }
}


// Single call: one tile per workgroup. Tile i takes row block i % mtiles and
// column block i / mtiles, so the row blocks of consecutive workgroups --
// which the hardware deals out to the 8 XCDs in turn -- keep their
// activation rows within one XCD's L2 when mtiles is a multiple of 8.
template <int XT, int BITS>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const uint8_t* __restrict__ packed,
                                                         const uint16_t* __restrict__ scales, int64_t n, int64_t k,
                                                         const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
                                                         void* __restrict__ y, int64_t ldy, int yt, int mtiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int t = blockIdx.x, mb = t % mtiles, nb = t / mtiles;
  pf_tile<XT, BITS>(packed, f16_bits_to_float(scales[0]), n, k, x, m, ldx, y, ldy, yt, (int64_t)mb * PF_BM,
                    (int64_t)nb * PF_BN, smem);
}

// Prefill plan: the tiles of many products of one bit width in one persistent
// launch (one workgroup per CU). Plan order lists products by decreasing k,
// each product's tiles with the row block fastest. Tile t belongs to queue
// t % 8, one queue per XCD: with 8 row blocks (m = 2048) an XCD then runs one
// row block of every product, so its activation rows stay in its own L2,
// and the last round of each queue is made of short tiles. A workgroup takes
// tiles from its XCD's queue (a device counter), then from the others' until
// all are empty, so every tile is computed whatever the grid. The last
// workgroup to finish leaves the counters at zero for the next run.
constexpr int PP_QUEUES = 8;

template <int XT, int BITS>
__global__ __launch_bounds__(256, 1) void prefill_plan_kernel(const PrefillProblem* __restrict__ probs, int nprob,
                                                              int64_t total, uint32_t* __restrict__ sync) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_tile;  // tiles of one plan stay below 2^31
  __shared__ int s_prob;
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
      int p = 0;
      if (t < total) {
        int lo = 0, hi = nprob - 1;  // last product whose first tile is <= t
        while (lo < hi) {
          const int mid = (lo + hi + 1) / 2;
          if (probs[mid].tile0 <= t) lo = mid;
          else hi = mid - 1;
        }
        p = lo;
      }
      s_tile = (int)(t < total ? t : total);
      s_prob = p;
    }
    __syncthreads();
    // uniform values: read into scalar registers, so the tile's addressing
    // stays scalar
    const int64_t t = (int64_t)__builtin_amdgcn_readfirstlane(s_tile);
    const int pi = __builtin_amdgcn_readfirstlane(s_prob);
    __syncthreads();  // read before thread 0 takes the next tile
    if (t >= total) break;
    const PrefillProblem& pr = probs[pi];
    const int local = (int)(t - pr.tile0), mt = (int)pr.mtiles;
    const int nb = local / mt, mb = local - nb * mt;
    pf_tile<XT, BITS>(pr.packed, f16_bits_to_float(pr.scales[0]), pr.n, pr.k, pr.x, pr.m, pr.ldx, pr.y, pr.ldy,
                      pr.yt, (int64_t)mb * PF_BM, (int64_t)nb * PF_BN, smem);
  }
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(sync + PP_QUEUES, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
    for (int i = 0; i <= PP_QUEUES; ++i) __hip_atomic_store(sync + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// kernels of one bit width (instantiated in zq_prefill_b<BITS>.hip):
// plan ? prefill_plan_kernel : prefill_kernel, for activations of type xt
template <int BITS>
const void* prefill_fn(int xt, bool plan) {
  if (xt == XF16) return plan ? reinterpret_cast<const void*>(&prefill_plan_kernel<XF16, BITS>)
                              : reinterpret_cast<const void*>(&prefill_kernel<XF16, BITS>);
  return plan ? reinterpret_cast<const void*>(&prefill_plan_kernel<XBF16, BITS>)
              : reinterpret_cast<const void*>(&prefill_kernel<XBF16, BITS>);
}
const void* prefill_fn_b2(int xt, bool plan);
const void* prefill_fn_b4(int xt, bool plan);
const void* prefill_fn_b8(int xt, bool plan);

}  // namespace zq
