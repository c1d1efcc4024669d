// zq_prefill.hip -- MFMA kernel for prefill-sized batches (m > 64) with one
// scale per tensor: Y = X * dequant(W)^T, codes of 2, 4 or 8 bits.
//
// The ZSE wiki article ("ZSE - open-source движок для запуска LLM локально на
// GPU - 2026", sections "Компилятор GPU-ядер (zse-compiler)" and "Оркестратор и
// GPU-ядра") lists a dequantizing matmul and a shared-memory tiled matmul, and
// zQuantize (openclawradar articles, section "Componentes da arquitetura";
// lavx article, section "Technical Architecture") picks INT2..INT8 per tensor.
// Prefill is compute-bound (2 * 2048 flop per weight byte at m = 2048), so the
// design is a bf16/fp16 MFMA GEMM for gfx950 with the dequantization fused
// into the staging of the weight tile:
//   * a workgroup (8 waves, 2 x 4) computes a 256 x 256 tile of Y; each wave
//     128 x 64 as 4 x 2 MFMA 32x32x16 tiles (128 fp32 accumulators per lane,
//     in the accumulation registers), so two waves share each SIMD and hide
//     each other's LDS and memory waits;
//   * K runs in steps of 64. Activations go through LDS: the 256 x 64 tile of
//     step kt + 2 is loaded into registers while step kt computes, and step
//     kt + 1 is written to the other of two LDS stages at the end of step kt
//     (16-byte pieces XOR-swizzled by row: conflict-free writes and MFMA
//     fragment reads);
//   * weights bypass LDS (its bandwidth, ~128-155 bytes per clock per CU, is
//     the other limit of this design): each lane loads the 32 codes of its
//     own fragment row straight into registers, one step ahead, and decodes
//     them per MFMA with the magic-number decoder (code + BIAS as an exact
//     16-bit value, pairs (i, i + E/2) of a packed dword). The activations
//     are permuted into that same order when staged, so the MFMA sums
//     x * (q + BIAS) with matching pairs;
//   * every activation row's sum over K is accumulated while staging; the
//     epilogue stores s * (acc - BIAS * rowsum).
#include <algorithm>

#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace zq {

constexpr int P2_BM = 256, P2_BN = 256, P2_BK = 64;
constexpr int P2_TILE = 256 * 128;            // bytes of one 256-row x 64-k 16-bit activation tile
constexpr int P2_LDS = 2 * P2_TILE + 256 * 4;  // two stages + row sums

template <int XT>
__device__ __forceinline__ f16v p2_mfma(u4 a, u4 b, f16v c) {
  if constexpr (XT == XF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

// byte offset of 16-byte piece (row r, kc = k/8 within the 64-k step)
__device__ __forceinline__ int p2_off(int r, int kc) { return r * 128 + ((kc ^ (r & 7)) << 4); }

// Activations of one 16-k span (natural order, p0 = k 0..7, p1 = k 8..15) ->
// the two 8-element MFMA slots in the decoder's pair order for BITS:
//   INT4: slot g = k 8g + [0,4,1,5,2,6,3,7]
//   INT8: slot g = k 8g + [0,2,1,3,4,6,5,7]
//   INT2: slot g = k 4g + [0,8,1,9,2,10,3,11]
template <int BITS>
__device__ __forceinline__ void p2_perm(const u4& p0, const u4& p1, u4& s0, u4& s1) {
  // INT8: one v_perm_b32 each (byte selectors: 0-3 pick bytes of a, 4-7 of
  // b). INT2/INT4 keep shift-and-mask forms, which measured faster there.
  auto lo_lo = [](uint32_t a, uint32_t b) {
    if constexpr (BITS == 8) return __builtin_amdgcn_perm(b, a, 0x05040100u);
    else return (a & 0xFFFFu) | (b << 16);
  };
  auto hi_hi = [](uint32_t a, uint32_t b) {
    if constexpr (BITS == 8) return __builtin_amdgcn_perm(b, a, 0x07060302u);
    else return (a >> 16) | (b & 0xFFFF0000u);
  };
  if constexpr (BITS == 4) {
    s0 = u4{lo_lo(p0[0], p0[2]), hi_hi(p0[0], p0[2]), lo_lo(p0[1], p0[3]), hi_hi(p0[1], p0[3])};
    s1 = u4{lo_lo(p1[0], p1[2]), hi_hi(p1[0], p1[2]), lo_lo(p1[1], p1[3]), hi_hi(p1[1], p1[3])};
  } else if constexpr (BITS == 8) {
    s0 = u4{lo_lo(p0[0], p0[1]), hi_hi(p0[0], p0[1]), lo_lo(p0[2], p0[3]), hi_hi(p0[2], p0[3])};
    s1 = u4{lo_lo(p1[0], p1[1]), hi_hi(p1[0], p1[1]), lo_lo(p1[2], p1[3]), hi_hi(p1[2], p1[3])};
  } else {
    s0 = u4{lo_lo(p0[0], p1[0]), hi_hi(p0[0], p1[0]), lo_lo(p0[1], p1[1]), hi_hi(p0[1], p1[1])};
    s1 = u4{lo_lo(p0[2], p1[2]), hi_hi(p0[2], p1[2]), lo_lo(p0[3], p1[3]), hi_hi(p0[3], p1[3])};
  }
}

// sum of the 8 activations of a piece (v_dot2 against (1, 1))
template <int XT>
__device__ __forceinline__ float p2_sum8(const u4& p, float acc) {
  constexpr uint32_t ONES = XT == XF16 ? 0x3C003C00u : 0x3F803F80u;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = dot2<XT>(p[i], ONES, acc);
  return acc;
}

// Codes of one MFMA step kk for a lane's fragment: the lane holds 32 codes of
// its weight row (k 32g .. 32g+31 of the 64-k step, g = lane / 32) as
// INT4: one u4, INT8: two u4, INT2: one u2 (in a u4, upper half unused);
// step kk takes codes 8kk .. 8kk+7 of them, decoded in pair order, which
// matches activation piece kc = 4g + kk staged by p2_perm.
//
// bf16 INT4: a pair (code i, code i + 4) of a dword moves, by one shift (none
// for i = 0), to bits 3:0 of each 16-bit half; there it is the low fraction
// bits of the bf16 number 128, whose unit in the last place is 1:
// (t & M) | 0x4300 is the exact value 128 + u, u = q + 8 the code with its
// sign bit flipped. The flip folds into the masking, ((t ^ S) & M) | O ==
// (t & M) ^ ((S & M) ^ O): one v_bitop3 per pair; BIAS = 136.
// bf16 INT2: a pair (code i, code i + 8) moves to bits 3:2, fraction bits of
// the bf16 number 32 with unit 1: 32 + u, u = q + 2, BIAS = 34, again one
// v_bitop3 per pair and a shift for three of the four. (Bits 1:0 under 128
// cost the same but carry a 4 times larger offset into the fp32 sums, which
// for INT2's small weights came to a fifth of the tolerance at k = 18944;
// bits 6:5 under 4 need a fourth shift, 4 % slower.)
// BIAS is removed in the epilogue. fp16 activations keep the decoder with
// the offset 16 + u: with 1024 + u the fp32 sums of long rows would carry ten
// more bits of offset.
// INT8 (256 code values do not fit a bf16 fraction): byte -> float -> the
// upper 16 bits, exact; BIAS = 128.
template <int XT, int BITS>
struct P2Dec {
  static constexpr bool FAST = XT == XBF16 && BITS <= 4;
  static constexpr float BIAS = !FAST ? Decoder<XT, BITS>::BIAS : BITS == 4 ? 136.f : 34.f;
  static constexpr uint32_t M = BITS == 4 ? 0x000F000Fu : 0x000C000Cu;
  static constexpr uint32_t K = BITS == 4 ? 0x00080008u ^ 0x43004300u : 0x00080008u ^ 0x42004200u;

  static __device__ __forceinline__ u4 frag(const u4 (&c)[2], int kk) {
    using Dc = Decoder<XT, BITS>;
    constexpr uint32_t S = Codes<BITS>::SIGNS;
    if constexpr (FAST && BITS == 4) {
      const uint32_t v = c[0][kk];
      return u4{(v & M) ^ K, ((v >> 4) & M) ^ K, ((v >> 8) & M) ^ K, ((v >> 12) & M) ^ K};
    } else if constexpr (FAST) {
      const uint32_t v = c[0][kk >> 1] >> ((kk & 1) * 8);  // pairs 0..3 or 4..7
      return u4{((v << 2) & M) ^ K, (v & M) ^ K, ((v >> 2) & M) ^ K, ((v >> 4) & M) ^ K};
    } else if constexpr (BITS == 4) {
      const uint32_t v = c[0][kk] ^ S;
      return u4{Dc::template pair<0>(v), Dc::template pair<1>(v), Dc::template pair<2>(v), Dc::template pair<3>(v)};
    } else if constexpr (BITS == 8 && XT == XBF16) {
      // bytes I and I + 2 of a dword -> exact floats -> their upper halves,
      // joined by one v_perm_b32
      const uint32_t v0 = c[kk >> 1][2 * (kk & 1)] ^ S, v1 = c[kk >> 1][2 * (kk & 1) + 1] ^ S;
      auto pr = [](uint32_t v, int i) __attribute__((always_inline)) {
        const float lo = (float)((v >> (8 * i)) & 0xFFu), hi = (float)((v >> (8 * (i + 2))) & 0xFFu);
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
      };
      return u4{pr(v0, 0), pr(v0, 1), pr(v1, 0), pr(v1, 1)};
    } else if constexpr (BITS == 8) {
      const uint32_t v0 = c[kk >> 1][2 * (kk & 1)] ^ S, v1 = c[kk >> 1][2 * (kk & 1) + 1] ^ S;
      return u4{Dc::template pair<0>(v0), Dc::template pair<1>(v0), Dc::template pair<0>(v1),
                Dc::template pair<1>(v1)};
    } else {
      const uint32_t v = c[0][kk >> 1] ^ S;
      if (kk & 1)
        return u4{Dc::template pair<4>(v), Dc::template pair<5>(v), Dc::template pair<6>(v), Dc::template pair<7>(v)};
      return u4{Dc::template pair<0>(v), Dc::template pair<1>(v), Dc::template pair<2>(v), Dc::template pair<3>(v)};
    }
  }
};

// One 256 x 256 tile of Y (rows m0.., columns n0..) by the workgroup's
// WGM x WGN waves; wave (wm, wn) computes rows 256/WGM * wm.. and columns
// 256/WGN * wn.. of the tile as FI x FJ MFMA 32x32 tiles. Uses P2_LDS bytes
// of `smem`; ends with every wave past its last LDS access.
template <int XT, int BITS, int WGM, int WGN>
__device__ __forceinline__ void p2_tile(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
                                        int64_t n, int64_t k, const uint16_t* __restrict__ x, int64_t m, int64_t ldx,
                                        void* __restrict__ y, int64_t ldy, int yt, int64_t m0, int64_t n0,
                                        uint8_t* smem) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int TM = P2_BM / WGM, TN = P2_BN / WGN, FI = TM / 32, FJ = TN / 32;
  constexpr int SPT = 1024 / NT;            // 16-k activation spans per thread per step
  constexpr int CB = 8 * BITS;              // code bytes of one row per 64-k step
  constexpr int NB = BITS == 8 ? 2 : 1;     // 16-byte code loads per lane per fragment
  // the thread index goes through an empty asm: in the persistent plan
  // kernel this keeps lane-dependent offsets from being hoisted out of the
  // tile loop, where they would hold registers across it (and spill)
  int tid_ = threadIdx.x;
  __asm__ volatile("" : "+v"(tid_));
  const int tid = tid_, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = lane >> 5;
  const int64_t rowbytes = k * BITS / 8;
  const int64_t KT = k / P2_BK;
  float* rowsum = reinterpret_cast<float*>(smem + 2 * P2_TILE);

  // activation staging: spans (row = s/4, 16-k span s%4), s = it*NT + tid.
  // Rows past m re-read row m - 1: they only feed output rows past m, which
  // are not stored.
  const uint16_t* xrow[SPT];
#pragma unroll
  for (int it = 0; it < SPT; ++it) {
    const int s = it * NT + tid;
    const int64_t r = m0 + (s >> 2);
    xrow[it] = x + (r < m ? r : m - 1) * ldx + 16 * (s & 3);
  }
  // weight fragments of this wave: rows n0 + TN wn + 32 j + lane % 32, bytes
  // CB/2 * g of each step
  const uint8_t* wfr[FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int64_t r = n0 + wn * TN + 32 * j + (lane & 31);
    wfr[j] = packed + (r < n ? r : n - 1) * rowbytes + (CB / 2) * g;
  }

  // two register sets: tile kt + 2 is loaded while tile kt computes (codes
  // loaded two steps ahead measured slower: the third set of registers
  // costs more than the latency it hides)
  u4 xa0[SPT][2], xa1[SPT][2], wb0[FJ][2], wb1[FJ][2];
  float rs[SPT];
#pragma unroll
  for (int it = 0; it < SPT; ++it) rs[it] = 0.f;
  auto load_x = [&](int64_t kt, u4 (&xa)[SPT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < SPT; ++it) {
      const u4* p = reinterpret_cast<const u4*>(xrow[it] + kt * P2_BK);
      xa[it][0] = *to_global(p);
      xa[it][1] = *to_global(p + 1);
    }
  };
  auto load_w = [&](int64_t kt, u4 (&wb)[FJ][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const uint8_t* q = wfr[j] + kt * CB;
      if constexpr (BITS == 2) {
        const u2 t = __builtin_nontemporal_load(to_global(reinterpret_cast<const u2*>(q)));
        wb[j][0] = u4{t[0], t[1], 0u, 0u};
      } else {
#pragma unroll
        for (int i = 0; i < NB; ++i) wb[j][i] = __builtin_nontemporal_load(to_global(reinterpret_cast<const u4*>(q) + i));
      }
    }
  };
  // stage activation span `it` of a tile into LDS stage st
  auto stage_span = [&](uint8_t* st, const u4 (&xa)[SPT][2], int it) __attribute__((always_inline)) {
    const int s = it * NT + tid, r = s >> 2, sp = s & 3;
    const u4 p0 = xa[it][0], p1 = xa[it][1];
    rs[it] = p2_sum8<XT>(p1, p2_sum8<XT>(p0, rs[it]));
    u4 s0, s1;
    p2_perm<BITS>(p0, p1, s0, s1);
    *reinterpret_cast<u4*>(st + p2_off(r, 2 * sp)) = s0;
    *reinterpret_cast<u4*>(st + p2_off(r, 2 * sp + 1)) = s1;
  };

  f16v acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f16v{};

  auto read_a = [&](const uint8_t* cur, int kk, u4 (&a)[FI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
      a[i] = *reinterpret_cast<const u4*>(cur + p2_off(wm * TM + 32 * i + (lane & 31), 4 * g + kk));
  };
  // one K step: the tile in LDS stage kt & 1 with weight codes `wb`. The
  // fragments of step kk + 1 are read before the MFMAs of step kk; the
  // activations of tile kt + 1 (`nxa`) are staged into the other stage
  // between the MFMA steps.
  auto kstep = [&](int64_t kt, const u4 (&wb)[FJ][2], const u4 (&nxa)[SPT][2], u4 (&lxa)[SPT][2],
                   u4 (&lwb)[FJ][2]) __attribute__((always_inline)) {
    const uint8_t* cur = smem + (kt & 1) * P2_TILE;
    uint8_t* nxt = smem + ((kt + 1) & 1) * P2_TILE;
    const bool stage_next = kt + 1 < KT;
    if (kt + 2 < KT) load_x(kt + 2, lxa);  // tile kt's activations are already staged
    u4 a0[FI], a1[FI];
    read_a(cur, 0, a0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u4 (&a)[FI] = (kk & 1) ? a1 : a0;
      u4 (&an)[FI] = (kk & 1) ? a0 : a1;
      if (kk < 3) read_a(cur, kk + 1, an);
      u4 b[FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) b[j] = P2Dec<XT, BITS>::frag(wb[j], kk);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = p2_mfma<XT>(a[i], b[j], acc[i][j]);
      // spread this thread's spans over the 4 MFMA steps
#pragma unroll
      for (int it = 0; it < SPT; ++it)
        if (stage_next && (it * 4) / SPT == kk) stage_span(nxt, nxa, it);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 2 < KT) load_w(kt + 2, lwb);  // tile kt's codes are consumed
    __syncthreads();
  };

  load_x(0, xa0);
  load_w(0, wb0);
  if (KT > 1) {
    load_x(1, xa1);
    load_w(1, wb1);
  }
#pragma unroll
  for (int it = 0; it < SPT; ++it) stage_span(smem, xa0, it);
  __syncthreads();
  for (int64_t kt = 0; kt < KT; kt += 2) {
    kstep(kt, wb0, xa1, xa0, wb0);  // compute tile kt (codes in set 0); stage kt+1 (set 1); load kt+2 into set 0
    if (kt + 1 < KT) kstep(kt + 1, wb1, xa0, xa1, wb1);
  }

  // row sums: the 4 spans of a row are 4 consecutive threads
#pragma unroll
  for (int it = 0; it < SPT; ++it) {
    float v = rs[it];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    if ((tid & 3) == 0) rowsum[it * (NT / 4) + (tid >> 2)] = v;
  }
  __syncthreads();

  using Dc = P2Dec<XT, BITS>;
  const float s = f16_bits_to_float(scales[0]);
  // D layout of 32x32: value r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < FI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * TM + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
      const int64_t row = m0 + rl;
      const float corr = Dc::BIAS * rowsum[rl];
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int64_t col = n0 + wn * TN + 32 * j + (lane & 31);
        if (row < m && col < n) store_y(y, row * ldy + col, s * (acc[i][j][r] - corr), yt);
      }
    }
  }
  __syncthreads();  // the row sums are read: the next tile may reuse the LDS
}

template <int XT, int BITS, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_prefill2_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, int64_t n, int64_t k,
    const uint16_t* __restrict__ x, int64_t m, int64_t ldx, void* __restrict__ y, int64_t ldy, int yt) {
  extern __shared__ __align__(16) uint8_t smem[];
  p2_tile<XT, BITS, WGM, WGN>(packed, scales, n, k, x, m, ldx, y, ldy, yt, (int64_t)blockIdx.y * P2_BM,
                              (int64_t)blockIdx.x * P2_BN, smem);
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

template <int XT, int BITS, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_prefill_plan_kernel(const PrefillProblem* __restrict__ probs,
                                                                           int nprob, int64_t total,
                                                                           uint32_t* __restrict__ sync) {
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
    // stays scalar (LDS reads are taken as per-lane values otherwise)
    const int64_t t = (int64_t)__builtin_amdgcn_readfirstlane(s_tile);
    const int pi = __builtin_amdgcn_readfirstlane(s_prob);
    __syncthreads();  // read before thread 0 takes the next tile
    if (t >= total) break;
    const PrefillProblem& pr = probs[pi];
    const int local = (int)(t - pr.tile0), mt = (int)pr.mtiles;
    const int nb = local / mt, mb = local - nb * mt;
    p2_tile<XT, BITS, WGM, WGN>(pr.packed, pr.scales, pr.n, pr.k, pr.x, pr.m, pr.ldx, pr.y, pr.ldy, pr.yt,
                                (int64_t)mb * P2_BM, (int64_t)nb * P2_BN, smem);
  }
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(sync + PP_QUEUES, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
    for (int i = 0; i <= PP_QUEUES; ++i) __hip_atomic_store(sync + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

bool gemm_prefill2_supported(const GemmArgs& a) {
  if (a.group != 0 || a.m <= 64 || a.k % P2_BK != 0 || a.k == 0) return false;
  if (((uintptr_t)a.x & 15) || ((a.ldx * 2) & 15) || ((uintptr_t)a.packed & 15)) return false;
  return true;
}

#ifndef ZQ_P2_WGM
#define ZQ_P2_WGM 2
#define ZQ_P2_WGN 4
#endif

template <int XT, int BITS>
static hipError_t p2_launch(const GemmArgs& a) {
  constexpr int WGM = ZQ_P2_WGM, WGN = ZQ_P2_WGN;
  const void* fn = reinterpret_cast<const void*>(&gemm_prefill2_kernel<XT, BITS, WGM, WGN>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, P2_LDS);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.n + P2_BN - 1) / P2_BN), (unsigned)((a.m + P2_BM - 1) / P2_BM));
  hipLaunchKernelGGL((gemm_prefill2_kernel<XT, BITS, WGM, WGN>), grid, dim3(64 * WGM * WGN), P2_LDS, a.stream,
                     a.packed, a.scales, a.n, a.k, a.x, a.m, a.ldx, a.y, a.ldy, a.yt);
  return hipGetLastError();
}

bool prefill_plan_supported(const GemmArgs& a) { return a.zeros == nullptr && gemm_prefill2_supported(a); }

template <int XT, int BITS>
static hipError_t pp_launch(const PrefillProblem* dev_probs, int nprob, int64_t total, uint32_t* sync,
                            hipStream_t stream) {
  constexpr int WGM = ZQ_P2_WGM, WGN = ZQ_P2_WGN;
  const void* fn = reinterpret_cast<const void*>(&gemm_prefill_plan_kernel<XT, BITS, WGM, WGN>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, P2_LDS);
  if (e != hipSuccess) return e;
  const int64_t G = std::min<int64_t>(stream_grid(), total);
  hipLaunchKernelGGL((gemm_prefill_plan_kernel<XT, BITS, WGM, WGN>), dim3((unsigned)G), dim3(64 * WGM * WGN),
                     P2_LDS, stream, dev_probs, nprob, total, sync);
  return hipGetLastError();
}

hipError_t launch_prefill_plan(const PrefillProblem* dev_probs, int nprob, int64_t total, int xt, int bits,
                               uint32_t* sync, hipStream_t stream) {
  if (xt == XF16) {
    if (bits == 2) return pp_launch<XF16, 2>(dev_probs, nprob, total, sync, stream);
    if (bits == 4) return pp_launch<XF16, 4>(dev_probs, nprob, total, sync, stream);
    return pp_launch<XF16, 8>(dev_probs, nprob, total, sync, stream);
  }
  if (bits == 2) return pp_launch<XBF16, 2>(dev_probs, nprob, total, sync, stream);
  if (bits == 4) return pp_launch<XBF16, 4>(dev_probs, nprob, total, sync, stream);
  return pp_launch<XBF16, 8>(dev_probs, nprob, total, sync, stream);
}

hipError_t launch_gemm_prefill2(const GemmArgs& a) {
  if (a.xt == XF16) {
    if (a.bits == 2) return p2_launch<XF16, 2>(a);
    if (a.bits == 4) return p2_launch<XF16, 4>(a);
    return p2_launch<XF16, 8>(a);
  }
  if (a.bits == 2) return p2_launch<XBF16, 2>(a);
  if (a.bits == 4) return p2_launch<XBF16, 4>(a);
  return p2_launch<XBF16, 8>(a);
}

}  // namespace zq
