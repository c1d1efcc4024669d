// zq_mstream_impl.hpp -- persistent MFMA kernel for batched decode: 2..32
// activation rows against INT4 weights, for one product or a whole plan.
// Host launchers: zq_mstream.hip; instantiations: zq_mstream_t1.hip (16
// activation rows per MFMA tile) and zq_mstream_t2.hip (32).
//
// The ZSE wiki article ("ZSE - open-source движок для запуска LLM локально на
// GPU - 2026", sections "Честные ограничения" and "Перспективы") names
// concurrent INT4 decode of a few sequences as the engine's weak spot, and
// its section "Оркестратор и GPU-ядра" a wave-64 INT4 GEMV for single
// tokens. With 2..32 activation rows the weights are still streamed once
// (3.9 flop per weight byte per activation row, far below the MFMA/HBM
// balance of ~312), but a dot product per row on the vector ALU would cost
// more instructions than the memory time allows. Here the contraction runs on
// gfx950 MFMA (16x16x32, fp16 or bf16 inputs, fp32 accumulation):
//
//   * the activations are the A operand (16 activation rows per tile), the
//     decoded weight codes the B operand: MFMA output column n is weight row
//     n of the tile, so each lane multiplies by the group scale of the one
//     weight row it loaded;
//   * weights are loaded with one load instruction covering 4 rows x 256
//     contiguous bytes (16 lanes per row); in the MFMA layout one instruction
//     would cover 16 rows x 64 bytes, which streams ~25% slower from HBM. The
//     wave then moves each 16-row tile through a padded LDS scratch so that
//     lane (row n, slot g) holds the 16 bytes (32 codes) of row n at byte
//     64*group + 16*g; those codes feed 4 MFMAs, 8 codes each, in the
//     decoder's pair order; activations are staged in LDS in that same order,
//     so A and B agree on k;
//   * codes become exact 16-bit values with a constant offset (a nibble
//     placed in a binary16/bfloat16 fraction); the offset's contribution,
//     BE * (sum of x at even k) + BO * (sum at odd k) per activation row and
//     group, is staged with the activations and enters the first MFMA of the
//     group as its C operand, negated, so the MFMA output is the group's
//     exact-input dot product;
//   * a workgroup (16 waves for up to 16 activation rows, 8 for more) owns
//     a contiguous range of the segment's row space; it walks it in blocks
//     of up to 256 rows inside one product (wave w takes 16-row tile w, or
//     tiles w and w + 8 with 8 waves) and each block in chunks
//     of 512 k: activations of the next chunk are loaded into registers and
//     the weights of the next chunk are in flight while the current chunk is
//     computed; the activation buffers in LDS are double buffered;
//   * outputs of a block are stored when its last chunk is done.
#pragma once
#include "zq_stream_impl.hpp"

namespace zq {

// One 16-row activation tile (M <= 16): 16 waves with one 16-row weight
// tile each per block; two (M = 17..32): 8 waves with two each, since the
// second tile's accumulators and fragments do not fit 128 VGPRs. Both walk
// 256-row blocks and use the same transpose scratch. At M = 2..16 the 16
// waves streamed 11-23 % faster than 8.
template <int MT>
__host__ __device__ constexpr int ms_threads() { return MT == 1 ? 1024 : 512; }
template <int MT>
__host__ __device__ constexpr int ms_tw() { return MT == 1 ? 1 : 2; }  // 16-row tiles per wave per block
constexpr int MS_KC = 512;       // k per chunk (4 groups of 128)
constexpr int MS_BLOCK = 256;  // rows per block: waves x tiles per wave x 16
static_assert(ms_threads<1>() / 64 * ms_tw<1>() * 16 == MS_BLOCK && ms_threads<2>() / 64 * ms_tw<2>() * 16 == MS_BLOCK,
              "both tile counts walk the same blocks");
// items whose weights are in flight ahead of the one computed: 1 (64 KB per
// CU) streamed 0.4-1 % faster than 2 at M = 2..64, with ~40 fewer VGPRs
constexpr int MS_AHEAD = 1;

// LDS bytes of one activation chunk buffer: A fragments [gs][mt][d][g][m][8]
// (16 bytes each), the negated offset sums [gs][mt][m] (fp32) and, for
// asymmetric weights, the plain sums [gs][mt][m] (fp32).
__host__ __device__ constexpr int mstream_xbuf_bytes(int mt) { return mt * (4 * 4 * 4 * 16 * 16 + 2 * 4 * 16 * 4); }
// Weight transpose scratch of one wave: per tile, 4 loads x 4 rows x 16
// pieces of 16 bytes, each 16-piece row padded by 16 bytes (272 bytes) so
// that both the row-wise writes and the tile-column reads are conflict-free.
constexpr int MS_TROW = 272, MS_TLOAD = 4 * MS_TROW, MS_TTILE = 4 * MS_TLOAD;
constexpr int MS_WSCR_ALL = (MS_BLOCK / 16) * MS_TTILE;  // all waves' scratch of one workgroup

__host__ __device__ inline size_t mstream_lds_bytes(int mt, int nrec) {
  return (size_t)nrec * PROD_REC_BYTES + 2 * (size_t)mstream_xbuf_bytes(mt) + (size_t)MS_WSCR_ALL;
}

// INT4 decoder for the MFMA kernel: raw packed dword -> 4 dwords of packed
// 16-bit values, pair p holding codes (p, p + 4) as u + magic, u = q + 8 for
// signed codes (the sign flip folded into the mask: ((v ^ S) & M) | O ==
// (v & M) ^ ((S & M) ^ O)) and u = the code itself for unsigned
// (asymmetric) ones.
//  fp16: pairs 0, 2 as 1024 + u (nibble in fraction bits 3:0), pairs 1, 3 as
//        64 + u (nibble in bits 7:4, exponent 2^6); offsets 1032 / 72
//        (asymmetric 1024 / 64).
//  bf16: every pair as 128 + u (nibble in fraction bits 3:0); offset 136
//        (asymmetric 128).
template <int XT, bool ASYM = false>
struct MDec {
  static constexpr float FLIP = ASYM ? 0.f : 8.f;
  static constexpr float BE = (XT == XF16 ? 1024.f : 128.f) + FLIP;  // pairs of even k
  static constexpr float BO = (XT == XF16 ? 64.f : 128.f) + FLIP;    // pairs of odd k
  static constexpr uint32_t S0 = ASYM ? 0u : 0x00080008u, S1 = ASYM ? 0u : 0x00800080u;
  static __device__ __forceinline__ u4 decode(uint32_t v) {
    u4 r;
    if constexpr (XT == XF16) {
      const uint32_t t = v >> 8;
      r[0] = (v & 0x000F000Fu) ^ (S0 ^ 0x64006400u);
      r[1] = (v & 0x00F000F0u) ^ (S1 ^ 0x54005400u);
      r[2] = (t & 0x000F000Fu) ^ (S0 ^ 0x64006400u);
      r[3] = (t & 0x00F000F0u) ^ (S1 ^ 0x54005400u);
    } else {
      r[0] = (v & 0x000F000Fu) ^ (S0 ^ 0x43004300u);
      r[1] = ((v >> 4) & 0x000F000Fu) ^ (S0 ^ 0x43004300u);
      r[2] = ((v >> 8) & 0x000F000Fu) ^ (S0 ^ 0x43004300u);
      r[3] = ((v >> 12) & 0x000F000Fu) ^ (S0 ^ 0x43004300u);
    }
    return r;
  }
};

template <int XT>
__device__ __forceinline__ f4 ms_mfma(u4 a, u4 b, f4 c) {
  if constexpr (XT == XF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

// seg: segment; probs: problem table (nullptr: `single`); wr: {first, last}
// problem of the segment touched by this workgroup; m: activation rows
// (<= 16 * MT).
// COH: activations and outputs cross phases (agent-coherent accesses); a
// template parameter so the main loop has one fixed number of loads.
// ASYM: unsigned codes with a zero point per group (w = q * s + z): each
// group adds z * (sum of the group's activations) to every output of its row.
template <int XT, bool GROUPED, int MT, bool COH, bool ASYM = false>
__device__ __forceinline__ void run_msegment(const StreamPhase& seg, const StreamProblem* probs,
                                             const StreamProblem& single, int2 wr, int m, uint8_t* smem,
                                             uint32_t* sync, uint32_t wait_target) {
  static_assert(!ASYM || GROUPED, "zero points come per 128-group");
  constexpr bool coherent = COH;
  using D = MDec<XT, ASYM>;
  constexpr int NT = ms_threads<MT>();
  constexpr int NWV = NT / 64;  // waves
  constexpr int TW = ms_tw<MT>();
  constexpr int XB = mstream_xbuf_bytes(MT);
  constexpr int PPT = MT * 16 * 64 / NT;  // activation pieces (8 values) per thread per chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n16 = lane & 15;  // weight row within a tile / activation row of an A fragment
  const int g = lane >> 4;    // k slot of the lane in an MFMA
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x;
  const int64_t N = seg.n_total, k = seg.k;
  const int32_t NC = (int32_t)(k / MS_KC);  // chunks per row
  const int64_t rowbytes = k / 2;
  const int32_t GS = (int32_t)(k / 128);
  const int64_t w = blockIdx.x;
  const int32_t r0 = (int32_t)(w * N / G), r1 = (int32_t)((w + 1) * N / G);
  if (r1 == r0) return;  // uniform
  const int nrec = wr.y - wr.x + 1;

  ProdRec* rec = reinterpret_cast<ProdRec*>(smem);
  uint8_t* xbuf = smem + (size_t)nrec * sizeof(ProdRec);
  uint8_t* wscr = xbuf + 2 * XB + wv * TW * MS_TTILE;  // this wave's transpose scratch
  for (int i = tid; i < nrec; i += NT) {
    const StreamProblem& p = probs ? probs[seg.first + wr.x + i] : single;
    rec[i] = make_rec(p, rowbytes, GS, GROUPED);
  }
  __syncthreads();

  // ---- the workgroup's item sequence: blocks of <= 256 rows inside one
  // product, each in NC chunks. Item state is workgroup-uniform.
  struct Item {
    int32_t pi, b0, b1, c;
  };
  auto first_item = [&]() __attribute__((always_inline)) {
    Item it;
    it.pi = rec_of(rec, nrec, r0);
    it.b0 = r0;
    it.b1 = min(min(r0 + MS_BLOCK, r1), rec[it.pi].pend);
    it.c = 0;
    return it;
  };
  auto valid = [&](const Item& it) __attribute__((always_inline)) { return it.b0 < r1; };
  auto next_item = [&](Item it) __attribute__((always_inline)) {
    if (++it.c < NC) return it;
    it.c = 0;
    it.b0 = it.b1;
    if (it.b0 >= rec[it.pi].pend) ++it.pi;
    it.b1 = it.b0 < r1 ? min(min(it.b0 + MS_BLOCK, r1), rec[min(it.pi, nrec - 1)].pend) : it.b0;
    return it;
  };
  // the next item, or the same one past the end (a valid stand-in address)
  auto next_or_same = [&](const Item& it) __attribute__((always_inline)) {
    const Item nx = next_item(it);
    return valid(nx) ? nx : it;
  };

  // ---- weight stream: 4 register slots per lane, tile and item in flight,
  // for this wave's TW tiles; slot 4TWh + 4t + s holds rows 4s..4s+3 of tile
  // t of an item (of parity h when two are in flight; lane l: row 4s + l/16,
  // bytes 16*(l%16) of the chunk). Slots are refilled with the item MS_AHEAD
  // ahead as soon as they are moved to LDS.
  // Loads are unconditional (tiles past a block's end re-read its last row),
  // so the compiler counts them exactly.
  u4 slot[4 * TW * MS_AHEAD];
  u2 sc[TW * MS_AHEAD], zc[TW * MS_AHEAD];
  auto w_ptr = [&](const Item& it, int t, int s4) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
    const int32_t row = min(it.b0 + (wv + NWV * t) * 16 + 4 * s4 + (lane >> 4), it.b1 - 1);
    return reinterpret_cast<const u4*>(pr.wbase + (int64_t)row * rowbytes + (int64_t)it.c * 256) + (lane & 15);
  };
  auto s_ptr = [&](const Item& it, int t) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
    const int32_t row = min(it.b0 + (wv + NWV * t) * 16 + n16, it.b1 - 1);
    return reinterpret_cast<const u2*>(pr.sbase + (int64_t)row * GS + 4 * it.c);
  };
  auto z_ptr = [&](const Item& it, int t) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
    const int32_t row = min(it.b0 + (wv + NWV * t) * 16 + n16, it.b1 - 1);
    return reinterpret_cast<const u2*>(pr.zbase + (int64_t)row * GS + 4 * it.c);
  };

  // ---- activations of one item: MT*16 rows x 512 k, PPT pieces per thread
  u4 xr[PPT];
  auto load_x = [&](const Item& it) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = i * NT + tid;
      const int mm = p >> 6, k8 = p & 63;
      // rows past m re-read row 0 and are zeroed when stored
      xr[i] = load_x16(pr.x + (int64_t)(mm < m ? mm : 0) * pr.ldx + (int64_t)it.c * MS_KC + 8 * k8, coherent);
    }
  };
  auto store_x = [&](uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = i * NT + tid;
      const int mm = p >> 6, k8 = p & 63;
      const int gs = k8 >> 4, gg = (k8 >> 2) & 3, d = k8 & 3, mt = mm >> 4, m16 = mm & 15;
      const bool live = mm < m;
      const uint32_t a0 = live ? xr[i][0] : 0u, a1 = live ? xr[i][1] : 0u;
      const uint32_t a2 = live ? xr[i][2] : 0u, a3 = live ? xr[i][3] : 0u;
      // natural order x0..x7 -> decoder pair order (0,4),(1,5),(2,6),(3,7)
      u4 piece;
      piece[0] = (a0 & 0xFFFFu) | (a2 << 16);
      piece[1] = (a0 >> 16) | (a2 & 0xFFFF0000u);
      piece[2] = (a1 & 0xFFFFu) | (a3 << 16);
      piece[3] = (a1 >> 16) | (a3 & 0xFFFF0000u);
      *reinterpret_cast<u4*>(buf + ((((gs * MT + mt) * 4 + d) * 4 + gg) * 16 + m16) * 16) = piece;
      const float se = x_bits_to_float<XT>((uint16_t)(a0 & 0xFFFFu)) + x_bits_to_float<XT>((uint16_t)(a1 & 0xFFFFu)) +
                       x_bits_to_float<XT>((uint16_t)(a2 & 0xFFFFu)) + x_bits_to_float<XT>((uint16_t)(a3 & 0xFFFFu));
      const float so = x_bits_to_float<XT>((uint16_t)(a0 >> 16)) + x_bits_to_float<XT>((uint16_t)(a1 >> 16)) +
                       x_bits_to_float<XT>((uint16_t)(a2 >> 16)) + x_bits_to_float<XT>((uint16_t)(a3 >> 16));
      float corr = D::BE * se + D::BO * so;
      float sum = se + so;
      // the 16 pieces of one (row, group) are 16 aligned consecutive threads
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        corr += __shfl_xor(corr, o, 64);
        if constexpr (ASYM) sum += __shfl_xor(sum, o, 64);
      }
      if ((k8 & 15) == 0) {
        *reinterpret_cast<float*>(buf + MT * 16384 + ((gs * MT + mt) * 16 + m16) * 4) = -corr;
        if constexpr (ASYM) *reinterpret_cast<float*>(buf + MT * 16640 + ((gs * MT + mt) * 16 + m16) * 4) = sum;
      }
    }
  };

  f4 acc[TW][MT];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f4{0.f, 0.f, 0.f, 0.f};

  auto epilogue = [&](const Item& it) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int32_t row = it.b0 + (wv + NWV * t) * 16 + n16;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int mm = mt * 16 + 4 * g + j;
          if (mm < m && row < it.b1)
            store_y_coherent(pr.y, (int64_t)mm * pr.ldy + (row - pr.roff), acc[t][mt][j] * pr.tscale, pr.yt,
                             coherent);
          acc[t][mt][j] = 0.f;
        }
      }
    }
  };

  // One item of parity H: x for it is in LDS buffer H; the slots hold its
  // weights. Loads the next item's activations and refills the slots with
  // the item MS_AHEAD ahead (`nx`, or `pf2` two ahead), then stages the
  // activations and waits for the workgroup.
  auto process = [&]<int H>(const Item& it, const Item& nx, const Item& pf2) __attribute__((always_inline)) {
    const uint8_t* buf = xbuf + H * XB;
    constexpr int SB = MS_AHEAD == 2 ? 4 * TW * H : 0, CB2 = MS_AHEAD == 2 ? TW * H : 0;
    const Item& pf = MS_AHEAD == 2 ? pf2 : nx;
    load_x(nx);
    // this item's weights -> the wave's scratch; refill the slots at once
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        *reinterpret_cast<u4*>(wscr + t * MS_TTILE + s4 * MS_TLOAD + (lane >> 4) * MS_TROW + (lane & 15) * 16) =
            slot[SB + 4 * t + s4];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        slot[SB + 4 * t + s4] = __builtin_nontemporal_load(to_global(w_ptr(pf, t, s4)));
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int gs = 0; gs < 4; ++gs) {
      u4 a[MT][4];
      f4 cneg[MT], xsum[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
          a[mt][d] = *reinterpret_cast<const u4*>(buf + ((((gs * MT + mt) * 4 + d) * 4 + g) * 16 + n16) * 16);
        cneg[mt] = *reinterpret_cast<const f4*>(buf + MT * 16384 + ((gs * MT + mt) * 16 + 4 * g) * 4);
        if constexpr (ASYM)
          xsum[mt] = *reinterpret_cast<const f4*>(buf + MT * 16640 + ((gs * MT + mt) * 16 + 4 * g) * 4);
      }
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        // row n16 of the tile, bytes 64 gs + 16 g: load n16/4, row n16%4, piece 4 gs + g
        const u4 wq = *reinterpret_cast<const u4*>(wscr + t * MS_TTILE + (n16 >> 2) * MS_TLOAD +
                                                   (n16 & 3) * MS_TROW + (4 * gs + g) * 16);
        if (it.b0 + (wv + NWV * t) * 16 < it.b1) {  // wave-uniform: the tile has rows
          u4 bw[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) bw[d] = D::decode(wq[d]);
          float s = 1.f, z = 0.f;
          if constexpr (GROUPED) {
            const uint32_t sw = sc[CB2 + t][gs >> 1];
            s = f16_bits_to_float((uint16_t)((gs & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
          }
          if constexpr (ASYM) {
            const uint32_t zw = zc[CB2 + t][gs >> 1];
            z = f16_bits_to_float((uint16_t)((gs & 1) ? (zw >> 16) : (zw & 0xFFFFu)));
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            f4 dd = cneg[mt];
#pragma unroll
            for (int d = 0; d < 4; ++d) dd = ms_mfma<XT>(a[mt][d], bw[d], dd);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if constexpr (GROUPED) acc[t][mt][j] = __builtin_fmaf(s, dd[j], acc[t][mt][j]);
              else acc[t][mt][j] += dd[j];
              if constexpr (ASYM) acc[t][mt][j] = __builtin_fmaf(z, xsum[mt][j], acc[t][mt][j]);
            }
          }
        }
        if constexpr (GROUPED)
          if (gs == 3) sc[CB2 + t] = *to_global(s_ptr(pf, t));
        if constexpr (ASYM)
          if (gs == 3) zc[CB2 + t] = *to_global(z_ptr(pf, t));
      }
    }
    if (it.c == NC - 1) epilogue(it);
    store_x(xbuf + (H ^ 1) * XB);
    __syncthreads();  // also orders this wave's scratch reads before the next item's writes
  };

  // ---- prologue: the first MS_AHEAD items' weights (they do not depend on
  // earlier phases), then the phase wait, then the first activations
  Item cur = first_item();
  Item nx = next_or_same(cur);
#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      slot[4 * t + s4] = __builtin_nontemporal_load(to_global(w_ptr(cur, t, s4)));
      if constexpr (MS_AHEAD == 2) slot[(MS_AHEAD - 1) * 4 * TW + 4 * t + s4] = __builtin_nontemporal_load(to_global(w_ptr(nx, t, s4)));
    }
    if constexpr (GROUPED) {
      sc[t] = *to_global(s_ptr(cur, t));
      if constexpr (MS_AHEAD == 2) sc[(MS_AHEAD - 1) * TW + t] = *to_global(s_ptr(nx, t));
    }
    if constexpr (ASYM) {
      zc[t] = *to_global(z_ptr(cur, t));
      if constexpr (MS_AHEAD == 2) zc[(MS_AHEAD - 1) * TW + t] = *to_global(z_ptr(nx, t));
    }
  }
  if (sync) {
    if (tid == 0) {
      uint32_t polls = 0;
      while (__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < wait_target) {
        __builtin_amdgcn_s_sleep(1);
        if (++polls > (1u << 24)) {  // bounded: record the failure and go on
          __hip_atomic_fetch_or(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
  }
  load_x(cur);
  store_x(xbuf);
  __syncthreads();

  // ---- main loop: two items per trip so slot and buffer indices are static
  Item pf = next_or_same(nx);
  while (true) {
    nx = next_item(cur);
    process.template operator()<0>(cur, valid(nx) ? nx : cur, pf);
    if (!valid(nx)) break;
    cur = nx;
    pf = next_or_same(pf);
    nx = next_item(cur);
    process.template operator()<1>(cur, valid(nx) ? nx : cur, pf);
    if (!valid(nx)) break;
    cur = nx;
    pf = next_or_same(pf);
  }
  __syncthreads();  // LDS is reused by the next segment
}

// variant = (x fp16 ? 0 : 3) + (asymmetric ? 2 : grouped ? 1 : 0); 6 = a mix
__host__ __device__ inline int mstream_variant(int xt, int group, int asym) {
  return (xt == XF16 ? 0 : 3) + (asym ? 2 : group ? 1 : 0);
}
constexpr int MVAR_ANY = 6;

template <int MT, int V>
__device__ __forceinline__ void mrun_variant(const StreamPhase& seg, const StreamProblem* probs,
                                             const StreamProblem& single, int2 wr, int m, uint8_t* smem,
                                             uint32_t* sync, uint32_t wt, bool coh) {
  constexpr int XT = V < 3 ? XF16 : XBF16;
  constexpr bool ASYM = V % 3 == 2, GROUPED = V % 3 != 0;
  if (coh) run_msegment<XT, GROUPED, MT, true, ASYM>(seg, probs, single, wr, m, smem, sync, wt);
  else run_msegment<XT, GROUPED, MT, false, ASYM>(seg, probs, single, wr, m, smem, sync, wt);
}

template <int MT, int VAR>
__device__ __forceinline__ void mseg_dispatch(const StreamPhase& seg, const StreamProblem* probs,
                                              const StreamProblem& single, int2 wr, int m, uint8_t* smem,
                                              uint32_t* sync, uint32_t wt, bool coh) {
  if constexpr (VAR != MVAR_ANY) {
    mrun_variant<MT, VAR>(seg, probs, single, wr, m, smem, sync, wt, coh);
  } else {
    switch (mstream_variant(seg.xt, seg.group, seg.asym)) {
      case 0: mrun_variant<MT, 0>(seg, probs, single, wr, m, smem, sync, wt, coh); break;
      case 1: mrun_variant<MT, 1>(seg, probs, single, wr, m, smem, sync, wt, coh); break;
      case 2: mrun_variant<MT, 2>(seg, probs, single, wr, m, smem, sync, wt, coh); break;
      case 3: mrun_variant<MT, 3>(seg, probs, single, wr, m, smem, sync, wt, coh); break;
      case 4: mrun_variant<MT, 4>(seg, probs, single, wr, m, smem, sync, wt, coh); break;
      default: mrun_variant<MT, 5>(seg, probs, single, wr, m, smem, sync, wt, coh); break;
    }
  }
}

// Same launch contract as gemv_stream_kernel, plus the activation row count.
template <int MT, int VAR>
__global__ __launch_bounds__(ms_threads<MT>()) void gemm_mstream_kernel(
    const StreamPhase* __restrict__ segs, int nseg, const StreamProblem* __restrict__ probs,
    const int2* __restrict__ wranges, StreamPhase single_seg, StreamProblem single_prob, uint32_t* sync, int m) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t G = gridDim.x;
  if (!segs) {
    mseg_dispatch<MT, VAR>(single_seg, nullptr, single_prob, make_int2(0, 0), m, smem, nullptr, 0, false);
    return;
  }
  // data crosses phases only when some segment waits: only then do the
  // activations and outputs need agent-coherent (L2-bypassing) accesses
  bool coh = false;
  for (int s = 0; s < nseg; ++s) coh = coh || segs[s].wait;
  uint32_t waits = 0;
  for (int s = 0; s < nseg; ++s) {
    const StreamPhase seg = segs[s];
    uint32_t* ws = nullptr;
    if (seg.wait) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++waits;
      ws = sync;
    }
    const int2 wr = wranges[(int64_t)s * G + blockIdx.x];
    mseg_dispatch<MT, VAR>(seg, probs, single_prob, wr, m, smem, ws, waits * G, coh);
  }
  if (waits) {
    __syncthreads();
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1) {
      __hip_atomic_store(sync + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int MT>
static const void* mstream_fn_var(int var) {
  switch (var) {
    case 0: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, 0>);
    case 1: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, 1>);
    case 2: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, 2>);
    case 3: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, 3>);
    case 4: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, 4>);
    case 5: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, 5>);
    default: return reinterpret_cast<const void*>(&gemm_mstream_kernel<MT, MVAR_ANY>);
  }
}

const void* mstream_kernel_t1(int var);
const void* mstream_kernel_t2(int var);

}  // namespace zq
