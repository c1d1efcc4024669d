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
//   * weights are loaded with buffer loads, one instruction covering 4 rows
//     x 256 contiguous bytes (16 lanes per row); in the MFMA layout one
//     instruction would cover 16 rows x 64 bytes, which streams ~25% slower
//     from HBM. The wave then moves each 16-row tile through a padded LDS
//     scratch so that lane (row n, slot g) holds the 16 bytes (32 codes) of
//     row n at byte 64*group + 16*g; those codes feed 4 MFMAs, 8 codes each,
//     in the decoder's pair order; activations are staged in LDS in that
//     same order, so A and B agree on k;
//   * codes become exact 16-bit values with a constant offset (a nibble
//     placed in a binary16/bfloat16 fraction); the offset's contribution,
//     BE * (sum of x at even k) + BO * (sum at odd k) per activation row and
//     group, is staged with the activations and enters the first MFMA of the
//     group as its C operand, negated, so the MFMA output is the group's
//     exact-input dot product;
//   * a workgroup of 16 waves owns a contiguous range of the segment's row
//     space; it walks it in blocks of up to 512 rows inside one product
//     (256 for asymmetric weights), each block in chunks of 512 k and each
//     chunk in 256-row halves; wave w takes 16-row tile w of each half.
//     The next item's weights are in flight while the current one is
//     computed; the next chunk's activations are loaded during a chunk's
//     last half and staged into the other of two LDS buffers;
//   * outputs of a half are stored when its last chunk is done.
#pragma once
#include "zq_stream_impl.hpp"

namespace zq {

// 16 waves per workgroup; wave w takes 16-row weight tile w of each
// 256-row half block, against one 16-row activation tile (M <= 16) or two
// (M = 17..32). With two, the activation fragments are read from LDS one
// tile at a time, so both tiles' accumulators fit 128 VGPRs. 16 waves
// streamed 11-23 % faster than 8 at M = 2..16 and 8-11 % faster at
// M = 17..32 (where 8 waves had held two weight tiles each).
template <int MT>
__host__ __device__ constexpr int ms_threads() { return 1024; }
// Weight tiles a wave takes in turn against the same staged activations: a
// block is 512 rows, walked as two 256-row halves per chunk, so the
// activations are staged (and re-read from L2) once per 512 rows instead of
// once per 256, with one workgroup barrier per chunk (M = 17..32: 5-6 %
// faster, M = 8..16: 2-3 %). Zero points need more registers: asymmetric
// weights keep 256-row blocks.
template <int MT, bool ASYM>
__host__ __device__ constexpr int ms_tp() { return ASYM ? 1 : 2; }
constexpr int MS_KC = 512;    // k per chunk (4 groups of 128)
constexpr int MS_HALF = 256;  // rows of one half of a block: 16 waves x 16 rows
static_assert(ms_threads<1>() / 64 * 16 == MS_HALF && ms_threads<2>() / 64 * 16 == MS_HALF,
              "one weight tile per wave and half");

// LDS bytes of one activation chunk buffer: A fragments [gs][mt][d][g][m][8]
// (16 bytes each; row m of fragment (d, g) at slot m ^ (4 d + g), so that a
// wave staging one activation row writes 16 different bank groups with 16
// consecutive lanes, while the 16 lanes of an MFMA read still cover one
// 256-byte run), the negated offset sums [gs][mt][m] (fp32) and, for
// asymmetric weights, the plain sums [gs][mt][m] (fp32).
__host__ __device__ constexpr int mstream_xbuf_bytes(int mt) { return mt * (4 * 4 * 4 * 16 * 16 + 2 * 4 * 16 * 4); }
// Weight transpose scratch of one wave: per tile, 4 loads x 4 rows x 16
// pieces of 16 bytes, each 16-piece row padded by 16 bytes (272 bytes) so
// that both the row-wise writes and the tile-column reads are conflict-free.
constexpr int MS_TROW = 272, MS_TLOAD = 4 * MS_TROW, MS_TTILE = 4 * MS_TLOAD;
constexpr int MS_WSCR_ALL = (MS_HALF / 16) * MS_TTILE;  // all waves' scratch of one workgroup

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
  // (BE, BO) and (1, 1) as 16-bit pairs of the activation type
  static constexpr uint32_t BW = XT == XF16 ? (ASYM ? 0x54006400u : 0x54806408u) : (ASYM ? 0x43004300u : 0x43084308u);
  static constexpr uint32_t ONE = XT == XF16 ? 0x3C003C00u : 0x3F803F80u;
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
// (<= 16 * MT); sync (non-null): a phase wait not performed yet by this
// workgroup. Returns false when the workgroup has no rows in the segment (it
// then read nothing and the wait stays pending for its next segment).
// COH: activations and outputs cross phases (agent-coherent accesses); a
// template parameter so the main loop has one fixed number of loads.
// ASYM: unsigned codes with a zero point per group (w = q * s + z): each
// group adds z * (sum of the group's activations) to every output of its row.
template <int XT, bool GROUPED, int MT, bool COH, bool ASYM = false>
__device__ __forceinline__ bool run_msegment(const StreamPhase& seg, const StreamProblem* probs,
                                             const StreamProblem& single, int2 wr, int m, uint8_t* smem,
                                             uint32_t* sync, uint32_t wait_target) {
  static_assert(!ASYM || GROUPED, "zero points come per 128-group");
  constexpr bool coherent = COH;
  using D = MDec<XT, ASYM>;
  constexpr int NT = ms_threads<MT>();
  constexpr int XB = mstream_xbuf_bytes(MT);
  constexpr int PPT = MT * 16 * 64 / NT;  // activation pieces (8 values) per thread per chunk
  constexpr int TP = ms_tp<MT, ASYM>();
  constexpr int BLOCK = TP * MS_HALF;  // rows per block

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
  if (r1 == r0) return false;  // uniform: no rows here, a pending wait stays pending
  const int nrec = wr.y - wr.x + 1;

  ProdRec* rec = reinterpret_cast<ProdRec*>(smem);
  uint8_t* xbuf = smem + (size_t)nrec * sizeof(ProdRec);
  uint8_t* wscr = xbuf + 2 * XB + wv * MS_TTILE;  // this wave's transpose scratch
  for (int i = tid; i < nrec; i += NT) {
    const StreamProblem& p = probs ? probs[seg.first + wr.x + i] : single;
    rec[i] = make_rec(p, rowbytes, GS, GROUPED);
  }
  __syncthreads();

  // ---- the workgroup's item sequence: blocks of <= BLOCK rows inside one
  // product, each in NC chunks of TP halves (h). Item state is
  // workgroup-uniform.
  struct Item {
    int32_t pi, b0, b1, c, h;
  };
  // record fields come from LDS: readfirstlane tells the compiler they are
  // the same in every lane, so the item state stays in scalar registers
  auto pend_of = [&](int i) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(rec[i].pend); };
  auto first_item = [&]() __attribute__((always_inline)) {
    Item it;
    it.pi = __builtin_amdgcn_readfirstlane(rec_of(rec, nrec, r0));
    it.b0 = r0;
    it.b1 = min(min(r0 + BLOCK, r1), pend_of(it.pi));
    it.c = 0;
    it.h = 0;
    return it;
  };
  auto valid = [&](const Item& it) __attribute__((always_inline)) { return it.b0 < r1; };
  auto next_item = [&](Item it) __attribute__((always_inline)) {
    if (++it.h < TP) return it;
    it.h = 0;
    if (++it.c < NC) return it;
    it.c = 0;
    it.b0 = it.b1;
    if (it.b0 >= pend_of(it.pi)) ++it.pi;
    it.b1 = it.b0 < r1 ? min(min(it.b0 + BLOCK, r1), pend_of(min(it.pi, nrec - 1))) : it.b0;
    return it;
  };

  // ---- fetch state of the item whose weights, scales and activations are
  // being loaded. Buffer loads: a descriptor per block (weights, scales, zero
  // points: the block's rows only) or per product (activations: m rows), a
  // scalar offset per item and a per-lane offset that is fixed for the
  // segment. Lane l of a weight load takes row 4 s + l/16 of the wave's tile
  // (slot s), bytes 16 (l % 16) of the chunk. Rows past the block's end and
  // activation rows past m lie outside their descriptor and read as zeros
  // (their outputs are never stored), so every load is unconditional and
  // the compiler counts them exactly.
  __amdgpu_buffer_rsrc_t f_w, f_s, f_z, f_x;
  int32_t f_wo, f_so, f_xo;  // scalar byte offsets of the item
  int32_t f_ldxb;  // activation row pitch in bytes
  const uint32_t wvo = (uint32_t)(lane >> 4) * (uint32_t)rowbytes + (uint32_t)(lane & 15) * 16;
  const uint32_t svo = (uint32_t)n16 * (uint32_t)(GS * 2);
  const uint32_t xvo = (uint32_t)lane * 16;
  // Descriptor words must sit in scalar registers: a descriptor held in
  // vector registers turns every load into a loop over lanes. Record fields
  // read from LDS are the same in every lane, which readfirstlane states.
  auto uni = [](const void* p) __attribute__((always_inline)) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  };
  auto rsrc = [&](const void* base, uint32_t bytes) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uni(base)), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
  };
  auto fetch_block = [&](const Item& it) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
    const uint32_t rows = (uint32_t)(it.b1 - it.b0);
    f_w = rsrc(uni(pr.wbase) + (int64_t)it.b0 * rowbytes, rows * (uint32_t)rowbytes);
    if constexpr (GROUPED) f_s = rsrc(uni(pr.sbase) + (int64_t)it.b0 * GS * 2, rows * (uint32_t)(GS * 2));
    if constexpr (ASYM) f_z = rsrc(uni(pr.zbase) + (int64_t)it.b0 * GS * 2, rows * (uint32_t)(GS * 2));
    f_ldxb = __builtin_amdgcn_readfirstlane((int32_t)pr.ldx * 2);
    f_x = rsrc(uni(pr.x), (uint32_t)m * (uint32_t)f_ldxb);
    f_wo = (it.h * MS_HALF + wv * 16) * (int32_t)rowbytes + it.c * 256;
    f_so = (it.h * MS_HALF + wv * 16) * GS * 2 + it.c * 8;
    f_xo = it.c * MS_KC * 2;
  };
  // move the fetch state from item `from` to the next item `to`
  auto fetch_advance = [&](const Item& from, const Item& to) __attribute__((always_inline)) {
    if (to.b0 != from.b0) {  // uniform: a new block
      fetch_block(to);
    } else if (to.c == from.c) {  // the next half of the same chunk
      f_wo += MS_HALF * (int32_t)rowbytes;
      f_so += MS_HALF * GS * 2;
    } else {  // the first half of the next chunk
      f_wo += 256 - (TP - 1) * MS_HALF * (int32_t)rowbytes;
      f_so += 8 - (TP - 1) * MS_HALF * GS * 2;
      f_xo += MS_KC * 2;
    }
  };
  constexpr int AUX_NT = 2, AUX_COH = 16;  // cache policy: nontemporal; agent-coherent (sc1)

  // ---- weight stream: 4 register slots per lane hold the next item's
  // weights (64 KB per workgroup); they are refilled as soon as the current
  // item's are moved to the wave's LDS scratch. One item ahead streamed
  // 0.4-1 % faster than two at M = 2..64, with ~40 fewer VGPRs.
  u4 slot[4];
  u2 sc = u2{0u, 0u}, zc = u2{0u, 0u};
  auto fetch_weights = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      slot[s4] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                            f_w, (int)wvo, f_wo + s4 * 4 * (int32_t)rowbytes, AUX_NT));
  };
  auto fetch_scales = [&]() __attribute__((always_inline)) {
    if constexpr (GROUPED) sc = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(f_s, (int)svo, f_so, 0));
    if constexpr (ASYM) zc = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(f_z, (int)svo, f_so, 0));
  };

  // ---- activations of one item: MT*16 rows x 512 k, PPT pieces per thread
  u4 xr[PPT];
  auto load_x = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int mm = i * (NT / 64) + wv;  // activation row of piece i (uniform)
      xr[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(f_x, (int)xvo, mm * f_ldxb + f_xo,
                                                                           coherent ? AUX_COH : 0));
    }
  };
  auto store_x = [&](uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = i * NT + tid;
      const int mm = p >> 6, k8 = p & 63;
      const int gs = k8 >> 4, gg = (k8 >> 2) & 3, d = k8 & 3, mt = mm >> 4, m16 = mm & 15;
      const uint32_t a0 = xr[i][0], a1 = xr[i][1], a2 = xr[i][2], a3 = xr[i][3];
      // natural order x0..x7 -> decoder pair order (0,4),(1,5),(2,6),(3,7)
      u4 piece;
      piece[0] = (a0 & 0xFFFFu) | (a2 << 16);
      piece[1] = (a0 >> 16) | (a2 & 0xFFFF0000u);
      piece[2] = (a1 & 0xFFFFu) | (a3 << 16);
      piece[3] = (a1 >> 16) | (a3 & 0xFFFF0000u);
      *reinterpret_cast<u4*>(buf + ((((gs * MT + mt) * 4 + d) * 4 + gg) * 16 + (m16 ^ (4 * d + gg))) * 16) = piece;
      // BE * (x at even k) + BO * (x at odd k), as dot products of pairs
      float corr = dot2<XT>(a0, D::BW, dot2<XT>(a1, D::BW, dot2<XT>(a2, D::BW, dot2<XT>(a3, D::BW, 0.f))));
      float sum = 0.f;
      if constexpr (ASYM)
        sum = dot2<XT>(a0, D::ONE, dot2<XT>(a1, D::ONE, dot2<XT>(a2, D::ONE, dot2<XT>(a3, D::ONE, 0.f))));
      // the 16 pieces of one (row, group) are the 16 lanes of a DPP row
      corr = row16_sum(corr);
      if constexpr (ASYM) sum = row16_sum(sum);
      if ((k8 & 15) == 0) {
        *reinterpret_cast<float*>(buf + MT * 16384 + ((gs * MT + mt) * 16 + m16) * 4) = -corr;
        if constexpr (ASYM) *reinterpret_cast<float*>(buf + MT * 16640 + ((gs * MT + mt) * 16 + m16) * 4) = sum;
      }
    }
  };

  f4 acc[TP][MT];
#pragma unroll
  for (int t = 0; t < TP; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f4{0.f, 0.f, 0.f, 0.f};

  auto epilogue = [&]<int T>(const Item& it) __attribute__((always_inline)) {
    const ProdRec& pr = rec[it.pi];
    const int32_t row = it.b0 + T * MS_HALF + wv * 16 + n16;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mm = mt * 16 + 4 * g + j;
        if (mm < m && row < it.b1)
          store_y_coherent(pr.y, (int64_t)mm * pr.ldy + (row - pr.roff), acc[T][mt][j] * pr.tscale, pr.yt,
                           coherent);
        acc[T][mt][j] = 0.f;
      }
    }
  };

  // One item (half T of a chunk of parity H): the chunk's activations are in
  // LDS buffer H, the item's weights in the slots and its scales in sc/zc;
  // the fetch state points at the next item (or at this one again when it
  // is the last). Moves this item's weights to the scratch and refills the
  // slots, computes; in a chunk's last half it also loads the next chunk's
  // activations, stages them into the other buffer and waits for the
  // workgroup (the only barrier of the chunk: each wave's scratch is its
  // own, and the activation buffers alternate by chunk).
  auto process = [&]<int H, int T>(const Item& it) __attribute__((always_inline)) {
    constexpr bool last_half = T == TP - 1;
    const uint8_t* buf = xbuf + H * XB;
    if constexpr (last_half) load_x();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      *reinterpret_cast<u4*>(wscr + s4 * MS_TLOAD + (lane >> 4) * MS_TROW + (lane & 15) * 16) = slot[s4];
    fetch_weights();
    __builtin_amdgcn_wave_barrier();
    const u2 scur = sc, zcur = zc;
    fetch_scales();
    const bool rows = it.b0 + T * MS_HALF + wv * 16 < it.b1;  // wave-uniform: the tile has rows
    // two activation tiles: waves in their MFMA section issue first (their
    // staging and loads at the default priority); M = 17..32 0.3-1.2 % faster, no
    // gain with one tile
    if constexpr (MT == 2) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int gs = 0; gs < 4; ++gs) {
      __builtin_amdgcn_sched_barrier(0);
      // row n16 of the tile, bytes 64 gs + 16 g: load n16/4, row n16%4, piece 4 gs + g
      const u4 wq = *reinterpret_cast<const u4*>(wscr + (n16 >> 2) * MS_TLOAD + (n16 & 3) * MS_TROW + (4 * gs + g) * 16);
      if (rows) {
        u4 bw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = D::decode(wq[d]);
        float s = 1.f, z = 0.f;
        if constexpr (GROUPED) {
          const uint32_t sw = scur[gs >> 1];
          s = f16_bits_to_float((uint16_t)((gs & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
        }
        if constexpr (ASYM) {
          const uint32_t zw = zcur[gs >> 1];
          z = f16_bits_to_float((uint16_t)((gs & 1) ? (zw >> 16) : (zw & 0xFFFFu)));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          u4 a[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            a[d] = *reinterpret_cast<const u4*>(buf + ((((gs * MT + mt) * 4 + d) * 4 + g) * 16 + (n16 ^ (4 * d + g))) * 16);
          f4 dd = *reinterpret_cast<const f4*>(buf + MT * 16384 + ((gs * MT + mt) * 16 + 4 * g) * 4);
          f4 xsum;
          if constexpr (ASYM) xsum = *reinterpret_cast<const f4*>(buf + MT * 16640 + ((gs * MT + mt) * 16 + 4 * g) * 4);
#pragma unroll
          for (int d = 0; d < 4; ++d) dd = ms_mfma<XT>(a[d], bw[d], dd);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (GROUPED) acc[T][mt][j] = __builtin_fmaf(s, dd[j], acc[T][mt][j]);
            else acc[T][mt][j] += dd[j];
            if constexpr (ASYM) acc[T][mt][j] = __builtin_fmaf(z, xsum[j], acc[T][mt][j]);
          }
        }
      }
    }
    if constexpr (MT == 2) __builtin_amdgcn_s_setprio(0);
    if (it.c == NC - 1) epilogue.template operator()<T>(it);
    if constexpr (last_half) {
      store_x(xbuf + (H ^ 1) * XB);
      __syncthreads();
    }
  };

  // ---- prologue: the first item's weights and scales (they do not depend
  // on earlier phases), then the phase wait, then the first activations
  Item cur = first_item();
  fetch_block(cur);
  fetch_weights();
  fetch_scales();
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
  load_x();
  store_x(xbuf);
  __syncthreads();

  // ---- main loop: two chunks (2 TP items) per trip so the buffer and half
  // indices are static; the fetch state moves to the next item before each
  // one is processed (past the last item it stays, and the loads repeat
  // valid addresses). Every block starts at half 0 of chunk 0 and has
  // NC * TP items, so the item at each position has that position's half.
  auto step = [&]<int H, int T>() __attribute__((always_inline)) {
    const Item nx = next_item(cur);
    const bool more = valid(nx);
    if (more) fetch_advance(cur, nx);
    process.template operator()<H, T>(cur);
    cur = nx;
    return more;
  };
  auto chunk = [&]<int H>() __attribute__((always_inline)) {
    bool more = true;
    [&]<int... T>(std::integer_sequence<int, T...>) __attribute__((always_inline)) {
      ((more = more && step.template operator()<H, T>()), ...);
    }(std::make_integer_sequence<int, TP>{});
    return more;
  };
  while (true) {
    if (!chunk.template operator()<0>()) break;
    if (!chunk.template operator()<1>()) break;
  }
  __syncthreads();  // LDS is reused by the next segment
  return true;
}

// variant = (x fp16 ? 0 : 3) + (asymmetric ? 2 : grouped ? 1 : 0); 6 = a mix
__host__ __device__ inline int mstream_variant(int xt, int group, int asym) {
  return (xt == XF16 ? 0 : 3) + (asym ? 2 : group ? 1 : 0);
}
constexpr int MVAR_ANY = 6;

template <int MT, int V>
__device__ __forceinline__ bool mrun_variant(const StreamPhase& seg, const StreamProblem* probs,
                                             const StreamProblem& single, int2 wr, int m, uint8_t* smem,
                                             uint32_t* sync, uint32_t wt, bool coh) {
  constexpr int XT = V < 3 ? XF16 : XBF16;
  constexpr bool ASYM = V % 3 == 2, GROUPED = V % 3 != 0;
  if (coh) return run_msegment<XT, GROUPED, MT, true, ASYM>(seg, probs, single, wr, m, smem, sync, wt);
  return run_msegment<XT, GROUPED, MT, false, ASYM>(seg, probs, single, wr, m, smem, sync, wt);
}

template <int MT, int VAR>
__device__ __forceinline__ bool mseg_dispatch(const StreamPhase& seg, const StreamProblem* probs,
                                              const StreamProblem& single, int2 wr, int m, uint8_t* smem,
                                              uint32_t* sync, uint32_t wt, bool coh) {
  if constexpr (VAR != MVAR_ANY) {
    return mrun_variant<MT, VAR>(seg, probs, single, wr, m, smem, sync, wt, coh);
  } else {
    switch (mstream_variant(seg.xt, seg.group, seg.asym)) {
      case 0: return mrun_variant<MT, 0>(seg, probs, single, wr, m, smem, sync, wt, coh);
      case 1: return mrun_variant<MT, 1>(seg, probs, single, wr, m, smem, sync, wt, coh);
      case 2: return mrun_variant<MT, 2>(seg, probs, single, wr, m, smem, sync, wt, coh);
      case 3: return mrun_variant<MT, 3>(seg, probs, single, wr, m, smem, sync, wt, coh);
      case 4: return mrun_variant<MT, 4>(seg, probs, single, wr, m, smem, sync, wt, coh);
      default: return mrun_variant<MT, 5>(seg, probs, single, wr, m, smem, sync, wt, coh);
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
  uint32_t* pending = nullptr;  // a phase wait not performed yet (see gemv_stream_kernel)
  for (int s = 0; s < nseg; ++s) {
    const StreamPhase seg = segs[s];
    if (seg.wait) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++waits;
      pending = sync;
    }
    const int2 wr = wranges[(int64_t)s * G + blockIdx.x];
    if (mseg_dispatch<MT, VAR>(seg, probs, single_prob, wr, m, smem, pending, waits * G, coh)) pending = nullptr;
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
