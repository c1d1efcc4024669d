// zq_stream_impl.hpp -- persistent, load-balanced decode kernel (1..4
// activation rows) for one weight matrix or for a whole list of them in one
// launch. Host launchers: zq_stream.hip; instantiations: zq_stream_m1..m4.hip.
//
// Prior art: the wave-64 INT4 GEMV with 128-bit weight loads of the ZSE wiki
// article ("ZSE - open-source движок для запуска LLM локально на GPU - 2026",
// section "Оркестратор и GPU-ядра"), which also captures the decode launch
// sequence in a graph to cut launch cost. On gfx950 every launch and every
// dependent step costs microseconds, more than streaming a 7B k/v matrix, so
// this kernel stays resident (one workgroup per CU) and streams a list of
// products as a few long segments.
//
// A segment is a run of products that share K, code width, scale layout and
// activation type; their rows are concatenated into one row space and
// workgroup w streams rows [w*N/G, (w+1)*N/G) of it -- one contiguous range
// that may cover several products. A segment may have to wait until every
// workgroup has stored the outputs of the segments before it (a device-wide
// counter), so outputs of one phase can feed the next; data that crosses such
// a wait is stored and loaded with agent-coherent (sc1) accesses, and the
// counter is a relaxed agent atomic after an s_waitcnt: an agent-scope
// release/acquire fence writes back or invalidates the XCD's whole L2.
//
// Inside a workgroup's range:
//   * the products it touches are described by records in LDS; the
//     activations of each are staged in LDS in decoder order (see Decoder)
//     with two sums per 128-wide group of k (even and odd k) that remove the
//     decoder's constant offsets (applied by the group's first lane);
//   * its 16-lane groups each get an equal, contiguous run of 16-chunk steps
//     (a step = 256 contiguous bytes of one row), so work is balanced to one
//     chunk per lane whatever the shapes;
//   * every lane keeps ST_U chunks (and their group scales) in flight; loads
//     are issued unconditionally -- past its run a lane re-reads a cached
//     chunk and discards it -- so the compiler waits for exactly one load
//     per step, and the main loop has a workgroup-uniform trip count;
//   * a group reduces its 16 lane partials with four DPP steps whenever its
//     run leaves a row: a row that lies inside the run is stored at once; a
//     row split between runs leaves a tail partial and head partials that are
//     summed in group order after the loop, so results are run-to-run
//     identical.
#pragma once
#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace zq {

// chunks in flight per lane: 4 (64 KB per CU at 1024 threads) streamed the
// 7B, 32B and tensor-parallel stacks 2-5 % faster than 8; 2 and 3 were no
// better than 4
constexpr int ST_U = 4;
// 1024 threads (16 waves, 128 VGPRs) for one activation row; 512 threads
// (256 VGPRs) when each lane keeps 2..4 rows of partials.
template <int MR>
constexpr int st_threads() { return MR == 1 ? 1024 : 512; }

// Fast decoder for the stream kernel.
//  fp16 INT4: pairs (0,4),(2,6) put the nibble in the fraction's low bits
//    (value 1024 + u), pairs (1,5),(3,7) in bits 7:4 (value 64 + u); one shift
//    by 8 serves the upper two pairs. u = q + 8. Offsets: even k 1032, odd 72.
//  fp16 INT8: bytes in the fraction's low 8 bits: value 1024 + u, u = q + 128.
//  bf16 INT4: every pair's nibbles in the fraction's low 4 bits (value
//    128 + u, u = q + 8) after shifts by 0, 4, 8 and 12; offset 136 for all k.
//  everything else: the generic Decoder (one offset for all k).
// ASYM: unsigned codes (u = code, no sign flip), so every offset is smaller
// by 2^(BITS-1): fp16 INT4 1024 / 64, generic 2^BITS.
template <int XT, int BITS, bool ASYM = false>
struct FastDec {
  static constexpr float SYM_BE = (XT == XF16 && BITS == 4)    ? 1032.f
                                  : (XT == XF16 && BITS == 8)  ? 1152.f
                                  : (XT == XBF16 && BITS == 4) ? 136.f
                                                               : Decoder<XT, BITS>::BIAS;
  static constexpr float SYM_BO = (XT == XF16 && BITS == 4) ? 72.f : SYM_BE;
  static constexpr float BE = ASYM ? SYM_BE - (float)(1 << (BITS - 1)) : SYM_BE;
  static constexpr float BO = ASYM ? SYM_BO - (float)(1 << (BITS - 1)) : SYM_BO;
  static constexpr uint32_t FLIP4 = ASYM ? 0u : 0x00080008u;  // sign flip of the low-nibble pairs
  static constexpr uint32_t FLIP4H = ASYM ? 0u : 0x00800080u;  // ... of the high-nibble pairs
  static constexpr uint32_t FLIP8 = ASYM ? 0u : 0x00800080u;
  // dot of one raw packed dword (codes not yet sign-flipped) with its
  // activation pairs. The sign flip is folded into the masking:
  // ((v ^ S) & M) | O == (v & M) ^ ((S & M) ^ O), one v_bitop3 per pair.
  static __device__ __forceinline__ float dot(uint32_t v, const uint32_t* xq, float d) {
    if constexpr (XT == XF16 && BITS == 4) {
      const uint32_t t = v >> 8;
      d = dot2<XF16>((v & 0x000F000Fu) ^ (FLIP4 ^ 0x64006400u), xq[0], d);
      d = dot2<XF16>((v & 0x00F000F0u) ^ (FLIP4H ^ 0x54005400u), xq[1], d);
      d = dot2<XF16>((t & 0x000F000Fu) ^ (FLIP4 ^ 0x64006400u), xq[2], d);
      d = dot2<XF16>((t & 0x00F000F0u) ^ (FLIP4H ^ 0x54005400u), xq[3], d);
      return d;
    } else if constexpr (XT == XBF16 && BITS == 4) {
      d = dot2<XBF16>((v & 0x000F000Fu) ^ (FLIP4 ^ 0x43004300u), xq[0], d);
      d = dot2<XBF16>(((v >> 4) & 0x000F000Fu) ^ (FLIP4 ^ 0x43004300u), xq[1], d);
      d = dot2<XBF16>(((v >> 8) & 0x000F000Fu) ^ (FLIP4 ^ 0x43004300u), xq[2], d);
      d = dot2<XBF16>(((v >> 12) & 0x000F000Fu) ^ (FLIP4 ^ 0x43004300u), xq[3], d);
      return d;
    } else if constexpr (XT == XF16 && BITS == 8) {
      d = dot2<XF16>((v & 0x00FF00FFu) ^ (FLIP8 ^ 0x64006400u), xq[0], d);
      d = dot2<XF16>(((v >> 8) & 0x00FF00FFu) ^ (FLIP8 ^ 0x64006400u), xq[1], d);
      return d;
    } else {
      using D = Decoder<XT, BITS>;
      if constexpr (!ASYM) v ^= Codes<BITS>::SIGNS;
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((d = dot2<XT>(D::template pair<I>(v), xq[I], d)), ...);
      }(std::make_integer_sequence<int, Codes<BITS>::PAIRS>{});
      return d;
    }
  }
};

// One product as the workgroup sees it (LDS record, 80 bytes).
struct ProdRec {
  const uint8_t* wbase;   // packed - roff * rowbytes: index by segment row
  const uint16_t* sbase;  // grouped: scales - roff * (k/128); per tensor: unused
  const uint16_t* zbase;  // asymmetric: zeros - roff * (k/128); else unused
  const uint16_t* x;
  void* y;
  int64_t ldx, ldy;
  int32_t roff, pend;     // rows [roff, pend) of the segment row space
  int32_t yt;
  float tscale;           // per-tensor scale (1 when grouped)
  int64_t pad;
};
constexpr int PROD_REC_BYTES = 80;
static_assert(sizeof(ProdRec) == PROD_REC_BYTES, "LDS record layout");

// Activation block of one 16-chunk step: for each row m, PC rows of 16
// 16-byte pieces, then the (even, odd) sums of the step's 128-wide groups.
__host__ __device__ inline size_t stream_block_bytes(int bits, int64_t mr) {
  const int64_t wpc = 128 / bits, pc = wpc / 8, ng = 16 * wpc / 128;
  return (size_t)(mr * pc * 256 + mr * ng * 8);
}

// LDS bytes of one workgroup's view of a segment touching nrec products
__host__ __device__ inline size_t stream_seg_lds(int bits, int64_t mr, int64_t k, int nrec) {
  const int64_t C = k / (128 / bits);
  const int nw = mr == 1 ? 16 : 8;  // waves
  return (size_t)nrec * PROD_REC_BYTES + (size_t)nrec * ((C + 15) / 16) * stream_block_bytes(bits, mr) +
         (size_t)nw * (8 + 32 * mr);
}

// 16 bytes of activations, optionally with agent-coherent loads (the buffer
// may have been written by another workgroup before the phase wait).
__device__ __forceinline__ u4 load_x16(const uint16_t* p, bool coherent) {
  if (!coherent) return *to_global(reinterpret_cast<const u4*>(p));
  gptr<const uint32_t> q = to_global(reinterpret_cast<const uint32_t*>(p));
  u4 r;
  r[0] = __hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r[1] = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r[2] = __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r[3] = __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return r;
}
__device__ __forceinline__ uint16_t load_x2(const uint16_t* p, bool coherent) {
  if (!coherent) return *to_global(p);
  return __hip_atomic_load(to_global(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_y_coherent(void* y, int64_t idx, float v, int yt, bool coherent) {
  if (yt == YF32) {
    gptr<float> d = to_global(reinterpret_cast<float*>(y)) + idx;
    if (coherent) __hip_atomic_store(d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *d = v;
  } else {
    const uint16_t h = yt == YF16 ? float_to_f16_bits(v) : float_to_bf16_bits(v);
    gptr<uint16_t> d = to_global(reinterpret_cast<uint16_t*>(y)) + idx;
    if (coherent) __hip_atomic_store(d, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *d = h;
  }
}

// Record of product p for a segment (device table entry or the single product).
__device__ __forceinline__ ProdRec make_rec(const StreamProblem& p, int64_t rowbytes, int64_t GS, bool grouped) {
  ProdRec r;
  r.wbase = p.packed - p.row_off * rowbytes;
  r.sbase = p.scales - (grouped ? p.row_off * GS : 0);
  r.zbase = p.zeros ? p.zeros - p.row_off * GS : nullptr;
  r.x = p.x;
  r.y = p.y;
  r.ldx = p.ldx;
  r.ldy = p.ldy;
  r.roff = (int32_t)p.row_off;
  r.pend = (int32_t)(p.row_off + p.n);
  r.yt = p.yt;
  r.tscale = grouped ? 1.f : f16_bits_to_float(*to_global(p.scales));
  return r;
}

// Record index (0..nrec-1) owning a segment row: last record with roff <= row.
__device__ __forceinline__ int rec_of(const ProdRec* rec, int nrec, int32_t row) {
  int i = 0;
  for (int t = 1; t < nrec; ++t) i = rec[t].roff <= row ? t : i;
  return i;
}

// seg: segment description; probs: the problem table (nullptr: `single`);
// wr: {first, last} problem (within the segment) touched by this workgroup;
// sync (non-null): a phase wait this workgroup has not performed yet, done
// before its first activation load. Returns false when the workgroup has no
// rows in the segment: it then read nothing, and a pending wait stays pending
// for its next segment.
//
// Work split inside the workgroup: rows [r0, r1) form quads of 4 rows; a
// quad-step is one 16-chunk column block of a quad (4 x 256 contiguous-row
// bytes). Each wave takes an equal, contiguous run of quad-steps (quad-major),
// its 16-lane group q4 handling row 4*quad + q4, so all four groups of a wave
// cross row ends together: every branch of the main loop is wave-uniform.
template <int XT, int BITS, bool GROUPED, int MR, bool ASYM = false>
__device__ __forceinline__ bool run_segment(const StreamPhase& seg, const StreamProblem* probs,
                                            const StreamProblem& single, int2 wr, uint8_t* smem,
                                            uint32_t* sync, uint32_t wait_target, bool coherent) {
  using CD = Codes<BITS>;
  using FD = FastDec<XT, BITS, ASYM>;
  static_assert(!ASYM || GROUPED, "zero points come per 128-group");
  constexpr int NT = st_threads<MR>();
  constexpr int NW = NT / 64;      // waves
  constexpr int WPC = 128 / BITS;  // weights per 16-byte chunk
  constexpr int PC = WPC / 8;      // activation pieces per chunk
  constexpr int CPG = 128 / WPC;   // chunks per 128-group
  constexpr int SPS = 16 / CPG;    // scale entries per step
  constexpr int U = ST_U;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane & 15;
  const int q4 = lane >> 4;
  // wave index as a scalar: the run bookkeeping below is wave-uniform and
  // then lives in SGPRs with scalar branches
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the segment's rows are split over its own number of workgroups (the
  // launch may have more, for larger segments): the same split as a single
  // call on the segment alone
  const int G = seg.grid > 0 && seg.grid < (int)gridDim.x ? seg.grid : (int)gridDim.x;
  const int64_t N = seg.n_total, k = seg.k;
  const int32_t C = (int32_t)(k / WPC);
  const int32_t CB = (C + 15) / 16;     // column blocks (steps) per row
  const int32_t CT = C - (CB - 1) * 16;  // chunks in a row's last step (1..16)
  const int32_t CP = CB * 16;            // chunks per row with the last step padded
  const int64_t rowbytes = (int64_t)C * 16;
  const int32_t GS = (int32_t)(k / 128);
  const int64_t w = blockIdx.x;
  if (w >= G) return false;  // uniform: the segment's rows go to fewer workgroups
  const int32_t r0 = (int32_t)(w * N / G), r1 = (int32_t)((w + 1) * N / G);
  const int32_t R = r1 - r0;
  if (R == 0) return false;  // uniform: this workgroup has no rows in the segment
  const int nrec = wr.y - wr.x + 1;

  // ---- LDS layout
  ProdRec* rec = reinterpret_cast<ProdRec*>(smem);
  // activation slot of one product: blocks of 16 chunks (one step); block b
  // holds, for each row m, PC rows of 16 pieces (piece t of chunk 16b+jj at
  // (m*PC + t)*256 + jj*16), then for each row m the NG (even, odd) sums of
  // the block's groups at MR*PC*256 + (m*NG + g)*8
  constexpr int NG = 16 / CPG;                     // groups per block
  constexpr int BS = MR * PC * 256 + MR * NG * 8;  // bytes per block
  const size_t slot_bytes = (size_t)CB * BS;
  uint8_t* xbase = smem + (size_t)nrec * sizeof(ProdRec);
  int32_t* head_q = reinterpret_cast<int32_t*>(xbase + nrec * slot_bytes);  // [NW] quad of the head
  int32_t* tail_q = head_q + NW;                                           // [NW]
  float* head_val = reinterpret_cast<float*>(tail_q + NW);                 // [NW][4][MR]
  float* tail_val = head_val + NW * 4 * MR;                                // [NW][4][MR]

  // ---- product records of this workgroup's range
  for (int i = tid; i < nrec; i += NT) {
    const StreamProblem& p = probs ? probs[seg.first + wr.x + i] : single;
    rec[i] = make_rec(p, rowbytes, GS, GROUPED);
  }
  if (tid < NW) {
    head_q[tid] = -1;
    tail_q[tid] = -1;
  }
  __syncthreads();

  // this wave's run of quad-steps
  const int32_t NQ = (R + 3) / 4;
  const int64_t T = (int64_t)NQ * CB;
  const int64_t s0 = (int64_t)wv * T / NW, s1 = (int64_t)(wv + 1) * T / NW;
  const int64_t nsteps = (T + NW - 1) / NW;  // uniform trip count (runs differ by at most 1)

  // row of this lane in quad qd (rows past the range re-read the last row)
  auto quad_row = [&](int32_t qd) __attribute__((always_inline)) -> int32_t {
    const int32_t rr = r0 + 4 * qd + q4;
    return rr < r1 ? rr : r1 - 1;
  };
  auto rec_at = [&](int32_t row) __attribute__((always_inline)) -> int {
    return rec_of(rec, nrec, row);
  };

  // ---- producer: weight chunks (and group scales) of the run, ST_U ahead.
  // Within a quad row the lane's pointers advance by one step (256 bytes,
  // 16/CPG scales); at a block wrap they move to the lane's row of the next
  // quad. At the end of its run a wave keeps re-reading its last chunks
  // (cached); the consumer discards those. When a row's last step is partial
  // (C % 16 != 0), its lanes past the row's end re-read the row's last chunk
  // (and its group's scale): their activations are staged as zeros.
  const int32_t tdel = j >= CT ? CT - 1 - j : 0;                // u4 units
  const int32_t sdel = j >= CT ? (CT - 1) / CPG - j / CPG : 0;  // scale units
  const int64_t tdel_b = (int64_t)tdel * 16, sdel_b = (int64_t)sdel * 2;  // bytes
  const bool ragged = CT != 16;
  int32_t lq = (int32_t)(s0 / CB), lb = (int32_t)(s0 % CB);
  if (s1 == s0) { lq = 0; lb = 0; }  // empty run: a valid stand-in address
  int32_t lrow = quad_row(lq);
  int lpi = rec_at(lrow);
  const bool last0 = lb == CB - 1;
  const u4* lptr =
      reinterpret_cast<const u4*>(rec[lpi].wbase + (int64_t)lrow * rowbytes) + lb * 16 + j + (last0 ? tdel : 0);
  const uint16_t* lsp =
      GROUPED ? rec[lpi].sbase + (int64_t)lrow * GS + lb * SPS + j / CPG + (last0 ? sdel : 0) : nullptr;
  // zero points sit at the same index in their own [n][k/128] array
  auto zdiff = [&](int pi_) __attribute__((always_inline)) -> int64_t {
    return ((int64_t)(uintptr_t)rec[pi_].zbase - (int64_t)(uintptr_t)rec[pi_].sbase) / 2;
  };
  int64_t zoff = ASYM ? zdiff(lpi) : 0;
  int32_t lleft = (int32_t)(s1 - s0);  // quad-steps not yet requested
  auto next_chunk = [&](u4& wvv, uint16_t& sv, uint16_t& zv) __attribute__((always_inline)) {
    wvv = __builtin_nontemporal_load(to_global(lptr));
    if constexpr (GROUPED) sv = *to_global(lsp);
    if constexpr (ASYM) zv = *to_global(lsp + zoff);
    if (lleft > 1) {  // wave-uniform
      --lleft;
      if (++lb == CB) {
        lb = 0;
        ++lq;
        lrow = quad_row(lq);
        while (lrow >= rec[lpi].pend) ++lpi;
        lptr = reinterpret_cast<const u4*>(rec[lpi].wbase + (int64_t)lrow * rowbytes) + j + (CB == 1 ? tdel : 0);
        if constexpr (GROUPED) lsp = rec[lpi].sbase + (int64_t)lrow * GS + j / CPG + (CB == 1 ? sdel : 0);
        if constexpr (ASYM) zoff = zdiff(lpi);
      } else {
        lptr += 16;
        if constexpr (GROUPED) lsp += SPS;
        if (ragged && lb == CB - 1) {  // wave-uniform: the row's partial last step
          // an empty volatile asm keeps this a scalar branch: folded into
          // per-step selects, the rare adjustment costs six VALU ops a step
          __asm__ volatile("");
          lptr = reinterpret_cast<const u4*>(reinterpret_cast<const uint8_t*>(lptr) + tdel_b);
          if constexpr (GROUPED)
            lsp = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(lsp) + sdel_b);
        }
      }
    } else {
      lleft = 0;
    }
  };

  // ---- activation staging: piece idx -> (record, m, chunk, piece), over
  // the padded row (CP chunks); pieces of chunks c >= C are zeros
  constexpr int XR = MR == 1 ? 1 : 4;  // pieces per thread per round
  const int64_t per_slot = (int64_t)MR * CP * PC;
  const int64_t P = nrec * per_slot;
  auto piece_of = [&](int64_t idx, int& slot, int& m, int64_t& c, int& t) __attribute__((always_inline)) {
    slot = (int)(idx / per_slot);
    int64_t rem = idx - (int64_t)slot * per_slot;
    m = (int)(rem / ((int64_t)CP * PC));
    rem -= (int64_t)m * CP * PC;
    c = rem / PC;
    t = (int)(rem - c * PC);
  };
  u4 xraw[XR];
  auto load_x_round = [&](int64_t it0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      int64_t idx = (it0 + i) * NT + tid;
      idx = idx < P ? idx : 0;
      int slot, m, t;
      int64_t c;
      piece_of(idx, slot, m, c, t);
      if (c >= C) c = 0;  // padding: a valid address, zeroed when stored
      const uint16_t* xr = rec[slot].x + (int64_t)m * rec[slot].ldx + c * WPC;
      if constexpr (BITS == 4 || BITS == 8) {
        xraw[i] = load_x16(xr + 8 * t, coherent);
      } else {
        // INT2: the piece's 8 activations are spread over 16 consecutive ones
        uint16_t v[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const int pp = 8 * t + h, q = pp % CD::E, e = q / 2 + (q % 2) * (CD::E / 2);
          v[h] = load_x2(xr + (pp / CD::E) * CD::E + e, coherent);
        }
        xraw[i][0] = v[0] | ((uint32_t)v[1] << 16);
        xraw[i][1] = v[2] | ((uint32_t)v[3] << 16);
        xraw[i][2] = v[4] | ((uint32_t)v[5] << 16);
        xraw[i][3] = v[6] | ((uint32_t)v[7] << 16);
      }
    }
  };
  auto store_x_round = [&](int64_t it0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      if ((it0 + i) * NT >= P) break;  // uniform: no live piece in this or later rounds
      const int64_t idx = (it0 + i) * NT + tid;
      const bool live = idx < P;
      int slot, m, t;
      int64_t c;
      piece_of(live ? idx : 0, slot, m, c, t);
      const bool pad = c >= C;
      const uint32_t a0 = pad ? 0u : xraw[i][0], a1 = pad ? 0u : xraw[i][1];
      const uint32_t a2 = pad ? 0u : xraw[i][2], a3 = pad ? 0u : xraw[i][3];
      uint16_t v[8];
      if constexpr (BITS == 4) {  // decoder order (0,4,1,5,2,6,3,7)
        v[0] = a0 & 0xFFFF; v[1] = a2 & 0xFFFF; v[2] = a0 >> 16; v[3] = a2 >> 16;
        v[4] = a1 & 0xFFFF; v[5] = a3 & 0xFFFF; v[6] = a1 >> 16; v[7] = a3 >> 16;
      } else if constexpr (BITS == 8) {  // decoder order (0,2,1,3,4,6,5,7)
        v[0] = a0 & 0xFFFF; v[1] = a1 & 0xFFFF; v[2] = a0 >> 16; v[3] = a1 >> 16;
        v[4] = a2 & 0xFFFF; v[5] = a3 & 0xFFFF; v[6] = a2 >> 16; v[7] = a3 >> 16;
      } else {  // already gathered in decoder order
        v[0] = a0 & 0xFFFF; v[1] = a0 >> 16; v[2] = a1 & 0xFFFF; v[3] = a1 >> 16;
        v[4] = a2 & 0xFFFF; v[5] = a2 >> 16; v[6] = a3 & 0xFFFF; v[7] = a3 >> 16;
      }
      float se = 0.f, so = 0.f;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const int pp = 8 * t + h, q = pp % CD::E, e = q / 2 + (q % 2) * (CD::E / 2);
        const int kk = (pp / CD::E) * CD::E + e;
        const float f = x_bits_to_float<XT>(v[h]);
        if (kk & 1) so += f;
        else se += f;
      }
      uint8_t* blk = xbase + slot * slot_bytes + (size_t)(c / 16) * BS + (c % 16) * 16;
      if (live) {
        u4 piece;
        piece[0] = v[0] | ((uint32_t)v[1] << 16);
        piece[1] = v[2] | ((uint32_t)v[3] << 16);
        piece[2] = v[4] | ((uint32_t)v[5] << 16);
        piece[3] = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<u4*>(blk + (m * PC + t) * 256) = piece;
      }
      // the 16 pieces of a 128-group are 16 consecutive, 16-aligned piece
      // indices (k/8 is a multiple of 16), hence 16 aligned lanes, all live
      // or all not
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        se += __shfl_xor(se, o, 64);
        so += __shfl_xor(so, o, 64);
      }
      if (live && ((c % CPG) * PC + t) == 0) {
        uint8_t* sums = xbase + slot * slot_bytes + (size_t)(c / 16) * BS + MR * PC * 256;
        *reinterpret_cast<f2*>(sums + (m * NG + (c % 16) / CPG) * 8) = f2{se, so};
      }
    }
  };

  // ---- prologue: activations (after the dependency wait when there is one)
  // go out before most of the weights, so they are not queued behind them
  constexpr int U0 = 2;
  u4 buf[U];
  uint16_t sbuf[U], zbuf[U];
  if (!sync) load_x_round(0);
#pragma unroll
  for (int u = 0; u < U0; ++u) next_chunk(buf[u], sbuf[u], zbuf[u]);
  if (sync) {
    // weights and scales do not depend on earlier phases: the whole window
    // goes out before the wait, so it streams while the earlier phase ends
#pragma unroll
    for (int u = U0; u < U; ++u) next_chunk(buf[u], sbuf[u], zbuf[u]);
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
    load_x_round(0);
    store_x_round(0);
  } else {
    store_x_round(0);
#pragma unroll
    for (int u = U0; u < U; ++u) next_chunk(buf[u], sbuf[u], zbuf[u]);
  }
  for (int64_t it0 = XR; it0 * NT < P; it0 += XR) {
    load_x_round(it0);
    store_x_round(it0);
  }
  __syncthreads();

  // ---- consumer
  int32_t cq = (int32_t)(s0 / CB), cb = (int32_t)(s0 % CB);
  int32_t row = quad_row(cq);
  bool row_ok = r0 + 4 * cq + q4 < r1;
  int pi = rec_at(row);
  const uint8_t* slot0 = xbase + pi * slot_bytes + j * 16;  // block 0 of this product, lane j
  const uint8_t* xp8 = slot0 + (size_t)cb * BS;            // block of the current step
  bool split_head = cb != 0;  // the run starts inside a quad
  // the first lane of each group removes the group's decoder offsets
  const int sdelta = MR * PC * 256 + (j / CPG) * 8 - j * 16;  // sums of lane j's group, from xp8
  const bool gfirst = j % CPG == 0;
  const float fe = gfirst ? FD::BE : 0.f, fo = gfirst ? FD::BO : 0.f;
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;

  for (int64_t sb = 0; sb < nsteps; sb += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u4 wq = buf[u];
      const uint16_t sv = sbuf[u];
      const uint16_t zv = zbuf[u];
      next_chunk(buf[u], sbuf[u], zbuf[u]);  // the chunk U steps ahead (or the stand-in)
      if (s0 + sb + u < s1) {       // wave-uniform
        float sc = 1.f, zs = 0.f;
        if constexpr (GROUPED) sc = f16_bits_to_float(sv);
        // zero point term z * (sum of the group's x), added by the group's first lane
        if constexpr (ASYM) zs = gfirst ? f16_bits_to_float(zv) : 0.f;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          // activation pairs of dword dw are pairs [dw*PAIRS, (dw+1)*PAIRS) of
          // the chunk's pieces; read each 16-byte piece just before first use
          uint32_t xp[4 * PC];
          float d = 0.f;
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
#pragma unroll
            for (int t = (dw * CD::PAIRS) / 4; t < ((dw + 1) * CD::PAIRS + 3) / 4; ++t) {
              if ((dw * CD::PAIRS) % 4 == 0 || t > (dw * CD::PAIRS) / 4) {
                const u4 pc = *reinterpret_cast<const u4*>(xp8 + (m * PC + t) * 256);
                xp[4 * t + 0] = pc[0];
                xp[4 * t + 1] = pc[1];
                xp[4 * t + 2] = pc[2];
                xp[4 * t + 3] = pc[3];
              }
            }
            d = FD::dot(wq[dw], xp + dw * CD::PAIRS, d);
          }
          const f2 xsm = *reinterpret_cast<const f2*>(xp8 + sdelta + m * NG * 8);
          const float part = d - fe * xsm[0] - fo * xsm[1];
          if constexpr (GROUPED) acc[m] = __builtin_fmaf(sc, part, acc[m]);
          else acc[m] += part;
          if constexpr (ASYM) acc[m] = __builtin_fmaf(zs, xsm[0] + xsm[1], acc[m]);
        }
        xp8 += BS;
        if (++cb == CB) {  // wave-uniform: the four rows of this quad end
          const ProdRec& pr = rec[pi];
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const float v = row16_sum(acc[m]);
            acc[m] = 0.f;
            if (j == 0) {
              if (split_head) head_val[(wv * 4 + q4) * MR + m] = v;
              else if (row_ok)
                store_y_coherent(pr.y, (int64_t)m * pr.ldy + (row - pr.roff), v * pr.tscale, pr.yt, coherent);
            }
          }
          if (split_head && lane == 0) head_q[wv] = cq;
          split_head = false;
          cb = 0;
          ++cq;
          row = quad_row(cq);
          row_ok = r0 + 4 * cq + q4 < r1;
          if (row >= rec[pi].pend) {
            while (row >= rec[pi].pend) ++pi;
            slot0 = xbase + pi * slot_bytes + j * 16;
          }
          xp8 = slot0;
        }
      }
    }
  }
  if (s1 > s0 && cb != 0) {  // the run ends inside a quad
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float v = row16_sum(acc[m]);
      if (j == 0) {
        if (split_head) head_val[(wv * 4 + q4) * MR + m] = v;  // started and ended in one quad
        else tail_val[(wv * 4 + q4) * MR + m] = v;
      }
    }
    if (lane == 0) {
      if (split_head) head_q[wv] = cq;
      else tail_q[wv] = cq;
    }
  }
  __syncthreads();

  // ---- quads split between runs: tail of the wave that began the quad plus
  // the heads of the following waves, in wave order; one thread per row
  if (tid < NW * 4) {
    const int w0 = tid >> 2, r4 = tid & 3;
    const int32_t qd = tail_q[w0];
    const int32_t rr = r0 + 4 * qd + r4;
    if (qd >= 0 && rr < r1) {
      float v[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) v[m] = tail_val[(w0 * 4 + r4) * MR + m];
      for (int w2 = w0 + 1; w2 < NW; ++w2) {
        const bool empty = (int64_t)w2 * T / NW == (int64_t)(w2 + 1) * T / NW;
        if (empty) continue;  // waves with empty runs hold no piece of any quad
        if (head_q[w2] != qd) break;
#pragma unroll
        for (int m = 0; m < MR; ++m) v[m] += head_val[(w2 * 4 + r4) * MR + m];
      }
      const ProdRec& pr = rec[rec_at(rr)];
#pragma unroll
      for (int m = 0; m < MR; ++m)
        store_y_coherent(pr.y, (int64_t)m * pr.ldy + (rr - pr.roff), v[m] * pr.tscale, pr.yt, coherent);
    }
  }
  __syncthreads();  // LDS is reused by the next segment
  return true;
}

// variant = (x fp16 ? 0 : 6) + (bits 2/4/8 -> 0/2/4) + (grouped ? 1 : 0);
// asymmetric (grouped, bits 2/4): 12 + (x fp16 ? 0 : 2) + (bits 4 ? 1 : 0)
__host__ __device__ inline int stream_variant(int xt, int bits, int group, int asym) {
  if (asym) return 12 + (xt == XF16 ? 0 : 2) + (bits == 4 ? 1 : 0);
  return (xt == XF16 ? 0 : 6) + (bits == 2 ? 0 : bits == 4 ? 2 : 4) + (group ? 1 : 0);
}
constexpr int VAR_ANY = 16;

template <int MR, int V>
__device__ __forceinline__ bool run_variant(const StreamPhase& seg, const StreamProblem* probs,
                                            const StreamProblem& single, int2 wr, uint8_t* smem,
                                            uint32_t* sync, uint32_t wt, bool coh) {
  if constexpr (V >= 12) {
    constexpr int XT = V < 14 ? XF16 : XBF16;
    constexpr int BITS = (V & 1) ? 4 : 2;
    return run_segment<XT, BITS, true, MR, true>(seg, probs, single, wr, smem, sync, wt, coh);
  } else {
    constexpr int XT = V < 6 ? XF16 : XBF16;
    constexpr int BITS = (V % 6) / 2 == 0 ? 2 : (V % 6) / 2 == 1 ? 4 : 8;
    constexpr bool GROUPED = (V % 2) == 1;
    return run_segment<XT, BITS, GROUPED, MR>(seg, probs, single, wr, smem, sync, wt, coh);
  }
}

template <int MR, int VAR>
__device__ __forceinline__ bool seg_dispatch(const StreamPhase& seg, const StreamProblem* probs,
                                             const StreamProblem& single, int2 wr, uint8_t* smem,
                                             uint32_t* sync, uint32_t wt, bool coh) {
  if constexpr (VAR != VAR_ANY) {
    return run_variant<MR, VAR>(seg, probs, single, wr, smem, sync, wt, coh);
  } else {
    switch (stream_variant(seg.xt, seg.bits, seg.group, seg.asym)) {
      case 0: return run_variant<MR, 0>(seg, probs, single, wr, smem, sync, wt, coh);
      case 1: return run_variant<MR, 1>(seg, probs, single, wr, smem, sync, wt, coh);
      case 2: return run_variant<MR, 2>(seg, probs, single, wr, smem, sync, wt, coh);
      case 3: return run_variant<MR, 3>(seg, probs, single, wr, smem, sync, wt, coh);
      case 4: return run_variant<MR, 4>(seg, probs, single, wr, smem, sync, wt, coh);
      case 5: return run_variant<MR, 5>(seg, probs, single, wr, smem, sync, wt, coh);
      case 6: return run_variant<MR, 6>(seg, probs, single, wr, smem, sync, wt, coh);
      case 7: return run_variant<MR, 7>(seg, probs, single, wr, smem, sync, wt, coh);
      case 8: return run_variant<MR, 8>(seg, probs, single, wr, smem, sync, wt, coh);
      case 9: return run_variant<MR, 9>(seg, probs, single, wr, smem, sync, wt, coh);
      case 10: return run_variant<MR, 10>(seg, probs, single, wr, smem, sync, wt, coh);
      case 11: return run_variant<MR, 11>(seg, probs, single, wr, smem, sync, wt, coh);
      case 12: return run_variant<MR, 12>(seg, probs, single, wr, smem, sync, wt, coh);
      case 13: return run_variant<MR, 13>(seg, probs, single, wr, smem, sync, wt, coh);
      case 14: return run_variant<MR, 14>(seg, probs, single, wr, smem, sync, wt, coh);
      default: return run_variant<MR, 15>(seg, probs, single, wr, smem, sync, wt, coh);
    }
  }
}

// Single product: segs == nullptr, `single_seg` and `single_prob` by value.
// Plan: nseg segments, the problem table, per-(segment, workgroup) problem
// ranges wranges[s * G + w] = {first, last} (within the segment), and
// sync = {done counter, error word, finished workgroups}; the counters are
// zero when a run starts and the run leaves them zero. VAR fixes the format (VAR_ANY: a mix).
template <int MR, int VAR>
__global__ __launch_bounds__(st_threads<MR>()) void gemv_stream_kernel(
    const StreamPhase* __restrict__ segs, int nseg, const StreamProblem* __restrict__ probs,
    const int2* __restrict__ wranges, StreamPhase single_seg, StreamProblem single_prob, uint32_t* sync) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t G = gridDim.x;
  if (!segs) {
    seg_dispatch<MR, VAR>(single_seg, nullptr, single_prob, make_int2(0, 0), smem, nullptr, 0, false);
    return;
  }
  // data crosses phases only when some segment waits: only then do the
  // activations and outputs need agent-coherent (L2-bypassing) accesses
  bool coh = false;
  for (int s = 0; s < nseg; ++s) coh = coh || segs[s].wait;
  uint32_t waits = 0;
  // a phase wait this workgroup has not performed yet: the poll happens in
  // the first later segment where the workgroup has rows, since segments of
  // one phase may spread their rows over different numbers of workgroups
  uint32_t* pending = nullptr;
  for (int s = 0; s < nseg; ++s) {
    const StreamPhase seg = segs[s];
    if (seg.wait) {
      // this workgroup's outputs of the previous phase are stored
      // (agent-coherent): wait for them to complete, count the workgroup done
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ++waits;
      pending = sync;
    }
    const int2 wr = wranges[(int64_t)s * G + blockIdx.x];
    if (seg_dispatch<MR, VAR>(seg, probs, single_prob, wr, smem, pending, waits * G, coh)) pending = nullptr;
  }
  if (waits) {
    // leave the counter at zero for the next run: the last workgroup to get
    // here knows that no workgroup polls it any more
    __syncthreads();
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1) {
      __hip_atomic_store(sync + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sync + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int MR, int VAR>
static const void* stream_fn() {
  return reinterpret_cast<const void*>(&gemv_stream_kernel<MR, VAR>);
}

template <int MR>
static const void* stream_fn_var(int var) {
  switch (var) {
    case 0: return stream_fn<MR, 0>();
    case 1: return stream_fn<MR, 1>();
    case 2: return stream_fn<MR, 2>();
    case 3: return stream_fn<MR, 3>();
    case 4: return stream_fn<MR, 4>();
    case 5: return stream_fn<MR, 5>();
    case 6: return stream_fn<MR, 6>();
    case 7: return stream_fn<MR, 7>();
    case 8: return stream_fn<MR, 8>();
    case 9: return stream_fn<MR, 9>();
    case 10: return stream_fn<MR, 10>();
    case 11: return stream_fn<MR, 11>();
    case 12: return stream_fn<MR, 12>();
    case 13: return stream_fn<MR, 13>();
    case 14: return stream_fn<MR, 14>();
    case 15: return stream_fn<MR, 15>();
    default: return stream_fn<MR, VAR_ANY>();
  }
}

// kernels for MR activation rows, one translation unit each (zq_stream_m*.hip)
const void* stream_kernel_m1(int var);
const void* stream_kernel_m2(int var);
const void* stream_kernel_m3(int var);
const void* stream_kernel_m4(int var);

}  // namespace zq
