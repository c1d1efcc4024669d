// zq_gemv.hip -- vector-ALU kernels of the quantized linear layer for few
// activation rows (decode), and the general kernel for shapes the fast paths
// do not take.
//
// The decode kernel follows the idea of the wave-64 INT4 GEMV with 128-bit
// weight loads that the ZSE wiki article ("ZSE - open-source движок для запуска
// LLM локально на GPU - 2026", section "Оркестратор и GPU-ядра") names as the
// main small-batch kernel on AMD; its layout here is designed for gfx950:
//   * a wave covers 4 weight rows, 16 lanes per row; every lane loads whole
//     16-byte chunks (global_load_dwordx4), so each instruction reads four
//     256-byte row segments; U chunks per lane are in flight at once;
//   * activations are staged once per workgroup in LDS, already permuted into
//     the pair order of the code decoder and laid out [piece][chunk] so the 16
//     lanes of a row read consecutive 16-byte pieces (no bank conflicts);
//     the staging also stores each chunk's activation sum;
//   * codes become exact fp16/bf16 pairs (two VALU ops per pair, see
//     Decoder) and are dotted with v_dot2_f32_{f16,bf16}; the decoder's
//     constant offset is removed once per chunk with the staged sum; the
//     group scale multiplies the chunk partial (a chunk never spans groups);
//   * the 16 per-lane partials of a row are reduced with four DPP steps;
//   * workgroups are persistent: each stages x once and then walks the row
//     quads in a grid-stride loop.
#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace zq {

constexpr int GEMV_THREADS = 256;

template <int XT, int BITS, int MR, bool GROUPED, int U>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_valu_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales, int64_t n,
    int64_t k, const uint16_t* __restrict__ x, int64_t ldx, void* __restrict__ y,
    int64_t ldy, int yt) {
  using D = Decoder<XT, BITS>;
  using CD = Codes<BITS>;
  constexpr int WPC = 128 / BITS;       // weights per 16-byte chunk
  constexpr int PC = WPC / 8;           // 16-byte activation pieces per chunk
  constexpr int CPG = 128 / WPC;        // chunks per 128-group
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t C = k / WPC;            // chunks per row
  u4* xs = reinterpret_cast<u4*>(smem);                       // [MR][PC][C]
  float* xsum = reinterpret_cast<float*>(smem + (size_t)MR * PC * C * 16);  // [MR][C]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;
  const int64_t units = (n + 3) >> 2;
  const int64_t rowbytes = C * 16;

  // First unit of this wave: start its weight loads before staging x.
  int64_t unit = (int64_t)blockIdx.x * 4 + wave;
  const int64_t ustride = (int64_t)gridDim.x * 4;

  // ---- stage x: piece (m, c, t) holds the 8 activations that meet the 16-bit
  // pairs of piece t of chunk c, in decoder order.
  {
    const int64_t P = (int64_t)MR * C * PC;
    const int64_t iters = (P + GEMV_THREADS - 1) / GEMV_THREADS;
    for (int64_t it = 0; it < iters; ++it) {
      const int64_t idx = it * GEMV_THREADS + tid;
      float psum = 0.f;
      u4 piece = {0, 0, 0, 0};
      int m = 0;
      int64_t c = 0;
      int t = 0;
      const bool live = idx < P;
      if (live) {
        m = (int)(idx / (C * PC));
        const int64_t rem = idx - (int64_t)m * C * PC;
        c = rem / PC;
        t = (int)(rem - c * PC);
        const uint16_t* xr = x + (int64_t)m * ldx + c * WPC;
        uint16_t v[8];
        if constexpr (BITS == 4 || BITS == 8) {
          // the piece covers 8 consecutive activations: one 16-byte load
          const u4 raw = *reinterpret_cast<const u4*>(xr + 8 * t);
          const uint16_t* r = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            const int p = 8 * t + h, q = p % CD::E, e = q / 2 + (q % 2) * (CD::E / 2);
            v[h] = r[(p / CD::E) * CD::E + e - 8 * t];
          }
        } else {
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            const int p = 8 * t + h, q = p % CD::E, e = q / 2 + (q % 2) * (CD::E / 2);
            v[h] = xr[(p / CD::E) * CD::E + e];
          }
        }
#pragma unroll
        for (int h = 0; h < 8; ++h) psum += x_bits_to_float<XT>(v[h]);
        piece[0] = v[0] | ((uint32_t)v[1] << 16);
        piece[1] = v[2] | ((uint32_t)v[3] << 16);
        piece[2] = v[4] | ((uint32_t)v[5] << 16);
        piece[3] = v[6] | ((uint32_t)v[7] << 16);
        xs[((int64_t)m * PC + t) * C + c] = piece;
      }
      // sum the PC pieces of a chunk: they sit on PC consecutive lanes
#pragma unroll
      for (int o = 1; o < PC; o <<= 1) psum += __shfl_xor(psum, o, 64);
      if (live && t == 0) xsum[(int64_t)m * C + c] = psum;
    }
  }
  __syncthreads();

  float tensor_scale = 1.f;
  if constexpr (!GROUPED) tensor_scale = f16_bits_to_float(scales[0]);

  for (; unit < units; unit += ustride) {
    const int64_t row = unit * 4 + (lane >> 4);
    const bool rv = row < n;
    const u4* wr = reinterpret_cast<const u4*>(packed + (rv ? row : 0) * rowbytes);
    const uint16_t* sr = scales + (GROUPED ? (rv ? row : 0) * (C / CPG) : 0);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;

    for (int64_t c0 = j; c0 < C; c0 += 16 * U) {
      u4 w[U];
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + 16 * u;
        if (rv && c < C) {
          w[u] = __builtin_nontemporal_load(wr + c);
          s[u] = GROUPED ? f16_bits_to_float(sr[c / CPG]) : 1.f;
        } else {
          w[u] = u4{0, 0, 0, 0};
          s[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + 16 * u;
        if (c < C) {
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            uint32_t xp[4 * PC];
#pragma unroll
            for (int t = 0; t < PC; ++t) {
              const u4 pc = xs[((int64_t)m * PC + t) * C + c];
              xp[4 * t + 0] = pc[0];
              xp[4 * t + 1] = pc[1];
              xp[4 * t + 2] = pc[2];
              xp[4 * t + 3] = pc[3];
            }
            float d = 0.f;
#pragma unroll
            for (int dw = 0; dw < 4; ++dw) {
              const uint32_t v = w[u][dw] ^ CD::SIGNS;
              const uint32_t* xq = xp + dw * CD::PAIRS;
              [&]<int... I>(std::integer_sequence<int, I...>) {
                ((d = dot2<XT>(D::template pair<I>(v), xq[I], d)), ...);
              }(std::make_integer_sequence<int, CD::PAIRS>{});
            }
            const float part = d - D::BIAS * xsum[(int64_t)m * C + c];
            if constexpr (GROUPED) acc[m] = __builtin_fmaf(s[u], part, acc[m]);
            else acc[m] += part;
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float v = row16_sum(acc[m]) * tensor_scale;
      if (rv && j == 0) store_y(y, (int64_t)m * ldy + row, v, yt);
    }
  }
}

// ---------------------------------------------------------------------------
// General kernel: one wave per output (m, row); byte-granular reads, any K
// that the format allows, any alignment. Same arithmetic contract (fp32 sums
// of x * q * s), different order.
// Asymmetric weights (zeros != nullptr): unsigned codes, w = q * s + z.
template <int XT>
__global__ __launch_bounds__(256) void gemm_general_kernel(
    const uint8_t* __restrict__ packed, int bits, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, int group, int64_t n, int64_t k, const uint16_t* __restrict__ x,
    int64_t m, int64_t ldx, void* __restrict__ y, int64_t ldy, int yt) {
  const int lane = threadIdx.x & 63;
  const int64_t out = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (out >= m * n) return;  // whole wave leaves together
  const int64_t mi = out / n, r = out - mi * n;
  const int per = 8 / bits;
  const int64_t rowbytes = k / per;
  const int64_t G = group ? k / group : 0;
  float acc = 0.f;
  for (int64_t c = lane; c < k; c += 64) {
    const uint32_t byte = packed[r * rowbytes + c / per];
    const int i = (int)(c % per);
    int f = (int)((byte >> (i * bits)) & ((1u << bits) - 1u));
    if (!zeros && f >= (1 << (bits - 1))) f -= (1 << bits);
    const int64_t si = group ? r * G + c / group : 0;
    const float s = f16_bits_to_float(scales[si]);
    const float wv = zeros ? __builtin_fmaf((float)f, s, f16_bits_to_float(zeros[si])) : (float)f * s;
    acc = __builtin_fmaf(x_bits_to_float<XT>(x[mi * ldx + c]), wv, acc);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) store_y(y, mi * ldy + r, acc, yt);
}

__global__ void zero_rows_kernel(uint8_t* __restrict__ y, int esz, int64_t m, int64_t n,
                                 int64_t ldy) {
  const int64_t total = m * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / n, c = i - r * n;
    if (esz == 4) reinterpret_cast<float*>(y)[r * ldy + c] = 0.f;
    else reinterpret_cast<uint16_t*>(y)[r * ldy + c] = 0;
  }
}

// ---------------------------------------------------------------------------
// Host launchers

hipError_t launch_zero_rows(void* y, int esz, int64_t m, int64_t n, int64_t ldy, hipStream_t s) {
  int64_t blocks = (m * n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks > 0)
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint8_t*)y, esz,
                       m, n, ldy);
  return hipGetLastError();
}

static int gemv_blocks(const void* fn, size_t lds, int64_t units) {
  const DeviceInfo& di = device_info();
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, GEMV_THREADS, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t want = (units + 3) / 4;
  const int64_t cap = (int64_t)di.num_cus * per_cu;
  return (int)(want < cap ? want : cap);
}

template <int XT, int BITS, int MR, bool GROUPED>
static hipError_t launch_valu(const GemmArgs& a) {
  constexpr int U = 8;
  constexpr int WPC = 128 / BITS;
  constexpr int PC = WPC / 8;
  const int64_t C = a.k / WPC;
  const size_t lds = (size_t)MR * C * (PC * 16 + 4);
  auto fn = gemv_valu_kernel<XT, BITS, MR, GROUPED, U>;
  const int64_t units = (a.n + 3) / 4;
  const int blocks = gemv_blocks(reinterpret_cast<const void*>(fn), lds, units);
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(GEMV_THREADS), lds, a.stream, a.packed, a.scales,
                     a.n, a.k, a.x, a.ldx, a.y, a.ldy, a.yt);
  return hipGetLastError();
}

size_t gemv_valu_lds_bytes(int bits, int64_t m, int64_t k) {
  const int WPC = 128 / bits, PC = WPC / 8;
  return (size_t)m * (k / WPC) * (PC * 16 + 4);
}

template <int XT, int BITS, bool GROUPED>
static hipError_t launch_valu_m(const GemmArgs& a) {
  switch (a.m) {
    case 1: return launch_valu<XT, BITS, 1, GROUPED>(a);
    case 2: return launch_valu<XT, BITS, 2, GROUPED>(a);
    case 3: return launch_valu<XT, BITS, 3, GROUPED>(a);
    default: return launch_valu<XT, BITS, 4, GROUPED>(a);
  }
}

template <int XT, int BITS>
static hipError_t launch_valu_g(const GemmArgs& a) {
  return a.group ? launch_valu_m<XT, BITS, true>(a) : launch_valu_m<XT, BITS, false>(a);
}

hipError_t launch_gemv_valu(const GemmArgs& a) {
  if (a.xt == XF16) {
    switch (a.bits) {
      case 2: return launch_valu_g<XF16, 2>(a);
      case 4: return launch_valu_g<XF16, 4>(a);
      default: return launch_valu_g<XF16, 8>(a);
    }
  }
  switch (a.bits) {
    case 2: return launch_valu_g<XBF16, 2>(a);
    case 4: return launch_valu_g<XBF16, 4>(a);
    default: return launch_valu_g<XBF16, 8>(a);
  }
}

hipError_t launch_gemm_general(const GemmArgs& a) {
  const int64_t outs = a.m * a.n;
  const int64_t blocks = (outs + 3) / 4;
  if (a.xt == XF16)
    hipLaunchKernelGGL(gemm_general_kernel<XF16>, dim3((uint32_t)blocks), dim3(256), 0, a.stream,
                       a.packed, a.bits, a.scales, a.zeros, a.group, a.n, a.k, a.x, a.m, a.ldx, a.y, a.ldy,
                       a.yt);
  else
    hipLaunchKernelGGL(gemm_general_kernel<XBF16>, dim3((uint32_t)blocks), dim3(256), 0, a.stream,
                       a.packed, a.bits, a.scales, a.zeros, a.group, a.n, a.k, a.x, a.m, a.ldx, a.y, a.ldy,
                       a.yt);
  return hipGetLastError();
}

}  // namespace zq
