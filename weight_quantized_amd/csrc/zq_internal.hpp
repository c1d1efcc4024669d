// zq_internal.hpp -- host-side interfaces between the C-ABI layer (zq_api.hip)
// and the kernel launchers of libzq.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zq {

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
  int num_xcds = 8;
};
// Properties of the current device, queried once per device and cached.
const DeviceInfo& device_info();

// One validated problem Y[m][n] = X[m][k] * dequant(W)^T, all device pointers.
struct GemmArgs {
  const uint8_t* packed;
  const uint16_t* scales;
  const uint16_t* zeros = nullptr;  // asymmetric weights: fp16 zero points, [n][k/128]
  int bits, group;
  int64_t n, k;
  const uint16_t* x;
  int xt;  // XF16 / XBF16
  int64_t m, ldx;
  void* y;
  int yt;  // YF32 / YF16 / YBF16
  int64_t ldy;
  hipStream_t stream;
};

// One product of the persistent decode kernel (device pointers).
struct StreamProblem {
  const uint8_t* packed;
  const uint16_t* zeros;  // asymmetric weights (unsigned codes): zero points, else nullptr
  const uint16_t* scales;
  const uint16_t* x;
  void* y;
  int64_t n, k, ldx, ldy;
  int64_t row_off;  // first row in its segment's concatenated row space
  int32_t bits, group, xt, yt;
};
// A segment of a plan: consecutive products of one phase that share k, bits,
// group and activation type. wait = 1: the segment starts its arithmetic
// only after every workgroup has stored all earlier segments' outputs.
struct StreamPhase {
  int32_t first, count;  // problems [first, first + count) of the problem table
  int64_t n_total, k;
  int32_t bits, group, xt, wait;
  int32_t asym;          // unsigned codes with zero points
  int32_t grid;          // decode kernel: workgroups that share the segment's rows (0: all)
};
constexpr size_t STREAM_LDS_MAX = 160 * 1024;
int stream_grid();  // workgroups of a stream launch (one per CU)
// workgroups for a segment of n rows: at most one per CU, and no more than
// give each wave about one step of 4 rows x 256 bytes (small products are
// latency-bound: fewer, fuller workgroups start sooner)
int stream_grid_for(int bits, int64_t m, int64_t n, int64_t k);
// persistent, balanced kernel (1 <= m <= 4, rows of whole 256-byte steps)
bool stream_supported(int bits, int group, int64_t m, int64_t n, int64_t k);
size_t stream_lds_bytes(int bits, int64_t m, int64_t k, int nrec);
int stream_variant_of(int xt, int bits, int group, int asym);
constexpr int STREAM_VAR_ANY = 16;  // a plan mixing formats
hipError_t launch_stream_single(const StreamProblem& p, int64_t m, hipStream_t stream);
// dev_ranges[s * stream_grid() + w] = {first, last} product (within segment s)
// that workgroup w touches; variant: one format code (stream_variant_of) for
// every segment, or STREAM_VAR_ANY for a mix; sync = 3 device words
hipError_t launch_stream_plan(const StreamPhase* dev_segs, int nseg, const StreamProblem* dev_probs,
                              const int2* dev_ranges, int64_t m, int variant, size_t lds, uint32_t* sync,
                              bool waits, int grid, hipStream_t stream);

// persistent MFMA kernel for batched decode: INT4, 2 <= m <= 32, k a
// multiple of 512, 16-byte aligned codes and activations, 8-byte aligned
// group scales
constexpr int MSTREAM_MIN_M = 2;  // measured faster than the VALU kernel from 2 rows on
bool mstream_supported(const void* packed, const uint16_t* scales, const uint16_t* zeros, int bits, int group,
                       int64_t m, int64_t k, const void* x, int64_t ldx);
size_t mstream_lds(int64_t m, int nrec);
int mstream_variant_of(int xt, int group, int asym);
constexpr int MSTREAM_VAR_ANY = 6;  // the variant of a plan that mixes formats
hipError_t launch_mstream_single(const StreamProblem& p, int64_t m, hipStream_t stream);
hipError_t launch_mstream_plan(const StreamPhase* dev_segs, int nseg, const StreamProblem* dev_probs,
                               const int2* dev_ranges, int64_t m, int variant, size_t lds, uint32_t* sync,
                               bool waits, hipStream_t stream);

// vector-ALU kernel for m <= 4 with x staged in LDS
size_t gemv_valu_lds_bytes(int bits, int64_t m, int64_t k);
hipError_t launch_gemv_valu(const GemmArgs& a);
// prefill MFMA kernel: m > 16, symmetric codes, one scale per tensor (k a
// multiple of 64) or per row and 128 k
bool gemm_prefill_supported(const GemmArgs& a);
hipError_t launch_gemm_prefill(const GemmArgs& a);
// rows of the kernel's output tiles for m activation rows (32, 64 or 128)
int prefill_tile_m(int64_t m);
// One product of a prefill plan (device pointers): its prefill_tile_m(m) x
// PREFILL_TILE_N tiles are plan tiles [tile0, tile0 + mtiles * ntiles), row
// block fastest.
struct PrefillProblem {
  const uint8_t* packed;
  const uint16_t* scales;
  const uint16_t* x;
  void* y;
  int64_t m, n, k, ldx, ldy;
  int64_t tile0, mtiles;
  int32_t bits, yt, group;
};
constexpr int PREFILL_TILE_N = 256;
// persistent launch over the `total` tiles of products of one bit width and
// group size (m activation rows); xt: their activations' type; sync:
// PREFILL_SYNC_WORDS device words (tile counters, finished workgroups), zero
// before the first run
constexpr int PREFILL_SYNC_WORDS = 16;
hipError_t launch_prefill_plan(const PrefillProblem* dev_probs, int nprob, int64_t total, int xt, int bits,
                               int group, int64_t m, uint32_t* sync, hipStream_t stream);
// MFMA kernels for larger m
bool gemm_mfma_supported(const GemmArgs& a);
hipError_t launch_gemm_mfma(const GemmArgs& a);
// general kernel: any legal shape and alignment
hipError_t launch_gemm_general(const GemmArgs& a);
// Y rows of n zeros (a fill kernel, so it is safe under stream capture)
hipError_t launch_zero_rows(void* y, int esz, int64_t m, int64_t n, int64_t ldy, hipStream_t s);

// pack / unpack
struct PackArgs {
  const void* w;
  int wt;  // 0 = int8 codes, 1 = f16, 2 = bf16, 3 = f32
  int64_t n, k;
  int bits, group;
  const uint16_t* scales;  // scales used for quantizing (given or computed)
  const uint16_t* zeros;   // asymmetric: zero points used for quantizing, else nullptr
  uint8_t* packed;
  uint32_t* flags;         // device: [0] error bits, [1] absmax bits
  hipStream_t stream;
};
enum : uint32_t { FLAG_NONFINITE = 1u, FLAG_SCALE_RANGE = 2u, FLAG_CODE_RANGE = 4u };
hipError_t launch_compute_scales(const PackArgs& a, uint16_t* scales_out);
hipError_t launch_quantize_pack(const PackArgs& a);
hipError_t launch_unpack(const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros, int bits,
                         int group, int64_t n, int64_t k, void* out, int out_dtype, hipStream_t stream);
// asymmetric weights (unsigned codes, fp16 scale and zero per 128-group)
hipError_t launch_compute_scales_zeros(const PackArgs& a, uint16_t* scales_out, uint16_t* zeros_out);
hipError_t launch_quantize_pack_asym(const PackArgs& a);

}  // namespace zq
