// zq_api.hip -- the C-ABI of libzq.so (declared in include/zq.h): argument
// validation, kernel choice and error reporting. Every check runs before the
// first HIP call, so invalid calls never touch the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <tuple>
#include <vector>

#include "zq.h"
#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace {
// rows of the mid-batch chunk that starts at row r0 of m: 32, but never a
// last chunk of one row (the batched-decode kernel takes 2..32)
int64_t chunk_rows(int64_t m, int64_t r0) { return m - r0 == 33 ? 31 : std::min<int64_t>(32, m - r0); }


thread_local char g_err[512] = "";

zq_status fail(zq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

zq_status ok() {
  g_err[0] = 0;
  return ZQ_OK;
}

zq_status hip_fail(hipError_t e, const char* where) {
  return fail(ZQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool bits_supported(int bits) { return bits == 2 || bits == 4 || bits == 8; }

// Format checks shared by every call that takes a weight shape.
zq_status check_format(int bits, int group, int64_t n, int64_t k) {
  if (!bits_supported(bits)) return fail(ZQ_ERR_UNSUPPORTED, "bits=%d not in {2,4,8}", bits);
  if (group != 0 && group != 128) return fail(ZQ_ERR_UNSUPPORTED, "group=%d not in {0,128}", group);
  if (n < 0 || k < 0) return fail(ZQ_ERR_INVALID_ARG, "negative size n=%lld k=%lld", (long long)n, (long long)k);
  if (group && k % group) return fail(ZQ_ERR_UNSUPPORTED, "k=%lld not a multiple of group %d", (long long)k, group);
  if (k % (8 / bits)) return fail(ZQ_ERR_UNSUPPORTED, "k=%lld not a multiple of %d codes per byte", (long long)k, 8 / bits);
  return ZQ_OK;
}

zq_status check_weight(const zq_weight* W) {
  if (!W) return fail(ZQ_ERR_INVALID_ARG, "null weight descriptor");
  zq_status s = check_format(W->bits, W->group, W->n, W->k);
  if (s) return s;
  if (W->n > 0 && W->k > 0 && (!W->packed || !W->scales))
    return fail(ZQ_ERR_INVALID_ARG, "null packed or scales pointer");
  if (W->zeros && (W->bits == 8 || W->group != 128))
    return fail(ZQ_ERR_UNSUPPORTED, "asymmetric weights take bits 2 or 4 and group 128");
  return ZQ_OK;
}

std::mutex g_dev_mu;
std::vector<zq::DeviceInfo> g_devs;

// ---- device flag words of the pack kernels: [0] error bits, [1] tensor absmax
constexpr int PACK_FLAG_WORDS = 2;

// Scratch of zq_pack_noalloc: a file-scope device array, one copy per GPU,
// holding the pack kernels' flag words (every shape needs the same two).
// Host code never passes `scratch` itself (in host code the name is only a
// stand-in); the device address comes from hipGetSymbolAddress, taken once
// per device with that device current and kept in g_scratch.
constexpr int NOALLOC_SCRATCH_WORDS = 64;  // 256 bytes per device
static __device__ __align__(256) uint32_t scratch[NOALLOC_SCRATCH_WORDS];
std::mutex g_scratch_mu;
std::vector<uint32_t*> g_scratch;  // per device: address of `scratch`, or null before the first call

hipError_t scratch_address(uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Argument checks of zq_pack (before any HIP call).
zq_status check_pack(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits, int group,
                     const uint16_t* scales_in, void* packed_out, uint16_t* scales_out) {
  zq_status st = check_format(bits, group, n, k);
  if (st) return st;
  if (w_dtype != ZQ_I8 && w_dtype != ZQ_F16 && w_dtype != ZQ_BF16 && w_dtype != ZQ_F32)
    return fail(ZQ_ERR_INVALID_ARG, "w_dtype=%d not accepted", (int)w_dtype);
  const bool empty = n == 0 || k == 0;
  if (!empty && (!w || !packed_out)) return fail(ZQ_ERR_INVALID_ARG, "null w or packed_out");
  if (w_dtype != ZQ_I8 && !scales_in && !scales_out)
    return fail(ZQ_ERR_INVALID_ARG, "float weights need scales_in or scales_out");
  return ZQ_OK;
}

// The work of zq_pack on checked arguments, with `flags` (PACK_FLAG_WORDS
// device words, used only for non-empty shapes) as the kernels' flag buffer:
// cleared by a fill kernel, then read back after the stream is synchronised.
zq_status pack_body(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits, int group,
                    const uint16_t* scales_in, void* packed_out, uint16_t* scales_out, void* stream,
                    uint32_t* flags) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t ns = zq_num_scales(group, n, k);
  hipError_t e;
  if (scales_in && scales_out && scales_in != scales_out && ns > 0) {
    e = hipMemcpyAsync(scales_out, scales_in, (size_t)ns * 2, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "copy scales");
  }
  if (n == 0 || k == 0) {
    if (w_dtype != ZQ_I8 && !scales_in && ns > 0) {
      // an empty tensor has absmax 0: its scales are +0
      e = hipMemsetAsync(scales_out, 0, (size_t)ns * 2, s);
      if (e != hipSuccess) return hip_fail(e, "zero scales");
    }
    e = hipStreamSynchronize(s);
    return e == hipSuccess ? ok() : hip_fail(e, "sync");
  }
  zq::PackArgs a;
  a.w = w;
  a.wt = (int)w_dtype;
  a.n = n;
  a.k = k;
  a.bits = bits;
  a.group = group;
  a.scales = scales_in ? scales_in : scales_out;
  a.zeros = nullptr;
  a.packed = (uint8_t*)packed_out;
  a.flags = flags;
  a.stream = s;
  uint32_t host_flags[PACK_FLAG_WORDS] = {0, 0};
  e = zq::launch_zero_rows(flags, 4, 1, PACK_FLAG_WORDS, PACK_FLAG_WORDS, s);
  if (e == hipSuccess && w_dtype != ZQ_I8 && !scales_in) e = zq::launch_compute_scales(a, scales_out);
  if (e == hipSuccess) e = zq::launch_quantize_pack(a);
  if (e == hipSuccess) e = hipMemcpyAsync(host_flags, flags, sizeof host_flags, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "pack");
  if (host_flags[0] & zq::FLAG_NONFINITE) return fail(ZQ_ERR_RANGE, "non-finite weight or scale");
  if (host_flags[0] & zq::FLAG_SCALE_RANGE) return fail(ZQ_ERR_RANGE, "scale beyond the fp16 range");
  if (host_flags[0] & zq::FLAG_CODE_RANGE) return fail(ZQ_ERR_RANGE, "code outside the %d-bit range", bits);
  return ok();
}

}  // namespace

namespace zq {
const DeviceInfo& device_info() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_devs.size() <= dev) g_devs.resize(dev + 1);
  DeviceInfo& d = g_devs[dev];
  if (d.device < 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    d.num_cus = cus;
    d.device = dev;
  }
  return d;
}
}  // namespace zq

extern "C" {

size_t zq_packed_bytes(int bits, int64_t n, int64_t k) {
  if (!bits_supported(bits) || n < 0 || k < 0) return 0;
  return (size_t)(n * k * bits / 8);
}

int64_t zq_num_scales(int group, int64_t n, int64_t k) {
  if (group == 0) return 1;
  if (group != 128 || n < 0 || k < 0) return -1;
  return n * (k / 128);
}

const char* zq_status_string(zq_status s) {
  switch (s) {
    case ZQ_OK: return "ok";
    case ZQ_ERR_INVALID_ARG: return "invalid argument";
    case ZQ_ERR_UNSUPPORTED: return "unsupported format or shape";
    case ZQ_ERR_RANGE: return "value out of range";
    case ZQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* zq_last_error(void) { return g_err; }

zq_status zq_pack(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits, int group,
                  const uint16_t* scales_in, void* packed_out, uint16_t* scales_out, void* stream) {
  zq_status st = check_pack(w, w_dtype, n, k, bits, group, scales_in, packed_out, scales_out);
  if (st) return st;
  if (n == 0 || k == 0) return pack_body(w, w_dtype, n, k, bits, group, scales_in, packed_out, scales_out, stream,
                                         nullptr);
  uint32_t* flags = nullptr;
  hipError_t e = hipMalloc(&flags, PACK_FLAG_WORDS * sizeof(uint32_t));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc flags");
  st = pack_body(w, w_dtype, n, k, bits, group, scales_in, packed_out, scales_out, stream, flags);
  char keep[sizeof g_err];
  memcpy(keep, g_err, sizeof keep);
  hipError_t ef = hipFree(flags);
  if (st) return fail(st, "%s", keep);
  if (ef != hipSuccess) return hip_fail(ef, "hipFree flags");
  return ok();
}

zq_status zq_pack_noalloc(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits, int group,
                          const uint16_t* scales_in, void* packed_out, uint16_t* scales_out, void* stream) {
  zq_status st = check_pack(w, w_dtype, n, k, bits, group, scales_in, packed_out, scales_out);
  if (st) return st;
  static_assert(PACK_FLAG_WORDS <= NOALLOC_SCRATCH_WORDS, "the pack flags fit the static scratch");
  uint32_t* flags = nullptr;
  if (n > 0 && k > 0) {
    hipError_t e = scratch_address(&flags);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  }
  return pack_body(w, w_dtype, n, k, bits, group, scales_in, packed_out, scales_out, stream, flags);
}

zq_status zq_pack_asym(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits,
                       const uint16_t* scales_in, const uint16_t* zeros_in, void* packed_out,
                       uint16_t* scales_out, uint16_t* zeros_out, void* stream) {
  if (bits != 2 && bits != 4) return fail(ZQ_ERR_UNSUPPORTED, "asymmetric weights take bits 2 or 4 (bits=%d)", bits);
  zq_status st = check_format(bits, 128, n, k);
  if (st) return st;
  if (w_dtype != ZQ_I8 && w_dtype != ZQ_F16 && w_dtype != ZQ_BF16 && w_dtype != ZQ_F32)
    return fail(ZQ_ERR_INVALID_ARG, "w_dtype=%d not accepted", (int)w_dtype);
  const bool empty = n == 0 || k == 0;
  if (!empty && (!w || !packed_out)) return fail(ZQ_ERR_INVALID_ARG, "null w or packed_out");
  if ((scales_in == nullptr) != (zeros_in == nullptr))
    return fail(ZQ_ERR_INVALID_ARG, "scales_in and zeros_in go together");
  if (w_dtype == ZQ_I8 && !scales_in && (!scales_out || !zeros_out) && !empty)
    return fail(ZQ_ERR_INVALID_ARG, "integer codes need scales_in and zeros_in");
  if (!scales_in && (!scales_out || !zeros_out))
    return fail(ZQ_ERR_INVALID_ARG, "float weights need scales_in/zeros_in or scales_out/zeros_out");
  hipStream_t s = (hipStream_t)stream;
  const int64_t ns = n * (k / 128);
  hipError_t e;
  if (scales_in && scales_out && zeros_out && ns > 0) {
    if (scales_in != scales_out) {
      e = hipMemcpyAsync(scales_out, scales_in, (size_t)ns * 2, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "copy scales");
    }
    if (zeros_in != zeros_out) {
      e = hipMemcpyAsync(zeros_out, zeros_in, (size_t)ns * 2, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "copy zeros");
    }
  }
  if (empty) {
    e = hipStreamSynchronize(s);
    return e == hipSuccess ? ok() : hip_fail(e, "sync");
  }
  uint32_t* flags = nullptr;
  e = hipMalloc(&flags, 2 * sizeof(uint32_t));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc flags");
  zq::PackArgs a;
  a.w = w;
  a.wt = (int)w_dtype;
  a.n = n;
  a.k = k;
  a.bits = bits;
  a.group = 128;
  a.scales = scales_in ? scales_in : scales_out;
  a.zeros = zeros_in ? zeros_in : zeros_out;
  a.packed = (uint8_t*)packed_out;
  a.flags = flags;
  a.stream = s;
  uint32_t host_flags[2] = {0, 0};
  e = hipMemsetAsync(flags, 0, 2 * sizeof(uint32_t), s);
  if (e == hipSuccess && w_dtype != ZQ_I8 && !scales_in) e = zq::launch_compute_scales_zeros(a, scales_out, zeros_out);
  if (e == hipSuccess) e = zq::launch_quantize_pack_asym(a);
  if (e == hipSuccess) e = hipMemcpyAsync(host_flags, flags, sizeof host_flags, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipError_t ef = hipFree(flags);
  if (e != hipSuccess) return hip_fail(e, "pack");
  if (ef != hipSuccess) return hip_fail(ef, "hipFree flags");
  if (host_flags[0] & zq::FLAG_NONFINITE) return fail(ZQ_ERR_RANGE, "non-finite weight, scale or zero");
  if (host_flags[0] & zq::FLAG_SCALE_RANGE) return fail(ZQ_ERR_RANGE, "scale or zero beyond the fp16 range");
  if (host_flags[0] & zq::FLAG_CODE_RANGE) return fail(ZQ_ERR_RANGE, "code outside [0, %d]", (1 << bits) - 1);
  return ok();
}

zq_status zq_unpack(const zq_weight* W, void* out, zq_dtype out_dtype, void* stream) {
  zq_status st = check_weight(W);
  if (st) return st;
  if (out_dtype != ZQ_I8 && out_dtype != ZQ_F16 && out_dtype != ZQ_BF16 && out_dtype != ZQ_F32)
    return fail(ZQ_ERR_INVALID_ARG, "out_dtype=%d not accepted", (int)out_dtype);
  if (W->n > 0 && W->k > 0 && !out) return fail(ZQ_ERR_INVALID_ARG, "null out");
  hipError_t e = zq::launch_unpack((const uint8_t*)W->packed, W->scales, W->zeros, W->bits, W->group,
                                   W->n, W->k, out, (int)out_dtype, (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "unpack launch");
}

zq_status zq_gemm(const zq_weight* W, const void* X, zq_dtype x_dtype, int64_t m, int64_t ldx,
                  void* Y, zq_dtype y_dtype, int64_t ldy, void* stream) {
  zq_status st = check_weight(W);
  if (st) return st;
  if (x_dtype != ZQ_F16 && x_dtype != ZQ_BF16)
    return fail(ZQ_ERR_INVALID_ARG, "x_dtype=%d not accepted (F16 or BF16)", (int)x_dtype);
  if (y_dtype != ZQ_F32 && y_dtype != ZQ_F16 && y_dtype != ZQ_BF16)
    return fail(ZQ_ERR_INVALID_ARG, "y_dtype=%d not accepted (F32, F16 or BF16)", (int)y_dtype);
  if (m < 0) return fail(ZQ_ERR_INVALID_ARG, "negative m");
  if (ldx < W->k || ldy < W->n) return fail(ZQ_ERR_INVALID_ARG, "ldx < k or ldy < n");
  if (m == 0 || W->n == 0) return ok();
  if (!Y || (W->k > 0 && !X)) return fail(ZQ_ERR_INVALID_ARG, "null X or Y");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (W->k == 0) {
    // empty sums: zero rows of Y
    e = zq::launch_zero_rows(Y, y_dtype == ZQ_F32 ? 4 : 2, m, W->n, ldy, s);
    return e == hipSuccess ? ok() : hip_fail(e, "zero Y");
  }
  zq::GemmArgs a;
  a.packed = (const uint8_t*)W->packed;
  a.scales = W->scales;
  a.zeros = W->zeros;
  a.bits = W->bits;
  a.group = W->group;
  a.n = W->n;
  a.k = W->k;
  a.x = (const uint16_t*)X;
  a.xt = x_dtype == ZQ_F16 ? zq::XF16 : zq::XBF16;
  a.m = m;
  a.ldx = ldx;
  a.y = Y;
  a.yt = y_dtype == ZQ_F32 ? zq::YF32 : y_dtype == ZQ_F16 ? zq::YF16 : zq::YBF16;
  a.ldy = ldy;
  a.stream = s;
  const int64_t rowbytes = W->k * W->bits / 8;
  const bool aligned16 = ((uintptr_t)W->packed & 15) == 0 && rowbytes % 16 == 0 &&
                         ((uintptr_t)X & 15) == 0 && (m == 1 || (ldx * 2) % 16 == 0);
  // asymmetric weights: the vector-ALU stream kernel (m = 1), the MFMA
  // batched-decode kernel (INT4) or the general kernel
  const bool asym = W->zeros != nullptr;
  // the batched-decode kernel streams the weights fastest up to 32 rows;
  // past that, and for the formats it does not take, symmetric codes go to
  // the prefill tiles (32, 64 or 128 rows high)
  const bool mstream_ok = m >= zq::MSTREAM_MIN_M && m <= 32 &&
                          zq::mstream_supported(W->packed, W->scales, W->zeros, W->bits, W->group, m, W->k, X, ldx);
  const bool use_prefill = !mstream_ok && !asym && aligned16 && zq::gemm_prefill_supported(a);
  const bool use_mstream = !use_prefill && mstream_ok;
  // other m > 32 (asymmetric codes): 32-row chunks on the batched-decode
  // kernel
  const bool use_chunks = !use_prefill && m > 32 &&
                          zq::mstream_supported(W->packed, W->scales, W->zeros, W->bits, W->group, 32, W->k, X, ldx);
  if (use_chunks) {
    const int ysz = y_dtype == ZQ_F32 ? 4 : 2;
    e = hipSuccess;
    for (int64_t r0 = 0, mc = 0; r0 < m && e == hipSuccess; r0 += mc) {
      mc = chunk_rows(m, r0);
      zq::StreamProblem p{};
      p.packed = a.packed;
      p.scales = a.scales;
      p.zeros = a.zeros;
      p.x = a.x + r0 * ldx;
      p.y = (uint8_t*)Y + r0 * ldy * ysz;
      p.n = a.n;
      p.k = a.k;
      p.ldx = ldx;
      p.ldy = ldy;
      p.bits = a.bits;
      p.group = a.group;
      p.xt = a.xt;
      p.yt = a.yt;
      e = zq::launch_mstream_single(p, mc, s);
    }
    return e == hipSuccess ? ok() : hip_fail(e, "gemm launch");
  }
  const bool use_stream = !use_mstream && m <= 4 && aligned16 &&
                          zq::stream_supported(W->bits, W->group, m, W->n, W->k);
  if (use_stream || use_mstream) {
    zq::StreamProblem p{};
    p.packed = a.packed;
    p.scales = a.scales;
    p.zeros = a.zeros;
    p.x = a.x;
    p.y = a.y;
    p.n = a.n;
    p.k = a.k;
    p.ldx = a.ldx;
    p.ldy = a.ldy;
    p.bits = a.bits;
    p.group = a.group;
    p.xt = a.xt;
    p.yt = a.yt;
    p.row_off = 0;
    e = use_stream ? zq::launch_stream_single(p, m, s) : zq::launch_mstream_single(p, m, s);
  } else if (!asym && m <= 4 && aligned16 && zq::gemv_valu_lds_bytes(W->bits, m, W->k) <= 64 * 1024)
    e = zq::launch_gemv_valu(a);
  else if (use_prefill)
    e = zq::launch_gemm_prefill(a);
  else if (!asym && aligned16 && zq::gemm_mfma_supported(a))
    e = zq::launch_gemm_mfma(a);
  else
    e = zq::launch_gemm_general(a);
  return e == hipSuccess ? ok() : hip_fail(e, "gemm launch");
}

}  // extern "C"

struct zq_plan_s {
  zq::StreamPhase* segs = nullptr;     // device
  zq::StreamProblem* probs = nullptr;  // device
  int2* ranges = nullptr;              // device: [segment][workgroup] {first, last}
  uint32_t* sync = nullptr;            // device: counter, error word, finished workgroups
  int nseg = 0;
  bool waits = false;  // some segment waits for an earlier phase
  bool mfma = false;   // the MFMA batched-decode kernel (m >= MSTREAM_MIN_M)
  int64_t m = 1;
  int variant = 0;  // the kernel variant of the plan's one format, or the mixed-format one
  int grid = 0;     // workgroups of the launch (the ranges table has one entry per segment and workgroup)
  size_t lds = 0;
  // prefill plans (m > 16): one tile queue per bit width and group size, run
  // in turn
  static constexpr int PREFILL_KINDS = 6;
  bool prefill = false;
  zq::PrefillProblem* pprobs = nullptr;  // device, grouped by bit width and group size
  int xt = 0;
  int ngroup = 0;
  int gfirst[PREFILL_KINDS] = {}, gcount[PREFILL_KINDS] = {}, gbits[PREFILL_KINDS] = {}, ggroup[PREFILL_KINDS] = {};
  int64_t gtotal[PREFILL_KINDS] = {};  // tiles
  // mid-batch plans (32 < m): plans of at most 32 activation rows each, run in turn
  std::vector<zq_plan_s*> chunks;
};

namespace {
// products of segment `sg` touched by workgroup w of the launch's G: rows
// [w*N/Gs, (w+1)*N/Gs) for the Gs = sg.grid (or G) workgroups that share the
// segment, none for the others
void seg_ranges(const zq::StreamPhase& sg, const std::vector<zq::StreamProblem>& probs, int G,
                std::vector<int2>& out) {
  const int64_t N = sg.n_total;
  const int Gs = sg.grid > 0 && sg.grid < G ? sg.grid : G;
  int lo = 0;
  for (int w = 0; w < G; ++w) {
    const int64_t r0 = w * N / Gs, r1 = (w + 1) * N / Gs;
    if (w >= Gs || r1 == r0) {
      out.push_back(make_int2(0, 0));
      continue;
    }
    while (lo + 1 < sg.count && probs[sg.first + lo + 1].row_off <= r0) ++lo;
    int hi = lo;
    while (hi + 1 < sg.count && probs[sg.first + hi + 1].row_off < r1) ++hi;
    out.push_back(make_int2(lo, hi));
  }
}

// The products a prefill plan takes for 16 < m <= 64 (batched decode): valid
// weights, symmetric codes, one phase and activation type, the prefill
// kernel's shapes and alignment. Other lists go to the batched-decode
// kernel, which also takes several phases.
bool prefill_plannable(const zq_problem* problems, int count, int64_t m) {
  for (int i = 0; i < count; ++i) {
    const zq_problem& q = problems[i];
    if (check_weight(&q.w) || q.w.zeros || q.phase != problems[0].phase || q.x_dtype != problems[0].x_dtype ||
        (q.x_dtype != ZQ_F16 && q.x_dtype != ZQ_BF16) || q.ldx < q.w.k || q.ldy < q.w.n || q.w.n == 0 ||
        q.w.k == 0 || !q.x || !q.y)
      return false;
    zq::GemmArgs a{};
    a.packed = (const uint8_t*)q.w.packed;
    a.scales = q.w.scales;
    a.zeros = q.w.zeros;
    a.bits = q.w.bits;
    a.group = q.w.group;
    a.n = q.w.n;
    a.k = q.w.k;
    a.x = (const uint16_t*)q.x;
    a.m = m;
    a.ldx = q.ldx;
    if (!zq::gemm_prefill_supported(a)) return false;
  }
  return true;
}

// A prefill plan (m > 16): every product with symmetric codes, one scale per
// tensor (k a multiple of 64) or per row and 128 k, 16-byte aligned codes and
// activations, one activation type, one phase.
zq_status create_prefill_plan(const zq_problem* problems, int count, int64_t m, zq_plan* plan_out) {
  std::vector<zq::PrefillProblem> pp(count);
  std::vector<int> order(count);
  for (int i = 0; i < count; ++i) {
    const zq_problem& q = problems[i];
    zq_status st = check_weight(&q.w);
    if (st) return fail(st, "problem %d: %s", i, g_err);
    if (q.x_dtype != ZQ_F16 && q.x_dtype != ZQ_BF16)
      return fail(ZQ_ERR_INVALID_ARG, "problem %d: x_dtype must be F16 or BF16", i);
    if (q.y_dtype != ZQ_F32 && q.y_dtype != ZQ_F16 && q.y_dtype != ZQ_BF16)
      return fail(ZQ_ERR_INVALID_ARG, "problem %d: y_dtype must be F32, F16 or BF16", i);
    if (q.ldx < q.w.k || q.ldy < q.w.n) return fail(ZQ_ERR_INVALID_ARG, "problem %d: ldx < k or ldy < n", i);
    if (q.w.n == 0 || q.w.k == 0 || !q.x || !q.y)
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: empty shapes and null pointers are not planned", i);
    if (q.x_dtype != problems[0].x_dtype)
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: a prefill plan takes one activation type", i);
    if (q.phase != problems[0].phase)
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: a prefill plan has one phase", i);
    zq::GemmArgs a{};
    a.packed = (const uint8_t*)q.w.packed;
    a.scales = q.w.scales;
    a.zeros = q.w.zeros;
    a.bits = q.w.bits;
    a.group = q.w.group;
    a.n = q.w.n;
    a.k = q.w.k;
    a.x = (const uint16_t*)q.x;
    a.m = m;
    a.ldx = q.ldx;
    if (!zq::gemm_prefill_supported(a))
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: prefill plans need symmetric codes, k a multiple of 64 (of 128 "
                  "with group scales) and 16-byte aligned codes and activations", i);
    zq::PrefillProblem& p = pp[i];
    p = zq::PrefillProblem{};
    p.packed = a.packed;
    p.scales = a.scales;
    p.x = a.x;
    p.y = q.y;
    p.m = m;
    p.n = q.w.n;
    p.k = q.w.k;
    p.ldx = q.ldx;
    p.ldy = q.ldy;
    p.mtiles = (m + zq::prefill_tile_m(m) - 1) / zq::prefill_tile_m(m);
    p.bits = q.w.bits;
    p.group = q.w.group;
    p.yt = q.y_dtype == ZQ_F32 ? zq::YF32 : q.y_dtype == ZQ_F16 ? zq::YF16 : zq::YBF16;
    order[i] = i;
  }
  // one queue per bit width and group size (a kernel each); within it the
  // longest tiles first, so the last round of the queue is made of short ones
  std::stable_sort(order.begin(), order.end(), [&](int u, int v) {
    if (pp[u].bits != pp[v].bits) return pp[u].bits < pp[v].bits;
    if (pp[u].group != pp[v].group) return pp[u].group < pp[v].group;
    return pp[u].k > pp[v].k;
  });
  std::vector<zq::PrefillProblem> sorted(count);
  zq_plan_s* plan = new zq_plan_s;
  plan->prefill = true;
  plan->m = m;
  plan->xt = problems[0].x_dtype == ZQ_F16 ? zq::XF16 : zq::XBF16;
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    sorted[i] = pp[order[i]];
    if (i == 0 || sorted[i].bits != sorted[i - 1].bits || sorted[i].group != sorted[i - 1].group) {
      plan->gfirst[plan->ngroup] = i;
      plan->gbits[plan->ngroup] = sorted[i].bits;
      plan->ggroup[plan->ngroup] = sorted[i].group;
      ++plan->ngroup;
      total = 0;
    }
    sorted[i].tile0 = total;
    total += sorted[i].mtiles * ((sorted[i].n + zq::PREFILL_TILE_N - 1) / zq::PREFILL_TILE_N);
    plan->gcount[plan->ngroup - 1] += 1;
    plan->gtotal[plan->ngroup - 1] = total;
    if (total >= (int64_t)1 << 31) {
      delete plan;
      return fail(ZQ_ERR_UNSUPPORTED, "too many tiles in one plan");
    }
  }
  hipError_t e = hipMalloc(&plan->pprobs, sizeof(zq::PrefillProblem) * count);
  const size_t sync_bytes = zq_plan_s::PREFILL_KINDS * zq::PREFILL_SYNC_WORDS * sizeof(uint32_t);
  if (e == hipSuccess) e = hipMalloc(&plan->sync, sync_bytes);
  if (e == hipSuccess)
    e = hipMemcpy(plan->pprobs, sorted.data(), sizeof(zq::PrefillProblem) * count, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(plan->sync, 0, sync_bytes);
  if (e != hipSuccess) {
    (void)hipFree(plan->pprobs);
    (void)hipFree(plan->sync);
    delete plan;
    return hip_fail(e, "plan allocation");
  }
  *plan_out = plan;
  return ok();
}
}  // namespace

namespace {
// A mid-batch plan (32 < m <= 64, or asymmetric codes at any m > 32; INT4
// products the MFMA batched-decode kernel takes): the rows go in chunks of
// 32 (the last one shorter), each chunk a plan of its own over all products;
// the weights stream once per chunk.
zq_status create_chunked_plan(const zq_problem* problems, int count, int64_t m, zq_plan* plan_out) {
  for (int i = 0; i < count; ++i) {
    const zq_problem& q = problems[i];
    zq_status st = check_weight(&q.w);
    if (st) return fail(st, "problem %d: %s", i, g_err);
    if (!zq::mstream_supported(q.w.packed, q.w.scales, q.w.zeros, q.w.bits, q.w.group, 32, q.w.k, q.x, q.ldx))
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: plans with m > 32 need INT4 codes, k a multiple of 512, "
                  "16-byte aligned codes and activations and 8-byte aligned scales (for m > 64: symmetric "
                  "codes)", i);
  }
  zq_plan_s* plan = new zq_plan_s;
  plan->m = m;
  std::vector<zq_problem> sub(problems, problems + count);
  for (int64_t r0 = 0, mc = 0; r0 < m; r0 += mc) {
    mc = chunk_rows(m, r0);
    for (int i = 0; i < count; ++i) {
      const zq_problem& q = problems[i];
      const int ysz = q.y_dtype == ZQ_F32 ? 4 : 2;
      sub[i].x = (const uint16_t*)q.x + r0 * q.ldx;
      sub[i].y = (uint8_t*)q.y + r0 * q.ldy * ysz;
    }
    zq_plan c = nullptr;
    zq_status st = zq_plan_create(sub.data(), count, mc, &c);
    if (st) {
      char keep[sizeof g_err];
      memcpy(keep, g_err, sizeof keep);
      zq_plan_destroy(plan);
      return fail(st, "rows %lld..: %s", (long long)r0, keep);
    }
    plan->chunks.push_back(c);
  }
  *plan_out = plan;
  return ok();
}
}  // namespace

extern "C" {

zq_status zq_plan_create(const zq_problem* problems, int count, int64_t m, zq_plan* plan_out) {
  if (!plan_out) return fail(ZQ_ERR_INVALID_ARG, "null plan_out");
  *plan_out = nullptr;
  if (count < 1 || !problems) return fail(ZQ_ERR_INVALID_ARG, "empty problem list");
  if (m < 1) return fail(ZQ_ERR_UNSUPPORTED, "plans take m >= 1 (m=%lld)", (long long)m);
  if (m > 64) {
    // symmetric codes: the prefill tile queues
    bool prefill = true;
    for (int i = 0; i < count && prefill; ++i) prefill = !problems[i].w.zeros;
    if (prefill) return create_prefill_plan(problems, count, m, plan_out);
    return create_chunked_plan(problems, count, m, plan_out);
  }
  if (m > 32) {
    if (prefill_plannable(problems, count, m)) return create_prefill_plan(problems, count, m, plan_out);
    return create_chunked_plan(problems, count, m, plan_out);
  }
  // 16 < m <= 32: the batched-decode kernel when every product suits it,
  // else the prefill tiles when they take the list
  if (m > 16) {
    bool ms = true;
    for (int i = 0; i < count && ms; ++i) {
      const zq_problem& q = problems[i];
      ms = !check_weight(&q.w) &&
           zq::mstream_supported(q.w.packed, q.w.scales, q.w.zeros, q.w.bits, q.w.group, m, q.w.k, q.x, q.ldx);
    }
    if (!ms && prefill_plannable(problems, count, m)) return create_prefill_plan(problems, count, m, plan_out);
  }
  // the MFMA kernel when every product suits it; for m <= 4 the vector-ALU
  // kernel takes the other formats
  bool mfma = m >= zq::MSTREAM_MIN_M;
  if (mfma && m <= 4) {
    for (int i = 0; i < count && mfma; ++i) {
      const zq_problem& q = problems[i];
      mfma = zq::mstream_supported(q.w.packed, q.w.scales, q.w.zeros, q.w.bits, q.w.group, m, q.w.k, q.x, q.ldx);
    }
  }
  std::vector<zq::StreamProblem> probs(count);
  std::vector<zq::StreamPhase> segs;
  for (int i = 0; i < count; ++i) {
    const zq_problem& q = problems[i];
    zq_status st = check_weight(&q.w);
    if (st) return fail(st, "problem %d: %s", i, g_err);
    if (i > 0 && q.phase < problems[i - 1].phase)
      return fail(ZQ_ERR_INVALID_ARG, "problem %d: phases must not decrease", i);
    if (q.x_dtype != ZQ_F16 && q.x_dtype != ZQ_BF16)
      return fail(ZQ_ERR_INVALID_ARG, "problem %d: x_dtype must be F16 or BF16", i);
    if (q.y_dtype != ZQ_F32 && q.y_dtype != ZQ_F16 && q.y_dtype != ZQ_BF16)
      return fail(ZQ_ERR_INVALID_ARG, "problem %d: y_dtype must be F32, F16 or BF16", i);
    if (q.ldx < q.w.k || q.ldy < q.w.n) return fail(ZQ_ERR_INVALID_ARG, "problem %d: ldx < k or ldy < n", i);
    if (q.w.n == 0 || q.w.k == 0 || !q.x || !q.y)
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: empty shapes and null pointers are not planned", i);
    const bool aligned = ((uintptr_t)q.w.packed & 15) == 0 && ((uintptr_t)q.x & 15) == 0 &&
                         (m == 1 || (q.ldx * 2) % 16 == 0);
    if (mfma) {
      if (!zq::mstream_supported(q.w.packed, q.w.scales, q.w.zeros, q.w.bits, q.w.group, m, q.w.k, q.x, q.ldx))
        return fail(ZQ_ERR_UNSUPPORTED, "problem %d: plans with m > 4 need INT4 codes, k a multiple of 512, "
                    "16-byte aligned codes and activations and 8-byte aligned scales", i);
    } else if (!aligned || !zq::stream_supported(q.w.bits, q.w.group, m, q.w.n, q.w.k)) {
      return fail(ZQ_ERR_UNSUPPORTED, "problem %d: needs 16-byte alignment, k a multiple of 128 "
                  "and activations that fit in LDS", i);
    }
  }
  // Products of one phase do not depend on each other: order them by format
  // (activation type, bit width, scale group, zero points, then k from the
  // longest rows down), stably, so that each format of a phase is one
  // segment. Few large segments keep every workgroup's load pipeline full; a
  // segment boundary drains it. Short rows last: a segment of short rows is
  // bound by load latency, and starting the launch with it cost the
  // tensor-parallel 7B share 2 % (K = 896 first: 5205 GB/s; last: 5311).
  std::vector<int> order(count);
  for (int i = 0; i < count; ++i) order[i] = i;
  auto fmt_key = [&](int i) {
    const zq_problem& q = problems[i];
    return std::make_tuple(q.x_dtype, q.w.bits, q.w.group, q.w.zeros ? 1 : 0, -q.w.k);
  };
  for (int a = 0; a < count;) {
    int b = a + 1;
    while (b < count && problems[b].phase == problems[a].phase) ++b;
    std::stable_sort(order.begin() + a, order.begin() + b, [&](int u, int v) { return fmt_key(u) < fmt_key(v); });
    a = b;
  }
  for (int i = 0; i < count; ++i) {
    const zq_problem& q = problems[order[i]];
    const int xt = q.x_dtype == ZQ_F16 ? zq::XF16 : zq::XBF16;
    // a new segment when the phase or the format changes
    const bool same_phase = i > 0 && q.phase == problems[order[i - 1]].phase;
    bool new_segment = !same_phase;
    if (same_phase) {
      const zq::StreamPhase& sg = segs.back();
      new_segment = sg.k != q.w.k || sg.bits != q.w.bits || sg.group != q.w.group || sg.xt != xt ||
                    sg.asym != (q.w.zeros ? 1 : 0);
    }
    if (new_segment) {
      zq::StreamPhase sg{};
      sg.first = i;
      sg.k = q.w.k;
      sg.bits = q.w.bits;
      sg.group = q.w.group;
      sg.xt = xt;
      sg.asym = q.w.zeros ? 1 : 0;
      sg.wait = (i > 0 && !same_phase) ? 1 : 0;
      segs.push_back(sg);
    }
    zq::StreamPhase& sg = segs.back();
    zq::StreamProblem& p = probs[i];
    p = zq::StreamProblem{};
    p.packed = (const uint8_t*)q.w.packed;
    p.scales = q.w.scales;
    p.zeros = q.w.zeros;
    p.x = (const uint16_t*)q.x;
    p.y = q.y;
    p.n = q.w.n;
    p.k = q.w.k;
    p.ldx = q.ldx;
    p.ldy = q.ldy;
    p.row_off = sg.n_total;
    p.bits = q.w.bits;
    p.group = q.w.group;
    p.xt = xt;
    p.yt = q.y_dtype == ZQ_F32 ? zq::YF32 : q.y_dtype == ZQ_F16 ? zq::YF16 : zq::YBF16;
    sg.count += 1;
    sg.n_total += q.w.n;
  }
  // Workgroups: one per CU, fewer for plans whose largest segment is small.
  // Split segments whose workgroup ranges would stage too many activation
  // buffers for LDS: halve them (no wait between the halves) until they fit.
  int G = zq::stream_grid();
  if (!mfma) {
    G = 1;
    for (zq::StreamPhase& sg : segs) {
      sg.grid = zq::stream_grid_for(sg.bits, m, sg.n_total, sg.k);
      G = std::max(G, sg.grid);
    }
  }
  std::vector<zq::StreamPhase> fitted;
  std::vector<int2> ranges;
  size_t lds = 0;
  for (size_t si = 0; si < segs.size(); ++si) {
    std::vector<zq::StreamPhase> todo{segs[si]};
    while (!todo.empty()) {
      zq::StreamPhase sg = todo.back();
      todo.pop_back();
      // row offsets relative to this (possibly split) segment
      int64_t off = 0;
      for (int i = 0; i < sg.count; ++i) {
        probs[sg.first + i].row_off = off;
        off += probs[sg.first + i].n;
      }
      sg.n_total = off;
      if (!mfma) sg.grid = zq::stream_grid_for(sg.bits, m, sg.n_total, sg.k);
      std::vector<int2> r;
      seg_ranges(sg, probs, G, r);
      int maxrec = 1;
      for (const int2& v : r) maxrec = std::max(maxrec, v.y - v.x + 1);
      const size_t need = mfma ? zq::mstream_lds(m, maxrec) : zq::stream_lds_bytes(sg.bits, m, sg.k, maxrec);
      if (need > zq::STREAM_LDS_MAX) {
        if (sg.count == 1)
          return fail(ZQ_ERR_UNSUPPORTED, "problem %d needs %zu bytes of LDS (max %zu)", order[sg.first], need,
                      zq::STREAM_LDS_MAX);
        zq::StreamPhase a = sg, b = sg;
        a.count = sg.count / 2;
        b.first = sg.first + a.count;
        b.count = sg.count - a.count;
        b.wait = 0;
        todo.push_back(b);  // processed after a (stack order)
        todo.push_back(a);
        continue;
      }
      fitted.push_back(sg);
      ranges.insert(ranges.end(), r.begin(), r.end());
      lds = std::max(lds, need);
    }
  }
  int variant = -1;
  for (const zq::StreamPhase& sg : fitted) {
    const int v = mfma ? zq::mstream_variant_of(sg.xt, sg.group, sg.asym)
                       : zq::stream_variant_of(sg.xt, sg.bits, sg.group, sg.asym);
    variant = (variant == -1 || variant == v) ? v : (mfma ? zq::MSTREAM_VAR_ANY : zq::STREAM_VAR_ANY);
  }
  zq_plan_s* plan = new zq_plan_s;
  plan->nseg = (int)fitted.size();
  plan->m = m;
  plan->lds = lds;
  plan->grid = G;
  plan->variant = variant;
  for (const zq::StreamPhase& sg : fitted) plan->waits = plan->waits || sg.wait;
  plan->mfma = mfma;
  hipError_t e = hipMalloc(&plan->segs, sizeof(zq::StreamPhase) * fitted.size());
  if (e == hipSuccess) e = hipMalloc(&plan->probs, sizeof(zq::StreamProblem) * probs.size());
  if (e == hipSuccess) e = hipMalloc(&plan->ranges, sizeof(int2) * ranges.size());
  if (e == hipSuccess) e = hipMalloc(&plan->sync, 3 * sizeof(uint32_t));
  if (e == hipSuccess)
    e = hipMemcpy(plan->segs, fitted.data(), sizeof(zq::StreamPhase) * fitted.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(plan->probs, probs.data(), sizeof(zq::StreamProblem) * probs.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(plan->ranges, ranges.data(), sizeof(int2) * ranges.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(plan->sync, 0, 3 * sizeof(uint32_t));
  if (e != hipSuccess) {
    (void)hipFree(plan->segs);
    (void)hipFree(plan->probs);
    (void)hipFree(plan->ranges);
    (void)hipFree(plan->sync);
    delete plan;
    return hip_fail(e, "plan allocation");
  }
  *plan_out = plan;
  return ok();
}

zq_status zq_plan_run(zq_plan plan, void* stream) {
  if (!plan) return fail(ZQ_ERR_INVALID_ARG, "null plan");
  if (!plan->chunks.empty()) {
    for (zq_plan c : plan->chunks) {
      const zq_status st = zq_plan_run(c, stream);
      if (st) return st;
    }
    return ok();
  }
  if (plan->prefill) {
    hipError_t e = hipSuccess;
    for (int g = 0; g < plan->ngroup && e == hipSuccess; ++g)
      e = zq::launch_prefill_plan(plan->pprobs + plan->gfirst[g], plan->gcount[g], plan->gtotal[g], plan->xt,
                                  plan->gbits[g], plan->ggroup[g], plan->m, plan->sync + zq::PREFILL_SYNC_WORDS * g,
                                  (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "plan launch");
  }
  hipError_t e = plan->mfma
                     ? zq::launch_mstream_plan(plan->segs, plan->nseg, plan->probs, plan->ranges, plan->m,
                                               plan->variant, plan->lds, plan->sync, plan->waits, (hipStream_t)stream)
                     : zq::launch_stream_plan(plan->segs, plan->nseg, plan->probs, plan->ranges, plan->m,
                                              plan->variant, plan->lds, plan->sync, plan->waits, plan->grid,
                                              (hipStream_t)stream);
  return e == hipSuccess ? ok() : hip_fail(e, "plan launch");
}

zq_status zq_plan_check(zq_plan plan) {
  if (!plan) return fail(ZQ_ERR_INVALID_ARG, "null plan");
  for (zq_plan c : plan->chunks) {
    const zq_status st = zq_plan_check(c);
    if (st) return st;
  }
  if (!plan->chunks.empty()) return ok();
  uint32_t w[2] = {0, 0};
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(w, plan->sync, sizeof w, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "plan check");
  if (plan->prefill) return ok();  // no phase waits (its words are tile counters)
  if (w[1]) return fail(ZQ_ERR_HIP, "a phase wait gave up: outputs of that run are invalid");
  return ok();
}

zq_status zq_plan_destroy(zq_plan plan) {
  if (!plan) return ok();
  zq_status cst = ZQ_OK;
  for (zq_plan c : plan->chunks) {
    const zq_status st = zq_plan_destroy(c);
    if (st && !cst) cst = st;
  }
  if (!plan->chunks.empty()) {
    delete plan;
    return cst ? fail(cst, "plan destroy") : ok();
  }
  hipError_t e = hipDeviceSynchronize();
  hipError_t e1 = hipFree(plan->segs);
  if (e1 == hipSuccess) e1 = hipFree(plan->probs);
  if (e1 == hipSuccess) e1 = hipFree(plan->ranges);
  if (e1 == hipSuccess) e1 = hipFree(plan->pprobs);
  hipError_t e2 = hipFree(plan->sync);
  delete plan;
  if (e != hipSuccess) return hip_fail(e, "plan destroy sync");
  if (e1 != hipSuccess) return hip_fail(e1, "plan destroy");
  if (e2 != hipSuccess) return hip_fail(e2, "plan destroy");
  return ok();
}

zq_status zq_gemv(const zq_weight* W, const void* x, zq_dtype x_dtype, void* y, zq_dtype y_dtype,
                  void* stream) {
  zq_status st = check_weight(W);
  if (st) return st;
  return zq_gemm(W, x, x_dtype, 1, W->k, y, y_dtype, W->n, stream);
}

}  // extern "C"
