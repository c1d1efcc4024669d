// zq_api.hip -- the C-ABI of libzq.so (declared in include/zq.h): argument
// validation, kernel choice and error reporting. Every check runs before the
// first HIP call, so invalid calls never touch the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/zq.h"
#include "zq_device.hpp"
#include "zq_internal.hpp"

namespace {

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
  return ZQ_OK;
}

std::mutex g_dev_mu;
std::vector<zq::DeviceInfo> g_devs;

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
  zq_status st = check_format(bits, group, n, k);
  if (st) return st;
  if (w_dtype != ZQ_I8 && w_dtype != ZQ_F16 && w_dtype != ZQ_BF16 && w_dtype != ZQ_F32)
    return fail(ZQ_ERR_INVALID_ARG, "w_dtype=%d not accepted", (int)w_dtype);
  const bool empty = n == 0 || k == 0;
  if (!empty && (!w || !packed_out)) return fail(ZQ_ERR_INVALID_ARG, "null w or packed_out");
  if (w_dtype != ZQ_I8 && !scales_in && !scales_out)
    return fail(ZQ_ERR_INVALID_ARG, "float weights need scales_in or scales_out");
  hipStream_t s = (hipStream_t)stream;
  const int64_t ns = zq_num_scales(group, n, k);
  hipError_t e;
  if (scales_in && scales_out && scales_in != scales_out && ns > 0) {
    e = hipMemcpyAsync(scales_out, scales_in, (size_t)ns * 2, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "copy scales");
  }
  if (empty) {
    if (w_dtype != ZQ_I8 && !scales_in && ns > 0) {
      // an empty tensor has absmax 0: its scales are +0
      e = hipMemsetAsync(scales_out, 0, (size_t)ns * 2, s);
      if (e != hipSuccess) return hip_fail(e, "zero scales");
    }
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
  a.group = group;
  a.scales = scales_in ? scales_in : scales_out;
  a.packed = (uint8_t*)packed_out;
  a.flags = flags;
  a.stream = s;
  uint32_t host_flags[2] = {0, 0};
  e = hipMemsetAsync(flags, 0, 2 * sizeof(uint32_t), s);
  if (e == hipSuccess && w_dtype != ZQ_I8 && !scales_in) e = zq::launch_compute_scales(a, scales_out);
  if (e == hipSuccess) e = zq::launch_quantize_pack(a);
  if (e == hipSuccess) e = hipMemcpyAsync(host_flags, flags, sizeof host_flags, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipError_t ef = hipFree(flags);
  if (e != hipSuccess) return hip_fail(e, "pack");
  if (ef != hipSuccess) return hip_fail(ef, "hipFree flags");
  if (host_flags[0] & zq::FLAG_NONFINITE) return fail(ZQ_ERR_RANGE, "non-finite weight or scale");
  if (host_flags[0] & zq::FLAG_SCALE_RANGE) return fail(ZQ_ERR_RANGE, "scale beyond the fp16 range");
  if (host_flags[0] & zq::FLAG_CODE_RANGE) return fail(ZQ_ERR_RANGE, "code outside the %d-bit range", bits);
  return ok();
}

zq_status zq_unpack(const zq_weight* W, void* out, zq_dtype out_dtype, void* stream) {
  zq_status st = check_weight(W);
  if (st) return st;
  if (out_dtype != ZQ_I8 && out_dtype != ZQ_F16 && out_dtype != ZQ_BF16 && out_dtype != ZQ_F32)
    return fail(ZQ_ERR_INVALID_ARG, "out_dtype=%d not accepted", (int)out_dtype);
  if (W->n > 0 && W->k > 0 && !out) return fail(ZQ_ERR_INVALID_ARG, "null out");
  hipError_t e = zq::launch_unpack((const uint8_t*)W->packed, W->scales, W->bits, W->group, W->n,
                                   W->k, out, (int)out_dtype, (hipStream_t)stream);
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
  if (m <= 4 && aligned16 && zq::gemv_valu_lds_bytes(W->bits, m, W->k) <= 64 * 1024)
    e = zq::launch_gemv_valu(a);
  else if (aligned16 && zq::gemm_mfma_supported(a))
    e = zq::launch_gemm_mfma(a);
  else
    e = zq::launch_gemm_general(a);
  return e == hipSuccess ? ok() : hip_fail(e, "gemm launch");
}

zq_status zq_gemv(const zq_weight* W, const void* x, zq_dtype x_dtype, void* y, zq_dtype y_dtype,
                  void* stream) {
  zq_status st = check_weight(W);
  if (st) return st;
  return zq_gemm(W, x, x_dtype, 1, W->k, y, y_dtype, W->n, stream);
}

}  // extern "C"
