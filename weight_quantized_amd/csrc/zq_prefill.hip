// zq_prefill.hip -- host launchers of the prefill MFMA kernels (m > 64, one
// scale per tensor); tile and kernels in zq_prefill_impl.hpp.
#include "zq_prefill_impl.hpp"

namespace zq {

static const void* prefill_fn_for(int bits, int xt, bool plan) {
  return bits == 2 ? prefill_fn_b2(xt, plan) : bits == 4 ? prefill_fn_b4(xt, plan) : prefill_fn_b8(xt, plan);
}

// The tile addresses its activations and codes through 32-bit buffer
// offsets from the tile's first row: 256 rows of either must stay below 4 GB.
bool gemm_prefill2_supported(const GemmArgs& a) {
  if (a.group != 0 || a.m <= 64 || a.k % PF_BK != 0 || a.k == 0) return false;
  if (((uintptr_t)a.x & 15) || ((a.ldx * 2) & 15) || ((uintptr_t)a.packed & 15)) return false;
  if ((int64_t)PF_BM * a.ldx * 2 >= ((int64_t)1 << 32) || (int64_t)PF_BN * a.k * a.bits / 8 >= ((int64_t)1 << 32))
    return false;
  return true;
}

bool prefill_plan_supported(const GemmArgs& a) { return a.zeros == nullptr && gemm_prefill2_supported(a); }

hipError_t launch_gemm_prefill2(const GemmArgs& a) {
  const void* fn = prefill_fn_for(a.bits, a.xt, false);
  const int lds = pf_lds(a.bits);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int mtiles = (int)((a.m + PF_BM - 1) / PF_BM);
  const int64_t tiles = (int64_t)mtiles * ((a.n + PF_BN - 1) / PF_BN);
  const uint8_t* packed = a.packed;
  const uint16_t* scales = a.scales;
  int64_t n = a.n, k = a.k, m = a.m, ldx = a.ldx, ldy = a.ldy;
  const uint16_t* x = a.x;
  void* y = a.y;
  int yt = a.yt;
  void* args[] = {&packed, &scales, &n, &k, &x, &m, &ldx, &y, &ldy, &yt, &mtiles};
  return hipLaunchKernel(fn, dim3((unsigned)tiles), dim3(256), args, lds, a.stream);
}

hipError_t launch_prefill_plan(const PrefillProblem* dev_probs, int nprob, int64_t total, int xt, int bits,
                               uint32_t* sync, hipStream_t stream) {
  const void* fn = prefill_fn_for(bits, xt, true);
  const int lds = pf_lds(bits);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int64_t G = std::min<int64_t>(stream_grid(), total);
  void* args[] = {(void*)&dev_probs, &nprob, &total, &sync};
  return hipLaunchKernel(fn, dim3((unsigned)G), dim3(256), args, lds, stream);
}

}  // namespace zq
