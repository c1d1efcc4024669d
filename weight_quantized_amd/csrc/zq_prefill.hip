// zq_prefill.hip -- host launchers of the prefill MFMA kernels (m > 64, one
// scale per tensor or per row and 128 k); tile and kernels in
// zq_prefill_impl.hpp.
#include "zq_prefill_impl.hpp"

namespace zq {

static_assert(PREFILL_TILE_M == PF_BM && PREFILL_TILE_N == PF_BN, "plan tiles are the kernel's");

static const void* prefill_fn_for(int bits, int xt, bool plan, bool gs) {
  return bits == 2 ? prefill_fn_b2(xt, plan, gs) : bits == 4 ? prefill_fn_b4(xt, plan, gs)
                                                             : prefill_fn_b8(xt, plan, gs);
}

// The tile addresses its activations and codes through 32-bit buffer
// offsets from the tile's first row: 128 rows of activations and 256 rows of
// codes must stay below 4 GB. A single call's grid is (row blocks, column
// blocks): at most 65535 column blocks.
bool gemm_prefill_supported(const GemmArgs& a) {
  if (a.zeros != nullptr || a.m <= 64 || a.k == 0) return false;
  if (a.group == 0 ? a.k % PF_BK != 0 : (a.group != PF_GROUP || a.k % PF_GROUP != 0)) return false;
  if (((uintptr_t)a.x & 15) || ((a.ldx * 2) & 15) || ((uintptr_t)a.packed & 15) || ((uintptr_t)a.scales & 1))
    return false;
  if ((int64_t)PF_BM * a.ldx * 2 >= ((int64_t)1 << 32) || (int64_t)PF_BN * a.k * a.bits / 8 >= ((int64_t)1 << 32))
    return false;
  return (a.n + PF_BN - 1) / PF_BN <= 65535 && (a.m + PF_BM - 1) / PF_BM < ((int64_t)1 << 31);
}

static hipError_t set_lds(const void* fn, int lds) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

hipError_t launch_gemm_prefill(const GemmArgs& a) {
  const void* fn = prefill_fn_for(a.bits, a.xt, false, a.group != 0);
  const int lds = pf_lds(a.bits);
  hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  const int64_t mtiles = (a.m + PF_BM - 1) / PF_BM, ntiles = (a.n + PF_BN - 1) / PF_BN;
  const uint8_t* packed = a.packed;
  const uint16_t* scales = a.scales;
  int64_t n = a.n, k = a.k, m = a.m, ldx = a.ldx, ldy = a.ldy;
  const uint16_t* x = a.x;
  void* y = a.y;
  int yt = a.yt;
  void* args[] = {&packed, &scales, &n, &k, &x, &m, &ldx, &y, &ldy, &yt};
  return hipLaunchKernel(fn, dim3((unsigned)mtiles, (unsigned)ntiles), dim3(256), args, lds, a.stream);
}

// two workgroups per CU stay resident (LDS and registers are sized for it)
hipError_t launch_prefill_plan(const PrefillProblem* dev_probs, int nprob, int64_t total, int xt, int bits,
                               int group, uint32_t* sync, hipStream_t stream) {
  const void* fn = prefill_fn_for(bits, xt, true, group != 0);
  const int lds = pf_lds(bits);
  hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  const int64_t G = std::min<int64_t>(2 * (int64_t)stream_grid(), total);
  void* args[] = {(void*)&dev_probs, &nprob, &total, &sync};
  return hipLaunchKernel(fn, dim3((unsigned)G), dim3(256), args, lds, stream);
}

}  // namespace zq
