// zq_prefill.hip -- host launchers of the prefill MFMA kernels (m > 16, one
// scale per tensor or per row and 128 k); tile and kernels in
// zq_prefill_impl.hpp.
#include "zq_prefill_impl.hpp"

namespace zq {

static_assert(PREFILL_TILE_N == PF_BN, "plan tiles are the kernel's");

static const void* prefill_fn_for(int bits, int xt, bool plan, bool gs, int fi) {
  return bits == 2 ? prefill_fn_b2(xt, plan, gs, fi) : bits == 4 ? prefill_fn_b4(xt, plan, gs, fi)
                                                                 : prefill_fn_b8(xt, plan, gs, fi);
}

int prefill_tile_m(int64_t m) { return pf_bm(pf_fi(m)); }

// The tile addresses its activations and codes through 32-bit buffer
// offsets from the tile's first row: a tile's rows of activations and 256
// rows of codes must stay below 4 GB. A single call's grid is (row blocks,
// column blocks): at most 65535 column blocks.
bool gemm_prefill_supported(const GemmArgs& a) {
  if (a.zeros != nullptr || a.m <= 16 || a.k == 0) return false;
  if (a.group == 0 ? a.k % PF_BK != 0 : (a.group != PF_GROUP || a.k % PF_GROUP != 0)) return false;
  if (((uintptr_t)a.x & 15) || ((a.ldx * 2) & 15) || ((uintptr_t)a.packed & 15) || ((uintptr_t)a.scales & 1))
    return false;
  const int64_t bm = prefill_tile_m(a.m);
  if (bm * a.ldx * 2 >= ((int64_t)1 << 32) || (int64_t)PF_BN * a.k * a.bits / 8 >= ((int64_t)1 << 32)) return false;
  return (a.n + PF_BN - 1) / PF_BN <= 65535 && (a.m + bm - 1) / bm < ((int64_t)1 << 31);
}

static hipError_t set_lds(const void* fn, int lds) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

hipError_t launch_gemm_prefill(const GemmArgs& a) {
  const int fi = pf_fi(a.m);
  const void* fn = prefill_fn_for(a.bits, a.xt, false, a.group != 0, fi);
  const int lds = pf_lds(a.bits, fi);
  hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  const int64_t mtiles = (a.m + pf_bm(fi) - 1) / pf_bm(fi), ntiles = (a.n + PF_BN - 1) / PF_BN;
  const uint8_t* packed = a.packed;
  const uint16_t* scales = a.scales;
  int64_t n = a.n, k = a.k, m = a.m, ldx = a.ldx, ldy = a.ldy;
  const uint16_t* x = a.x;
  void* y = a.y;
  int yt = a.yt;
  void* args[] = {&packed, &scales, &n, &k, &x, &m, &ldx, &y, &ldy, &yt};
  return hipLaunchKernel(fn, dim3((unsigned)mtiles, (unsigned)ntiles), dim3(256), args, lds, a.stream);
}

// as many workgroups as stay resident (LDS and registers are sized for
// pf_wpc per CU)
hipError_t launch_prefill_plan(const PrefillProblem* dev_probs, int nprob, int64_t total, int xt, int bits,
                               int group, int64_t m, uint32_t* sync, hipStream_t stream) {
  const int fi = pf_fi(m);
  const void* fn = prefill_fn_for(bits, xt, true, group != 0, fi);
  const int lds = pf_lds(bits, fi);
  hipError_t e = set_lds(fn, lds);
  if (e != hipSuccess) return e;
  const int64_t G = std::min<int64_t>((int64_t)pf_wpc(bits, fi) * stream_grid(), total);
  void* args[] = {(void*)&dev_probs, &nprob, &total, &sync};
  return hipLaunchKernel(fn, dim3((unsigned)G), dim3(256), args, lds, stream);
}

}  // namespace zq
