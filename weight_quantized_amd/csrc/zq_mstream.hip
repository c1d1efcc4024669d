// zq_mstream.hip -- host launchers of the persistent MFMA batched-decode
// kernel (templates in zq_mstream_impl.hpp, instantiated in
// zq_mstream_t1.hip and zq_mstream_t2.hip).
#include "zq_mstream_impl.hpp"

namespace zq {

bool mstream_supported(const void* packed, const uint16_t* scales, const uint16_t* zeros, int bits, int group,
                       int64_t m, int64_t k, const void* x, int64_t ldx) {
  if (bits != 4 || m < 2 || m > 32 || k <= 0 || k % MS_KC != 0) return false;
  // buffer descriptors and 32-bit signed offsets: a 512-row block of codes
  // and the m activation rows stay below 2 GB
  if (2 * MS_HALF * (k / 2) >= ((int64_t)1 << 31) || m * ldx * 2 >= ((int64_t)1 << 31)) return false;
  if (((uintptr_t)packed & 15) || ((uintptr_t)x & 15) || ((ldx * 2) & 15)) return false;
  if (group && ((uintptr_t)scales & 7)) return false;
  if (zeros && (!group || ((uintptr_t)zeros & 7))) return false;
  return mstream_lds(m, 1) <= STREAM_LDS_MAX;
}

size_t mstream_lds(int64_t m, int nrec) { return mstream_lds_bytes(m <= 16 ? 1 : 2, nrec); }

int mstream_variant_of(int xt, int group, int asym) { return mstream_variant(xt, group, asym); }
static_assert(MVAR_ANY == MSTREAM_VAR_ANY, "the host and the kernels agree on the mixed-format variant");

static const void* mstream_kernel_for(int64_t m, int var) {
  return m <= 16 ? mstream_kernel_t1(var) : mstream_kernel_t2(var);
}

static hipError_t ms_lds_attr(const void* fn, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_mstream_single(const StreamProblem& p, int64_t m, hipStream_t stream) {
  StreamPhase seg{};
  seg.first = 0;
  seg.count = 1;
  seg.n_total = p.n;
  seg.k = p.k;
  seg.bits = p.bits;
  seg.group = p.group;
  seg.xt = p.xt;
  seg.asym = p.zeros ? 1 : 0;
  StreamProblem pp = p;
  pp.row_off = 0;
  const void* fn = mstream_kernel_for(m, mstream_variant(p.xt, p.group, seg.asym));
  const size_t lds = mstream_lds(m, 1);
  hipError_t e = ms_lds_attr(fn, lds);
  if (e != hipSuccess) return e;
  // one 16-row tile per workgroup at least; at most one workgroup per CU
  const int64_t tiles = (p.n + 15) / 16;
  const int grid = (int)(tiles < stream_grid() ? tiles : stream_grid());
  const StreamPhase* none = nullptr;
  const StreamProblem* noprobs = nullptr;
  const int2* noranges = nullptr;
  int nseg = 1;
  uint32_t* nosync = nullptr;
  int mi = (int)m;
  void* args[] = {&none, &nseg, &noprobs, &noranges, &seg, &pp, &nosync, &mi};
  return hipLaunchKernel(fn, dim3(grid), dim3(m <= 16 ? ms_threads<1>() : ms_threads<2>()), args, lds, stream);
}

hipError_t launch_mstream_plan(const StreamPhase* dev_segs, int nseg, const StreamProblem* dev_probs,
                               const int2* dev_ranges, int64_t m, int variant, size_t lds, uint32_t* sync,
                               bool waits, hipStream_t stream) {
  const void* fn = mstream_kernel_for(m, variant);
  hipError_t e = ms_lds_attr(fn, lds);
  if (e != hipSuccess) return e;
  StreamPhase dseg{};
  StreamProblem dpr{};
  int mi = (int)m;
  void* args[] = {(void*)&dev_segs, &nseg, (void*)&dev_probs, (void*)&dev_ranges, &dseg, &dpr, &sync, &mi};
  const dim3 grid(stream_grid()), block(m <= 16 ? ms_threads<1>() : ms_threads<2>());
  if (waits) return hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)lds, stream);
  return hipLaunchKernel(fn, grid, block, args, lds, stream);
}

}  // namespace zq
