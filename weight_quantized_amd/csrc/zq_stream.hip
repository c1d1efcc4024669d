// zq_stream.hip -- host launchers of the persistent decode kernel (kernel
// templates in zq_stream_impl.hpp, instantiated in zq_stream_m1..m4.hip).
#include "zq_stream_impl.hpp"

namespace zq {

int stream_grid() { return device_info().num_cus; }

int stream_grid_for(int bits, int64_t m, int64_t n, int64_t k) {
  const int64_t steps = (n + 3) / 4 * ((k / (128 / bits) + 15) / 16);  // quad-steps of the segment
  const int64_t waves = m == 1 ? 16 : 8;
  const int64_t g = (steps + waves - 1) / waves;
  return (int)(g < 1 ? 1 : g < stream_grid() ? g : stream_grid());
}

int stream_variant_of(int xt, int bits, int group, int asym) { return stream_variant(xt, bits, group, asym); }
static_assert(VAR_ANY == STREAM_VAR_ANY, "variant numbering");

size_t stream_lds_bytes(int bits, int64_t m, int64_t k, int nrec) { return stream_seg_lds(bits, m, k, nrec); }

bool stream_supported(int bits, int group, int64_t m, int64_t n, int64_t k) {
  (void)group;
  (void)n;
  if (m < 1 || m > 4 || k % 128 != 0 || k == 0) return false;  // whole 128-groups; a row's last step may be partial
  return stream_seg_lds(bits, m, k, 1) <= STREAM_LDS_MAX;
}

static const void* stream_kernel_for(int64_t m, int var) {
  switch (m) {
    case 1: return stream_kernel_m1(var);
    case 2: return stream_kernel_m2(var);
    case 3: return stream_kernel_m3(var);
    default: return stream_kernel_m4(var);
  }
}

static hipError_t ensure_lds_attr(const void* fn, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_stream_single(const StreamProblem& p, int64_t m, hipStream_t stream) {
  StreamPhase seg{};
  seg.first = 0;
  seg.count = 1;
  seg.n_total = p.n;
  seg.k = p.k;
  seg.bits = p.bits;
  seg.group = p.group;
  seg.xt = p.xt;
  StreamProblem pp = p;
  pp.row_off = 0;
  seg.asym = p.zeros ? 1 : 0;
  seg.grid = stream_grid_for(p.bits, m, p.n, p.k);
  const void* fn = stream_kernel_for(m, stream_variant(p.xt, p.bits, p.group, seg.asym));
  const size_t lds = stream_seg_lds(p.bits, m, p.k, 1);
  hipError_t e = ensure_lds_attr(fn, lds);
  if (e != hipSuccess) return e;
  const StreamPhase* none = nullptr;
  const StreamProblem* noprobs = nullptr;
  const int2* noranges = nullptr;
  int nseg = 1;
  uint32_t* nosync = nullptr;
  void* args[] = {&none, &nseg, &noprobs, &noranges, &seg, &pp, &nosync};
  return hipLaunchKernel(fn, dim3(seg.grid), dim3(m == 1 ? 1024 : 512), args, lds, stream);
}

hipError_t launch_stream_plan(const StreamPhase* dev_segs, int nseg, const StreamProblem* dev_probs,
                              const int2* dev_ranges, int64_t m, int variant, size_t lds, uint32_t* sync,
                              bool waits, int grid_size, hipStream_t stream) {
  const void* fn = stream_kernel_for(m, variant);
  hipError_t e = ensure_lds_attr(fn, lds);
  if (e != hipSuccess) return e;
  StreamPhase dseg{};
  StreamProblem dpr{};
  void* args[] = {(void*)&dev_segs, &nseg, (void*)&dev_probs, (void*)&dev_ranges, &dseg, &dpr, &sync};
  const dim3 grid(grid_size), block(m == 1 ? 1024 : 512);
  // workgroups wait for each other only across phases: only then must they
  // all be resident at once
  if (waits) return hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)lds, stream);
  return hipLaunchKernel(fn, grid, block, args, lds, stream);
}

}  // namespace zq
