// zq_prefill_b2.hip -- the prefill kernels for 2-bit codes (one translation unit per
// bit width, so the builds run in parallel)
#include "zq_prefill_impl.hpp"

namespace zq {
const void* prefill_fn_b2(int xt, bool plan, bool gs, int fi) { return prefill_fn<2>(xt, plan, gs, fi); }
}  // namespace zq
