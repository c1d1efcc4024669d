// zq_prefill_b8.hip -- the prefill kernels for 8-bit codes (one translation unit per
// bit width, so the builds run in parallel)
#include "zq_prefill_impl.hpp"

namespace zq {
const void* prefill_fn_b8(int xt, bool plan, bool gs, int fi) { return prefill_fn<8>(xt, plan, gs, fi); }
}  // namespace zq
