// zq_mstream_t1.hip -- instantiations of the persistent MFMA batched-decode
// kernel with 1 tile(s) of 16 activation rows (one translation unit each
// keeps builds parallel).
#include "zq_mstream_impl.hpp"

namespace zq {
const void* mstream_kernel_t1(int var) { return mstream_fn_var<1>(var); }
}  // namespace zq
