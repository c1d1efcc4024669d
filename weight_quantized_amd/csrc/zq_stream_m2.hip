// zq_stream_m2.hip -- instantiations of the persistent decode kernel for
// 2 activation rows (one translation unit per row count keeps builds parallel).
#include "zq_stream_impl.hpp"

namespace zq {
const void* stream_kernel_m2(int var) { return stream_fn_var<2>(var); }
}  // namespace zq
