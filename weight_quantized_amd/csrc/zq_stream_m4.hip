// zq_stream_m4.hip -- instantiations of the persistent decode kernel for
// 4 activation rows (one translation unit per row count keeps builds parallel).
#include "zq_stream_impl.hpp"

namespace zq {
const void* stream_kernel_m4(int var) { return stream_fn_var<4>(var); }
}  // namespace zq
