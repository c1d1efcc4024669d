// zq_stream_m3.hip -- instantiations of the persistent decode kernel for
// 3 activation rows (one translation unit per row count keeps builds parallel).
#include "zq_stream_impl.hpp"

namespace zq {
const void* stream_kernel_m3(int var) { return stream_fn_var<3>(var); }
}  // namespace zq
