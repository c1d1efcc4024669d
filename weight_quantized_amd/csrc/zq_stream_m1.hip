// zq_stream_m1.hip -- instantiations of the persistent decode kernel for
// 1 activation row (one translation unit per row count keeps builds parallel).
#include "zq_stream_impl.hpp"

namespace zq {
const void* stream_kernel_m1(int var) { return stream_fn_var<1>(var); }
}  // namespace zq
