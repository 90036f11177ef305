// kern_i64.hip -- kernels instantiated for one input dtype (i64); each input
// dtype has its own translation unit so the library builds in parallel.
#define RK_UNIT unit_kern_i64
#include "rk_kernels.hpp"

namespace rk {
int launch_in_i64(const Launch &L) { return run_in<int64_t>(L); }
}  // namespace rk
