// kern_i32.hip -- kernels instantiated for one input dtype (i32); each input
// dtype has its own translation unit so the library builds in parallel.
#define RK_UNIT unit_kern_i32
#include "rk_kernels.hpp"

namespace rk {
int launch_in_i32(const Launch &L) { return run_in<int32_t>(L); }
}  // namespace rk
