// kern_f32.hip -- kernels instantiated for one input dtype (f32); each input
// dtype has its own translation unit so the library builds in parallel.
#define RK_UNIT unit_kern_f32
#include "rk_kernels.hpp"

namespace rk {
int launch_in_f32(const Launch &L) { return run_in<float>(L); }
}  // namespace rk
