// kern_f16.hip -- kernels instantiated for one input dtype (f16); each input
// dtype has its own translation unit so the library builds in parallel.
#define RK_UNIT unit_kern_f16
#include "rk_kernels.hpp"

namespace rk {
int launch_in_f16(const Launch &L) { return run_in<f16_in>(L); }
}  // namespace rk
