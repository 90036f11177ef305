// kern_f64.hip -- kernels instantiated for one input dtype (f64); each input
// dtype has its own translation unit so the library builds in parallel.
#define RK_UNIT unit_kern_f64
#include "rk_kernels.hpp"

namespace rk {
int launch_in_f64(const Launch &L) { return run_in<double>(L); }
}  // namespace rk
