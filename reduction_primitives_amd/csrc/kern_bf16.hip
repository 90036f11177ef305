// kern_bf16.hip -- kernels instantiated for one input dtype (bf16); each input
// dtype has its own translation unit so the library builds in parallel.
#define RK_UNIT unit_kern_bf16
#include "rk_kernels.hpp"

namespace rk {
int launch_in_bf16(const Launch &L) { return run_in<bf16_in>(L); }
}  // namespace rk
