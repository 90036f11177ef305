// scan_i32.hip -- scan kernels instantiated for one input dtype (i32).
#define RK_UNIT unit_scan_i32
#include "rk_scan.hpp"

namespace rk {
int launch_scan_in_i32(const ScanLaunch &L) { return run_scan_in<int32_t>(L); }
}  // namespace rk
