// scan_f32.hip -- scan kernels instantiated for one input dtype (f32).
#define RK_UNIT unit_scan_f32
#include "rk_scan.hpp"

namespace rk {
int launch_scan_in_f32(const ScanLaunch &L) { return run_scan_in<float>(L); }
}  // namespace rk
