// scan_f16.hip -- scan kernels instantiated for one input dtype (f16).
#define RK_UNIT unit_scan_f16
#include "rk_scan.hpp"

namespace rk {
int launch_scan_in_f16(const ScanLaunch &L) { return run_scan_in<f16_in>(L); }
}  // namespace rk
