// scan_f64.hip -- scan kernels instantiated for one input dtype (f64).
#define RK_UNIT unit_scan_f64
#include "rk_scan.hpp"

namespace rk {
int launch_scan_in_f64(const ScanLaunch &L) { return run_scan_in<double>(L); }
}  // namespace rk
