// scan_i64.hip -- scan kernels instantiated for one input dtype (i64).
#define RK_UNIT unit_scan_i64
#include "rk_scan.hpp"

namespace rk {
int launch_scan_in_i64(const ScanLaunch &L) { return run_scan_in<int64_t>(L); }
}  // namespace rk
