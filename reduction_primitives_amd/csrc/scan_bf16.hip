// scan_bf16.hip -- scan kernels instantiated for one input dtype (bf16).
#define RK_UNIT unit_scan_bf16
#include "rk_scan.hpp"

namespace rk {
int launch_scan_in_bf16(const ScanLaunch &L) { return run_scan_in<bf16_in>(L); }
}  // namespace rk
