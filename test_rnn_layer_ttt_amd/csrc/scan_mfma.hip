// MFMA chunk scan (d = 64).  Not built yet: every call goes to the VALU scan.
#include "scan_common.h"

namespace ttt {
bool scan_mfma_supports(const ScanArgs&) { return false; }
hipError_t launch_scan_mfma(const ScanArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
