// Matrix-core dual-form chunk scan with the two-layer inner model (gfx950).
#include "scan_common.h"

namespace ttt {

bool mlp_mfma_supports(const ScanArgs&) { return false; }

hipError_t launch_mlp_mfma(const ScanArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ttt
