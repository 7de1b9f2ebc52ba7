// The vector-ALU backward's entry, for the dispatcher.
#pragma once

#include "scan_common.h"

namespace ttt {

// Backward of the scan on the vector ALUs: d in {16, 32, 64, 128}, the
// per-token modes and the dual form with any chunk length, from the record of
// either forward kernel (delta_t of every token and the running W before every
// kRecTile-th token); hipErrorNotSupported for any other d.
hipError_t launch_bwd_valu(const BwdArgs& a, hipStream_t stream);

}  // namespace ttt
