// MXFP8 grouped GEMMs (placeholder until the scaled-MFMA kernels land).
#include "kernels.h"

namespace moe {
hipError_t launch_mx_gateup(const MxArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mx_down(const MxArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace moe
