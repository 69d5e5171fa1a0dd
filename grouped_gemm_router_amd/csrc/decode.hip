// Small-token expert MLP (placeholder: runs the general grouped GEMMs).
#include "kernels.h"

namespace moe {
hipError_t launch_decode_mlp(const GemmArgs& a, hipStream_t s) {
  hipError_t e = launch_fwd_gateup(a, s);
  if (e == hipSuccess) e = launch_fwd_down(a, s);
  return e;
}
}  // namespace moe
