// Placeholder: linear-layer kernels land in the next commit.
#include "common.hpp"
#include "kernels.hpp"

namespace qlora {
size_t fwd_workspace_bytes(int64_t, int64_t, int64_t, int32_t) { return 0; }
size_t bwd_workspace_bytes(int64_t, int64_t, int64_t, int32_t) { return 0; }
hipError_t launch_linear_fwd(const LinearArgs&, const Codebook&, const uint16_t*, uint16_t*, float*, void*,
                             hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_linear_bwd(const LinearArgs&, const Codebook&, const uint16_t*, const uint16_t*, const float*,
                             uint16_t*, uint16_t*, uint16_t*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace qlora
