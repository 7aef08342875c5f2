// Stand-ins for the HIP kernel launchers, for the host-only build of the
// library that the sanitizer test compiles with g++ (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code: argument validation, the
// scheduler, the NSP planner).  Reaching a launcher there means a call got
// past validation on a machine without the kernels: it reports failure.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace vl {

hipError_t launch_sp_permute(const void*, void*, int64_t, int32_t, int32_t, int32_t, int32_t, int,
                             hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_sp_qkv(const QkvTensors&, int64_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                         int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_mfma_probe(int32_t, int32_t, float*, hipStream_t) { return hipErrorNotSupported; }
int64_t mfma_probe_flops(int32_t iters, int32_t n_wg) {
  return int64_t(iters) * int64_t(n_wg);
}
hipError_t launch_lse_merge(int32_t, const void* const*, const float* const*, int32_t, int64_t,
                            int32_t, int32_t, void*, float*, int32_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attn_fwd(const AttnShape&, const void*, const void*, const void*, const ItemMap&,
                           int32_t, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_attn_bwd(const AttnShape&, const void*, const void*, const void*, const void*,
                           const void*, const float*, const ItemMap&, const ItemMap&, int32_t,
                           void*, void*, void*, float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t noalloc_scratch(void**) { return hipErrorNotSupported; }

}  // namespace vl
