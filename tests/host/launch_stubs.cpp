// Kernel-launch entry points for the host-only build of the library (tests/test_host_build.py): the C ABI
// layer (aah_api.cpp) and the planner (workplan.cpp) compiled by a plain C++ compiler, with sanitizers,
// and linked against these instead of the HIP kernels.  Every launch reports that no device is present, so
// a call that passes its argument checks fails with AAH_ERR_HIP, exactly as the real library does on a
// machine without a GPU; the validation and planning code under test runs unchanged.
#include <hip/hip_runtime_api.h>

#include "kernels.hpp"

namespace aah {

int fwd_bf16_resident(int) { return 0; }
int bwd_dq_resident(int) { return 0; }
int bwd_dkdv_resident(int) { return 0; }

hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, float*, float*, float*, const WorkItem*, int,
                           const int32_t*, const int32_t*, const AttnShape&, const FwdSplit*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, float*, float*, const WorkItem*,
                          int, const int32_t*, const int32_t*, const AttnShape&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_preprocess(const void*, const void*, const float*, bool, float*, float*, const AttnShape&,
                                 hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_dkdv_bf16(const void*, const void*, const void*, const void*, const float*, const float*, void*,
                                void*, const WorkItem*, int, const int32_t*, const int32_t*, const AttnShape&,
                                hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_dq_bf16(const void*, const void*, const void*, const void*, const void*, const float*, float*,
                              float*, void*, const WorkItem*, int, const int32_t*, const int32_t*, const AttnShape&,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_dkdv_bf16_split(const void*, const void*, const void*, const void*, const float*, const float*,
                                      void*, void*, const WorkItem*, int, const int32_t*, const int32_t*,
                                      const AttnShape&, const BwdSplit&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_dq_bf16_split(const void*, const void*, const void*, const void*, const void*, const float*,
                                    float*, float*, void*, const WorkItem*, int, const int32_t*, const int32_t*,
                                    const AttnShape&, const BwdSplit&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_dq_simple(const float*, const float*, const float*, const float*, const float*, const float*,
                                float*, const WorkItem*, int, const int32_t*, const int32_t*, const AttnShape&,
                                hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_dkdv_simple(const float*, const float*, const float*, const float*, const float*, const float*,
                                  float*, float*, const WorkItem*, int, const int32_t*, const int32_t*,
                                  const AttnShape&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_head_features(const void*, const void*, const void*, bool, const float*, const float*,
                                const int32_t*, int, int, int, int, int, float, bool, float*, float*, double*,
                                hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_bf16(const void*, const void*, const void*, void*, void*, const int32_t*,
                              const DecodePlanView&, int, int, int, float, void*, float*, int32_t*, float*,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_cache_fill_bf16(const void*, const void*, void*, void*, const DecodePlanView&, int, int, int,
                                  hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_decode_noalloc_bf16(const void*, const void*, const void*, void*, void*, const int32_t*,
                                      const NoAllocHeads&, int, int, int, int, int, int, int, float, void*, float*,
                                      hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace aah
