// Host-only stand-ins for the kernel launchers, so that the C ABI layer
// (sv_api.cpp) and the planner (sv_plan.cpp) can be built and exercised under
// AddressSanitizer / UndefinedBehaviorSanitizer on a machine without a GPU.
// Nothing here touches memory behind the pointers it receives.
#include "sv_internal.h"

namespace sv {

hipError_t launch_attention(const AttnPlan&, const AttnPtrs&, hipStream_t) { return hipSuccess; }
hipError_t launch_accept(int, int, int, const float*, const int32_t*, int32_t*, int32_t*,
                         int32_t*, const int32_t*, int32_t*, void*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_accept_tree(int, int, int, const float*, const int32_t*, const int32_t*,
                              int32_t*, int32_t*, int32_t*, int32_t*, const int32_t*, int32_t*,
                              void*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_accept_sampled(int, int, int, float, const float*, const float*,
                                 const int32_t*, const float*, const float*, int32_t*, int32_t*,
                                 const int32_t*, int32_t*, void*, hipStream_t) {
  return hipSuccess;
}
size_t draft_signals_workspace_bytes(int rows, int V) {
  return (size_t)rows * (size_t)argmax_chunks(V) * 32u;
}
hipError_t launch_draft_signals(int, int, float, const float*, float*, float*, int32_t*, int,
                                float, int, void*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_kv_append(const AppendPlan&, const void*, const void*, void*, void*, float*,
                            float*, const int32_t*, const int32_t*, int32_t*, const int32_t*,
                            hipStream_t) {
  return hipSuccess;
}
hipError_t launch_ceiling_read(const void*, size_t, int, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_ceiling_mfma(int, int, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_ceiling_exp2(int, int, float*, hipStream_t) { return hipSuccess; }

static unsigned char g_fake_scratch[256];
hipError_t accept_scratch(void** ptr) {
  *ptr = g_fake_scratch;
  return hipSuccess;
}

}  // namespace sv

extern "C" const char* hipGetErrorString(hipError_t) { return "stub error string"; }
