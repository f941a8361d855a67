// Host-only stand-ins for the library's launchers and planner, linked with
// csrc/mx_api.cpp into a library built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_abi_sanitized.py). They let the C
// ABI's argument checking run on a machine without a GPU: every launch
// "succeeds" without touching its pointers, plans have a fixed name and no
// GEMM asks for a workspace. Test infrastructure only; no compute happens here.
#include "mx_launch.h"

namespace mx {

hipError_t launch_quantize(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, int, int, const uint32_t*,
                           int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_quantize_batch(const QuantBatchItem*, int, int, uint32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_layernorm_quantize(const float*, int64_t, int64_t, int64_t, const float*, const float*, float,
                                     uint8_t*, uint8_t*, int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_quantize_dual(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*,
                                int, const float*, float, int, uint64_t, uint64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gemm_mx(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, void*, int64_t, int64_t,
                          int64_t, int, const uint16_t*, int, float*, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gemm_mx_gelu_quant(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t,
                                     int64_t, int, const uint16_t*, uint8_t*, uint8_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gemm_nvfp4(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, void*, int64_t, int64_t,
                             int64_t, const uint16_t*, int, float*, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_splitk_reduce(const float*, int, int64_t, int64_t, const uint16_t*, void*, int, hipStream_t) {
  return hipSuccess;
}
int64_t gemm_mx_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }
int64_t gemm_nvfp4_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }
hipError_t scratch_buffer(void** ptr) {
  alignas(256) static unsigned char host_stand_in[256];
  *ptr = host_stand_in;
  return hipSuccess;
}
const char* plan_gemm_mx(int64_t, int64_t, int64_t, int, int64_t) { return "stub plan"; }
const char* plan_gemm_nvfp4(int64_t, int64_t, int64_t, int64_t) { return "stub plan"; }

}  // namespace mx

extern "C" const char* hipGetErrorString(hipError_t) { return "stub error"; }
