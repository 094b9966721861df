// Test-only stand-ins for the library's kernel launchers, linked with the C
// ABI's argument checks (api.cpp) and the launch planning (plans.cpp) into a
// host-only library built with AddressSanitizer and UBSan. No GPU, no device
// code: each launcher only counts its call and returns the error the test
// asks for, so a test can force the launch-failure path (QG_ERR_HIP) and see
// that nothing else was enqueued after it.
#include <stdint.h>

#include "qg_internal.h"

namespace {
int g_fail = 0;          // 1: every launch fails; 2: the scratch lookup fails
long g_calls = 0;        // launcher calls since the last reset
alignas(256) unsigned char g_fake_scratch[256];   // never dereferenced by a stub

hipError_t launched() {
  ++g_calls;
  return g_fail == 1 ? hipErrorLaunchFailure : hipSuccess;
}
}  // namespace

extern "C" void qg_test_fail_launches(int mode) { g_fail = mode; }
extern "C" long qg_test_launch_calls(void) { return g_calls; }
extern "C" void qg_test_reset(void) {
  g_calls = 0;
  g_fail = 0;
}

namespace qg {

hipError_t launch_gemm_prefill(int, const PrefillPlan&, const void*, bool, const void*,
                               const void*, bool, bool, void*, int64_t, int64_t, int64_t, void*,
                               hipStream_t) {
  return launched();
}
hipError_t launch_rtn_scales(int, const void*, bool, int64_t, int64_t, void*, hipStream_t) {
  return launched();
}
hipError_t launch_pack_to_grid(int, const void*, bool, const void*, bool, int64_t, int64_t, void*,
                               hipStream_t) {
  return launched();
}
hipError_t launch_prepack(int, const int8_t*, int64_t, int64_t, void*, hipStream_t) {
  return launched();
}
hipError_t launch_unpack(int, const void*, int64_t, int64_t, int8_t*, hipStream_t) {
  return launched();
}
hipError_t launch_fake_quant(int, const void*, bool, const void*, bool, void*, int, int64_t,
                             int64_t, hipStream_t) {
  return launched();
}
hipError_t launch_dequant(int, const void*, const void*, bool, void*, bool, int64_t, int64_t,
                          hipStream_t) {
  return launched();
}
hipError_t launch_gemm_small(int, const SmallPlan&, const void*, bool, const GroupArgs&, bool,
                             bool, int64_t, int64_t, void*, hipStream_t) {
  return launched();
}
hipError_t launch_prepack_scales(const void*, int64_t, int64_t, void*, hipStream_t) {
  return launched();
}
hipError_t launch_swa_attention(const SwaPlan&, const void*, const void*, const void*,
                                const int32_t*, void*, int64_t, int64_t, int64_t, int64_t, float,
                                void*, hipStream_t) {
  return launched();
}
hipError_t launch_read_stream(const void*, int64_t, int, void*, hipStream_t) { return launched(); }
hipError_t launch_gemv(int, const void*, bool, const GroupArgs&, bool, bool, int64_t, int64_t,
                       hipStream_t) {
  return launched();
}
hipError_t scratch_for_stream(hipStream_t, void** ptr) {
  if (g_fail == 2) return hipErrorInvalidSymbol;
  *ptr = g_fake_scratch;
  return hipSuccess;
}

}  // namespace qg
