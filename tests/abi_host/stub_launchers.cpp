// Stand-ins for the kernel launchers, for the host-only check of the C ABI
// (check_abi.cpp): each records that a launch was requested and returns
// success, or a launch error once a set number of launches has been requested.
// Nothing is dereferenced, so the ABI's argument checks run on fake device
// addresses under the address and undefined-behaviour sanitizers.
#include "stub_launchers.hpp"

namespace stub {
int launches = 0;
int fail_from = -1;   // launch index from which launches fail (-1: never)
bool scratch_fails = false;
}  // namespace stub

static hipError_t record() {
  const int n = stub::launches++;
  return (stub::fail_from >= 0 && n >= stub::fail_from) ? hipErrorLaunchFailure : hipSuccess;
}

namespace nvfp4 {
hipError_t launch_quantize_act(const uint16_t*, int64_t, int64_t, int64_t, const float*, uint8_t*, uint8_t*, float*,
                               void*, hipStream_t) {
  return record();
}
hipError_t launch_pack_weight(const float*, int64_t, int64_t, int64_t, const nvfp4_segment*, int, uint8_t*, uint8_t*,
                              float*, void*, hipStream_t) {
  return record();
}
hipError_t launch_weight_to_canonical(const uint8_t*, const uint8_t*, int64_t, int64_t, uint8_t*, uint8_t*,
                                      hipStream_t) {
  return record();
}
hipError_t launch_gemm_skinny(const uint8_t*, const uint8_t*, const float*, int, int, const uint8_t*, const uint8_t*,
                              int, const SegTable&, const float*, float*, int64_t, hipStream_t) {
  return record();
}
hipError_t launch_fill_zero(float*, int, int, int64_t, hipStream_t) { return record(); }
hipError_t launch_linear_decode(const uint16_t*, int64_t, const float*, uint8_t*, uint8_t*, float*, int, int,
                                const uint8_t*, const uint8_t*, int, const SegTable&, const float*, float*, int64_t,
                                hipStream_t) {
  return record();
}
hipError_t launch_gemm_mfma(const uint8_t*, const uint8_t*, const float*, int, int, const uint8_t*, const uint8_t*,
                            int, const SegTable&, const float*, float*, int64_t, hipStream_t) {
  return record();
}
hipError_t launch_pack_weight_gate_up(const float*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, float*, void*,
                                      hipStream_t) {
  return record();
}
hipError_t launch_gemm_swiglu_quantize(const uint8_t*, const uint8_t*, const float*, int, int, const uint8_t*,
                                       const uint8_t*, int, const float*, const float*, uint8_t*, uint8_t*, float*,
                                       hipStream_t) {
  return record();
}
hipError_t launch_swiglu(const float*, int64_t, int64_t, int64_t, uint16_t*, int64_t, hipStream_t) { return record(); }
hipError_t launch_amax_observe(const uint16_t*, int64_t, int64_t, int64_t, float*, void*, hipStream_t) {
  return record();
}
hipError_t launch_quantize_stats(const uint16_t*, int64_t, int64_t, int64_t, const float*, uint32_t*, hipStream_t) {
  return record();
}
hipError_t launch_convert_sweep(int, uint32_t, int64_t, uint8_t*, hipStream_t) { return record(); }
// the allocation-free scratch: a fake device address, or a lookup error
hipError_t scratch_for_stream(hipStream_t, void** out) {
  if (stub::scratch_fails) return hipErrorInvalidSymbol;
  *out = reinterpret_cast<void*>(uintptr_t(1) << 44);
  return hipSuccess;
}
hipError_t launch_kv_fp8_encode(const uint16_t*, int64_t, const float*, uint8_t*, hipStream_t) { return record(); }
hipError_t launch_kv_fp8_decode(const uint8_t*, int64_t, const float*, uint16_t*, hipStream_t) { return record(); }
hipError_t launch_read_probe(const void*, int64_t, int, uint32_t*, hipStream_t) { return record(); }
}  // namespace nvfp4
