// Host-only check of the C ABI's argument handling, built with the address and
// undefined-behaviour sanitizers against the stand-in launchers: every
// rejected call returns its status without requesting a launch, accepted calls
// request the expected launches, and a launch the runtime rejects is reported
// as NVFP4_EHIP.  Buffers are fake device addresses, never dereferenced.
// Prints one line per failed case and "ok <n>" at the end; exits non-zero on
// any failure.
#include <cstdint>
#include <cstdio>
#include <functional>
#include <vector>

#include "../../include/nvfp4.h"
#include "stub_launchers.hpp"

namespace {

const uintptr_t A = uintptr_t(1) << 40;
template <class T = void>
T* at(uintptr_t mb, uintptr_t off = 0) {
  return reinterpret_cast<T*>(A + (mb << 20) + off);
}

struct Case {
  const char* name;
  std::function<nvfp4_status()> call;
  nvfp4_status want;
  int launches;        // launches requested
  int fail_from = -1;  // stand-in launches fail from this index on
};

nvfp4_segment one[1] = {{0, 32}};
nvfp4_segment two16[2] = {{0, 16}, {17, 32}};

nvfp4_status q(const void* x, int64_t M, int64_t K, int64_t ldx, const float* amax, uint8_t* c, uint8_t* s, float* g,
               void* ws = nullptr, size_t wsb = 0) {
  return nvfp4_quantize_act(x, M, K, ldx, amax, c, s, g, ws, wsb, nullptr);
}
nvfp4_status gm(int64_t M, int64_t K, int64_t N, const nvfp4_segment* sg, int nseg, float* out, int64_t ldo,
                const uint8_t* a = at<uint8_t>(0), const float* wg = at<float>(5), const float* ag = at<float>(2)) {
  return nvfp4_gemm(a, at<uint8_t>(1), ag, M, K, at<uint8_t>(3), at<uint8_t>(4), N, sg, wg, nseg, out, ldo, nullptr);
}
nvfp4_status lin(const void* x, int64_t M, int64_t K, int64_t ldx, const float* amax, float* out, void* ws = nullptr,
                 size_t wsb = 0, uint8_t* ac = at<uint8_t>(64), float* ag = at<float>(96)) {
  nvfp4_segment sg[1] = {{0, 32}};
  return nvfp4_linear(x, M, K, ldx, amax, ac, at<uint8_t>(80), ag, at<uint8_t>(128), at<uint8_t>(160), 32, sg,
                      at<float>(192), 1, out, 32, ws, wsb, nullptr);
}

}  // namespace

int main() {
  const size_t qws = nvfp4_quantize_act_workspace_bytes(4096, 4096);
  std::vector<Case> cases = {
      // ---- nvfp4_quantize_act
      {"quant ok", [] { return q(at(0), 4, 32, 32, nullptr, at<uint8_t>(1), at<uint8_t>(2), at<float>(3)); }, NVFP4_OK, 1},
      {"quant M<0", [] { return q(at(0), -1, 32, 32, nullptr, at<uint8_t>(1), at<uint8_t>(2), at<float>(3)); }, NVFP4_EINVAL, 0},
      {"quant K%16", [] { return q(at(0), 4, 24, 32, nullptr, at<uint8_t>(1), at<uint8_t>(2), at<float>(3)); }, NVFP4_ESHAPE, 0},
      {"quant x misaligned", [] { return q(at(0, 8), 4, 32, 32, nullptr, at<uint8_t>(1), at<uint8_t>(2), at<float>(3)); }, NVFP4_EALIGN, 0},
      {"quant g_dec misaligned", [] { return q(at(0), 4, 32, 32, nullptr, at<uint8_t>(1), at<uint8_t>(2), at<float>(3, 4)); }, NVFP4_EALIGN, 0},
      {"quant amax misaligned", [] { return q(at(0), 4, 32, 32, at<float>(4, 4), at<uint8_t>(1), at<uint8_t>(2), at<float>(3)); }, NVFP4_EALIGN, 0},
      {"quant codes over x", [] { return q(at(0), 4, 32, 32, nullptr, at<uint8_t>(0, 16), at<uint8_t>(2), at<float>(3)); }, NVFP4_EINVAL, 0},
      {"quant ws missing", [] { return q(at(0), 4096, 4096, 4096, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96)); }, NVFP4_EWORKSPACE, 0},
      {"quant ws over x", [qws] { return q(at(0), 4096, 4096, 4096, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at(1), qws); }, NVFP4_EINVAL, 0},
      {"quant ws ok", [qws] { return q(at(0), 4096, 4096, 4096, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at(128), qws); }, NVFP4_OK, 1},
      {"quant static no ws", [] { return q(at(0), 4096, 4096, 4096, at<float>(100), at<uint8_t>(64), at<uint8_t>(80), at<float>(96)); }, NVFP4_OK, 1},
      {"quant empty", [] { return q(nullptr, 0, 32, 32, nullptr, nullptr, nullptr, at<float>(3)); }, NVFP4_OK, 1},
      {"quant launch fails", [] { return q(at(0), 4, 32, 32, nullptr, at<uint8_t>(1), at<uint8_t>(2), at<float>(3)); }, NVFP4_EHIP, 1, 0},
      // ---- nvfp4_gemm
      {"gemm ok", [] { return gm(4, 32, 32, one, 1, at<float>(6), 32); }, NVFP4_OK, 1},
      {"gemm M=0", [] { return gm(0, 32, 32, one, 1, nullptr, 32); }, NVFP4_OK, 0},
      {"gemm K=0 out null", [] { return gm(4, 0, 32, one, 1, nullptr, 32); }, NVFP4_EINVAL, 0},
      {"gemm K=0 out misaligned", [] { return gm(4, 0, 32, one, 1, at<float>(6, 4), 32); }, NVFP4_EALIGN, 0},
      {"gemm K=0 fill", [] { return gm(4, 0, 32, one, 1, at<float>(6), 32); }, NVFP4_OK, 1},
      {"gemm segments gap", [] { return gm(4, 32, 32, two16, 2, at<float>(6), 32); }, NVFP4_ESEGMENTS, 0},
      {"gemm a_g misaligned", [] { return gm(4, 32, 32, one, 1, at<float>(6), 32, at<uint8_t>(0), at<float>(5), at<float>(2, 4)); }, NVFP4_EALIGN, 0},
      {"gemm w_g misaligned", [] { return gm(4, 32, 32, one, 1, at<float>(6), 32, at<uint8_t>(0), at<float>(5, 8)); }, NVFP4_EALIGN, 0},
      {"gemm out over weights", [] { return gm(4, 32, 32, one, 1, at<float>(3, 256), 32); }, NVFP4_EINVAL, 0},
      {"gemm MFMA 4 GiB", [] { return gm(1 << 20, 8192, 32, one, 1, at<float>(6), 32); }, NVFP4_ESHAPE, 0},
      {"gemm launch fails", [] { return gm(4, 32, 32, one, 1, at<float>(6), 32); }, NVFP4_EHIP, 1, 0},
      // ---- nvfp4_linear
      {"linear decode ok", [] { return lin(at(0), 4, 32, 32, nullptr, at<float>(224)); }, NVFP4_OK, 1},
      {"linear large ok", [qws] { return lin(at(0), 4096, 4096, 4096, nullptr, at<float>(224), at(300), qws); }, NVFP4_OK, 2},
      {"linear ws over x", [qws] { return lin(at(0), 4096, 4096, 4096, nullptr, at<float>(224), at(1), qws); }, NVFP4_EINVAL, 0},
      {"linear ws over weights", [qws] { return lin(at(0), 4096, 4096, 4096, nullptr, at<float>(224), at(128), qws); }, NVFP4_EINVAL, 0},
      {"linear ws over out", [qws] { return lin(at(0), 4096, 4096, 4096, nullptr, at<float>(224), at(224, 64), qws); }, NVFP4_EINVAL, 0},
      {"linear ws misaligned", [qws] { return lin(at(0), 4096, 4096, 4096, nullptr, at<float>(224), at(300, 4), qws); }, NVFP4_EALIGN, 0},
      {"linear static ws unused", [] { return lin(at(0), 4096, 4096, 4096, at<float>(250), at<float>(224), at(0, 64), 16); }, NVFP4_OK, 2},
      {"linear K=0 out null", [] { return lin(nullptr, 4, 0, 32, nullptr, nullptr); }, NVFP4_EINVAL, 0},
      {"linear K=0 out misaligned", [] { return lin(nullptr, 4, 0, 32, nullptr, at<float>(224, 4)); }, NVFP4_EALIGN, 0},
      {"linear K=0 ok", [] { return lin(nullptr, 4, 0, 32, nullptr, at<float>(224)); }, NVFP4_OK, 2},
      {"linear M=0 ok", [] { return lin(nullptr, 0, 32, 32, nullptr, nullptr); }, NVFP4_OK, 1},
      {"linear g_dec over out", [] { return lin(at(0), 4, 32, 32, nullptr, at<float>(224), nullptr, 0, at<uint8_t>(64), at<float>(224, 16)); }, NVFP4_EINVAL, 0},
      {"linear codes over x", [] { return lin(at(0), 4, 32, 32, nullptr, at<float>(224), nullptr, 0, at<uint8_t>(0, 32)); }, NVFP4_EINVAL, 0},
      {"linear decode launch fails", [] { return lin(at(0), 4, 32, 32, nullptr, at<float>(224)); }, NVFP4_EHIP, 1, 0},
      // the GEMM launch after an enqueued quantizer is rejected: EHIP (the header
      // says the kernels before it may already be enqueued)
      {"linear second launch fails", [qws] { return lin(at(0), 4096, 4096, 4096, nullptr, at<float>(224), at(300), qws); }, NVFP4_EHIP, 2, 1},
      // ---- nvfp4_linear_noalloc: the library's scratch in place of the workspace
      {"noalloc large ok", [] { nvfp4_segment sg[1] = {{0, 32}}; return nvfp4_linear_noalloc(at(0), 4096, 4096, 4096, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at<uint8_t>(128), at<uint8_t>(160), 32, sg, at<float>(192), 1, at<float>(224), 32, nullptr); }, NVFP4_OK, 2},
      {"noalloc decode ok", [] { nvfp4_segment sg[1] = {{0, 32}}; return nvfp4_linear_noalloc(at(0), 4, 32, 32, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at<uint8_t>(128), at<uint8_t>(160), 32, sg, at<float>(192), 1, at<float>(224), 32, nullptr); }, NVFP4_OK, 1},
      {"noalloc bad shape", [] { nvfp4_segment sg[1] = {{0, 32}}; return nvfp4_linear_noalloc(at(0), 4, 24, 32, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at<uint8_t>(128), at<uint8_t>(160), 32, sg, at<float>(192), 1, at<float>(224), 32, nullptr); }, NVFP4_ESHAPE, 0},
      {"noalloc out over x", [] { nvfp4_segment sg[1] = {{0, 32}}; return nvfp4_linear_noalloc(at(0), 4096, 4096, 4096, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at<uint8_t>(128), at<uint8_t>(160), 32, sg, at<float>(192), 1, at<float>(16), 32, nullptr); }, NVFP4_EINVAL, 0},
      {"noalloc scratch lookup fails", [] { stub::scratch_fails = true; nvfp4_segment sg[1] = {{0, 32}}; const nvfp4_status s = nvfp4_linear_noalloc(at(0), 4, 32, 32, nullptr, at<uint8_t>(64), at<uint8_t>(80), at<float>(96), at<uint8_t>(128), at<uint8_t>(160), 32, sg, at<float>(192), 1, at<float>(224), 32, nullptr); stub::scratch_fails = false; return s; }, NVFP4_EHIP, 0},
      // ---- pack, swiglu, calibration, KV codec
      {"pack ok", [] { return nvfp4_pack_weight(at<float>(0), 32, 32, 32, one, 1, at<uint8_t>(1), at<uint8_t>(2), at<float>(3), at(4), 4096, nullptr); }, NVFP4_OK, 1},
      {"pack ws misaligned", [] { return nvfp4_pack_weight(at<float>(0), 32, 32, 32, one, 1, at<uint8_t>(1), at<uint8_t>(2), at<float>(3), at(4, 4), 4096, nullptr); }, NVFP4_EALIGN, 0},
      {"pack g over ws", [] { return nvfp4_pack_weight(at<float>(0), 32, 32, 32, one, 1, at<uint8_t>(1), at<uint8_t>(2), at<float>(4, 16), at(4), 4096, nullptr); }, NVFP4_EINVAL, 0},
      {"swiglu ok", [] { return nvfp4_swiglu(at<float>(0), 4, 64, 128, at(1), 64, nullptr); }, NVFP4_OK, 1},
      {"swiglu gu misaligned", [] { return nvfp4_swiglu(at<float>(0, 4), 4, 64, 128, at(1), 64, nullptr); }, NVFP4_EALIGN, 0},
      {"swiglu h misaligned", [] { return nvfp4_swiglu(at<float>(0), 4, 64, 128, at(1, 2), 64, nullptr); }, NVFP4_EALIGN, 0},
      {"swiglu h over gu", [] { return nvfp4_swiglu(at<float>(0), 4, 64, 128, at(0, 64), 64, nullptr); }, NVFP4_EINVAL, 0},
      {"swiglu-quantize amax misaligned", [] { return nvfp4_gemm_swiglu_quantize(at<uint8_t>(0), at<uint8_t>(1), at<float>(2), 32, 32, at<uint8_t>(3), at<uint8_t>(4), 128, at<float>(5), at<float>(6, 4), at<uint8_t>(7), at<uint8_t>(8), at<float>(9), nullptr); }, NVFP4_EALIGN, 0},
      {"swiglu-quantize ok", [] { return nvfp4_gemm_swiglu_quantize(at<uint8_t>(0), at<uint8_t>(1), at<float>(2), 32, 32, at<uint8_t>(3), at<uint8_t>(4), 128, at<float>(5), at<float>(6), at<uint8_t>(7), at<uint8_t>(8), at<float>(9), nullptr); }, NVFP4_OK, 1},
      {"stats counts misaligned", [] { return nvfp4_quantize_stats(at(0), 4, 32, 32, at<float>(1), at<uint32_t>(2, 4), nullptr); }, NVFP4_EALIGN, 0},
      {"stats ok", [] { return nvfp4_quantize_stats(at(0), 4, 32, 32, at<float>(1), at<uint32_t>(2), nullptr); }, NVFP4_OK, 1},
      {"observe running misaligned", [] { return nvfp4_amax_observe(at(0), 4, 32, 32, at<float>(1, 4), at(2), 4096, nullptr); }, NVFP4_EALIGN, 0},
      {"observe ok", [] { return nvfp4_amax_observe(at(0), 4, 32, 32, at<float>(1), at(2), 4096, nullptr); }, NVFP4_OK, 1},
      {"kv encode amax misaligned", [] { return nvfp4_kv_fp8_encode(at(0), 64, at<float>(1, 4), at<uint8_t>(2), nullptr); }, NVFP4_EALIGN, 0},
      {"kv decode ok", [] { return nvfp4_kv_fp8_decode(at<uint8_t>(0), 64, at<float>(1), at(2), nullptr); }, NVFP4_OK, 1},
      {"kv decode launch fails", [] { return nvfp4_kv_fp8_decode(at<uint8_t>(0), 64, at<float>(1), at(2), nullptr); }, NVFP4_EHIP, 1, 0},
  };
  int bad = 0;
  for (const Case& c : cases) {
    stub::launches = 0;
    stub::fail_from = c.fail_from;
    const nvfp4_status s = c.call();
    if (s != c.want || stub::launches != c.launches) {
      std::printf("FAIL %s: status %d (want %d), launches %d (want %d)\n", c.name, (int)s, (int)c.want,
                  stub::launches, c.launches);
      ++bad;
    }
  }
  if (nvfp4_abi_version() != NVFP4_ABI_VERSION || !nvfp4_status_str(NVFP4_EHIP)) ++bad;
  std::printf("%s %zu\n", bad ? "failed" : "ok", cases.size());
  return bad ? 1 : 0;
}
