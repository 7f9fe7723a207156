// C ABI of the NVFP4 W4A4 linear layer: argument validation and dispatch.
// Every check runs on the host before anything is enqueued, so a non-OK status
// means no work was launched and no HIP call was made.
#include <stdint.h>

#include <cstring>

#include "common.hpp"

namespace {

using nvfp4::round_up;

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // kernel index math is 32-bit per dimension

// Leading dimensions are bounded like the other sizes, so that the extents
// (rows - 1) * ld + cols computed below stay far inside int64.
bool ld_ok(int64_t ld, int64_t cols) { return ld >= cols && ld < kMaxDim; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p + n) and [q, q + m) overlap (both non-empty)?
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

nvfp4_status check_segments(const nvfp4_segment* segs, int32_t nseg, int64_t N) {
  if (!segs || nseg < 1 || nseg > NVFP4_MAX_SEGMENTS) return NVFP4_ESEGMENTS;
  int64_t pos = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].n_begin != pos || segs[i].n_end <= segs[i].n_begin) return NVFP4_ESEGMENTS;
    pos = segs[i].n_end;
  }
  return pos == N ? NVFP4_OK : NVFP4_ESEGMENTS;
}

nvfp4_status launched(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_str(int s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument (null pointer, negative size or overlapping buffers)";
    case NVFP4_ESHAPE: return "invalid shape (K must be a multiple of 16; leading dimension too small; size too large)";
    case NVFP4_EALIGN: return "misaligned buffer (16-byte alignment required; bf16 leading dimension must be a multiple of 8)";
    case NVFP4_ESEGMENTS: return "invalid segment table (must tile [0, N) in order, 1..16 segments)";
    case NVFP4_EWORKSPACE: return "workspace missing or too small";
    case NVFP4_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t nvfp4_quantize_act_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return nvfp4::quantize_act_workspace(M, K);
}

nvfp4_status nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                uint8_t* codes, uint8_t* scales, float* g_dec_out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (M < 0 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || !ld_ok(ldx, K)) return NVFP4_ESHAPE;
  if (!g_dec_out) return NVFP4_EINVAL;
  const bool empty = (M == 0 || K == 0);
  if (!empty && (!x_bf16 || !codes || !scales)) return NVFP4_EINVAL;
  if (!empty && (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales) || ldx % 8 != 0))
    return NVFP4_EALIGN;
  const size_t need = nvfp4::quantize_act_workspace(M, K);
  if (!amax_in && need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_EWORKSPACE;
  // outputs (codes, scales, g_dec, and the workspace the dynamic mode writes)
  // must not overlap each other or the inputs (x, amax_in)
  const size_t xb = empty ? 0 : (size_t)((M - 1) * ldx + K) * 2, cb = (size_t)(M * K / 2), sb = (size_t)(M * K / 16);
  const void* outs[4] = {codes, scales, g_dec_out, amax_in ? nullptr : workspace};
  const size_t osz[4] = {cb, sb, 4, amax_in ? 0 : need};
  const void* ins[2] = {x_bf16, amax_in};
  const size_t isz[2] = {xb, 4};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlap(outs[i], osz[i], ins[j], isz[j])) return NVFP4_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return NVFP4_EINVAL;
  }
  return launched(nvfp4::launch_quantize_act(static_cast<const uint16_t*>(x_bf16), M, K, ldx, amax_in, codes,
                                             scales, g_dec_out, workspace, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_packed_weight_bytes(int64_t N, int64_t K, size_t* codes_bytes, size_t* scales_bytes) {
  if (N < 0 || K < 0 || !codes_bytes || !scales_bytes) return NVFP4_EINVAL;
  if (K % 16 != 0 || N >= kMaxDim || K >= kMaxDim) return NVFP4_ESHAPE;
  const int64_t Np = round_up(N, nvfp4::kStrip), Kp = round_up(K, nvfp4::kTileK);
  *codes_bytes = (size_t)(Np * Kp / 2);
  *scales_bytes = (size_t)(Np * Kp / 16);
  return NVFP4_OK;
}

size_t nvfp4_pack_weight_workspace_bytes(int64_t N, int64_t K, int32_t nseg) {
  if (N < 0 || K < 0 || nseg < 1 || nseg > NVFP4_MAX_SEGMENTS) return 0;
  return nvfp4::pack_weight_workspace(N, K, nseg);
}

nvfp4_status nvfp4_pack_weight(const float* w, int64_t N, int64_t K, int64_t ldw, const nvfp4_segment* segs,
                               int32_t nseg, uint8_t* w_codes, uint8_t* w_scales, float* w_g_dec,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 1 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || N >= kMaxDim || K >= kMaxDim || !ld_ok(ldw, K)) return NVFP4_ESHAPE;
  if ((!w && K > 0) || !w_codes || !w_scales || !w_g_dec) return NVFP4_EINVAL;
  const nvfp4_status ss = check_segments(segs, nseg, N);
  if (ss != NVFP4_OK) return ss;
  if (!aligned16(w) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(w_g_dec)) return NVFP4_EALIGN;
  const size_t need = nvfp4::pack_weight_workspace(N, K, nseg);
  if (!workspace || workspace_bytes < need) return NVFP4_EWORKSPACE;
  size_t cb = 0, sb = 0;
  nvfp4_packed_weight_bytes(N, K, &cb, &sb);
  const size_t wb = (size_t)((N - 1) * ldw + K) * 4;
  if (overlap(w, wb, w_codes, cb) || overlap(w, wb, w_scales, sb) || overlap(w_codes, cb, w_scales, sb) ||
      overlap(w_g_dec, nseg * 4, w, wb) || overlap(w_g_dec, nseg * 4, w_codes, cb) ||
      overlap(w_g_dec, nseg * 4, w_scales, sb) || overlap(workspace, need, w, wb) ||
      overlap(workspace, need, w_codes, cb) || overlap(workspace, need, w_scales, sb) ||
      overlap(workspace, need, w_g_dec, nseg * 4))
    return NVFP4_EINVAL;
  return launched(nvfp4::launch_pack_weight(w, N, K, ldw, segs, nseg, w_codes, w_scales, w_g_dec, workspace,
                                            static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_weight_to_canonical(const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, int64_t K,
                                       uint8_t* codes, uint8_t* scales, void* stream) {
  if (N < 0 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || N >= kMaxDim || K >= kMaxDim) return NVFP4_ESHAPE;
  if (N == 0 || K == 0) return NVFP4_OK;
  if (!w_codes || !w_scales || !codes || !scales) return NVFP4_EINVAL;
  if (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(codes) || !aligned16(scales)) return NVFP4_EALIGN;
  return launched(nvfp4::launch_weight_to_canonical(w_codes, w_scales, N, K, codes, scales,
                                                    static_cast<hipStream_t>(stream)));
}

// The MFMA GEMM (M > 16) addresses each operand buffer with 32-bit byte offsets:
// the activation codes (M * K / 2 bytes) and the packed weight codes must each
// stay below 4 GiB (their scales are an eighth of that).
static bool mfma_operands_fit(int64_t M, int64_t K, int64_t N) {
  size_t cb = 0, sb = 0;
  nvfp4_packed_weight_bytes(N, K, &cb, &sb);
  return (uint64_t)M * (uint64_t)(K / 2) < (1ull << 32) && (uint64_t)cb < (1ull << 32);
}

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec, int64_t M,
                        int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                        const nvfp4_segment* segs, const float* w_g_dec, int32_t nseg, float* out, int64_t ldo,
                        void* stream) {
  if (M < 0 || K < 0 || N < 1) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim || !ld_ok(ldo, N)) return NVFP4_ESHAPE;
  if (M > 16 && !mfma_operands_fit(M, K, N)) return NVFP4_ESHAPE;
  const nvfp4_status ss = check_segments(segs, nseg, N);
  if (ss != NVFP4_OK) return ss;
  if (M == 0) return NVFP4_OK;
  if (K == 0) {  // empty sum: out = 0; no operand is read
    if (!out) return NVFP4_EINVAL;
    if (!aligned16(out)) return NVFP4_EALIGN;
    return launched(nvfp4::launch_fill_zero(out, (int)M, (int)N, ldo, static_cast<hipStream_t>(stream)));
  }
  if (!a_codes || !a_scales || !a_g_dec || !w_codes || !w_scales || !w_g_dec || !out) return NVFP4_EINVAL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(out))
    return NVFP4_EALIGN;
  size_t cb = 0, sb = 0;
  nvfp4_packed_weight_bytes(N, K, &cb, &sb);
  const size_t ob = (size_t)((M - 1) * ldo + N) * 4;
  if (overlap(out, ob, a_codes, (size_t)(M * K / 2)) || overlap(out, ob, a_scales, (size_t)(M * K / 16)) ||
      overlap(out, ob, a_g_dec, 4) || overlap(out, ob, w_codes, cb) || overlap(out, ob, w_scales, sb) ||
      overlap(out, ob, w_g_dec, (size_t)nseg * 4))
    return NVFP4_EINVAL;
  nvfp4::SegTable st{};
  st.nseg = nseg;
  for (int i = 0; i < nseg; ++i) st.end[i] = segs[i].n_end;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nvfp4::gemm_prefers_skinny(M, K, N))
    return launched(nvfp4::launch_gemm_skinny(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales,
                                              (int)N, st, w_g_dec, out, ldo, s));
  return launched(nvfp4::launch_gemm_mfma(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N,
                                          st, w_g_dec, out, ldo, s));
}

int nvfp4_gemm_form(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return -1;
  return nvfp4::gemm_prefers_skinny(M, K, N) ? 0 : 1;
}

// ---- nvfp4_linear: the workspace holds the quantizer's amax partials (large inputs only)
size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return nvfp4::quantize_act_workspace(M, K);
}

nvfp4_status nvfp4_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                          uint8_t* a_codes, uint8_t* a_scales, float* a_g_dec, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t N, const nvfp4_segment* segs, const float* w_g_dec,
                          int32_t nseg, float* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (M < 0 || K < 0 || N < 1) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim || !ld_ok(ldx, K) || !ld_ok(ldo, N))
    return NVFP4_ESHAPE;
  if (M > 16 && !mfma_operands_fit(M, K, N)) return NVFP4_ESHAPE;
  const nvfp4_status ss = check_segments(segs, nseg, N);
  if (ss != NVFP4_OK) return ss;
  if (!a_g_dec) return NVFP4_EINVAL;
  const size_t need = nvfp4_linear_workspace_bytes(M, K);
  if (!amax_in && need > 0 && (!workspace || workspace_bytes < need)) return NVFP4_EWORKSPACE;
  if (workspace && !aligned16(workspace)) return NVFP4_EALIGN;
  if (M == 0 || K == 0) {   // nothing to encode or nothing to sum: the separate calls cover both
    const nvfp4_status q = nvfp4_quantize_act(x_bf16, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, workspace,
                                              workspace_bytes, stream);
    if (q != NVFP4_OK || M == 0) return q;
    return nvfp4_gemm(a_codes, a_scales, a_g_dec, M, K, w_codes, w_scales, N, segs, w_g_dec, nseg, out, ldo,
                      stream);
  }
  if (!x_bf16 || !a_codes || !a_scales || !w_codes || !w_scales || !w_g_dec || !out) return NVFP4_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) ||
      !aligned16(w_scales) || !aligned16(out) || ldx % 8 != 0)
    return NVFP4_EALIGN;
  size_t cb = 0, sb = 0;
  nvfp4_packed_weight_bytes(N, K, &cb, &sb);
  const size_t xb = (size_t)((M - 1) * ldx + K) * 2, acb = (size_t)(M * K / 2), asb = (size_t)(M * K / 16);
  const size_t ob = (size_t)((M - 1) * ldo + N) * 4;
  const void* outs[4] = {a_codes, a_scales, a_g_dec, out};
  const size_t osz[4] = {acb, asb, 4, ob};
  const void* ins[6] = {x_bf16, w_codes, w_scales, w_g_dec, workspace, amax_in};
  const size_t isz[6] = {xb, cb, sb, (size_t)nseg * 4, need, 4};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], osz[i], ins[j], isz[j])) return NVFP4_EINVAL;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return NVFP4_EINVAL;
  }
  nvfp4::SegTable st{};
  st.nseg = nseg;
  for (int i = 0; i < nseg; ++i) st.end[i] = segs[i].n_end;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nvfp4::linear_decode_fits(M, K))
    return launched(nvfp4::launch_linear_decode(static_cast<const uint16_t*>(x_bf16), ldx, amax_in, a_codes, a_scales,
                                                a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N, st, w_g_dec, out,
                                                ldo, s));
  const hipError_t e = nvfp4::launch_quantize_act(static_cast<const uint16_t*>(x_bf16), M, K, ldx, amax_in, a_codes,
                                                  a_scales, a_g_dec, workspace, s);
  if (e != hipSuccess) return NVFP4_EHIP;
  if (nvfp4::gemm_prefers_skinny(M, K, N))
    return launched(nvfp4::launch_gemm_skinny(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N,
                                              st, w_g_dec, out, ldo, s));
  return launched(nvfp4::launch_gemm_mfma(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N,
                                          st, w_g_dec, out, ldo, s));
}

// ---- fused gate+up GEMM with the SwiGLU -> NVFP4 epilogue
nvfp4_status nvfp4_pack_weight_gate_up(const float* w, int64_t I, int64_t K, int64_t ldw, uint8_t* w_codes,
                                       uint8_t* w_scales, float* w_g_dec, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (I < 1 || K < 0) return NVFP4_EINVAL;
  if (I % 128 != 0 || K % 16 != 0 || K < 16 || 2 * I >= kMaxDim || K >= kMaxDim || !ld_ok(ldw, K))
    return NVFP4_ESHAPE;
  if (!w || !w_codes || !w_scales || !w_g_dec) return NVFP4_EINVAL;
  if (!aligned16(w) || !aligned16(w_codes) || !aligned16(w_scales)) return NVFP4_EALIGN;
  const size_t need = nvfp4::pack_weight_workspace(2 * I, K, 2);
  if (!workspace || workspace_bytes < need) return NVFP4_EWORKSPACE;
  size_t cb = 0, sb = 0;
  nvfp4_packed_weight_bytes(2 * I, K, &cb, &sb);
  const size_t wb = (size_t)((2 * I - 1) * ldw + K) * 4;
  if (overlap(w, wb, w_codes, cb) || overlap(w, wb, w_scales, sb) || overlap(w_codes, cb, w_scales, sb) ||
      overlap(workspace, need, w_codes, cb) || overlap(workspace, need, w_scales, sb) ||
      overlap(workspace, need, w, wb) || overlap(workspace, need, w_g_dec, 8) ||
      overlap(w_g_dec, 8, w_codes, cb) || overlap(w_g_dec, 8, w_scales, sb) || overlap(w_g_dec, 8, w, wb))
    return NVFP4_EINVAL;
  return launched(nvfp4::launch_pack_weight_gate_up(w, I, K, ldw, w_codes, w_scales, w_g_dec, workspace,
                                                    static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec,
                                        int64_t M, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                                        int64_t I, const float* w_g_dec, const float* amax_h, uint8_t* h_codes,
                                        uint8_t* h_scales, float* h_g_dec, void* stream) {
  if (M < 0 || K < 0 || I < 1) return NVFP4_EINVAL;
  if (I % 128 != 0 || K % 16 != 0 || K < 16 || M >= kMaxDim || K >= kMaxDim || 2 * I >= kMaxDim)
    return NVFP4_ESHAPE;
  if (!mfma_operands_fit(M, K, 2 * I)) return NVFP4_ESHAPE;
  if (!amax_h || !h_g_dec) return NVFP4_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) return launched(nvfp4::launch_quantize_act(nullptr, 0, 0, 0, amax_h, nullptr, nullptr, h_g_dec,
                                                         nullptr, s));
  if (!a_codes || !a_scales || !a_g_dec || !w_codes || !w_scales || !w_g_dec || !h_codes || !h_scales)
    return NVFP4_EINVAL;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(h_codes) || !aligned16(h_scales))
    return NVFP4_EALIGN;
  size_t cb = 0, sb = 0;
  nvfp4_packed_weight_bytes(2 * I, K, &cb, &sb);
  const size_t hcb = (size_t)(M * I / 2), hsb = (size_t)(M * I / 16);
  const void* outs[3] = {h_codes, h_scales, h_g_dec};
  const size_t osz[3] = {hcb, hsb, 4};
  const void* ins[7] = {a_codes, a_scales, a_g_dec, w_codes, w_scales, w_g_dec, amax_h};
  const size_t isz[7] = {(size_t)(M * K / 2), (size_t)(M * K / 16), 4, cb, sb, 8, 4};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlap(outs[i], osz[i], ins[j], isz[j])) return NVFP4_EINVAL;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], osz[i], outs[j], osz[j])) return NVFP4_EINVAL;
  }
  return launched(nvfp4::launch_gemm_swiglu_quantize(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales,
                                                     (int)I, w_g_dec, amax_h, h_codes, h_scales, h_g_dec, s));
}

nvfp4_status nvfp4_swiglu(const float* gu, int64_t M, int64_t I, int64_t ldgu, void* h_bf16, int64_t ldh,
                          void* stream) {
  if (M < 0 || I < 0) return NVFP4_EINVAL;
  if (M >= kMaxDim || I >= kMaxDim || !ld_ok(ldgu, 2 * I) || !ld_ok(ldh, I)) return NVFP4_ESHAPE;
  if (M == 0 || I == 0) return NVFP4_OK;
  if (!gu || !h_bf16) return NVFP4_EINVAL;
  const size_t gb = (size_t)((M - 1) * ldgu + 2 * I) * 4, hb = (size_t)((M - 1) * ldh + I) * 2;
  if (overlap(gu, gb, h_bf16, hb)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_swiglu(gu, M, I, ldgu, static_cast<uint16_t*>(h_bf16), ldh,
                                       static_cast<hipStream_t>(stream)));
}

// ---- static-scale calibration
size_t nvfp4_amax_observe_workspace_bytes(int64_t M, int64_t K) {
  (void)M;
  (void)K;
  return nvfp4::amax_observe_workspace();
}

nvfp4_status nvfp4_amax_observe(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, float* running_amax,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || !ld_ok(ldx, K)) return NVFP4_ESHAPE;
  if (!running_amax) return NVFP4_EINVAL;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x_bf16) return NVFP4_EINVAL;
  if (!aligned16(x_bf16) || ldx % 8 != 0) return NVFP4_EALIGN;
  const size_t need = nvfp4::amax_observe_workspace();
  if (!workspace || workspace_bytes < need) return NVFP4_EWORKSPACE;
  const size_t xb = (size_t)((M - 1) * ldx + K) * 2;
  if (overlap(x_bf16, xb, running_amax, 4) || overlap(workspace, need, running_amax, 4) ||
      overlap(workspace, need, x_bf16, xb))
    return NVFP4_EINVAL;
  return launched(nvfp4::launch_amax_observe(static_cast<const uint16_t*>(x_bf16), M, K, ldx, running_amax,
                                             workspace, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_stats(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                  uint32_t* counts, void* stream) {
  if (M < 0 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || !ld_ok(ldx, K)) return NVFP4_ESHAPE;
  if (!amax_in || !counts) return NVFP4_EINVAL;
  const bool empty = (M == 0 || K == 0);
  if (!empty && !x_bf16) return NVFP4_EINVAL;
  if (!empty && (!aligned16(x_bf16) || ldx % 8 != 0)) return NVFP4_EALIGN;
  if (!empty && overlap(x_bf16, (size_t)((M - 1) * ldx + K) * 2, counts, 8)) return NVFP4_EINVAL;
  if (overlap(amax_in, 4, counts, 8)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_quantize_stats(static_cast<const uint16_t*>(x_bf16), M, K, ldx, amax_in, counts,
                                               static_cast<hipStream_t>(stream)));
}

// ---- calibrated FP8 KV-cache codec
nvfp4_status nvfp4_kv_fp8_encode(const void* x_bf16, int64_t n, const float* amax, uint8_t* codes, void* stream) {
  if (n < 0) return NVFP4_EINVAL;
  if (n >= ((int64_t)1 << 48)) return NVFP4_ESHAPE;
  if (n == 0) return NVFP4_OK;
  if (!x_bf16 || !amax || !codes) return NVFP4_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(codes)) return NVFP4_EALIGN;
  if (overlap(x_bf16, (size_t)n * 2, codes, (size_t)n) || overlap(amax, 4, codes, (size_t)n)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_kv_fp8_encode(static_cast<const uint16_t*>(x_bf16), n, amax, codes,
                                              static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_kv_fp8_decode(const uint8_t* codes, int64_t n, const float* amax, void* out_bf16, void* stream) {
  if (n < 0) return NVFP4_EINVAL;
  if (n >= ((int64_t)1 << 48)) return NVFP4_ESHAPE;
  if (n == 0) return NVFP4_OK;
  if (!codes || !amax || !out_bf16) return NVFP4_EINVAL;
  if (!aligned16(codes) || !aligned16(out_bf16)) return NVFP4_EALIGN;
  if (overlap(codes, (size_t)n, out_bf16, (size_t)n * 2) || overlap(amax, 4, out_bf16, (size_t)n * 2))
    return NVFP4_EINVAL;
  return launched(nvfp4::launch_kv_fp8_decode(codes, n, amax, static_cast<uint16_t*>(out_bf16),
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
