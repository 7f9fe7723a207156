// C ABI of the NVFP4 W4A4 linear layer: argument validation and dispatch.
//
// Each entry point validates all of its arguments on the host (no HIP call)
// before it enqueues anything, so every status other than NVFP4_EHIP means
// nothing was launched.  NVFP4_EHIP means the HIP runtime rejected a launch;
// a call that enqueues several kernels may already have enqueued the ones
// before the rejected launch (their outputs are then unspecified).
//
// This file sees only the host-side header launch.hpp: it compiles as plain
// C++ against the HIP runtime API.
#include <stdint.h>

#include <initializer_list>

#include "launch.hpp"

namespace {

using nvfp4::round_up;

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // kernel index math is 32-bit per dimension

// Leading dimensions are bounded like the other sizes, so that the extents
// (rows - 1) * ld + cols computed below stay far inside int64.
bool ld_ok(int64_t ld, int64_t cols) { return ld >= cols && ld < kMaxDim; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A device buffer a call touches: base pointer and extent in bytes (0 = not
// touched by this call).
struct Buf {
  const void* p;
  size_t n;
};

bool overlap(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
  return x < y + b.n && y < x + a.n;
}

// No buffer a call writes overlaps another one it writes or one it reads
// (inputs may share memory with each other).
template <int NO, int NI>
bool disjoint(const Buf (&outs)[NO], const Buf (&ins)[NI]) {
  for (int i = 0; i < NO; ++i) {
    for (int j = 0; j < NI; ++j)
      if (overlap(outs[i], ins[j])) return false;
    for (int j = i + 1; j < NO; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

// Every non-null pointer of the list is 16-byte aligned.
bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
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

nvfp4::SegTable seg_table(const nvfp4_segment* segs, int32_t nseg) {
  nvfp4::SegTable st{};
  st.nseg = nseg;
  for (int i = 0; i < nseg; ++i) st.end[i] = segs[i].n_end;
  return st;
}

nvfp4_status launched(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

// Bytes spanned by `rows` rows of `cols` elements of `elem` bytes at row stride ld.
size_t extent(int64_t rows, int64_t cols, int64_t ld, size_t elem) {
  return (rows == 0 || cols == 0) ? 0 : (size_t)((rows - 1) * ld + cols) * elem;
}

size_t packed_codes(int64_t N, int64_t K) {
  return (size_t)(round_up(N, nvfp4::kStrip) * round_up(K, nvfp4::kTileK) / 2);
}
size_t packed_scales(int64_t N, int64_t K) {
  return (size_t)(round_up(N, nvfp4::kStrip) * round_up(K, nvfp4::kTileK) / 16);
}

// The MFMA GEMM (M > 16) addresses each operand buffer with 32-bit byte offsets:
// the activation codes (M * K / 2 bytes) and the packed weight codes must each
// stay below 4 GiB (their scales are an eighth of that).
bool mfma_operands_fit(int64_t M, int64_t K, int64_t N) {
  return (uint64_t)M * (uint64_t)(K / 2) < (1ull << 32) && (uint64_t)packed_codes(N, K) < (1ull << 32);
}

// ---- per-call validation (host only) ------------------------------------------

nvfp4_status check_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                const uint8_t* codes, const uint8_t* scales, const float* g_dec_out,
                                const void* workspace, size_t workspace_bytes) {
  if (M < 0 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || !ld_ok(ldx, K)) return NVFP4_ESHAPE;
  if (!g_dec_out) return NVFP4_EINVAL;
  const bool empty = (M == 0 || K == 0);
  if (!empty && (!x || !codes || !scales)) return NVFP4_EINVAL;
  if (!all_aligned({x, codes, scales, g_dec_out, amax_in}) || (!empty && ldx % 8 != 0)) return NVFP4_EALIGN;
  const size_t need = nvfp4::quantize_act_workspace(M, K);
  const bool uses_ws = !amax_in && need > 0;
  if (uses_ws && (!workspace || workspace_bytes < need)) return NVFP4_EWORKSPACE;
  if (uses_ws && !aligned16(workspace)) return NVFP4_EALIGN;
  const Buf outs[] = {{codes, (size_t)(M * K / 2)}, {scales, (size_t)(M * K / 16)}, {g_dec_out, 4},
                      {workspace, uses_ws ? need : 0}};
  const Buf ins[] = {{x, extent(M, K, ldx, 2)}, {amax_in, 4}};
  return disjoint(outs, ins) ? NVFP4_OK : NVFP4_EINVAL;
}

nvfp4_status check_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec, int64_t M,
                        int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                        const nvfp4_segment* segs, const float* w_g_dec, int32_t nseg, const float* out,
                        int64_t ldo) {
  if (M < 0 || K < 0 || N < 1) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim || !ld_ok(ldo, N)) return NVFP4_ESHAPE;
  if (M > 16 && !mfma_operands_fit(M, K, N)) return NVFP4_ESHAPE;
  const nvfp4_status ss = check_segments(segs, nseg, N);
  if (ss != NVFP4_OK) return ss;
  if (M == 0) return NVFP4_OK;                      // nothing is read or written
  if (!out) return NVFP4_EINVAL;
  if (K > 0 && (!a_codes || !a_scales || !a_g_dec || !w_codes || !w_scales || !w_g_dec)) return NVFP4_EINVAL;
  if (!all_aligned({a_codes, a_scales, a_g_dec, w_codes, w_scales, w_g_dec, out})) return NVFP4_EALIGN;
  if (K == 0) return NVFP4_OK;                      // empty sum: out = 0, no operand is read
  const Buf outs[] = {{out, extent(M, N, ldo, 4)}};
  const Buf ins[] = {{a_codes, (size_t)(M * K / 2)}, {a_scales, (size_t)(M * K / 16)}, {a_g_dec, 4},
                     {w_codes, packed_codes(N, K)}, {w_scales, packed_scales(N, K)}, {w_g_dec, (size_t)nseg * 4}};
  return disjoint(outs, ins) ? NVFP4_OK : NVFP4_EINVAL;
}

nvfp4_status check_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                          const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec,
                          const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, const nvfp4_segment* segs,
                          const float* w_g_dec, int32_t nseg, const float* out, int64_t ldo, const void* workspace,
                          size_t workspace_bytes) {
  // sizes and the segment table first, then each half on its own (the GEMM
  // half reads the codes the quantizer writes) ...
  if (M < 0 || K < 0 || N < 1) return NVFP4_EINVAL;
  if (K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim || !ld_ok(ldx, K) || !ld_ok(ldo, N))
    return NVFP4_ESHAPE;
  if (M > 16 && !mfma_operands_fit(M, K, N)) return NVFP4_ESHAPE;
  nvfp4_status s = check_segments(segs, nseg, N);
  if (s != NVFP4_OK) return s;
  s = check_quantize_act(x, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, workspace,
                                      workspace_bytes);
  if (s != NVFP4_OK) return s;
  s = check_gemm(a_codes, a_scales, a_g_dec, M, K, w_codes, w_scales, N, segs, w_g_dec, nseg, out, ldo);
  if (s != NVFP4_OK) return s;
  // ... and across the halves: nothing the call writes overlaps anything else it touches
  const size_t need = nvfp4::quantize_act_workspace(M, K);
  const bool uses_ws = !amax_in && need > 0;
  const bool empty = (M == 0 || K == 0);
  const Buf outs[] = {{a_codes, (size_t)(M * K / 2)}, {a_scales, (size_t)(M * K / 16)}, {a_g_dec, 4},
                      {out, M == 0 ? 0 : extent(M, N, ldo, 4)}, {workspace, uses_ws ? need : 0}};
  const Buf ins[] = {{x, extent(M, K, ldx, 2)}, {amax_in, 4}, {w_codes, empty ? 0 : packed_codes(N, K)},
                     {w_scales, empty ? 0 : packed_scales(N, K)}, {w_g_dec, empty ? 0 : (size_t)nseg * 4}};
  return disjoint(outs, ins) ? NVFP4_OK : NVFP4_EINVAL;
}

}  // namespace

namespace nvfp4 {
hipError_t launch_read_probe(const void* buf, int64_t bytes, int workgroups, uint32_t* sink, hipStream_t stream);
}  // namespace nvfp4

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
  const nvfp4_status s =
      check_quantize_act(x_bf16, M, K, ldx, amax_in, codes, scales, g_dec_out, workspace, workspace_bytes);
  if (s != NVFP4_OK) return s;
  return launched(nvfp4::launch_quantize_act(static_cast<const uint16_t*>(x_bf16), M, K, ldx, amax_in, codes,
                                             scales, g_dec_out, workspace, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_packed_weight_bytes(int64_t N, int64_t K, size_t* codes_bytes, size_t* scales_bytes) {
  if (N < 0 || K < 0 || !codes_bytes || !scales_bytes) return NVFP4_EINVAL;
  if (K % 16 != 0 || N >= kMaxDim || K >= kMaxDim) return NVFP4_ESHAPE;
  *codes_bytes = packed_codes(N, K);
  *scales_bytes = packed_scales(N, K);
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
  if (!all_aligned({w, w_codes, w_scales, w_g_dec})) return NVFP4_EALIGN;
  const size_t need = nvfp4::pack_weight_workspace(N, K, nseg);
  if (!workspace || workspace_bytes < need) return NVFP4_EWORKSPACE;
  if (!aligned16(workspace)) return NVFP4_EALIGN;
  const Buf outs[] = {{w_codes, packed_codes(N, K)}, {w_scales, packed_scales(N, K)}, {w_g_dec, (size_t)nseg * 4},
                      {workspace, need}};
  const Buf ins[] = {{w, extent(N, K, ldw, 4)}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_pack_weight(w, N, K, ldw, segs, nseg, w_codes, w_scales, w_g_dec, workspace,
                                            static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_weight_to_canonical(const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, int64_t K,
                                       uint8_t* codes, uint8_t* scales, void* stream) {
  if (N < 0 || K < 0) return NVFP4_EINVAL;
  if (K % 16 != 0 || N >= kMaxDim || K >= kMaxDim) return NVFP4_ESHAPE;
  if (N == 0 || K == 0) return NVFP4_OK;
  if (!w_codes || !w_scales || !codes || !scales) return NVFP4_EINVAL;
  if (!all_aligned({w_codes, w_scales, codes, scales})) return NVFP4_EALIGN;
  const Buf outs[] = {{codes, (size_t)(N * K / 2)}, {scales, (size_t)(N * K / 16)}};
  const Buf ins[] = {{w_codes, packed_codes(N, K)}, {w_scales, packed_scales(N, K)}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_weight_to_canonical(w_codes, w_scales, N, K, codes, scales,
                                                    static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec, int64_t M,
                        int64_t K, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                        const nvfp4_segment* segs, const float* w_g_dec, int32_t nseg, float* out, int64_t ldo,
                        void* stream) {
  const nvfp4_status s =
      check_gemm(a_codes, a_scales, a_g_dec, M, K, w_codes, w_scales, N, segs, w_g_dec, nseg, out, ldo);
  if (s != NVFP4_OK || M == 0) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (K == 0) return launched(nvfp4::launch_fill_zero(out, (int)M, (int)N, ldo, st));
  const nvfp4::SegTable tab = seg_table(segs, nseg);
  if (nvfp4::gemm_prefers_skinny(M, K, N))
    return launched(nvfp4::launch_gemm_skinny(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales,
                                              (int)N, tab, w_g_dec, out, ldo, st));
  return launched(nvfp4::launch_gemm_mfma(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N,
                                          tab, w_g_dec, out, ldo, st));
}

int nvfp4_gemm_form(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return -1;
  if (nvfp4::gemm_prefers_skinny(M, K, N)) return 0;
  return nvfp4::mfma_narrow(M, N) ? 2 : 1;
}

// ---- nvfp4_linear: the workspace holds the quantizer's amax partials (large inputs only)
size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return nvfp4::quantize_act_workspace(M, K);
}

static nvfp4_status linear_impl(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                uint8_t* a_codes, uint8_t* a_scales, float* a_g_dec, const uint8_t* w_codes,
                                const uint8_t* w_scales, int64_t N, const nvfp4_segment* segs, const float* w_g_dec,
                                int32_t nseg, float* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const nvfp4_status s = check_linear(x_bf16, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, w_codes, w_scales,
                                      N, segs, w_g_dec, nseg, out, ldo, workspace, workspace_bytes);
  if (s != NVFP4_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const nvfp4::SegTable tab = seg_table(segs, nseg);
  if (M > 0 && nvfp4::linear_decode_fits(M, K))
    return launched(nvfp4::launch_linear_decode(x, ldx, amax_in, a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes,
                                                w_scales, (int)N, tab, w_g_dec, out, ldo, st));
  // the quantizer, then the GEMM (for M == 0 only g_dec is written; for K == 0
  // the GEMM zero-fills out)
  if (nvfp4::launch_quantize_act(x, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, workspace, st) != hipSuccess)
    return NVFP4_EHIP;
  if (M == 0) return NVFP4_OK;
  if (K == 0) return launched(nvfp4::launch_fill_zero(out, (int)M, (int)N, ldo, st));
  if (nvfp4::gemm_prefers_skinny(M, K, N))
    return launched(nvfp4::launch_gemm_skinny(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N,
                                              tab, w_g_dec, out, ldo, st));
  return launched(nvfp4::launch_gemm_mfma(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales, (int)N,
                                          tab, w_g_dec, out, ldo, st));
}

nvfp4_status nvfp4_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                          uint8_t* a_codes, uint8_t* a_scales, float* a_g_dec, const uint8_t* w_codes,
                          const uint8_t* w_scales, int64_t N, const nvfp4_segment* segs, const float* w_g_dec,
                          int32_t nseg, float* out, int64_t ldo, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return linear_impl(x_bf16, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, w_codes, w_scales, N, segs, w_g_dec,
                     nseg, out, ldo, workspace, workspace_bytes, stream);
}

// The same with the library's own scratch (one static device array per GPU)
// in place of the caller's workspace: no allocation anywhere in the call.
nvfp4_status nvfp4_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                  uint8_t* a_codes, uint8_t* a_scales, float* a_g_dec, const uint8_t* w_codes,
                                  const uint8_t* w_scales, int64_t N, const nvfp4_segment* segs,
                                  const float* w_g_dec, int32_t nseg, float* out, int64_t ldo, void* stream) {
  if (M >= 0 && K >= 0 && nvfp4::quantize_act_workspace(M, K) > nvfp4::kScratchBytes) return NVFP4_EWORKSPACE;
  void* scratch = nullptr;
  if (nvfp4::scratch_for_stream(static_cast<hipStream_t>(stream), &scratch) != hipSuccess) return NVFP4_EHIP;
  return linear_impl(x_bf16, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, w_codes, w_scales, N, segs, w_g_dec,
                     nseg, out, ldo, scratch, nvfp4::kScratchBytes, stream);
}

// ---- fused gate+up GEMM with the SwiGLU -> NVFP4 epilogue
nvfp4_status nvfp4_pack_weight_gate_up(const float* w, int64_t I, int64_t K, int64_t ldw, uint8_t* w_codes,
                                       uint8_t* w_scales, float* w_g_dec, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (I < 1 || K < 0) return NVFP4_EINVAL;
  if (I % 128 != 0 || K % 16 != 0 || K < 16 || 2 * I >= kMaxDim || K >= kMaxDim || !ld_ok(ldw, K))
    return NVFP4_ESHAPE;
  if (!w || !w_codes || !w_scales || !w_g_dec) return NVFP4_EINVAL;
  if (!all_aligned({w, w_codes, w_scales, w_g_dec})) return NVFP4_EALIGN;
  const size_t need = nvfp4::pack_weight_workspace(2 * I, K, 2);
  if (!workspace || workspace_bytes < need) return NVFP4_EWORKSPACE;
  if (!aligned16(workspace)) return NVFP4_EALIGN;
  const Buf outs[] = {{w_codes, packed_codes(2 * I, K)}, {w_scales, packed_scales(2 * I, K)}, {w_g_dec, 8},
                      {workspace, need}};
  const Buf ins[] = {{w, extent(2 * I, K, ldw, 4)}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
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
  if (M > 0 && (!a_codes || !a_scales || !a_g_dec || !w_codes || !w_scales || !w_g_dec || !h_codes || !h_scales))
    return NVFP4_EINVAL;
  if (!all_aligned({a_codes, a_scales, a_g_dec, w_codes, w_scales, w_g_dec, amax_h, h_codes, h_scales, h_g_dec}))
    return NVFP4_EALIGN;
  const Buf outs[] = {{h_codes, (size_t)(M * I / 2)}, {h_scales, (size_t)(M * I / 16)}, {h_g_dec, 4}};
  const Buf ins[] = {{a_codes, (size_t)(M * K / 2)}, {a_scales, (size_t)(M * K / 16)}, {a_g_dec, M ? 4u : 0u},
                     {w_codes, M ? packed_codes(2 * I, K) : 0}, {w_scales, M ? packed_scales(2 * I, K) : 0},
                     {w_g_dec, M ? 8u : 0u}, {amax_h, 4}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0)
    return launched(nvfp4::launch_quantize_act(nullptr, 0, 0, 0, amax_h, nullptr, nullptr, h_g_dec, nullptr, s));
  return launched(nvfp4::launch_gemm_swiglu_quantize(a_codes, a_scales, a_g_dec, (int)M, (int)K, w_codes, w_scales,
                                                     (int)I, w_g_dec, amax_h, h_codes, h_scales, h_g_dec, s));
}

nvfp4_status nvfp4_swiglu(const float* gu, int64_t M, int64_t I, int64_t ldgu, void* h_bf16, int64_t ldh,
                          void* stream) {
  if (M < 0 || I < 0) return NVFP4_EINVAL;
  if (M >= kMaxDim || I >= kMaxDim || !ld_ok(ldgu, 2 * I) || !ld_ok(ldh, I)) return NVFP4_ESHAPE;
  if (M == 0 || I == 0) return NVFP4_OK;
  if (!gu || !h_bf16) return NVFP4_EINVAL;
  if (!all_aligned({gu, h_bf16})) return NVFP4_EALIGN;
  const Buf outs[] = {{h_bf16, extent(M, I, ldh, 2)}};
  const Buf ins[] = {{gu, extent(M, 2 * I, ldgu, 4)}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
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
  if (!aligned16(running_amax)) return NVFP4_EALIGN;
  if (M == 0 || K == 0) return NVFP4_OK;
  if (!x_bf16) return NVFP4_EINVAL;
  if (!aligned16(x_bf16) || ldx % 8 != 0) return NVFP4_EALIGN;
  const size_t need = nvfp4::amax_observe_workspace();
  if (!workspace || workspace_bytes < need) return NVFP4_EWORKSPACE;
  if (!aligned16(workspace)) return NVFP4_EALIGN;
  const Buf outs[] = {{running_amax, 4}, {workspace, need}};
  const Buf ins[] = {{x_bf16, extent(M, K, ldx, 2)}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
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
  if (!all_aligned({x_bf16, amax_in, counts}) || (!empty && ldx % 8 != 0)) return NVFP4_EALIGN;
  const Buf outs[] = {{counts, 8}};
  const Buf ins[] = {{x_bf16, extent(M, K, ldx, 2)}, {amax_in, 4}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_quantize_stats(static_cast<const uint16_t*>(x_bf16), M, K, ldx, amax_in, counts,
                                               static_cast<hipStream_t>(stream)));
}

// ---- calibrated FP8 KV-cache codec
nvfp4_status nvfp4_kv_fp8_encode(const void* x_bf16, int64_t n, const float* amax, uint8_t* codes, void* stream) {
  if (n < 0) return NVFP4_EINVAL;
  if (n >= ((int64_t)1 << 48)) return NVFP4_ESHAPE;
  if (n == 0) return NVFP4_OK;
  if (!x_bf16 || !amax || !codes) return NVFP4_EINVAL;
  if (!all_aligned({x_bf16, amax, codes})) return NVFP4_EALIGN;
  const Buf outs[] = {{codes, (size_t)n}};
  const Buf ins[] = {{x_bf16, (size_t)n * 2}, {amax, 4}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_kv_fp8_encode(static_cast<const uint16_t*>(x_bf16), n, amax, codes,
                                              static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_kv_fp8_decode(const uint8_t* codes, int64_t n, const float* amax, void* out_bf16, void* stream) {
  if (n < 0) return NVFP4_EINVAL;
  if (n >= ((int64_t)1 << 48)) return NVFP4_ESHAPE;
  if (n == 0) return NVFP4_OK;
  if (!codes || !amax || !out_bf16) return NVFP4_EINVAL;
  if (!all_aligned({codes, amax, out_bf16})) return NVFP4_EALIGN;
  const Buf outs[] = {{out_bf16, (size_t)n * 2}};
  const Buf ins[] = {{codes, (size_t)n}, {amax, 4}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_kv_fp8_decode(codes, n, amax, static_cast<uint16_t*>(out_bf16),
                                              static_cast<hipStream_t>(stream)));
}

// ---- diagnostic: the device conversion steps over a range of bit patterns
nvfp4_status nvfp4_convert_sweep(int32_t op, uint32_t first_bits, int64_t n, uint8_t* out, void* stream) {
  if (op < 0 || op > 2 || n < 0) return NVFP4_EINVAL;
  if ((uint64_t)first_bits + (uint64_t)n > (1ull << 32)) return NVFP4_ESHAPE;
  if (n == 0) return NVFP4_OK;
  if (!out) return NVFP4_EINVAL;
  if (!aligned16(out)) return NVFP4_EALIGN;
  return launched(nvfp4::launch_convert_sweep(op, first_bits, n, out, static_cast<hipStream_t>(stream)));
}

// ---- diagnostic: the read rate of a bare stream (stream_probe.hip)
nvfp4_status nvfp4_read_probe(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (bytes < 0 || workgroups < 1 || workgroups > 65536) return NVFP4_EINVAL;
  if (bytes % 16 != 0 || bytes >= ((int64_t)1 << 40)) return NVFP4_ESHAPE;
  if (!buf || !sink) return NVFP4_EINVAL;
  if (!all_aligned({buf, sink})) return NVFP4_EALIGN;
  const Buf outs[] = {{sink, (size_t)workgroups * 4}};
  const Buf ins[] = {{buf, (size_t)bytes}};
  if (!disjoint(outs, ins)) return NVFP4_EINVAL;
  return launched(nvfp4::launch_read_probe(buf, bytes, workgroups, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
