// Host-side view of the gfx950 NVFP4 kernels: layout constants, the segment
// table passed to the GEMM kernels, and one launcher per kernel family.  The
// C ABI (api.cpp) sees only this header, so it compiles as plain C++ against
// the HIP runtime API, with no device code.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// ---- layout constants -------------------------------------------------------
constexpr int kBlock = 16;        // elements per E4M3 scale
constexpr int kTileK = 128;       // k extent of one weight chunk
constexpr int kStrip = 16;        // rows (output columns) of one weight chunk
constexpr int kChunkCodes = kStrip * kTileK / 2;        // 1024 bytes
constexpr int kChunkScales = kStrip * kTileK / kBlock;  // 128 bytes
constexpr float kGMax = 2688.0f;  // 6 * 448

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

constexpr int kCUs = 256;         // compute units of a gfx950 (MI355X) device

// Host-side sizes shared by the launchers and the dispatch code.
constexpr int kPartials = 1024;             // amax workgroups of the two-pass activation quantizer
constexpr int64_t kSmallElems = 1 << 17;    // single-launch activation quantizer up to 128K elements
constexpr int kSegParts = 256;              // amax workgroups per weight segment (packer)
constexpr size_t kScratchBytes = kPartials * sizeof(uint32_t) + 16;   // nvfp4_linear_noalloc's scratch
constexpr int kMaxDevices = 64;             // GPUs whose scratch address is cached

// Strips of 16 output columns per workgroup (1..3) of the M <= 16 weight-
// streaming GEMM: the fewest strips on the busiest CU -- a launch of more than
// 256 workgroups puts a second one on some CUs -- with ties going to more strips
// per workgroup (fewer, longer weight streams).  Measured at K = 5120 (us per
// launch, M = 1, skinny GEMM; S = 1 / 2 / 3): N = 2048 3.9 / 4.7 / 5.7,
// N = 5120 5.7 / 5.0 / 5.8, N = 8192 6.0 / 5.7 / 6.3, N = 12288 8.5 / 9.0 / 7.8;
// the one-launch layer follows the same pattern.
inline int skinny_strips(int64_t nstrips) {
  int best = 3;
  int64_t cost = 0;
  for (int s = 3; s >= 1; --s) {
    const int64_t wgs = (nstrips + s - 1) / s;
    const int64_t c = (wgs + kCUs - 1) / kCUs * s;
    if (s == 3 || c < cost) {
      best = s;
      cost = c;
    }
  }
  return best;
}

// Waves of a weight-streaming workgroup (skinny GEMM, row blocks, one-launch
// layer) that split its k tiles, wave w taking tiles w, w + W, w + 2W, ...: the
// count fixes the fp32 summation order, so every weight-streaming form takes it
// from K and N alone and their results stay bit-identical.  Sixteen waves (four
// per SIMD) keep more of the weight stream in flight per CU, which pays where
// the M <= 16 launch leaves CUs idle and each wave has more than five tiles (us
// per skinny launch at M = 1, 8 / 16 waves: K = 17408, N = 5120 15.9 / 14.9;
// N = 2048 11.6 / 10.6; K = 6144, N = 5120 9.0 / 8.5); with every CU busy it
// does not (K = 10240, N = 12288: 15.0 / 15.1), nor at K = 5120 (N = 12288:
// 9.0 / 11.9).
inline int stream_waves(int64_t K, int64_t N) {
  if (K <= 8 * 5 * kTileK) return 8;
  const int64_t nstrips = (N + kStrip - 1) / kStrip;
  const int s = skinny_strips(nstrips);
  return (nstrips + s - 1) / s < kCUs ? 16 : 8;
}

// Rows of the one-launch decode layer for a K (0: none): each wave keeps its k
// tiles' activation blocks for every row in registers and in a wave-private LDS
// area, so longer K takes fewer rows.
inline int decode_max_rows(int64_t K) {
  if (K <= 5 * 8 * kTileK) return 16;                // K <= 5120
  if (K <= 10 * 8 * kTileK) return 8;                // K <= 10240
  if (K <= 20 * 8 * kTileK) return 4;                // K <= 20480
  return 0;
}

// Activation k tiles per wave (U: 5, 10 or 20) of the one-launch layer with nw
// waves; within decode_max_rows the wave-private area (MAXM * U tiles of 80
// bytes) fits LDS and the lane's block registers (MAXM * U / 8 steps of two
// 16-byte chunks) fit the register file, 128 VGPRs per lane at sixteen waves.
inline int decode_tiles_per_wave(int64_t K, int nw) {
  const int64_t per = ((K + kTileK - 1) / kTileK + nw - 1) / nw;
  return per <= 5 ? 5 : (per <= 10 ? 10 : 20);
}

// The MFMA GEMM's two tile forms: 256 x 256 (eight waves, one workgroup per
// CU) and the narrow 256 x 128 (four waves doing the same per-wave work, two
// workgroups per CU).  Their duration in rounds of the wide form (one 256 x 256
// tile per CU): the wide form takes ceil(tiles / 256); the narrow form runs 512
// workgroups per round, and a last round of at most 256 workgroups puts one on
// each of as many CUs (half the work per CU at a lower rate per wave), which
// costs kNarrowLoneRound of a round: measured 0.76-0.79 at K = 5120, N = 12288
// (M = 256 / 512: 96 / 192 narrow workgroups, 79 / 82 us, against 103 us for a
// round of 96 wide ones).
constexpr double kNarrowLoneRound = 0.78;
inline double mfma_rounds(int64_t M, int64_t N, bool narrow) {
  const int64_t num_m = (M + 255) / 256;
  if (!narrow) return (double)((num_m * ((N + 255) / 256) + kCUs - 1) / kCUs);
  const int64_t t = num_m * ((N + 127) / 128), rem = t % (2 * kCUs);
  return (double)(t / (2 * kCUs)) + (rem == 0 ? 0.0 : (rem <= kCUs ? kNarrowLoneRound : 1.0));
}
// Columns a form covers with whole tiles where its last, ragged tile column
// would cost an extra round (that column then runs as the row-blocked
// weight-streaming GEMM); N otherwise.
inline int64_t mfma_main_columns(int64_t M, int64_t N, bool narrow) {
  const int64_t tn = narrow ? 128 : 256, n_full = N / tn * tn;
  return (n_full > 0 && n_full < N && mfma_rounds(M, n_full, narrow) < mfma_rounds(M, n_full + tn, narrow)) ? n_full
                                                                                                          : N;
}
inline double mfma_cost(int64_t M, int64_t N, bool narrow) {
  return mfma_rounds(M, mfma_main_columns(M, N, narrow), narrow);
}
// The narrow form where it takes fewer rounds (a partial last round of wide
// tiles); the wide form on ties.
inline bool mfma_narrow(int64_t M, int64_t N) { return mfma_cost(M, N, true) < mfma_cost(M, N, false); }

// Rows per weight pass of the row-blocked weight-streaming GEMM: 16 for outputs
// of at most 8 strips (there the activation work dominates: the 64 ragged
// columns of the GDN in-projection take 12.9 us in 16-row passes with 2 strips
// per workgroup and 15.3 us in 64-row passes with 1), else 32 up to 32 rows and
// 64 beyond.
inline int rows_per_pass(int64_t M, int64_t N) {
  if ((N + kStrip - 1) / kStrip <= 8) return 16;
  return M <= 32 ? 32 : 64;
}

// Segment table passed by value to the GEMM kernels: column -> module index.
struct SegTable {
  int32_t end[NVFP4_MAX_SEGMENTS];  // exclusive end column of each segment
  int32_t nseg;
};
}  // namespace nvfp4

// ---- host-side launchers (one per kernel family), defined in the .hip files --
namespace nvfp4 {
hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const float* amax_in, uint8_t* codes, uint8_t* scales,
                               float* g_dec_out, void* workspace, hipStream_t stream);
size_t quantize_act_workspace(int64_t M, int64_t K);

hipError_t launch_pack_weight(const float* w, int64_t N, int64_t K, int64_t ldw,
                              const nvfp4_segment* segs, int nseg,
                              uint8_t* w_codes, uint8_t* w_scales, float* w_g_dec,
                              void* workspace, hipStream_t stream);
size_t pack_weight_workspace(int64_t N, int64_t K, int nseg);
hipError_t launch_weight_to_canonical(const uint8_t* w_codes, const uint8_t* w_scales,
                                      int64_t N, int64_t K, uint8_t* codes, uint8_t* scales,
                                      hipStream_t stream);

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g,
                              int M, int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                              const SegTable& st, const float* w_g, float* out, int64_t ldo,
                              hipStream_t stream);
hipError_t launch_fill_zero(float* out, int M, int N, int64_t ldo, hipStream_t stream);
// One-launch decode-form linear layer (activation quantization fused into the
// skinny GEMM); valid when linear_decode_fits(M, K).
bool linear_decode_fits(int64_t M, int64_t K);
// nvfp4_gemm's form for M rows: the weight-streaming skinny GEMM (over 16-row
// blocks when M > 16) or the MFMA GEMM.
bool gemm_prefers_skinny(int64_t M, int64_t K, int64_t N);
hipError_t launch_linear_decode(const uint16_t* x, int64_t ldx, const float* amax_in, uint8_t* a_codes,
                                uint8_t* a_scales, float* a_g, int M, int K, const uint8_t* w_codes,
                                const uint8_t* w_scales, int N, const SegTable& st, const float* w_g, float* out,
                                int64_t ldo, hipStream_t stream);
hipError_t launch_gemm_mfma(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g,
                            int M, int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                            const SegTable& st, const float* w_g, float* out, int64_t ldo,
                            hipStream_t stream);
hipError_t launch_pack_weight_gate_up(const float* w, int64_t I, int64_t K, int64_t ldw, uint8_t* w_codes,
                                      uint8_t* w_scales, float* w_g_dec, void* workspace, hipStream_t stream);
hipError_t launch_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M,
                                       int K, const uint8_t* w_codes, const uint8_t* w_scales, int I,
                                       const float* w_g, const float* amax_h, uint8_t* h_codes,
                                       uint8_t* h_scales, float* h_g_dec, hipStream_t stream);
hipError_t launch_swiglu(const float* gu, int64_t M, int64_t I, int64_t ldgu, uint16_t* h, int64_t ldh,
                         hipStream_t stream);
size_t amax_observe_workspace();
hipError_t launch_amax_observe(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float* running,
                               void* workspace, hipStream_t stream);
hipError_t launch_quantize_stats(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                 uint32_t* counts, hipStream_t stream);
// Device address of the current GPU's (or `stream`'s GPU's) copy of the
// allocation-free scratch (kScratchBytes), looked up once per device.
hipError_t scratch_for_stream(hipStream_t stream, void** out);
hipError_t launch_convert_sweep(int op, uint32_t first, int64_t n, uint8_t* out, hipStream_t stream);
hipError_t launch_kv_fp8_encode(const uint16_t* x, int64_t n, const float* amax, uint8_t* codes,
                                hipStream_t stream);
hipError_t launch_kv_fp8_decode(const uint8_t* codes, int64_t n, const float* amax, uint16_t* out,
                                hipStream_t stream);
}  // namespace nvfp4
