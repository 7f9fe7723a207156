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
constexpr int kDecMaxM = 16;                // rows of the one-launch decode layer
constexpr size_t kScratchBytes = kPartials * sizeof(uint32_t) + 16;   // nvfp4_linear_noalloc's scratch
constexpr int kMaxDevices = 64;             // GPUs whose scratch address is cached

// k tiles per wave (U) of the one-launch decode layer for an M x K input, 0
// when it has no instance: the wave-private activation area (MAXM * U tiles of
// 80 bytes) must fit LDS and the lane's block registers (MAXM * U / 8 steps of
// two 16-byte chunks) the register file, so longer K takes fewer rows.
inline int decode_tiles_per_wave(int64_t M, int64_t K) {
  if (K <= 8 * 5 * kTileK) return 5;               // K <= 5120: every row bound
  if (K <= 8 * 10 * kTileK && M <= 8) return 10;   // K <= 10240
  if (K <= 8 * 20 * kTileK && M <= 4) return 20;   // K <= 20480
  return 0;
}

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
