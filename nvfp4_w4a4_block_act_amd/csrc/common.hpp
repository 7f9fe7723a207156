// Shared device helpers and layout constants for the gfx950 NVFP4 kernels.
//
// NVFP4 (Summary page "Summary of 'Why Gated DeltaNet Survives 4-Bit
// Quantization'", Background, item 1): E2M1 element codes, one E4M3 scale per
// 16 elements, one FP32 scale per tensor.  Bit layouts are the OCP ones:
// E2M1 = sign | 2-bit exponent (bias 1) | 1-bit mantissa, magnitudes
// 0, .5, 1, 1.5, 2, 3, 4, 6; E4M3FN = sign | 4-bit exponent (bias 7) | 3-bit
// mantissa, subnormals m * 2^-9, largest finite 448 (0x7E).
#pragma once

#include <hip/hip_runtime.h>
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

// Segment table passed by value to the GEMM kernels: column -> module index.
struct SegTable {
  int32_t end[NVFP4_MAX_SEGMENTS];  // exclusive end column of each segment
  int32_t nseg;
};

__device__ __forceinline__ int seg_of(const SegTable& st, int n) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < NVFP4_MAX_SEGMENTS - 1; ++i)
    s += (i < st.nseg - 1 && n >= st.end[i]) ? 1 : 0;
  return s;
}

// ---- E4M3FN -----------------------------------------------------------------
// Round a non-negative binary32 s (finite or +inf) to the nearest E4M3FN
// magnitude code, ties to even mantissa, saturating at 448 (0x7E).  gfx950's
// v_cvt_pk_fp8_f32 rounds to nearest even on OCP E4M3FN; with its input clamped
// to 448 it equals this rule for every binary32 value (checked exhaustively on
// the device for all values in [0, 448], subnormals included; larger inputs and
// +inf clamp to 448).
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0x7Fu;
}

// Exact binary32 value of an E4M3FN magnitude code 0..0x7E (v_cvt_f32_fp8 is
// exact for every code, checked exhaustively on the device).
__device__ __forceinline__ float e4m3_value(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// ---- decode to fp16 ---------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// Weight chunk layout (16 rows n x 128 k): the 16 code bytes holding row n's k
// group g (k in [32g, 32g + 32)) sit at byte (g * 16 + n) * 16, the two scale
// bytes of blocks 2g, 2g + 1 at byte (g * 16 + n) * 2.  Lane l = g * 16 + n of a
// wave therefore reads bytes [16 l, 16 l + 16) of a chunk: one fully coalesced
// 1 KB wave load that lands in the 16 x 16 x 32 MFMA operand layout.
__host__ __device__ inline int64_t chunk_code_off(int n, int g) { return (int64_t)(g * kStrip + n) * 16; }
__host__ __device__ inline int64_t chunk_scale_off(int n, int g) { return (int64_t)(g * kStrip + n) * 2; }

// fp16 bit pattern (c << 7) read as an IEEE half is exactly E4M3(c) * 2^-8 for
// every code 0..0x7E (normal codes map onto fp16 normals, E4M3 subnormals onto
// fp16 subnormals).  scale_pair(c) puts that half in both lanes of a half2.
__device__ __forceinline__ half2_t scale_pair(uint32_t c) {
  const uint32_t b = (c & 0x7Fu) * 0x00800080u;           // (c << 7) | (c << 23)
  return __builtin_bit_cast(half2_t, b);
}

// 8 E2M1 codes (one dword, low nibble first) times one E4M3 scale as 8 exact
// fp16 values.  The fp4 converter with scale 2^8 yields E2M1 * 256 exactly;
// the packed fp16 multiply by E4M3 * 2^-8 then gives E2M1 * E4M3, exact because
// every such product has at most 6 significant bits and lies in [2^-10, 2688],
// inside fp16's normal range.
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t s2) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s2;
  const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint32_t u4_dword_sel(uint4 v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

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
hipError_t launch_kv_fp8_encode(const uint16_t* x, int64_t n, const float* amax, uint8_t* codes,
                                hipStream_t stream);
hipError_t launch_kv_fp8_decode(const uint8_t* codes, int64_t n, const float* amax, uint16_t* out,
                                hipStream_t stream);
}  // namespace nvfp4
