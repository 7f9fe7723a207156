// Device-side NVFP4 encode steps shared by the activation quantizer, the weight
// packer and the one-launch decode-form linear kernel.
//
// The rule (Summary page "Summary of 'Why Gated DeltaNet Survives 4-Bit
// Quantization'", Background, item 1, with the readings stated in
// include/nvfp4.h): the per-tensor scale maps the tensor maximum onto 6 * 448;
// per 16-element block t = fl(bmax / 6), s = fl(t * g_enc), scale = E4M3 RNE of
// s (saturating, t == 0 gives 0); per element y = fl(|x| * fl(g_enc / s_dec)),
// code = E2M1 RNE of y (saturating at 6) with the sign of x.  Files including
// this header are built with -ffp-contract=off and correctly rounded fp32
// division, so every step is one binary32 rounding.
#pragma once

#include "common.hpp"

namespace nvfp4 {

// ---- block encoder ------------------------------------------------------------
// x: the 16 values of one block as binary32 (exactly widened), bmax = max|x|.
// Returns the E4M3 scale code; writes the 16 element codes (8 bytes) to out.
__device__ __forceinline__ uint32_t encode_block(const float (&x)[16], float bmax, float g_enc,
                                                 uint2& out) {
  const float t = bmax / 6.0f;
  const uint32_t sc = (t != 0.0f) ? e4m3_encode_rne_sat(t * g_enc) : 0u;
  const float sdec = e4m3_value(sc);
  // sdec == 0: every magnitude is 0; x * 0 keeps the sign bit, which the fp4
  // converter then emits on its own.
  const float rb = (sdec != 0.0f) ? g_enc / sdec : 0.0f;
  float y[16];
  if (__builtin_isinf(rb)) {
    // g_enc overflowed (tensor maximum below ~1e-35): 0 * inf would be NaN,
    // but a zero element encodes to magnitude 0.
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = (x[i] == 0.0f) ? x[i] : x[i] * rb;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = x[i] * rb;
  }
  uint32_t lo = 0, hi = 0;
  lo = e2m1_pack_pair<0>(lo, y[0], y[1]);
  lo = e2m1_pack_pair<1>(lo, y[2], y[3]);
  lo = e2m1_pack_pair<2>(lo, y[4], y[5]);
  lo = e2m1_pack_pair<3>(lo, y[6], y[7]);
  hi = e2m1_pack_pair<0>(hi, y[8], y[9]);
  hi = e2m1_pack_pair<1>(hi, y[10], y[11]);
  hi = e2m1_pack_pair<2>(hi, y[12], y[13]);
  hi = e2m1_pack_pair<3>(hi, y[14], y[15]);
  out = make_uint2(lo, hi);
  return sc;
}

// Per-tensor encode factor from amax; amax == 0 makes every block's scale 0.
__device__ __forceinline__ float g_enc_of(float amax) {
  return (amax == 0.0f) ? 0.0f : kGMax / amax;
}

// ---- |x| maximum of bf16 data on bit patterns ------------------------------------
// For finite bf16, |x| orders exactly like (bits & 0x7FFF) as an unsigned
// integer; the two halves of a word are compared with one packed 16-bit max.
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2_t absmax_pk(uint4 v, u16x2_t m) {
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu));
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu));
}

// max(m, largest |x| bit pattern among the 8 bf16 of v)
__device__ __forceinline__ uint32_t absmax_bits(uint4 v, uint32_t m) {
  const u16x2_t p = absmax_pk(v, u16x2_t{0, 0});
  return max(m, (uint32_t)max(p.x, p.y));
}

// ---- fast exact encoder for bf16 blocks ------------------------------------------
// Both divisions of the rule are done as a multiply by a correctly rounded
// reciprocal y = RN(1/d) followed by Markstein's correction (P. Markstein, "Computation
// of elementary functions on the IBM RISC System/6000 processor", IBM J. Res. Dev.
// 34(1), 1990): q = RN(a y), r = a - d q (exact with a fused multiply-add),
// q' = RN(q + r y) = RN(a / d).  Exhaustive checks (the CPU test suite rebuilds
// them) confirm it for a = every bf16 value with d = 6, and for every binary32
// significand a with d = every E4M3 significand.  The second division is only
// taken through this path while g_enc lies in [2^-60, 2^60], so that no
// quotient or remainder leaves the normal range; other tensors (amax outside
// about [2.3e-15, 3.1e21]) use the plain correctly rounded divisions.
constexpr float kRcp6 = 0x1.555556p-3f;     // RN(1/6)

__device__ __forceinline__ float div_rn(float a, float d, float y) {
  const float q = a * y;
  const float r = __builtin_fmaf(-d, q, a);
  return __builtin_fmaf(r, y, q);
}

// rtab[c] = RN(1 / E4M3 value of c) for the codes 1..126; rtab[0] = 0 turns a
// zero scale into rb = 0 (q = 0, r = a, q' = a * 0 = 0).  Filled by the first
// 128 threads; the caller synchronizes before use.
__device__ __forceinline__ void fill_rcp_table(float* rtab) {
  const int c = threadIdx.x;
  if (c < 128) rtab[c] = (c == 0 || c == 127) ? 0.0f : 1.0f / e4m3_value(c);
}

// Per-tensor encode context; `fast` must be uniform across the workgroup.
struct EncCtx {
  float g_enc;
  bool fast;
  const float* rtab;   // LDS reciprocal table
};

__device__ __forceinline__ EncCtx make_ctx(float amax, const float* rtab) {
  const float g = g_enc_of(amax);
  const uint32_t gb = __builtin_amdgcn_readfirstlane(__float_as_uint(g));
  const float gu = __uint_as_float(gb);
  return EncCtx{gu, gu >= 0x1p-60f && gu <= 0x1p60f, rtab};
}

// Encode one bf16 block given as two 16-byte chunks (element 2 i in the low
// half of word i): returns the scale code and the 8 code bytes in `c`.  Works
// pair by pair on the packed words to keep few values live.
#define NVFP4_PAIR(W, I, SEL, MUL) \
  W = e2m1_pack_pair<SEL>(W, MUL(__uint_as_float(d[I] << 16)), MUL(__uint_as_float(d[I] & 0xFFFF0000u)))
#define NVFP4_PAIRS(MUL)                                                                               \
  NVFP4_PAIR(lo, 0, 0, MUL); NVFP4_PAIR(lo, 1, 1, MUL); NVFP4_PAIR(lo, 2, 2, MUL);                   \
  NVFP4_PAIR(lo, 3, 3, MUL); NVFP4_PAIR(hi, 4, 0, MUL); NVFP4_PAIR(hi, 5, 1, MUL);                   \
  NVFP4_PAIR(hi, 6, 2, MUL); NVFP4_PAIR(hi, 7, 3, MUL)
#define NVFP4_MUL(v) ((v) * rb)
#define NVFP4_MUL_KEEP_ZERO(v) (((v) == 0.0f) ? (v) : (v) * rb)

// Same, given the block's |x| maximum as a bf16 bit pattern (absmax_bits of the
// two chunks), for callers that already have it.
__device__ __forceinline__ uint32_t encode_bf16_block_max(uint4 v0, uint4 v1, uint32_t bmax_bits, const EncCtx& cx,
                                                          uint2& c) {
  const uint32_t d[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  const float bmax = __uint_as_float(bmax_bits << 16);
  uint32_t lo = 0, hi = 0, sc;
  if (__builtin_expect(cx.fast, 1)) {   // keeps the rare exact-division path out of line
    const float t = div_rn(bmax, 6.0f, kRcp6);
    sc = e4m3_encode_rne_sat(t * cx.g_enc);   // t == 0 gives code 0
    const float rb = div_rn(cx.g_enc, e4m3_value(sc), cx.rtab[sc]);
    NVFP4_PAIRS(NVFP4_MUL);
  } else {
    // the rule with plain correctly rounded divisions (see encode_block)
    const float t = bmax / 6.0f;
    sc = (t != 0.0f) ? e4m3_encode_rne_sat(t * cx.g_enc) : 0u;
    const float sdec = e4m3_value(sc);
    const float rb = (sdec != 0.0f) ? cx.g_enc / sdec : 0.0f;
    if (__builtin_isinf(rb)) {
      NVFP4_PAIRS(NVFP4_MUL_KEEP_ZERO);
    } else {
      NVFP4_PAIRS(NVFP4_MUL);
    }
  }
  c = make_uint2(lo, hi);
  return sc;
}

__device__ __forceinline__ uint32_t encode_bf16_block(uint4 v0, uint4 v1, const EncCtx& cx, uint2& c) {
  return encode_bf16_block_max(v0, v1, absmax_bits(v0, absmax_bits(v1, 0u)), cx, c);
}
#undef NVFP4_MUL_KEEP_ZERO
#undef NVFP4_MUL
#undef NVFP4_PAIRS
#undef NVFP4_PAIR

// Same, storing 8 code bytes and 1 scale byte.
__device__ __forceinline__ void encode_bf16_chunks(uint4 v0, uint4 v1, const EncCtx& cx,
                                                   uint8_t* __restrict__ code_dst, uint8_t* __restrict__ scale_dst) {
  uint2 c;
  const uint32_t sc = encode_bf16_block(v0, v1, cx, c);
  *reinterpret_cast<uint2*>(code_dst) = c;
  *scale_dst = (uint8_t)sc;
}

__device__ __forceinline__ uint32_t block_reduce_max(uint32_t v, uint32_t* red) {

#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = max(r, red[i]);
  __syncthreads();
  return r;
}


}  // namespace nvfp4
