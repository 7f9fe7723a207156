// Decode-form W4A4 GEMM (M <= 16): weight-streaming, HBM-bound.
//
// out[m][n] = fl(acc * fl(a_g * w_g[seg(n)])) with acc the fp32 sum over k of
// exact E2M1*E4M3 products -- the W4A4 GEMM on NVFP4 operands (Summary page,
// Background, item 1) with the per-module global-scale epilogue that repairs
// the fused-GEMM scale mismatch (paper abstract; Glonce article, "Who it
// affects"; aiany page, "Mechanistic notes").
//
// Design (gfx950):
//  * each weight byte is read from HBM exactly once: 0.5625 B per weight
//    (codes + scales); a workgroup of four waves owns `SW` strips of 16 output
//    columns, and its waves split the K tiles of those strips (split-K inside
//    the workgroup, reduced through LDS), so ~1.5 waves per SIMD each keep
//    several KB of independent 16-byte loads in flight;
//  * the 16 x 16 x 32 fp16 MFMA does the arithmetic with M padded to 16:
//    lane l holds row/column l % 16 and the 32 k of group g = l / 16 of a
//    128-k tile.  A K-permutation shared by both operands makes each lane's
//    operand bytes contiguous: MFMA j of a tile covers k = 32g + 8j + e, so a
//    lane's 16-byte load of canonical codes feeds four MFMAs.  Both operands
//    are decoded exactly to fp16 in registers (fp4 converter + packed fp16
//    multiply by the E4M3 scale); no LDS staging, since each weight is used
//    once;
//  * the epilogue applies the per-segment scale during the cross-wave sum.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

constexpr int kSkWaves = 4;
constexpr int kSkThreads = 64 * kSkWaves;

// 16 contiguous code bytes (32 elements) of activation row m starting at
// element k0; zero past K.  `al16` says whether rows start 16-byte aligned.
__device__ __forceinline__ uint4 load_act_codes(const uint8_t* __restrict__ a, int64_t m, int K, int k0,
                                                bool al16) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (k0 >= K) return v;
  const uint8_t* p = a + m * (K / 2) + k0 / 2;
  if (k0 + 32 <= K) {
    if (al16) {
      v = *reinterpret_cast<const uint4*>(p);
    } else {
      const uint2 x0 = reinterpret_cast<const uint2*>(p)[0];
      const uint2 x1 = reinterpret_cast<const uint2*>(p)[1];
      v = make_uint4(x0.x, x0.y, x1.x, x1.y);
    }
  } else {  // k0 + 16 == K: the last block of the row
    const uint2 x0 = *reinterpret_cast<const uint2*>(p);
    v.x = x0.x;
    v.y = x0.y;
  }
  return v;
}

// Two scale bytes (blocks k0/16 and k0/16 + 1) of activation row m; zero past K.
__device__ __forceinline__ uint32_t load_act_scales(const uint8_t* __restrict__ s, int64_t m, int K, int k0) {
  if (k0 >= K) return 0u;
  const uint8_t* p = s + m * (K / kBlock) + k0 / kBlock;
  uint32_t r = p[0];
  if (k0 + 16 < K) r |= (uint32_t)p[1] << 8;
  return r;
}

template <int SW, int U>
__global__ __launch_bounds__(kSkThreads) void gemm_skinny_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
  __shared__ float red[kSkWaves][SW][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int tiles = (K + kTileK - 1) / kTileK;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int strip0 = blockIdx.x * SW;
  const bool arow = r < M;
  const bool al16 = (K % 32) == 0;

  float4_t acc[SW];
#pragma unroll
  for (int s = 0; s < SW; ++s) acc[s] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = wave; t0 < tiles; t0 += kSkWaves * U) {
    uint4 av[U], wv[U][SW];
    uint32_t as[U], ws[U][SW];
    // issue every load of this batch first
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * kSkWaves;
      const int k0 = t * kTileK + 32 * g;
      const bool tv = t < tiles;
      av[u] = (tv && arow) ? load_act_codes(a_codes, r, K, k0, al16) : make_uint4(0u, 0u, 0u, 0u);
      as[u] = (tv && arow) ? load_act_scales(a_scales, r, K, k0) : 0u;
#pragma unroll
      for (int s = 0; s < SW; ++s) {
        const int strip = strip0 + s;
        if (tv && strip < nstrips) {
          const int64_t chunk = (int64_t)strip * tiles + t;
          wv[u][s] = *reinterpret_cast<const uint4*>(w_codes + chunk * kChunkCodes + r * 64 + g * 16);
          ws[u][s] = *reinterpret_cast<const uint16_t*>(w_scales + chunk * kChunkScales + r * 8 + g * 2);
        } else {
          wv[u][s] = make_uint4(0u, 0u, 0u, 0u);
          ws[u][s] = 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const half2_t sa0 = scale_h2(as[u] & 0xFF), sa1 = scale_h2(as[u] >> 8);
      const half8_t A0 = decode8(av[u].x, sa0), A1 = decode8(av[u].y, sa0);
      const half8_t A2 = decode8(av[u].z, sa1), A3 = decode8(av[u].w, sa1);
#pragma unroll
      for (int s = 0; s < SW; ++s) {
        const half2_t sb0 = scale_h2(ws[u][s] & 0xFF), sb1 = scale_h2(ws[u][s] >> 8);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, decode8(wv[u][s].x, sb0), acc[s], 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, decode8(wv[u][s].y, sb0), acc[s], 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, decode8(wv[u][s].z, sb1), acc[s], 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, decode8(wv[u][s].w, sb1), acc[s], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int s = 0; s < SW; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][s][i][lane] = acc[s][i];
  __syncthreads();

  // thread -> (i, l): output row 4 * (l / 16) + i, column l % 16 of each strip
  const int i = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int row = 4 * (l >> 4) + i;
  if (row >= M) return;
  const float ag = *a_g;
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const int n = (strip0 + s) * kStrip + (l & 15);
    if (n >= N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) v += red[w][s][i][l];
    out[(int64_t)row * ldo + n] = v * (ag * w_g[seg_of(st, n)]);
  }
}

__global__ void fill_zero_kernel(float* __restrict__ out, int M, int N, int64_t ldo) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x)
    out[(i / N) * ldo + i % N] = 0.0f;
}

hipError_t launch_fill_zero(float* out, int M, int N, int64_t ldo, hipStream_t stream) {
  const int64_t total = (int64_t)M * N;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
  fill_zero_kernel<<<grid, 256, 0, stream>>>(out, M, N, ldo);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M,
                              int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                              const SegTable& st, const float* w_g, float* out, int64_t ldo,
                              hipStream_t stream) {
  constexpr int SW = 2, U = 5;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int grid = (nstrips + SW - 1) / SW;
  gemm_skinny_kernel<SW, U><<<grid, kSkThreads, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes, w_scales,
                                                             N, st, w_g, out, ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
