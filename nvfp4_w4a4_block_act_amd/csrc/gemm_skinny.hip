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

// Activation fragment of one lane for a full 128-k tile: row `row`, k in
// [t * 128 + 32 g, + 32).  Codes are 16 bytes (one 16-byte load when rows are
// 16-byte aligned, i.e. K % 32 == 0), scales two bytes.
template <bool AL16>
__device__ __forceinline__ void load_a_full(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, int t,
                                            uint4& v, uint32_t& sc) {
  if constexpr (AL16) {
    v = *reinterpret_cast<const uint4*>(ac + t * 64);
    sc = *reinterpret_cast<const uint16_t*>(as + t * 8);
  } else {
    const uint2 x0 = reinterpret_cast<const uint2*>(ac + t * 64)[0];
    const uint2 x1 = reinterpret_cast<const uint2*>(ac + t * 64)[1];
    v = make_uint4(x0.x, x0.y, x1.x, x1.y);
    sc = (uint32_t)as[t * 8] | ((uint32_t)as[t * 8 + 1] << 8);
  }
}

// Same for the ragged last tile (K % 128 != 0): zero past K (K % 16 == 0).
__device__ __forceinline__ void load_a_tail(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, int t,
                                            int k0, int K, uint4& v, uint32_t& sc) {
  v = make_uint4(0u, 0u, 0u, 0u);
  sc = 0u;
  if (k0 >= K) return;
  const uint2 x0 = reinterpret_cast<const uint2*>(ac + t * 64)[0];
  v.x = x0.x;
  v.y = x0.y;
  sc = as[t * 8];
  if (k0 + 16 < K) {
    const uint2 x1 = reinterpret_cast<const uint2*>(ac + t * 64)[1];
    v.z = x1.x;
    v.w = x1.y;
    sc |= (uint32_t)as[t * 8 + 1] << 8;
  }
}

// One 128-k tile for one strip: four 16x16x32 MFMAs on exactly decoded operands.
__device__ __forceinline__ void tile_mfma(const half8_t (&A)[4], uint4 w, uint32_t wsc, float4_t& acc) {
  const half2_t s0 = scale_pair(wsc & 0xFF), s1 = scale_pair(wsc >> 8);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], decode8(w.x, s0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], decode8(w.y, s0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2], decode8(w.z, s1), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[3], decode8(w.w, s1), acc, 0, 0, 0);
}

__device__ __forceinline__ void decode_a(uint4 v, uint32_t sc, uint32_t amask, half8_t (&A)[4]) {
  sc &= amask;                    // padded rows (m >= M) decode to zeros
  const half2_t s0 = scale_pair(sc & 0xFF), s1 = scale_pair(sc >> 8);
  A[0] = decode8(v.x, s0);
  A[1] = decode8(v.y, s0);
  A[2] = decode8(v.z, s1);
  A[3] = decode8(v.w, s1);
}

// S strips of 16 columns per workgroup, NW waves splitting the k tiles
// (wave w takes tiles w, w + NW, ...), U tiles per load batch.
template <int S, int NW, int U, bool AL16>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
  __shared__ float red[NW][S][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int tiles = (K + kTileK - 1) / kTileK;       // tiles of the packed weight
  const int full = K / kTileK;                       // tiles with no k tail
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int strip0 = blockIdx.x * S;

  // A: row r (clamped; padded rows are zeroed through their scale)
  const int arow = min(r, M - 1);
  const uint32_t amask = (r < M) ? 0xFFFFu : 0u;
  const uint8_t* ac = a_codes + (int64_t)arow * (K / 2) + g * 16;
  const uint8_t* as = a_scales + (int64_t)arow * (K / kBlock) + g * 2;
  // W: strip pointers (clamped; columns past N are never stored)
  const uint8_t* wc[S];
  const uint8_t* ws[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t strip = min(strip0 + s, nstrips - 1);
    wc[s] = w_codes + strip * tiles * kChunkCodes + lane * 16;
    ws[s] = w_scales + strip * tiles * kChunkScales + lane * 2;
  }

  float4_t acc[S];
#pragma unroll
  for (int s = 0; s < S; ++s) acc[s] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Batches of U tiles; every load of a batch is issued before any decode, and the
  // batch has no branches (tiles past the end are clamped and their activation
  // scales zeroed), so the waits before each tile's MFMAs stay progressive.
  for (int t0 = wave; t0 < full; t0 += NW * U) {
    uint4 av[U], wv[U][S];
    uint32_t asc[U], wsc[U][S];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + u * NW, full - 1);
      load_a_full<AL16>(ac, as, t, av[u], asc[u]);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        wv[u][s] = *reinterpret_cast<const uint4*>(wc[s] + (int64_t)t * kChunkCodes);
        wsc[u][s] = *reinterpret_cast<const uint16_t*>(ws[s] + (int64_t)t * kChunkScales);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t live = (t0 + u * NW < full) ? amask : 0u;
      half8_t A[4];
      decode_a(av[u], asc[u], live, A);
#pragma unroll
      for (int s = 0; s < S; ++s) tile_mfma(A, wv[u][s], wsc[u][s], acc[s]);
    }
  }
  if (full < tiles && wave == full % NW) {           // ragged last tile
    const int t = full;
    uint4 v;
    uint32_t sc;
    load_a_tail(ac, as, t, t * kTileK + 32 * g, K, v, sc);
    half8_t A[4];
    decode_a(v, sc, amask, A);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint4 w = *reinterpret_cast<const uint4*>(wc[s] + (int64_t)t * kChunkCodes);
      const uint32_t wsv = *reinterpret_cast<const uint16_t*>(ws[s] + (int64_t)t * kChunkScales);
      tile_mfma(A, w, wsv, acc[s]);
    }
  }

#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][s][i][lane] = acc[s][i];
  __syncthreads();

  // output element e = (s, i, l): row 4 * (l / 16) + i, column (strip0 + s) * 16 + l % 16
  const float ag = *a_g;
  for (int e = threadIdx.x; e < S * 256; e += 64 * NW) {
    const int s = e >> 8, i = (e >> 6) & 3, l = e & 63;
    const int row = 4 * (l >> 4) + i;
    const int n = (strip0 + s) * kStrip + (l & 15);
    if (row >= M || n >= N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][s][i][l];
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
  constexpr int S = 3, NW = 8, U = 5;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int grid = (nstrips + S - 1) / S;
  if (K % 32 == 0)
    gemm_skinny_kernel<S, NW, U, true><<<grid, 64 * NW, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes,
                                                                      w_scales, N, st, w_g, out, ldo);
  else
    gemm_skinny_kernel<S, NW, U, false><<<grid, 64 * NW, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes,
                                                                       w_scales, N, st, w_g, out, ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
