// Prefill-form W4A4 GEMM (M > 16): matrix-core bound.
//
// Same result as the skinny path: out = fl(acc * fl(a_g * w_g[seg(n)])), acc
// the fp32 sum of exact E2M1*E4M3 products (Summary page, Background, item 1;
// per-module epilogue from the paper abstract and the Glonce article, "Who it
// affects").
//
// Why fp16 MFMA and not the fp4 MFMA: gfx950's block-scaled fp4 MFMA takes one
// power-of-two (E8M0) scale per 32 k, while NVFP4 carries a non-power-of-two
// E4M3 scale per 16 k.  Decoding E2M1 x E4M3 to fp16 is exact (every product
// has at most 6 significant bits and lies in [2^-10, 2688]), so the 16-bit
// MFMA computes exact products with fp32 accumulation, at the dense fp16 rate.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile; its four
// waves each own 64 x 64 (2 x 2 MFMA 32x32x16 tiles).  Per 128-k tile the
// workgroup loads 8 KB of activation codes (canonical rows) and eight 1 KB
// weight chunks (+ scales), decodes them once to fp16 into LDS (row stride
// padded by 16 bytes so the 16-byte operand reads of 8 consecutive rows hit
// distinct banks), and double-buffers LDS so the next tile's global loads and
// decode overlap the current tile's MFMAs.
#include "common.hpp"

namespace nvfp4 {

constexpr int kBM = 128, kBN = 128;
constexpr int kLdsRow = kTileK + 8;          // halfs per LDS row (272 bytes)
constexpr int kMfThreads = 256;

__device__ __forceinline__ uint4 ld_act16(const uint8_t* __restrict__ a, int64_t m, int K, int k0, bool al16) {
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
  } else {
    const uint2 x0 = *reinterpret_cast<const uint2*>(p);
    v.x = x0.x;
    v.y = x0.y;
  }
  return v;
}

__device__ __forceinline__ uint32_t ld_act_sc2(const uint8_t* __restrict__ s, int64_t m, int K, int k0) {
  if (k0 >= K) return 0u;
  const uint8_t* p = s + m * (K / kBlock) + k0 / kBlock;
  uint32_t r = p[0];
  if (k0 + 16 < K) r |= (uint32_t)p[1] << 8;
  return r;
}

// Decode one 32-element unit (16 code bytes, 2 scale bytes) into an LDS row segment.
__device__ __forceinline__ void decode_unit_to_lds(uint4 v, uint32_t sc, _Float16* dst) {
  const half2_t s0 = scale_h2(sc & 0xFF), s1 = scale_h2((sc >> 8) & 0xFF);
  half8_t* d = reinterpret_cast<half8_t*>(dst);
  d[0] = decode8(v.x, s0);
  d[1] = decode8(v.y, s0);
  d[2] = decode8(v.z, s1);
  d[3] = decode8(v.w, s1);
}

__global__ __launch_bounds__(kMfThreads, 1) void gemm_mfma_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) _Float16 sA[2][kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) _Float16 sB[2][kBN * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles = (K + kTileK - 1) / kTileK;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int tiles_n = (N + kBN - 1) / kBN;
  // workgroup -> output tile, column-tile fastest so concurrently running
  // workgroups share the same activation rows
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const bool al16 = (K % 32) == 0;

  // loader units: u = tid and tid + 256; activation unit = (row u/4, group u%4),
  // weight unit = (strip u/64, row (u/4)%16, group u%4)
  uint4 ra[2], rw[2];
  uint32_t rsa[2], rsw[2];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = tid + h * kMfThreads;
      const int row = u >> 2, g = u & 3;
      const int k0 = t * kTileK + 32 * g;
      const int m = m0 + row;
      const bool mv = m < M;
      ra[h] = mv ? ld_act16(a_codes, m, K, k0, al16) : make_uint4(0u, 0u, 0u, 0u);
      rsa[h] = mv ? ld_act_sc2(a_scales, m, K, k0) : 0u;
      const int strip = n0 / kStrip + (u >> 6);
      const int r = (u >> 2) & 15;
      if (strip < nstrips) {
        const int64_t chunk = (int64_t)strip * tiles + t;
        rw[h] = *reinterpret_cast<const uint4*>(w_codes + chunk * kChunkCodes + r * 64 + g * 16);
        rsw[h] = *reinterpret_cast<const uint16_t*>(w_scales + chunk * kChunkScales + r * 8 + g * 2);
      } else {
        rw[h] = make_uint4(0u, 0u, 0u, 0u);
        rsw[h] = 0u;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = tid + h * kMfThreads;
      const int row = u >> 2, g = u & 3;
      decode_unit_to_lds(ra[h], rsa[h], &sA[buf][row * kLdsRow + 32 * g]);
      decode_unit_to_lds(rw[h], rsw[h], &sB[buf][row * kLdsRow + 32 * g]);
    }
  };

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int lrow = lane & 31, lk = 8 * (lane >> 5);
  for (int t = 0; t < tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < tiles) load_tile(t + 1);
    const _Float16* A = sA[buf];
    const _Float16* B = sB[buf];
#pragma unroll
    for (int kk = 0; kk < kTileK / 16; ++kk) {
      half8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&A[(wm * 64 + i * 32 + lrow) * kLdsRow + kk * 16 + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(&B[(wn * 64 + j * 32 + lrow) * kLdsRow + kk * 16 + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (t + 1 < tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of each 32x32 tile
  const float ag = *a_g;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + lrow;
    if (n >= N) continue;
    const float alpha = ag * w_g[seg_of(st, n)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M) out[(int64_t)m * ldo + n] = acc[i][j][r] * alpha;
      }
  }
}

hipError_t launch_gemm_mfma(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M, int K,
                            const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                            const float* w_g, float* out, int64_t ldo, hipStream_t stream) {
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  gemm_mfma_kernel<<<tiles_m * tiles_n, kMfThreads, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes, w_scales,
                                                                 N, st, w_g, out, ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
