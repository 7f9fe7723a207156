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
// MFMA computes exact products with fp32 accumulation at the dense fp16 rate.
//
// Tiling (512 threads, 256 x 256 output tile, k tile 128):
//  * eight waves in a 4 (M) x 2 (N) grid, each owning 64 x 128 = 2 x 4 MFMA
//    32x32x16 tiles (128 fp32 accumulators per lane);
//  * activations are decoded straight into MFMA operand registers by the wave
//    that uses them: under a K-permutation shared by both operands (MFMA step
//    j of a tile takes k = 64 h + 8 j + e for lane group h = lane / 32), each
//    lane's operand bytes are 32 contiguous bytes of a canonical row, loaded
//    one k tile ahead;
//  * weights (shared by the four M-waves) are loaded two k tiles ahead as
//    fully coalesced 1 KB chunk reads, decoded once per workgroup to fp16 and
//    written to a double-buffered LDS tile (row stride 272 bytes: the 16-byte
//    operand reads of 16 consecutive lanes hit distinct banks); the decode of
//    tile t + 1 is interleaved with the MFMAs of tile t;
//  * workgroups are numbered XCD-major, then in groups of four row panels, so
//    the 32 workgroups resident on an XCD share one activation slab in its L2
//    while they stream weight column panels.
#include "common.hpp"

namespace nvfp4 {

constexpr int kBM = 256, kBN = 256;
constexpr int kMfWaves = 8, kMfThreads = 64 * kMfWaves;
constexpr int kLdsRow = kTileK + 8;                  // halfs per LDS row
constexpr int kGroupM = 4;

struct RawA {                                          // one lane's activation bytes for one k tile
  uint4 c[2][2];                                       // [row tile][16-byte half]
  uint32_t s[2];                                       // 4 scale bytes per row tile
};

struct RawW {                                          // one thread's two weight slots for one k tile
  uint4 c[2];
  uint32_t s[2];
};

template <bool AL>
__device__ __forceinline__ void load_a_tile(const uint8_t* const (&ap)[2], const uint8_t* const (&asp)[2], int t,
                                            RawA& r) {
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const uint8_t* p = ap[rt] + (int64_t)t * 64;
    const uint8_t* q = asp[rt] + (int64_t)t * 8;
    if constexpr (AL) {
      r.c[rt][0] = reinterpret_cast<const uint4*>(p)[0];
      r.c[rt][1] = reinterpret_cast<const uint4*>(p)[1];
      r.s[rt] = *reinterpret_cast<const uint32_t*>(q);
    } else {
      const uint2* p2 = reinterpret_cast<const uint2*>(p);
      const uint2 x0 = p2[0], x1 = p2[1], x2 = p2[2], x3 = p2[3];
      r.c[rt][0] = make_uint4(x0.x, x0.y, x1.x, x1.y);
      r.c[rt][1] = make_uint4(x2.x, x2.y, x3.x, x3.y);
      r.s[rt] = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
    }
  }
}

// Ragged last tile: per 16-element block, load only blocks that start before K.
__device__ __forceinline__ void load_a_tail(const uint8_t* const (&ap)[2], const uint8_t* const (&asp)[2], int t,
                                            int kbase, int K, RawA& r) {
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const uint8_t* p = ap[rt] + (int64_t)t * 64;
    const uint8_t* q = asp[rt] + (int64_t)t * 8;
    uint32_t d[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t s = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (kbase + 16 * b < K) {
        const uint2 x = reinterpret_cast<const uint2*>(p)[b];
        d[2 * b] = x.x;
        d[2 * b + 1] = x.y;
        s |= (uint32_t)q[b] << (8 * b);
      }
    }
    r.c[rt][0] = make_uint4(d[0], d[1], d[2], d[3]);
    r.c[rt][1] = make_uint4(d[4], d[5], d[6], d[7]);
    r.s[rt] = s;
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4 (&c)[2], int j) {
  const uint4 v = c[j >> 2];
  switch (j & 3) {
    case 0: return v.x;
    case 1: return v.y;
    case 2: return v.z;
    default: return v.w;
  }
}

template <bool AL>
__global__ __launch_bounds__(kMfThreads, 1) void gemm_mfma_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) _Float16 sB[2][kBN * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles = (K + kTileK - 1) / kTileK, full = K / kTileK;
  const int nstrips = (N + kStrip - 1) / kStrip;

  // ---- workgroup -> output tile: XCD-major numbering, then grouped row panels
  const int num_m = (M + kBM - 1) / kBM, num_n = (N + kBN - 1) / kBN;
  const int nwg = num_m * num_n;
  int pid = blockIdx.x;
  if (nwg % 8 == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int per_group = kGroupM * num_n;
  const int first_m = (pid / per_group) * kGroupM;
  const int gsz = min(num_m - first_m, kGroupM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * kBM, n0 = tn * kBN;

  // ---- activation lane constants: rows m0 + wm*64 + rt*32 + i, k group h
  const int i = lane & 31, h = lane >> 5;
  const uint8_t* ap[2];
  const uint8_t* asp[2];
  uint32_t amask[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = m0 + wm * 64 + rt * 32 + i;
    const int rc = min(row, M - 1);
    ap[rt] = a_codes + (int64_t)rc * (K / 2) + 32 * h;
    asp[rt] = a_scales + (int64_t)rc * (K / kBlock) + 4 * h;
    amask[rt] = row < M ? 0xFFFFFFFFu : 0u;    // padded rows decode to zeros
  }
  // ---- weight slots: slot q = tid + 512 * s covers strip q / 64, chunk lane q % 64
  const uint8_t* wp[2];
  const uint8_t* wsp[2];
  int woff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int q = tid + kMfThreads * s;
    const int64_t strip = min(n0 / kStrip + (q >> 6), nstrips - 1);
    const int c = q & 63;
    wp[s] = w_codes + strip * tiles * kChunkCodes + c * 16;
    wsp[s] = w_scales + strip * tiles * kChunkScales + c * 2;
    woff[s] = ((q >> 6) * kStrip + (c & 15)) * kLdsRow + (c >> 4) * 32;   // LDS row n, k group g
  }

  auto load_w = [&](int t, RawW& r) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      r.c[s] = *reinterpret_cast<const uint4*>(wp[s] + (int64_t)t * kChunkCodes);
      r.s[s] = *reinterpret_cast<const uint16_t*>(wsp[s] + (int64_t)t * kChunkScales);
    }
  };
  auto store_w_part = [&](const RawW& r, int stage, int part) {   // part 0..7: slot part/4, dword part%4
    const int s = part >> 2, d = part & 3;
    const uint32_t sc = (d < 2) ? (r.s[s] & 0xFF) : (r.s[s] >> 8);
    const uint32_t w = (d == 0) ? r.c[s].x : (d == 1) ? r.c[s].y : (d == 2) ? r.c[s].z : r.c[s].w;
    *reinterpret_cast<half8_t*>(&sB[stage][woff[s] + 8 * d]) = decode8(w, scale_pair(sc));
  };
  auto load_a = [&](int t, RawA& r) {
    if (t < full) load_a_tile<AL>(ap, asp, t, r);
    else load_a_tail(ap, asp, t, t * kTileK + 64 * h, K, r);
  };

  float16_t acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rt][c][r] = 0.f;

  RawA ra0, ra1;
  RawW rw0, rw1;
  load_a(0, ra0);
  load_w(0, rw0);
  if (tiles > 1) load_w(1, rw1);
#pragma unroll
  for (int p = 0; p < 8; ++p) store_w_part(rw0, 0, p);
  __syncthreads();

  const int brow = wn * 128 + i;                       // this lane's B row within the tile (+ 32 c)
  // One k tile: MFMAs on tile t (activations in `acur`, weights in LDS stage t & 1)
  // while tile t + 1's activations load into `anext`, tile t + 2's weights into
  // `wload` and tile t + 1's weights (`wstore`) are decoded into the other stage.
  auto step = [&](int t, const RawA& acur, RawA& anext, RawW& wload, const RawW& wstore) {
    const int cur = t & 1;
    if (t + 1 < tiles) load_a(t + 1, anext);
    if (t + 2 < tiles) load_w(t + 2, wload);
    const _Float16* B = sB[cur];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half8_t af[2], bf[4];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const uint32_t sc = (acur.s[rt] & amask[rt]) >> (8 * (j >> 1));
        af[rt] = decode8(dword_of(acur.c[rt], j), scale_pair(sc & 0xFF));
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        bf[c] = *reinterpret_cast<const half8_t*>(&B[(brow + 32 * c) * kLdsRow + 64 * h + 8 * j]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[rt][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[rt], bf[c], acc[rt][c], 0, 0, 0);
      if (t + 1 < tiles) store_w_part(wstore, cur ^ 1, j);
    }
    __syncthreads();
  };
  for (int t = 0; t < tiles; t += 2) {
    step(t, ra0, ra1, rw0, rw1);
    if (t + 1 < tiles) step(t + 1, ra1, ra0, rw1, rw0);
  }

  // ---- epilogue: lane holds rows 8*(r/4) + 4*h + r%4, column i of each 32x32 tile
  const float ag = *a_g;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int n = n0 + wn * 128 + 32 * c + i;
    if (n >= N) continue;
    const float alpha = ag * w_g[seg_of(st, n)];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) out[(int64_t)m * ldo + n] = acc[rt][c][r] * alpha;
      }
  }
}

hipError_t launch_gemm_mfma(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M, int K,
                            const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                            const float* w_g, float* out, int64_t ldo, hipStream_t stream) {
  const int grid = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (K % 64 == 0)
    gemm_mfma_kernel<true><<<grid, kMfThreads, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes, w_scales, N,
                                                            st, w_g, out, ldo);
  else
    gemm_mfma_kernel<false><<<grid, kMfThreads, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes, w_scales, N,
                                                             st, w_g, out, ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
