// Device pieces of the weight-streaming GEMMs shared by gemm_skinny.hip and
// gemm_mfma.hip: the lane's activation fragments, the weight strip pointers and
// the row-blocked GEMM over 16 MT rows (rows_block).  Operand layouts and the
// MFMA lane mapping are described at the top of gemm_skinny.hip.
#pragma once

#include <cstdint>
#include <type_traits>

#include "common.hpp"

namespace nvfp4 {

constexpr int kSkNW = 8;   // waves of the M <= 16 workgroup (sixteen where stream_waves says so)
constexpr int kSkU = 5;    // k tiles per outer iteration of a wave

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

// The caller's early load of the per-segment scales (see reduce_store): lane
// t < nseg of each wave keeps w_g[t].  Branch-free (every thread reads a valid
// entry), so the kernel's argument loads are not split around a branch at
// kernel start; issue it after the first activation and weight loads.
__device__ __forceinline__ float load_segment_scale(const float* __restrict__ w_g, const SegTable& st) {
  return w_g[min((int)(threadIdx.x & 63), st.nseg - 1)];
}

// Weight pointers of lane `lane` for the S strips starting at strip0 (clamped;
// columns past N are never stored).
template <int S>
__device__ __forceinline__ void strip_pointers(const uint8_t* w_codes, const uint8_t* w_scales, int strip0, int nstrips,
                                               int tiles, int lane, const uint8_t* (&wc)[S], const uint8_t* (&ws)[S]) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t strip = min(strip0 + s, nstrips - 1);
    wc[s] = w_codes + strip * tiles * kChunkCodes + lane * 16;
    ws[s] = w_scales + strip * tiles * kChunkScales + lane * 2;
  }
}

// ---- the same weight stream for more than 16 rows.
// Workgroup b takes strip group b % groups of the block of 16 MT rows
// b / groups: each weight fragment is decoded once and multiplied by the MT
// row tiles' activations, so the packed weight is streamed once per 16 MT rows.
// Used by nvfp4_gemm where too few 256 x 256 tiles would fill the chip for the
// MFMA GEMM.  The kernel reproduces the summation order of gemm_skinny_kernel
// with NW * VW waves on NW waves: wave w keeps VW accumulator sets, set j
// playing wave w + NW j (tile t goes to set (t / NW) % VW, so each set sees its
// tiles in the same ascending order), and the cross-wave sums of the sets are
// chained in wave order in each thread's registers.  Every accumulator thus
// sees the same MFMA sequence, and every output the same fp32 additions, as in
// the skinny kernel, so each row's result is bit-identical to that kernel's,
// while the waves stream the weight in the same order as with one set (the
// 64-row instances would not fit in the 128 VGPRs a lane has at sixteen waves).
template <int S, int NW, int MT>
__device__ __forceinline__ void reduce_rows_set(const float4_t (&acc)[S][MT], float (&red)[NW][S][MT][4][64],
                                                 float (&part)[(16 * MT * S * kStrip + 64 * NW - 1) / (64 * NW)],
                                                 int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][s][mt][i][lane] = acc[s][mt][i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < (16 * MT * S * kStrip + 64 * NW - 1) / (64 * NW); ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    if (e < rows * S * kStrip) {
      const int row = e / (S * kStrip), c = e % (S * kStrip);
      const int mt = row >> 4, rr = row & 15;
      const int s = c / kStrip, l = (rr >> 2) * kStrip + c % kStrip;
      float v = part[i];
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][s][mt][rr & 3][l];
      part[i] = v;
    }
  }
}

// Strips per workgroup of gemm_rows_kernel: every workgroup decodes its S weight
// fragments and its MT activation tiles per k tile, so the busiest CU's work is
// ceil(workgroups / 256) * (S + MT); the fewest, ties to larger S (fewer
// activation re-decodes).  E.g. N = 34816, M = 128: S = 3 (1452 workgroups).
// 16-row passes (MT = 1, outputs of at most 8 strips: rows_per_pass) may take
// four strips: the 64 ragged columns of the GDN in-projection (M = 4096) then
// run as 256 workgroups that each decode their activation rows once, 1.6 us
// faster than 512 workgroups of two strips (four alternating runs on one box,
// bit-identical).  Host code, used by the launchers of both GEMM sources.
inline int pick_strips_rows(int nstrips, int64_t blocks, int mt) {
  const int smax = mt == 1 ? 4 : 3;
  int best = smax;
  int64_t cost = 0;
  for (int s = smax; s >= 1; --s) {
    const int64_t wgs = (int64_t)(nstrips + s - 1) / s * blocks;
    const int64_t c = (wgs + kCUs - 1) / kCUs * (s + mt);
    if (s == smax || c < cost) {
      best = s;
      cost = c;
    }
  }
  return best;
}

// The workgroup body of gemm_rows_kernel for workgroup index `bid`: a kernel of
// its own (gemm_skinny.hip) or the extra workgroups of an MFMA GEMM launch that
// take its ragged last tile column (gemm_mfma.hip).  64 NW threads.
template <int S, int NW, int VW, int U, bool AL16, int MT>
__device__ __forceinline__ void rows_block(
    int bid, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_g, int M, int K, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, int N, const SegTable& st, const float* __restrict__ w_g,
    float* __restrict__ out, int64_t ldo) {
  constexpr int kDepth = 2;
  constexpr int kPer = (16 * MT * S * kStrip + 64 * NW - 1) / (64 * NW);
  static_assert(U >= kDepth, "pipeline depth");
  static_assert(VW == 1 || VW == 2, "one or two accumulator sets (eight or sixteen waves)");
  static_assert(U % VW == 0, "tile u of an outer iteration belongs to accumulator set u % VW");
  static_assert(S * kStrip <= 64, "one lane of wave 0 per column");
  __shared__ float red[NW][S][MT][4][64];
  __shared__ float scol[S * kStrip];
  const float ag = *a_g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int tiles = (K + kTileK - 1) / kTileK;
  const int full = K / kTileK;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int groups = (nstrips + S - 1) / S;
  const int rb = bid / groups;                // block of 16 MT rows
  const int strip0 = (bid - rb * groups) * S;
  const int64_t row0 = (int64_t)rb * 16 * MT;
  const int rows = (int)min((int64_t)16 * MT, (int64_t)M - row0);

  // A: row tile mt, row r (clamped; padded rows are zeroed through their scale)
  const uint8_t* ac[MT];
  const uint8_t* as[MT];
  uint32_t amask[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = 16 * mt + r;
    const int64_t arow = row0 + min(row, rows - 1);
    amask[mt] = (row < rows) ? 0xFFFFu : 0u;
    ac[mt] = a_codes + arow * (K / 2) + g * 16;
    as[mt] = a_scales + arow * (K / kBlock) + g * 2;
  }
  const uint8_t* wc[S];
  const uint8_t* ws[S];
  strip_pointers<S>(w_codes, w_scales, strip0, nstrips, tiles, lane, wc, ws);
  const float wgv = load_segment_scale(w_g, st);

  // accumulator set j of wave w plays wave w + NW j of the NW * VW-wave order:
  // tile t goes to set (t / NW) % VW
  float4_t acc[VW][S][MT];
#pragma unroll
  for (int j = 0; j < VW; ++j)
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[j][s][mt] = float4_t{0.f, 0.f, 0.f, 0.f};

  // one batch: the weight fragments of the S strips, decoded once, against the
  // MT row tiles' activation fragments (same MFMA order as tile_mfma).  With two
  // accumulator sets and more row tiles than strips, the strips' fragments are
  // decoded first and the row tiles one at a time, which holds fewer operands
  // in registers; every accumulator sees the same MFMA sequence either way.
  auto batch = [&](float4_t (&c)[S][MT], const uint4 (&av)[MT], const uint32_t (&asc)[MT], bool live,
                   const uint4 (&w)[S], const uint32_t (&wsv)[S]) {
    if constexpr (VW > 1 && MT > S) {
      half8_t B[S][4];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const half2_t s0 = scale_pair(wsv[s] & 0xFF), s1 = scale_pair(wsv[s] >> 8);
        B[s][0] = decode8(w[s].x, s0);
        B[s][1] = decode8(w[s].y, s0);
        B[s][2] = decode8(w[s].z, s1);
        B[s][3] = decode8(w[s].w, s1);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        half8_t A[4];
        decode_a(av[mt], asc[mt], live ? amask[mt] : 0u, A);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[0], B[s][0], c[s][mt], 0, 0, 0);
          c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[1], B[s][1], c[s][mt], 0, 0, 0);
          c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[2], B[s][2], c[s][mt], 0, 0, 0);
          c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[3], B[s][3], c[s][mt], 0, 0, 0);
        }
      }
      return;
    }
    half8_t A[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) decode_a(av[mt], asc[mt], live ? amask[mt] : 0u, A[mt]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const half2_t s0 = scale_pair(wsv[s] & 0xFF), s1 = scale_pair(wsv[s] >> 8);
      const half8_t B0 = decode8(w[s].x, s0), B1 = decode8(w[s].y, s0);
      const half8_t B2 = decode8(w[s].z, s1), B3 = decode8(w[s].w, s1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][0], B0, c[s][mt], 0, 0, 0);
        c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][1], B1, c[s][mt], 0, 0, 0);
        c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][2], B2, c[s][mt], 0, 0, 0);
        c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][3], B3, c[s][mt], 0, 0, 0);
      }
    }
  };

  // U tiles per iteration; the last iteration, whose tiles past the end are
  // clamped, skips their decode and MFMAs (a uniform branch, kept out of the
  // main loop so that its waits stay progressive)
  auto iteration = [&](int t0, auto guarded) {
    uint4 av[U][MT];
    uint32_t asc[U][MT];
    uint4 wv[U][S];
    uint32_t wsc[U][S];
    auto request = [&](int u) {
      const int t = min(t0 + u * NW, full - 1);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        wv[u][s] = *reinterpret_cast<const uint4*>(wc[s] + (int64_t)t * kChunkCodes);
        wsc[u][s] = *reinterpret_cast<const uint16_t*>(ws[s] + (int64_t)t * kChunkScales);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) load_a_full<AL16>(ac[mt], as[mt], t, av[u][mt], asc[u][mt]);
    };
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {              // in batch order, so that the waits stay progressive
      request(u);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!decltype(guarded)::value || t0 + u * NW < full) batch(acc[u % VW], av[u], asc[u], true, wv[u], wsc[u]);
      __builtin_amdgcn_sched_barrier(0);
      if (u + kDepth < U) request(u + kDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int t0 = wave;
  for (; t0 + (U - 1) * NW < full; t0 += NW * U) iteration(t0, std::false_type{});
  if (t0 < full) iteration(t0, std::true_type{});
  if (full < tiles && wave == full % NW) {           // ragged last tile
    const int t = full;
    uint4 av[MT], w[S];
    uint32_t asc[MT], wsv[S];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) load_a_tail(ac[mt], as[mt], t, t * kTileK + 32 * g, K, av[mt], asc[mt]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      w[s] = *reinterpret_cast<const uint4*>(wc[s] + (int64_t)t * kChunkCodes);
      wsv[s] = *reinterpret_cast<const uint16_t*>(ws[s] + (int64_t)t * kChunkScales);
    }
    if ((t / NW) % VW == 0)                          // the set of tile t
      batch(acc[0], av, asc, true, w, wsv);
    else
      batch(acc[VW - 1], av, asc, true, w, wsv);
  }

  if (wave == 0) {                                   // column scales, read after the first barrier
    const int n = min(strip0 * kStrip + min(lane, S * kStrip - 1), N - 1);
    const float wcol = __shfl(wgv, seg_of(st, n), 64);
    if (lane < S * kStrip) scol[lane] = wcol;
  }
  // cross-wave sums in the order of the NW * VW waves, chained over the sets
  float part[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) part[i] = 0.f;
#pragma unroll
  for (int j = 0; j < VW; ++j) {
    if (j > 0) __syncthreads();                      // the previous set's sums are read
    reduce_rows_set<S, NW, MT>(acc[j], red, part, rows);
  }
  float* const o = out + row0 * ldo;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + i * 64 * NW;
    if (e < rows * S * kStrip) {
      const int row = e / (S * kStrip), c = e % (S * kStrip);
      const int n = strip0 * kStrip + c;
      if (n < N) o[(int64_t)row * ldo + n] = part[i] * (ag * scol[c]);
    }
  }
}

}  // namespace nvfp4
