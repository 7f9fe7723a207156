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
//    (codes + scales); a workgroup of eight waves (sixteen for some long-K
//    shapes, as stream_waves sets) owns S strips of 16 output columns (S = 1..3
//    chosen per N by skinny_strips: 3 for N = 12288, i.e. 256 workgroups, one
//    per CU), and its waves split the K tiles of those strips
//    (split-K inside the workgroup, reduced through LDS); each wave keeps two
//    batches (one k tile of the S strips each) in flight, requesting batch
//    u + 2 after the MFMAs of batch u;
//  * the 16 x 16 x 32 fp16 MFMA does the arithmetic with M padded to 16:
//    lane l holds row/column l % 16 and the 32 k of group g = l / 16 of a
//    128-k tile.  A K-permutation shared by both operands makes each lane's
//    operand bytes contiguous: MFMA j of a tile covers k = 32g + 8j + e, so a
//    lane's 16-byte load of canonical codes feeds four MFMAs.  Both operands
//    are decoded exactly to fp16 in registers (fp4 converter + packed fp16
//    multiply by the E4M3 scale); no LDS staging, since each weight is used
//    once;
//  * the weight loads of the M <= 16 kernels carry the non-temporal hint (each
//    byte is read once per call, and a model's weights do not fit the
//    last-level cache between calls): 0.4-0.8 us faster per call at K = 5120,
//    N = 12288.  The row-blocked kernel keeps plain loads: its later row passes
//    find the weight in the last-level cache (the hint made M = 256 12% slower);
//  * the epilogue applies the per-segment scale during the cross-wave sum;
//  * for decode-sized activations a second kernel also quantizes them inside
//    the same launch (linear_decode_kernel below).
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "common.hpp"
#include "quant_device.hpp"

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

// Cross-wave sum of the per-wave partial tiles and the epilogue.  Only live
// outputs are visited: e = row * (16 S) + c for row < M, c = 16 s + l % 16, so
// consecutive threads store consecutive columns of one row.  MFMA lane l holds
// rows 4 (l / 16) + i in acc[s][i], i.e. output (row, c) is partial
// red[w][s][row % 4][16 (row / 4) + c % 16] of wave w.  The result is
// fl(sum * fl(a_g * w_g[seg(n)])).  The per-segment scales were loaded at
// kernel start (wgv: lane t < nseg of every wave holds w_g[t]) so the epilogue
// does not wait on memory behind the weight stream; wave 0 turns them into
// column scales (one cross-lane read per column) before the barrier, while the
// other waves finish their tiles, and they reach the other threads through LDS
// with the partial tiles.
template <int S, int NW>
__device__ __forceinline__ void reduce_store(const float4_t (&acc)[S], float (&red)[NW][S][4][64],
                                             float (&scol)[S * kStrip], float wgv, int strip0, int M, int N,
                                             const SegTable& st, float ag, float* __restrict__ out, int64_t ldo) {
  static_assert(S * kStrip <= 64, "one lane of wave 0 per column");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const int n = min(strip0 * kStrip + min(lane, S * kStrip - 1), N - 1);
    const float wc = __shfl(wgv, seg_of(st, n), 64);
    if (lane < S * kStrip) scol[lane] = wc;
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][s][i][lane] = acc[s][i];
  __syncthreads();
  for (int e = threadIdx.x; e < M * S * kStrip; e += 64 * NW) {
    const int row = e / (S * kStrip), c = e % (S * kStrip);
    const int n = strip0 * kStrip + c;
    if (n >= N) continue;
    const int s = c / kStrip, l = (row >> 2) * kStrip + c % kStrip;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][s][row & 3][l];
    out[(int64_t)row * ldo + n] = v * (ag * scol[c]);
  }
}

// The caller's early load of the per-segment scales (see reduce_store): lane
// t < nseg of each wave keeps w_g[t].  Branch-free (every thread reads a valid
// entry), so the kernel's argument loads are not split around a branch at
// kernel start; issue it after the first activation and weight loads.
__device__ __forceinline__ float load_segment_scale(const float* __restrict__ w_g, const SegTable& st) {
  return w_g[min((int)(threadIdx.x & 63), st.nseg - 1)];
}

// Issue priority of this wave (s_setprio takes an immediate; p is a constant
// after unrolling).  The two waves sharing a SIMD otherwise issue oldest first,
// so the younger one falls behind and its weight batches end the stream alone.
// With the priority lowered after each batch, a wave that is behind outranks
// its partner until it catches up; the results do not change.
__device__ __forceinline__ void set_issue_priority(int p) {
  switch (p < 0 ? 0 : (p > 3 ? 3 : p)) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
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

// The skinny GEMM of one workgroup: S strips of 16 columns, NW waves splitting
// the k tiles (wave w takes tiles w, w + NW, ...), U tiles per outer iteration.
// Software pipeline: a batch is one tile of the S strips, and a wave keeps two
// batches in flight (batch u + 2 is requested after the MFMAs of batch u).
// Requesting every batch up front instead lets the memory system accept the
// loads first come, first served: the first waves of a workgroup get all their
// data early, the last wave gets all of it at the end of the stream and then
// has its whole decode and MFMA work left (about 1 us of tail).  Every load is
// unconditional (tiles past the end are clamped), so the waits before each
// batch's MFMAs stay progressive; the clamped tiles of the last iteration skip
// their decode and MFMAs.
template <int S, int NW, int U, bool AL16, bool TAIL>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
  constexpr int kDepth = 2;
  static_assert(U >= kDepth, "pipeline depth");
  __shared__ float red[NW][S][4][64];
  __shared__ float scol[S * kStrip];
  const float ag = *a_g;
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
  const uint8_t* wc[S];
  const uint8_t* ws[S];
  strip_pointers<S>(w_codes, w_scales, strip0, nstrips, tiles, lane, wc, ws);
  const float wgv = load_segment_scale(w_g, st);

  float4_t acc[S];
#pragma unroll
  for (int s = 0; s < S; ++s) acc[s] = float4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (!TAIL) {
    // the general loop: tiles past the end are clamped and decoded with zero
    // scales; the fastest form where every wave's tiles fill whole iterations
    for (int t0 = wave; t0 < full; t0 += NW * U) {
      // activation fragments first (a few hundred bytes, L2-resident after the
      // first workgroups), then the first two weight batches
      uint4 av[U];
      uint32_t asc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) load_a_full<AL16>(ac, as, min(t0 + u * NW, full - 1), av[u], asc[u]);
      uint4 wv[U][S];
      uint32_t wsc[U][S];
      auto request = [&](int u) {
        const int t = min(t0 + u * NW, full - 1);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          wv[u][s] = ld_stream16(wc[s] + (int64_t)t * kChunkCodes);
          wsc[u][s] = ld_stream2(ws[s] + (int64_t)t * kChunkScales);
        }
      };
#pragma unroll
      for (int u = 0; u < kDepth; ++u) request(u);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t live = (t0 + u * NW < full) ? amask : 0u;
        half8_t A[4];
        decode_a(av[u], asc[u], live, A);
#pragma unroll
        for (int s = 0; s < S; ++s) tile_mfma(A, wv[u][s], wsc[u][s], acc[s]);
        __builtin_amdgcn_sched_barrier(0);
        if (u + kDepth < U) request(u + kDepth);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // some wave's last iteration is partial: that iteration, peeled, skips the
    // clamped tiles' decode and MFMAs (a uniform branch, kept out of the main
    // loop so that its waits stay progressive)
    auto iteration = [&](int t0, auto guarded) {
      uint4 av[U];
      uint32_t asc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) load_a_full<AL16>(ac, as, min(t0 + u * NW, full - 1), av[u], asc[u]);
      __builtin_amdgcn_sched_barrier(0);
      uint4 wv[U][S];
      uint32_t wsc[U][S];
      auto request = [&](int u) {
        const int t = min(t0 + u * NW, full - 1);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          wv[u][s] = ld_stream16(wc[s] + (int64_t)t * kChunkCodes);
          wsc[u][s] = ld_stream2(ws[s] + (int64_t)t * kChunkScales);
        }
      };
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {            // in batch order, so that the waits stay progressive
        request(u);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!decltype(guarded)::value || t0 + u * NW < full) {
          half8_t A[4];
          decode_a(av[u], asc[u], amask, A);
#pragma unroll
          for (int s = 0; s < S; ++s) tile_mfma(A, wv[u][s], wsc[u][s], acc[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u + kDepth < U) request(u + kDepth);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int t0 = wave;
    for (; t0 + (U - 1) * NW < full; t0 += NW * U) iteration(t0, std::false_type{});
    if (t0 < full) iteration(t0, std::true_type{});
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
      const uint4 w = ld_stream16(wc[s] + (int64_t)t * kChunkCodes);
      const uint32_t wsv = ld_stream2(ws[s] + (int64_t)t * kChunkScales);
      tile_mfma(A, w, wsv, acc[s]);
    }
  }
  reduce_store<S, NW>(acc, red, scol, wgv, strip0, M, N, st, ag, out, ldo);
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

template <int S, int NW, int VW, int U, bool AL16, int MT>
__global__ __launch_bounds__(64 * NW) void gemm_rows_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
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
  const int rb = blockIdx.x / groups;                // block of 16 MT rows
  const int strip0 = (blockIdx.x - rb * groups) * S;
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

// ---- decode-form linear layer in one launch (M <= 16 at K <= 5120, fewer rows
// for longer K).  The activation quantizer and the skinny GEMM above in a single
// kernel: the tensor is at most 81920 bf16 values (16 x 5120, 8 x 10240 or
// 4 x 20480), and a separate quantizer launch costs about
// 5 us of launch and latency for a few KB of work on this chip.  Wave w of a
// workgroup multiplies only k tiles w, w + NW, ..., so it needs the quantized
// activations of those tiles alone: each wave loads and encodes exactly those
// blocks (all rows) itself, spread over its 64 lanes, and hands them to the
// MFMA lane layout through a wave-private LDS area.  The only workgroup barrier
// before the MFMAs is the tensor-amax reduction (the scale rule needs the amax
// of the whole tensor, which the waves hold between them); no wave waits for
// another wave's encode, so its weight decode and MFMAs overlap the rest of the
// weight stream.  Every workgroup encodes the tensor's blocks (redundantly;
// the bf16 input is L2-resident after the first reads) and workgroup 0 also
// writes the canonical codes, scales and g_dec.  Steps:
//  1. each lane loads its bf16 blocks: slot i = lane + 64 q is row i / (8 U),
//     tile u = (i / 8) % U, block j = i % 8 of that tile, i.e. block column
//     (w + NW u) * 8 + j; groups of eight lanes read 256 contiguous bytes;
//  2. the wave requests its first weight batch (one k tile of its S strips);
//  3. amax: per-lane maximum, wave reduction, one barrier (which also
//     publishes the reciprocal table of the fast encoder);
//  4. each lane encodes its blocks into the wave's LDS area; the second weight
//     batch is requested after the first encode step;
//  5. the MFMA tiles read their activation operand from the wave's LDS area,
//     software-pipelined with two weight batches in flight (batch u + 2 is
//     requested after the MFMAs of batch u; see the skinny GEMM above).
// MAXM bounds the rows a launch may have: the encode steps are unrolled over
// MAXM rows' slots, and smaller instantiations (less code to fetch at each
// launch) are measurably faster for small M.  BAL lowers each wave's issue
// priority after each batch of step 5 (set_issue_priority).  The results are
// bit-identical to the activation quantizer followed by the skinny GEMM.
constexpr int kDecRowBytes = kTileK / 2 + 16;   // LDS bytes per row of one tile (padded)

template <int S, int NW, int U, int MAXM, bool BAL, bool TAIL>
__global__ __launch_bounds__(64 * NW) void linear_decode_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ amax_in, uint8_t* __restrict__ a_codes,
    uint8_t* __restrict__ a_scales, float* __restrict__ a_g, int M, int K, const uint8_t* __restrict__ w_codes,
    const uint8_t* __restrict__ w_scales, int N, SegTable st, const float* __restrict__ w_g,
    float* __restrict__ out, int64_t ldo) {
  constexpr int kSlots = MAXM * U * (kTileK / kBlock);   // block slots of one wave
  constexpr int kQ = (kSlots + 63) / 64;
  static_assert(U >= 2, "two weight batches in flight");
  static_assert(kQ <= 32, "one bit of `live` per encode step");
  __shared__ float red[NW][S][4][64];
  // wave-private activation tiles, row-major over (row, tile): slot group
  // v = row * U + u holds the 8 blocks of row `row` in the wave's tile u
  __shared__ __align__(16) uint8_t lcodes[NW][MAXM * U][kDecRowBytes];
  __shared__ __align__(4) uint8_t lscales[NW][MAXM * U][kTileK / kBlock];
  __shared__ float rtab[128];
  __shared__ uint32_t wmax[NW];
  __shared__ float scol[S * kStrip];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = K / kBlock;
  const int nslot = M * U * (kTileK / kBlock);   // live slots: rows < M
  const int tiles = (K + kTileK - 1) / kTileK;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int strip0 = blockIdx.x * S;

  // 1. this wave's activation blocks; bit q of `live` marks a block to encode
  uint4 xv[kQ][2];
  uint32_t live = 0;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    xv[q][0] = xv[q][1] = make_uint4(0u, 0u, 0u, 0u);
    if (64 * q < nslot) {                          // uniform
      const int i = lane + 64 * q;
      const int row = i / (8 * U), u = (i >> 3) % U;
      const int c = (wave + NW * u) * 8 + (i & 7);
      if (i < nslot && c < nb) {
        const uint4* p = reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + (int64_t)c * kBlock);
        xv[q][0] = p[0];
        xv[q][1] = p[1];
        live |= 1u << q;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. the first weight batch: batch u is tile t = wave + NW u of the S strips
  //    (clamped past the end; its activation scales are zeroed then)
  const uint8_t* wc[S];
  const uint8_t* ws[S];
  strip_pointers<S>(w_codes, w_scales, strip0, nstrips, tiles, lane, wc, ws);
  uint4 wv[U][S];
  uint32_t wsc[U][S];
  auto request = [&](int u) {
    const int t = min(wave + NW * u, tiles - 1);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      wv[u][s] = ld_stream16(wc[s] + (int64_t)t * kChunkCodes);
      wsc[u][s] = ld_stream2(ws[s] + (int64_t)t * kChunkScales);
    }
  };
  request(0);
  __builtin_amdgcn_sched_barrier(0);
  const float wgv = load_segment_scale(w_g, st);

  // 3. reciprocal table, block maxima (kept for the encode) and tensor amax
  //    (max of |x| as bf16 bit patterns); the waves together hold every block
  fill_rcp_table(rtab);
  uint32_t bm[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) bm[q] = absmax_bits(xv[q][0], absmax_bits(xv[q][1], 0u));
  float amax;
  if (amax_in) {
    amax = *amax_in;
    __syncthreads();
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) m = max(m, bm[q]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = max(m, wmax[w]);
    amax = __uint_as_float(m << 16);
  }
  const EncCtx cx = make_ctx(amax, rtab);
  const float g_dec = amax / kGMax;
  const bool writer = blockIdx.x == 0;
  if (writer && tid == 0) *a_g = g_dec;

  // 4. encode this wave's blocks into its LDS area (workgroup 0 also writes the
  //    canonical codes and scales); the second weight batch goes out after the
  //    first encode step
  uint8_t* const lc = &lcodes[wave][lane >> 3][(lane & 7) * 8];   // slot group (lane >> 3) + 8 q
  uint8_t* const ls = &lscales[wave][lane >> 3][lane & 7];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (64 * q < nslot) {                          // uniform
      if ((live >> q) & 1u) {
        uint2 cd;
        const uint32_t sc = encode_bf16_block_max(xv[q][0], xv[q][1], bm[q], cx, cd);
        *reinterpret_cast<uint2*>(lc + q * 8 * kDecRowBytes) = cd;
        ls[q * 8 * (kTileK / kBlock)] = (uint8_t)sc;
        if (writer) {
          const int i = lane + 64 * q;
          const int row = i / (8 * U), c = (wave + NW * ((i >> 3) % U)) * 8 + (i & 7);
          *reinterpret_cast<uint2*>(a_codes + (int64_t)row * (K / 2) + c * 8) = cd;
          a_scales[(int64_t)row * nb + c] = (uint8_t)sc;
        }
      }
    }
    if (q == 0) request(1);
  }
  if constexpr (BAL) set_issue_priority(3);
  // the lanes of this wave read each other's LDS writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // 5. MFMAs, software-pipelined: batch u + 2 is requested after the MFMAs of
  //    batch u.  Lane (r, g) of tile t takes row r, k in [t * 128 + 32 g, + 32)
  const int r = lane & 15, g = lane >> 4;
  const int arow = min(r, M - 1);
  float4_t acc[S];
#pragma unroll
  for (int s = 0; s < S; ++s) acc[s] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (!TAIL) {                           // every wave has U tiles
      const int t = min(wave + NW * u, tiles - 1);
      const int k0 = t * kTileK + 32 * g;
      const bool live0 = (wave + NW * u < tiles) && (r < M) && (k0 < K);
      const bool live1 = live0 && (k0 + kBlock < K);
      const uint4 cv = *reinterpret_cast<const uint4*>(&lcodes[wave][arow * U + u][16 * g]);
      const uint32_t s2 = *reinterpret_cast<const uint16_t*>(&lscales[wave][arow * U + u][2 * g]);
      const uint32_t sc = s2 & ((live0 ? 0xFFu : 0u) | (live1 ? 0xFF00u : 0u));
      half8_t A[4];
      decode_a(cv, sc, 0xFFFFu, A);
#pragma unroll
      for (int s = 0; s < S; ++s) tile_mfma(A, wv[u][s], wsc[u][s], acc[s]);
    } else if (wave + NW * u < tiles) {              // uniform: tiles past the end only complete their loads
      const int t = wave + NW * u;
      const int k0 = t * kTileK + 32 * g;
      const bool live0 = (r < M) && (k0 < K);
      const bool live1 = live0 && (k0 + kBlock < K);
      const uint4 cv = *reinterpret_cast<const uint4*>(&lcodes[wave][arow * U + u][16 * g]);
      const uint32_t s2 = *reinterpret_cast<const uint16_t*>(&lscales[wave][arow * U + u][2 * g]);
      const uint32_t sc = s2 & ((live0 ? 0xFFu : 0u) | (live1 ? 0xFF00u : 0u));
      half8_t A[4];
      decode_a(cv, sc, 0xFFFFu, A);
#pragma unroll
      for (int s = 0; s < S; ++s) tile_mfma(A, wv[u][s], wsc[u][s], acc[s]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (u + 2 < U) request(u + 2);             // two batches in flight
    if constexpr (BAL) set_issue_priority(U - 2 - u);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (BAL) __builtin_amdgcn_s_setprio(0);
  reduce_store<S, NW>(acc, red, scol, wgv, strip0, M, N, st, g_dec, out, ldo);
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

constexpr int kSkNW = 8, kSkU = 5;

template <int S, int NW>
static void launch_skinny_nw(int grid, hipStream_t stream, const uint8_t* a_codes, const uint8_t* a_scales,
                             const float* a_g, int M, int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                             const SegTable& st, const float* w_g, float* out, int64_t ldo) {
  // the peeled loop where some wave's last iteration is partial
  const bool tail = (K / kTileK) % (NW * kSkU) != 0;
#define NVFP4_SKINNY_LAUNCH(AL, T)                                                                               \
  gemm_skinny_kernel<S, NW, kSkU, AL, T><<<grid, 64 * NW, 0, stream>>>(a_codes, a_scales, a_g, M, K, w_codes, \
                                                                      w_scales, N, st, w_g, out, ldo)
  if (K % 32 == 0) {
    if (tail) NVFP4_SKINNY_LAUNCH(true, true);
    else NVFP4_SKINNY_LAUNCH(true, false);
  } else {
    if (tail) NVFP4_SKINNY_LAUNCH(false, true);
    else NVFP4_SKINNY_LAUNCH(false, false);
  }
#undef NVFP4_SKINNY_LAUNCH
}

template <int S>
static void launch_skinny(int nstrips, hipStream_t stream, const uint8_t* a_codes, const uint8_t* a_scales,
                          const float* a_g, int M, int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                          const SegTable& st, const float* w_g, float* out, int64_t ldo) {
  const int grid = (nstrips + S - 1) / S;
  if (stream_waves(K, N) == 16)
    launch_skinny_nw<S, 16>(grid, stream, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
  else
    launch_skinny_nw<S, 8>(grid, stream, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
}

// Row blocks run eight waves; a sixteen-wave order takes two accumulator sets
// (VW = 2) and four tiles per iteration, two per set.
template <int S, int MT, int VW>
static void launch_rows_vw(int grid, hipStream_t stream, const uint8_t* a_codes, const uint8_t* a_scales,
                           const float* a_g, int M, int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                           const SegTable& st, const float* w_g, float* out, int64_t ldo) {
  constexpr int U = VW == 1 ? kSkU : 4;             // a whole number of tiles per accumulator set
  if (K % 32 == 0)
    gemm_rows_kernel<S, kSkNW, VW, U, true, MT><<<grid, 64 * kSkNW, 0, stream>>>(
        a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
  else
    gemm_rows_kernel<S, kSkNW, VW, U, false, MT><<<grid, 64 * kSkNW, 0, stream>>>(
        a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
}

template <int S, int MT>
static void launch_rows(int nstrips, int64_t blocks, hipStream_t stream, const uint8_t* a_codes,
                        const uint8_t* a_scales, const float* a_g, int M, int K, const uint8_t* w_codes,
                        const uint8_t* w_scales, int N, const SegTable& st, const float* w_g, float* out,
                        int64_t ldo) {
  static_assert(kSkNW == 8, "row blocks replay sixteen-wave orders with eight waves");
  const int grid = (int)((nstrips + S - 1) / S * blocks);
  if (stream_waves(K, N) == 16)
    launch_rows_vw<S, MT, 2>(grid, stream, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
  else
    launch_rows_vw<S, MT, 1>(grid, stream, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
}

// Strips per workgroup of gemm_rows_kernel: every workgroup decodes its S weight
// fragments and its MT activation tiles per k tile, so the busiest CU's work is
// ceil(workgroups / 256) * (S + MT); the fewest, ties to larger S (fewer
// activation re-decodes).  E.g. N = 34816, M = 128: S = 3 (1452 workgroups).
static int pick_strips_rows(int nstrips, int64_t blocks, int mt) {
  int best = 3;
  int64_t cost = 0;
  for (int s = 3; s >= 1; --s) {
    const int64_t wgs = (int64_t)(nstrips + s - 1) / s * blocks;
    const int64_t c = (wgs + kCUs - 1) / kCUs * (s + mt);
    if (s == 3 || c < cost) {
      best = s;
      cost = c;
    }
  }
  return best;
}

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M,
                              int K, const uint8_t* w_codes, const uint8_t* w_scales, int N,
                              const SegTable& st, const float* w_g, float* out, int64_t ldo,
                              hipStream_t stream) {
  const int nstrips = (N + kStrip - 1) / kStrip;
  if (M <= 16) {
#define NVFP4_SKINNY(S) launch_skinny<S>(nstrips, stream, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo)
    switch (skinny_strips(nstrips)) {
      case 1: NVFP4_SKINNY(1); break;
      case 2: NVFP4_SKINNY(2); break;
      default: NVFP4_SKINNY(3);
    }
#undef NVFP4_SKINNY
    return hipGetLastError();
  }
  const int rp = rows_per_pass(M, N);
  const int64_t blocks = (M + rp - 1) / rp;
  const int s = pick_strips_rows(nstrips, blocks, rp / 16);
  if ((nstrips + s - 1) / s * blocks > INT32_MAX) return hipErrorInvalidValue;
#define NVFP4_ROWS(S, MT) launch_rows<S, MT>(nstrips, blocks, stream, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo)
  if (rp == 16) {
    switch (s) {
      case 1: NVFP4_ROWS(1, 1); break;
      case 2: NVFP4_ROWS(2, 1); break;
      default: NVFP4_ROWS(3, 1);
    }
  } else if (rp == 32) {
    switch (s) {
      case 1: NVFP4_ROWS(1, 2); break;
      case 2: NVFP4_ROWS(2, 2); break;
      default: NVFP4_ROWS(3, 2);
    }
  } else {
    switch (s) {
      case 1: NVFP4_ROWS(1, 4); break;
      case 2: NVFP4_ROWS(2, 4); break;
      default: NVFP4_ROWS(3, 4);
    }
  }
#undef NVFP4_ROWS
  return hipGetLastError();
}

// One instantiation per row bound.  The issue-priority balancing of the waves
// measured about 0.4 us per launch faster for the 1-row instantiation at
// K = 5120, N = 12288, slower for 2 to 6 rows and no better for 8 or 16 (or in
// the skinny GEMM).
template <int S, int NW, int U, int MAXM>
static bool launch_decode(int nstrips, hipStream_t stream, const uint16_t* x, int64_t ldx, const float* amax_in,
                          uint8_t* a_codes, uint8_t* a_scales, float* a_g, int M, int K, const uint8_t* w_codes,
                          const uint8_t* w_scales, int N, const SegTable& st, const float* w_g, float* out,
                          int64_t ldo) {
  const int grid = (nstrips + S - 1) / S;
  if ((K + kTileK - 1) / kTileK == NW * U)           // every wave has U tiles
    linear_decode_kernel<S, NW, U, MAXM, MAXM == 1 && NW == 8, false><<<grid, 64 * NW, 0, stream>>>(
        x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
  else
    linear_decode_kernel<S, NW, U, MAXM, MAXM == 1 && NW == 8, true><<<grid, 64 * NW, 0, stream>>>(
        x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo);
  return true;
}

// The row-bound instance for M (rows 1, 4, 8, 16; as decode_max_rows allows,
// 16 rows while NW * U covers 40 tiles, 8 up to 80 and 4 up to 160).  False: no
// instance.
template <int S, int NW, int U>
static bool launch_decode_rows(int nstrips, hipStream_t stream, const uint16_t* x, int64_t ldx,
                               const float* amax_in, uint8_t* a_codes, uint8_t* a_scales, float* a_g, int M, int K,
                               const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                               const float* w_g, float* out, int64_t ldo) {
#define NVFP4_DECODE(MAXM)                                                                                       \
  launch_decode<S, NW, U, MAXM>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, \
                                N, st, w_g, out, ldo)
  if (M == 1) return NVFP4_DECODE(1);
  if (M <= 4) return NVFP4_DECODE(4);
  if constexpr (NW * U <= 80) {
    if (M <= 8) return NVFP4_DECODE(8);
    if constexpr (NW * U <= 40) {
      if (M <= 16) return NVFP4_DECODE(16);
    }
  }
#undef NVFP4_DECODE
  return false;
}

template <int S, int NW>
static bool launch_decode_nw(int nstrips, hipStream_t stream, const uint16_t* x, int64_t ldx,
                             const float* amax_in, uint8_t* a_codes, uint8_t* a_scales, float* a_g, int M, int K,
                             const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                             const float* w_g, float* out, int64_t ldo) {
  switch (decode_tiles_per_wave(K, NW)) {
    case 5:
      return launch_decode_rows<S, NW, 5>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes,
                                          w_scales, N, st, w_g, out, ldo);
    case 10:
      return launch_decode_rows<S, NW, 10>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes,
                                           w_scales, N, st, w_g, out, ldo);
    default:
      if constexpr (NW == 8)
        return launch_decode_rows<S, NW, 20>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K,
                                             w_codes, w_scales, N, st, w_g, out, ldo);
      return false;                                  // sixteen waves cover K <= 20480 with U <= 10
  }
}

template <int S>
static bool launch_decode_tiles(int nstrips, hipStream_t stream, const uint16_t* x, int64_t ldx,
                                const float* amax_in, uint8_t* a_codes, uint8_t* a_scales, float* a_g, int M, int K,
                                const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                                const float* w_g, float* out, int64_t ldo) {
  if (M < 1 || M > decode_max_rows(K)) return false;
  if (stream_waves(K, N) == 16)
    return launch_decode_nw<S, 16>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales,
                                   N, st, w_g, out, ldo);
  return launch_decode_nw<S, 8>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N,
                                st, w_g, out, ldo);
}

hipError_t launch_linear_decode(const uint16_t* x, int64_t ldx, const float* amax_in, uint8_t* a_codes,
                                uint8_t* a_scales, float* a_g, int M, int K, const uint8_t* w_codes,
                                const uint8_t* w_scales, int N, const SegTable& st, const float* w_g, float* out,
                                int64_t ldo, hipStream_t stream) {
  const int nstrips = (N + kStrip - 1) / kStrip;
  bool ok;
  switch (skinny_strips(nstrips)) {
    case 1:
      ok = launch_decode_tiles<1>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N,
                                  st, w_g, out, ldo);
      break;
    case 2:
      ok = launch_decode_tiles<2>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N,
                                  st, w_g, out, ldo);
      break;
    default:
      ok = launch_decode_tiles<3>(nstrips, stream, x, ldx, amax_in, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N,
                                  st, w_g, out, ldo);
  }
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

}  // namespace nvfp4
