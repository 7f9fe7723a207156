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
#include "rows_body.hpp"

namespace nvfp4 {

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

// ---- the same weight stream for more than 16 rows (rows_block in rows_body.hpp).
template <int S, int NW, int VW, int U, bool AL16, int MT>
__global__ __launch_bounds__(64 * NW) void gemm_rows_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N,
    SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo) {
  rows_block<S, NW, VW, U, AL16, MT>(blockIdx.x, a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out,
                                     ldo);
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
// writes g_dec and, after its outputs, the canonical codes and scales.  Steps:
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
  // PSC: the wave's S x U weight scale chunks (128 bytes each) are fetched by two
  // 16-byte loads per lane at kernel start (eight chunks per load) and handed to
  // the MFMA lanes through a wave-private LDS area, instead of one 2-byte load
  // per lane, strip and tile in each batch.  Measured at K = 5120, N = 12288
  // (three alternating runs on one box, us per launch): M = 1 8.27 -> 7.95,
  // M = 4 8.61 -> 8.54, M = 16 12.79 -> 12.89, so the 8- and 16-row instances
  // keep the per-batch loads.
  constexpr bool PSC = S * U <= 16 && NW == 8 && MAXM <= 4;
  __shared__ __align__(16) uint8_t lwsc[NW][PSC ? 16 : 1][kChunkScales];
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
  uint4 scp[2];                                      // PSC: chunk c = s U + u of the wave (c = 8 j + lane / 8)
  if constexpr (PSC) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = min(8 * j + (lane >> 3), S * U - 1);
      const int sc = c / U, u = c - sc * U;
      const int64_t strip = min(strip0 + sc, nstrips - 1);
      const int t = min(wave + NW * u, tiles - 1);
      scp[j] = ld_stream16(w_scales + (strip * tiles + t) * kChunkScales + (lane & 7) * 16);
    }
  }
  auto request = [&](int u) {
    const int t = min(wave + NW * u, tiles - 1);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      wv[u][s] = ld_stream16(wc[s] + (int64_t)t * kChunkCodes);
      if constexpr (!PSC) wsc[u][s] = ld_stream2(ws[s] + (int64_t)t * kChunkScales);
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

  // 4. encode this wave's blocks into its LDS area (workgroup 0 stores them as
  //    the canonical codes and scales at the end); the second weight batch goes
  //    out after the first encode step
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
      }
    }
    if (q == 0) request(1);
  }
  if constexpr (PSC) {                               // lane l of load j held bytes 16 l of chunks 8 j ..
    uint4* const dst = reinterpret_cast<uint4*>(&lwsc[wave][0][0]);
    dst[lane] = scp[0];
    dst[64 + lane] = scp[1];
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
      for (int s = 0; s < S; ++s)
        tile_mfma(A, wv[u][s], PSC ? (uint32_t)*reinterpret_cast<const uint16_t*>(&lwsc[wave][s * U + u][2 * lane])
                                   : wsc[u][s], acc[s]);
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
      for (int s = 0; s < S; ++s)
        tile_mfma(A, wv[u][s], PSC ? (uint32_t)*reinterpret_cast<const uint16_t*>(&lwsc[wave][s * U + u][2 * lane])
                                   : wsc[u][s], acc[s]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (u + 2 < U) request(u + 2);             // two batches in flight
    if constexpr (BAL) set_issue_priority(U - 2 - u);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (BAL) __builtin_amdgcn_s_setprio(0);
  reduce_store<S, NW>(acc, red, scol, wgv, strip0, M, N, st, g_dec, out, ldo);
  // workgroup 0 stores g_dec and the canonical codes and scales last, the codes
  // from each lane's own slots in its wave's LDS area: a store counts against
  // the same in-order counter as the weight loads, so stores issued during the
  // encode would make the weight batches behind them wait for their round trips
  if (writer) {
    if (tid == 0) *a_g = g_dec;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (64 * q < nslot && ((live >> q) & 1u)) {
        const int i = lane + 64 * q;
        const int row = i / (8 * U), c = (wave + NW * ((i >> 3) % U)) * 8 + (i & 7);
        *reinterpret_cast<uint2*>(a_codes + (int64_t)row * (K / 2) + c * 8) =
            *reinterpret_cast<const uint2*>(lc + q * 8 * kDecRowBytes);
        a_scales[(int64_t)row * nb + c] = ls[q * 8 * (kTileK / kBlock)];
      }
    }
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
      case 3: NVFP4_ROWS(3, 1); break;
      default: NVFP4_ROWS(4, 1);
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
