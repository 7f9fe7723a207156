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
//  * K-permutation shared by both operands: MFMA step j of a tile takes
//    k = 64 h + 8 j + e for lane group h = lane / 32, so a lane's activation
//    operand for a step is one dword of canonical codes and its weight operand
//    one 16-byte piece of a decoded row;
//  * activation codes: 16 KB per k tile loaded coalesced (four lanes per
//    64-byte row segment) into registers, written one tile later to a
//    double-buffered LDS tile, read back by the wave that needs them and
//    decoded to fp16 in registers; their scales go straight to the lanes;
//  * weights (shared by the four M-waves): coalesced chunk reads, loaded two k
//    tiles ahead, decoded once per workgroup to fp16 into double-buffered LDS
//    half-tiles (64 k each: MFMA steps 0-3 use k groups 0 and 2 of a chunk,
//    steps 4-7 groups 1 and 3); the decode of the next half-tile is
//    interleaved with the MFMAs of the current one.  Rows are padded to 144
//    bytes, so the 16-byte operand reads of 16 consecutive lanes hit distinct
//    banks and each step's reads are constant offsets from one base;
//  * the activation tile is XOR-swizzled at 16-byte granularity (piece p of row
//    r at p ^ ((r >> 1 ^ r >> 2) & 3)) so its coalesced writes and its operand
//    reads are bank-conflict free without padding;
//  * workgroups are numbered XCD-major, then in groups of four row panels, so
//    the 32 workgroups resident on an XCD share one activation slab in its L2
//    while they stream weight column panels;
//  * a narrow form (NWN = 1) runs the same per-wave work on a 256 x 128 tile
//    of four waves, two workgroups per CU, where 256 x 256 tiles would leave a
//    partial last round (mfma_narrow); each output sees the same MFMA
//    sequence, so the two forms give bit-identical results.
#include <algorithm>

#include "common.hpp"
#include "quant_device.hpp"
#include "rows_body.hpp"

namespace nvfp4 {

constexpr int kBM = 256, kBN = 256;
constexpr int kMfWaves = 8, kMfThreads = 64 * kMfWaves;
// The narrow form: a 256 x 128 tile of four waves (one N-wave), each wave's
// work exactly as in the 256 x 256 form, two workgroups per CU.
constexpr int kBNNarrow = 128, kMfThreadsNarrow = 256;
constexpr int kGroupM = 4;
constexpr int kHalfRow = 9;                            // uint4 pieces per LDS weight row (8 + 1 pad)

__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Buffer loads: the base address and size live in a resource descriptor (scalar
// registers), each lane keeps a fixed 32-bit byte offset, and the per-k-tile
// step is a scalar offset, so advancing to the next tile costs no vector
// instructions.  Offsets are 32-bit: every operand buffer must be below 4 GiB
// (checked by the launcher).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_u4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 buf_u2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_u8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Per-thread coalesced activation slots: slot q = tid + threads * s covers row
// q / 4 of the tile and its 16-byte piece q % 4 (NS = 1024 / threads slots).
template <int NS>
struct ASlots {
  uint32_t off[NS];                                    // byte offset of the piece in tile 0
  int lds[NS];                                         // uint4 index inside an LDS stage
  int koff[NS];                                        // k offset of the piece inside a tile
};

template <bool AL16, bool TAIL, int NS>
__device__ __forceinline__ void load_a_codes(__amdgpu_buffer_rsrc_t ra, const ASlots<NS>& as, int t, int full, int K,
                                             uint4 (&r)[NS]) {
  const uint32_t soff = (uint32_t)t * 64u;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (TAIL && t == full) {
      const int k0 = t * kTileK + as.koff[s];
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (k0 < K) {
        const uint2 x0 = buf_u2(ra, as.off[s], soff);
        v.x = x0.x;
        v.y = x0.y;
        if (k0 + 16 < K) {
          const uint2 x1 = buf_u2(ra, as.off[s] + 8u, soff);
          v.z = x1.x;
          v.w = x1.y;
        }
      }
      r[s] = v;
    } else if (AL16) {
      r[s] = buf_u4(ra, as.off[s], soff);
    } else {
      const uint2 x0 = buf_u2(ra, as.off[s], soff), x1 = buf_u2(ra, as.off[s] + 8u, soff);
      r[s] = make_uint4(x0.x, x0.y, x1.x, x1.y);
    }
  }
}

// A lane's four scale bytes (blocks 4h .. 4h + 3 of the tile) for each row tile.
template <bool AL4, bool TAIL>
__device__ __forceinline__ void load_a_scales(__amdgpu_buffer_rsrc_t rs, const uint32_t (&so)[2], int t, int full,
                                              int kbase, int K, uint32_t (&r)[2]) {
  const uint32_t soff = (uint32_t)t * 8u;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (TAIL && t == full) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (kbase + 16 * b < K) v |= buf_u8(rs, so[rt] + b, soff) << (8 * b);
      r[rt] = v;
    } else if (AL4) {
      r[rt] = buf_u32(rs, so[rt], soff);
    } else {
      r[rt] = buf_u8(rs, so[rt], soff) | (buf_u8(rs, so[rt] + 1, soff) << 8) | (buf_u8(rs, so[rt] + 2, soff) << 16) |
              (buf_u8(rs, so[rt] + 3, soff) << 24);
    }
  }
}

// Weight slots: thread tid owns chunk row n = tid % 16 of strip tid / 32 and the
// k groups g = 2 * ((tid / 16) % 2) + s for s = 0, 1; slot s is decoded into the
// half-tile s (groups 0 and 2 feed MFMA steps 0-3, groups 1 and 3 steps 4-7).
struct WSlots {
  uint32_t off[2];                                     // byte offset of the slot's codes in tile 0
  uint32_t soff[2];                                    // byte offset of its two scales in tile 0
  int lds;                                             // uint4 index of this thread's row + piece 4 * (g / 2)
};

struct RawW {
  uint4 c[2];
  uint32_t s[2];
};

__device__ __forceinline__ void load_w_tile(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, const WSlots& ws,
                                            int t, RawW& r) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    r.c[s] = buf_u4(rc, ws.off[s], (uint32_t)t * kChunkCodes);
    r.s[s] = buf_u16(rs, ws.soff[s], (uint32_t)t * kChunkScales);
  }
}

// Decode dword d of slot s (one 8-element piece) into its half-tile stage.
__device__ __forceinline__ void store_w_piece(const WSlots& ws, const RawW& r, int s, int d, uint4* stage) {
  const uint32_t sc = (d < 2) ? (r.s[s] & 0xFF) : ((r.s[s] >> 8) & 0xFF);
  const uint32_t w = u4_dword_sel(r.c[s], d);
  stage[ws.lds + d] = __builtin_bit_cast(uint4, decode8(w, scale_pair(sc)));
}

// Column offset (inside the wave's column base) of the wave's MFMA column tile c.
// Plain: four adjacent 32-column tiles.  Gate/up (SW): tiles 0, 1 are 64 gate
// columns and tiles 2, 3 the 64 up columns 128 further on, so each lane holds the
// gate and up values of the same output element.
template <bool SW>
__device__ __forceinline__ constexpr int wtile_col(int c) { return SW ? (c >> 1) * 128 + (c & 1) * 32 : 32 * c; }

// Four MFMA steps (one half-tile, global steps 4 * HALF .. 4 * HALF + 3) on the
// activation codes of LDS stage `sa` and the decoded weights of half-stage `sw`,
// while one weight piece per step of the next half-tile is decoded into `sw_next`.
template <int HALF, bool SW>
__device__ __forceinline__ void mfma_half(const uint4* sa, const uint4* sw, const uint32_t (&asc)[2],
                                          const uint32_t (&amask)[2], int arow0, int bbase, int h,
                                          const WSlots& ws, const RawW& wstore, int wslot, uint4* sw_next,
                                          float16_t (&acc)[2][4]) {
  uint4 araw[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = arow0 + 32 * rt;
    araw[rt] = sa[r * 4 + ((2 * h + HALF) ^ swz_a(r))];
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = 4 * HALF + jj;
    half8_t af[2], bf[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const uint32_t sc = ((asc[rt] & amask[rt]) >> (8 * (j >> 1))) & 0xFF;
      af[rt] = decode8(u4_dword_sel(araw[rt], jj), scale_pair(sc));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      bf[c] = __builtin_bit_cast(half8_t, sw[bbase + wtile_col<SW>(c) * kHalfRow + jj]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[rt][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[rt], bf[c], acc[rt][c], 0, 0, 0);
    store_w_piece(ws, wstore, wslot, jj, sw_next);
  }
}

// Epilogues of the MFMA GEMM.
enum MfmaEpilogue : int {
  kEpiStore = 0,     // out[m][n] = acc * fl(a_g * w_g[seg(n)])
  kEpiSwiglu = 2,    // gate/up weights interleaved; emit NVFP4(bf16(silu(g) * u)) instead of fp32
};

// Outputs of the SwiGLU -> NVFP4 epilogue: the down projection's activations.
struct SwigluOut {
  const float* amax;   // calibrated maximum of h (device scalar)
  uint8_t* codes;      // [M][I/2] canonical
  uint8_t* scales;     // [M][I/16]
  float* g_dec;        // amax / 2688
  int I;               // intermediate size (gate rows = up rows = I)
};

// bf16 bits of a finite float (round to nearest even).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// The MLP's gate nonlinearity on fp32 values: h = silu(g) * u, silu(z) = z / (1 + e^-z).
__device__ __forceinline__ float swiglu_f32(float g, float u) { return g / (1.0f + expf(-g)) * u; }

constexpr int kHRow = 128 + 8;   // bf16 per LDS row of the SwiGLU tile (16-byte pad)

// The ragged last tile column of a launch whose whole tiles fill their last
// round, run by workgroups nmain.. of the same launch as the row-blocked
// weight-streaming GEMM (rows_block over 16-row blocks of RS strips): they start
// as the whole tiles' workgroups finish, with no second launch.
struct RaggedCols {
  const uint8_t* w_codes;   // the strips of columns n_full..
  const uint8_t* w_scales;
  const float* w_g;         // module scales from the first module with such columns
  float* out;               // output column n_full
  SegTable st;              // segment table shifted to column n_full
  int N;                    // ragged columns
  int nmain;                // workgroups of the whole tiles
};

// One launch covers output columns [n_lo, n_hi) (n_lo a multiple of 256).  With
// kEpiSwiglu the weight is the interleaved
// gate/up packing (columns 256 t .. 256 t + 127 are gate rows 128 t .., the next
// 128 the matching up rows), and the workgroup writes the NVFP4 encoding of
// h[m][j] = bf16(silu(g) * u) for its 128 j instead of fp32 output.
// NWN: waves along N (2: the 256 x 256 tile of eight waves; 1: the narrow
// 256 x 128 tile of four waves, two workgroups per CU).  RS > 0: workgroups
// from rg.nmain on run the ragged column (RaggedCols) with RS strips each.
template <bool AL16, bool AL4, bool TAIL, int EPI, int NWN, int RS>
__global__ __launch_bounds__(256 * NWN, 3 - NWN) void gemm_mfma_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, const float* __restrict__ a_g,
    int M, int K, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N, int n_lo,
    int n_hi, SegTable st, const float* __restrict__ w_g, float* __restrict__ out, int64_t ldo, SwigluOut so,
    RaggedCols rg) {
  constexpr bool SW = EPI == kEpiSwiglu;
  if constexpr (RS > 0) {
    static_assert(NWN == 2 && AL16 && !TAIL && !SW, "ragged workgroups: 512 threads, whole k tiles");
    if ((int)blockIdx.x >= rg.nmain) {             // uniform per workgroup
      rows_block<RS, 8, 1, kSkU, true, 1>((int)blockIdx.x - rg.nmain, a_codes, a_scales, a_g, M, K, rg.w_codes,
                                          rg.w_scales, rg.N, rg.st, rg.w_g, rg.out, ldo);
      return;
    }
  }
  constexpr int kThreads = 256 * NWN, kTileN = 128 * NWN, NS = 1024 / kThreads;
  static_assert(!SW || NWN == 2, "the SwiGLU epilogue pairs gate and up columns of a 256-column tile");
  __shared__ uint4 sW[2][kTileN * kHalfRow];           // decoded weight half-tiles, 2 x 36 KB (2 x 18 KB narrow)
  __shared__ uint4 sA[2][kBM * 4];                     // activation codes, 2 x 16 KB

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int tiles = (K + kTileK - 1) / kTileK, full = K / kTileK;
  const int nstrips = (N + kStrip - 1) / kStrip;
  const int tb = 0, te = tiles;                        // the workgroup's k tiles

  // ---- workgroup -> output tile: XCD-major numbering, then grouped row panels
  const int num_m = (M + kBM - 1) / kBM, num_n = (n_hi - n_lo + kTileN - 1) / kTileN;
  const int nwg = num_m * num_n;
  int pid = blockIdx.x;
  if (nwg % 8 == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int per_group = kGroupM * num_n;
  const int first_m = (pid / per_group) * kGroupM;
  const int gsz = min(num_m - first_m, kGroupM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int m0 = tm * kBM, n0 = n_lo + tn * kTileN;

  // ---- activation code slots (coalesced loads) and this lane's scale rows
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_codes, (uint32_t)((int64_t)M * (K / 2)));
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(a_scales, (uint32_t)((int64_t)M * (K / kBlock)));
  ASlots<NS> as;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int q = tid + kThreads * s;
    const int r = q >> 2, p = q & 3;
    const int rc = min(m0 + r, M - 1);
    as.off[s] = (uint32_t)rc * (uint32_t)(K / 2) + 16u * p;
    as.lds[s] = r * 4 + (p ^ swz_a(r));
    as.koff[s] = 32 * p;
  }
  const int i = lane & 31, h = lane >> 5;
  uint32_t asp[2];
  uint32_t amask[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = m0 + wm * 64 + rt * 32 + i;
    asp[rt] = (uint32_t)min(row, M - 1) * (uint32_t)(K / kBlock) + 4u * h;
    amask[rt] = row < M ? 0xFFFFFFFFu : 0u;    // padded rows decode to zeros
  }
  // ---- weight slots
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_codes, (uint32_t)((int64_t)nstrips * tiles * kChunkCodes));
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(w_scales, (uint32_t)((int64_t)nstrips * tiles * kChunkScales));
  WSlots ws;
  {
    const int sl = tid >> 5, n = tid & 15, gg = (tid >> 4) & 1;
    const uint32_t strip = (uint32_t)min(n0 / kStrip + sl, nstrips - 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = 2 * gg + s;
      ws.off[s] = strip * (uint32_t)tiles * kChunkCodes + (uint32_t)chunk_code_off(n, g);
      ws.soff[s] = strip * (uint32_t)tiles * kChunkScales + (uint32_t)chunk_scale_off(n, g);
    }
    ws.lds = (sl * kStrip + n) * kHalfRow + 4 * gg;
  }

  float16_t acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rt][c][r] = 0.f;

  const int last = te - 1;
  const int kb = 64 * h;
  const int arow0 = wm * 64 + i;
  const int bbase = (wn * (SW ? 64 : 128) + i) * kHalfRow + 4 * h;
  uint4 an[NS];                                         // activation codes in flight (next tile)
  uint32_t sc0[2];                                      // activation scales of tile 0
  RawW rw0, rw1;                                        // weights of tiles 0 and 1
  {
    uint4 a0[NS];
    load_a_codes<AL16, TAIL>(ra, as, tb, full, K, a0);
    load_a_scales<AL4, TAIL>(ras, asp, tb, full, tb * kTileK + kb, K, sc0);
    load_w_tile(rw, rws, ws, tb, rw0);
    load_a_codes<AL16, TAIL>(ra, as, min(tb + 1, last), full, K, an);
    load_w_tile(rw, rws, ws, min(tb + 1, last), rw1);
#pragma unroll
    for (int d = 0; d < 4; ++d) store_w_piece(ws, rw0, 0, d, sW[0]);
#pragma unroll
    for (int s = 0; s < NS; ++s) sA[0][as.lds[s]] = a0[s];
  }
  __syncthreads();

  // Per tile t (two half-tiles): half 0 runs MFMA steps 0-3 on sW[0] while the
  // second half of tile t's weights (rwc, slot 1) is decoded into sW[1] and
  // tile t + 1's activation codes are written to the other activation stage;
  // half 1 runs steps 4-7 on sW[1] while the first half of tile t + 1's weights
  // (rwn, slot 0) is decoded into sW[0].  Tile t + 1's scales load at the top
  // of tile t, tile t + 2's codes after half 0 and tile t + 2's weights after
  // half 1.  Tile indices are clamped to the last tile, so every load is
  // unconditional and in bounds.  The loop body is one tile; the raw register
  // sets change roles through plain copies at its end.
  uint32_t scc[2] = {sc0[0], sc0[1]};
  RawW rwc = rw0, rwn = rw1;
  for (int t = tb; t < te; ++t) {
    const uint4* sa = sA[(t - tb) & 1];
    uint4* sa_next = sA[(t - tb + 1) & 1];
    uint32_t scn[2];
    load_a_scales<AL4, TAIL>(ras, asp, min(t + 1, last), full, min(t + 1, last) * kTileK + kb, K, scn);
    mfma_half<0, SW>(sa, sW[0], scc, amask, arow0, bbase, h, ws, rwc, 1, sW[1], acc);
#pragma unroll
    for (int s = 0; s < NS; ++s) sa_next[as.lds[s]] = an[s];
    load_a_codes<AL16, TAIL>(ra, as, min(t + 2, last), full, K, an);
    __syncthreads();
    mfma_half<1, SW>(sa, sW[1], scc, amask, arow0, bbase, h, ws, rwn, 0, sW[0], acc);
    rwc = rwn;
    load_w_tile(rw, rws, ws, min(t + 2, last), rwn);
    scc[0] = scn[0];
    scc[1] = scn[1];
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 8*(r/4) + 4*h + r%4, column i of each 32x32 tile
  const float ag = *a_g;
  if constexpr (SW) {
    // h = bf16(silu(g) * u) for the tile's 256 rows x 128 j, staged in LDS (the
    // weight stages are free once every wave has left the loop), then encoded
    // block by block exactly as the activation quantizer encodes a bf16 tensor.
    uint16_t* hs = reinterpret_cast<uint16_t*>(&sW[0][0]);
    float* rtab = reinterpret_cast<float*>(&sA[0][0]);
    const float alpha_g = ag * w_g[0], alpha_u = ag * w_g[1];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ml = wm * 64 + rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const int jl = wn * 64 + 32 * c + i;
          hs[ml * kHRow + jl] = bf16_rne(swiglu_f32(acc[rt][c][r] * alpha_g, acc[rt][c + 2][r] * alpha_u));
        }
    fill_rcp_table(rtab);
    __syncthreads();
    const float amax = *so.amax;
    const EncCtx cx = make_ctx(amax, rtab);
    if (blockIdx.x == 0 && tid == 0) *so.g_dec = amax / kGMax;
    const int j0 = n0 / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = tid + kMfThreads * q;          // 256 rows x 8 blocks of 16 j
      const int row = b >> 3, jb = b & 7;
      const int m = m0 + row;
      if (m >= M) continue;
      const uint4* src = reinterpret_cast<const uint4*>(hs + row * kHRow + jb * 16);
      uint2 cw;
      const uint32_t sc = encode_bf16_block(src[0], src[1], cx, cw);
      const int64_t j = j0 + jb * 16;
      *reinterpret_cast<uint2*>(so.codes + (int64_t)m * (so.I / 2) + j / 2) = cw;
      so.scales[(int64_t)m * (so.I / kBlock) + j / kBlock] = (uint8_t)sc;
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int n = n0 + wn * 128 + 32 * c + i;
    if (n >= n_hi) continue;
    const float alpha = ag * w_g[seg_of(st, n)];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) {
          out[(int64_t)m * ldo + n] = acc[rt][c][r] * alpha;
        }
      }
  }
}

// ---- unfused SwiGLU of a gate+up output (columns [0, I) gate, [I, 2I) up) to bf16,
// with the same fp32 arithmetic as the fused epilogue.
__global__ void swiglu_kernel(const float* __restrict__ gu, int64_t M, int I, int64_t ldgu,
                              uint16_t* __restrict__ hout, int64_t ldh) {
  const int64_t total = M * I;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / I;
    const int j = (int)(e - m * I);
    hout[m * ldh + j] = bf16_rne(swiglu_f32(gu[m * ldgu + j], gu[m * ldgu + I + j]));
  }
}

hipError_t launch_swiglu(const float* gu, int64_t M, int64_t I, int64_t ldgu, uint16_t* h, int64_t ldh,
                         hipStream_t stream) {
  const int64_t total = M * I;
  if (total == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 256 * 16);
  swiglu_kernel<<<grid, 256, 0, stream>>>(gu, M, (int)I, ldgu, h, ldh);
  return hipGetLastError();
}

// One form of the MFMA GEMM over all N columns (NWN = 2: 256 x 256 tiles; 1: the
// narrow 256 x 128 tiles).
template <int NWN>
static hipError_t launch_mfma_form(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M, int K,
                                   const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                                   const float* w_g, float* out, int64_t ldo, hipStream_t stream) {
  constexpr int kTileN = 128 * NWN, kThreads = 256 * NWN;
  const int num_m = (M + kBM - 1) / kBM;
  const int n_full = N / kTileN * kTileN;              // columns covered by whole tiles
  const int tiles = (K + kTileK - 1) / kTileK;
  // A ragged last tile column costs a whole extra round of workgroups when the
  // whole tiles fill their last round (e.g. 16 x 48 = 768 = 3 x 256).  Then the
  // whole tiles run alone and the ragged strips -- a tall, narrow product with
  // a weight slice of a few hundred KB -- run as the weight-streaming GEMM over
  // row blocks, with the segment table shifted to them.  On the GDN
  // in-projection (4096 x 64 ragged columns, K = 5120: 16-row blocks, 2 strips
  // per workgroup) that takes 11-13 us, where a K-split of the 256 x 256 tile
  // with fp32 atomics into a zeroed output took 29 us; the result is
  // deterministic.
  const int n_main = (int)mfma_main_columns(M, N, NWN == 1);
  const bool ragged = n_main < N;
  const int grid = num_m * ((n_main + kTileN - 1) / kTileN);
  // The ragged strips as the row-blocked GEMM: its segment table shifted to them.
  SegTable sr{};
  int first = 0;                                       // first module with columns at or past n_full
  int64_t rstrip = 0;
  if (ragged) {
    while (st.end[first] <= n_full) ++first;
    sr.nseg = st.nseg - first;
    for (int i = 0; i < sr.nseg; ++i) sr.end[i] = st.end[first + i] - n_full;
    rstrip = n_full / kStrip;
  }
  const int nr = N - n_full;
  // Merged into this launch where the ragged part takes 16-row blocks in the
  // eight-wave order and every k tile is whole (the GDN in-projection: 64
  // columns, 256 workgroups of 4 strips after the 768 whole tiles); otherwise a
  // second launch of the same kernel (gemm_rows_kernel) follows.
  if constexpr (NWN == 2) {
    if (ragged && K % kTileK == 0 && rows_per_pass(M, nr) == 16 && stream_waves(K, nr) == 8) {
      const int rstrips = (nr + kStrip - 1) / kStrip;
      const int64_t blocks = (M + 15) / 16;
      const int rs = pick_strips_rows(rstrips, blocks, 1);
      const int64_t rwgs = (int64_t)(rstrips + rs - 1) / rs * blocks;
      if (grid + rwgs <= INT32_MAX) {
        const RaggedCols rg{w_codes + rstrip * tiles * kChunkCodes, w_scales + rstrip * tiles * kChunkScales,
                            w_g + first, out + n_full, sr, nr, grid};
        const int g2 = (int)(grid + rwgs);
#define NVFP4_MFMA_RAGGED(RS)                                                                                   \
  gemm_mfma_kernel<true, true, false, kEpiStore, 2, RS><<<g2, kThreads, 0, stream>>>(                          \
      a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, 0, n_main, st, w_g, out, ldo, SwigluOut{}, rg)
        switch (rs) {
          case 1: NVFP4_MFMA_RAGGED(1); break;
          case 2: NVFP4_MFMA_RAGGED(2); break;
          case 3: NVFP4_MFMA_RAGGED(3); break;
          default: NVFP4_MFMA_RAGGED(4);
        }
#undef NVFP4_MFMA_RAGGED
        return hipGetLastError();
      }
    }
  }
#define NVFP4_MFMA_LAUNCH(A16, A4, T, EPI, GRID, NLO, NHI)                                                      \
  gemm_mfma_kernel<A16, A4, T, EPI, NWN, 0><<<GRID, kThreads, 0, stream>>>(a_codes, a_scales, a_g, M, K,        \
                                                                           w_codes, w_scales, N, NLO, NHI, st,  \
                                                                           w_g, out, ldo, SwigluOut{},          \
                                                                           RaggedCols{})
#define NVFP4_MFMA_DISPATCH(EPI, GRID, NLO, NHI)                                                                 \
  if (K % kTileK == 0) NVFP4_MFMA_LAUNCH(true, true, false, EPI, GRID, NLO, NHI);                               \
  else if (K % 64 == 0) NVFP4_MFMA_LAUNCH(true, true, true, EPI, GRID, NLO, NHI);                               \
  else if (K % 32 == 0) NVFP4_MFMA_LAUNCH(true, false, true, EPI, GRID, NLO, NHI);                              \
  else NVFP4_MFMA_LAUNCH(false, false, true, EPI, GRID, NLO, NHI)
  NVFP4_MFMA_DISPATCH(kEpiStore, grid, 0, n_main);
  if (ragged) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gemm_skinny(a_codes, a_scales, a_g, M, K, w_codes + rstrip * tiles * kChunkCodes,
                              w_scales + rstrip * tiles * kChunkScales, nr, sr, w_g + first, out + n_full, ldo,
                              stream);
  }
#undef NVFP4_MFMA_DISPATCH
#undef NVFP4_MFMA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M, int K,
                            const uint8_t* w_codes, const uint8_t* w_scales, int N, const SegTable& st,
                            const float* w_g, float* out, int64_t ldo, hipStream_t stream) {
  if (mfma_narrow(M, N))
    return launch_mfma_form<1>(a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo, stream);
  return launch_mfma_form<2>(a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, st, w_g, out, ldo, stream);
}

hipError_t launch_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g, int M,
                                       int K, const uint8_t* w_codes, const uint8_t* w_scales, int I,
                                       const float* w_g, const float* amax_h, uint8_t* h_codes,
                                       uint8_t* h_scales, float* h_g_dec, hipStream_t stream) {
  const int N = 2 * I;
  const int grid = ((M + kBM - 1) / kBM) * (N / kBN);
  SegTable st{};
  st.nseg = 2;
  st.end[0] = I;
  st.end[1] = N;
  const SwigluOut so{amax_h, h_codes, h_scales, h_g_dec, I};
#define NVFP4_SWIGLU_LAUNCH(A16, A4, T)                                                                          \
  gemm_mfma_kernel<A16, A4, T, kEpiSwiglu, 2, 0><<<grid, kMfThreads, 0, stream>>>(                               \
      a_codes, a_scales, a_g, M, K, w_codes, w_scales, N, 0, N, st, w_g, nullptr, 0, so, RaggedCols{})
  if (K % kTileK == 0) NVFP4_SWIGLU_LAUNCH(true, true, false);
  else if (K % 64 == 0) NVFP4_SWIGLU_LAUNCH(true, true, true);
  else if (K % 32 == 0) NVFP4_SWIGLU_LAUNCH(true, false, true);
  else NVFP4_SWIGLU_LAUNCH(false, false, true);
#undef NVFP4_SWIGLU_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
