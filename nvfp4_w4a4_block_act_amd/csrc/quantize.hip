// NVFP4 encoder kernels: on-the-fly activation quantization (bf16 in) and the
// per-module weight encoder's block step (fp32 in).
//
// Format: Summary page ("Summary of 'Why Gated DeltaNet Survives 4-Bit
// Quantization'"), Background, item 1 -- E2M1 elements, an E4M3 scale per 16
// elements from the block maximum / 6, an FP32 scale per tensor.  The FP32
// scale maps the tensor maximum onto 6 * 448 = 2688; every rounding below is
// one binary32 operation (this file is built with -ffp-contract=off and the
// default correctly rounded fp32 division), so the codes are bit-identical to
// the step-by-step definition in include/nvfp4.h.
//
// Work decomposition (HBM-bound: read 2 B, write 0.5625 B per element):
//  * one thread encodes one 16-element block per loop trip: two 16-byte bf16
//    loads (a wave reads 2 KB contiguous), block max on the bit patterns,
//    two correctly rounded divisions per block (reciprocal multiply plus one
//    fused-multiply-add correction), one multiply per element and
//    the gfx950 fp4 converter (v_cvt_scalef32_pk_fp4_f32 with unit scale
//    rounds to nearest even and saturates at 6, exactly the E2M1 rule);
//  * one block per thread and a grid that covers the tensor (up to 2^28
//    blocks; larger tensors loop): on the 32768 x 17408 down-projection input
//    this encodes at 259 us against 314 us for eight workgroups per CU looping
//    over the blocks;
//  * dynamic amax of large tensors: a partial-max kernel (four 16-byte loads in
//    flight per thread per trip: 188 us against 220 us with one) writes one
//    value per workgroup into the workspace, a one-workgroup kernel reduces
//    them to the maximum (also in the workspace), and the encoder reads it like
//    a calibrated one (exact, order-independent, no atomics, no memset); with
//    at most kFuseParts partial maxima (tensors up to ~2M elements) every
//    encode workgroup reduces them itself instead, one launch fewer (with the
//    1024 partials of a prefill-sized tensor that measured slower);
//  * small tensors (decode-sized activations) use a single launch in which
//    every 1024-thread workgroup recomputes the whole-tensor maximum from L2
//    with all of its loads in flight at once.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "quant_device.hpp"

namespace nvfp4 {

constexpr int kQThreads = 256;
constexpr int kAmaxLoads = 4;                // amax pass: 16-byte loads in flight per thread
constexpr int64_t kMaxEncodeGrid = 1 << 20;  // encoder workgroups (blocks beyond loop)
constexpr int kFuseParts = 64;               // partial maxima an encode workgroup reduces itself

// Tensors whose bf16 bytes exceed the 256 MB last-level cache are streamed (ST):
// the maximum pass and the encode pass read x, and the encode pass writes the
// codes and scales, with the non-temporal hint, since none of those bytes
// survive in a cache until they are used again (32768 x 17408: maximum pass
// 212 -> 187 us; calibrated-scale call 260 -> 246 us, where the hint on the
// stores is what counts).  Smaller tensors keep plain accesses, so the encode
// pass finds what the maximum pass has just read (the hint made 4096 x 5120
// 9% slower).
constexpr int64_t kStreamBytes = int64_t(256) << 20;

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Encode the bf16 block at p into its 8 code bytes at cdst and its scale byte at sdst.
template <bool ST>
__device__ __forceinline__ void encode_block_to(const uint16_t* __restrict__ p, uint8_t* __restrict__ cdst,
                                                uint8_t* __restrict__ sdst, const EncCtx& cx) {
  if constexpr (ST) {
    uint2 c;
    const uint32_t sc = encode_bf16_block(ld_stream16(p), ld_stream16(p + 8), cx, c);
    u32x2_t w;
    w.x = c.x;
    w.y = c.y;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(cdst));
    __builtin_nontemporal_store((uint8_t)sc, sdst);
  } else {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    encode_bf16_chunks(q[0], q[1], cx, cdst, sdst);
  }
}

// Encode the bf16 block (m, b) of x.
template <bool ST>
__device__ __forceinline__ void encode_block_at(const uint16_t* __restrict__ x, int64_t ldx, int K, int64_t m,
                                                int b, const EncCtx& cx, uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales) {
  encode_block_to<ST>(x + m * ldx + (int64_t)b * kBlock, codes + m * (K / 2) + (int64_t)b * 8,
                      scales + m * (K / kBlock) + b, cx);
}

// ---- whole-tensor |x| maximum on bf16 bit patterns ------------------------------
// For finite bf16, |x| orders exactly like (bits & 0x7FFF) as an unsigned integer.
// 8-element (16-byte) chunks of the M x K tensor, row-major over the valid
// region; each trip issues kAmaxLoads chunk loads before reducing any.
template <bool ST>
__device__ __forceinline__ uint32_t chunk_absmax(const uint16_t* __restrict__ x, int64_t ldx, int K,
                                                 int64_t M, int64_t first, int64_t stride) {
  const int64_t cpr = K / 8;
  const int64_t total = M * cpr;
  uint32_t m = 0;
  for (int64_t c0 = first; c0 < total; c0 += kAmaxLoads * stride) {
    uint4 v[kAmaxLoads];
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) {
      const int64_t c = c0 + u * stride;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (c < total) {
        const int64_t r = c / cpr;
        const int64_t k = (c - r * cpr) * 8;
        v[u] = ST ? ld_stream16(x + r * ldx + k) : *reinterpret_cast<const uint4*>(x + r * ldx + k);
      }
    }
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) m = absmax_bits(v[u], m);
  }
  return m;
}

// The same over a contiguous tensor (ldx == K) seen as one flat run of chunks:
// workgroup b takes the contiguous share [b * per, min((b + 1) * per, total)),
// its lanes consecutive chunks, kAmaxLoads loads in flight per lane, with no
// row / column arithmetic per chunk.
template <bool ST>
__device__ __forceinline__ uint32_t flat_absmax(const uint16_t* __restrict__ x, int64_t total) {
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = min(lo + per, total);
  const uint4* p = reinterpret_cast<const uint4*>(x);
  uint32_t m = 0;
  int64_t c = lo + threadIdx.x;
  for (; c + (kAmaxLoads - 1) * kQThreads < hi; c += kAmaxLoads * kQThreads) {
    uint4 v[kAmaxLoads];
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) v[u] = ST ? ld_stream16(p + c + u * kQThreads) : p[c + u * kQThreads];
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) m = absmax_bits(v[u], m);
  }
  for (; c < hi; c += kQThreads) m = absmax_bits(ST ? ld_stream16(p + c) : p[c], m);
  return m;
}

template <bool ST>
__global__ __launch_bounds__(kQThreads) void amax_partial_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                 int K, int64_t ldx,
                                                                 uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kQThreads / 64];
  const uint32_t m = (ldx == K) ? flat_absmax<ST>(x, M * (K / 8))   // uniform
                                : chunk_absmax<ST>(x, ldx, K, M, (int64_t)blockIdx.x * blockDim.x + threadIdx.x,
                                                   (int64_t)gridDim.x * blockDim.x);
  const uint32_t r = block_reduce_max(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = r;
}

// *amax_out = the largest of the nparts partial maxima (bf16 bit patterns).
__global__ __launch_bounds__(kQThreads) void amax_finalize_kernel(const uint32_t* __restrict__ partial, int nparts,
                                                                  float* __restrict__ amax_out) {
  __shared__ uint32_t red[kQThreads / 64];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, partial[i]);
  m = block_reduce_max(m, red);
  if (threadIdx.x == 0) *amax_out = __uint_as_float(m << 16);
}

// Encode with the tensor maximum: *amax (calibrated, or the dynamic one the two
// kernels above left in the workspace), or, with `partial`, the largest of the
// nparts partial maxima (bf16 bit patterns), reduced by every workgroup.
template <bool ST>
__global__ __launch_bounds__(kQThreads) void quantize_act_kernel(
    const uint16_t* __restrict__ x, int64_t M, int K, int64_t ldx, const float* __restrict__ amax_in,
    const uint32_t* __restrict__ partial, int nparts, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ g_dec_out) {
  __shared__ float rtab[128];
  __shared__ uint32_t red[kQThreads / 64];
  fill_rcp_table(rtab);
  float amax;
  if (partial) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, partial[i]);
    amax = __uint_as_float(block_reduce_max(m, red) << 16);   // its barriers also publish rtab
  } else {
    amax = *amax_in;
    __syncthreads();
  }
  const EncCtx cx = make_ctx(amax, rtab);
  if (blockIdx.x == 0 && threadIdx.x == 0) *g_dec_out = amax / kGMax;

  const int nb = K / kBlock;
  const int64_t total = M * nb;
  const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (int64_t)gridDim.x * blockDim.x;
  if (ldx == K) {
    // contiguous: block i of the flat tensor is row i / nb, block i % nb, and its
    // codes and scales sit at i * 8 and i in the canonical layout
    for (int64_t i = first; i < total; i += stride) encode_block_to<ST>(x + i * kBlock, codes + i * 8, scales + i, cx);
  } else {
    for (int64_t i = first; i < total; i += stride) {
      const int64_t m = i / nb;
      const int b = (int)(i - m * nb);
      encode_block_at<ST>(x, ldx, K, m, b, cx, codes, scales);
    }
  }
}

// Decode-sized tensors (M * K <= kSmallElems): one launch, at most 8 workgroups
// of 1024 threads.  Thread t of workgroup b encodes block i = 1024 b + t, whose
// two 16-byte chunks are chunks 2i and 2i + 1 of the row-major chunk order.
// Every workgroup reads the whole tensor once for the maximum, all loads in
// flight at once: thread t takes chunk slots (2048 b + 2t + h + 2048 j) mod
// 16384 for h = 0, 1 and j = 0..7, which cover every slot and start with its
// own block, so the encode step needs no second load.
constexpr int kSmallThreads = 1024;
constexpr int kSmallSlots = 16384;                  // chunks of 8 elements

__global__ __launch_bounds__(kSmallThreads) void quantize_act_small_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, float inv_cpr, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ g_dec_out) {
  __shared__ uint32_t red[kSmallThreads / 64];
  __shared__ float rtab[128];
  fill_rcp_table(rtab);
  const int cpr = K / 8;
  const int total = M * cpr;
  uint4 v[16];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (2048 * (int)blockIdx.x + 2 * (int)threadIdx.x + h + 2048 * j) & (kSmallSlots - 1);
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (c < total) {
        // c / cpr via a float reciprocal, corrected to exact (c < 2^24)
        int r = (int)((float)c * inv_cpr);
        int k = c - r * cpr;
        if (k < 0) { --r; k += cpr; }
        if (k >= cpr) { ++r; k -= cpr; }
        val = *reinterpret_cast<const uint4*>(x + (int64_t)r * ldx + (int64_t)k * 8);
      }
      v[2 * j + h] = val;
    }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // per 16-bit half: a packed pair must not be compared as one 32-bit word
    const uint32_t a0 = max(v[j].x & 0x7FFFu, (v[j].x >> 16) & 0x7FFFu);
    const uint32_t a1 = max(v[j].y & 0x7FFFu, (v[j].y >> 16) & 0x7FFFu);
    const uint32_t a2 = max(v[j].z & 0x7FFFu, (v[j].z >> 16) & 0x7FFFu);
    const uint32_t a3 = max(v[j].w & 0x7FFFu, (v[j].w >> 16) & 0x7FFFu);
    m = max(m, max(max(a0, a1), max(a2, a3)));
  }
  const float amax = __uint_as_float(block_reduce_max(m, red) << 16);
  const EncCtx cx = make_ctx(amax, rtab);
  if (blockIdx.x == 0 && threadIdx.x == 0) *g_dec_out = amax / kGMax;
  const int nb = K / kBlock;
  const int i = blockIdx.x * kSmallThreads + threadIdx.x;
  if (i < M * nb) {
    const int row = i / nb, b = i - row * nb;
    encode_bf16_chunks(v[0], v[1], cx, codes + (int64_t)row * (K / 2) + (int64_t)b * 8,
                       scales + (int64_t)row * nb + b);
  }
}

__global__ void g_dec_only_kernel(const float* __restrict__ amax_in, float* __restrict__ g_dec_out) {
  *g_dec_out = amax_in ? *amax_in / kGMax : 0.0f;
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const float* amax_in, uint8_t* codes, uint8_t* scales,
                               float* g_dec_out, void* workspace, hipStream_t stream) {
  const int64_t blocks = M * (K / kBlock);
  if (blocks == 0) {
    g_dec_only_kernel<<<1, 1, 0, stream>>>(amax_in, g_dec_out);
    return hipGetLastError();
  }
  // One block per thread (grid-stride beyond kMaxEncodeGrid workgroups).
  const int grid = (int)std::min<int64_t>((blocks + kQThreads - 1) / kQThreads, kMaxEncodeGrid);
  const bool st = M * K * 2 > kStreamBytes;
  auto encode = [&](const float* amax, const uint32_t* partial, int nparts) {
    if (st)
      quantize_act_kernel<true><<<grid, kQThreads, 0, stream>>>(x, M, (int)K, ldx, amax, partial, nparts, codes,
                                                                scales, g_dec_out);
    else
      quantize_act_kernel<false><<<grid, kQThreads, 0, stream>>>(x, M, (int)K, ldx, amax, partial, nparts, codes,
                                                                 scales, g_dec_out);
  };
  if (amax_in) {
    encode(amax_in, nullptr, 0);
  } else if (M * K <= kSmallElems) {
    const int grid = (int)((blocks + kSmallThreads - 1) / kSmallThreads);
    quantize_act_small_kernel<<<grid, kSmallThreads, 0, stream>>>(x, (int)M, (int)K, ldx, 1.0f / (float)(K / 8),
                                                                   codes, scales, g_dec_out);
  } else {
    uint32_t* partial = static_cast<uint32_t*>(workspace);
    const int64_t chunks = M * (K / 8);
    int pgrid = (int)std::max<int64_t>(1, std::min<int64_t>(kPartials, chunks / (kQThreads * 16)));
    // mid-size tensors: at most kFuseParts partials, each workgroup two chunks per thread
    if (pgrid <= kFuseParts) pgrid = (int)std::max<int64_t>(1, std::min<int64_t>(kFuseParts, chunks / (kQThreads * 2)));
    float* amax = reinterpret_cast<float*>(partial + kPartials);
    if (st)
      amax_partial_kernel<true><<<pgrid, kQThreads, 0, stream>>>(x, M, (int)K, ldx, partial);
    else
      amax_partial_kernel<false><<<pgrid, kQThreads, 0, stream>>>(x, M, (int)K, ldx, partial);
    if (pgrid <= kFuseParts) {
      encode(nullptr, partial, pgrid);
    } else {
      amax_finalize_kernel<<<1, kQThreads, 0, stream>>>(partial, pgrid, amax);
      encode(amax, nullptr, 0);
    }
  }
  return hipGetLastError();
}

// ---- static-scale calibration -------------------------------------------------------
// Observer: running = max(running, max |x|), from the partial maxima above.
__global__ __launch_bounds__(kQThreads) void amax_observe_finalize_kernel(const uint32_t* __restrict__ partial,
                                                                          int nparts, float* __restrict__ running) {
  __shared__ uint32_t red[kQThreads / 64];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = max(m, partial[i]);
  m = block_reduce_max(m, red);
  if (threadIdx.x == 0) *running = fmaxf(*running, __uint_as_float(m << 16));
}

hipError_t launch_amax_observe(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float* running,
                               void* workspace, hipStream_t stream) {
  if (M * K == 0) return hipSuccess;
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  const int64_t chunks = M * (K / 8);
  const int pgrid = (int)std::max<int64_t>(1, std::min<int64_t>(kPartials, chunks / (kQThreads * 16)));
  amax_partial_kernel<false><<<pgrid, kQThreads, 0, stream>>>(x, M, (int)K, ldx, partial);
  amax_observe_finalize_kernel<<<1, kQThreads, 0, stream>>>(partial, pgrid, running);
  return hipGetLastError();
}

// Saturation statistics under a static maximum, in the encoder's own binary32
// steps: counts[0] += blocks whose unrounded scale fl(fl(bmax / 6) * g_enc)
// exceeds 448, counts[1] += elements with y = fl(|x| * fl(g_enc / s_dec)) >= 7
// (past the midpoint from 6 to the next grid value 8: cut rather than rounded to
// 6, which happens in saturated blocks and in blocks with E4M3 subnormal scales).
__global__ __launch_bounds__(kQThreads) void quantize_stats_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                   int K, int64_t ldx,
                                                                   const float* __restrict__ amax_in,
                                                                   uint32_t* __restrict__ counts) {
  const float g_enc = g_enc_of(*amax_in);
  const int nb = K / kBlock;
  const int64_t total = M * nb;
  uint32_t sat = 0, clip = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / nb;
    const int b = (int)(i - m * nb);
    const uint4* p = reinterpret_cast<const uint4*>(x + m * ldx + (int64_t)b * kBlock);
    const uint4 v0 = p[0], v1 = p[1];
    const uint32_t d[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const float bmax = __uint_as_float(absmax_bits(v0, absmax_bits(v1, 0u)) << 16);
    const float t = bmax / 6.0f;
    const float s = t * g_enc;
    sat += (s > 448.0f) ? 1u : 0u;
    const uint32_t sc = (t != 0.0f) ? e4m3_encode_rne_sat(s) : 0u;
    const float sdec = e4m3_value(sc);
    const float rb = (sdec != 0.0f) ? g_enc / sdec : 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      clip += (__uint_as_float((d[e] << 16) & 0x7FFF0000u) * rb >= 7.0f) ? 1u : 0u;
      clip += (__uint_as_float(d[e] & 0x7FFF0000u) * rb >= 7.0f) ? 1u : 0u;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sat += (uint32_t)__shfl_xor((int)sat, o, 64);
    clip += (uint32_t)__shfl_xor((int)clip, o, 64);
  }
  if ((threadIdx.x & 63) == 0 && (sat | clip)) {
    atomicAdd(&counts[0], sat);
    atomicAdd(&counts[1], clip);
  }
}

hipError_t launch_quantize_stats(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                 uint32_t* counts, hipStream_t stream) {
  const hipError_t e = launch_fill_zero(reinterpret_cast<float*>(counts), 1, 2, 2, stream);
  if (e != hipSuccess) return e;
  const int64_t blocks = M * (K / kBlock);
  if (blocks == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((blocks + kQThreads - 1) / kQThreads, 256 * 8);
  quantize_stats_kernel<<<grid, kQThreads, 0, stream>>>(x, M, (int)K, ldx, amax_in, counts);
  return hipGetLastError();
}

// ---- allocation-free scratch --------------------------------------------------------
// The two-pass quantizer's workspace (partial maxima, then the maximum) for the
// entry point that allocates nothing: a file-scope device array, one copy per
// GPU, held until the process ends.  Its device address is looked up once per
// device and cached; kernels receive that address, never the host-side name.
// Calls that overlap on one GPU share it and race (the caller orders them).
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_for_stream(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = (dev != cur) ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// ---- conversion sweep (diagnostic) ------------------------------------------------
// For the binary32 value v_i with bit pattern first + i, i < n (values 2 j and
// 2 j + 1 form one pair, the first in the low half, as the encoders pair them):
//   op 0: out[i] = E2M1 code of v_i through e2m1_pack_pair (the element step);
//   op 1: out[i] = E4M3 code of v_i through e4m3_pair_rne_sat (the block-scale
//         step and the KV-cache codec);
//   op 2: out[2 i .. 2 i + 1] = fp16 bits (little endian) of the GEMMs' exact
//         decode (decode8 with scale_pair) of E2M1 code (first + i) & 15 times
//         E4M3 code ((first + i) >> 4) & 127.
__global__ __launch_bounds__(kQThreads) void convert_sweep_kernel(int op, uint32_t first, int64_t n,
                                                                 uint8_t* __restrict__ out) {
  const int64_t pairs = (n + 1) / 2;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < pairs; j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i0 = 2 * j;
    const bool two = i0 + 1 < n;
    const uint32_t b0 = first + (uint32_t)i0, b1 = two ? b0 + 1 : b0;
    if (op == 0) {
      const uint32_t c = e2m1_pack_pair<0>(0u, __uint_as_float(b0), __uint_as_float(b1));
      out[i0] = (uint8_t)(c & 15u);
      if (two) out[i0 + 1] = (uint8_t)((c >> 4) & 15u);
    } else if (op == 1) {
      const uint32_t c = e4m3_pair_rne_sat(__uint_as_float(b0), __uint_as_float(b1));
      out[i0] = (uint8_t)(c & 0xFFu);
      if (two) out[i0 + 1] = (uint8_t)(c >> 8);
    } else {
      const uint32_t h0 = __builtin_bit_cast(uint16_t, decode8(b0 & 15u, scale_pair((b0 >> 4) & 127u))[0]);
      const uint32_t h1 = __builtin_bit_cast(uint16_t, decode8(b1 & 15u, scale_pair((b1 >> 4) & 127u))[0]);
      *reinterpret_cast<uint16_t*>(out + 2 * i0) = (uint16_t)h0;
      if (two) *reinterpret_cast<uint16_t*>(out + 2 * i0 + 2) = (uint16_t)h1;
    }
  }
}

hipError_t launch_convert_sweep(int op, uint32_t first, int64_t n, uint8_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(((n + 1) / 2 + kQThreads - 1) / kQThreads, 256 * 64);
  convert_sweep_kernel<<<grid, kQThreads, 0, stream>>>(op, first, n, out);
  return hipGetLastError();
}

// ---- weights: per-module encode into the tiled layout ----------------------------
// partial[s * kSegParts + p] = max |w| bits over rows p, p + kSegParts, ... of
// segment s: workgroup p walks its rows, its threads the row's 16-byte pieces
// (four loads in flight per trip) when every row starts 16-byte aligned
// (ldw % 4 == 0), else single floats.
static_assert(kSegParts == kQThreads, "the packer reduces one partial per thread");
__global__ __launch_bounds__(kQThreads) void seg_amax_kernel(const float* __restrict__ w, int K, int64_t ldw,
                                                             SegTable st, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kQThreads / 64];
  const int s = blockIdx.y;
  const int64_t r0 = (s == 0) ? 0 : st.end[s - 1];
  const int64_t rows = st.end[s] - r0;
  const bool vec = (ldw % 4) == 0;
  uint32_t m = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* row = w + (r0 + r) * ldw;
    if (vec) {
      const int k4 = K / 4;
      for (int j0 = threadIdx.x; j0 < k4; j0 += 4 * kQThreads) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j0 + u * kQThreads;
          v[u] = j < k4 ? reinterpret_cast<const float4*>(row)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          m = max(m, max(max(__float_as_uint(v[u].x) & 0x7FFFFFFFu, __float_as_uint(v[u].y) & 0x7FFFFFFFu),
                         max(__float_as_uint(v[u].z) & 0x7FFFFFFFu, __float_as_uint(v[u].w) & 0x7FFFFFFFu)));
      }
    } else {
      for (int k = threadIdx.x; k < K; k += kQThreads) m = max(m, __float_as_uint(row[k]) & 0x7FFFFFFFu);
    }
  }
  const uint32_t r = block_reduce_max(m, red);
  if (threadIdx.x == 0) partial[s * kSegParts + blockIdx.x] = r;
}

// One thread per 16-element block of the padded Np x Kp weight.  With ilv = I > 0
// the weight is a fused gate+up pair (rows [0, I) gate, [I, 2I) up, segments 0
// and 1) packed interleaved: packed row n holds module (n / 128) % 2, row
// (n / 256) * 128 + n % 128 of it, so every 256-row tile pairs 128 gate rows
// with the matching 128 up rows.
__global__ __launch_bounds__(kQThreads) void pack_weight_kernel(
    const float* __restrict__ w, int N, int K, int64_t ldw, int Np, int Kp, SegTable st, int ilv,
    const uint32_t* __restrict__ partial, uint8_t* __restrict__ w_codes, uint8_t* __restrict__ w_scales,
    float* __restrict__ w_g_dec) {
  __shared__ float s_genc[NVFP4_MAX_SEGMENTS];
  __shared__ uint32_t red[kQThreads / 64];
  for (int s = 0; s < st.nseg; ++s) {                // each segment's maximum from its partials
    const float amax = __uint_as_float(block_reduce_max(partial[s * kSegParts + threadIdx.x], red));
    if (threadIdx.x == 0) {
      s_genc[s] = g_enc_of(amax);
      if (blockIdx.x == 0) w_g_dec[s] = amax / kGMax;
    }
  }
  __syncthreads();
  const int nbk = Kp / kBlock;
  const int64_t total = (int64_t)Np * nbk;
  const int tiles = Kp / kTileK;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / nbk);
    const int b = (int)(i - (int64_t)n * nbk);
    uint2 c = make_uint2(0u, 0u);
    uint32_t sc = 0;
    const int mod = (n >> 7) & 1;
    const int src = ilv ? mod * ilv + ((n >> 8) << 7) + (n & 127) : n;
    if (n < N && b * kBlock < K) {
      const float* p = w + (int64_t)src * ldw + (int64_t)b * kBlock;
      float xf[16];
      float bmax = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        xf[j] = p[j];
        bmax = fmaxf(bmax, fabsf(xf[j]));
      }
      sc = encode_block(xf, bmax, s_genc[ilv ? mod : seg_of(st, n)], c);
    }
    const int64_t chunk = (int64_t)(n / kStrip) * tiles + b / (kTileK / kBlock);
    const int r = n % kStrip, bb = b % (kTileK / kBlock);   // block bb of the chunk: group bb / 2
    *reinterpret_cast<uint2*>(w_codes + chunk * kChunkCodes + chunk_code_off(r, bb >> 1) + (bb & 1) * 8) = c;
    w_scales[chunk * kChunkScales + chunk_scale_off(r, bb >> 1) + (bb & 1)] = (uint8_t)sc;
  }
}

__global__ __launch_bounds__(kQThreads) void weight_to_canonical_kernel(
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales, int N, int K, int Kp,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int nb = K / kBlock;
  const int64_t total = (int64_t)N * nb;
  const int tiles = Kp / kTileK;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / nb);
    const int b = (int)(i - (int64_t)n * nb);
    const int64_t chunk = (int64_t)(n / kStrip) * tiles + b / (kTileK / kBlock);
    const int r = n % kStrip, bb = b % (kTileK / kBlock);
    const uint2 c = *reinterpret_cast<const uint2*>(w_codes + chunk * kChunkCodes + chunk_code_off(r, bb >> 1) +
                                                    (bb & 1) * 8);
    *reinterpret_cast<uint2*>(codes + (int64_t)n * (K / 2) + (int64_t)b * 8) = c;
    scales[(int64_t)n * nb + b] = w_scales[chunk * kChunkScales + chunk_scale_off(r, bb >> 1) + (bb & 1)];
  }
}

static hipError_t pack_weight_impl(const float* w, int64_t N, int64_t K, int64_t ldw, const SegTable& st,
                                   int ilv, uint8_t* w_codes, uint8_t* w_scales, float* w_g_dec, void* workspace,
                                   hipStream_t stream) {
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  seg_amax_kernel<<<dim3(kSegParts, st.nseg), kQThreads, 0, stream>>>(w, (int)K, ldw, st, partial);
  const int64_t Np = round_up(N, kStrip), Kp = round_up(K, kTileK);
  const int64_t total = Np * (Kp / kBlock);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((total + kQThreads - 1) / kQThreads, 256 * 16));
  pack_weight_kernel<<<grid, kQThreads, 0, stream>>>(w, (int)N, (int)K, ldw, (int)Np, (int)Kp, st, ilv, partial,
                                                     w_codes, w_scales, w_g_dec);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const float* w, int64_t N, int64_t K, int64_t ldw,
                              const nvfp4_segment* segs, int nseg, uint8_t* w_codes,
                              uint8_t* w_scales, float* w_g_dec, void* workspace,
                              hipStream_t stream) {
  SegTable st{};
  st.nseg = nseg;
  for (int i = 0; i < nseg; ++i) st.end[i] = segs[i].n_end;
  return pack_weight_impl(w, N, K, ldw, st, 0, w_codes, w_scales, w_g_dec, workspace, stream);
}

hipError_t launch_pack_weight_gate_up(const float* w, int64_t I, int64_t K, int64_t ldw, uint8_t* w_codes,
                                      uint8_t* w_scales, float* w_g_dec, void* workspace, hipStream_t stream) {
  SegTable st{};
  st.nseg = 2;
  st.end[0] = (int32_t)I;
  st.end[1] = (int32_t)(2 * I);
  return pack_weight_impl(w, 2 * I, K, ldw, st, (int)I, w_codes, w_scales, w_g_dec, workspace, stream);
}

hipError_t launch_weight_to_canonical(const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                      int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t total = N * (K / kBlock);
  if (total == 0) return hipSuccess;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((total + kQThreads - 1) / kQThreads, 256 * 16));
  weight_to_canonical_kernel<<<grid, kQThreads, 0, stream>>>(w_codes, w_scales, (int)N, (int)K,
                                                             (int)round_up(K, kTileK), codes, scales);
  return hipGetLastError();
}

}  // namespace nvfp4
