// Read-rate probe: the HBM read rate a stream of a given size reaches on this
// chip with the access pattern of the decode-form GEMMs' weight stream
// (non-temporal 16-byte loads, each workgroup reading one contiguous region,
// several loads in flight per lane).  It is the ceiling those GEMMs are set
// against: a decode GEMM reads its packed weight once per call, so it cannot be
// faster than a bare read of the same bytes by as many workgroups.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

constexpr int kProbeThreads = 512;
constexpr int kProbeDepth = 4;   // loads in flight per lane

// Workgroup b reads 16-byte chunks [b * per, min((b + 1) * per, n16)), lane t
// chunks t, t + 512, ... of it, and stores the XOR of every word it read to
// sink[b] (which keeps the loads live and lets a test check that every chunk
// was read exactly once).
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                   int64_t per, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kProbeThreads / 64];
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = min(lo + per, n16);
  uint32_t x = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (kProbeDepth - 1) * kProbeThreads < hi; i += kProbeDepth * kProbeThreads) {
    uint4 v[kProbeDepth];
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) v[d] = ld_stream16(p + i + d * kProbeThreads);
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) x ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  for (; i < hi; i += kProbeThreads) {
    const uint4 v = ld_stream16(p + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, int workgroups, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per = (n16 + workgroups - 1) / workgroups;
  read_probe_kernel<<<workgroups, kProbeThreads, 0, stream>>>(static_cast<const uint4*>(buf), n16, per, sink);
  return hipGetLastError();
}

}  // namespace nvfp4
