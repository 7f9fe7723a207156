// Host-side dispatch of the NVFP4 kernels: workspace sizes and the choice of
// GEMM form.  Plain C++ (no device code), so the C ABI and this logic can be
// built and checked on the host alone.
#include <algorithm>

#include "launch.hpp"

namespace nvfp4 {

size_t quantize_act_workspace(int64_t M, int64_t K) {
  // the partial maxima, then the maximum itself
  return (M * K > kSmallElems) ? kPartials * sizeof(uint32_t) + 16 : 0;
}

size_t amax_observe_workspace() { return kPartials * sizeof(uint32_t); }

size_t pack_weight_workspace(int64_t, int64_t, int nseg) { return (size_t)nseg * kSegParts * sizeof(uint32_t); }

bool gemm_prefers_skinny(int64_t M, int64_t K, int64_t N) {
  if (M <= 16) return true;
  // Cost models measured at K = 5120 (N = 5120, 12288, 34816):
  //  * the MFMA GEMM needs about 256 tiles of 256 x 256 to fill the chip; a
  //    round of them costs ~2.5 us per 128-k tile however few run (94-128 us
  //    for M = 17..256), a partial round of its 256 x 128 tiles 0.78 of that
  //    (mfma_cost takes the cheaper tiling);
  //  * the row-blocked weight-streaming GEMM streams the packed weight once per
  //    32 or 64 rows at ~6 TB/s (later passes find it in the 256 MB last-level
  //    cache) and decodes both operands for every MFMA, ~4.6e-15 s per
  //    multiply-add over the rows it computes (N = 12288: 9.4 us at M = 17,
  //    17.6 us at M = 64, 64 us at M = 256, 125 us at M = 512 against 110 us for
  //    the MFMA GEMM).
  const double ktiles = (double)((K + kTileK - 1) / kTileK);
  const double t_mfma = std::min(mfma_cost(M, N, false), mfma_cost(M, N, true)) * ktiles * 2.5e-6;
  const int rp = rows_per_pass(M, N);
  const double passes = (double)((M + rp - 1) / rp);
  const double t_stream = passes * (double)N * (double)K * 0.5625 / 6e12;
  const double t_mac = passes * rp * (double)N * (double)K * 4.6e-15;
  return std::max(t_stream, t_mac) + 3e-6 < t_mfma;
}

bool linear_decode_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= decode_max_rows(K) && K >= kBlock;
}

}  // namespace nvfp4
