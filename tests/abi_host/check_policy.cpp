// Host-only check of the launch rules in launch.hpp: the wave count of the
// weight-streaming kernels (it fixes their fp32 summation order), the one-launch
// layer's row bounds and k tiles per wave, and the choice between the MFMA
// GEMM's two tilings.  Pins the documented values, and checks over a sweep of
// shapes that every (M, K) the one-launch layer accepts has a kernel instance:
// its waves times tiles per wave cover K, and its row bound is one that exists
// for that product (16 rows up to 40 tiles per workgroup, 8 up to 80, 4 up to
// 160).  Prints one line per failed case and "ok <n>" at the end.
#include <cstdio>

#include "../../nvfp4_w4a4_block_act_amd/csrc/launch.hpp"

using namespace nvfp4;

static int fails = 0, checks = 0;
#define EXPECT(c)                                           \
  do {                                                      \
    ++checks;                                               \
    if (!(c)) {                                             \
      ++fails;                                              \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);      \
    }                                                       \
  } while (0)

int main() {
  // strips per workgroup of the M <= 16 launch
  EXPECT(skinny_strips(768) == 3);     // N = 12288: 256 workgroups
  EXPECT(skinny_strips(320) == 2);     // N = 5120: 160
  EXPECT(skinny_strips(128) == 1);     // N = 2048: 128
  EXPECT(skinny_strips(44) == 1);      // N = 700: 44
  // wave count: eight up to K = 5120 and wherever the launch fills the CUs
  EXPECT(stream_waves(5120, 12288) == 8);
  EXPECT(stream_waves(5120, 2048) == 8);
  EXPECT(stream_waves(5136, 700) == 16);
  EXPECT(stream_waves(17408, 5120) == 16);
  EXPECT(stream_waves(17408, 2048) == 16);
  EXPECT(stream_waves(6144, 5120) == 16);
  EXPECT(stream_waves(10240, 12288) == 8);   // 256 workgroups
  EXPECT(stream_waves(10240, 12300) == 8);   // 257 workgroups
  EXPECT(stream_waves(17408, 700) == 16);
  // one-launch row bounds and tiles per wave
  EXPECT(decode_max_rows(5120) == 16 && decode_max_rows(5136) == 8 && decode_max_rows(10240) == 8);
  EXPECT(decode_max_rows(10256) == 4 && decode_max_rows(20480) == 4 && decode_max_rows(20496) == 0);
  EXPECT(decode_tiles_per_wave(5120, 8) == 5 && decode_tiles_per_wave(10240, 8) == 10);
  EXPECT(decode_tiles_per_wave(17408, 8) == 20 && decode_tiles_per_wave(10240, 16) == 5);
  EXPECT(decode_tiles_per_wave(17408, 16) == 10 && decode_tiles_per_wave(20480, 16) == 10);
  // MFMA tilings: narrow tiles only where they save a partial round
  EXPECT(mfma_narrow(512, 12288) && mfma_narrow(4096, 5120) && mfma_narrow(1536, 12288));
  EXPECT(!mfma_narrow(1024, 12288) && !mfma_narrow(8192, 34816) && !mfma_narrow(32768, 5120));
  EXPECT(!mfma_narrow(4096, 12352));                 // both forms: three rounds plus the ragged strips
  EXPECT(mfma_main_columns(4096, 12352, false) == 12288 && mfma_main_columns(4096, 12352, true) == 12288);
  EXPECT(mfma_main_columns(300, 32808, false) == 32768 && mfma_main_columns(1536, 12300, true) == 12300);
  EXPECT(mfma_rounds(512, 12288, false) == 1.0 && mfma_rounds(512, 12288, true) == kNarrowLoneRound);
  // every accepted one-launch shape has an instance
  const int64_t Ns[] = {16, 700, 2048, 5120, 8192, 12288, 12300, 34816};
  for (int64_t N : Ns)
    for (int64_t K = 16; K <= 20480 + 256; K += 16)
      for (int64_t M = 1; M <= 16; ++M) {
        if (M > decode_max_rows(K)) continue;
        const int nw = stream_waves(K, N), u = decode_tiles_per_wave(K, nw);
        const int64_t tiles = (K + kTileK - 1) / kTileK;
        const bool covers = (int64_t)nw * u >= tiles;
        const bool instance = (nw == 8 || u <= 10) && (nw * u <= 40 || (nw * u <= 80 && M <= 8) || M <= 4);
        ++checks;
        if (!covers || !instance) {
          ++fails;
          std::printf("FAIL M=%lld K=%lld N=%lld: waves %d, tiles per wave %d\n", (long long)M, (long long)K,
                      (long long)N, nw, u);
          if (fails > 20) return 1;
        }
      }
  if (fails) return 1;
  std::printf("ok %d\n", checks);
  return 0;
}
