// Host sweep of the C ABI's size limits against the buffer windows the kernels
// build (mixed_precision_int8_amd/csrc/ranges.h, used by both): every shape
// that the admission checks accept must give windows of at most 2^31 bytes, so
// that the kernels' "reads as zero" offset 2^31 lies past every window, and the
// first shape past each limit must be rejected. Built by tests/test_ranges.py.
#include <cstdio>
#include <initializer_list>

#include "../mixed_precision_int8_amd/csrc/ranges.h"

using namespace llmint8;

static int failures = 0;
static long checked = 0;
#define EXPECT(c)                                                                        \
  do {                                                                                   \
    if (!(c)) {                                                                          \
      if (++failures < 20) std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #c); \
    }                                                                                    \
  } while (0)

static bool fits(uint64_t bytes) { return bytes <= kRsrcMaxBytes && bytes <= kOobOffset; }

static void linear_case(int64_t T, int64_t K, int64_t N) {
  if (admit_linear(T, K, N) != LLMINT8_OK) return;
  ++checked;
  if (T > 0) EXPECT(fits(scan_window_bytes((int)T, (int)K, scan_row_groups((int)T))));
  EXPECT(fits(gemm_window_bytes((int)K)));
  EXPECT(fits(gemv_window_bytes((int)K)));
  if (admit_backward(T, K, N) == LLMINT8_OK) EXPECT(fits(backward_window_bytes((int)N)));
}

int main() {
  // int8 forward and backward: every K, T and N at and around each limit and
  // the scan's row-group boundaries
  for (int64_t K = 16; K <= kMaxK + 16; K += 16) {
    const int64_t Tmax = (kTwo31 - 1) / K, Nmax = (kTwo31 - 1) / K;
    for (int64_t T : {int64_t(0), int64_t(1), int64_t(511), int64_t(512), int64_t(513), int64_t(4095),
                      int64_t(4096), int64_t(4097), Tmax / 8, Tmax / 2, Tmax - 1, Tmax, Tmax + 1})
      for (int64_t N : {int64_t(1), int64_t(8), int64_t(4096), Nmax - 1, Nmax, Nmax + 1})
        linear_case(T, K, N);
    EXPECT(admit_linear(Tmax + 1, K, 16) != LLMINT8_OK);
    EXPECT(admit_linear(1, K, Nmax + 1) != LLMINT8_OK);
  }
  EXPECT(admit_linear(1, kMaxK + 16, 16) != LLMINT8_OK);
  // the scan window over every admitted T of a few K (the row groups change with T)
  for (int64_t K : {int64_t(16), int64_t(4096), int64_t(8192), int64_t(14336), int64_t(65536)})
    for (int64_t T = 1; T * K < kTwo31; T += (K >= 4096 ? 1 : 97)) {
      ++checked;
      EXPECT(fits(scan_window_bytes((int)T, (int)K, scan_row_groups((int)T))));
    }
  // blockwise codecs: the largest vectors per lane any block size takes (16 for
  // fp32 blocks of 4096) and the admission edge of n
  for (int vpl = 1; vpl <= 16; vpl *= 2) EXPECT(fits(codec_window_bytes(vpl)));
  for (int64_t block = 64; block <= 4096; block *= 2) {
    EXPECT(admit_blockwise(int64_t(1) << 30, block) == LLMINT8_OK);
    EXPECT(admit_blockwise((int64_t(1) << 30) + 16, block) != LLMINT8_OK);
    EXPECT(admit_4bit(kTwo31 - 16, block) == LLMINT8_OK);
    EXPECT(admit_4bit(kTwo31, block) != LLMINT8_OK);
  }
  EXPECT(admit_blockwise(4096, 96) != LLMINT8_OK && admit_blockwise(4096, 8192) != LLMINT8_OK);
  // 4-bit linear: X windows of 16 rows and the whole code matrix
  for (int64_t K = 128; K <= kLinear4MaxK + 128; K = K < 65536 ? K + 128 : K * 2) {
    const int64_t Tmax = (kTwo31 - 1) / K, Nmax = (kTwo31 - 1) / K;
    for (int64_t T : {int64_t(1), int64_t(15), int64_t(16), int64_t(17), Tmax, Tmax + 1})
      for (int64_t N : {int64_t(1), Nmax, Nmax + 1}) {
        if (admit_linear_4bit(T, K, N) != LLMINT8_OK) continue;
        ++checked;
        EXPECT(fits(linear4_x_window_bytes((int)T, (int)K)));
        EXPECT(fits(linear4_w_window_bytes((int)N, (int)K)));
      }
  }
  EXPECT(admit_linear_4bit(1, 2 * kLinear4MaxK, 1) != LLMINT8_OK);
  if (failures) {
    std::fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  std::printf("ranges ok: %ld shapes\n", checked);
  return 0;
}
