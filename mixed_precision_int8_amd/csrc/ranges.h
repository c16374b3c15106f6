// Size limits of the C ABI and the byte windows of the buffer resources that
// the kernels build over caller memory. Not part of the public ABI.
//
// A raw buffer load whose offset reaches the resource's size returns zero, and
// the kernels rely on that for ragged edges: a load that must read as zero
// uses the offset kOobOffset = 2^31. That offset is out of range only while
// the resource spans at most 2^31 bytes, so every window a kernel builds is
// bounded by kRsrcMaxBytes. The admission checks of the C ABI and the window
// sizes of the kernels are both written here, once, so that a host test can
// sweep every admitted shape against the windows the kernels will build.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/llmint8.h"

namespace llmint8 {

constexpr uint64_t kRsrcMaxBytes = uint64_t(1) << 31;
constexpr uint32_t kOobOffset = 0x80000000u;  // reads zero in any window of <= kRsrcMaxBytes

constexpr int kMaxK = 65536;          // bitmap prefix tables live in LDS
constexpr int kScanMaxGroups = 8;     // row groups of the column scan (partial bitmaps)
constexpr int kScanRowsPerStep = 512; // rows one scan thread step covers (64 rows x 8 loads)
constexpr int kLinear4MaxK = 1 << 26; // 4-bit linear: 16 rows of X stay within one window
constexpr int64_t kTwo31 = int64_t(1) << 31;

__host__ __device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- admission (host): LLMINT8_OK, or the status the C ABI returns

// int8 forward and weight quantization: X [T, K], Wq [N, K], Y [T, N]
inline int admit_linear(int64_t T, int64_t K, int64_t N) {
  if (T < 0 || K <= 0 || N <= 0) return LLMINT8_ERR_INVALID_ARG;
  if (K % 16 != 0 || K > kMaxK) return LLMINT8_ERR_UNSUPPORTED;
  if (N * K >= kTwo31 || T * K >= kTwo31) return LLMINT8_ERR_UNSUPPORTED;
  if (T * N >= 16 * kTwo31) return LLMINT8_ERR_UNSUPPORTED;  // T < 2^27, N < 2^27: no overflow
  return LLMINT8_OK;
}

// input gradient: also N % 8 == 0 and N <= kMaxK (rows of 2N bytes per tile)
inline int admit_backward(int64_t T, int64_t K, int64_t N) {
  const int st = admit_linear(T, K, N);
  if (st != LLMINT8_OK) return st;
  if (N % 8 != 0 || N > kMaxK) return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

// a power of two in [64, 4096]
inline bool codec_block_ok(int64_t block) {
  return block >= 64 && block <= 4096 && (block & (block - 1)) == 0;
}

// blockwise 8-bit codec: n elements of elem_bytes (2 or 4)
inline int admit_blockwise(int64_t n, int64_t block) {
  if (n < 0 || block <= 0) return LLMINT8_ERR_INVALID_ARG;
  if (!codec_block_ok(block) || n % 16 != 0 || n > (int64_t(1) << 30)) return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

// 4-bit weight codec: n 16-bit elements
inline int admit_4bit(int64_t n, int64_t block) {
  if (n < 0 || block <= 0) return LLMINT8_ERR_INVALID_ARG;
  if (!codec_block_ok(block) || n % 16 != 0 || n >= kTwo31) return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

// 4-bit linear: X [T, K], codes [N, K / 2]
inline int admit_linear_4bit(int64_t T, int64_t K, int64_t N) {
  if (T < 0 || K <= 0 || N <= 0) return LLMINT8_ERR_INVALID_ARG;
  if (K % 128 != 0 || K > kLinear4MaxK || N * K >= kTwo31 || T * K >= kTwo31)
    return LLMINT8_ERR_UNSUPPORTED;
  return LLMINT8_OK;
}

// ---- windows (host and device): bytes of each resource a kernel builds

// column scan: row groups and the window of one group's rows
__host__ __device__ inline int scan_row_groups(int T) {
  const int g = (int)ceil_div64(T, kScanRowsPerStep);
  return g < 1 ? 1 : (g > kScanMaxGroups ? kScanMaxGroups : g);
}
__host__ __device__ inline int scan_rows_per_group(int T, int groups) {
  return (int)ceil_div64(T, groups);
}
__host__ __device__ inline uint64_t scan_window_bytes(int T, int K, int groups) {
  return (uint64_t)scan_rows_per_group(T, groups) * (uint64_t)K * 2u;
}

// blockwise codecs: one wavefront iteration covers 64 lanes x vpl 16-byte vectors
__host__ __device__ inline uint64_t codec_window_bytes(int vpl) { return 64u * 16u * (uint64_t)vpl; }

// 4-bit linear: the 16 rows of X one workgroup reads, and the whole code matrix
__host__ __device__ inline uint64_t linear4_x_window_bytes(int T, int K) {
  return (uint64_t)(T < 16 ? T : 16) * (uint64_t)K * 2u;
}
__host__ __device__ inline uint64_t linear4_w_window_bytes(int N, int K) {
  return (uint64_t)N * (uint64_t)K / 2u;
}

// int8 GEMM operands (the tallest tile has 352 rows), fused decode kernel
// weight rows (16), input-gradient GEMM operands (256 rows of 2N bytes)
__host__ __device__ inline uint64_t gemm_window_bytes(int K) { return 352u * (uint64_t)K; }
__host__ __device__ inline uint64_t gemv_window_bytes(int K) { return 16u * (uint64_t)K; }
__host__ __device__ inline uint64_t backward_window_bytes(int N) { return 256u * 2u * (uint64_t)N; }

}  // namespace llmint8
