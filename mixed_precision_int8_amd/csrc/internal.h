// Internal declarations shared by the host dispatcher and the kernel files.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "ranges.h"

namespace llmint8 {

constexpr int kOutChunk = 32;       // outlier columns per fp16 MFMA k-step
constexpr int kWsChunks = 16;       // outlier chunks a standard workspace materializes (512 columns)
constexpr size_t kWsAlign = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace regions of the GEMM route (byte offsets from the workspace base).
//   parts  uint32 [kScanMaxGroups][KW]      per-row-group column bitmaps
//   bitmap uint32 [KW]                      final outlier bitmap
//   count  int32  [1]                       |O|
//   idx    int32  [K]                       ascending outlier columns
//   aX     fp32   [T]                       row statistic
//   Xq     int8   [T, K]                    quantized activations
//   Xo     16-bit [chunks][T][32]           outlier activations, chunk-major, zero padded
//   Wd     16-bit [chunks][N][32]           dequantized outlier weight columns, same layout
// (16-bit: the activation type, fp16 or bf16) with KW = ceil(K/32) words. Xo
// and Wd hold the first `chunks` chunks of 32 outlier columns; the epilogue
// forms any chunk past them from X and Wq directly (same values, fewer reuse).
// The fixed part (up to Xq) does not depend on the data; a workspace of
// gemm_workspace_bytes(T, K, N) materializes min(ceil(K/32), kWsChunks) chunks,
// and a larger one as many more as fit.
struct WsLayout {
  size_t parts, bitmap, count, idx, aX, Xq, Xo, Wd, total;
  int chunks;
};

inline WsLayout ws_layout(int64_t T, int64_t K, int64_t N, int64_t chunks) {
  WsLayout L;
  const int64_t KW = ceil_div(K, 32);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, kWsAlign);
    return o;
  };
  L.parts = take(sizeof(uint32_t) * kScanMaxGroups * KW);
  L.bitmap = take(sizeof(uint32_t) * KW);
  L.count = take(sizeof(int32_t) * 4);
  L.idx = take(sizeof(int32_t) * K);
  L.aX = take(sizeof(float) * (T > 0 ? T : 1));
  L.Xq = take((size_t)T * K);
  L.Xo = take(sizeof(uint16_t) * chunks * kOutChunk * (size_t)T);
  L.Wd = take(sizeof(uint16_t) * chunks * kOutChunk * (size_t)N);
  L.total = off;
  L.chunks = (int)chunks;
  return L;
}

// bytes of one materialized chunk (Xo and Wd, each region rounded up)
inline size_t ws_chunk_bytes(int64_t T, int64_t N) { return 2 * kOutChunk * (size_t)(T + N); }
// the standard GEMM workspace: min(ceil(K/32), kWsChunks) chunks
inline size_t gemm_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  return ws_layout(T, K, N, std::min<int64_t>(ceil_div(K, kOutChunk), kWsChunks)).total;
}
// the layout of a workspace of `bytes` (>= the fixed part plus one chunk): as
// many chunks as fit, up to ceil(K/32); chunks = 0 when not even one fits
inline WsLayout ws_layout_for(int64_t T, int64_t K, int64_t N, size_t bytes) {
  const int64_t KC = ceil_div(K, kOutChunk);
  int64_t lo = 0, hi = KC;  // largest chunk count whose layout fits
  if (ws_layout(T, K, N, 0).total > bytes) return ws_layout(T, K, N, 0);
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (ws_layout(T, K, N, mid).total <= bytes) lo = mid; else hi = mid - 1;
  }
  return ws_layout(T, K, N, lo);
}

// Pointers into a workspace, plus optional debug destinations.
struct LinearArgs {
  const uint16_t* X;
  const int8_t* Wq;
  const float* sW;
  uint16_t* Y;
  int T, K, N;
  float thr;
  int bf16;              // activation type: 0 fp16, 1 bf16 (X, bias, Y, Xo, Wd)
  const uint16_t* bias;  // [N] in the activation type, or null
  // workspace
  uint32_t* parts;
  uint32_t* bitmap;
  int32_t* count;
  int32_t* idx;
  float* aX;
  int8_t* Xq;
  uint16_t* Xo;
  uint16_t* Wd;
  int wchunks;  // outlier chunks held in Xo / Wd (>= 1); later chunks are formed in the epilogue
  // debug outputs (nullable)
  uint32_t* dbg_bitmap;
  int32_t* dbg_idx;
  int32_t* dbg_count;
  int8_t* dbg_Xq;
  float* dbg_aX;
  int32_t* dbg_C;
};

// Operands of the input gradient dX = dY . Wdeq.
struct BwdArgs {
  const uint16_t* dY;  // 16-bit [T, N]
  const int8_t* Wq;    // int8 [N, K] and its scales [N] (dequantized on the fly)
  const float* sW;
  uint16_t* dX;        // 16-bit [T, K]
  int T, K, N;
  int bf16;            // 16-bit type: 0 fp16, 1 bf16
};

// The forward on the library's static scratch (no workspace argument): after
// every argument check passes on the GEMM route, `scratch` gives the current
// device's scratch address; the fixed part of the layout and one outlier chunk
// must fit in scratch_bytes (LLMINT8_ERR_WORKSPACE otherwise).
typedef hipError_t (*ScratchSource)(void** address);
int linear_static_scratch(const void* X, int dtype, int64_t T, int64_t K, const int8_t* Wq,
                          const float* sW, int64_t N, float threshold, const void* bias, void* Y,
                          ScratchSource scratch, size_t scratch_bytes, void* stream);

// Launchers (each enqueues exactly one kernel on `stream`).
hipError_t launch_quantize_weight(const uint16_t* W, int N, int K, int8_t* Wq, float* sW, bool bf16,
                                  hipStream_t stream);
uint32_t threshold_code(float thr, bool bf16);  // smallest 16-bit |x| code whose value reaches thr
hipError_t launch_scan(const LinearArgs& a, int groups, hipStream_t stream);
hipError_t launch_prepare(const LinearArgs& a, int groups, int num_cus, hipStream_t stream);
// int8 GEMM tiles (N x T): 256x256, 192x256, 256x128, 128x128, 352x256; the
// host picks one by cost unless `tile` (0..kGemmTiles-1) forces it.
constexpr int kGemmTiles = 5;
int choose_gemm_tile(int64_t T, int64_t N, int num_cus);  // host: the cost model's candidate
hipError_t launch_gemm(const LinearArgs& a, int num_cus, hipStream_t stream, int tile = -1);
int gemv_max_rows(int K);
hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream);
hipError_t launch_dequant_t(const int8_t* Wq, const float* sW, int N, int K, uint16_t* WdT,
                            bool bf16, hipStream_t stream);
// dX = dY . Wdeq in one kernel, Wq dequantized into the 16-bit operand on the fly
hipError_t launch_backward_dq(const BwdArgs& a, int num_cus, hipStream_t stream);
hipError_t launch_quantize_blockwise(const void* x, bool f32, int n, int block, int8_t* q,
                                     float* absmax, int num_cus, hipStream_t stream);
hipError_t launch_dequantize_blockwise(const int8_t* q, const float* absmax, int n, int block,
                                       void* out, bool f32, int num_cus, hipStream_t stream);


// 4-bit weights (NF4 / FP4): a code book and its quantizer's decision table.
struct Code4 {
  float value[16];   // value of each code
  float mid[15];     // midpoints between adjacent distinct levels, ascending (+inf when unused)
  uint32_t rank_lo;  // code of the level of rank r (r < 8) in nibble r
  uint32_t rank_hi;  // code of the level of rank r (8 <= r < 16) in nibble r - 8
};
bool code_book_4bit(int quant_type, Code4* out);  // false for an unknown type (host)

// Operands of the 4-bit linear Y = X . Wdeq^T (+ bias).
struct FourBitArgs {
  const uint16_t* X;     // [T, K], 16-bit
  const uint8_t* W4;     // [N, K] codes, two per byte, even index in the low nibble
  const float* absmax;   // one per block of the flat weight
  const uint16_t* bias;  // [N] or null
  uint16_t* Y;           // [T, N]
  int T, K, N, block_shift;
};
hipError_t launch_quantize_4bit(const uint16_t* w, bool bf16, int n, int block, const Code4& book,
                                uint8_t* packed, float* absmax, int num_cus, hipStream_t stream);
hipError_t launch_dequantize_4bit(const uint8_t* packed, const float* absmax, int n, int block,
                                  const Code4& book, uint16_t* out, bool bf16, int num_cus,
                                  hipStream_t stream);
hipError_t launch_linear_4bit(const FourBitArgs& a, const Code4& book, bool bf16, int num_cus,
                              hipStream_t stream);

}  // namespace llmint8
