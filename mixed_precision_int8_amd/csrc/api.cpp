// Host side of the C ABI declared in include/llmint8.h: argument validation,
// workspace carving, kernel-route choice and launches on the caller's stream.
// Nothing here allocates device memory, synchronises the host or copies device
// data to the host; validation runs before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/llmint8.h"
#include "internal.h"

using namespace llmint8;

namespace {

thread_local int g_last_hip_error = 0;

llmint8_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LLMINT8_OK;
  g_last_hip_error = (int)e;
  return LLMINT8_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// size limits: ranges.h (shared with the kernels' buffer windows)
llmint8_status check_sizes(int64_t T, int64_t K, int64_t N) { return admit_linear(T, K, N); }

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

llmint8_status validate_linear(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                               const float* sW, int64_t N, float threshold, void* Y,
                               void* workspace, size_t workspace_bytes, int dtype,
                               const void* bias) {
  llmint8_status st = check_sizes(T, K, N);
  if (st != LLMINT8_OK) return st;
  if (dtype != LLMINT8_DTYPE_F16 && dtype != LLMINT8_DTYPE_BF16) return LLMINT8_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 2)) return LLMINT8_ERR_INVALID_ARG;
  if (std::isnan(threshold) || !(threshold > 0.0f)) return LLMINT8_ERR_INVALID_ARG;
  if (!Wq || !sW) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(Wq, 16) || !aligned(sW, 4)) return LLMINT8_ERR_INVALID_ARG;
  if (T == 0) return LLMINT8_OK;
  if (!X || !Y) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Y, 16)) return LLMINT8_ERR_INVALID_ARG;
  return LLMINT8_OK;
}

// The GEMM route's workspace: present, aligned, and at least the standard size.
llmint8_status validate_workspace(int64_t T, int64_t K, int64_t N, void* workspace,
                                  size_t workspace_bytes) {
  if (!workspace || !aligned(workspace, kWsAlign)) return LLMINT8_ERR_INVALID_ARG;
  if (workspace_bytes < gemm_workspace_bytes(T, K, N)) return LLMINT8_ERR_WORKSPACE;
  return LLMINT8_OK;
}

LinearArgs make_args(const void* X, int64_t T, int64_t K, const int8_t* Wq, const float* sW,
                     int64_t N, float threshold, void* Y, void* workspace, size_t workspace_bytes,
                     int dtype, const void* bias) {
  LinearArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.Wq = Wq;
  a.sW = sW;
  a.Y = static_cast<uint16_t*>(Y);
  a.T = (int)T;
  a.K = (int)K;
  a.N = (int)N;
  a.thr = threshold;
  a.bf16 = dtype == LLMINT8_DTYPE_BF16 ? 1 : 0;
  a.bias = static_cast<const uint16_t*>(bias);
  if (!workspace) return a;  // the fused decode route
  const WsLayout L = ws_layout_for(T, K, N, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  a.parts = reinterpret_cast<uint32_t*>(ws + L.parts);
  a.bitmap = reinterpret_cast<uint32_t*>(ws + L.bitmap);
  a.count = reinterpret_cast<int32_t*>(ws + L.count);
  a.idx = reinterpret_cast<int32_t*>(ws + L.idx);
  a.aX = reinterpret_cast<float*>(ws + L.aX);
  a.Xq = reinterpret_cast<int8_t*>(ws + L.Xq);
  a.Xo = reinterpret_cast<uint16_t*>(ws + L.Xo);
  a.Wd = reinterpret_cast<uint16_t*>(ws + L.Wd);
  a.wchunks = L.chunks;
  return a;
}

int choose_path(int path, int64_t T, int64_t K) {
  if (path == LLMINT8_PATH_AUTO) return T <= gemv_max_rows((int)K) ? LLMINT8_PATH_GEMV : LLMINT8_PATH_GEMM;
  return path == LLMINT8_PATH_GEMV ? LLMINT8_PATH_GEMV : LLMINT8_PATH_GEMM;
}

static_assert(LLMINT8_PATH_GEMM_352x256 - LLMINT8_PATH_GEMM_256x256 + 1 == kGemmTiles,
              "one path value per GEMM tile, in the order of launch_gemm's candidates");
// A forced GEMM tile from the path argument, or -1 (the cost model picks).
int forced_tile(int path) {
  return path >= LLMINT8_PATH_GEMM_256x256 && path < LLMINT8_PATH_GEMM_256x256 + kGemmTiles
             ? path - LLMINT8_PATH_GEMM_256x256
             : -1;
}

// The whole forward; `events` (nullable) are recorded around each kernel.
llmint8_status run_linear(const void* X, int64_t T, int64_t K, const int8_t* Wq, const float* sW,
                          int64_t N, float threshold, void* Y, void* workspace,
                          size_t workspace_bytes, void* stream_ptr, int path,
                          uint32_t* dbg_bitmap, int32_t* dbg_idx, int32_t* dbg_count,
                          int8_t* dbg_Xq, float* dbg_aX, int32_t* dbg_C,
                          void* const* events, int n_events, int* kernels_launched,
                          int dtype = LLMINT8_DTYPE_F16, const void* bias = nullptr,
                          ScratchSource scratch = nullptr) {
  if (kernels_launched) *kernels_launched = 0;
  llmint8_status st = validate_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes,
                                      dtype, bias);
  if (st != LLMINT8_OK) return st;
  if (path != LLMINT8_PATH_AUTO && path != LLMINT8_PATH_GEMM && path != LLMINT8_PATH_GEMV &&
      forced_tile(path) < 0)
    return LLMINT8_ERR_INVALID_ARG;
  const int route = choose_path(path, T, K);
  if (route == LLMINT8_PATH_GEMV && T > gemv_max_rows((int)K)) return LLMINT8_ERR_UNSUPPORTED;
  const int nk = route == LLMINT8_PATH_GEMV ? 1 : 3;
  if (events && n_events < nk + 1) return LLMINT8_ERR_INVALID_ARG;
  if (T == 0) return LLMINT8_OK;
  // the fused decode kernel keeps everything in LDS: no workspace
  if (route == LLMINT8_PATH_GEMM) {
    if (scratch) {
      // the library's static scratch: the fixed part and one outlier chunk must fit
      if (ws_layout(T, K, N, 1).total > workspace_bytes) return LLMINT8_ERR_WORKSPACE;
      const hipError_t se = scratch(&workspace);
      if (se != hipSuccess) return hip_status(se);
    } else {
      st = validate_workspace(T, K, N, workspace, workspace_bytes);
      if (st != LLMINT8_OK) return st;
    }
  }

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  LinearArgs a = route == LLMINT8_PATH_GEMM
                     ? make_args(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, dtype, bias)
                     : make_args(X, T, K, Wq, sW, N, threshold, Y, nullptr, 0, dtype, bias);
  a.dbg_C = dbg_C;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) : hipSuccess;
  };
  const int cus = device_cu_count();
  hipError_t e = mark(0);
  if (e != hipSuccess) return hip_status(e);
  if (route == LLMINT8_PATH_GEMV) {
    a.dbg_bitmap = dbg_bitmap;
    a.dbg_idx = dbg_idx;
    a.dbg_count = dbg_count;
    a.dbg_Xq = dbg_Xq;
    a.dbg_aX = dbg_aX;
    e = launch_gemv(a, stream);
    if (e == hipSuccess) e = mark(1);
    if (e != hipSuccess) return hip_status(e);
    if (kernels_launched) *kernels_launched = 1;
    return LLMINT8_OK;
  }
  const int groups = scan_row_groups((int)T);
  e = launch_scan(a, groups, stream);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess) e = launch_prepare(a, groups, cus, stream);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) e = launch_gemm(a, cus, stream, forced_tile(path));
  if (e == hipSuccess) e = mark(3);
  if (e != hipSuccess) return hip_status(e);
  if (kernels_launched) *kernels_launched = 3;
  // intermediate copies for the debug entry point (device to device, async)
  const size_t KW = (size_t)ceil_div(K, 32);
  if (dbg_bitmap) e = hipMemcpyAsync(dbg_bitmap, a.bitmap, KW * 4, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && dbg_idx)
    e = hipMemcpyAsync(dbg_idx, a.idx, (size_t)K * 4, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && dbg_count)
    e = hipMemcpyAsync(dbg_count, a.count, 4, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && dbg_Xq)
    e = hipMemcpyAsync(dbg_Xq, a.Xq, (size_t)T * K, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && dbg_aX)
    e = hipMemcpyAsync(dbg_aX, a.aX, (size_t)T * 4, hipMemcpyDeviceToDevice, stream);
  return hip_status(e);
}

// dY rows and WdT rows (2N bytes) are copied in whole 16-byte pieces, and a tile's
// rows x 2N bytes must stay within one buffer window
llmint8_status check_backward_sizes(int64_t T, int64_t K, int64_t N) { return admit_backward(T, K, N); }

// dX = dY . Wdeq in one kernel (Wq dequantized on the fly); no workspace.
llmint8_status run_backward_input(const void* dY, int64_t T, int64_t K, const int8_t* Wq,
                                  const float* sW, int64_t N, void* dX, void* stream_ptr,
                                  void* const* events, int n_events, int* kernels_launched,
                                  int dtype = LLMINT8_DTYPE_F16) {
  if (kernels_launched) *kernels_launched = 0;
  llmint8_status st = check_backward_sizes(T, K, N);
  if (st != LLMINT8_OK) return st;
  if (dtype != LLMINT8_DTYPE_F16 && dtype != LLMINT8_DTYPE_BF16) return LLMINT8_ERR_INVALID_ARG;
  if (!Wq || !sW || !aligned(Wq, 16) || !aligned(sW, 4)) return LLMINT8_ERR_INVALID_ARG;
  if (events && n_events < 2) return LLMINT8_ERR_INVALID_ARG;
  if (T == 0) return LLMINT8_OK;
  if (!dY || !dX) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(dY, 16) || !aligned(dX, 16)) return LLMINT8_ERR_INVALID_ARG;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) : hipSuccess;
  };
  BwdArgs a{};
  a.dY = static_cast<const uint16_t*>(dY);
  a.Wq = Wq;
  a.sW = sW;
  a.dX = static_cast<uint16_t*>(dX);
  a.T = (int)T;
  a.K = (int)K;
  a.N = (int)N;
  a.bf16 = dtype == LLMINT8_DTYPE_BF16 ? 1 : 0;
  hipError_t e = mark(0);
  if (e == hipSuccess) e = launch_backward_dq(a, device_cu_count(), stream);
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return hip_status(e);
  if (kernels_launched) *kernels_launched = 1;
  return LLMINT8_OK;
}

}  // namespace

namespace llmint8 {
llmint8_status linear_static_scratch(const void* X, int dtype, int64_t T, int64_t K, const int8_t* Wq,
                                     const float* sW, int64_t N, float threshold, const void* bias,
                                     void* Y, ScratchSource scratch, size_t scratch_bytes, void* stream) {
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, nullptr, scratch_bytes, stream, LLMINT8_PATH_AUTO,
                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, dtype,
                    bias, scratch);
}
}  // namespace llmint8

extern "C" {

llmint8_status llmint8_quantize_weight_ex(const void* W, int dtype, int64_t N, int64_t K, int8_t* Wq,
                                          float* sW, void* stream) {
  llmint8_status st = check_sizes(0, K, N);
  if (st != LLMINT8_OK) return st;
  if (dtype != LLMINT8_DTYPE_F16 && dtype != LLMINT8_DTYPE_BF16) return LLMINT8_ERR_INVALID_ARG;
  if (!W || !Wq || !sW) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(sW, 4)) return LLMINT8_ERR_INVALID_ARG;
  return hip_status(launch_quantize_weight(static_cast<const uint16_t*>(W), (int)N, (int)K, Wq, sW,
                                           dtype == LLMINT8_DTYPE_BF16, static_cast<hipStream_t>(stream)));
}

llmint8_status llmint8_quantize_weight(const void* W, int64_t N, int64_t K, int8_t* Wq, float* sW,
                                       void* stream) {
  return llmint8_quantize_weight_ex(W, LLMINT8_DTYPE_F16, N, K, Wq, sW, stream);
}

size_t llmint8_workspace_bytes_path(int64_t T, int64_t K, int64_t N, int path) {
  if (check_sizes(T, K, N) != LLMINT8_OK) return 0;
  if (path != LLMINT8_PATH_AUTO && path != LLMINT8_PATH_GEMM && path != LLMINT8_PATH_GEMV &&
      forced_tile(path) < 0)
    return 0;
  if (T == 0 || choose_path(path, T, K) == LLMINT8_PATH_GEMV) return 0;
  return gemm_workspace_bytes(T, K, N);
}

size_t llmint8_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  return llmint8_workspace_bytes_path(T, K, N, LLMINT8_PATH_AUTO);
}

llmint8_status llmint8_linear(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                              const float* sW, int64_t N, float threshold, void* Y,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, stream,
                    LLMINT8_PATH_AUTO, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, 0, nullptr);
}

llmint8_status llmint8_linear_ex(const void* X, int dtype, int64_t T, int64_t K, const int8_t* Wq,
                                 const float* sW, int64_t N, float threshold, const void* bias,
                                 void* Y, void* workspace, size_t workspace_bytes, void* stream) {
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, stream,
                    LLMINT8_PATH_AUTO, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, 0, nullptr, dtype, bias);
}

llmint8_status llmint8_linear_debug_ex(const void* X, int dtype, int64_t T, int64_t K,
                                       const int8_t* Wq, const float* sW, int64_t N, float threshold,
                                       const void* bias, void* Y, void* workspace,
                                       size_t workspace_bytes, void* stream, int path,
                                       uint32_t* outlier_bitmap, int32_t* outlier_idx,
                                       int32_t* outlier_count, int8_t* Xq, float* aX, int32_t* C) {
  if ((outlier_bitmap && !aligned(outlier_bitmap, 4)) || (outlier_idx && !aligned(outlier_idx, 4)) ||
      (outlier_count && !aligned(outlier_count, 4)) || (Xq && !aligned(Xq, 16)) ||
      (aX && !aligned(aX, 4)) || (C && !aligned(C, 16)))
    return LLMINT8_ERR_INVALID_ARG;
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, stream, path,
                    outlier_bitmap, outlier_idx, outlier_count, Xq, aX, C, nullptr, 0, nullptr,
                    dtype, bias);
}

llmint8_status llmint8_linear_timed_ex(const void* X, int dtype, int64_t T, int64_t K,
                                       const int8_t* Wq, const float* sW, int64_t N, float threshold,
                                       const void* bias, void* Y, void* workspace,
                                       size_t workspace_bytes, void* stream, int path,
                                       void* const* events, int n_events, int* kernels_launched) {
  if (!events || n_events < 2) return LLMINT8_ERR_INVALID_ARG;
  for (int i = 0; i < n_events && i < 4; ++i)
    if (!events[i]) return LLMINT8_ERR_INVALID_ARG;
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, stream, path,
                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, events, n_events,
                    kernels_launched, dtype, bias);
}

llmint8_status llmint8_linear_debug(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                    const float* sW, int64_t N, float threshold, void* Y,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int path, uint32_t* outlier_bitmap, int32_t* outlier_idx,
                                    int32_t* outlier_count, int8_t* Xq, float* aX, int32_t* C) {
  if ((outlier_bitmap && !aligned(outlier_bitmap, 4)) || (outlier_idx && !aligned(outlier_idx, 4)) ||
      (outlier_count && !aligned(outlier_count, 4)) || (Xq && !aligned(Xq, 16)) ||
      (aX && !aligned(aX, 4)) || (C && !aligned(C, 16)))
    return LLMINT8_ERR_INVALID_ARG;
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, stream, path,
                    outlier_bitmap, outlier_idx, outlier_count, Xq, aX, C, nullptr, 0, nullptr);
}

llmint8_status llmint8_linear_timed(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                    const float* sW, int64_t N, float threshold, void* Y,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int path, void* const* events, int n_events,
                                    int* kernels_launched) {
  if (!events || n_events < 2) return LLMINT8_ERR_INVALID_ARG;
  for (int i = 0; i < n_events && i < 4; ++i)
    if (!events[i]) return LLMINT8_ERR_INVALID_ARG;
  return run_linear(X, T, K, Wq, sW, N, threshold, Y, workspace, workspace_bytes, stream, path,
                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, events, n_events,
                    kernels_launched);
}

size_t llmint8_backward_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  (void)T;
  (void)K;
  (void)N;
  return 0;  // the weight is dequantized on the fly; nothing is staged in memory
}

llmint8_status llmint8_dequantize_weight_t_ex(const int8_t* Wq, const float* sW, int64_t N,
                                              int64_t K, void* WdT, int dtype, void* stream) {
  llmint8_status st = check_backward_sizes(0, K, N);
  if (st != LLMINT8_OK) return st;
  if (dtype != LLMINT8_DTYPE_F16 && dtype != LLMINT8_DTYPE_BF16) return LLMINT8_ERR_INVALID_ARG;
  if (!Wq || !sW || !WdT) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(Wq, 16) || !aligned(sW, 4) || !aligned(WdT, 16)) return LLMINT8_ERR_INVALID_ARG;
  return hip_status(launch_dequant_t(Wq, sW, (int)N, (int)K, static_cast<uint16_t*>(WdT),
                                     dtype == LLMINT8_DTYPE_BF16, static_cast<hipStream_t>(stream)));
}

llmint8_status llmint8_dequantize_weight_t(const int8_t* Wq, const float* sW, int64_t N, int64_t K,
                                           void* WdT, void* stream) {
  return llmint8_dequantize_weight_t_ex(Wq, sW, N, K, WdT, LLMINT8_DTYPE_F16, stream);
}

llmint8_status llmint8_linear_backward_input_ex(const void* dY, int dtype, int64_t T, int64_t K,
                                                const int8_t* Wq, const float* sW, int64_t N,
                                                void* dX, void* workspace, size_t workspace_bytes,
                                                void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return run_backward_input(dY, T, K, Wq, sW, N, dX, stream, nullptr, 0, nullptr, dtype);
}

llmint8_status llmint8_linear_backward_input(const void* dY, int64_t T, int64_t K, const int8_t* Wq,
                                             const float* sW, int64_t N, void* dX, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return run_backward_input(dY, T, K, Wq, sW, N, dX, stream, nullptr, 0, nullptr);
}

llmint8_status llmint8_linear_backward_input_timed(const void* dY, int64_t T, int64_t K,
                                                   const int8_t* Wq, const float* sW, int64_t N,
                                                   void* dX, void* workspace, size_t workspace_bytes,
                                                   void* stream, void* const* events, int n_events,
                                                   int* kernels_launched) {
  if (!events || n_events < 2) return LLMINT8_ERR_INVALID_ARG;
  for (int i = 0; i < 2; ++i)
    if (!events[i]) return LLMINT8_ERR_INVALID_ARG;
  (void)workspace;
  (void)workspace_bytes;
  return run_backward_input(dY, T, K, Wq, sW, N, dX, stream, events, n_events, kernels_launched);
}

static llmint8_status check_blockwise(int dtype, int64_t n, int64_t block) {
  // the codec takes fp16 or fp32 tensors
  if (dtype != LLMINT8_DTYPE_F16 && dtype != LLMINT8_DTYPE_F32) return LLMINT8_ERR_INVALID_ARG;
  return admit_blockwise(n, block);
}

llmint8_status llmint8_quantize_blockwise(const void* x, int dtype, int64_t n, int64_t block,
                                          int8_t* q, float* absmax, void* stream) {
  llmint8_status st = check_blockwise(dtype, n, block);
  if (st != LLMINT8_OK) return st;
  if (n == 0) return LLMINT8_OK;
  if (!x || !q || !absmax) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(absmax, 4)) return LLMINT8_ERR_INVALID_ARG;
  return hip_status(launch_quantize_blockwise(x, dtype == LLMINT8_DTYPE_F32, (int)n, (int)block, q,
                                              absmax, device_cu_count(),
                                              static_cast<hipStream_t>(stream)));
}

llmint8_status llmint8_dequantize_blockwise(const int8_t* q, const float* absmax, int64_t n,
                                            int64_t block, void* out, int dtype, void* stream) {
  llmint8_status st = check_blockwise(dtype, n, block);
  if (st != LLMINT8_OK) return st;
  if (n == 0) return LLMINT8_OK;
  if (!q || !absmax || !out) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(absmax, 4)) return LLMINT8_ERR_INVALID_ARG;
  return hip_status(launch_dequantize_blockwise(q, absmax, (int)n, (int)block, out,
                                                dtype == LLMINT8_DTYPE_F32, device_cu_count(),
                                                static_cast<hipStream_t>(stream)));
}

static llmint8_status check_4bit(int dtype, int quant_type, int64_t n, int64_t block) {
  if (dtype != LLMINT8_DTYPE_F16 && dtype != LLMINT8_DTYPE_BF16) return LLMINT8_ERR_INVALID_ARG;
  if (quant_type != LLMINT8_QUANT_NF4 && quant_type != LLMINT8_QUANT_FP4) return LLMINT8_ERR_INVALID_ARG;
  return admit_4bit(n, block);
}

llmint8_status llmint8_code_book_4bit(int quant_type, float* values) {
  if (!values) return LLMINT8_ERR_INVALID_ARG;
  Code4 book;
  if (!code_book_4bit(quant_type, &book)) return LLMINT8_ERR_INVALID_ARG;
  for (int c = 0; c < 16; ++c) values[c] = book.value[c];
  return LLMINT8_OK;
}

llmint8_status llmint8_quantize_4bit(const void* W, int dtype, int64_t n, int64_t block,
                                     int quant_type, uint8_t* packed, float* absmax, void* stream) {
  llmint8_status st = check_4bit(dtype, quant_type, n, block);
  if (st != LLMINT8_OK) return st;
  if (n == 0) return LLMINT8_OK;
  if (!W || !packed || !absmax) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(absmax, 4)) return LLMINT8_ERR_INVALID_ARG;
  Code4 book;
  code_book_4bit(quant_type, &book);
  return hip_status(launch_quantize_4bit(static_cast<const uint16_t*>(W), dtype == LLMINT8_DTYPE_BF16,
                                         (int)n, (int)block, book, packed, absmax, device_cu_count(),
                                         static_cast<hipStream_t>(stream)));
}

llmint8_status llmint8_dequantize_4bit(const uint8_t* packed, const float* absmax, int64_t n,
                                       int64_t block, int quant_type, void* out, int dtype,
                                       void* stream) {
  llmint8_status st = check_4bit(dtype, quant_type, n, block);
  if (st != LLMINT8_OK) return st;
  if (n == 0) return LLMINT8_OK;
  if (!packed || !absmax || !out) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(packed, 16) || !aligned(absmax, 4) || !aligned(out, 16)) return LLMINT8_ERR_INVALID_ARG;
  Code4 book;
  code_book_4bit(quant_type, &book);
  return hip_status(launch_dequantize_4bit(packed, absmax, (int)n, (int)block, book,
                                           static_cast<uint16_t*>(out), dtype == LLMINT8_DTYPE_BF16,
                                           device_cu_count(), static_cast<hipStream_t>(stream)));
}

llmint8_status llmint8_linear_4bit(const void* X, int dtype, int64_t T, int64_t K,
                                   const uint8_t* packed, const float* absmax, int64_t block,
                                   int quant_type, int64_t N, const void* bias, void* Y,
                                   void* stream) {
  if (T < 0 || K <= 0 || N <= 0) return LLMINT8_ERR_INVALID_ARG;
  llmint8_status st = check_4bit(dtype, quant_type, 0, block);
  if (st != LLMINT8_OK) return st;
  st = admit_linear_4bit(T, K, N);
  if (st != LLMINT8_OK) return st;
  if (T == 0) return LLMINT8_OK;
  if (!X || !packed || !absmax || !Y) return LLMINT8_ERR_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(absmax, 4) || !aligned(Y, 2) ||
      (bias && !aligned(bias, 2)))
    return LLMINT8_ERR_INVALID_ARG;
  Code4 book;
  code_book_4bit(quant_type, &book);
  int shift = 0;
  while ((int64_t(1) << shift) < block) ++shift;
  FourBitArgs a;
  a.X = static_cast<const uint16_t*>(X);
  a.W4 = packed;
  a.absmax = absmax;
  a.bias = static_cast<const uint16_t*>(bias);
  a.Y = static_cast<uint16_t*>(Y);
  a.T = (int)T;
  a.K = (int)K;
  a.N = (int)N;
  a.block_shift = shift;
  return hip_status(launch_linear_4bit(a, book, dtype == LLMINT8_DTYPE_BF16, device_cu_count(),
                                       static_cast<hipStream_t>(stream)));
}

int llmint8_gemm_tile(int64_t T, int64_t N) {
  if (T <= 0 || N <= 0) return LLMINT8_ERR_INVALID_ARG;
  return LLMINT8_PATH_GEMM_256x256 + choose_gemm_tile(T, N, device_cu_count());
}

int llmint8_gemv_max_rows(int64_t K) {
  if (K <= 0 || K % 16 != 0 || K > kMaxK) return 0;
  return gemv_max_rows((int)K);
}

const char* llmint8_status_string(llmint8_status status) {
  switch (status) {
    case LLMINT8_OK: return "ok";
    case LLMINT8_ERR_INVALID_ARG: return "invalid argument";
    case LLMINT8_ERR_UNSUPPORTED: return "unsupported shape";
    case LLMINT8_ERR_WORKSPACE: return "workspace too small";
    case LLMINT8_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int llmint8_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
