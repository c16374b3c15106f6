// Measurement helper of the benchmark, not part of the method and not part of
// libllmint8: the peak rate of the matrix-core instruction the int8 GEMM is
// built on (v_mfma_i32_32x32x32_i8), so that the GEMM's rate can be set against
// what the chip delivers at its running clock as well as against the published
// peak. Built on its own as libllmint8_probe.so; only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 4;  // independent accumulators per wavefront

// Each wavefront issues iters x kProbeChains MFMAs from register operands, with
// no memory traffic, then stores one checksum per thread.
__global__ __launch_bounds__(kProbeThreads) void kp_mfma_i8(int iters, int32_t* __restrict__ out) {
  const v4i a = {(int)threadIdx.x, 1, 2, 3}, b = {3, 2, 1, (int)threadIdx.x};
  v16i c[kProbeChains] = {};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += c[j][0] + c[j][15];
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// Enqueues `blocks` workgroups of 256 threads on `stream` (a hipStream_t); each
// of their 4 wavefronts issues iters x 4 MFMAs (65536 int8 operations each),
// then every thread writes one checksum to out (int32 [blocks * 256], device).
// Returns 0, -1 for blocks <= 0, iters <= 0 or a null / misaligned out, or -4
// when the launch fails.
extern "C" __attribute__((visibility("default"))) int llmint8_bench_probe_mfma_i8(int blocks, int iters,
                                                                                int32_t* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out || (reinterpret_cast<uintptr_t>(out) & 3u) != 0) return -1;
  hipLaunchKernelGGL(kp_mfma_i8, dim3(blocks), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
