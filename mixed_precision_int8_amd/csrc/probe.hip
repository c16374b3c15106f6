// Measurement helper, not part of the method: the peak rate of the matrix-core
// instruction the int8 GEMM is built on (v_mfma_i32_32x32x32_i8), so that the
// GEMM's rate can be set against what the chip delivers at its running clock
// as well as against the published peak.
#include "internal.h"

namespace llmint8 {

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

hipError_t launch_probe_mfma_i8(int blocks, int iters, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(kp_mfma_i8, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, out);
  return hipGetLastError();
}

}  // namespace llmint8
