// The LLM.int8() forward for callers that cannot allocate device memory or
// pass a workspace (code under HIP graph capture, tight serving loops): its
// scratch is a file-scope device array of kScratchBytes, one copy per GPU,
// held from the library's first use on that GPU until the process ends.
//
// Host code never uses the array's name as a device address: on each device,
// at the entry point's first call there (with that device current), the
// array's address is taken once with hipGetSymbolAddress and kept, and only
// that address is handed to the kernels. Nothing here calls hipMalloc,
// hipFree or an allocating library routine.
//
// The kernels write every scratch word they read within the same call (per-row
// group column bitmaps, the outlier set, row statistics, int8 rows and the
// zero-padded outlier operands), so nothing has to be cleared between calls.
// Every call on one GPU shares that GPU's array: calls that overlap on one GPU
// (on different streams, or from different threads) race.
#include <mutex>

#include "../../include/llmint8.h"
#include "internal.h"

namespace llmint8 {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace llmint8

extern "C" llmint8_status llmint8_linear_noalloc(const void* X, int dtype, int64_t T, int64_t K,
                                                 const int8_t* Wq, const float* sW, int64_t N,
                                                 float threshold, const void* bias, void* Y,
                                                 void* stream) {
  return llmint8::linear_static_scratch(X, dtype, T, K, Wq, sW, N, threshold, bias, Y,
                                        llmint8::scratch_address, llmint8::kScratchBytes, stream);
}

extern "C" size_t llmint8_noalloc_scratch_bytes(void) { return llmint8::kScratchBytes; }
