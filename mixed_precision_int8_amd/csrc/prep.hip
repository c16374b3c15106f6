// Quantization-side kernels of the LLM.int8() forward on gfx950:
//   kw_quantize_rows  vector-wise int8 weight quantization, once at load time
//   ka_scan           outlier feature-column scan over X (per row group)
//   ka_prepare        row absmax over non-outlier columns, int8 quantization of
//                     X, gather of the outlier activations and of the
//                     dequantized outlier weight columns
// Sources: "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
// Explained", sections 2 and 3; "bitsandbytes: GPU-Accelerated Inference and
// Training at Lower Bit Depths", "How LLM.int8() quantizes weights and
// activations"; "bitsandbytes" glossary, introduction (load-time quantization).
//
// All three are HBM-bound streaming kernels: 16-byte coalesced loads, |x| taken
// on the fp16 bit pattern (exact), wavefront reductions, and the outlier bitmap
// plus its prefix counts kept in LDS.
#include <cmath>

#include "device_util.h"
#include "internal.h"

namespace llmint8 {

// ---------------------------------------------------------------------------
// Weight quantization: one wavefront per output row.
//   sW[n] = max_k |W[n,k]|,  Wq[n,k] = rne(fl32(W[n,k] * fl32(127 / sW[n])))
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kw_quantize_rows(const uint16_t* __restrict__ W, int N,
                                                        int K, int8_t* __restrict__ Wq,
                                                        float* __restrict__ sW) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wave;
  if (n >= N) return;
  const uint4* row = reinterpret_cast<const uint4*>(W + (size_t)n * K);
  const int chunks = K >> 3;
  v2u16 m2 = {0, 0};
  for (int c = lane; c < chunks; c += 64) {
    v2u16 a[4];
    abs_codes(row[c], a);
    m2 = __builtin_elementwise_max(m2, __builtin_elementwise_max(
                                           __builtin_elementwise_max(a[0], a[1]),
                                           __builtin_elementwise_max(a[2], a[3])));
  }
  const int m = wave_max_i(max((int)m2.x, (int)m2.y));
  const float b = half_bits_to_float((uint32_t)m);
  const float s = m > 0 ? 127.0f / b : 0.0f;
  uint2* out = reinterpret_cast<uint2*>(Wq + (size_t)n * K);
  for (int c = lane; c < chunks; c += 64) out[c] = quantize8(row[c], s, 0u);
  if (lane == 0) sW[n] = b;
}

hipError_t launch_quantize_weight(const uint16_t* W, int N, int K, int8_t* Wq, float* sW,
                                  hipStream_t stream) {
  const int blocks = (N + 3) / 4;
  hipLaunchKernelGGL(kw_quantize_rows, dim3(blocks), dim3(256), 0, stream, W, N, K, Wq, sW);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Outlier column scan. Block (x, g) covers columns [64x, 64x+64) for the rows
// of row group g; 8 lanes span one 128-byte row segment, 64 rows per pass. The
// per-column maximum |x| code is kept with packed u16 max and compared with the
// threshold once at the end: |x| >= thr  <=>  code(|x|) >= hthr, where hthr is
// the smallest fp16 magnitude code whose value reaches thr (computed on the
// host), so the decision is the fp32 comparison, taken exactly.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 512;
constexpr int kScanUnroll = 8;

__global__ __launch_bounds__(kScanThreads) void ka_scan(const uint16_t* __restrict__ X, int T,
                                                        int K, uint32_t hthr,
                                                        uint32_t* __restrict__ parts, int KW) {
  __shared__ uint32_t words[2];
  const int tid = threadIdx.x;
  const int c = tid & 7;
  const int r = tid >> 3;
  const int col = blockIdx.x * 64 + c * 8;
  const int G = gridDim.y, g = blockIdx.y;
  const int rows_per = (T + G - 1) / G;
  const int t0 = g * rows_per;
  const int t1 = min(T, t0 + rows_per);
  if (tid < 2) words[tid] = 0u;
  v2u16 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  if (col < K) {
    const uint16_t* base = X + col;
    int t = t0 + r;
    for (; t + 64 * (kScanUnroll - 1) < t1; t += 64 * kScanUnroll) {
      uint4 v[kScanUnroll];
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u)
        v[u] = *reinterpret_cast<const uint4*>(base + (size_t)(t + 64 * u) * K);
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        v2u16 a[4];
        abs_codes(v[u], a);
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = __builtin_elementwise_max(m[i], a[i]);
      }
    }
    for (; t < t1; t += 64) {
      v2u16 a[4];
      abs_codes(*reinterpret_cast<const uint4*>(base + (size_t)t * K), a);
#pragma unroll
      for (int i = 0; i < 4; ++i) m[i] = __builtin_elementwise_max(m[i], a[i]);
    }
  }
  uint32_t bits = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bits |= (uint32_t)(m[i].x >= hthr) << (2 * i);
    bits |= (uint32_t)(m[i].y >= hthr) << (2 * i + 1);
  }
  __syncthreads();
  if (bits) atomicOr(&words[c >> 2], bits << ((c & 3) * 8));
  __syncthreads();
  if (tid < 2) {
    const int w = blockIdx.x * 2 + tid;
    if (w < KW) parts[(size_t)g * KW + w] = words[tid];
  }
}

int scan_row_groups(int T, int K, int num_cus) {
  const int slices = (K + 63) / 64;
  int g = (2 * num_cus + slices - 1) / slices;
  g = g < 1 ? 1 : (g > kScanMaxGroups ? kScanMaxGroups : g);
  const int max_by_rows = (T + 255) / 256;  // keep >= 256 rows per group
  if (g > max_by_rows) g = max_by_rows < 1 ? 1 : max_by_rows;
  return g;
}

uint32_t threshold_code(float thr) {
  // smallest fp16 magnitude code h (0..0x7c00) with value(h) >= thr; 0x7c00 (inf)
  // when no finite fp16 reaches thr. Codes are ordered like their values.
  auto value = [](uint32_t h) -> double {
    const uint32_t e = (h >> 10) & 31u, f = h & 1023u;
    if (e == 31) return INFINITY;
    if (e == 0) return std::ldexp((double)f, -24);
    return std::ldexp((double)(1024 + f), (int)e - 25);
  };
  uint32_t lo = 0, hi = 0x7c00;  // invariant: value(hi) >= thr (inf >= anything)
  if (value(lo) >= thr) return 0;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (value(mid) >= (double)thr) hi = mid; else lo = mid;
  }
  return hi;
}

hipError_t launch_scan(const LinearArgs& a, int groups, hipStream_t stream) {
  const int KW = (a.K + 31) / 32;
  dim3 grid((a.K + 63) / 64, groups);
  hipLaunchKernelGGL(ka_scan, grid, dim3(kScanThreads), 0, stream, a.X, a.T, a.K,
                     threshold_code(a.thr), a.parts, KW);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prepare: every block rebuilds the outlier bitmap (OR of the row-group parts)
// and its per-word prefix counts in LDS. Block 0 publishes bitmap, idx and
// count. Blocks [0, nq) then quantize rows of X (one wavefront per row) and
// gather the outlier activations; blocks [nq, nq+nw) gather and dequantize the
// outlier columns of the stored int8 weight.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 256;
constexpr int kMaxKW = kMaxK / 32;

__device__ __forceinline__ uint32_t chunk_skip_mask(const uint32_t* bm, int c) {
  return (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu;
}

__global__ __launch_bounds__(kPrepThreads) void ka_prepare(LinearArgs a, int groups, int nq) {
  __shared__ uint32_t bm[kMaxKW];
  __shared__ int pre[kMaxKW];
  __shared__ int wave_tot[kPrepThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, K = a.K, N = a.N;
  const int KW = (K + 31) >> 5;

  for (int w = tid; w < KW; w += kPrepThreads) {
    uint32_t v = 0u;
    for (int g = 0; g < groups; ++g) v |= a.parts[(size_t)g * KW + w];
    bm[w] = v;
  }
  __syncthreads();
  // exclusive prefix of per-word popcounts: contiguous word ranges per thread
  const int per = (KW + kPrepThreads - 1) / kPrepThreads;
  const int w0 = min(KW, tid * per), w1 = min(KW, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(bm[w]);
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kPrepThreads / 64; ++i) {
    base += (i < wave) ? wave_tot[i] : 0;
    total += wave_tot[i];
  }
  int run = base + incl - local;
  for (int w = w0; w < w1; ++w) {
    pre[w] = run;
    run += __popc(bm[w]);
  }
  __syncthreads();
  const int count = total;
  const int opad = (count + kOutChunk - 1) / kOutChunk * kOutChunk;

  if (blockIdx.x == 0) {
    for (int w = tid; w < KW; w += kPrepThreads) {
      a.bitmap[w] = bm[w];
      uint32_t bits = bm[w];
      int j = pre[w];
      while (bits) {
        const int b = __builtin_ctz(bits);
        a.idx[j++] = w * 32 + b;
        bits &= bits - 1u;
      }
    }
    if (tid == 0) a.count[0] = count;
  }

  if ((int)blockIdx.x < nq) {
    // ---- activations: one wavefront per row
    const int chunks = K >> 3;
    for (int t = blockIdx.x * 4 + wave; t < T; t += nq * 4) {
      const uint4* row = reinterpret_cast<const uint4*>(a.X + (size_t)t * K);
      int m = 0;
      for (int c = lane; c < chunks; c += 64) {
        const uint4 v = row[c];
        const uint32_t skip = chunk_skip_mask(bm, c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int code = (int)((w[i >> 1] >> ((i & 1) * 16)) & 0x7fffu);
          m = ((skip >> i) & 1u) ? m : max(m, code);
        }
      }
      m = wave_max_i(m);
      const float ax = half_bits_to_float((uint32_t)m);
      const float s = m > 0 ? 127.0f / ax : 0.0f;
      uint2* out = reinterpret_cast<uint2*>(a.Xq + (size_t)t * K);
      for (int c = lane; c < chunks; c += 64) out[c] = quantize8(row[c], s, chunk_skip_mask(bm, c));
      if (lane == 0) a.aX[t] = ax;
      if (count) {
        const uint16_t* xrow = a.X + (size_t)t * K;
        for (int w = lane; w < KW; w += 64) {
          uint32_t bits = bm[w];
          int j = pre[w];
          while (bits) {
            const int b = __builtin_ctz(bits);
            a.Xo[((size_t)(j / kOutChunk) * T + t) * kOutChunk + (j % kOutChunk)] = xrow[w * 32 + b];
            ++j;
            bits &= bits - 1u;
          }
        }
        for (int j = count + lane; j < opad; j += 64)
          a.Xo[((size_t)(j / kOutChunk) * T + t) * kOutChunk + (j % kOutChunk)] = 0;
      }
    }
  } else {
    // ---- outlier weight columns: Wd[n,j] = fp16(fl32(fl32(Wq[n,idx_j] * sW[n]) / 127))
    if (count == 0) return;
    const int nw = gridDim.x - nq;
    for (int n = (blockIdx.x - nq) * 4 + wave; n < N; n += nw * 4) {
      const float b = a.sW[n];
      const int8_t* wrow = a.Wq + (size_t)n * K;
      for (int w = lane; w < KW; w += 64) {
        uint32_t bits = bm[w];
        int j = pre[w];
        while (bits) {
          const int bb = __builtin_ctz(bits);
          const float q = (float)wrow[w * 32 + bb];
          a.Wd[((size_t)(j / kOutChunk) * N + n) * kOutChunk + (j % kOutChunk)] =
              float_to_half_bits((q * b) / 127.0f);
          ++j;
          bits &= bits - 1u;
        }
      }
      for (int j = count + lane; j < opad; j += 64)
        a.Wd[((size_t)(j / kOutChunk) * N + n) * kOutChunk + (j % kOutChunk)] = 0;
    }
  }
}

hipError_t launch_prepare(const LinearArgs& a, int groups, int num_cus, hipStream_t stream) {
  int nq = (a.T + 3) / 4;
  if (nq > 4 * num_cus) nq = 4 * num_cus;
  if (nq < 1) nq = 1;
  int nw = (a.N + 3) / 4;
  if (nw > 2 * num_cus) nw = 2 * num_cus;
  hipLaunchKernelGGL(ka_prepare, dim3(nq + nw), dim3(kPrepThreads), 0, stream, a, groups, nq);
  return hipGetLastError();
}

}  // namespace llmint8
