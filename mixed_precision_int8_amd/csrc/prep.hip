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
template <bool BF16>
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
  const float b = Act16<BF16>::to_f32((uint32_t)m);
  const float s = m > 0 ? 127.0f / b : 0.0f;
  uint2* out = reinterpret_cast<uint2*>(Wq + (size_t)n * K);
  for (int c = lane; c < chunks; c += 64) out[c] = Act16<BF16>::quantize8(row[c], s, ~0u, ~0u);
  if (lane == 0) sW[n] = b;
}

hipError_t launch_quantize_weight(const uint16_t* W, int N, int K, int8_t* Wq, float* sW, bool bf16,
                                  hipStream_t stream) {
  const int blocks = (N + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(kw_quantize_rows<true>, dim3(blocks), dim3(256), 0, stream, W, N, K, Wq, sW);
  else
    hipLaunchKernelGGL(kw_quantize_rows<false>, dim3(blocks), dim3(256), 0, stream, W, N, K, Wq, sW);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Outlier column scan. Block (x, g) covers columns [64x, 64x+64) for the rows
// of row group g; 8 lanes span one 128-byte row segment and 64 rows are read
// per load, kScanLoads loads in flight per thread. The per-column maximum |x|
// code is kept with packed u16 max and compared with the threshold once at
// the end: |x| >= thr  <=>  code(|x|) >= hthr, where hthr is the smallest
// 16-bit (fp16 or bf16) magnitude code whose value reaches thr (computed on
// the host), so the decision is the fp32 comparison, taken exactly.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 512;
constexpr int kScanLoads = 8;

__global__ __launch_bounds__(kScanThreads) void ka_scan(const uint16_t* __restrict__ X, int T,
                                                        int K, uint32_t hthr,
                                                        uint32_t* __restrict__ parts, int KW) {
  __shared__ uint32_t words[2];
  const int tid = threadIdx.x;
  const int c = tid & 7;
  const int r = tid >> 3;
  const int col = blockIdx.x * 64 + c * 8;
  const int G = gridDim.y, g = blockIdx.y;
  const int rows_per = scan_rows_per_group(T, G);
  const int t0 = g * rows_per;
  const int rows = min(T, t0 + rows_per) - t0;
  if (tid < 2) words[tid] = 0u;
  v2u16 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  if (col < K && rows > 0) {
    // one window per row group, at most scan_window_bytes (< 2^31), so that
    // kOobOffset lies past it
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(X + (size_t)t0 * K, (uint32_t)((size_t)rows * K * 2));
    for (int tb = r; tb < rows; tb += 64 * kScanLoads) {
      uint4 v[kScanLoads];
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) {  // rows past the group read as zero
        const int t = tb + 64 * u;
        const uint32_t off = t < rows ? (uint32_t)(((size_t)t * K + col) * 2) : kOobOffset;
        v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
      }
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) {
        v2u16 a[4];
        abs_codes(v[u], a);
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = __builtin_elementwise_max(m[i], a[i]);
      }
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

static_assert(64 * kScanLoads == kScanRowsPerStep, "rows per scan step");

uint32_t threshold_code(float thr, bool bf16) {
  // smallest 16-bit magnitude code h with value(h) >= thr; the infinity code
  // (0x7c00 fp16, 0x7f80 bf16) when no finite value reaches thr. Codes are
  // ordered like their values.
  auto value = [bf16](uint32_t h) -> double {
    if (bf16) {
      const uint32_t e = (h >> 7) & 255u, f = h & 127u;
      if (e == 255) return INFINITY;
      if (e == 0) return std::ldexp((double)f, -133);
      return std::ldexp((double)(128 + f), (int)e - 134);
    }
    const uint32_t e = (h >> 10) & 31u, f = h & 1023u;
    if (e == 31) return INFINITY;
    if (e == 0) return std::ldexp((double)f, -24);
    return std::ldexp((double)(1024 + f), (int)e - 25);
  };
  uint32_t lo = 0, hi = bf16 ? 0x7f80u : 0x7c00u;  // invariant: value(hi) >= thr (inf >= anything)
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
                     threshold_code(a.thr, a.bf16 != 0), a.parts, KW);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prepare. Every block ORs the row-group parts into the outlier bitmap in LDS.
//   gather blocks [0, ng) come first in the grid, so that their small bitmap
//     reads are issued ahead of the quantization blocks' loads of X on the
//     same CUs. They build the per-word prefix counts of the bitmap and the
//     ascending outlier indices in LDS, then one thread per (row, 8
//     consecutive outliers) fills the chunk-major outlier activations
//     Xo [KC][T][32] and the dequantized outlier weight columns Wd [KC][N][32]
//     (zero past |O|), all gathers in flight together. Gather block 0
//     publishes bitmap, idx and count.
//   quantization blocks [ng, ng + nq): one wavefront per row of X at a time;
//     a row is held in registers (CPL 16-byte chunks per lane, the row's
//     length rounded up to a template capacity), reduced to its absmax over
//     the kept columns, quantized and written as int8. Each wavefront takes
//     rows wave, wave + W, ... (W quantization wavefronts) with two register
//     buffers: the next row's loads are in flight while the current row is
//     reduced and its codes are stored, so stores and loads overlap when a
//     wavefront has several rows (up to 8192 columns per row); rows of up to
//     16384 columns have one buffer (CPL = 32, 128 registers). Rows longer
//     than the largest capacity (CPL = 0) are read twice from memory, which
//     keeps the kernel's registers low enough for all its blocks to stay
//     resident.
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 256;
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
constexpr int kMaxKW = kMaxK / 32;
constexpr int kIdxCap = 4096;  // outlier indices kept in LDS by the gather blocks

__device__ __forceinline__ uint32_t chunk_skip_mask(const uint32_t* bm, int c) {
  return (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu;
}

// masked absmax code of one 16-byte chunk (8 fp16 values, skipped ones excluded)
__device__ __forceinline__ uint32_t chunk_kept_max(const uint4& v, uint32_t skip) {
  const uint32_t m0 = expand4(~skip & 0xfu), m1 = expand4((~skip >> 4) & 0xfu);
  // byte masks -> 16-bit masks: element i kept iff byte i of m0/m1 is 0xff
  const uint32_t k0 = __builtin_amdgcn_perm(0u, m0, 0x01010000u), k1 = __builtin_amdgcn_perm(0u, m0, 0x03030202u);
  const uint32_t k2 = __builtin_amdgcn_perm(0u, m1, 0x01010000u), k3 = __builtin_amdgcn_perm(0u, m1, 0x03030202u);
  v2u16 mx = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(v2u16, v.x & 0x7fff7fffu & k0),
                                __builtin_bit_cast(v2u16, v.y & 0x7fff7fffu & k1)),
      __builtin_elementwise_max(__builtin_bit_cast(v2u16, v.z & 0x7fff7fffu & k2),
                                __builtin_bit_cast(v2u16, v.w & 0x7fff7fffu & k3)));
  return max((uint32_t)mx.x, (uint32_t)mx.y);
}

// One row of X held in registers: chunk lane + 64 u in v[u] (chunks past the row read as zero)
template <int CPL>
__device__ __forceinline__ void load_row_regs(const LinearArgs& a, int t, int lane, uint4 (&v)[CPL]) {
  const int K = a.K, cpl = ((K >> 3) + 63) >> 6;
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X + (size_t)t * K, (uint32_t)(K * 2));
#pragma unroll
  for (int u = 0; u < CPL; ++u)
    if (u < cpl) v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, (uint32_t)((lane + 64 * u) * 16), 0, 0));
}

// The outlier flags of a lane's chunks c = lane + 64 u, the same for every
// row: read from the bitmap once (all reads in flight together) and packed
// four chunks' 8-bit masks to a register. Read for every chunk from LDS, the
// masks had cost the 8-chunk kernel eight LDS round trips per row in
// sequence.
template <int CPL>
__device__ __forceinline__ void load_skip_masks(const uint32_t* bm, int lane, int KC,
                                                uint32_t (&sk)[(CPL + 3) / 4]) {
  uint32_t w[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) w[u] = lane + 64 * u < KC ? bm[(lane >> 2) + 16 * u] : 0u;
#pragma unroll
  for (int j = 0; j < (CPL + 3) / 4; ++j) {
    uint32_t x = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * j + i < CPL) x |= ((w[4 * j + i] >> ((lane & 3) * 8)) & 0xffu) << (8 * i);
    sk[j] = x;
  }
}
// the mask of chunk u: from the packed registers (8 chunks per lane), else
// from the bitmap in LDS (longer rows: registers for their masks would cost
// the rows' register buffers occupancy)
template <int CPL>
__device__ __forceinline__ uint32_t skip_of(const uint32_t (&sk)[(CPL + 3) / 4], const uint32_t* bm, int lane,
                                            int u) {
  if constexpr (CPL <= 8) return (sk[u >> 2] >> ((u & 3) * 8)) & 0xffu;
  else return chunk_skip_mask(bm, lane + 64 * u);
}

// absmax over the kept columns, quantization and the stores of row t (held in v)
template <bool BF16, int CPL>
__device__ __forceinline__ void quantize_row_regs(const LinearArgs& a, const uint32_t (&sk)[(CPL + 3) / 4],
                                                  const uint32_t* bm, int t, int lane, const uint4 (&v)[CPL]) {
  const int K = a.K, KC = K >> 3, cpl = (KC + 63) >> 6;
  // past 8 chunks the masks come from LDS, four chunks' words per round trip
  constexpr int GM = CPL <= 8 ? 1 : 4;
  auto masks = [&](int u0, uint32_t (&mk)[GM]) {
    if constexpr (CPL <= 8) {
      mk[0] = skip_of<CPL>(sk, bm, lane, u0);
    } else {
      uint32_t w[GM];
#pragma unroll
      for (int i = 0; i < GM; ++i) w[i] = lane + 64 * (u0 + i) < KC ? bm[(lane >> 2) + 16 * (u0 + i)] : 0u;
#pragma unroll
      for (int i = 0; i < GM; ++i) mk[i] = (w[i] >> ((lane & 3) * 8)) & 0xffu;
    }
  };
  uint32_t m = 0u;
#pragma unroll
  for (int u0 = 0; u0 < CPL; u0 += GM) {
    uint32_t mk[GM];
    masks(u0, mk);
#pragma unroll
    for (int i = 0; i < GM; ++i) {
      const int u = u0 + i, c = lane + 64 * u;
      if (u < cpl && c < KC) m = max(m, chunk_kept_max(v[u], mk[i]));
    }
  }
  m = wave_max_u16x2(m) & 0xffffu;
  const float ax = Act16<BF16>::to_f32(m);
  const float s = m ? 127.0f / ax : 0.0f;
  uint2* out = reinterpret_cast<uint2*>(a.Xq + (size_t)t * K);
  // Codes of 8 chunks into 8 register pairs, then their 8 stores: a store's
  // data registers are not written again while it is in flight, so no chunk
  // waits for the previous chunk's store to complete (with one register pair
  // reused per chunk the compiler waited for every store).
  constexpr int G = CPL < 8 ? CPL : 8;
#pragma unroll
  for (int u0 = 0; u0 < CPL; u0 += G) {
    uint2 q[G];
#pragma unroll
    for (int i0 = 0; i0 < G; i0 += GM) {
      uint32_t mk[GM];
      masks(u0 + i0, mk);
#pragma unroll
      for (int i = i0; i < i0 + GM; ++i) {
        const int u = u0 + i, c = lane + 64 * u;
        if (u < cpl && c < KC) {
          const uint32_t skip = mk[i - i0];
          q[i] = Act16<BF16>::quantize8(v[u], s, expand4(~skip & 0xfu), expand4((~skip >> 4) & 0xfu));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int u = u0 + i, c = lane + 64 * u;
      // non-temporal: the codes are not read again by this kernel (ka_prepare
      // 12.0 -> 11.4 us at the 2048 x 4096 prefill input; the whole call about
      // 0.5 us faster, the GEMM that reads them next a little slower)
      if (u < cpl && c < KC) __builtin_nontemporal_store(v2u32{q[i].x, q[i].y}, reinterpret_cast<v2u32*>(out) + c);
    }
  }
  if (lane == 0) a.aX[t] = ax;
}

// rows longer than any register capacity: read twice (maximum, then codes)
template <bool BF16>
__device__ __forceinline__ void quantize_row_mem(const LinearArgs& a, const uint32_t* bm, int t, int lane) {
  const int K = a.K, KC = K >> 3;
  const uint4* row = reinterpret_cast<const uint4*>(a.X + (size_t)t * K);
  uint2* out = reinterpret_cast<uint2*>(a.Xq + (size_t)t * K);
  uint32_t m = 0u;
  for (int c = lane; c < KC; c += 64) m = max(m, chunk_kept_max(row[c], chunk_skip_mask(bm, c)));
  m = wave_max_u16x2(m) & 0xffffu;
  const float ax = Act16<BF16>::to_f32(m);
  const float s = m ? 127.0f / ax : 0.0f;
  for (int c = lane; c < KC; c += 64) {
    const uint32_t skip = chunk_skip_mask(bm, c);
    out[c] = Act16<BF16>::quantize8(row[c], s, expand4(~skip & 0xfu), expand4((~skip >> 4) & 0xfu));
  }
  if (lane == 0) a.aX[t] = ax;
}

// ONE: a single register buffer, for rows of 32 chunks per lane (two would not
// fit) and, with 16 chunks, for grids where every wavefront has at most one row
// (the second buffer would never be used, and without it more workgroups stay
// resident)
template <bool BF16, int CPL, bool ONE>
__global__ __launch_bounds__(kPrepThreads) void ka_prepare(LinearArgs a, int groups, int nq) {
  __shared__ uint32_t bm[kMaxKW];
  __shared__ int pre[kMaxKW];
  __shared__ int wave_tot[kPrepThreads / 64];
  __shared__ uint16_t idx_s[kIdxCap];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, K = a.K, N = a.N;
  const int KW = (K + 31) >> 5;
  const int ng = gridDim.x - nq;  // gather blocks come first: their bitmap reads then
  const bool quant = (int)blockIdx.x >= ng;  // queue ahead of the quantization blocks' X loads

  // quantization blocks start their first row's loads before anything else
  const int row0 = (blockIdx.x - ng) * 4 + wave;
  const int W = nq * 4;  // quantization wavefronts
  constexpr int CB = CPL > 0 ? CPL : 1;
  uint4 v0[CB], v1[ONE ? 1 : CB];
  if (CPL > 0 && quant && row0 < T) load_row_regs<CB>(a, row0, lane, v0);
  // the row groups' partial bitmaps, all loads in flight before the first OR
  for (int w = tid; w < KW; w += kPrepThreads) {
    uint32_t p[kScanMaxGroups];
#pragma unroll
    for (int g = 0; g < kScanMaxGroups; ++g) p[g] = g < groups ? a.parts[(size_t)g * KW + w] : 0u;
    uint32_t x = 0u;
#pragma unroll
    for (int g = 0; g < kScanMaxGroups; ++g) x |= p[g];
    bm[w] = x;
  }
  __syncthreads();

  if (quant) {
    uint32_t sk[(CB + 3) / 4];
    if constexpr (CPL > 0 && CPL <= 8) load_skip_masks<CB>(bm, lane, K >> 3, sk);
    // ---- activations: rows row0, row0 + W, ...; two register buffers alternate
    if constexpr (CPL > 0 && ONE) {
      // one register buffer: any next row's loads follow the current row's stores
      for (int t = row0; t < T; t += W) {
        if (t != row0) load_row_regs<CB>(a, t, lane, v0);
        quantize_row_regs<BF16, CB>(a, sk, bm, t, lane, v0);
      }
    } else if constexpr (CPL > 0) {
      for (int t = row0; t < T; t += 2 * W) {
        const int t1 = t + W;
        if (t1 < T) load_row_regs<CB>(a, t1, lane, v1);
        quantize_row_regs<BF16, CB>(a, sk, bm, t, lane, v0);
        if (t1 >= T) break;
        if (t1 + W < T) load_row_regs<CB>(a, t1 + W, lane, v0);
        quantize_row_regs<BF16, CB>(a, sk, bm, t1, lane, v1);
      }
    } else {
      for (int t = row0; t < T; t += W) quantize_row_mem<BF16>(a, bm, t, lane);
    }
    return;
  }

  // ---- gather blocks: exclusive prefix of per-word popcounts
  const int per = (KW + kPrepThreads - 1) / kPrepThreads;
  const int w0 = min(KW, tid * per), w1 = min(KW, w0 + per);
  int local = 0;
  for (int w = w0; w < w1; ++w) local += __popc(bm[w]);
  const int incl = wave_incl_sum(local);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, count = 0;
#pragma unroll
  for (int i = 0; i < kPrepThreads / 64; ++i) {
    base += (i < wave) ? wave_tot[i] : 0;
    count += wave_tot[i];
  }
  int run = base + incl - local;
  for (int w = w0; w < w1; ++w) {
    pre[w] = run;
    uint32_t bits = bm[w];
    while (bits) {  // ascending outlier columns, as far as the LDS table reaches
      if (run < kIdxCap) idx_s[run] = (uint16_t)(w * 32 + __builtin_ctz(bits));
      ++run;
      bits &= bits - 1u;
    }
  }
  __syncthreads();
  const int gb = blockIdx.x;
  if (gb == 0) {
    for (int w = tid; w < KW; w += kPrepThreads) {
      a.bitmap[w] = bm[w];
      uint32_t bits = bm[w];
      int j = pre[w];
      while (bits) {
        a.idx[j++] = w * 32 + __builtin_ctz(bits);
        bits &= bits - 1u;
      }
    }
    if (tid == 0) a.count[0] = count;
  }
  if (count == 0) return;

  // one item = (row of Xo or Wd, group of 8 consecutive outliers), for the
  // chunks the workspace holds (the GEMM epilogue forms any later chunk itself)
  const int ngrp = min((count + kOutChunk - 1) / kOutChunk, a.wchunks) * (kOutChunk / 8);
  const int items = (T + N) * ngrp;  // < 2^31: T, N < 2^31 / K and ngrp <= K / 8
  for (int it = gb * kPrepThreads + tid; it < items; it += ng * kPrepThreads) {
    const int row = it / ngrp;
    const int jg = it - row * ngrp;
    const int j0 = jg * 8;
    if (j0 >= count) {  // a group wholly past |O| (chunk padding): zeros, no loads
      const size_t dst = row < T ? ((size_t)(j0 / kOutChunk) * T + row) * kOutChunk + (j0 % kOutChunk)
                                 : ((size_t)(j0 / kOutChunk) * N + (row - T)) * kOutChunk + (j0 % kOutChunk);
      *reinterpret_cast<uint4*>((row < T ? a.Xo : a.Wd) + dst) = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    // column of each outlier j0 .. j0+7 (index 0 past |O|, masked later):
    // from the LDS table, or beyond it by a binary search for the word holding
    // it (last word with pre[w] <= j), all 8 searches advancing together,
    // then the (j - pre[w])-th set bit of that word
    int h[8];
    const int nvalid = min(8, max(0, count - j0));
    if (j0 + 8 <= kIdxCap) {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = idx_s[min(j0 + e, count - 1)];
    } else {
      int lo[8], hi[8], jj[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        jj[e] = min(j0 + e, count - 1);
        lo[e] = 0;
        hi[e] = KW - 1;
      }
      for (int span = KW; span > 1; span = (span + 1) >> 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int mid = (lo[e] + hi[e] + 1) >> 1;
          if (lo[e] < hi[e]) {
            if (pre[mid] <= jj[e]) lo[e] = mid; else hi[e] = mid - 1;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t bits = bm[lo[e]];
        for (int r = jj[e] - pre[lo[e]]; r > 0; --r) bits &= bits - 1u;
        h[e] = lo[e] * 32 + __builtin_ctz(bits);
      }
    }
    // all 8 gathers are issued unconditionally (index 0 past |O|, masked
    // afterwards) so that they are in flight together
    uint16_t val[8];
    if (row < T) {
      const uint16_t* xr = a.X + (size_t)row * K;
      uint16_t g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = xr[h[e]];
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = e < nvalid ? g[e] : (uint16_t)0;
      const size_t dst = ((size_t)(j0 / kOutChunk) * T + row) * kOutChunk + (j0 % kOutChunk);
      *reinterpret_cast<uint4*>(a.Xo + dst) = make_uint4(val[0] | ((uint32_t)val[1] << 16), val[2] | ((uint32_t)val[3] << 16),
                                                           val[4] | ((uint32_t)val[5] << 16), val[6] | ((uint32_t)val[7] << 16));
    } else {
      // Wd[n,j] = r16(fl32(fl32(Wq[n,idx_j] * sW[n]) / 127)), r16 the activation type's rounding
      const int n = row - T;
      const float b = a.sW[n];
      const int8_t* wr = a.Wq + (size_t)n * K;
      int8_t g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = wr[h[e]];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        val[e] = e < nvalid ? Act16<BF16>::from_f32(((float)g[e] * b) / 127.0f) : (uint16_t)0;
      const size_t dst = ((size_t)(j0 / kOutChunk) * N + n) * kOutChunk + (j0 % kOutChunk);
      *reinterpret_cast<uint4*>(a.Wd + dst) = make_uint4(val[0] | ((uint32_t)val[1] << 16), val[2] | ((uint32_t)val[3] << 16),
                                                           val[4] | ((uint32_t)val[5] << 16), val[6] | ((uint32_t)val[7] << 16));
    }
  }
}

template <bool BF16>
static hipError_t launch_prepare_dt(const LinearArgs& a, int groups, dim3 grid, int nq, hipStream_t stream) {
  const int cpl = ((a.K >> 3) + 63) >> 6;  // 16-byte chunks per lane of one row
  // every quantization wavefront has at most one row: the 16-chunk kernel then
  // takes one buffer (127 registers, not 224: twice the resident workgroups;
  // 39.3 -> 36.4 us at the 4096 x 8192 input). The 8-chunk kernel keeps two
  // (119 registers; with one, 78, the 2048 x 4096 prefill call measured slower).
  const bool one = a.T <= 4 * nq;
#define PREP(C, O) hipLaunchKernelGGL((ka_prepare<BF16, C, O>), grid, dim3(kPrepThreads), 0, stream, a, groups, nq)
  if (cpl <= 8) {
    PREP(8, false);
  } else if (cpl <= 16) {
    if (one) PREP(16, true); else PREP(16, false);
  } else if (cpl <= 32) {
    PREP(32, true);
  } else {
    PREP(0, false);
  }
#undef PREP
  return hipGetLastError();
}

hipError_t launch_prepare(const LinearArgs& a, int groups, int num_cus, hipStream_t stream) {
  // quantization wavefronts: one row each (every row's loads in flight at
  // once), at most 16 per CU
  int nq = (int)ceil_div(a.T, 4);
  if (nq > 4 * num_cus) nq = 4 * num_cus;
  if (nq < 1) nq = 1;
  // gather work for up to 32 outliers; more are covered by the grid-stride loop
  int ng = (int)ceil_div((int64_t)(a.T + a.N) * (kOutChunk / 8), kPrepThreads);
  if (ng > 2 * num_cus) ng = 2 * num_cus;
  if (ng < 1) ng = 1;
  const dim3 grid(nq + ng);
  return a.bf16 ? launch_prepare_dt<true>(a, groups, grid, nq, stream)
                : launch_prepare_dt<false>(a, groups, grid, nq, stream);
}

}  // namespace llmint8
