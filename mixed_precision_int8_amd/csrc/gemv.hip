// Fused decode-shaped forward (T <= 16 rows) of the LLM.int8() layer on gfx950.
//
// One kernel does every step for a small batch of rows: outlier column scan,
// row absmax over the non-outlier columns, int8 quantization of X into LDS,
// the int8 product, the dequantization and the 16-bit outlier product
// ("Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
// Explained", sections 2 and 3; "bitsandbytes: GPU-Accelerated Inference and
// Training at Lower Bit Depths", "How LLM.int8() quantizes weights and
// activations").
//
// At T <= 16 the call is bound by streaming the int8 weight from HBM, so the
// kernel is built around that stream. A 256-thread block owns 16 output rows;
// its 4 wavefronts split K and each issues its first 16 x 16-byte weight loads
// into registers before anything else, so the HBM traffic is in flight while
// the block scans and quantizes the (small, L2-resident) X. The int8 dot
// products run on v_mfma_i32_16x16x64_i8 with the 16 weight rows as the A
// operand and the (zero-padded) quantized rows of X, read from LDS, as B.
// Partial int32 sums of the 4 wavefronts are added exactly through LDS; the
// outlier columns go through v_mfma_f32_16x16x32_f16 on top of the
// dequantized int8 part.
#include "device_util.h"
#include "internal.h"

namespace llmint8 {

constexpr int kGemvRowsN = 16;
constexpr int kGemvBatch = 16;  // k-steps (64 bytes each) held in registers per batch
constexpr int kLdsLimit = 160 * 1024;

struct GemvLds {
  int xq, bm, idx, red, arow, total, kp;
};

__host__ __device__ inline GemvLds gemv_lds(int T, int K) {
  GemvLds L;
  const int KW = (K + 31) / 32;
  L.kp = K + 16;  // row pitch of the quantized rows: shifts banks between rows
  int off = 0;
  L.xq = off;
  off += (T * L.kp + 15) / 16 * 16;
  L.bm = off;
  off += (KW * 4 + 15) / 16 * 16;
  L.idx = off;
  off += (K * 2 + 15) / 16 * 16;
  L.red = off;
  off += 3 * 64 * 16;
  L.arow = off;
  off += 16 * 4;
  L.total = off;
  return L;
}

int gemv_max_rows(int K) {
  if (K <= 0) return 0;
  for (int t = kGemvRowsN; t >= 1; --t)
    if (gemv_lds(t, K).total <= kLdsLimit - 256) return t;
  return 0;
}

__global__ __launch_bounds__(256, 1) void kd_gemv(LinearArgs a, uint32_t hthr, int kq) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int T = a.T, K = a.K, N = a.N;
  const GemvLds L = gemv_lds(T, K);
  int8_t* xq = reinterpret_cast<int8_t*>(lds + L.xq);
  uint32_t* bm = reinterpret_cast<uint32_t*>(lds + L.bm);
  uint16_t* idxl = reinterpret_cast<uint16_t*>(lds + L.idx);
  v4i* red = reinterpret_cast<v4i*>(lds + L.red);
  float* arow = reinterpret_cast<float*>(lds + L.arow);
  __shared__ int wave_tot[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fi = lane & 15, fg = lane >> 4;
  const int KW = (K + 31) >> 5;
  const int n0 = blockIdx.x * kGemvRowsN;
  const int rows_n = min(kGemvRowsN, N - n0);

  // ---- 1. start streaming this wavefront's share of the 16 weight rows
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.Wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const int kbeg = wave * kq;
  const int kend = min(K, kbeg + kq);
  const int steps = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  const int nbatch = (steps + kGemvBatch - 1) / kGemvBatch;
  const uint32_t rowoff = (uint32_t)(fi * K);
  auto load_batch = [&](v4i* w, int b) {
#pragma unroll
    for (int s = 0; s < kGemvBatch; ++s) {
      const int k = kbeg + (b * kGemvBatch + s) * 64 + fg * 16;
      const uint32_t off = k < kend ? rowoff + (uint32_t)k : kOobOffset;
      w[s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
    }
  };
  v4i w0[kGemvBatch], w1[kGemvBatch];
  if (nbatch > 0) load_batch(w0, 0);

  // ---- 2. outlier columns of X (all T rows), into an LDS bitmap
  for (int w = tid; w < KW; w += 256) bm[w] = 0u;
  __syncthreads();
  for (int c = tid; c < (K >> 3); c += 256) {
    v2u16 m[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    for (int t = 0; t < T; ++t) {
      v2u16 ab[4];
      abs_codes(*reinterpret_cast<const uint4*>(a.X + (size_t)t * K + c * 8), ab);
#pragma unroll
      for (int i = 0; i < 4; ++i) m[i] = __builtin_elementwise_max(m[i], ab[i]);
    }
    uint32_t bits = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bits |= (uint32_t)(m[i].x >= hthr) << (2 * i);
      bits |= (uint32_t)(m[i].y >= hthr) << (2 * i + 1);
    }
    if (bits) atomicOr(&bm[c >> 2], bits << ((c & 3) * 8));
  }
  __syncthreads();

  // ---- 3. ascending outlier list (prefix counts over bitmap words)
  const int per = (KW + 255) / 256;
  const int w0i = min(KW, tid * per), w1i = min(KW, w0i + per);
  int local = 0;
  for (int w = w0i; w < w1i; ++w) local += __popc(bm[w]);
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, count = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    base += (i < wave) ? wave_tot[i] : 0;
    count += wave_tot[i];
  }
  {
    int j = base + incl - local;
    for (int w = w0i; w < w1i; ++w) {
      uint32_t bits = bm[w];
      while (bits) {
        const int bb = __builtin_ctz(bits);
        idxl[j] = (uint16_t)(w * 32 + bb);
        if (blockIdx.x == 0 && a.dbg_idx) a.dbg_idx[j] = w * 32 + bb;
        ++j;
        bits &= bits - 1u;
      }
      if (blockIdx.x == 0 && a.dbg_bitmap) a.dbg_bitmap[w] = bm[w];
    }
  }
  if (blockIdx.x == 0 && tid == 0 && a.dbg_count) a.dbg_count[0] = count;

  // ---- 4. row statistic and int8 rows of X into LDS (one wavefront per row)
  for (int t = wave; t < T; t += 4) {
    const uint4* row = reinterpret_cast<const uint4*>(a.X + (size_t)t * K);
    int m = 0;
    for (int c = lane; c < (K >> 3); c += 64) {
      const uint4 v = row[c];
      const uint32_t skip = (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu;
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int code = (int)((wv[i >> 1] >> ((i & 1) * 16)) & 0x7fffu);
        m = ((skip >> i) & 1u) ? m : max(m, code);
      }
    }
    m = wave_max_i(m);
    const float ax = half_bits_to_float((uint32_t)m);
    const float s = m > 0 ? 127.0f / ax : 0.0f;
    for (int c = lane; c < (K >> 3); c += 64) {
      const uint2 q = quantize8(row[c], s, (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu);
      *reinterpret_cast<uint2*>(xq + t * L.kp + c * 8) = q;
      if (blockIdx.x == 0 && a.dbg_Xq) *reinterpret_cast<uint2*>(a.dbg_Xq + (size_t)t * K + c * 8) = q;
    }
    if (lane == 0) {
      arow[t] = ax;
      if (blockIdx.x == 0 && a.dbg_aX) a.dbg_aX[t] = ax;
    }
  }
  __syncthreads();

  // ---- 5. int8 product of this wavefront's K range
  v4i acc = {0, 0, 0, 0};
  const bool trow = fi < T;
  const int8_t* xrow = xq + fi * L.kp;
  auto compute_batch = [&](const v4i* w, int b) {
#pragma unroll
    for (int s = 0; s < kGemvBatch; ++s) {
      const int k = kbeg + (b * kGemvBatch + s) * 64 + fg * 16;
      v4i xf = {0, 0, 0, 0};
      if (trow && k < kend) xf = *reinterpret_cast<const v4i*>(xrow + k);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[s], xf, acc, 0, 0, 0);
    }
  };
  for (int b = 0; b < nbatch; b += 2) {
    if (b + 1 < nbatch) load_batch(w1, b + 1);
    compute_batch(w0, b);
    if (b + 1 < nbatch) {
      if (b + 2 < nbatch) load_batch(w0, b + 2);
      compute_batch(w1, b + 1);
    }
  }

  // ---- 6. exact sum of the 4 partial products
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += red[w * 64 + lane];

  // ---- 7. dequantize, outlier product, fp16 store. Lane holds rows (n)
  // n0 + 4*fg + v of column (t) fi.
  const int n = n0 + 4 * fg;
  const int t = fi;
  if (a.dbg_C && t < T) {
    for (int v = 0; v < 4; ++v)
      if (n + v < N) a.dbg_C[(size_t)t * N + n + v] = acc[v];
  }
  const float at = t < T ? arow[t] : 0.0f;
  v4f y;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float b = n + v < N ? a.sW[n + v] * (1.0f / 16129.0f) : 0.0f;
    y[v] = (float)acc[v] * (at * b);
  }
  if (count) {
    const int nr = n0 + fi;  // weight row of this lane in the A operand
    const bool nok = nr < N;
    const float br = nok ? a.sW[nr] : 0.0f;
    const int8_t* wrow = a.Wq + (size_t)min(nr, N - 1) * K;
    const uint16_t* xr = a.X + (size_t)min(t, T - 1) * K;
    for (int c = 0; c < count; c += kOutChunk) {
      v8h wf, xf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = c + fg * 8 + e;
        const bool ok = j < count;
        const int h = ok ? (int)idxl[j] : 0;
        const float q = (float)wrow[h];
        wf[e] = (ok && nok) ? (_Float16)((q * br) / 127.0f) : (_Float16)0.0f;
        xf[e] = (ok && t < T) ? __builtin_bit_cast(_Float16, xr[h]) : (_Float16)0.0f;
      }
      y = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, xf, y, 0, 0, 0);
    }
  }
  if (t < T) {
    uint16_t* dst = a.Y + (size_t)t * N + n;
    if ((N & 3) == 0 && n + 3 < N) {
      uint2 p;
      p.x = (uint32_t)float_to_half_bits(y[0]) | ((uint32_t)float_to_half_bits(y[1]) << 16);
      p.y = (uint32_t)float_to_half_bits(y[2]) | ((uint32_t)float_to_half_bits(y[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = p;
    } else {
      for (int v = 0; v < 4; ++v)
        if (n + v < N) dst[v] = float_to_half_bits(y[v]);
    }
  }
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream) {
  const GemvLds L = gemv_lds(a.T, a.K);
  if (L.total > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kd_gemv),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             kLdsLimit - 256);
    if (e != hipSuccess) return e;
  }
  const int kq = (int)(ceil_div(ceil_div(a.K, 4), 64) * 64);
  const int blocks = (int)ceil_div(a.N, kGemvRowsN);
  hipLaunchKernelGGL(kd_gemv, dim3(blocks), dim3(256), L.total, stream, a, threshold_code(a.thr), kq);
  return hipGetLastError();
}

}  // namespace llmint8
