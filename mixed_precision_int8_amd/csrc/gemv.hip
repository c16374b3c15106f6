// Fused decode-shaped forward (T <= 16 rows) of the LLM.int8() layer on gfx950.
//
// One kernel does every step for a small batch of rows: outlier column scan,
// row absmax over the non-outlier columns, int8 quantization of X, the int8
// product, the dequantization and the 16-bit outlier product ("Hugging Face
// Quantization with bitsandbytes: 4-bit & 8-bit Models Explained", sections 2
// and 3; "bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit
// Depths", "How LLM.int8() quantizes weights and activations").
//
// At T <= 16 the call streams the int8 weight from HBM once; what it adds on
// top is the latency of the X-dependent steps, which a wavefront executes at
// about one instruction per 4 cycles. A 512-thread block owns 16 output rows
// and splits into two roles:
//   * 4 stream wavefronts issue the block's weight loads into registers at
//     once (16 x 16-byte loads per lane). Issuing that much stalls the issuing
//     wavefront for about a microsecond, which is about when X has landed.
//   * 4 X wavefronts copy X into LDS (buffer_load ... lds) meanwhile.
//   * Then all 8 wavefronts work on X: a thread owns 8-column chunks across
//     all T rows, decides their outlier flags on its own (column absmax >=
//     threshold), takes the rows' maxima over its kept columns in the same
//     pass (packed u16 arithmetic on 16-bit magnitude codes), and after one block-wide
//     reduction quantizes its chunks into LDS.
//   * The stream wavefronts then multiply their quarter of K on
//     v_mfma_i32_16x16x64_i8 (16 weight rows as A, int8 rows of X as B) and
//     leave int32 partial sums in LDS. Meanwhile X wavefront 0, which has
//     compacted the outlier indices and gathered the weight bytes of the
//     first 32 outlier columns, computes the 16-bit outlier product on
//     v_mfma_f32_16x16x32_f16; it finally sums the partials, dequantizes and
//     stores Y in the activation type (fp16 or bf16).
// The kernel is instantiated per row capacity TB (1, 2, 4, 8, 16 >= T) so
// that per-row loops are resolved at compile time.
#include <atomic>

#include "device_util.h"
#include "internal.h"

namespace llmint8 {

constexpr int kGemvRowsN = 16;
constexpr int kGemvBatch = 16;  // k-steps (64 bytes each) held in registers per batch
constexpr int kLdsLimit = 160 * 1024 - 1024;  // dynamic LDS; leaves room for the static part

struct GemvLds {
  int xs, xq, bm, idx, red, arow, rowred, cnt, total, kp;
};

__host__ __device__ inline GemvLds gemv_lds(int T, int K) {
  GemvLds L;
  const int KW = (K + 31) / 32;
  auto al = [](int v, int a) { return (v + a - 1) / a * a; };
  L.kp = K + 16;  // row pitch of the int8 rows: shifts banks between rows
  int off = 0;
  L.xs = off;  // X (fp16 or bf16), copied in 1 KB pieces
  off += al(T * K * 2, 1024);
  L.xq = off;
  off += al(T * L.kp, 16);
  L.bm = off;
  off += al(KW * 4, 16);
  L.idx = off;  // + 64 bytes: groups of 8 indices are read past the count
  off += al(K * 2 + 64, 16);
  L.red = off;  // partial products of the 4 stream wavefronts
  off += 4 * 64 * 16;
  L.arow = off;
  off += kGemvRowsN * 4;
  L.rowred = off;  // [8 wavefronts][8 row pairs] packed u16 maxima
  off += 8 * 8 * 4;
  L.cnt = off;
  off += 16;
  L.total = off;
  return L;
}

int gemv_max_rows(int K) {
  if (K <= 0) return 0;
  for (int t = kGemvRowsN; t >= 1; --t)
    if (gemv_lds(t, K).total <= kLdsLimit) return t;
  return 0;
}

__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wavefront's LDS
// operations (lgkmcnt) but not for its outstanding global loads, so the weight
// stream stays in flight across the prologue's barriers.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// The aligned dword holding weight byte `off`: a 32-bit load result needs no
// conversion, so it stays untouched in its register (and nothing waits for
// it) until the byte is extracted where it is used.
__device__ __forceinline__ uint32_t load_word_of(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off & ~3u, 0, 0);
}
__device__ __forceinline__ int byte_of(uint32_t word, int h) {
  return (int)(int8_t)(uint8_t)(word >> ((h & 3) * 8));
}

__device__ __forceinline__ v2u16 pk_max(v2u16 a, v2u16 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ v2u16 as_u16x2(uint32_t x) { return __builtin_bit_cast(v2u16, x); }
__device__ __forceinline__ uint32_t as_u32(v2u16 x) { return __builtin_bit_cast(uint32_t, x); }

template <int TB, bool BF16>
__global__ __launch_bounds__(512, 1) void kd_gemv(LinearArgs a, uint32_t hthr, int kq) {
  using A16 = Act16<BF16>;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int T = a.T, K = a.K, N = a.N;
  const GemvLds L = gemv_lds(T, K);
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(lds + L.xs);
  int8_t* xq = reinterpret_cast<int8_t*>(lds + L.xq);
  uint32_t* bm = reinterpret_cast<uint32_t*>(lds + L.bm);
  uint16_t* idxl = reinterpret_cast<uint16_t*>(lds + L.idx);
  v4i* red = reinterpret_cast<v4i*>(lds + L.red);
  float* arow = reinterpret_cast<float*>(lds + L.arow);
  uint32_t* rowred = reinterpret_cast<uint32_t*>(lds + L.rowred);
  int* cnt = reinterpret_cast<int*>(lds + L.cnt);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool xwave = wave < 4;  // wavefronts 0-3: X; 4-7: weight stream
  const int xt = tid & 255;     // thread index within its group of 4 wavefronts
  const int fi = lane & 15, fg = lane >> 4;
  const int KW = (K + 31) >> 5;
  const int KC = K >> 3;  // 16-byte chunks per row of X
  const int n0 = blockIdx.x * kGemvRowsN;
  const int rows_n = min(kGemvRowsN, N - n0);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.Wq + (size_t)n0 * K, (uint32_t)(rows_n * K));
  const uint32_t rowoff = (uint32_t)(fi * K);
  constexpr int NP = (TB + 1) / 2;  // row pairs packed as u16x2

  // stream wavefronts: their K range and the first batch of weight loads
  const int ww = wave & 3;
  const int kbeg = ww * kq;
  const int kend = min(K, kbeg + kq);
  const int steps = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  const int nbatch = (steps + kGemvBatch - 1) / kGemvBatch;
  auto load_batch = [&](v4i* w, int b) {
#pragma unroll
    for (int s = 0; s < kGemvBatch; ++s) {
      const int k = kbeg + (b * kGemvBatch + s) * 64 + fg * 16;
      const uint32_t off = k < kend ? rowoff + (uint32_t)k : kOobOffset;
      w[s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
    }
  };
  v4i w0[kGemvBatch], w1[kGemvBatch];
  float bs4[4] = {0.f, 0.f, 0.f, 0.f}, brow = 0.f;
  uint16_t bias4[4] = {0, 0, 0, 0};
  if (xwave) {
    // ---- 1. X -> LDS (1 KB per wavefront issue); wavefront 0 also fetches
    // the scales of the 16 weight rows (rows past N read as zero)
    const int xbytes = T * K * 2;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X, (uint32_t)xbytes);
    for (int blk = wave; blk * 1024 < xbytes; blk += 4)
      lds_copy16(rX, lds + L.xs + blk * 1024, (uint32_t)(blk * 1024 + lane * 16));
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t rS = make_rsrc(a.sW + n0, (uint32_t)(rows_n * 4));
      brow = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, (uint32_t)(fi * 4), 0, 0));
#pragma unroll
      for (int v = 0; v < 4; ++v)
        bs4[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, (uint32_t)((4 * fg + v) * 4), 0, 0));
      if (a.bias) {  // the bias of this lane's 4 output rows, for the epilogue
        const __amdgpu_buffer_rsrc_t rBias = make_rsrc(a.bias + n0, (uint32_t)(rows_n * 2));
#pragma unroll
        for (int v = 0; v < 4; ++v)
          bias4[v] = __builtin_amdgcn_raw_buffer_load_b16(rBias, (uint32_t)((4 * fg + v) * 2), 0, 0);
      }
    }
    for (int w = xt; w < KW; w += 256) bm[w] = 0u;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's part of X has landed
  } else {
    // ---- 2. the weight stream: 16 x 16-byte loads per lane, in flight while
    // the X wavefronts work (issuing them stalls only these wavefronts)
    load_batch(w0, 0);  // out-of-range steps read as zero
  }
  lds_barrier();  // A: X is in LDS, the bitmap is clear

  uint32_t g[8];
  {
    // ---- 3. all 8 wavefronts (the stream wavefronts have issued their loads
    // by now): a thread takes 8-column chunks across all rows: column absmax
    // -> outlier flags -> keep masks -> row maxima over the kept columns. All
    // values are 16-bit codes with the sign cleared, compared as packed u16.
    const v2u16 hthr2 = {(uint16_t)hthr, (uint16_t)hthr};
    v2u16 rmax[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) rmax[t] = v2u16{0, 0};
    for (int c = tid; c < KC; c += 512) {
      v2u16 ab[TB][4];
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const uint4 v = t < T ? *reinterpret_cast<const uint4*>(xs + t * K + c * 8) : uint4{0, 0, 0, 0};
        ab[t][0] = as_u16x2(v.x & 0x7fff7fffu);
        ab[t][1] = as_u16x2(v.y & 0x7fff7fffu);
        ab[t][2] = as_u16x2(v.z & 0x7fff7fffu);
        ab[t][3] = as_u16x2(v.w & 0x7fff7fffu);
      }
      uint32_t keep[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v2u16 cm = ab[0][i];
#pragma unroll
        for (int t = 1; t < TB; ++t) cm = pk_max(cm, ab[t][i]);
        // cm - thr is negative (sign bit set) exactly where the column is kept
        const v2u16 d = cm - hthr2;
        keep[i] = as_u32(__builtin_bit_cast(v2u16, __builtin_bit_cast(short2, d) >> (short)15));
      }
      if ((keep[0] & keep[1] & keep[2] & keep[3]) != 0xffffffffu) {
        uint32_t bits = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) bits |= (((~keep[i]) & 1u) | ((~keep[i] >> 15) & 2u)) << (2 * i);
        atomicOr(&bm[c >> 2], bits << ((c & 3) * 8));
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        v2u16 m = rmax[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) m = pk_max(m, as_u16x2(as_u32(ab[t][i]) & keep[i]));
        rmax[t] = m;
      }
    }
    // fold the two halves, pack row pairs, reduce over the wavefront
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (2 * p < T) {
        const uint32_t lo = max(rmax[2 * p].x, rmax[2 * p].y);
        const uint32_t hi = 2 * p + 1 < TB ? max(rmax[2 * p + 1].x, rmax[2 * p + 1].y) : 0u;
        const uint32_t r = wave_max_u16x2(lo | (hi << 16));
        if (lane == 0) rowred[wave * 8 + p] = r;
      }
    }
  }
  lds_barrier();  // B: bitmap and partial row maxima complete

  {
    // ---- 4. row scales: lane t (< T) of every wavefront combines the 8
    // partial maxima of row t; the scales then go to scalar registers
    float srow = 0.0f;
    if (lane < T) {
      uint32_t m = 0u;
#pragma unroll
      for (int w = 0; w < 8; ++w) m = max(m, (rowred[w * 8 + (lane >> 1)] >> ((lane & 1) * 16)) & 0xffffu);
      const float ax = A16::to_f32(m);
      srow = m ? 127.0f / ax : 0.0f;
      if (wave == 0) arow[lane] = ax;
    }
    float st[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t)
      st[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, srow), t));
    // int8 codes of this thread's chunks
    for (int c = tid; c < KC; c += 512) {
      const uint32_t skip = (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu;
      const uint32_t m0 = expand4(~skip & 0xfu), m1 = expand4((~skip >> 4) & 0xfu);
      uint4 v[TB];
#pragma unroll
      for (int t = 0; t < TB; ++t)
        if (t < T) v[t] = *reinterpret_cast<const uint4*>(xs + t * K + c * 8);
#pragma unroll
      for (int t = 0; t < TB; ++t)
        if (t < T) *reinterpret_cast<uint2*>(xq + t * L.kp + c * 8) = A16::quantize8(v[t], st[t], m0, m1);
    }
    // wavefront 0: compact the outlier indices (ascending), then gather the
    // weight bytes of the first 32 outlier columns for the epilogue
    if (wave == 0) {
      const int per = (KW + 63) / 64;
      const int w0i = min(KW, lane * per), w1i = min(KW, w0i + per);
      int local = 0;
      for (int w = w0i; w < w1i; ++w) local += __popc(bm[w]);
      const int incl = wave_incl_sum(local);
      const int count = __builtin_amdgcn_readlane(incl, 63);
      if (count) {
        int j = incl - local;
        for (int w = w0i; w < w1i; ++w) {
          uint32_t bits = bm[w];
          while (bits) {
            idxl[j++] = (uint16_t)(w * 32 + __builtin_ctz(bits));
            bits &= bits - 1u;
          }
        }
      }
      if (lane == 0) *cnt = count;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // the wavefront's index writes precede its reads
      const uint4 iv = *reinterpret_cast<const uint4*>(idxl + fg * 8);
      const uint32_t iw[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = (iw[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        g[e] = load_word_of(rW, fg * 8 + e < count ? rowoff + h : kOobOffset);
      }
    }
  }
  lds_barrier();  // C: int8 rows of X, row statistics and outlier indices ready

  if (!xwave) {
    // ---- 5. int8 product of this wavefront's K range; partial sums to LDS.
    // B operand lanes of rows past T read row T-1: they only feed output
    // columns t >= T, which are never stored. Steps past the range read
    // in-bounds X; their weights were loaded as zeros.
    v4i acc = {0, 0, 0, 0};
    const int8_t* xrow = xq + min(fi, T - 1) * L.kp;
    auto compute_batch = [&](const v4i* w, int b) {
      v4i xf[kGemvBatch];
#pragma unroll
      for (int s = 0; s < kGemvBatch; ++s) {
        const int k = min(kbeg + (b * kGemvBatch + s) * 64 + fg * 16, K - 16);
        xf[s] = *reinterpret_cast<const v4i*>(xrow + k);
      }
      __builtin_amdgcn_sched_barrier(0);  // all reads in flight before the first product
#pragma unroll
      for (int s = 0; s < kGemvBatch; ++s) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[s], xf[s], acc, 0, 0, 0);
    };
    for (int b = 0; b < nbatch; b += 2) {
      if (b + 1 < nbatch) load_batch(w1, b + 1);
      compute_batch(w0, b);
      if (b + 1 < nbatch) {
        if (b + 2 < nbatch) load_batch(w0, b + 2);
        compute_batch(w1, b + 1);
      }
    }
    red[ww * 64 + lane] = acc;
  }
  // X wavefront 0, while the stream wavefronts multiply: the 16-bit outlier
  // product, which needs only X and the gathered weight bytes. Lane holds
  // rows (n) n0 + 4*fg + v of column (t) fi.
  const int count = *cnt;
  const int t = fi;
  v4f yo = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0 && count) {
    const uint16_t* xr = xs + min(t, T - 1) * K;
    for (int c = 0; c < count; c += kOutChunk) {
      // 8 indices in one read (past `count` they are masked below), then the
      // 8 activation reads together
      const uint4 iv = *reinterpret_cast<const uint4*>(idxl + c + fg * 8);
      const uint32_t iw[4] = {iv.x, iv.y, iv.z, iv.w};
      int h[8];
      uint16_t xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[e] = c + fg * 8 + e < count ? (int)((iw[e >> 1] >> ((e & 1) * 16)) & 0xffffu) : 0;
        xv[e] = xr[h[e]];
      }
      uint16_t wf[8], xf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = c + fg * 8 + e < count;
        const uint32_t word = c == 0 ? g[e] : load_word_of(rW, ok ? rowoff + (uint32_t)h[e] : kOobOffset);
        wf[e] = A16::from_f32(((float)byte_of(word, h[e]) * brow) / 127.0f);
        xf[e] = (ok && t < T) ? xv[e] : (uint16_t)0;
      }
      const uint4 wf4 = make_uint4(wf[0] | ((uint32_t)wf[1] << 16), wf[2] | ((uint32_t)wf[3] << 16),
                                   wf[4] | ((uint32_t)wf[5] << 16), wf[6] | ((uint32_t)wf[7] << 16));
      const uint4 xf4 = make_uint4(xf[0] | ((uint32_t)xf[1] << 16), xf[2] | ((uint32_t)xf[3] << 16),
                                   xf[4] | ((uint32_t)xf[5] << 16), xf[6] | ((uint32_t)xf[7] << 16));
      yo = A16::mma16(wf4, xf4, yo);
    }
  }
  lds_barrier();  // D: the 4 partial products are in LDS

  // intermediate stages for inspection (first block only, off the timed path)
  if (blockIdx.x == 0) {
    for (int w = tid; w < KW; w += 512)
      if (a.dbg_bitmap) a.dbg_bitmap[w] = bm[w];
    for (int j = tid; j < count; j += 512)
      if (a.dbg_idx) a.dbg_idx[j] = idxl[j];
    if (tid == 0 && a.dbg_count) a.dbg_count[0] = count;
    if (tid < T && a.dbg_aX) a.dbg_aX[tid] = arow[tid];
    if (a.dbg_Xq)
      for (int i = tid; i < T * KC; i += 512) {
        const int t = i / KC, c = i - t * KC;
        *reinterpret_cast<uint2*>(a.dbg_Xq + (size_t)t * K + c * 8) =
            *reinterpret_cast<const uint2*>(xq + t * L.kp + c * 8);
      }
  }
  if (wave != 0) return;
  // exact sum of the 4 partial products
  v4i acc = red[lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) acc += red[w * 64 + lane];

  // ---- 6. dequantize, add the outlier product and the bias, round and store
  const int n = n0 + 4 * fg;
  if (a.dbg_C && t < T) {
    for (int v = 0; v < 4; ++v)
      if (n + v < N) a.dbg_C[(size_t)t * N + n + v] = acc[v];
  }
  const float at = t < T ? arow[t] : 0.0f;
  v4f y;
#pragma unroll
  for (int v = 0; v < 4; ++v) y[v] = (float)acc[v] * (at * (bs4[v] * (1.0f / 16129.0f))) + yo[v];
  if (a.bias) {
#pragma unroll
    for (int v = 0; v < 4; ++v) y[v] += A16::to_f32(bias4[v]);
  }
  if (t < T) {
    uint16_t* dst = a.Y + (size_t)t * N + n;
    if ((N & 3) == 0 && n + 3 < N) {
      uint2 p;
      p.x = (uint32_t)A16::from_f32(y[0]) | ((uint32_t)A16::from_f32(y[1]) << 16);
      p.y = (uint32_t)A16::from_f32(y[2]) | ((uint32_t)A16::from_f32(y[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = p;
    } else {
      for (int v = 0; v < 4; ++v)
        if (n + v < N) dst[v] = A16::from_f32(y[v]);
    }
  }
}

template <int TB, bool BF16>
static hipError_t launch_gemv_tb(const LinearArgs& a, hipStream_t stream) {
  const GemvLds L = gemv_lds(a.T, a.K);
  static std::atomic<int> attr_max{64 * 1024};  // dynamic LDS this instance is allowed so far
  if (L.total > attr_max.load()) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kd_gemv<TB, BF16>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
    if (e != hipSuccess) return e;
    int cur = attr_max.load();
    while (cur < L.total && !attr_max.compare_exchange_weak(cur, L.total)) {
    }
  }
  const int kq = (int)(ceil_div(ceil_div(a.K, 4), 64) * 64);
  const int blocks = (int)ceil_div(a.N, kGemvRowsN);
  hipLaunchKernelGGL((kd_gemv<TB, BF16>), dim3(blocks), dim3(512), L.total, stream, a,
                     threshold_code(a.thr, BF16), kq);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_gemv_dt(const LinearArgs& a, hipStream_t stream) {
  if (a.T <= 1) return launch_gemv_tb<1, BF16>(a, stream);
  if (a.T <= 2) return launch_gemv_tb<2, BF16>(a, stream);
  if (a.T <= 4) return launch_gemv_tb<4, BF16>(a, stream);
  if (a.T <= 8) return launch_gemv_tb<8, BF16>(a, stream);
  return launch_gemv_tb<16, BF16>(a, stream);
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_gemv_dt<true>(a, stream) : launch_gemv_dt<false>(a, stream);
}

}  // namespace llmint8
