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
//   * The scan: a thread owns 8-column chunks across all T rows, decides
//     their outlier flags on its own (column absmax >= threshold) and takes
//     the rows' maxima over its kept columns in the same pass (packed u16
//     arithmetic on 16-bit magnitude codes). At T = 1 the X wavefronts scan
//     alone, each the chunks it copied, while the stream wavefronts are still
//     issuing; for more rows all 8 wavefronts scan once those have issued.
//   * After one block-wide reduction all 8 wavefronts quantize their chunks
//     into LDS.
//   * The stream wavefronts then multiply their quarter of K on
//     v_mfma_i32_16x16x64_i8 (16 weight rows as A, int8 rows of X as B, four
//     independent accumulators) and leave int32 partial sums in LDS.
//     Meanwhile X wavefront 0, which has compacted the outlier indices,
//     gathers the weight bytes of the outlier columns and computes the 16-bit
//     outlier product on v_mfma_f32_16x16x32_f16; it finally sums the
//     partials, dequantizes and stores Y in the activation type (fp16 or
//     bf16).
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
  L.cnt = off;  // [0] outlier count, [1] X wavefronts' arrivals (T = 1)
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

// Keep masks of 8 columns from their magnitude codes (packed u16 pairs):
// cm - thr is negative (sign bit set) exactly where the column stays below the
// threshold. Both codes are below 2^15, so the packed difference cannot wrap.
__device__ __forceinline__ uint32_t keep_mask(v2u16 cm, v2u16 hthr2) {
  const v2u16 d = cm - hthr2;
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, __builtin_bit_cast(short2, d) >> (short)15));
}
// Outlier bits (bit j: column j reaches the threshold) of 8 columns from their keep masks.
__device__ __forceinline__ uint32_t outlier_bits(const uint32_t keep[4]) {
  uint32_t bits = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) bits |= (((~keep[i]) & 1u) | ((~keep[i] >> 15) & 2u)) << (2 * i);
  return bits;
}
__device__ __forceinline__ v2u16 as_u16x2(uint32_t x) { return __builtin_bit_cast(v2u16, x); }
__device__ __forceinline__ uint32_t as_u32(v2u16 x) { return __builtin_bit_cast(uint32_t, x); }
// Maxima over the wavefront of NV independent unsigned values, one DPP step
// for all of them before the next, so that the chains overlap instead of
// waiting out each other's latencies; the totals end in lane 63. Lanes that a
// step leaves without a source take 0, the identity of the maximum, so each
// step can be one v_max_u32 with a DPP operand.
template <int NV>
__device__ __forceinline__ void wave_max_u32_n(uint32_t (&v)[NV]) {
  auto step = [&](auto ctrl, auto row_mask) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      v[i] = max(v[i], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[i], decltype(ctrl)::value,
                                                              decltype(row_mask)::value, 0xF, false));
  };
  step(std::integral_constant<int, 0xB1>{}, std::integral_constant<int, 0xF>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{}, std::integral_constant<int, 0xF>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{}, std::integral_constant<int, 0xF>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{}, std::integral_constant<int, 0xF>{});  // row_mirror
  step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});  // row_bcast:15
  step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});  // row_bcast:31
}

template <int TB, bool BF16, int XM>
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
  int* xctr = cnt + 1;

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
  // With XS the X wavefronts scan (each its own copies of X) and quantize
  // alone, so that work waits neither for the stream wavefronts to finish
  // issuing nor for their loads. X wavefront w copies the 1 KB pieces w,
  // w + 4, ... of X, which hold the chunks 64w + 256i of every row when
  // there is one row or K is a multiple of 2048 (the host picks XS then).
  constexpr bool kXScan = XM != 0;               // the X wavefronts scan alone
  constexpr bool kXQuant = XM == 1 || XM == 3;   // ... and quantize alone (else all 8 wavefronts do, after barrier B)
  constexpr bool kXRegs = XM == 2 || XM == 3;    // X loaded into the X wavefronts' registers
  // XM 2 and 3: X is loaded into the X wavefronts' registers, each thread the
  // kCpt chunks it scans, and written to LDS by them; the kernel then has no
  // copy into LDS in flight that the stream wavefronts' LDS reads would wait on
  constexpr int kCpt = kXRegs ? (TB <= 2 ? 4 : 4096 / (TB * 256)) : 1;
  static_assert(!kXRegs || kCpt >= 1, "register-loaded X needs TB <= 16");
  uint4 xr[kCpt][TB];
  uint32_t xskip[kCpt];  // outlier flags of the thread's chunks (register-loaded X)
  constexpr int kScanWaves = kXScan ? 4 : 8;  // wavefronts that leave partial row maxima

  // stream wavefronts: their K range and the first batch of weight loads
  const int ww = wave & 3;
  const int kbeg = ww * kq;
  const int kend = min(K, kbeg + kq);
  const int steps = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  const int nbatch = (steps + kGemvBatch - 1) / kGemvBatch;
  // Whole lines (TB <= 2): 128 contiguous bytes per row per load; for the step pair (2p, 2p+1)
  // load w[2p] covers rows 0-7 and w[2p+1] rows 8-15, each row's 128 bytes
  // by 8 lanes. Lane (fg, fi) takes row fi & 7 (+ 8), bytes 16 * (fg + 4 *
  // (fi >> 3)) of the pair: lanes fi < 8 hold the first 64 bytes of their
  // row, lanes fi >= 8 the second 64 bytes of row fi - 8 (+ 8).
  // Up to 2 rows, where the weights landing is the critical path, a load covers
  // whole lines and each fragment takes two MFMAs (above). From 4 rows on the
  // product starts after the X work, when the weights have landed, and the
  // doubled MFMAs would be on the critical path (about 2000 instead of 1000
  // cycles per wavefront): lane (fg, fi) then loads row fi, bytes 16 fg of
  // the 64-byte step, one MFMA per fragment.
  constexpr bool kWholeLine = TB <= 2;
  // the outlier indices compacted by a stream wavefront before barrier C (the
  // form whose X wavefronts meet at the LDS counter and quantize alone), from
  // 4 rows on: with fewer rows the X work ends early and the compaction would
  // hold barrier C back instead
  constexpr bool kIdxByStream = XM == 3 && TB >= 4;
  // in the 16-row form X wavefront 3 compacts them after barrier B, before its
  // share of the quantization (it has the least scanning to do)
  constexpr bool kIdxByX3 = XM == 2;
  constexpr bool kEarlyIdx = kIdxByStream || kIdxByX3;
  auto load_batch = [&](v4i* w, int b) {
    if constexpr (kWholeLine) {
      const uint32_t r0 = (uint32_t)((fi & 7) * K), r1 = (uint32_t)((8 + (fi & 7)) * K);
#pragma unroll
      for (int p = 0; p < kGemvBatch / 2; ++p) {
        const int k = kbeg + (b * kGemvBatch + 2 * p) * 64 + fg * 16 + (fi >> 3) * 64;
        const bool in = k < kend;
        w[2 * p] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rW, in ? r0 + (uint32_t)k : kOobOffset, 0, 0));
        w[2 * p + 1] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rW, in ? r1 + (uint32_t)k : kOobOffset, 0, 0));
      }
    } else {
#pragma unroll
      for (int s = 0; s < kGemvBatch; ++s) {
        const int k = kbeg + (b * kGemvBatch + s) * 64 + fg * 16;
        w[s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rW, k < kend ? rowoff + (uint32_t)k : kOobOffset, 0, 0));
      }
    }
  };
  // ---- 3. the scan: a thread takes 8-column chunks across all rows: column
  // absmax -> outlier flags -> keep masks -> row maxima over the kept columns.
  // All values are 16-bit codes with the sign cleared, compared as packed u16.
  // Each scanning wavefront leaves its partial row maxima in rowred.
  // one chunk: its column maxima over the rows -> outlier bits into the
  // bitmap; the rows' maxima over its kept columns into rmax
  auto scan_chunk = [&](int c, const uint4* v, v2u16* rmax) -> uint32_t {
    const v2u16 hthr2 = {(uint16_t)hthr, (uint16_t)hthr};
    v2u16 ab[TB][4];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      ab[t][0] = as_u16x2(v[t].x & 0x7fff7fffu);
      ab[t][1] = as_u16x2(v[t].y & 0x7fff7fffu);
      ab[t][2] = as_u16x2(v[t].z & 0x7fff7fffu);
      ab[t][3] = as_u16x2(v[t].w & 0x7fff7fffu);
    }
    uint32_t keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v2u16 cm = ab[0][i];
#pragma unroll
      for (int t = 1; t < TB; ++t) cm = pk_max(cm, ab[t][i]);
      keep[i] = keep_mask(cm, hthr2);
    }
    const uint32_t bits = outlier_bits(keep);
    if (bits) atomicOr(&bm[c >> 2], bits << ((c & 3) * 8));
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      v2u16 m = rmax[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) m = pk_max(m, as_u16x2(as_u32(ab[t][i]) & keep[i]));
      rmax[t] = m;
    }
    return bits;
  };
  // fold the two halves, pack row pairs, reduce over the wavefront
  // (rows past T hold zeros, so every pair is reduced and only live ones stored)
  auto scan_finish = [&](const v2u16* rmax) {
    uint32_t r[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) r[t] = max(rmax[t].x, rmax[t].y);
    wave_max_u32_n<TB>(r);
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (2 * p < T && lane == 63) rowred[wave * 8 + p] = r[2 * p] | (2 * p + 1 < TB ? r[2 * p + 1] << 16 : 0u);
  };
  auto scan_chunks = [&](int first, int stride) {
    v2u16 rmax[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) rmax[t] = v2u16{0, 0};
    for (int c = first; c < KC; c += stride) {
      uint4 v[TB];
#pragma unroll
      for (int t = 0; t < TB; ++t)
        v[t] = t < T ? *reinterpret_cast<const uint4*>(xs + t * K + c * 8) : uint4{0, 0, 0, 0};
      scan_chunk(c, v, rmax);
    }
    scan_finish(rmax);
  };

  // ---- 4. row scales from the scanning wavefronts' partial maxima, and the
  // int8 codes of the chunks first, first + stride, ...
  // lane t (< T) of every calling wavefront combines the partial maxima of
  // row t; the scales then go to scalar registers
  auto row_scales = [&](float (&st)[TB]) {
    float srow = 0.0f;
    if (lane < T) {
      uint32_t m = 0u;
#pragma unroll
      for (int w = 0; w < kScanWaves; ++w) m = max(m, (rowred[w * 8 + (lane >> 1)] >> ((lane & 1) * 16)) & 0xffffu);
      const float ax = A16::to_f32(m);
      srow = m ? 127.0f / ax : 0.0f;
      if (wave == 0) arow[lane] = ax;
    }
#pragma unroll
    for (int t = 0; t < TB; ++t)
      st[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, srow), t));
  };
  auto quantize_chunks = [&](int first, int stride) {
    float st[TB];
    row_scales(st);
    // int8 codes of this thread's chunks
    for (int c = first; c < KC; c += stride) {
      uint4 v[TB];
#pragma unroll
      for (int t = 0; t < TB; ++t)
        if (t < T) v[t] = *reinterpret_cast<const uint4*>(xs + t * K + c * 8);
      uint32_t skip;
      if constexpr (TB == 1) {
        // one row: a column's maximum is its only value, so the outlier
        // flags follow from the chunk itself, as in the scan
        const v2u16 hthr2 = {(uint16_t)hthr, (uint16_t)hthr};
        const uint32_t keep[4] = {keep_mask(as_u16x2(v[0].x & 0x7fff7fffu), hthr2),
                                  keep_mask(as_u16x2(v[0].y & 0x7fff7fffu), hthr2),
                                  keep_mask(as_u16x2(v[0].z & 0x7fff7fffu), hthr2),
                                  keep_mask(as_u16x2(v[0].w & 0x7fff7fffu), hthr2)};
        skip = outlier_bits(keep);
      } else {
        skip = (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu;
      }
      const uint32_t m0 = expand4(~skip & 0xfu), m1 = expand4((~skip >> 4) & 0xfu);
#pragma unroll
      for (int t = 0; t < TB; ++t)
        if (__builtin_expect(t < T, 1)) *reinterpret_cast<uint2*>(xq + t * L.kp + c * 8) = A16::quantize8(v[t], st[t], m0, m1);
    }
  };

  // The same codes, one (row, chunk) item per thread and step, for the form
  // where every row is quantized by all 8 wavefronts: with few chunks per row,
  // splitting by chunk alone would leave most threads without work and the
  // rest with all rows. Each thread takes its row's scale from the partial
  // maxima itself (the same expression as row_scales, so the same value).
  auto quantize_items = [&](int first, int stride) {
    for (int i = first; i < T * KC; i += stride) {
      const int t = i / KC, c = i - t * KC;
      uint32_t m = 0u;
#pragma unroll
      for (int w = 0; w < kScanWaves; ++w) m = max(m, (rowred[w * 8 + (t >> 1)] >> ((t & 1) * 16)) & 0xffffu);
      const float ax = A16::to_f32(m);
      const float st = m ? 127.0f / ax : 0.0f;
      const uint4 v = *reinterpret_cast<const uint4*>(xs + t * K + c * 8);
      const uint32_t skip = (bm[c >> 2] >> ((c & 3) * 8)) & 0xffu;
      const uint32_t m0 = expand4(~skip & 0xfu), m1 = expand4((~skip >> 4) & 0xfu);
      *reinterpret_cast<uint2*>(xq + t * L.kp + c * 8) = A16::quantize8(v, st, m0, m1);
    }
    if (wave == 0 && lane < T) {  // the row statistic for the epilogue
      uint32_t m = 0u;
#pragma unroll
      for (int w = 0; w < kScanWaves; ++w) m = max(m, (rowred[w * 8 + (lane >> 1)] >> ((lane & 1) * 16)) & 0xffffu);
      arow[lane] = A16::to_f32(m);
    }
  };

  // ---- 5b. the outlier indices, ascending, compacted from the bitmap by one
  // wavefront; returns their count. The int8 product does not need them:
  // wavefront 0 compacts them after barrier C, beside the stream wavefronts'
  // products, unless a wavefront with slack has done so before C (kEarlyIdx).
  auto compact = [&]() -> int {
    const int per = (KW + 63) / 64;
    const int w0i = min(KW, lane * per), w1i = min(KW, w0i + per);
    // up to 4 words per lane (K <= 8192) are read once and kept in registers
    constexpr int kHeld = 4;
    uint32_t held[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i) held[i] = w0i + i < w1i ? bm[w0i + i] : 0u;
    int local = 0;
#pragma unroll
    for (int i = 0; i < kHeld; ++i) local += __popc(held[i]);
    for (int w = w0i + kHeld; w < w1i; ++w) local += __popc(bm[w]);
    const int incl = wave_incl_sum(local);
    const int count = __builtin_amdgcn_readlane(incl, 63);
    if (count) {
      int j = incl - local;
      for (int w = w0i; w < w1i; ++w) {
        const int i = w - w0i;
        uint32_t bits = i == 0 ? held[0] : i == 1 ? held[1] : i == 2 ? held[2] : i == 3 ? held[3] : bm[w];
        while (bits) {
          idxl[j++] = (uint16_t)(w * 32 + __builtin_ctz(bits));
          bits &= bits - 1u;
        }
      }
    }
    if (lane == 0) *cnt = count;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the index writes precede the wavefront's reads
    return count;
  };

  v4i w0[kGemvBatch], w1[kGemvBatch];
  float bs4[4] = {0.f, 0.f, 0.f, 0.f}, brow = 0.f;
  uint32_t bias4[4] = {0, 0, 0, 0};  // 16-bit values kept in whole registers: no packing waits for the loads
  // At T = 1 the X wavefronts synchronise among themselves through a counter
  // in LDS; the stream wavefronts meet them only at barrier C. The counter
  // is cleared before one block barrier at entry (E), which the X
  // wavefronts reach once their copies of X are issued and the stream
  // wavefronts before their first load: the copies of X enter the memory
  // pipeline ahead of the weight stream. The wait is bounded, so it always ends.
  auto x_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes are done
    if (lane == 0) __hip_atomic_fetch_add(xctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int spin = 0; spin < (1 << 22); ++spin) {
      if (__hip_atomic_load(xctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= 4) break;
      __builtin_amdgcn_s_sleep(1);
    }
  };
  if (xwave) {
    // ---- 1. X -> LDS (1 KB per wavefront issue); wavefront 0 also fetches
    // the scales of the 16 weight rows (rows past N read as zero)
    const int xbytes = T * K * 2;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X, (uint32_t)xbytes);
    if constexpr (kXRegs) {
      // into registers, each thread the chunks it scans (rows past T and
      // chunks past the row read as zero); written to LDS below
#pragma unroll
      for (int i = 0; i < kCpt; ++i) {
        const int c = xt + 256 * i;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const uint32_t off = c < KC && t < T ? (uint32_t)((t * K + c * 8) * 2) : kOobOffset;
          xr[i][t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
        }
      }
    } else {
      for (int blk = wave; blk * 1024 < xbytes; blk += 4)
        lds_copy16(rX, lds + L.xs + blk * 1024, (uint32_t)(blk * 1024 + lane * 16));
    }
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
    if constexpr (kXScan) {
      if (tid == 0) *xctr = 0;
      lds_barrier();  // E: the counter is clear; X and the scales are requested
    }
    if constexpr (kXScan) {
      // X wavefront w copied the 1 KB pieces w, w + 4, ... of the row, i.e.
      // chunks 64w + 256i + lane: it clears the bitmap words of those chunks
      // and scans them as soon as its own copies have landed. The stream
      // wavefronts, stalled issuing the weight loads, wait for none of it.
      for (int c = xt; c < KC; c += 256)
        if ((c & 3) == 0) bm[c >> 2] = 0u;
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's part of X has landed
      if constexpr (kXRegs) {
        v2u16 rmax[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) rmax[t] = v2u16{0, 0};
#pragma unroll
        for (int i = 0; i < kCpt; ++i) {
          const int c = xt + 256 * i;
          if (c < KC) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
              if (__builtin_expect(t < T, 1)) *reinterpret_cast<uint4*>(lds + L.xs + (t * K + c * 8) * 2) = xr[i][t];
            xskip[i] = scan_chunk(c, xr[i], rmax);
          }
        }
        scan_finish(rmax);
      } else {
        scan_chunks(xt, 256);
      }
      if constexpr (XM == 1) {
        x_sync();  // the 4 partial maxima and the whole bitmap are in LDS
        quantize_chunks(xt, 256);
      }
      if constexpr (XM == 3) {
        // codes straight from the registers; a chunk's outlier flags are the
        // scan's own (it saw every row of its columns)
        x_sync();  // the 4 partial maxima are in LDS
        float st[TB];
        row_scales(st);
#pragma unroll
        for (int i = 0; i < kCpt; ++i) {
          const int c = xt + 256 * i;
          if (c < KC) {
            const uint32_t m0 = expand4(~xskip[i] & 0xfu), m1 = expand4((~xskip[i] >> 4) & 0xfu);
#pragma unroll
            for (int t = 0; t < TB; ++t)
              if (__builtin_expect(t < T, 1)) *reinterpret_cast<uint2*>(xq + t * L.kp + c * 8) = A16::quantize8(xr[i][t], st[t], m0, m1);
          }
        }
      }
    } else {
      for (int w = xt; w < KW; w += 256) bm[w] = 0u;
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's part of X has landed
    }
  } else {
    // ---- 2. the weight stream: 16 x 16-byte loads per lane, in flight while
    // the X wavefronts work (issuing them stalls only these wavefronts)
    if constexpr (kXScan) lds_barrier();  // E
    load_batch(w0, 0);  // out-of-range steps read as zero
    if constexpr (kIdxByStream) {
      // The first stream wavefront, idle until its weights land, compacts the
      // outlier indices once the X wavefronts' scan is complete (the counter
      // reaches 4 after their bitmap updates), so that after barrier C
      // wavefront 0 starts straight at the gather. The wait is a relaxed read
      // of the LDS counter, with no ordering against memory, so the
      // wavefront's weight loads stay in flight. That suffices here: the X
      // wavefronts raise the counter only once their bitmap updates have
      // completed, and this wavefront's LDS reads of the bitmap issue after
      // the counter read has returned. The wait is bounded, so it always ends.
      if (wave == 4) {
        const __attribute__((address_space(3))) int* ctr = (const __attribute__((address_space(3))) int*)xctr;
        for (int spin = 0; spin < (1 << 22); ++spin) {
          if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= 4) break;
          __builtin_amdgcn_s_sleep(1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        compact();
      }
    }
  }
  if constexpr (!kXScan) {
    lds_barrier();  // A: X is in LDS, the bitmap is clear
    // all 8 wavefronts scan and quantize (the stream wavefronts have issued
    // their loads by now)
    scan_chunks(tid, 512);
  }
  if constexpr (!kXQuant) {
    lds_barrier();  // B: bitmap and partial row maxima complete
    if constexpr (XM == 2) {
      if (wave == 3) compact();  // the bitmap is complete at B
      quantize_items(tid, 512);
    } else {
      quantize_chunks(tid, 512);
    }
  }
  lds_barrier();  // C: int8 rows of X and the row statistics are ready

  if (!xwave) {
    // ---- 5. int8 product of this wavefront's K range; partial sums to LDS.
    // B operand lanes of rows past T hold zeros and read nothing: they only
    // feed output columns t >= T, which are never stored, and at small T the
    // LDS reads of the live lanes alone are a fraction of a full fragment's.
    // Steps past the range read in-bounds X; their weights were loaded as zeros.
    v4i acc4[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};  // independent chains
    const int8_t* xrow = xq + min(fi, T - 1) * L.kp;
    const bool live = fi < T;
    auto compute_batch = [&](const v4i* w, int b) {
      v4i xf[kGemvBatch];
#pragma unroll
      for (int s = 0; s < kGemvBatch; ++s) xf[s] = v4i{0, 0, 0, 0};
      if (live) {
#pragma unroll
        for (int s = 0; s < kGemvBatch; ++s) {
          const int k = min(kbeg + (b * kGemvBatch + s) * 64 + fg * 16, K - 16);
          xf[s] = *reinterpret_cast<const v4i*>(xrow + k);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // all reads in flight before the first product
      // Each whole-line fragment meets both halves of the X pair. Product
      // rows where the fragment's k range matches the X half are the valid
      // ones: acc4[0] rows 0-7 (weight rows 0-7, first halves), acc4[1]
      // rows 8-15 (weight rows 0-7, second halves), acc4[2] rows 0-7 (weight
      // rows 8-15, first halves), acc4[3] rows 8-15 (weight rows 8-15,
      // second halves); the other rows are discarded.
      if constexpr (kWholeLine) {
#pragma unroll
        for (int p = 0; p < kGemvBatch / 2; ++p) {
          acc4[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[2 * p], xf[2 * p], acc4[0], 0, 0, 0);
          acc4[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[2 * p], xf[2 * p + 1], acc4[1], 0, 0, 0);
          acc4[2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[2 * p + 1], xf[2 * p], acc4[2], 0, 0, 0);
          acc4[3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[2 * p + 1], xf[2 * p + 1], acc4[3], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < kGemvBatch; ++s)
          acc4[s & 3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[s], xf[s], acc4[s & 3], 0, 0, 0);
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
    // Output lane (fg, fi) holds rows 4 fg .. 4 fg + 3: lanes fg < 2 (rows
    // 0-7) add acc4[1] of the lane 32 above, lanes fg >= 2 (rows 8-15)
    // acc4[2] of the lane 32 below. Exact int32 sums.
    if constexpr (kWholeLine) {
      const v4i own = fg < 2 ? acc4[0] : acc4[3], give = fg < 2 ? acc4[2] : acc4[1];
      v4i other;
#pragma unroll
      for (int v = 0; v < 4; ++v) other[v] = __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, give[v]);
      red[ww * 64 + lane] = own + other;
    } else {
      red[ww * 64 + lane] = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
    }
  }
  // X wavefront 0, while the stream wavefronts multiply: the outlier indices,
  // then the 16-bit outlier product, which needs only X and the gathered
  // weight bytes. Lane holds rows (n) n0 + 4*fg + v of column (t) fi.
  const int t = fi;
  v4f yo = {0.f, 0.f, 0.f, 0.f};
  const float at = wave == 0 && t < T ? arow[t] : 0.0f;  // row statistic for the epilogue, read early
  const int count0 = wave != 0 ? 0 : kEarlyIdx ? __builtin_amdgcn_readfirstlane(*cnt) : compact();
  if (count0) {
    const int count = count0;
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
        const uint32_t word = load_word_of(rW, ok ? rowoff + (uint32_t)h[e] : kOobOffset);
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
  lds_barrier();  // D: the 4 partial products and the outlier indices are in LDS

  // intermediate stages for inspection (first block only, off the timed path)
  if (blockIdx.x == 0) {
    const int count = __builtin_amdgcn_readfirstlane(*cnt);
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
  v4f y;
#pragma unroll
  for (int v = 0; v < 4; ++v) y[v] = (float)acc[v] * (at * (bs4[v] * (1.0f / 16129.0f))) + yo[v];
  if (a.bias) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // An empty asm that may change the bias bits keeps their conversion
      // here. Moved up to the loads, it would wait there, and with the copies
      // of X issued before the bias, that wait holds the entry barrier.
      uint32_t b = bias4[v];
      asm volatile("" : "+v"(b));
      y[v] += A16::to_f32(b);
    }
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

template <int TB, bool BF16, int XM>
static hipError_t launch_gemv_tb(const LinearArgs& a, hipStream_t stream) {
  const GemvLds L = gemv_lds(a.T, a.K);
  static std::atomic<int> attr_max{64 * 1024};  // dynamic LDS this instance is allowed so far
  if (L.total > attr_max.load()) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kd_gemv<TB, BF16, XM>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
    if (e != hipSuccess) return e;
    int cur = attr_max.load();
    while (cur < L.total && !attr_max.compare_exchange_weak(cur, L.total)) {
    }
  }
  const int kq = (int)(ceil_div(ceil_div(a.K, 4), 64) * 64);
  const int blocks = (int)ceil_div(a.N, kGemvRowsN);
  hipLaunchKernelGGL((kd_gemv<TB, BF16, XM>), dim3(blocks), dim3(512), L.total, stream, a,
                     threshold_code(a.thr, BF16), kq);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_gemv_dt(const LinearArgs& a, hipStream_t stream) {
  // XM 3: X in the X wavefronts' registers (a thread holds kCpt chunks of TB
  // rows), they scan and quantize alone from the registers (up to 8 rows);
  // XM 2: the same loads, the X wavefronts scan and all 8 quantize (16 rows);
  // XM 1: X copied into LDS, the X wavefronts scan and quantize alone, when
  // their copies hold whole chunk columns; XM 0: all 8 scan and quantize
  const bool xs = a.K % 2048 == 0;
  if (a.T <= 1) return a.K <= 8192 ? launch_gemv_tb<1, BF16, 3>(a, stream) : launch_gemv_tb<1, BF16, 1>(a, stream);
  if (a.T <= 2)
    return a.K <= 8192 ? launch_gemv_tb<2, BF16, 3>(a, stream)
                       : xs ? launch_gemv_tb<2, BF16, 1>(a, stream) : launch_gemv_tb<2, BF16, 0>(a, stream);
  if (a.T <= 4)
    return a.K <= 8192 ? launch_gemv_tb<4, BF16, 3>(a, stream)
                       : xs ? launch_gemv_tb<4, BF16, 1>(a, stream) : launch_gemv_tb<4, BF16, 0>(a, stream);
  if (a.T <= 8)
    return a.K <= 4096 ? launch_gemv_tb<8, BF16, 3>(a, stream)
                       : xs ? launch_gemv_tb<8, BF16, 1>(a, stream) : launch_gemv_tb<8, BF16, 0>(a, stream);
  return a.K <= 2048 ? launch_gemv_tb<16, BF16, 2>(a, stream)
                     : xs ? launch_gemv_tb<16, BF16, 1>(a, stream) : launch_gemv_tb<16, BF16, 0>(a, stream);
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_gemv_dt<true>(a, stream) : launch_gemv_dt<false>(a, stream);
}

}  // namespace llmint8
