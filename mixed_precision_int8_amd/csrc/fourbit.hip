// 4-bit weights on gfx950: NF4 / FP4 code books, blockwise 4-bit quantization
// and dequantization, and the decode-shaped linear layer that dequantizes the
// weight on the fly ("bitsandbytes: GPU-Accelerated Inference and Training at
// Lower Bit Depths", introduction: FP4 and NF4 data types, blockwise scaling
// factors, 16-bit compute with the weights dequantized per operation;
// "Hugging Face Quantization with bitsandbytes ...", section 4: NF4 is fitted to
// normally distributed weights, FP4 is a generic 4-bit float).
//
// Code books, computed on the host in binary64 and rounded once to fp32:
//   NF4  standard-normal quantiles: eight levels above zero at probabilities
//        p_max + i (0.5 - p_max) / 8 (i = 0..7), seven below zero at the
//        mirrored probabilities p_max + i (0.5 - p_max) / 7 (i = 0..6), and an
//        exact zero, all divided by the quantile at p_max = 1 - (1/32 + 1/30)/2
//        (the published NormalFloat construction); code = ascending rank.
//   FP4  E2M1: sign, two exponent bits with bias 1, one mantissa bit, exponent 0
//        subnormal; divided by 6 so the largest magnitude is 1; code = 8 sign +
//        magnitude bits.
// Quantization of a block with maximum a: x = fl32(w / a) (0 when a = 0), and
// the code of the nearest level, found by counting the fp32 midpoints of
// adjacent distinct levels strictly below x (a tie takes the lower level; FP4
// uses its +0 code for zero). Two codes per byte, the even element in the low
// nibble. Dequantization: r16(fl32(value[code] * a)) in the 16-bit compute type.
//
// The linear Y = X . Wdeq^T (+ bias) streams the codes once: a workgroup owns
// 16 weight rows and its 16 wavefronts split K. Each lane loads 16 bytes of codes
// (32 codes of one row, one block) per 128-column step, dequantizes them through
// a 16-entry table in LDS and feeds v_mfma_f32_16x16x32_{f16,bf16} with the
// weight rows as A and up to 16 rows of X (read straight from L2) as B. The
// partial sums are added in a fixed order through LDS, the bias is added and Y
// is rounded once.
#include <algorithm>
#include <cmath>

#include "../../include/llmint8.h"
#include "device_util.h"
#include "internal.h"

namespace llmint8 {

// ------------------------------------------------------------------ code books (host)

namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

// Phi^-1(p) for p in [0.5, 1) by Newton's method from 0: Phi is concave on
// [0, inf), so the iterates rise monotonically to the root.
double normal_quantile_upper(double p) {
  const double inv_sqrt_2pi = 1.0 / std::sqrt(2.0 * 3.14159265358979323846);
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double nx = x - (normal_cdf(x) - p) / (inv_sqrt_2pi * std::exp(-0.5 * x * x));
    if (nx == x) break;
    x = nx;
  }
  return x;
}

bool build_code_book_4bit(int quant_type, Code4* out) {
  double v[16];
  if (quant_type == LLMINT8_QUANT_NF4) {
    const double pmax = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
    const double d = normal_quantile_upper(pmax);
    const double step_pos = (0.5 - pmax) / 8.0, step_neg = (0.5 - pmax) / 7.0;
    for (int i = 0; i < 7; ++i) v[i] = -normal_quantile_upper(pmax + i * step_neg) / d;
    v[7] = 0.0;
    for (int i = 0; i < 8; ++i) v[15 - i] = normal_quantile_upper(pmax + i * step_pos) / d;
  } else if (quant_type == LLMINT8_QUANT_FP4) {
    for (int c = 0; c < 16; ++c) {
      const int e = (c >> 1) & 3, m = c & 1;
      const double mag = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
      v[c] = ((c & 8) ? -mag : mag) / 6.0;
    }
  } else {
    return false;
  }
  for (int c = 0; c < 16; ++c) out->value[c] = (float)v[c];
  int order[16], nlev = 0;
  for (int c = 0; c < 16; ++c)
    if (!(out->value[c] == 0.0f && std::signbit(out->value[c]))) order[nlev++] = c;
  std::sort(order, order + nlev, [&](int x, int y) { return out->value[x] < out->value[y]; });
  for (int i = 0; i < 15; ++i) {
    if (i + 1 < nlev) {
      const float sum = out->value[order[i]] + out->value[order[i + 1]];
      out->mid[i] = sum * 0.5f;
    } else {
      out->mid[i] = INFINITY;
    }
  }
  out->rank_lo = out->rank_hi = 0;
  for (int r = 0; r < nlev; ++r) {
    if (r < 8) out->rank_lo |= (uint32_t)order[r] << (4 * r);
    else out->rank_hi |= (uint32_t)order[r] << (4 * (r - 8));
  }
  return true;
}

}  // namespace

// Each book is built once per process (thread-safe static initialisation): the
// NF4 book takes 15 quantile solves, too slow for every call of a decode step.
bool code_book_4bit(int quant_type, Code4* out) {
  static const Code4 nf4 = [] {
    Code4 c{};
    build_code_book_4bit(LLMINT8_QUANT_NF4, &c);
    return c;
  }();
  static const Code4 fp4 = [] {
    Code4 c{};
    build_code_book_4bit(LLMINT8_QUANT_FP4, &c);
    return c;
  }();
  if (quant_type == LLMINT8_QUANT_NF4) *out = nf4;
  else if (quant_type == LLMINT8_QUANT_FP4) *out = fp4;
  else return false;
  return true;
}

// ------------------------------------------------------------------ quantization (load time)

// One pass per block, as the 8-bit codec: LPB lanes per block, VPL 16-byte
// vectors (8 values) per lane in registers, a segmented lane maximum.
template <bool BF16, int LPB, int VPL>
__global__ __launch_bounds__(256) void kq4_blockwise(const uint16_t* __restrict__ w, int n, int nb,
                                                     Code4 book, uint8_t* __restrict__ packed,
                                                     float* __restrict__ absmax) {
  using A16 = Act16<BF16>;
  constexpr int VPB = LPB * VPL;
  constexpr int BPI = 64 / LPB;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPB, li = lane % LPB;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((size_t)n * 2));
  const int nvec = n / 8;
  for (int b0 = wave * BPI; b0 < nb; b0 += nwaves * BPI) {
    const int b = b0 + sub;
    uint4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int vi = b * VPB + i * LPB + li;
      v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rw, vi < nvec ? (uint32_t)vi * 16u : kOobOffset, 0, 0));
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint32_t x[4] = {v[i].x & 0x7fff7fffu, v[i].y & 0x7fff7fffu, v[i].z & 0x7fff7fffu,
                             v[i].w & 0x7fff7fffu};
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(x[j] & 0xffffu, x[j] >> 16));
    }
    m = segment_max_u32<LPB>(m);
    const float a = A16::to_f32(m);
    if (b >= nb) continue;
    if (li == 0) absmax[b] = a;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int vi = b * VPB + i * LPB + li;
      if (vi >= nvec) continue;
      const uint32_t x[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t out = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = A16::to_f32((x[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        const float xn = a > 0.0f ? f / a : 0.0f;
        uint32_t rank = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) rank += book.mid[j] < xn ? 1u : 0u;
        const uint32_t code =
            rank < 8 ? (book.rank_lo >> (4 * rank)) & 15u : (book.rank_hi >> (4 * (rank - 8))) & 15u;
        out |= code << (4 * e);
      }
      reinterpret_cast<uint32_t*>(packed)[vi] = out;
    }
  }
}

// ------------------------------------------------------------------ dequantization

// 8 codes (one word, element e in nibble e) -> 8 16-bit values r16(fl32(c * a)):
// an fp32 multiply per value, then one packed conversion (v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32, round to nearest even) per pair. The empty asm operands
// keep each product an fp32 value: otherwise the compiler may fold multiply and
// conversion into v_fma_mixlo_f16, which rounds the exact product to fp16 once
// and differs from the two roundings whenever fl32(c * a) lands on an fp16
// rounding midpoint.
// Byte SEL of w times 4 in one instruction (an SDWA operand select): the LDS
// byte offset of a table entry whose index sits alone in that byte.
template <int SEL>
__device__ __forceinline__ uint32_t byte_x4(uint32_t w) {
  uint32_t r;
  if constexpr (SEL == 0)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(w));
  else if constexpr (SEL == 1)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w));
  else if constexpr (SEL == 2)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}

template <bool BF16>
__device__ __forceinline__ uint4 dequant8(uint32_t cw, float a, const float* lut) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  // even codes alone in the bytes of `ev`, odd codes in `od`: one instruction per
  // table address instead of a shift and a mask
  const uint32_t ev = cw & 0x0f0f0f0fu, od = (cw >> 4) & 0x0f0f0f0fu;
  const uint32_t ae[4] = {byte_x4<0>(ev), byte_x4<1>(ev), byte_x4<2>(ev), byte_x4<3>(ev)};
  const uint32_t ao[4] = {byte_x4<0>(od), byte_x4<1>(od), byte_x4<2>(od), byte_x4<3>(od)};
  const char* base = reinterpret_cast<const char*>(lut);
  uint32_t o[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float lo = *reinterpret_cast<const float*>(base + ae[p]) * a;
    float hi = *reinterpret_cast<const float*>(base + ao[p]) * a;
    asm volatile("" : "+v"(lo), "+v"(hi));
    if constexpr (BF16) {
      b2 v;
      v.x = (__bf16)lo;
      v.y = (__bf16)hi;
      o[p] = __builtin_bit_cast(uint32_t, v);
    } else {
      h2 v;
      v.x = (_Float16)lo;
      v.y = (_Float16)hi;
      o[p] = __builtin_bit_cast(uint32_t, v);
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <bool BF16>
__global__ __launch_bounds__(256) void kdq4_blockwise(const uint8_t* __restrict__ packed,
                                                      const float* __restrict__ absmax, int n,
                                                      int block_shift, Code4 book,
                                                      uint16_t* __restrict__ out) {
  __shared__ float lut[16];
  if (threadIdx.x == 0) {
#pragma unroll
    for (int c = 0; c < 16; ++c) lut[c] = book.value[c];
  }
  __syncthreads();
  const int nvec = n / 8;
  for (int vi = blockIdx.x * 256 + threadIdx.x; vi < nvec; vi += gridDim.x * 256) {
    const float a = absmax[(vi * 8) >> block_shift];
    const uint32_t cw = reinterpret_cast<const uint32_t*>(packed)[vi];
    reinterpret_cast<uint4*>(out)[vi] = dequant8<BF16>(cw, a, lut);
  }
}

// ------------------------------------------------------------------ the 4-bit linear

constexpr int kN4Waves = 16;  // wavefronts per workgroup, splitting K
constexpr int kN4Unroll = 2;  // 128-column steps in flight per wavefront
// Two 1024-thread workgroups per CU need at most 64 VGPRs per lane (8 waves
// per SIMD); at 65 or more only one fits and the kernel runs ~40% slower.

template <bool BF16>
__global__ __launch_bounds__(kN4Waves * 64) void kn_gemv(FourBitArgs a, Code4 book) {
  using A16 = Act16<BF16>;
  __shared__ float lut[16];
  __shared__ float bias_l[16];
  __shared__ v4f part[kN4Waves][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  if (tid == 0) {
#pragma unroll
    for (int c = 0; c < 16; ++c) lut[c] = book.value[c];
  }
  // the block's 16 bias values, staged before the main loop (read in the
  // epilogue they would hold registers through it)
  if (tid >= 64 && tid < 80) {
    const int nb = n0 + tid - 64;
    bias_l[tid - 64] = a.bias && nb < a.N ? A16::to_f32(a.bias[nb]) : 0.0f;
  }
  const int r = lane & 15, g = lane >> 4;
  const int K = a.K;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const uint32_t nblocks = (uint32_t)(((size_t)a.N * K + (1u << a.block_shift) - 1) >> a.block_shift);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.W4, (uint32_t)a.N * row_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.absmax, nblocks * 4u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, (uint32_t)a.T * (uint32_t)K * 2u);
  const int n = n0 + r, t = t0 + r;
  const bool wvalid = n < a.N, xvalid = t < a.T;
  // lane (r, g) of step s holds row n's codes for columns 128 s + 32 g + [0, 32)
  // (word j: columns + 8 j + [0, 8), the k-slice of MFMA j) and row t's X there
  const uint32_t wbase = (uint32_t)n * row_bytes + 16u * g;
  const uint32_t ebase = (uint32_t)n * (uint32_t)K + 32u * g;
  const uint32_t xbase = ((uint32_t)t * (uint32_t)K + 32u * g) * 2u;
  const int steps = K / 128;
  const int per = (steps + kN4Waves - 1) / kN4Waves;
  const int s0 = min(steps, wave * per), s1 = min(steps, s0 + per);
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();
  struct Steps {
    uint4 cw[kN4Unroll];     // codes
    float sc[kN4Unroll];     // block maxima
    uint4 xb[kN4Unroll][4];  // X fragments
  };
  auto load = [&](Steps& b, int s) {
#pragma unroll
    for (int u = 0; u < kN4Unroll; ++u) {
      const int si = s + u;
      const bool ok = si < s1;
      b.cw[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rw, ok && wvalid ? wbase + 64u * si : kOobOffset, 0, 0));
      b.sc[u] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(
                     ra, ok && wvalid ? ((ebase + 128u * si) >> a.block_shift) * 4u : kOobOffset, 0, 0));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b.xb[u][j] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       rx, ok && xvalid ? xbase + 256u * si + 16u * j : kOobOffset, 0, 0));
    }
  };
  auto compute = [&](const Steps& b) {
#pragma unroll
    for (int u = 0; u < kN4Unroll; ++u) {
      const uint32_t c[4] = {b.cw[u].x, b.cw[u].y, b.cw[u].z, b.cw[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = A16::mma16(dequant8<BF16>(c[j], b.sc[u], lut), b.xb[u][j], acc);
    }
  };
  // written as load + compute per iteration; the compiler rotates the loop so
  // that the next iteration's loads are issued before this one's arithmetic
  for (int s = s0; s < s1; s += kN4Unroll) {
    Steps b;
    load(b, s);
    compute(b);
  }
  part[wave][lane] = acc;
  __syncthreads();
  // threads 0..255: output element (row 4 (l / 16) + v, column l % 16) of the
  // 16 x 16 block, l = tid % 64, v = tid / 64; partial sums added in wave order
  for (int e = tid; e < 256; e += kN4Waves * 64) {
    const int l = e & 63, v = e >> 6;
    float y = 0.0f;
#pragma unroll
    for (int w = 0; w < kN4Waves; ++w) y += part[w][l][v];
    const int nl = 4 * (l >> 4) + v;
    const int nn = n0 + nl, tt = t0 + (l & 15);
    if (nn < a.N && tt < a.T) a.Y[(size_t)tt * a.N + nn] = A16::from_f32(y + bias_l[nl]);
  }
}

// ------------------------------------------------------------------ launchers

namespace {
int log2_exact4(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}
}  // namespace

hipError_t launch_quantize_4bit(const uint16_t* w, bool bf16, int n, int block, const Code4& book,
                                uint8_t* packed, float* absmax, int num_cus, hipStream_t stream) {
  const int nb = (n + block - 1) / block;
  auto grid = [&](int lpb) {
    const int waves = (nb + 64 / lpb - 1) / (64 / lpb);
    return dim3(max(1, min((waves + 3) / 4, num_cus * 16)));
  };
#define L(B, LPB, VPL)                                                                        \
  hipLaunchKernelGGL((kq4_blockwise<B, (LPB), (VPL)>), grid(LPB), dim3(256), 0, stream, w, n, \
                     nb, book, packed, absmax)
#define CASES(B)                           \
  switch (block) {                         \
    case 64: L(B, 8, 1); break;            \
    case 128: L(B, 16, 1); break;          \
    case 256: L(B, 32, 1); break;          \
    case 512: L(B, 64, 1); break;          \
    case 1024: L(B, 64, 2); break;         \
    case 2048: L(B, 64, 4); break;         \
    case 4096: L(B, 64, 8); break;         \
    default: return hipErrorInvalidValue;  \
  }
  if (bf16) {
    CASES(true)
  } else {
    CASES(false)
  }
#undef CASES
#undef L
  return hipGetLastError();
}

hipError_t launch_dequantize_4bit(const uint8_t* packed, const float* absmax, int n, int block,
                                  const Code4& book, uint16_t* out, bool bf16, int num_cus,
                                  hipStream_t stream) {
  const int shift = log2_exact4(block);
  if (shift < 0) return hipErrorInvalidValue;
  const int nvec = n / 8;
  const int grid = max(1, min((nvec + 255) / 256, num_cus * 32));
  if (bf16) {
    hipLaunchKernelGGL(kdq4_blockwise<true>, dim3(grid), dim3(256), 0, stream, packed, absmax, n,
                       shift, book, out);
  } else {
    hipLaunchKernelGGL(kdq4_blockwise<false>, dim3(grid), dim3(256), 0, stream, packed, absmax, n,
                       shift, book, out);
  }
  return hipGetLastError();
}

hipError_t launch_linear_4bit(const FourBitArgs& a, const Code4& book, bool bf16, hipStream_t stream) {
  const dim3 grid((a.N + 15) / 16, (a.T + 15) / 16);
  if (bf16) {
    hipLaunchKernelGGL(kn_gemv<true>, grid, dim3(kN4Waves * 64), 0, stream, a, book);
  } else {
    hipLaunchKernelGGL(kn_gemv<false>, grid, dim3(kN4Waves * 64), 0, stream, a, book);
  }
  return hipGetLastError();
}

}  // namespace llmint8
