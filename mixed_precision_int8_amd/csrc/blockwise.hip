// Blockwise 8-bit codec on gfx950 ("bitsandbytes" glossary, "What it
// provides": tensors are quantized in blocks that each carry their own scaling
// factor, so an outlier only affects its own block; "bitsandbytes:
// GPU-Accelerated Inference and Training at Lower Bit Depths", 8-bit
// optimizers: block-wise quantization of the optimizer states).
//
//   a[b]  = max |x| over block b (block consecutive elements of the flat tensor)
//   q     = rne(fl32(x * fl32(127 / a[b])))           (0 for a zero block)
//   x'    = fl32(fl32(q * a[b]) / 127), rounded to the input dtype
//
// HBM-bound. Quantization: a wavefront covers 64 / LPB blocks at a time with
// LPB lanes per block and VPL 16-byte vectors per lane kept in registers: one
// pass over the data, a segmented lane reduction of the block maximum, the
// codes written as 8- or 4-byte pieces. Reads use buffer loads over a window
// that ends with the tensor, so a ragged last block reads zeros past the end
// without a branch. Dequantization is a
// flat grid-stride loop over output vectors.
#include "device_util.h"
#include "internal.h"

namespace llmint8 {

// 4 fp32 values -> 4 int8 codes rne(fl32(v * s)) in one word (|v * s| <= 127:
// adding 1.5 * 2^23 leaves the integer, rounded half to even, in the low bits)
__device__ __forceinline__ uint32_t quantize4_f32(const uint4& v, float s) {
  const float f[4] = {__builtin_bit_cast(float, v.x), __builtin_bit_cast(float, v.y),
                      __builtin_bit_cast(float, v.z), __builtin_bit_cast(float, v.w)};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, f[i] * s + 12582912.0f);
  const uint32_t lo = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// fl32(p / 127) for any fp32 p: the binary64 product with the binary64
// reciprocal is within 2^-52 (relative) of p / 127, while p / 127 is at least
// 2^-32 (relative) away from every midpoint between fp32 neighbours, so the
// final rounding to fp32 is the correctly rounded quotient.
__device__ __forceinline__ float div127(float p) { return (float)((double)p * (1.0 / 127.0)); }

// Every code and every dequantized value is written once and not read again by
// the kernel: the stores are non-temporal (their lines go to memory without
// lingering in L2). Measured on 45 M elements, three copies cycled:
// fp16 -> codes 26.7 -> 23.7 us, codes -> fp16 26.1 -> 20.7 us, codes -> fp32
// 44.0 -> 34.8 us, fp32 -> codes 44.0 -> 40.8 us, and 38.5 us with the fp32
// input read non-temporally as well (the same hint on the other loads was
// slower).
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

template <bool F32, int LPB, int VPL>
__global__ __launch_bounds__(256) void kq_blockwise(const void* __restrict__ x, int n, int nb,
                                                    int8_t* __restrict__ q, float* __restrict__ absmax) {
  constexpr int E = F32 ? 4 : 8;  // elements per 16-byte vector
  constexpr int kLoadPolicy = F32 ? 2 : 0;  // buffer cache policy: non-temporal reads of fp32 input
  constexpr int VPB = LPB * VPL;  // vectors per block
  constexpr int BPI = 64 / LPB;   // blocks per wavefront iteration
  static_assert(BPI * VPB * 16 == 1024 * VPL, "an iteration's window is codec_window_bytes(VPL)");
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPB, li = lane % LPB;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int nvec = n / E;
  for (int b0 = wave * BPI; b0 < nb; b0 += nwaves * BPI) {
    const int b = b0 + sub;
    // one window per iteration: the BPI blocks from b0, cut at the end of the
    // tensor (codec_window_bytes(VPL) bytes at most); vectors past it read as zero
    const int v0 = b0 * VPB;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(
        static_cast<const char*>(x) + (size_t)v0 * 16u, (uint32_t)min(BPI * VPB, nvec - v0) * 16u);
    uint4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int vl = sub * VPB + i * LPB + li;  // vector within the window
      v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)vl * 16u, 0, kLoadPolicy));
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (F32) {
        m = max(m, max(max(v[i].x & 0x7fffffffu, v[i].y & 0x7fffffffu),
                       max(v[i].z & 0x7fffffffu, v[i].w & 0x7fffffffu)));
      } else {
        const uint32_t w[4] = {v[i].x & 0x7fff7fffu, v[i].y & 0x7fff7fffu, v[i].z & 0x7fff7fffu,
                               v[i].w & 0x7fff7fffu};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0xffffu, w[j] >> 16));
      }
    }
    m = segment_max_u32<LPB>(m);
    const float a = F32 ? __builtin_bit_cast(float, m) : half_bits_to_float(m);
    const float s = a > 0.0f ? 127.0f / a : 0.0f;
    if (b < nb) {
      if (li == 0) absmax[b] = a;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int vi = b * VPB + i * LPB + li;
        if (vi >= nvec) continue;
        if (F32) {
          __builtin_nontemporal_store(quantize4_f32(v[i], s), reinterpret_cast<uint32_t*>(q) + vi);
        } else {
          const uint2 c = quantize8_masked(v[i], s, 0xffffffffu, 0xffffffffu);
          __builtin_nontemporal_store(v2u{c.x, c.y}, reinterpret_cast<v2u*>(q) + vi);
        }
      }
    }
  }
}

// Dequantization needs no reduction, so it runs flat: a grid-stride loop over
// 16-byte output vectors, each reading its codes (8 or 4 bytes) and its
// block's maximum.
template <bool F32>
__global__ __launch_bounds__(256) void kdq_blockwise(const int8_t* __restrict__ q,
                                                     const float* __restrict__ absmax, int n,
                                                     int block_shift, void* __restrict__ out) {
  constexpr int E = F32 ? 4 : 8;
  const int nvec = n / E;
  for (int vi = blockIdx.x * 256 + threadIdx.x; vi < nvec; vi += gridDim.x * 256) {
    const float a = absmax[(vi * E) >> block_shift];
    if (F32) {
      const uint32_t c = reinterpret_cast<const uint32_t*>(q)[vi];
      uint4 o;
      uint32_t* po = &o.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = (float)(int)(int8_t)((c >> (8 * j)) & 0xffu) * a;
        po[j] = __builtin_bit_cast(uint32_t, div127(p));
      }
      __builtin_nontemporal_store(__builtin_bit_cast(v4i, o), reinterpret_cast<v4i*>(out) + vi);
    } else {
      const uint2 c = reinterpret_cast<const uint2*>(q)[vi];
      const uint32_t w[2] = {c.x, c.y};
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = (float)(int)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xffu) * a;
        h[j] = float_to_half_bits(div127(p));
      }
      uint4 o;
      o.x = h[0] | (h[1] << 16);
      o.y = h[2] | (h[3] << 16);
      o.z = h[4] | (h[5] << 16);
      o.w = h[6] | (h[7] << 16);
      __builtin_nontemporal_store(__builtin_bit_cast(v4i, o), reinterpret_cast<v4i*>(out) + vi);
    }
  }
}

namespace {
int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}
int codec_grid(int nb, int blocks_per_wave_iter, int num_cus) {
  const int waves = (nb + blocks_per_wave_iter - 1) / blocks_per_wave_iter;
  const int wgs = (waves + 3) / 4;
  return max(1, min(wgs, num_cus * 16));
}
}  // namespace

#define LLMINT8_BW_CASES(F32, E)                                                           \
  switch (block) {                                                                         \
    case 64: L(F32, 64 / E < 64 ? 64 / E : 64, 64 / E <= 64 ? 1 : 64 / E / 64); break;     \
    case 128: L(F32, 128 / E < 64 ? 128 / E : 64, 128 / E <= 64 ? 1 : 128 / E / 64); break; \
    case 256: L(F32, 256 / E < 64 ? 256 / E : 64, 256 / E <= 64 ? 1 : 256 / E / 64); break; \
    case 512: L(F32, 512 / E < 64 ? 512 / E : 64, 512 / E <= 64 ? 1 : 512 / E / 64); break; \
    case 1024: L(F32, 64, 1024 / E / 64); break;                                           \
    case 2048: L(F32, 64, 2048 / E / 64); break;                                           \
    case 4096: L(F32, 64, 4096 / E / 64); break;                                           \
    default: return hipErrorInvalidValue;                                                  \
  }

hipError_t launch_quantize_blockwise(const void* x, bool f32, int n, int block, int8_t* q,
                                     float* absmax, int num_cus, hipStream_t stream) {
  const int nb = (n + block - 1) / block;
#define L(F, LPB, VPL)                                                                     \
  hipLaunchKernelGGL((kq_blockwise<F, (LPB), (VPL)>), dim3(codec_grid(nb, 64 / (LPB), num_cus)), \
                     dim3(256), 0, stream, x, n, nb, q, absmax)
  if (f32) {
    LLMINT8_BW_CASES(true, 4)
  } else {
    LLMINT8_BW_CASES(false, 8)
  }
#undef L
  return hipGetLastError();
}
#undef LLMINT8_BW_CASES

hipError_t launch_dequantize_blockwise(const int8_t* q, const float* absmax, int n, int block,
                                       void* out, bool f32, int num_cus, hipStream_t stream) {
  const int shift = log2_exact(block);
  if (shift < 0) return hipErrorInvalidValue;
  const int nvec = n / (f32 ? 4 : 8);
  const int grid = max(1, min((nvec + 255) / 256, num_cus * 32));
  if (f32) {
    hipLaunchKernelGGL(kdq_blockwise<true>, dim3(grid), dim3(256), 0, stream, q, absmax, n, shift, out);
  } else {
    hipLaunchKernelGGL(kdq_blockwise<false>, dim3(grid), dim3(256), 0, stream, q, absmax, n, shift, out);
  }
  return hipGetLastError();
}

}  // namespace llmint8
