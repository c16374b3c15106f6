// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ranges.h"

namespace llmint8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Buffer resource word 3 for raw (untyped) buffers on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  // v_cvt_f16_f32 rounds to nearest even in the default mode.
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);  // exact: bf16 is the top half of fp32
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  // v_cvt_pk_bf16_f32 rounds to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Maximum over aligned segments of LPB lanes (a power of two up to 64).
template <int LPB>
__device__ __forceinline__ uint32_t segment_max_u32(uint32_t v) {
#pragma unroll
  for (int off = LPB / 2; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// |x| codes of 8 16-bit values packed in a uint4, as 4 packed u16 pairs.
__device__ __forceinline__ void abs_codes(const uint4& v, v2u16 out[4]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = w[i] & 0x7fff7fffu;
    out[i] = __builtin_bit_cast(v2u16, a);
  }
}

// 4-bit mask -> 4 bytes of 0xff where the bit is set.
__device__ __forceinline__ uint32_t expand4(uint32_t b4) {
  return ((b4 * 0x00204081u) & 0x01010101u) * 0xffu;
}

// Quantize 8 fp16 values (uint4) with scale s: rne(fl32(x * s)), ANDed with
// the byte masks m0 (codes 0-3) and m1 (codes 4-7). fl32(x * s) is
// fma(x, s, +0) (v_fma_mix_f32 takes the fp16 operand directly); adding
// 1.5 * 2^23 then rounds it to an integer (ties to even) held in the low
// mantissa bits, whose low byte is the two's-complement int8 code while
// |x * s| < 2^22. v_perm_b32 gathers the bytes.
__device__ __forceinline__ uint2 quantize8_masked(const uint4& v, float s, uint32_t m0, uint32_t m1) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t h = (uint16_t)((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
    const float p = __builtin_fmaf((float)__builtin_bit_cast(_Float16, h), s, 0.0f);
    r[i] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
  }
  // perm(hi, lo, sel): selector bytes 0-3 pick bytes of `lo`, 4-7 of `hi`, 12 gives 0
  const uint32_t b01 = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
  const uint32_t b23 = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
  const uint32_t b45 = __builtin_amdgcn_perm(r[5], r[4], 0x0c0c0400u);
  const uint32_t b67 = __builtin_amdgcn_perm(r[7], r[6], 0x0c0c0400u);
  return make_uint2(__builtin_amdgcn_perm(b23, b01, 0x05040100u) & m0,
                    __builtin_amdgcn_perm(b67, b45, 0x05040100u) & m1);
}

// quantize8_masked for 8 bf16 values: each value is exact in fp32 (a shift),
// fl32(x * s) is one fp32 multiply, then the same rounding and byte gathering.
__device__ __forceinline__ uint2 quantize8_masked_bf16(const uint4& v, float s, uint32_t m0,
                                                       uint32_t m1) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t bits = (i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16);
    const float p = __builtin_bit_cast(float, bits) * s;
    r[i] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
  }
  const uint32_t b01 = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
  const uint32_t b23 = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
  const uint32_t b45 = __builtin_amdgcn_perm(r[5], r[4], 0x0c0c0400u);
  const uint32_t b67 = __builtin_amdgcn_perm(r[7], r[6], 0x0c0c0400u);
  return make_uint2(__builtin_amdgcn_perm(b23, b01, 0x05040100u) & m0,
                    __builtin_amdgcn_perm(b67, b45, 0x05040100u) & m1);
}

// The 16-bit activation type: fp16 or bf16. Magnitude codes (value & 0x7fff)
// order like the values for both, so outlier tests and maxima run on codes
// unchanged; only the conversions, the quantizer's operand form and the MFMA
// flavour of the 16-bit outlier product differ.
template <bool BF16>
struct Act16 {
  static __device__ __forceinline__ float to_f32(uint32_t h) {
    if constexpr (BF16) return bf16_bits_to_float(h);
    else return half_bits_to_float(h);
  }
  static __device__ __forceinline__ uint16_t from_f32(float f) {
    if constexpr (BF16) return float_to_bf16_bits(f);
    else return float_to_half_bits(f);
  }
  // two values rounded to the type and packed, x0 in the low half
  static __device__ __forceinline__ uint32_t pack2(float x0, float x1) {
    if constexpr (BF16) {
      typedef __bf16 v2 __attribute__((ext_vector_type(2)));
      return __builtin_bit_cast(uint32_t, v2{(__bf16)x0, (__bf16)x1});
    } else {
      typedef _Float16 v2 __attribute__((ext_vector_type(2)));
      return __builtin_bit_cast(uint32_t, v2{(_Float16)x0, (_Float16)x1});
    }
  }
  static __device__ __forceinline__ uint2 quantize8(const uint4& v, float s, uint32_t m0, uint32_t m1) {
    if constexpr (BF16) return quantize8_masked_bf16(v, s, m0, m1);
    else return quantize8_masked(v, s, m0, m1);
  }
  // 32x32 output block, k = 16 (8 values per lane of a and b)
  static __device__ __forceinline__ v16f_t mma32(const uint4& a, const uint4& b, v16f_t c) {
    if constexpr (BF16)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
  // 16x16 output block, k = 32 (8 values per lane of a and b)
  static __device__ __forceinline__ v4f mma16(const uint4& a, const uint4& b, v4f c) {
    if constexpr (BF16)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
};

// Maximum over the 64 lanes of two packed u16 values, result in every lane
// (DPP row reductions, then the row broadcasts, then lane 63).
__device__ __forceinline__ uint32_t wave_max_u16x2(uint32_t v) {
  auto pkmax = [](uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2u16, a),
                                                                  __builtin_bit_cast(v2u16, b)));
  };
  v = pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  v = pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = pkmax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum across the 64 lanes of a wavefront: shifts within each
// 16-lane row (lanes without a source add 0), then the running totals of rows
// 0 and 0..1 are broadcast forward with row_bcast15 / row_bcast31.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

}  // namespace llmint8
