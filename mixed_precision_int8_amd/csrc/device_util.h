// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llmint8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt == 0 only.
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);

// Buffer resource word 3 for raw (untyped) buffers on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;
// A buffer offset that is always out of range: loads from it return zero.
constexpr uint32_t kOobOffset = 0x80000000u;

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

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// |x| codes of 8 fp16 values packed in a uint4, as 4 packed u16 pairs.
__device__ __forceinline__ void abs_codes(const uint4& v, v2u16 out[4]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = w[i] & 0x7fff7fffu;
    out[i] = __builtin_bit_cast(v2u16, a);
  }
}

// Quantize 8 fp16 values (uint4) with scale s: rne(fl32(x * s)); values whose
// bit in `skip` is set give 0. Returns the 8 int8 codes packed in a uint2.
__device__ __forceinline__ uint2 quantize8(const uint4& v, float s, uint32_t skip) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = (w[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
    const float x = half_bits_to_float(h);
    int q = (int)__builtin_rintf(x * s);
    q = ((skip >> i) & 1u) ? 0 : q;
    out[i >> 2] |= ((uint32_t)q & 0xffu) << ((i & 3) * 8);
  }
  return make_uint2(out[0], out[1]);
}

}  // namespace llmint8
