// Device helpers shared by the kernels of libbt (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "bt_internal.h"

namespace bt {

struct bf16_t {
  uint16_t bits;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4_ __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const f16* p) { return (float)*p; }
__device__ __forceinline__ float load_f32(const bf16_t* p) { return __uint_as_float((uint32_t)p->bits << 16); }

// fp16 stores saturate at the largest finite value instead of overflowing to infinity.
__device__ __forceinline__ f16 to_f16(float x) { return (f16)fminf(fmaxf(x, -65504.f), 65504.f); }
__device__ __forceinline__ void store_from_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_from_f32(f16* p, float v) { *p = to_f16(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ f16 from_f32<f16>(float v) { return to_f16(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// exact-erf GELU
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Order-preserving map of a float to 32 bits, packed with the column so that the 64-bit maximum
// picks the largest value and, among equal values, the lowest column.
__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
  uint32_t u = __float_as_uint(v);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)k << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

}  // namespace bt
