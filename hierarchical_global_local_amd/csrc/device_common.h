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

// Operand layout of the fp16 GEMMs ("fragment order").  An M x K operand (weights: N x K) is cut
// into tiles of 16 rows x 32 columns; tile (g, s) holds 512 contiguous elements starting at
// (g * K/32 + s) * 512, and inside it the 8 elements k = 8q .. 8q+7 of row r (q < 4, r < 16) are
// the 16 bytes at element (16 q + r) * 8.  Those 16 bytes are exactly what lane 16 q + r of a wave
// holds as an operand of v_mfma_f32_16x16x32_f16, so one wave reads a whole operand tile with one
// fully contiguous 1 KB load, from HBM, L2 or LDS alike.  Rows are padded to a multiple of 16.
__device__ __forceinline__ size_t frag_off(int m, int k, int K) {
  return ((((size_t)(m >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (m & 15)) << 3) + (k & 7);
}
// Element index of (row m, column k) of an activation operand of width K: fragment order for the
// fp16 path, row-major for the fp32 path.
__device__ __forceinline__ size_t opnd_idx(const f16*, int m, int k, int K) { return frag_off(m, k, K); }
__device__ __forceinline__ size_t opnd_idx(const float*, int m, int k, int K) { return (size_t)m * K + k; }

// Stores 4 consecutive columns (k % 4 == 0) of an activation operand.
__device__ __forceinline__ void store4(float* base, size_t idx, float a, float b, float c, float d) {
  *(float4*)(base + idx) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(f16* base, size_t idx, float a, float b, float c, float d) {
  half4 w;
  w[0] = to_f16(a);
  w[1] = to_f16(b);
  w[2] = to_f16(c);
  w[3] = to_f16(d);
  *(half4*)(base + idx) = w;
}

// Maps the hardware workgroup id to a logical tile index so that the workgroups one XCD
// receives (ids x, x+8, x+16, ... go to XCD x) form one contiguous range of tiles.
__device__ __forceinline__ int xcd_contiguous_tile(int bid, int nb) {
  int per = nb >> 3, rem = nb & 7, x = bid & 7, i = bid >> 3;
  return x * per + min(x, rem) + i;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// GELU, 0.5 x (1 + erf(x / sqrt 2)), with erfc from Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
// t = 1 / (1 + p z), z >= 0, absolute error <= 1.5e-7 (far below the fp16 rounding of the result).
// 1 + erf(x / sqrt 2) is erfc(|x| / sqrt 2) for x < 0 (no cancellation) and 2 - erfc otherwise.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));  // hardware reciprocal (1 ulp)
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
                              0.254829592f);
  const float q = poly * __expf(-z * z);
  return 0.5f * x * (x < 0.f ? q : 2.0f - q);
}

// Order-preserving map of a float to 32 bits, packed with the column so that the 64-bit maximum
// picks the largest value and, among equal values, the lowest column.
__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
  uint32_t u = __float_as_uint(v);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)k << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

}  // namespace bt
