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

// Set to 1 by any fp16 conversion of an activation or cache value that is out of fp16's range or
// not finite (and is therefore clamped).  One flag per translation unit (each kernel file has its
// own copy); BT_DEFINE_CLAMP_FLAG_ACCESS gives the host a reader for it.
static __device__ unsigned int g_clamped;

// fp16 stores saturate at the largest finite value instead of overflowing to infinity.  (fmaxf and
// fminf return the other operand for a NaN, so a NaN becomes -65504.)  This form does not record
// the clamp: it is for values that cannot leave fp16's range by construction (attention outputs,
// convex combinations of fp16 values; probabilities; queries scaled by at most 1).
__device__ __forceinline__ f16 to_f16_bounded(float x) { return (f16)fminf(fmaxf(x, -65504.f), 65504.f); }

// The same conversion, recording a clamp (magnitude beyond 65504, or NaN) in the flag.
__device__ __forceinline__ f16 to_f16(float x) {
  if (!(fabsf(x) <= 65504.f)) g_clamped = 1u;
  return to_f16_bounded(x);
}

// Branch-free form for kernels that convert many values per thread: trk keeps the largest
// magnitude seen, as its bits shifted left by one (the sign dropped; infinities and NaN compare above
// every finite value), and clamp_note(trk) at the end of the kernel sets the flag once.
__device__ __forceinline__ f16 to_f16_trk(float x, uint32_t& trk) {
  trk = max(trk, __float_as_uint(x) << 1);
  return to_f16_bounded(x);
}
__device__ __forceinline__ void clamp_note(uint32_t trk) {
  if (trk > (0x477fe000u << 1)) g_clamped = 1u;  // 0x477fe000: the bits of 65504.0f
}

// Host access to the translation unit's clamp flag: copies it to *value and, with reset, clears it
// (both enqueued on st; the caller synchronises before reading *value).
#define BT_DEFINE_CLAMP_FLAG_ACCESS(fn)                                                           \
  hipError_t fn(unsigned int* value, bool reset, hipStream_t st) {                                \
    hipError_t e = hipMemcpyFromSymbolAsync(value, HIP_SYMBOL(g_clamped), sizeof(unsigned int), 0, \
                                            hipMemcpyDeviceToHost, st);                           \
    if (e != hipSuccess || !reset) return e;                                                      \
    static const unsigned int zero = 0u;                                                          \
    return hipMemcpyToSymbolAsync(HIP_SYMBOL(g_clamped), &zero, sizeof(unsigned int), 0,          \
                                  hipMemcpyHostToDevice, st);                                     \
  }
__device__ __forceinline__ void store_from_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_from_f32(f16* p, float v) { *p = to_f16(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ f16 from_f32<f16>(float v) { return to_f16(v); }

// Sum over each aligned group of 8 lanes on the DPP network (no LDS crossbar round trips): swap
// neighbours, swap pairs, then add the half-row mirror (lane i of a group reads lane 7 - i, which
// holds the other quad's sum).  The pairing is that of xor-shuffles by 1, 2 and 4, so every lane of
// the group gets the same, bit-identical sum.
__device__ __forceinline__ float sum8(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half mirror
  return v;
}
// Sum over each aligned group of N lanes (N = 8 or 16 on the DPP network, the 16-lane step adding
// the row mirror: lane i of a row reads lane 15 - i, the other half's sum; otherwise xor-shuffles),
// with the pairing of xor-shuffles by 1, 2, 4, ... so every lane of a group holds the same sum.
template <int N>
__device__ __forceinline__ float sum_lanes(float v) {
  if constexpr (N == 8) {
    return sum8(v);
  } else if constexpr (N == 16) {
    v = sum8(v);
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // row mirror
  } else {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
  }
}

// One DPP move of a 32-bit value: lanes of the rows in ROWS read lane CTRL's source, the others
// keep `old`.  0x142 / 0x143 broadcast lane 15 of each row to the next row / lane 31 to rows 2-3.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}

// Sum and maximum over the whole wave, in every lane: the 16-lane sums of sum_lanes, then row 1 adds
// row 0's and row 3 row 2's, row 3 adds row 1's (rows 0-1), and lane 63 is broadcast.  The pairing
// at every level is that of an xor butterfly, so the result does not depend on the lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = sum_lanes<16>(v);
  v += __uint_as_float(dpp_u32<0x142, 0xA>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x143, 0x8>(0u, __float_as_uint(v)));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  const uint32_t u = __float_as_uint(v);
  v = fmaxf(v, __uint_as_float(dpp_u32<0xB1, 0xF>(u, u)));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x4E, 0xF>(__float_as_uint(v), __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x141, 0xF>(__float_as_uint(v), __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x140, 0xF>(__float_as_uint(v), __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x142, 0xA>(__float_as_uint(v), __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x143, 0x8>(__float_as_uint(v), __float_as_uint(v))));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
// Largest 64-bit key of the wave, in every lane (the same levels as wave_max on both halves).
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_max_u64(unsigned long long v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const unsigned long long o = ((unsigned long long)dpp_u32<CTRL, ROWS>(hi, hi) << 32) | dpp_u32<CTRL, ROWS>(lo, lo);
  return o > v ? o : v;
}
// Largest 64-bit key over each aligned group of N lanes (N = 2, 4, 8, 16), in every lane of it.
template <int N>
__device__ __forceinline__ unsigned long long max_lanes_u64(unsigned long long v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "lane group");
  v = dpp_max_u64<0xB1, 0xF>(v);
  if constexpr (N >= 4) v = dpp_max_u64<0x4E, 0xF>(v);
  if constexpr (N >= 8) v = dpp_max_u64<0x141, 0xF>(v);
  if constexpr (N >= 16) v = dpp_max_u64<0x140, 0xF>(v);
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = dpp_max_u64<0xB1, 0xF>(v);
  v = dpp_max_u64<0x4E, 0xF>(v);
  v = dpp_max_u64<0x141, 0xF>(v);
  v = dpp_max_u64<0x140, 0xF>(v);
  v = dpp_max_u64<0x142, 0xA>(v);
  v = dpp_max_u64<0x143, 0x8>(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63), hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
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
// ... with the clamp recorded in a tracker (see to_f16_trk)
__device__ __forceinline__ void store4(float* base, size_t idx, float a, float b, float c, float d, uint32_t&) {
  store4(base, idx, a, b, c, d);
}
__device__ __forceinline__ void store4(f16* base, size_t idx, float a, float b, float c, float d, uint32_t& trk) {
  half4 w;
  w[0] = to_f16_trk(a, trk);
  w[1] = to_f16_trk(b, trk);
  w[2] = to_f16_trk(c, trk);
  w[3] = to_f16_trk(d, trk);
  *(half4*)(base + idx) = w;
}
// ... of values bounded by construction (attention outputs)
__device__ __forceinline__ void store4_bounded(float* base, size_t idx, float a, float b, float c, float d) {
  store4(base, idx, a, b, c, d);
}
__device__ __forceinline__ void store4_bounded(f16* base, size_t idx, float a, float b, float c, float d) {
  half4 w;
  w[0] = to_f16_bounded(a);
  w[1] = to_f16_bounded(b);
  w[2] = to_f16_bounded(c);
  w[3] = to_f16_bounded(d);
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
