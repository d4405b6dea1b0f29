// Skinny GEMM of libbt for decode shapes: C[M][N] = A[M][K] * W[N][K]^T with M <= 256 rows (the
// batch of a decode step), fp16 operands in fragment order (see frag_off), fp32 accumulation,
// the same fused epilogues as the LDS-tiled kernels of gemm.hip.
#include <algorithm>

#include "bt_internal.h"
#include "device_common.h"

namespace bt {

// For M <= 256 rows (the batch of a decode step) the GEMM is a stream over the weights.  One
// workgroup owns a slab of 16*NG output columns for ALL rows: MW waves along M (MG 16-row groups
// each) times KW waves along K.  Both operands are in fragment order and go straight from memory
// into MFMA operand registers (one contiguous 1 KB load per 16 x 32 tile, no LDS on the operand
// path), DEPTH K steps in flight per wave.  The KW partial tiles are summed once through LDS, in a
// fixed order, and the epilogue writes 8 consecutive columns per thread.  gridDim.y > 1 splits K
// over workgroups (EPI_RESID only): the partial products go to ep.part and the consumer adds them.
template <int MG, int MW, int NG, int KW, int MODE, int DEPTH = 2>
__global__ __launch_bounds__(64 * MW * KW) void k_gemm_skinny(const f16* __restrict__ A1, const f16* __restrict__ A2,
                                                              const f16* __restrict__ W, int M, int N, int K, Epi ep) {
  constexpr int R = 16 * MG * MW, C = 16 * NG, CLD = C + 4, NT = 64 * MW * KW;
  __shared__ __attribute__((aligned(16))) float red[KW * R * CLD];
  const int KS = K / 32, mgs = (M + 15) / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mw = wave % MW, kw = wave / MW;
  const int ng0 = blockIdx.x * NG, n0 = ng0 * 16;
  const f16* __restrict__ A = (MODE == EPI_QKV_GELU && n0 >= ep.n_split) ? A2 : A1;
  // K steps of this workgroup (split blockIdx.y of gridDim.y), then of this wave
  const int S = gridDim.y, sper = (KS + S - 1) / S;
  const int sb = blockIdx.y * sper, se = min(KS, sb + sper);
  const int wper = (se - sb + KW - 1) / KW;
  const int kb = min(se, sb + kw * wper), ke = min(se, kb + wper);

  const f16* ap[MG];
#pragma unroll
  for (int i = 0; i < MG; ++i) ap[i] = A + ((size_t)min(mw * MG + i, mgs - 1) * KS * 64 + lane) * 8;
  const f16* wp[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) wp[j] = W + ((size_t)(ng0 + j) * KS * 64 + lane) * 8;

  float4_ acc[MG][NG];
#pragma unroll
  for (int i = 0; i < MG; ++i)
#pragma unroll
    for (int j = 0; j < NG; ++j) acc[i][j] = float4_{0.f, 0.f, 0.f, 0.f};
  half8 ra[DEPTH][MG], rw[DEPTH][NG];
  auto load = [&](int s, int ks) {
#pragma unroll
    for (int i = 0; i < MG; ++i) ra[s][i] = *(const half8*)(ap[i] + (size_t)ks * 512);
#pragma unroll
    for (int j = 0; j < NG; ++j) rw[s][j] = *(const half8*)(wp[j] + (size_t)ks * 512);
  };
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
    if (kb + s < ke) load(s, kb + s);
  for (int k0 = kb; k0 < ke; k0 += DEPTH) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      if (k0 + s < ke) {
#pragma unroll
        for (int i = 0; i < MG; ++i)
#pragma unroll
          for (int j = 0; j < NG; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ra[s][i], rw[s][j], acc[i][j], 0, 0, 0);
        if (k0 + s + DEPTH < ke) load(s, k0 + s + DEPTH);
      }
    }
  }
  // partial tiles of the KW waves -> LDS [kw][row][col]
#pragma unroll
  for (int i = 0; i < MG; ++i)
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[(kw * R + (mw * MG + i) * 16 + 4 * (lane >> 4) + e) * CLD + j * 16 + (lane & 15)] = acc[i][j][e];
  __syncthreads();

  // epilogue: item = (row, 8 consecutive columns); every thread runs the same number of items so
  // that the row-wise shuffles of EPI_ARGMAX see whole groups
  constexpr int CPR = C / 8, ITEMS = R * CPR, ITER = (ITEMS + NT - 1) / NT;
  static_assert(64 % CPR == 0 && NT % 64 == 0, "a row's items sit in one wave");
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int it = 0; it < ITER; ++it) {
    const int item = tid + it * NT;
    const int rl = min(item, ITEMS - 1) / CPR, cl = (min(item, ITEMS - 1) % CPR) * 8;
    const int row = rl, col = n0 + cl;
    const bool live = item < ITEMS && row < M;
    float v[8];
    {
      float4 a0 = *(const float4*)&red[rl * CLD + cl], a1 = *(const float4*)&red[rl * CLD + cl + 4];
#pragma unroll
      for (int q = 1; q < KW; ++q) {
        const float4 b0 = *(const float4*)&red[(q * R + rl) * CLD + cl];
        const float4 b1 = *(const float4*)&red[(q * R + rl) * CLD + cl + 4];
        a0.x += b0.x, a0.y += b0.y, a0.z += b0.z, a0.w += b0.w;
        a1.x += b1.x, a1.y += b1.y, a1.z += b1.z, a1.w += b1.w;
      }
      v[0] = a0.x, v[1] = a0.y, v[2] = a0.z, v[3] = a0.w, v[4] = a1.x, v[5] = a1.y, v[6] = a1.z, v[7] = a1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= ep.wscale;
    if constexpr (MODE == EPI_QKV_GELU) {
      const float4 c0 = *(const float4*)(ep.bias + col), c1 = *(const float4*)(ep.bias + col + 4);
      v[0] += c0.x, v[1] += c0.y, v[2] += c0.z, v[3] += c0.w, v[4] += c1.x, v[5] += c1.y, v[6] += c1.z, v[7] += c1.w;
      if (live) {
        half8 w;
        if (n0 >= ep.n_split) {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16(gelu_erf(v[e]));
          *(half8*)((f16*)ep.out1 + frag_off(row, ep.act_col0 + (col - ep.n_split), ep.ld1)) = w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16(v[e]);
          *(half8*)((f16*)ep.out0 + (size_t)row * ep.ld0 + col) = w;
        }
      }
    } else if constexpr (MODE == EPI_RESID) {
      if (S > 1) {
        float* p = ep.part + ((size_t)blockIdx.y * M + row) * N + col;
        if (live) {
          *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
          *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
      } else {
        float* x = (float*)ep.out0 + (size_t)min(row, M - 1) * ep.ld0 + col;
        const float4 x0 = *(const float4*)x, x1 = *(const float4*)(x + 4);
        const float4 c0 = *(const float4*)(ep.bias + col), c1 = *(const float4*)(ep.bias + col + 4);
        const float4 d0 = *(const float4*)(ep.bias2 + col), d1 = *(const float4*)(ep.bias2 + col + 4);
        if (live) {
          *(float4*)x = make_float4(x0.x + (v[0] + c0.x + d0.x), x0.y + (v[1] + c0.y + d0.y),
                                    x0.z + (v[2] + c0.z + d0.z), x0.w + (v[3] + c0.w + d0.w));
          *(float4*)(x + 4) = make_float4(x1.x + (v[4] + c1.x + d1.x), x1.y + (v[5] + c1.y + d1.y),
                                          x1.z + (v[6] + c1.z + d1.z), x1.w + (v[7] + c1.w + d1.w));
        }
      }
    } else if constexpr (MODE == EPI_STORE) {
      float b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (ep.bias) {
        const float4 c0 = *(const float4*)(ep.bias + col), c1 = *(const float4*)(ep.bias + col + 4);
        b[0] = c0.x, b[1] = c0.y, b[2] = c0.z, b[3] = c0.w, b[4] = c1.x, b[5] = c1.y, b[6] = c1.z, b[7] = c1.w;
      }
      if (live) {
        float* o = (float*)ep.out0 + (size_t)row * ep.ld0 + col;
        *(float4*)o = make_float4(v[0] + b[0], v[1] + b[1], v[2] + b[2], v[3] + b[3]);
        *(float4*)(o + 4) = make_float4(v[4] + b[4], v[5] + b[5], v[6] + b[6], v[7] + b[7]);
      }
    } else {  // EPI_ARGMAX
      unsigned long long best = 0ull;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned long long k = argmax_key(v[e], col + e);
        if (col + e < ep.n_valid && k > best) best = k;
      }
      if (live && ep.out0) {
        float* o = (float*)ep.out0 + (size_t)row * ep.ld0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < ep.n_valid) o[col + e] = v[e];
      }
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) {
        const unsigned long long other = shfl_xor_u64(best, o);
        best = other > best ? other : best;
      }
      if (live && cl == 0) ep.keys[(size_t)row * ep.keys_ld + blockIdx.x] = best;
    }
  }
}

template <int MG, int MW, int NG, int KW>
static hipError_t launch_skinny_cfg(const void* A1, const void* A2, const void* W, int M, int N, int K, EpiMode mode,
                                    const Epi& ep, int S, hipStream_t st) {
  if (mode == EPI_ARGMAX && ep.nparts_out) *ep.nparts_out = N / (16 * NG);
  dim3 grid(N / (16 * NG), S), block(64 * MW * KW);
  const f16 *a1 = (const f16*)A1, *a2 = (const f16*)A2, *w = (const f16*)W;
  switch (mode) {
    case EPI_QKV_GELU:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_QKV_GELU>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_RESID>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_STORE>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_ARGMAX>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
  }
  return hipGetLastError();
}


// Which skinny configuration a GEMM of this shape runs (also the split count the consumer of
// EPI_RESID partials folds).  From a sweep of 34 configurations per decode shape on MI355X with
// the weights streamed from HBM: up to 4 row groups per wave, waves along M for more rows (16, 32,
// 64, 128, 256-row workgroups), K over 8 waves (4 when there are 2-4 row waves), 2 column groups
// per wave (4 at 128 rows when N is wide); the [out|down] GEMM (N = d_model) splits K over
// workgroups until ~192 of them stream the weights.
SkinnyPlan skinny_plan(int M, int N, int K, EpiMode mode) {
  SkinnyPlan p{};
  p.splits = 1;
  // The classifier of a batch above 128 rows has enough MFMA work to prefer the LDS-tiled kernel.
  p.ok = M >= 1 && M <= 256 && N % 32 == 0 && K % 32 == 0 && !(mode == EPI_ARGMAX && M > 128);
  if (!p.ok) return p;
  const int mgt = (M + 15) / 16;
  if (mgt <= 1) p.mg = 1, p.mw = 1;
  else if (mgt <= 2) p.mg = 2, p.mw = 1;
  else if (mgt <= 4) p.mg = 4, p.mw = 1;
  else if (mgt <= 8) p.mg = 4, p.mw = 2;
  else p.mg = 4, p.mw = 4;
  p.kw = p.mw == 1 ? 8 : 4;
  p.ng = (p.mw == 2 && N % 64 == 0 && N / 64 >= 224) ? 4 : 2;
  const int slabs = N / (16 * p.ng), ks = K / 32;
  if (mode == EPI_RESID && slabs < 128) {
    int s = std::min(16, (192 + slabs - 1) / slabs);
    s = std::max(1, std::min(s, ks / p.kw));
    const int per = (ks + s - 1) / s;
    p.splits = (ks + per - 1) / per;  // every split owns at least one K step
  }
  return p;
}

hipError_t launch_gemm_skinny(const SkinnyPlan& p, const void* A1, const void* A2, const void* W, int M, int N, int K,
                              EpiMode mode, const Epi& ep, hipStream_t st) {
  const int S = mode == EPI_RESID ? ep.splits : 1;
#define BT_SKINNY(MG, MW, NG, KW) \
  if (p.mg == MG && p.mw == MW && p.ng == NG && p.kw == KW)   \
    return launch_skinny_cfg<MG, MW, NG, KW>(A1, A2, W, M, N, K, mode, ep, S, st);
  BT_SKINNY(1, 1, 2, 8)
  BT_SKINNY(2, 1, 2, 8)
  BT_SKINNY(4, 1, 2, 8)
  BT_SKINNY(4, 2, 2, 4)
  BT_SKINNY(4, 2, 4, 4)
  BT_SKINNY(4, 4, 2, 4)
#undef BT_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace bt
