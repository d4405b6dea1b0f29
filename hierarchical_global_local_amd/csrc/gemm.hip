// GEMM kernels of libbt: C[M][N] = A[M][K] * W[N][K]^T with fused epilogues.
//
// fp16 operands: LDS-tiled MFMA (v_mfma_f32_16x16x32_f16, fp32 accumulation), 256 threads
// as a WM x WN grid of waves, BK = 64 with a double-buffered LDS stage fed by 16-byte global
// loads held in registers one K-step ahead.  Workgroup ids are remapped so that each of the 8
// XCDs walks a contiguous range of output tiles, grouped 8 M-tiles at a time, so that A and W
// tiles are re-read from that XCD's L2 rather than from HBM.
// fp32 operands (BT_FP32): a plain LDS-tiled VALU kernel with the same epilogues.
#include <cstdlib>

#include "bt_internal.h"
#include "device_common.h"

namespace bt {

template <int MODE, typename T>
__device__ __forceinline__ void epi_store(const Epi& ep, int row, int col, float v) {
  if constexpr (MODE == EPI_QKV_GELU) {
    v += ep.bias[col];
    if (col < ep.n_split)
      store_from_f32((T*)ep.out0 + (size_t)row * ep.ld0 + col, v);
    else
      store_from_f32((T*)ep.out1 + (size_t)row * ep.ld1 + ep.act_col0 + (col - ep.n_split), gelu_erf(v));
  } else if constexpr (MODE == EPI_RESID) {
    float* x = (float*)ep.out0 + (size_t)row * ep.ld0 + col;
    *x += v + ep.bias[col] + ep.bias2[col];
  } else if constexpr (MODE == EPI_STORE) {
    ((float*)ep.out0)[(size_t)row * ep.ld0 + col] = v + (ep.bias ? ep.bias[col] : 0.f);
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Maps the hardware workgroup id to a logical tile index so that the workgroups one XCD
// receives (ids x, x+8, x+16, ... go to XCD x) form one contiguous range of tiles.
__device__ __forceinline__ int xcd_contiguous_tile(int bid, int nb) {
  int per = nb >> 3, rem = nb & 7, x = bid & 7, i = bid >> 3;
  return x * per + min(x, rem) + i;
}

template <int BM, int BN, int WM, int WN, int MODE, int STAGES>
__global__ __launch_bounds__(256) void k_gemm_mfma(const f16* __restrict__ A1, const f16* __restrict__ A2, int lda,
                                                   const f16* __restrict__ W, int M, int N, int K, Epi ep) {
  constexpr int BK = 64, LDK = BK + 8;  // +16 B per LDS row: conflict-free 16-byte fragment reads
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int CA = BM * BK / 8 / 256, CB = BN * BK / 8 / 256;
  static_assert(WM * WN == 4 && FM >= 1 && FN >= 1 && CA >= 1 && CB >= 1, "tile");
  static_assert(STAGES == 1 || STAGES % 2 == 0, "register stages alternate the two LDS buffers");
  __shared__ __attribute__((aligned(16))) f16 smem[2 * (BM + BN) * LDK];
  f16(*As)[BM * LDK] = reinterpret_cast<f16(*)[BM * LDK]>(smem);
  f16(*Bs)[BN * LDK] = reinterpret_cast<f16(*)[BN * LDK]>(smem + 2 * BM * LDK);

  const int ntm = (M + BM - 1) / BM, ntn = N / BN;
  const int lt = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int split = lt % ep.splits, t = lt / ep.splits;  // K slices of one tile are neighbours
  constexpr int GM = 8;
  const int group = t / (GM * ntn), first_m = group * GM;
  const int gm = min(GM, ntm - first_m);
  const int r_in = t - group * GM * ntn;
  const int tm = first_m + r_in % gm, tn = r_in / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const f16* __restrict__ A = (MODE == EPI_QKV_GELU && n0 >= ep.n_split) ? A2 : A1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // STAGES K-steps of global loads are kept in flight in registers; each step's tile goes through
  // one of two LDS buffers.
  half8 ra[STAGES][CA], rb[STAGES][CB];
  auto gload = [&](int st, int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int c = tid + i * 256, r = c / (BK / 8), kc = c % (BK / 8);
      int row = min(m0 + r, M - 1);
      ra[st][i] = *(const half8*)(A + (size_t)row * lda + k0 + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      int c = tid + i * 256, r = c / (BK / 8), kc = c % (BK / 8);
      rb[st][i] = *(const half8*)(W + (size_t)(n0 + r) * K + k0 + kc * 8);
    }
  };
  auto sstore = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int c = tid + i * 256, r = c / (BK / 8), kc = c % (BK / 8);
      *(half8*)&As[buf][r * LDK + kc * 8] = ra[st][i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      int c = tid + i * 256, r = c / (BK / 8), kc = c % (BK / 8);
      *(half8*)&Bs[buf][r * LDK + kc * 8] = rb[st][i];
    }
  };

  float4_ acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = float4_{0.f, 0.f, 0.f, 0.f};

  const int nk_all = K / BK, per = (nk_all + ep.splits - 1) / ep.splits;
  const int kt0 = split * per, nk = min(nk_all, kt0 + per);  // this workgroup's K tiles [kt0, nk)
  auto mma = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      half8 af[FM], bw[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *(const half8*)&As[buf][(wm * TM + fm * 16 + (lane & 15)) * LDK + kk * 32 + (lane >> 4) * 8];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bw[fn] = *(const half8*)&Bs[buf][(wn * TN + fn * 16 + (lane & 15)) * LDK + kk * 32 + (lane >> 4) * 8];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bw[fn], acc[fm][fn], 0, 0, 0);
    }
  };
  if constexpr (STAGES == 1) {
    // one register stage (large tiles, where registers bound the occupancy): the next K step is
    // loaded while the current one is multiplied, then stored to the other LDS buffer
    gload(0, kt0 * BK);
    sstore(0, 0);
    __syncthreads();
    for (int kt = kt0; kt < nk; ++kt) {
      const int buf = (kt - kt0) & 1;
      if (kt + 1 < nk) gload(0, (kt + 1) * BK);
      mma(buf);
      if (kt + 1 < nk) sstore(0, buf ^ 1);
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
      if (kt0 + st < nk) gload(st, (kt0 + st) * BK);
    for (int kb = kt0; kb < nk; kb += STAGES) {
#pragma unroll
      for (int st = 0; st < STAGES; ++st) {
        const int kt = kb + st;
        if (kt < nk) {
          const int buf = st & 1;
          sstore(st, buf);
          if (kt + STAGES < nk) gload(st, (kt + STAGES) * BK);
          __syncthreads();
          mma(buf);
        }
      }
    }
  }

  // epilogue: lane holds C[4*(lane/16) + i][lane % 16] of each 16 x 16 tile
  constexpr bool kStaged = (MODE == EPI_QKV_GELU || MODE == EPI_RESID) && BM * (BN + 4) * 4 <= 2 * (BM + BN) * LDK * 2;
  if (kStaged && !(MODE == EPI_RESID && ep.splits > 1)) {
    // The finished tile goes through LDS so that global stores are whole 16-byte row segments
    // (split-K partials take the direct path below).
    constexpr int CLD = BN + 4;
    float* Cs = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done reading the operand tiles
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int cl = wn * TN + fn * 16 + (lane & 15);
      const float bias = ep.bias[n0 + cl] + (MODE == EPI_RESID ? ep.bias2[n0 + cl] : 0.f);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = wm * TM + fm * 16 + (lane >> 4) * 4 + i;
          float v = acc[fm][fn][i] * ep.wscale + bias;
          if constexpr (MODE == EPI_QKV_GELU)
            if (n0 >= ep.n_split) v = gelu_erf(v);
          Cs[rl * CLD + cl] = v;
        }
    }
    __syncthreads();
    if constexpr (MODE == EPI_QKV_GELU) {
      f16* dst;
      int ld, c0;
      if (n0 < ep.n_split) {
        dst = (f16*)ep.out0, ld = ep.ld0, c0 = n0;
      } else {
        dst = (f16*)ep.out1, ld = ep.ld1, c0 = ep.act_col0 + (n0 - ep.n_split);
      }
      constexpr int CH = (BM * BN / 8 + 255) / 256;  // 8-wide chunks per thread
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = tid + q * 256, rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
        if (c >= BM * BN / 8) break;
        if (m0 + rl < M) {
          half8 w;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16(Cs[rl * CLD + cl + e]);
          *(half8*)(dst + (size_t)(m0 + rl) * ld + c0 + cl) = w;
        }
      }
    } else {
      constexpr int CH = (BM * BN / 4 + 255) / 256;  // 4-wide chunks per thread
      float* X = (float*)ep.out0;
      float4 xo[CH];
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = min(tid + q * 256, BM * BN / 4 - 1), rl = c / (BN / 4), cl = (c % (BN / 4)) * 4;
        xo[q] = *(const float4*)(X + (size_t)min(m0 + rl, M - 1) * ep.ld0 + n0 + cl);
      }
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = tid + q * 256, rl = c / (BN / 4), cl = (c % (BN / 4)) * 4;
        if (c < BM * BN / 4 && m0 + rl < M) {
          const float* cs = &Cs[rl * CLD + cl];
          *(float4*)(X + (size_t)(m0 + rl) * ep.ld0 + n0 + cl) =
              make_float4(xo[q].x + cs[0], xo[q].y + cs[1], xo[q].z + cs[2], xo[q].w + cs[3]);
        }
      }
    }
  } else if constexpr (MODE == EPI_ARGMAX) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i;
        unsigned long long best = 0ull;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = n0 + wn * TN + fn * 16 + (lane & 15);
          const float v = acc[fm][fn][i] * ep.wscale;
          if (col < ep.n_valid) {
            if (ep.out0 && row < M) ((float*)ep.out0)[(size_t)row * ep.ld0 + col] = v;
            unsigned long long k = argmax_key(v, col);
            best = k > best ? k : best;
          }
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          unsigned long long other = shfl_xor_u64(best, o);
          best = other > best ? other : best;
        }
        if ((lane & 15) == 0 && row < M) ep.keys[(size_t)(tn * WN + wn) * ep.keys_ld + row] = best;
      }
  } else {
    // Loads the epilogue needs (biases per column, the residual per element) are issued for all of
    // this lane's outputs before any of them is used: no load sits behind a row guard, so they
    // overlap instead of each waiting for the previous one.  Rows past M are clamped for loads and
    // skipped for stores.
    float bc[FN], bc2[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = n0 + wn * TN + fn * 16 + (lane & 15);
      bc[fn] = (MODE == EPI_STORE && !ep.bias) ? 0.f : ep.bias[col];
      bc2[fn] = MODE == EPI_RESID ? ep.bias2[col] : 0.f;
    }
    if constexpr (MODE == EPI_RESID) {
      if (ep.splits > 1) {
        // split-K: partial products go to ep.part[split]; biases and residual are added by the consumer
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i;
              const int col = n0 + wn * TN + fn * 16 + (lane & 15);
              if (row < M) ep.part[((size_t)split * M + row) * N + col] = acc[fm][fn][i] * ep.wscale;
            }
        return;
      }
      float xo[FM][FN][4];
      float* X = (float*)ep.out0;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = min(m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i, M - 1);
            const int col = n0 + wn * TN + fn * 16 + (lane & 15);
            xo[fm][fn][i] = X[(size_t)row * ep.ld0 + col];
          }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i;
            const int col = n0 + wn * TN + fn * 16 + (lane & 15);
            if (row < M)
              X[(size_t)row * ep.ld0 + col] = xo[fm][fn][i] + (acc[fm][fn][i] * ep.wscale + bc[fn] + bc2[fn]);
          }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i;
            const int col = n0 + wn * TN + fn * 16 + (lane & 15);
            if (row >= M) continue;
            const float v = acc[fm][fn][i] * ep.wscale + bc[fn];
            if constexpr (MODE == EPI_QKV_GELU) {
              if (col < ep.n_split)
                ((f16*)ep.out0)[(size_t)row * ep.ld0 + col] = to_f16(v);
              else
                ((f16*)ep.out1)[(size_t)row * ep.ld1 + ep.act_col0 + (col - ep.n_split)] = to_f16(gelu_erf(v));
            } else {
              ((float*)ep.out0)[(size_t)row * ep.ld0 + col] = v;
            }
          }
    }
  }
}

// fp32 VALU GEMM: 64 x 64 tile, 256 threads with 4 x 4 outputs each, K staged 16 at a time.
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int lda, const float* __restrict__ W,
                                                  int M, int N, int K, Epi ep) {
  __shared__ float As[16][64 + 4], Ws[16][64 + 4];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  const int kchunk = (K + gridDim.z - 1) / gridDim.z;
  const int kbeg = blockIdx.z * kchunk, kend = min(K, kbeg + kchunk);
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      int r = e / 16, kk = e % 16;
      int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < kend) ? A[(size_t)gm * lda + gk] : 0.f;
      Ws[kk][r] = (gn < N && gk < kend) ? W[(size_t)gn * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = Ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    unsigned long long best = 0ull;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (row >= M || col >= N) continue;
      const float v = acc[i][j] * ep.wscale;
      if constexpr (MODE == EPI_ARGMAX) {
        if (col < ep.n_valid) {
          if (ep.out0) ((float*)ep.out0)[(size_t)row * ep.ld0 + col] = v;
          const unsigned long long k = argmax_key(v, col);
          best = k > best ? k : best;
        }
      } else if constexpr (MODE == EPI_RESID) {
        if (ep.splits > 1)
          ep.part[((size_t)blockIdx.z * M + row) * N + col] = v;
        else
          epi_store<MODE, float>(ep, row, col, v);
      } else {
        epi_store<MODE, float>(ep, row, col, v);
      }
    }
    if constexpr (MODE == EPI_ARGMAX)
      if (row < M) ep.keys[(size_t)(blockIdx.x * 16 + tx) * ep.keys_ld + row] = best;
  }
}

template <int BM, int BN, int WM, int WN, int STAGES>
static hipError_t launch_mfma_cfg(const void* A1, const void* A2, int lda, const void* W, int M, int N, int K,
                                  EpiMode mode, const Epi& ep, hipStream_t st) {
  if (mode == EPI_ARGMAX && ep.nparts_out) *ep.nparts_out = (N / BN) * WN;
  dim3 grid(((M + BM - 1) / BM) * (N / BN) * ep.splits), block(256);
  const f16 *a1 = (const f16*)A1, *a2 = (const f16*)A2, *w = (const f16*)W;
  switch (mode) {
    case EPI_QKV_GELU:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_QKV_GELU, STAGES>), grid, block, 0, st, a1, a2, lda, w, M, N, K, ep);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_RESID, STAGES>), grid, block, 0, st, a1, a2, lda, w, M, N, K, ep);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_STORE, STAGES>), grid, block, 0, st, a1, a2, lda, w, M, N, K, ep);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_ARGMAX, STAGES>), grid, block, 0, st, a1, a2, lda, w, M, N, K, ep);
      break;
  }
  return hipGetLastError();
}

static hipError_t launch_f32(const float* A, int lda, const float* W, int M, int N, int K, EpiMode mode,
                             const Epi& ep, hipStream_t st) {
  if (mode == EPI_ARGMAX && ep.nparts_out) *ep.nparts_out = ((N + 63) / 64) * 16;
  dim3 grid((N + 63) / 64, (M + 63) / 64, mode == EPI_RESID ? ep.splits : 1), block(256);
  switch (mode) {
    case EPI_QKV_GELU:
      hipLaunchKernelGGL(k_gemm_f32<EPI_QKV_GELU>, grid, block, 0, st, A, lda, W, M, N, K, ep);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL(k_gemm_f32<EPI_RESID>, grid, block, 0, st, A, lda, W, M, N, K, ep);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL(k_gemm_f32<EPI_STORE>, grid, block, 0, st, A, lda, W, M, N, K, ep);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL(k_gemm_f32<EPI_ARGMAX>, grid, block, 0, st, A, lda, W, M, N, K, ep);
      break;
  }
  return hipGetLastError();
}

// Split K only where the output tiles alone cannot fill the chip (decode: M is the batch).
int resid_splits(int M, int N, int K) {
  if (M > 1024) return 1;
  const int tiles = ((M + 63) / 64) * (N / 64 > 0 ? N / 64 : 1);
  const int nk = K / 64 > 0 ? K / 64 : 1;
  int s = std::min(std::min(16, nk), std::max(1, (512 + tiles - 1) / tiles));  // <= 16: the LayerNorm folds at most 16
  const int per = (nk + s - 1) / s;
  return (nk + per - 1) / per;  // every split gets at least one K tile of 64
}

hipError_t launch_gemm(bool f32, const void* A1, const void* A2, int lda, const void* W, int M, int N, int K,
                       EpiMode mode, const Epi& ep_in, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  Epi ep = ep_in;
  if (mode != EPI_RESID || ep.splits < 1) ep.splits = 1;
  if (f32) {
    if (mode == EPI_QKV_GELU) {
      // two launches: the q|k|v columns from A1, then the GELU columns from A2
      Epi e1 = ep;
      hipError_t err = launch_f32((const float*)A1, lda, (const float*)W, M, ep.n_split, K, mode, e1, st);
      if (err != hipSuccess) return err;
      Epi e2 = ep;
      e2.bias = ep.bias + ep.n_split;
      e2.n_split = 0;
      return launch_f32((const float*)A2, lda, (const float*)W + (size_t)ep.n_split * K, M, N - ep.n_split, K,
                        mode, e2, st);
    }
    return launch_f32((const float*)A1, lda, (const float*)W, M, N, K, mode, ep, st);
  }
  // fp16 MFMA path: K % 64 == 0, N % 32 == 0 and n_split on a tile boundary (checked at plan time)
  const bool split_ok128 = (mode != EPI_QKV_GELU) || (ep.n_split % 128 == 0);
  if ((M > 1024 || (M >= 256 && mode == EPI_ARGMAX)) && N % 128 == 0 && split_ok128 && ep.splits == 1)
    return launch_mfma_cfg<128, 128, 2, 2, 1>(A1, A2, lda, W, M, N, K, mode, ep, st);
  if (ep.splits > 1) return launch_mfma_cfg<64, 64, 2, 2, 4>(A1, A2, lda, W, M, N, K, mode, ep, st);
  const long tiles64 = (long)((M + 63) / 64) * (N / 64);
  if (N % 64 == 0 && tiles64 >= 512) return launch_mfma_cfg<64, 64, 2, 2, 4>(A1, A2, lda, W, M, N, K, mode, ep, st);
  const long tiles6432 = (long)((M + 63) / 64) * (N / 32);
  // decode shapes: small tiles keep several K steps in flight per workgroup
  if (tiles6432 >= 512) return launch_mfma_cfg<64, 32, 4, 1, 6>(A1, A2, lda, W, M, N, K, mode, ep, st);
  return launch_mfma_cfg<32, 32, 2, 2, 6>(A1, A2, lda, W, M, N, K, mode, ep, st);
}

}  // namespace bt
