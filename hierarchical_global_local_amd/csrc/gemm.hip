// GEMM kernels of libbt: C[M][N] = A[M][K] * W[N][K]^T with fused epilogues.
//
// fp16 operands (v_mfma_f32_16x16x32_f16, fp32 accumulation) are stored in fragment order (see
// frag_off): every 16 x 32 operand tile is one contiguous 1 KB block laid out as the wave's MFMA
// operand registers.
//  - LDS-tiled kernel (prefill, large M): 256 threads as a WM x WN grid of waves, BK = 64 staged
//    through two LDS buffers; tiles are copied into LDS as whole 1 KB blocks and read back with
//    conflict-free 16-byte reads, no swizzle or padding.  Workgroup ids are remapped so that each
//    of the 8 XCDs walks a contiguous range of output tiles, grouped 8 M-tiles at a time, so that A
//    and W tiles are re-read from that XCD's L2 rather than from HBM.
//  - skinny kernel (decode, M <= 256): operands go straight from memory into registers.
// fp32 operands (BT_FP32): a plain LDS-tiled VALU kernel with the same epilogues, row-major.
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

// Maps the hardware workgroup id to a logical tile index so that the workgroups one XCD
// receives (ids x, x+8, x+16, ... go to XCD x) form one contiguous range of tiles.
__device__ __forceinline__ int xcd_contiguous_tile(int bid, int nb) {
  int per = nb >> 3, rem = nb & 7, x = bid & 7, i = bid >> 3;
  return x * per + min(x, rem) + i;
}

template <int BM, int BN, int WM, int WN, int MODE, int STAGES>
__global__ __launch_bounds__(256) void k_gemm_mfma(const f16* __restrict__ A1, const f16* __restrict__ A2,
                                                   const f16* __restrict__ W, int M, int N, int K, Epi ep) {
  constexpr int BK = 64;                               // two 32-wide K steps per stage
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int CHA = BM / 16 * 2, CHB = BN / 16 * 2;  // 1 KB operand tiles per stage
  constexpr int CA = CHA / 4, CB = CHB / 4;            // tiles per thread: the 4 waves load 4 at a time
  static_assert(WM * WN == 4 && FM >= 1 && FN >= 1 && CA >= 1 && CB >= 1, "tile");
  static_assert(STAGES == 1 || STAGES % 2 == 0, "register stages alternate the two LDS buffers");
  constexpr bool kStagedMode = MODE == EPI_QKV_GELU || MODE == EPI_RESID;
  constexpr int OPND = 2 * (CHA + CHB) * 512;                // f16 elements: two stages of A and W tiles
  constexpr int EPIL = kStagedMode ? BM * (BN + 4) * 2 : 0;  // fp32 output tile, in f16 units
  __shared__ __attribute__((aligned(16))) f16 smem[OPND > EPIL ? OPND : EPIL];
  f16* As = smem;                  // [2][CHA][512]
  f16* Bs = smem + 2 * CHA * 512;  // [2][CHB][512]

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
  const int KS = K / 32, mgs = (M + 15) / 16, mg0 = m0 / 16, ng0 = n0 / 16;

  // STAGES K-steps of global loads are kept in flight in registers; each stage goes through one of
  // two LDS buffers.  Thread (wave, lane) moves 16 bytes of operand tiles wave, wave + 4, ...
  half8 ra[STAGES][CA], rb[STAGES][CB];
  auto gload = [&](int st, int kt) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = wave + 4 * i, mg = min(mg0 + (c >> 1), mgs - 1);
      ra[st][i] = *(const half8*)(A + ((size_t)(mg * KS + 2 * kt + (c & 1)) * 64 + lane) * 8);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = wave + 4 * i;
      rb[st][i] = *(const half8*)(W + ((size_t)((ng0 + (c >> 1)) * KS + 2 * kt + (c & 1)) * 64 + lane) * 8);
    }
  };
  auto sstore = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *(half8*)&As[(buf * CHA + wave + 4 * i) * 512 + lane * 8] = ra[st][i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *(half8*)&Bs[(buf * CHB + wave + 4 * i) * 512 + lane * 8] = rb[st][i];
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
    for (int kk = 0; kk < 2; ++kk) {
      half8 af[FM], bw[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *(const half8*)&As[(buf * CHA + (wm * FM + fm) * 2 + kk) * 512 + lane * 8];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bw[fn] = *(const half8*)&Bs[(buf * CHB + (wn * FN + fn) * 2 + kk) * 512 + lane * 8];
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
    gload(0, kt0);
    sstore(0, 0);
    __syncthreads();
    for (int kt = kt0; kt < nk; ++kt) {
      const int buf = (kt - kt0) & 1;
      if (kt + 1 < nk) gload(0, kt + 1);
      mma(buf);
      if (kt + 1 < nk) sstore(0, buf ^ 1);
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
      if (kt0 + st < nk) gload(st, kt0 + st);
    for (int kb = kt0; kb < nk; kb += STAGES) {
#pragma unroll
      for (int st = 0; st < STAGES; ++st) {
        const int kt = kb + st;
        if (kt < nk) {
          const int buf = st & 1;
          sstore(st, buf);
          if (kt + STAGES < nk) gload(st, kt + STAGES);
          __syncthreads();
          mma(buf);
        }
      }
    }
  }

  // epilogue: lane holds C[4*(lane/16) + i][lane % 16] of each 16 x 16 tile
  if (kStagedMode && !(MODE == EPI_RESID && ep.splits > 1)) {
    // The finished tile goes through LDS so that global stores are whole 16-byte segments.
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
      // q|k|v columns: row-major [M][ld0]; GELU columns: the [attn | gelu] operand in fragment order
      const bool gelu = n0 >= ep.n_split;
      constexpr int CH = (BM * BN / 8 + 255) / 256;  // 8-wide chunks per thread
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = tid + q * 256, rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
        if (c >= BM * BN / 8) break;
        const int row = m0 + rl;
        if (row < M) {
          half8 w;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16(Cs[rl * CLD + cl + e]);
          if (gelu)
            *(half8*)((f16*)ep.out1 + frag_off(row, ep.act_col0 + (n0 - ep.n_split) + cl, ep.ld1)) = w;
          else
            *(half8*)((f16*)ep.out0 + (size_t)row * ep.ld0 + n0 + cl) = w;
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
        if ((lane & 15) == 0 && row < M) ep.keys[(size_t)row * ep.keys_ld + tn * WN + wn] = best;
      }
  } else if constexpr (MODE == EPI_RESID) {
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
  } else {
    // EPI_STORE: fp32 output with an optional bias; the bias loads are issued before any store
    float bc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bc[fn] = ep.bias ? ep.bias[n0 + wn * TN + fn * 16 + (lane & 15)] : 0.f;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m0 + wm * TM + fm * 16 + (lane >> 4) * 4 + i;
          const int col = n0 + wn * TN + fn * 16 + (lane & 15);
          if (row < M) ((float*)ep.out0)[(size_t)row * ep.ld0 + col] = acc[fm][fn][i] * ep.wscale + bc[fn];
        }
  }
}

// ---------------------------------------------------------------- skinny GEMM (decode shapes)
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
      if (row < M) ep.keys[(size_t)row * ep.keys_ld + blockIdx.x * 16 + tx] = best;
  }
}

template <int BM, int BN, int WM, int WN, int STAGES>
static hipError_t launch_mfma_cfg(const void* A1, const void* A2, const void* W, int M, int N, int K, EpiMode mode,
                                  const Epi& ep, hipStream_t st) {
  if (mode == EPI_ARGMAX && ep.nparts_out) *ep.nparts_out = (N / BN) * WN;
  dim3 grid(((M + BM - 1) / BM) * (N / BN) * ep.splits), block(256);
  const f16 *a1 = (const f16*)A1, *a2 = (const f16*)A2, *w = (const f16*)W;
  switch (mode) {
    case EPI_QKV_GELU:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_QKV_GELU, STAGES>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_RESID, STAGES>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_STORE, STAGES>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, EPI_ARGMAX, STAGES>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
  }
  return hipGetLastError();
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

// Which fp16 kernel a GEMM of this shape runs (shared by launch_gemm and resid_splits, so that the
// split count the consumer folds is the one the kernel used).
struct GemmPlan {
  bool skinny;
  int mg, mw, ng, kw;  // skinny: waves and fragments
  int splits;          // K splits over workgroups (EPI_RESID only)
};

static GemmPlan plan_gemm(int M, int N, int K, EpiMode mode) {
  GemmPlan p{};
  p.splits = 1;
  // The skinny kernel streams the weights once for all M <= 256 rows.  The classifier of a batch
  // above 128 rows has enough MFMA work to prefer the LDS-tiled kernel.
  p.skinny = M <= 256 && N % 32 == 0 && K % 32 == 0 && !(mode == EPI_ARGMAX && M > 128);
  if (p.skinny) {
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
      // narrow outputs ([out|down]: N = d_model) split K so that ~192 workgroups stream the weights
      int s = std::min(16, (192 + slabs - 1) / slabs);
      s = std::max(1, std::min(s, ks / p.kw));
      const int per = (ks + s - 1) / s;
      p.splits = (ks + per - 1) / per;  // every split owns at least one K step
    }
    return p;
  }
  if (mode == EPI_RESID && M <= 1024) {
    const int tiles = ((M + 63) / 64) * std::max(1, N / 64);
    const int nk = std::max(1, K / 64);
    int s = std::min(std::min(16, nk), std::max(1, (512 + tiles - 1) / tiles));
    const int per = (nk + s - 1) / s;
    p.splits = (nk + per - 1) / per;
  }
  return p;
}

int resid_splits(int M, int N, int K) { return plan_gemm(M, N, K, EPI_RESID).splits; }

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
  // fp16 path: both operands in fragment order (their width is K)
  const GemmPlan p = plan_gemm(M, N, K, mode);
  if (mode == EPI_RESID && ep.splits != p.splits) ep.splits = p.splits;
  if (ep.splits > 1 && !ep.part) return hipErrorInvalidValue;
  if (p.skinny) {
    const int S = ep.splits;
#define BT_SKINNY(MG, MW, NG, KW) \
  if (p.mg == MG && p.mw == MW && p.ng == NG && p.kw == KW) return launch_skinny_cfg<MG, MW, NG, KW>(A1, A2, W, M, N, K, mode, ep, S, st);
    BT_SKINNY(1, 1, 2, 8)
    BT_SKINNY(2, 1, 2, 8)
    BT_SKINNY(4, 1, 2, 8)
    BT_SKINNY(4, 2, 2, 4)
    BT_SKINNY(4, 2, 4, 4)
    BT_SKINNY(4, 4, 2, 4)
#undef BT_SKINNY
    return hipErrorInvalidValue;
  }
  // LDS-tiled kernel: K % 64 == 0, N % 32 == 0 and n_split on a tile boundary (checked at plan time)
  const bool split_ok128 = (mode != EPI_QKV_GELU) || (ep.n_split % 128 == 0);
  if ((M > 1024 || (M >= 256 && mode == EPI_ARGMAX)) && N % 128 == 0 && split_ok128 && ep.splits == 1)
    return launch_mfma_cfg<128, 128, 2, 2, 1>(A1, A2, W, M, N, K, mode, ep, st);
  if (ep.splits > 1) return launch_mfma_cfg<64, 64, 2, 2, 4>(A1, A2, W, M, N, K, mode, ep, st);
  const long tiles64 = (long)((M + 63) / 64) * (N / 64);
  if (N % 64 == 0 && tiles64 >= 512) return launch_mfma_cfg<64, 64, 2, 2, 4>(A1, A2, W, M, N, K, mode, ep, st);
  const long tiles6432 = (long)((M + 63) / 64) * (N / 32);
  if (tiles6432 >= 512) return launch_mfma_cfg<64, 32, 4, 1, 6>(A1, A2, W, M, N, K, mode, ep, st);
  return launch_mfma_cfg<32, 32, 2, 2, 6>(A1, A2, W, M, N, K, mode, ep, st);
}

}  // namespace bt
