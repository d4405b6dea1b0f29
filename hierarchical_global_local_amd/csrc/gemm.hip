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
//  - large-tile kernel (prefill [q|k|v|up] and [out|down]): 256 x 128 tiles fed by direct
//    global -> LDS copies, two workgroups per CU;
//  - the skinny kernel for decode shapes (M <= 256) is in gemm_decode.hip.
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
      uint32_t trk = 0u;
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = tid + q * 256, rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
        if (c >= BM * BN / 8) break;
        const int row = m0 + rl;
        if (row < M) {
          half8 w;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16_trk(Cs[rl * CLD + cl + e], trk);
          if (gelu)
            *(half8*)((f16*)ep.out1 + frag_off(row, ep.act_col0 + (n0 - ep.n_split) + cl, ep.ld1)) = w;
          else
            *(half8*)((f16*)ep.out0 + (size_t)row * ep.ld0 + n0 + cl) = w;
        }
      }
      clamp_note(trk);
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
        best = max_lanes_u64<16>(best);
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

// ---------------------------------------------------------------- large-tile GEMM (prefill)
// With many rows (prefill: M = batch x prompt blocks) the GEMM is MFMA-bound, and what limits the
// 128 x 128 kernel is LDS read bandwidth (a 64 x 64 wave tile reads 8 KB of fragments per 16
// MFMAs) and global latency (one register stage of prefetch).  Here each of the 4 waves owns a
// 128 x TN tile (BN = 2 TN), which cuts the LDS bytes per MFMA, and the operand tiles travel
// global -> LDS directly (global_load_lds_dwordx4: a wave moves one 1 KB fragment-order tile per
// instruction, no registers) through a ring of NS stages, NS - 1 K steps in flight.  Used with
// BN = 128, NS = 3: 72 KB of LDS and <= 256 registers per lane, so two workgroups share a CU and
// one's epilogue overlaps the other's main loop (BN = 256, NS = 4 -- 128 x 128 per wave, one
// workgroup per CU -- measured slower on every prefill shape once that variant existed).
// Each wave waits for its own copies of a stage with an explicit vmcnt and the workgroup barrier
// publishes them; a slot is refilled only after the barrier that follows every wave's last use of
// it.  EPI_QKV_GELU and EPI_RESID (no split) only; the epilogue goes through LDS 128 rows at a time
// so that every global store is a whole 16-byte segment.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {  // s_waitcnt vmcnt(N), other counters untouched
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
// workgroup barrier without a memory fence (which would wait for every copy in flight); the empty
// asm statements keep the compiler from moving LDS accesses across it
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BN, int NS, int MODE>
__global__ __launch_bounds__(256, BN == 128 ? 2 : 1) void k_gemm_big(const f16* __restrict__ A1, const f16* __restrict__ A2,
                                                  const f16* __restrict__ W, int M, int N, int K, Epi ep) {
  constexpr int BM = 256, WN = 2;
  constexpr int TM = 128, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int CHA = BM / 16, CHB = BN / 16;  // 1 KB operand tiles per 32-wide K step
  constexpr int CA = CHA / 4, CB = CHB / 4;    // copies per wave per stage
  constexpr int PER = CA + CB;
  constexpr int STG = (CHA + CHB) * 512;       // f16 elements per stage
  constexpr int SR = TM, CLD = BN + 4;         // epilogue slab: one wave row of fp32
  constexpr int EPIL = SR * CLD * 2;
  static_assert(MODE == EPI_QKV_GELU || MODE == EPI_RESID || MODE == EPI_ARGMAX, "epilogue");
  static_assert((NS == 4 || NS == 3) && 2 * PER < 64, "ring: NS - 1 stages in flight");
  __shared__ __attribute__((aligned(16))) f16 smem[NS * STG > EPIL ? NS * STG : EPIL];

  const int ntm = (M + BM - 1) / BM, ntn = N / BN;
  const int t = xcd_contiguous_tile(blockIdx.x, gridDim.x);
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

  // K step ks -> ring slot ks % NS: A tiles (16-row groups of the tile) then W tiles
  auto issue = [&](int ks) {
    f16* st = smem + (ks % NS) * STG;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = wave + 4 * i, mg = min(mg0 + c, mgs - 1);
      __builtin_amdgcn_global_load_lds(A + ((size_t)(mg * KS + ks) * 64 + lane) * 8,
                                       (__attribute__((address_space(3))) void*)(st + c * 512), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = wave + 4 * i;
      __builtin_amdgcn_global_load_lds(W + ((size_t)((ng0 + c) * KS + ks) * 64 + lane) * 8,
                                       (__attribute__((address_space(3))) void*)(st + (CHA + c) * 512), 16, 0, 0);
    }
  };

  float4_ acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = float4_{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int q = 0; q < NS - 1; ++q)
    if (q < KS) issue(q);
  for (int ks = 0; ks < KS; ++ks) {
    // stage ks is complete once at most (stages issued after it) x PER copies are outstanding
    const int later = min(NS - 2, KS - 1 - ks);
    if (later >= 2) wait_vmcnt<2 * PER>();
    else if (later == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
    // after this barrier every wave has consumed (waited for and multiplied) its reads of step
    // ks - 1, so that step's slot can be refilled
    barrier_nofence();
    if (ks + NS - 1 < KS) issue(ks + NS - 1);
    const f16* st = smem + (ks % NS) * STG;
    // all fragments of the step are read before the first MFMA (the scheduling barrier keeps the
    // compiler from sinking the reads between MFMA groups, which would expose the LDS latency)
    half8 af[FM], bw[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bw[fn] = *(const half8*)&st[(CHA + wn * FN + fn) * 512 + lane * 8];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) af[fm] = *(const half8*)&st[(wm * FM + fm) * 512 + lane * 8];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[fm], bw[fn], acc[fm][fn], 0, 0, 0);
  }
  wait_vmcnt<0>();
  if constexpr (MODE == EPI_ARGMAX) {
    // classifier: per row, the largest (value, id) key of this wave's TN columns (ids >= n_valid
    // are padding), and the logits if requested
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
            const unsigned long long k = argmax_key(v, col);
            best = k > best ? k : best;
          }
        }
        best = max_lanes_u64<16>(best);
        if ((lane & 15) == 0 && row < M) ep.keys[(size_t)row * ep.keys_ld + tn * WN + wn] = best;
      }
    return;
  }
  __syncthreads();  // every wave is done with the ring before it becomes the epilogue's staging area

  // epilogue, one wave row (128 rows) of the tile at a time: the two waves owning it stage
  // acc * scale + bias in LDS, then all threads apply GELU (the up columns) and write whole 16-byte
  // segments, so that the transcendental work is spread over the whole workgroup
  float bias[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int col = n0 + wn * TN + fn * 16 + (lane & 15);
    if constexpr (MODE != EPI_ARGMAX) bias[fn] = ep.bias[col] + (MODE == EPI_RESID ? ep.bias2[col] : 0.f);
  }
  float* Cs = reinterpret_cast<float*>(smem);
  const bool gelu = MODE == EPI_QKV_GELU && n0 >= ep.n_split;
#pragma unroll
  for (int s = 0; s < BM / SR; ++s) {
    if (wm == s) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int cl = wn * TN + fn * 16 + (lane & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) Cs[(fm * 16 + (lane >> 4) * 4 + i) * CLD + cl] = acc[fm][fn][i] * ep.wscale + bias[fn];
        }
    }
    __syncthreads();
    const int r0 = m0 + s * SR;
    if constexpr (MODE == EPI_QKV_GELU) {
      constexpr int CH = SR * BN / 8 / 256;
      uint32_t trk = 0u;
#pragma unroll 4
      for (int q = 0; q < CH; ++q) {
        const int c = tid + q * 256, rl = c / (BN / 8), cl = (c % (BN / 8)) * 8;
        const int row = r0 + rl;
        if (row < M) {
          half8 w;
          if (gelu) {
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = to_f16_trk(gelu_erf(Cs[rl * CLD + cl + e]), trk);
            *(half8*)((f16*)ep.out1 + frag_off(row, ep.act_col0 + (n0 - ep.n_split) + cl, ep.ld1)) = w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = to_f16_trk(Cs[rl * CLD + cl + e], trk);
            *(half8*)((f16*)ep.out0 + (size_t)row * ep.ld0 + n0 + cl) = w;
          }
        }
      }
      clamp_note(trk);
    } else {
      // residual rows in groups of 8 float4 per thread: all loads of a group before its stores
      constexpr int CH = SR * BN / 4 / 256, G = 8;
      float* X = (float*)ep.out0;
#pragma unroll
      for (int q0 = 0; q0 < CH; q0 += G) {
        float4 xo[G];
#pragma unroll
        for (int q = 0; q < G; ++q) {
          const int c = tid + (q0 + q) * 256, rl = c / (BN / 4), cl = (c % (BN / 4)) * 4;
          xo[q] = *(const float4*)(X + (size_t)min(r0 + rl, M - 1) * ep.ld0 + n0 + cl);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
          const int c = tid + (q0 + q) * 256, rl = c / (BN / 4), cl = (c % (BN / 4)) * 4;
          if (r0 + rl < M) {
            const float* cs = &Cs[rl * CLD + cl];
            *(float4*)(X + (size_t)(r0 + rl) * ep.ld0 + n0 + cl) =
                make_float4(xo[q].x + cs[0], xo[q].y + cs[1], xo[q].z + cs[2], xo[q].w + cs[3]);
          }
        }
      }
    }
    __syncthreads();
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

template <int BN, int NS>
static hipError_t launch_big_cfg(const void* A1, const void* A2, const void* W, int M, int N, int K, EpiMode mode,
                                 const Epi& ep, hipStream_t st) {
  dim3 grid(((M + 255) / 256) * (N / BN)), block(256);
  const f16 *a1 = (const f16*)A1, *a2 = (const f16*)A2, *w = (const f16*)W;
  if (mode == EPI_QKV_GELU) {
    hipLaunchKernelGGL((k_gemm_big<BN, NS, EPI_QKV_GELU>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
  } else if (mode == EPI_RESID) {
    hipLaunchKernelGGL((k_gemm_big<BN, NS, EPI_RESID>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
  } else {
    if (ep.nparts_out) *ep.nparts_out = N / (BN / 2);  // one key per row and wave column half
    hipLaunchKernelGGL((k_gemm_big<BN, NS, EPI_ARGMAX>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
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

// Split count of a tiled-kernel GEMM (decode-size M above the skinny range): K is split over
// workgroups for EPI_RESID with at most 1024 rows until ~512 workgroups run.
static int tiled_resid_splits(int M, int N, int K) {
  if (M > 1024) return 1;
  const int tiles = ((M + 63) / 64) * std::max(1, N / 64);
  const int nk = std::max(1, K / 64);
  int s = std::min(std::min(16, nk), std::max(1, (512 + tiles - 1) / tiles));
  const int per = (nk + s - 1) / s;
  return (nk + per - 1) / per;
}

int resid_splits(int M, int N, int K) {
  const SkinnyPlan p = skinny_plan(M, N, K, EPI_RESID);
  return p.ok ? p.splits : tiled_resid_splits(M, N, K);
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
  // fp16 path: both operands in fragment order (their width is K)
  const SkinnyPlan sp = skinny_plan(M, N, K, mode);
  if (mode == EPI_RESID) ep.splits = sp.ok ? sp.splits : tiled_resid_splits(M, N, K);
  if (ep.splits > 1 && !ep.part) return hipErrorInvalidValue;
  if (sp.ok) return launch_gemm_skinny(sp, A1, A2, W, M, N, K, mode, ep, st);
  // Prefill [q|k|v|up] and [out|down] (fused epilogues): 256 x 128 tiles, 128 x 64 per wave, operand
  // tiles copied global -> LDS through a 3-stage ring (72 KB), two workgroups per CU so that one's
  // epilogue (GELU, staged stores) overlaps the other's main loop.  Measured against the 128 x 128
  // kernel: 573 -> 701 TFLOP/s on the prefill-heavy [q|k|v|up] (K = 768), 637 -> 801 on its
  // [out|down] (K = 3840, where the 256 x 256 variant at one workgroup per CU had been used); the
  // 1.2B prefill drops from 105 to 96 ms.
  if (M > 1024 && ep.splits == 1 && (mode == EPI_QKV_GELU || mode == EPI_RESID) && K % 64 == 0 && N % 128 == 0 &&
      (mode != EPI_QKV_GELU || ep.n_split % 128 == 0) && (long)((M + 255) / 256) * (N / 128) >= 512)
    return launch_big_cfg<128, 3>(A1, A2, W, M, N, K, mode, ep, st);
  // the classifier of a batch above the skinny kernel's 128 rows: the weights stream once
  if (mode == EPI_ARGMAX && M > 128 && K % 64 == 0 && N % 128 == 0)
    return launch_big_cfg<128, 3>(A1, A2, W, M, N, K, mode, ep, st);
  // 65-128 rows: one row tile of 128 x 128 (skinny_plan leaves these shapes to this kernel)
  if (mode == EPI_ARGMAX && M > 64 && K % 64 == 0 && N % 128 == 0)
    return launch_mfma_cfg<128, 128, 2, 2, 1>(A1, A2, W, M, N, K, mode, ep, st);
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

BT_DEFINE_CLAMP_FLAG_ACCESS(clamp_flag_gemm)

}  // namespace bt
