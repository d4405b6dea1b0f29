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
// One workgroup's tile: rows [16 mg0, 16 mg0 + R) x the 16 * NG columns of column slab `slab`, over
// the K steps [ks_lo, ks_hi) cut into `nsplit` equal ranges of which this is range `split`.
// EPI_RESID with to_part writes the partial products to ep.part slot `pslot`.  red: KW * R *
// (16 NG + 4) floats of LDS.
template <int MG, int MW, int NG, int KW>
constexpr int skinny_lds_floats() { return KW * (16 * MG * MW) * (16 * NG + 4); }

template <int MG, int MW, int NG, int KW, int MODE, int DEPTH>
__device__ __forceinline__ void skinny_tile(const f16* __restrict__ A1, const f16* __restrict__ A2,
                                            const f16* __restrict__ W, int M, int N, int K, const Epi& ep, int slab,
                                            int ks_lo, int ks_hi, int split, int nsplit, bool to_part, int pslot,
                                            float* __restrict__ red, int mg0 = 0) {
  constexpr int R = 16 * MG * MW, C = 16 * NG, CLD = C + 4, NT = 64 * MW * KW;
  const int KS = K / 32, mgs = (M + 15) / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mw = wave % MW, kw = wave / MW;
  const int ng0 = slab * NG, n0 = ng0 * 16;
  const f16* __restrict__ A = (MODE == EPI_QKV_GELU && n0 >= ep.n_split) ? A2 : A1;
  // K steps of this workgroup, then of this wave
  const int sper = (ks_hi - ks_lo + nsplit - 1) / nsplit;
  const int sb = min(ks_hi, ks_lo + split * sper), se = min(ks_hi, sb + sper);
  const int wper = (se - sb + KW - 1) / KW;
  const int kb = min(se, sb + kw * wper), ke = min(se, kb + wper);

  const f16* ap[MG];
#pragma unroll
  for (int i = 0; i < MG; ++i) ap[i] = A + ((size_t)min(mg0 + mw * MG + i, mgs - 1) * KS * 64 + lane) * 8;
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
    const int row = 16 * mg0 + rl, col = n0 + cl;
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
        uint32_t trk = 0u;
        if (n0 >= ep.n_split) {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16_trk(gelu_erf(v[e]), trk);
          *(half8*)((f16*)ep.out1 + frag_off(row, ep.act_col0 + (col - ep.n_split), ep.ld1)) = w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = to_f16_trk(v[e], trk);
          *(half8*)((f16*)ep.out0 + (size_t)row * ep.ld0 + col) = w;
        }
        clamp_note(trk);
      }
    } else if constexpr (MODE == EPI_RESID) {
      if (to_part) {
        float* p = ep.part + ((size_t)pslot * M + row) * N + col;
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
      best = max_lanes_u64<CPR>(best);
      if (live && cl == 0) ep.keys[(size_t)row * ep.keys_ld + slab] = best;
    }
  }
}

// grid (N / (16 NG), splits, row groups): gridDim.y > 1 splits K over workgroups (EPI_RESID only),
// whose partial products go to ep.part for the consumer to add; gridDim.z row groups of 16 MG MW
// rows each.  (Placing the row groups of one column slab on one XCD, so that its weight tiles come
// through one L2, measured slower: 9.9 instead of 9.2 us at 256 rows x 5376 x 768.)
template <int MG, int MW, int NG, int KW, int MODE, int DEPTH = 2>
__global__ __launch_bounds__(64 * MW * KW) void k_gemm_skinny(const f16* __restrict__ A1, const f16* __restrict__ A2,
                                                              const f16* __restrict__ W, int M, int N, int K, Epi ep) {
  __shared__ __attribute__((aligned(16))) float red[skinny_lds_floats<MG, MW, NG, KW>()];
  skinny_tile<MG, MW, NG, KW, MODE, DEPTH>(A1, A2, W, M, N, K, ep, blockIdx.x, 0, K / 32, blockIdx.y, gridDim.y,
                                           gridDim.y > 1, blockIdx.y, red, (int)blockIdx.z * MG * MW);
}

// ---------------------------------------------------------------- local attention + [out|down]
// Decode step of a token-decoder layer (one new local slot per row, head width 64): the token
// decoder's attention over its local window (prefix + the current block's tokens, summary page
// §3.4, The Token Decoder) is computed inside the [out|down] GEMM that consumes it, so that its
// latency overlaps the weight stream of the same launch instead of costing a launch of its own.
//  * attention workgroups (rb, hp, cp): rows [RB rb, RB rb + RB) (RB = 4 x waves: 32 with the 8-wave workgroups of
//    every plan),
//    query heads 2hp and 2hp + 1, output columns [128 cp, 128 cp + 128).  Half the waves take
//    each head, 8 rows per wave: lane = (row, 8 dimensions), rotary at the new slot, the new key
//    and value from the q | k | v row and the s0 cached ones from the local cache, softmax in base
//    2.  The outputs go to LDS in fragment order and feed 8 MFMAs per wave (column group
//    8 cp + wave % 8, the heads' four K steps); the products are partial sums (split hp) of the
//    residual update.  The workgroups with cp = 0 also write the new key (rotary applied,
//    rounded) and value to local slot s0 (first query head of a KV group).  A workgroup issues
//    its loads in the order it consumes them and the weight tiles last, so that waiting for the
//    attention's operands never waits for the weight stream.
//  * GEMM workgroups: the skinny tiles over the GELU columns [D, D + F) of the K range, K split
//    mlp_splits ways, partial slots H / 2 + split.
// All partials (H / 2 + mlp_splits of them) are folded, with both biases, by the next LayerNorm.

__device__ __forceinline__ void h8_to_f(const half8& v, float* o) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}

template <int MG, int MW, int NG, int KW, bool XA>
__global__ __launch_bounds__(64 * MW * KW) void k_attn_out(const f16* __restrict__ ACT, const f16* __restrict__ W,
                                                           int M, int N, int K, Epi ep, LocalStep ls, int n_attn,
                                                           int n_cp, int mlp_splits, int spread) {
  // attention tiles of RB rows: WPI waves per head (8 rows each), two heads
  constexpr int NWAVE = MW * KW, RB = 4 * NWAVE, RG = RB / 16, WPI = NWAVE / 2;
  static_assert(NWAVE == 8 || NWAVE == 16, "8 or 16 waves");
  // (XA: a second set of A tiles holds the cross-attention outputs)
  constexpr int LDS_GEMM = skinny_lds_floats<MG, MW, NG, KW>(), LDS_A = RG * 4 * 256,
                LDS_ATT = (XA ? 2 : 1) * LDS_A + 64 * NWAVE;
  __shared__ __attribute__((aligned(16))) float lds[LDS_GEMM > LDS_ATT ? LDS_GEMM : LDS_ATT];
  const int n_hp = ls.H / 2;
  // Workgroup id -> tile.  Workgroup ids x, x + 8, ... run on XCD x.  Attention group a = (rb, hp)
  // goes to XCD a % 8 with all n_cp of its column parts (the copies of its attention then share
  // that XCD's L2), and the GEMM tiles fill each XCD's remaining workgroups in order (consecutive
  // slabs of one K split share their operand rows).  spread = 0 (an XCD would hold more attention
  // tiles than workgroups): tiles in id order.
  const int nb = gridDim.x, n_grp = n_attn / n_cp;
  int t = blockIdx.x;
  if (spread) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int na = (n_grp / 8 + (x < n_grp % 8)) * n_cp;
    if (i < na) {
      t = ((i / n_cp) * 8 + x) * n_cp + i % n_cp;
    } else {
      const int before = x * (nb / 8) + min(x, nb % 8) - n_cp * (x * (n_grp / 8) + min(x, n_grp % 8));
      t = n_attn + before + (i - na);
    }
  }
  if (t >= n_attn) {
    // GEMM tile u: row group u / (slabs x splits) of 16 MG MW rows, then K split, then column slab
    const int slabs = N / (16 * NG), per_rg = slabs * mlp_splits;
    const int u = (t - n_attn) % per_rg, rg = (t - n_attn) / per_rg;
    skinny_tile<MG, MW, NG, KW, EPI_RESID, 2>(ACT, nullptr, W, M, N, K, ep, u % slabs, ls.H * 2,
                                              (XA ? ls.k_mlp : K) / 32, u / slabs, mlp_splits, true,
                                              n_hp + u / slabs, lds, rg * MG * MW);
    return;
  }
  const int cp = t % n_cp, hp = (t / n_cp) % n_hp, rb = t / (n_cp * n_hp);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KS = K / 32, ng = cp * 8 + (wave & 7);
  const int g = lane & 7, it = wave / WPI, lr = 8 * (wave % WPI) + (lane >> 3);
  const int r = rb * RB + lr, rc = min(r, M - 1);
  const int G = ls.H / ls.Hkv, s0 = ls.s0, h = 2 * hp + it, hk = h / G;
  const int crow = ls.rmap ? ls.rmap[rc] : rc;
  // Loads in the order they are consumed (a wait for one load is a wait for every earlier one):
  // q | k | v, the cached entries, the rotary row (one float per lane of every wave), then
  // the weight tiles, which only the MFMAs at the end need.
  const f16* __restrict__ qrow = ls.qkv + (size_t)rc * ls.ldq + 8 * g;
  const half8 qh = *(const half8*)(qrow + h * 64);
  const half8 kh = *(const half8*)(qrow + (ls.H + hk) * 64);
  const half8 vh = *(const half8*)(qrow + (ls.H + ls.Hkv + hk) * 64);
  // the rotary partners of this lane's dimensions (32 apart: lane g ^ 4 of the row's group of 8),
  // loaded rather than exchanged between lanes
  const int gp = 8 * ((g ^ 4) - g);
  const half8 qph = *(const half8*)(qrow + h * 64 + gp);
  const half8 kph = *(const half8*)(qrow + (ls.H + hk) * 64 + gp);
  // element offset of (cache row, KV head, entry 0, dimension 8g) in the local caches
  const size_t base = ((size_t)crow * ls.Hkv + hk) * ls.cap * 64 + 8 * g;
  half8 ch[8];  // cached keys 0..3, values 0..3 of the first group of four entries
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = min(u, max(s0 - 1, 0));  // clamped into the cached entries (masked below)
    ch[u] = *(const half8*)(ls.kc + base + (size_t)j * 64);
    ch[4 + u] = *(const half8*)(ls.vc + base + (size_t)j * 64);
  }
  const float rv = ((const float*)(ls.rope + (size_t)s0 * 32))[lane];
  // cross-attention operands: this lane's 8 dimensions of the query and, where the register
  // budget allows (8 waves: 256 registers a lane), of the first encoder state's key and value
  // (fp32) and the cross-attention weight tiles, issued with the rest
  constexpr bool XE = XA && NWAVE == 8;
  half8 xqh;
  float4 xk0[2], xv0[2];
  const float* xkb = nullptr;
  if constexpr (XA) {
    xqh = *(const half8*)(ls.qkv + (size_t)rc * ls.ldq + ls.xq_off + h * 64 + 8 * g);
    xkb = ls.xkv + (size_t)rc * ls.P * ls.xkv_ld + ls.xkv_off + hk * 64 + 8 * g;
  }
  if constexpr (XE) {
    xk0[0] = *(const float4*)xkb, xk0[1] = *(const float4*)(xkb + 4);
    xv0[0] = *(const float4*)(xkb + ls.Hkv * 64), xv0[1] = *(const float4*)(xkb + ls.Hkv * 64 + 4);
  }
  half8 rw[4], rwx[4];
  auto load_rwx = [&]() {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      rwx[ks] = *(const half8*)(W + (((size_t)ng * KS + ls.k_mlp / 32 + 4 * hp + ks) * 64 + lane) * 8);
  };
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) rw[ks] = *(const half8*)(W + (((size_t)ng * KS + 4 * hp + ks) * 64 + lane) * 8);
  if constexpr (XE) load_rwx();
  __builtin_amdgcn_sched_barrier(0);
  // each wave stages the rotary row in its own LDS slice (a wave's LDS accesses complete in order,
  // so no barrier: C1 decode 20.84 -> 20.76 ms against one staging for the workgroup)
  float* __restrict__ rope_s = lds + (XA ? 2 : 1) * LDS_A + 64 * wave;
  rope_s[lane] = rv;
  float cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float4 c = *(const float4*)(rope_s + 2 * ((8 * g) % 32) + 4 * e);
    cs[2 * e] = c.x, sn[2 * e] = c.y, cs[2 * e + 1] = c.z, sn[2 * e + 1] = c.w;
  }
  const bool first = g < 4;  // dimensions [0, 32): rotated with -sin
  const bool live = r < M;
  f16* __restrict__ at = (f16*)lds;  // A tiles [RG][4 K steps][512]
  float q[8], kn[8], vn[8], qpf[8], kpf[8];
  h8_to_f(qh, q);
  h8_to_f(kh, kn);
  h8_to_f(vh, vn);
  h8_to_f(qph, qpf);
  h8_to_f(kph, kpf);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float qp = __shfl_xor(q[e], 4, 64), kp = __shfl_xor(kn[e], 4, 64);
    q[e] = first ? q[e] * cs[e] - qp * sn[e] : q[e] * cs[e] + qp * sn[e];
    kn[e] = (float)to_f16(first ? kn[e] * cs[e] - kp * sn[e] : kn[e] * cs[e] + kp * sn[e]);
  }
  if (cp == 0 && live && h % G == 0) {
    half8 kw8;
#pragma unroll
    for (int e = 0; e < 8; ++e) kw8[e] = (f16)kn[e];
    *(half8*)(ls.kc + base + (size_t)s0 * 64) = kw8;
    *(half8*)(ls.vc + base + (size_t)s0 * 64) = vh;
  }
  // online softmax over the s0 cached keys (groups of four) and the new one (hardware exp2 of
  // differences from the running maximum, <= 0)
  float mrun = -INFINITY, lrun = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int j0 = 0; j0 < s0; j0 += 4) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + u, s0 - 1);
        ch[u] = *(const half8*)(ls.kc + base + (size_t)j * 64);
        ch[4 + u] = *(const half8*)(ls.vc + base + (size_t)j * 64);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float kv[8];
      h8_to_f(ch[u], kv);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(q[e], kv[e], dot);
      dot = sum8(dot);
      if (j0 + u < s0) {
        const float sc = dot * ls.scale_log2, mn = fmaxf(mrun, sc);
        const float corr = __builtin_amdgcn_exp2f(mrun - mn), p = __builtin_amdgcn_exp2f(sc - mn);
        h8_to_f(ch[4 + u], kv);
        lrun = lrun * corr + p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = o[e] * corr + p * kv[e];
        mrun = mn;
      }
    }
  }
  {
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(q[e], kn[e], dot);
    dot = sum8(dot);
    const float sc = dot * ls.scale_log2, mn = fmaxf(mrun, sc);
    const float corr = __builtin_amdgcn_exp2f(mrun - mn), p = __builtin_amdgcn_exp2f(sc - mn);
    lrun = lrun * corr + p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * corr + p * vn[e];
  }
  const float inv = live ? 1.0f / lrun : 0.f;
  half8 ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = to_f16_bounded(o[e] * inv);
  // A tile (row group lr / 16, K step 2 it + g / 4): element (row lr % 16, column 8 (g % 4) + e)
  *(half8*)(at + ((lr >> 4) * 4 + 2 * it + (g >> 2)) * 512 + ((g & 3) * 16 + (lr & 15)) * 8) = ov;
  if constexpr (XA) {
    // cross-attention of the same (row, head) over the P encoder states (no rotary embedding),
    // online softmax in base 2; the output goes to the second set of A tiles
    if constexpr (!XE) load_rwx();
    float xq[8];
    h8_to_f(xqh, xq);
    float xm = -INFINITY, xl = 0.f, xo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xo[e] = 0.f;
    for (int p = 0; p < ls.P; ++p) {
      float4 k4[2], v4[2];
      if (XE && p == 0) {
        k4[0] = xk0[0], k4[1] = xk0[1], v4[0] = xv0[0], v4[1] = xv0[1];
      } else {
        const float* kp = xkb + (size_t)p * ls.xkv_ld;
        k4[0] = *(const float4*)kp, k4[1] = *(const float4*)(kp + 4);
        v4[0] = *(const float4*)(kp + ls.Hkv * 64), v4[1] = *(const float4*)(kp + ls.Hkv * 64 + 4);
      }
      const float kk[8] = {k4[0].x, k4[0].y, k4[0].z, k4[0].w, k4[1].x, k4[1].y, k4[1].z, k4[1].w};
      const float vv[8] = {v4[0].x, v4[0].y, v4[0].z, v4[0].w, v4[1].x, v4[1].y, v4[1].z, v4[1].w};
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(xq[e], kk[e], dot);
      dot = sum8(dot);
      const float sc = dot * ls.scale_log2, mn = fmaxf(xm, sc);
      const float corr = __builtin_amdgcn_exp2f(xm - mn), pr = __builtin_amdgcn_exp2f(sc - mn);
      xl = xl * corr + pr;
#pragma unroll
      for (int e = 0; e < 8; ++e) xo[e] = xo[e] * corr + pr * vv[e];
      xm = mn;
    }
    const float xinv = live ? 1.0f / xl : 0.f;
    half8 xov;
#pragma unroll
    for (int e = 0; e < 8; ++e) xov[e] = to_f16_bounded(xo[e] * xinv);
    *(half8*)(at + LDS_A * 2 + ((lr >> 4) * 4 + 2 * it + (g >> 2)) * 512 + ((g & 3) * 16 + (lr & 15)) * 8) = xov;
  }
  __syncthreads();
  // the 16 x 16 output tiles (row groups rg0, rg0 + 1; column group ng) over the heads' 4 K steps
  const int rg0 = (wave >> 3) * 2;
  float4_ acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    acc[i] = float4_{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const half8*)(at + ((rg0 + i) * 4 + ks) * 512 + lane * 8),
                                                      rw[ks], acc[i], 0, 0, 0);
    if constexpr (XA) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            *(const half8*)(at + LDS_A * 2 + ((rg0 + i) * 4 + ks) * 512 + lane * 8), rwx[ks], acc[i], 0, 0, 0);
    }
  }
  const int col = ng * 16 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = rb * RB + (rg0 + i) * 16 + 4 * (lane >> 4) + e;
      if (row < M) ep.part[((size_t)hp * M + row) * N + col] = acc[i][e] * ep.wscale;
    }
}

template <int MG, int MW, int NG, int KW, bool XA>
static hipError_t launch_attn_out_cfg(const void* ACT, const void* W, int M, int N, int K, const Epi& ep,
                                      const LocalStep& ls, int mlp_splits, hipStream_t st) {
  constexpr int RB = 4 * MW * KW, RW = 16 * MG * MW;  // attention rows, GEMM rows per workgroup
  const int n_cp = N / 128, n_attn = (M + RB - 1) / RB * (ls.H / 2) * n_cp;
  const int n_gemm = N / (16 * NG) * mlp_splits * ((M + RW - 1) / RW), nb = n_attn + n_gemm, n_grp = n_attn / n_cp;
  const int spread = (n_grp + 7) / 8 * n_cp <= nb / 8;
  hipLaunchKernelGGL((k_attn_out<MG, MW, NG, KW, XA>), dim3(nb), dim3(64 * MW * KW), 0, st, (const f16*)ACT,
                     (const f16*)W, M, N, K, ep, ls, n_attn, n_cp, mlp_splits, spread);
  return hipGetLastError();
}

// Partial count of the fused launch (0: the shape does not run fused): H / 2 attention splits, and
// the GELU columns' K split so that attention and GEMM tiles together take at most about one
// workgroup per CU and each wave about 3 K steps (every split owning at least one K step, at most
// 16 partials).
// Workgroup shape of the fused launch: the skinny plan with all rows per workgroup up to 128 rows;
// above, 64-row GEMM workgroups (row groups) of 8 waves along K, and 32-row attention blocks.
static SkinnyPlan fused_plan(int M, int N, int K) {
  SkinnyPlan p = skinny_plan(M, N, K, EPI_RESID, false);
  if (p.ok && M > 128) p.mg = 4, p.mw = 1, p.ng = 2, p.kw = 8, p.rg = (M + 63) / 64;
  return p;
}

int attn_out_splits(int M, int N, int K, int H) {
  if (M < 1 || M > 256 || H < 2 || H % 2 || H > 30 || N != 64 * H || K <= N || (K - N) % 32) return 0;
  const SkinnyPlan p = fused_plan(M, N, K);
  if (!p.ok) return 0;
  const int rb = 4 * p.mw * p.kw, n_attn = (M + rb - 1) / rb * (H / 2) * (N / 128);
  const int slabs = N / (16 * p.ng) * ((M + 16 * p.mg * p.mw - 1) / (16 * p.mg * p.mw)), ks = (K - N) / 32;
  // (measured: fewer, longer splits win once each wave has about 3 K steps -- 64-row d=768 decode
  // 23.27 -> 23.10 ms at 4 splits instead of 7 -- the next LayerNorm then folds fewer partials; above
  // 128 rows the row groups already fill the chip and 2 splits beat 1, 3, 4 and 6: 256-row d=768
  // decode 583.5 -> 560.8 ms against 4, while 2 or 1 splits lose at 64 rows)
  int s = M > 128 ? 2 : std::min(16 - H / 2, std::max(1, (256 - n_attn) / slabs));
  s = std::min(s, std::max(1, ks / (3 * p.kw)));
  s = std::max(1, std::min(s, ks / p.kw));
  const int per = (ks + s - 1) / s;
  s = (ks + per - 1) / per;  // every split owns at least one K step
  return H / 2 + s;
}


hipError_t launch_attn_out_decode(const void* ACT, const void* W, int M, int N, int K, const Epi& ep,
                                  const LocalStep& ls, hipStream_t st) {
  const bool xa = ls.xkv != nullptr;
  const int total = attn_out_splits(M, N, xa ? ls.k_mlp : K, ls.H);
  if (total <= ls.H / 2 || total > 16 || !ep.part || ls.Hkv < 1 || ls.H % ls.Hkv || ls.s0 < 0 ||
      ls.s0 >= ls.cap || ls.ldq < (ls.H + 2 * ls.Hkv) * 64 || ls.ldq % 8)
    return hipErrorInvalidValue;
  if (xa && (ls.P < 1 || ls.k_mlp % 32 || ls.k_mlp + N != K || ls.xq_off % 8 || ls.xq_off + N > ls.ldq ||
             ls.xkv_ld % 4 || ls.xkv_off % 4))
    return hipErrorInvalidValue;
  const int mlp_splits = total - ls.H / 2;
  const SkinnyPlan p = fused_plan(M, N, xa ? ls.k_mlp : K);
#define BT_AO(MG, MW, NG, KW)                                                                               \
  if (p.mg == MG && p.mw == MW && p.ng == NG && p.kw == KW)                                               \
    return xa ? launch_attn_out_cfg<MG, MW, NG, KW, true>(ACT, W, M, N, K, ep, ls, mlp_splits, st)        \
              : launch_attn_out_cfg<MG, MW, NG, KW, false>(ACT, W, M, N, K, ep, ls, mlp_splits, st);
  BT_AO(1, 1, 2, 8)
  BT_AO(2, 1, 2, 8)
  BT_AO(4, 1, 2, 8)
  BT_AO(4, 2, 2, 4)
#undef BT_AO
  return hipErrorInvalidValue;
}

template <int MG, int MW, int NG, int KW, int DEPTH = 2>
static hipError_t launch_skinny_cfg(const void* A1, const void* A2, const void* W, int M, int N, int K, EpiMode mode,
                                    const Epi& ep, int S, int RG, hipStream_t st) {
  if (mode == EPI_ARGMAX && ep.nparts_out) *ep.nparts_out = N / (16 * NG);
  dim3 grid(N / (16 * NG), S, RG), block(64 * MW * KW);
  const f16 *a1 = (const f16*)A1, *a2 = (const f16*)A2, *w = (const f16*)W;
  switch (mode) {
    case EPI_QKV_GELU:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_QKV_GELU, DEPTH>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_RESID:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_RESID, DEPTH>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_STORE:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_STORE, DEPTH>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((k_gemm_skinny<MG, MW, NG, KW, EPI_ARGMAX, DEPTH>), grid, block, 0, st, a1, a2, w, M, N, K, ep);
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
SkinnyPlan skinny_plan(int M, int N, int K, EpiMode mode, bool row_groups) {
  SkinnyPlan p{};
  p.splits = 1;
  // The classifier of a batch above 64 rows has enough MFMA work to prefer the LDS-tiled kernels
  // (65-128 rows, 128 x 128 tiles, weights streamed from HBM: 26.4-28.4 instead of 32.9-36.7 us at
  // K = 768 and 57.8-58.8 instead of 68.6-73.6 us at K = 2048, vocabulary 50432).
  const bool tiled_head = mode == EPI_ARGMAX && M > 64 && N % 128 == 0 && K % 64 == 0;
  p.ok = M >= 1 && M <= 256 && N % 32 == 0 && K % 32 == 0 && !(mode == EPI_ARGMAX && M > 128) && !tiled_head;
  if (!p.ok) return p;
  const int mgt = (M + 15) / 16;
  if (row_groups && M > 128 && (mode == EPI_QKV_GELU || mode == EPI_RESID)) {
    // Above 128 rows every workgroup of the all-rows tile re-reads the whole activation operand
    // (256 rows x K) and too few of them fill the CUs: 64-row workgroups, 4 waves along K, three K
    // steps in flight.  Measured at 256 rows, weights streamed from HBM: [q|k|v|up] (5376 x 768)
    // 9.2 instead of 11.7 us per launch (7.8 instead of 9.3 from the Infinity Cache); [out|down]
    // (768 x 3840, 8 K splits) 8.1 instead of 9.1 us.
    p.mg = 4, p.mw = 1, p.ng = 2, p.kw = 4, p.depth = 3, p.rg = (M + 63) / 64;
    if (mode == EPI_RESID) {
      const int ks = K / 32, s = std::max(1, std::min(8, ks / p.kw)), per = (ks + s - 1) / s;
      p.splits = (ks + per - 1) / per;  // every split owns at least one K step
    }
    return p;
  }
  if (mode == EPI_ARGMAX && mgt > 2 && mgt <= 4) {
    // the classifier at 33-64 rows: 64 columns per workgroup over 2 waves along K, three K steps in
    // flight (measured at 64 rows x 50432 x 768, weights from HBM: 21.4 instead of 24.3 us)
    p.mg = 4, p.mw = 1, p.ng = 4, p.kw = 2, p.depth = 3;
    return p;
  }
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
  if (row_groups && mgt > 4 && mgt <= 8 &&
      ((mode == EPI_QKV_GELU && N % 64 == 0 && N / 64 >= 128) || (mode == EPI_RESID && N % 64 == 0 && N >= 2048))) {
    // 65-128 rows of a wide model: every byte a workgroup loads passes its CU's load path, which
    // bounds these launches (two row waves each loading the same weight tile, plus the activation
    // tile every slab re-reads).  One wave holds all 128 rows (no weight tile loaded twice) over 64
    // columns, 4 waves along K, and the [out|down] GEMM splits K 8 ways so that about 256 of these
    // workgroups stream its weights.  Measured on the 1.2B model's decode (128 rows, d = 2048):
    // 2648 -> 2460 ms per generation; [out|down] 22.5 -> 16.5 us per launch, [q|k|v|up] 22.3 -> 21.6.
    p.mg = 8, p.mw = 1, p.ng = 4, p.kw = 4;
    if (mode == EPI_RESID) {
      const int s = std::max(1, std::min(std::min(16, 256 / (N / 64)), ks / p.kw)), per = (ks + s - 1) / s;
      p.splits = (ks + per - 1) / per;
    }
  }
  return p;
}

hipError_t launch_gemm_skinny(const SkinnyPlan& p, const void* A1, const void* A2, const void* W, int M, int N, int K,
                              EpiMode mode, const Epi& ep, hipStream_t st) {
  const int S = mode == EPI_RESID ? ep.splits : 1;
  const int RG = std::max(1, p.rg);
  if (RG * 16 * p.mg * p.mw < M) return hipErrorInvalidValue;  // the row groups must cover every row
#define BT_SKINNY(MG, MW, NG, KW, D) \
  if (p.mg == MG && p.mw == MW && p.ng == NG && p.kw == KW && p.depth == D)   \
    return launch_skinny_cfg<MG, MW, NG, KW, D>(A1, A2, W, M, N, K, mode, ep, S, RG, st);
  BT_SKINNY(1, 1, 2, 8, 2)
  BT_SKINNY(2, 1, 2, 8, 2)
  BT_SKINNY(4, 1, 2, 8, 2)
  BT_SKINNY(4, 2, 2, 4, 2)
  BT_SKINNY(4, 2, 4, 4, 2)
  BT_SKINNY(4, 4, 2, 4, 2)
  BT_SKINNY(4, 1, 2, 4, 3)
  BT_SKINNY(4, 1, 4, 2, 3)
  BT_SKINNY(8, 1, 4, 4, 2)
#undef BT_SKINNY
  return hipErrorInvalidValue;
}

BT_DEFINE_CLAMP_FLAG_ACCESS(clamp_flag_gemm_decode)

}  // namespace bt
