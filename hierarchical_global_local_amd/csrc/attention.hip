// Attention kernels of libbt.
//
//  * k_rope_scatter: rotary embedding of prompt keys and scatter of K / V into the block-KV cache
//    (keys [slot][dh]; values in groups of 8 slots, each group transposed [dh][8], so that the
//    prefill P*V product and the decode value passes read 8 consecutive keys per 16-byte load).
//  * k_flash_prefill2: causal flash attention over block positions with MFMA (fp16 operands, fp32
//    softmax); computes S^T = K Q^T so that the probabilities come out of the MFMA already in the
//    operand layout of O^T = V^T P^T, with no LDS round trip.
//  * k_attn_decode_wave: memory-bound block-attention decode, fp16 multi-head: one wave per (row,
//    head, key split) streams a step's K and V^T together with 16-byte loads, wave-shuffle dot
//    products, online softmax in registers; split-KV partials merged by k_attn_combine with
//    log-sum-exp weights.  k_attn_decode (fp32, groups above 16 heads): one workgroup per unit,
//    K then V^T, softmax through LDS; k_attn_decode_mfma: grouped-query heads on MFMA.
//  * k_local_attn_step: the token decoder's local attention for one new slot (decode), one wave
//    per (row, head) with keys spread over lane groups, everything in registers;
//    k_local_attn: the same over several new slots (prefill tail), entries held in LDS.
//  * k_attn_naive: plain prefill attention for fp32 mode.
#include "bt_internal.h"
#include "device_common.h"

namespace bt {

constexpr float kLog2e = 1.4426950408889634f;
// Softmax weights use the hardware exp2 (__builtin_amdgcn_exp2f, v_exp_f32) directly: every
// argument is a difference from a running or final maximum (<= 0, or -inf giving 0), where the
// library exp2f only adds a denormal-range fix-up (compare, select, ldexp); a weight below 2^-126
// of the largest one is negligible.

// 8 consecutive elements as floats
__device__ __forceinline__ void load8(const f16* p, float* o) {
  half8 v = *(const half8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// the same with non-temporal loads (block-KV streams: they must not evict cached weights)
__device__ __forceinline__ void load8_nt(const f16* p, float* o) {
  half8 v = __builtin_nontemporal_load((const half8*)p);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void load8_nt(const float* p, float* o) {
  const float4_ a = __builtin_nontemporal_load((const float4_*)p), b = __builtin_nontemporal_load((const float4_*)(p + 4));
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = a[e], o[4 + e] = b[e];
}

template <typename T>
__device__ __forceinline__ T round_t(float v) { return from_f32<T>(v); }

// ---------------------------------------------------------------- block-KV addressing
// Entry j of cache row r, KV head hk: flat caches hold keys [row][head][cap][dh] and values in
// groups of 8 entries, each group transposed: [row][head][cap / 8][dh][8]; paged caches (ptab set)
// hold pages of 64 entries, keys [page][head][64][dh] and values [page][head][8][dh][8], entry j of
// row r in page ptab[r*pld + j/64].  A 16-byte load (fp16) takes 8 consecutive entries of one value
// dimension -- the operand shape of the P*V products -- while appending one entry touches the
// group's dh * 16 contiguous bytes instead of one cache line per dimension.
// nlim (paged prefill): entries at or past nlim[r] are not written or read (their pages may not
// exist).
struct KvPages {
  const int* ptab;
  int pld;
  const int* nlim;
};
__device__ __forceinline__ size_t kv_key(const KvPages& pg, int r, int hk, int j, int Hkv, int cap, int dh) {
  return pg.ptab ? (((size_t)pg.ptab[(size_t)r * pg.pld + (j >> 6)] * Hkv + hk) * 64 + (j & 63)) * dh
                 : (((size_t)r * Hkv + hk) * cap + j) * dh;
}
__device__ __forceinline__ size_t kv_val(const KvPages& pg, int r, int hk, int d, int j, int Hkv, int cap, int dh) {
  return pg.ptab ? ((((size_t)pg.ptab[(size_t)r * pg.pld + (j >> 6)] * Hkv + hk) * 8 + ((j & 63) >> 3)) * dh + d) * 8 +
                       (j & 7)
                 : ((((size_t)r * Hkv + hk) * (cap >> 3) + (j >> 3)) * dh + d) * 8 + (j & 7);
}

// ---------------------------------------------------------------- rotary + scatter (prefill)
// grid (ceil(m/64), Hkv, B); KV head hk of rows (b, i) of QKV [B*m][QW] goes to cache slot s0 + i.
template <typename T>
__global__ __launch_bounds__(256) void k_rope_scatter(const T* __restrict__ QKV, int m, int s0, int H, int Hkv, int dh,
                                                      const float2* __restrict__ rope, T* __restrict__ Kc,
                                                      T* __restrict__ Vc, int cap, int vt, const int* __restrict__ rmap,
                                                      KvPages pg) {
  __shared__ T vtile[64][129];
  const int hk = blockIdx.y, b = blockIdx.z, i0 = blockIdx.x * 64;
  const int half = dh / 2, tid = threadIdx.x;
  const size_t qw = (size_t)(H + 2 * Hkv) * dh, koff = (size_t)(H + hk) * dh, voff = (size_t)(H + Hkv + hk) * dh;
  const int cb = rmap ? rmap[b] : b;
  const size_t bh = (size_t)cb * Hkv + hk;
  // slots past the row's length (paged ragged prefill) are skipped
  const int cnt = min(64, min(m, pg.nlim ? pg.nlim[cb] - s0 : m) - i0);
  if (cnt <= 0) return;
  for (int e = tid; e < cnt * half; e += 256) {
    const int si = e / half, c = e % half, i = i0 + si, slot = s0 + i;
    const T* kr = QKV + ((size_t)b * m + i) * qw + koff;
    const float2 cs = rope[(size_t)slot * half + c];
    const float x1 = (float)kr[c], x2 = (float)kr[c + half];
    T* kd = Kc + kv_key(pg, cb, hk, slot, Hkv, cap, dh);
    kd[c] = round_t<T>(x1 * cs.x - x2 * cs.y);
    kd[c + half] = round_t<T>(x2 * cs.x + x1 * cs.y);
  }
  if (!vt) {
    for (int e = tid; e < cnt * dh; e += 256) {
      const int si = e / dh, d = e % dh, i = i0 + si;
      Vc[(bh * cap + s0 + i) * dh + d] = QKV[((size_t)b * m + i) * qw + voff + d];
    }
    return;
  }
  for (int e = tid; e < cnt * dh; e += 256) {
    const int si = e / dh, d = e % dh;
    vtile[si][d] = QKV[((size_t)b * m + i0 + si) * qw + voff + d];
  }
  __syncthreads();
  for (int e = tid; e < cnt * dh; e += 256) {
    const int d = e / cnt, si = e % cnt;
    Vc[kv_val(pg, cb, hk, d, s0 + i0 + si, Hkv, cap, dh)] = vtile[si][d];
  }
}

// fp16 block cache, slot offset s0 % 8 == 0: the same with 16-byte accesses.
// Keys: a thread takes 8 dimensions and their rotary partners (8 further by DH / 2) of one slot,
// with the 8 (cos, sin) pairs as 4 16-byte loads.  Values: the 64 x DH tile goes through LDS and
// leaves as 16-byte runs of 8 slots per dimension, one value group at a time (element stores for a
// ragged last run).
template <int DH>
__global__ __launch_bounds__(256) void k_rope_scatter_v(const f16* __restrict__ QKV, int m, int s0, int H, int Hkv,
                                                        const float2* __restrict__ rope, f16* __restrict__ Kc,
                                                        f16* __restrict__ Vc, int cap, const int* __restrict__ rmap,
                                                        KvPages pg) {
  constexpr int NC = DH / 8, HALF = DH / 2, VLD = DH + 8;
  __shared__ __attribute__((aligned(16))) f16 vtile[64 * VLD];
  const int hk = blockIdx.y, b = blockIdx.z, i0 = blockIdx.x * 64, tid = threadIdx.x;
  const size_t qw = (size_t)(H + 2 * Hkv) * DH, koff = (size_t)(H + hk) * DH, voff = (size_t)(H + Hkv + hk) * DH;
  const int cb = rmap ? rmap[b] : b;
  const int cnt = min(64, min(m, pg.nlim ? pg.nlim[cb] - s0 : m) - i0);
  if (cnt <= 0) return;
  // keys: items (slot si, chunk pair p < NC / 2)
  uint32_t trk = 0u;
  for (int e = tid; e < cnt * (NC / 2); e += 256) {
    const int si = e / (NC / 2), p = e % (NC / 2), slot = s0 + i0 + si;
    const f16* kr = QKV + ((size_t)b * m + i0 + si) * qw + koff + 8 * p;
    const half8 a = *(const half8*)kr, c = *(const half8*)(kr + HALF);
    const float4* rp = (const float4*)(rope + (size_t)slot * HALF + 8 * p);
    half8 oa, oc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 r = rp[q];  // (cos, sin) of dimensions 8p + 2q and 8p + 2q + 1
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e2 = 2 * q + u;
        const float cs = u ? r.z : r.x, sn = u ? r.w : r.y;
        const float x1 = (float)a[e2], x2 = (float)c[e2];
        oa[e2] = to_f16_trk(x1 * cs - x2 * sn, trk);
        oc[e2] = to_f16_trk(x2 * cs + x1 * sn, trk);
      }
    }
    f16* kd = Kc + kv_key(pg, cb, hk, slot, Hkv, cap, DH) + 8 * p;
    *(half8*)kd = oa;
    *(half8*)(kd + HALF) = oc;
  }
  clamp_note(trk);
  // values: rows of the tile into LDS (16 bytes per item), then 8-slot runs per dimension
  for (int e = tid; e < cnt * NC; e += 256) {
    const int si = e / NC, c = e % NC;
    *(half8*)(vtile + si * VLD + 8 * c) = *(const half8*)(QKV + ((size_t)b * m + i0 + si) * qw + voff + 8 * c);
  }
  __syncthreads();
  const int runs = (cnt + 7) / 8;
  for (int e = tid; e < DH * runs; e += 256) {  // consecutive threads: consecutive dimensions of a group
    const int d = e % DH, q = e / DH, n8 = min(8, cnt - 8 * q);
    f16* vd = Vc + kv_val(pg, cb, hk, d, s0 + i0 + 8 * q, Hkv, cap, DH);
    if (n8 == 8) {
      half8 w;
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = vtile[(8 * q + u) * VLD + d];
      *(half8*)vd = w;
    } else {
      for (int u = 0; u < n8; ++u) vd[u] = vtile[(8 * q + u) * VLD + d];
    }
  }
}

hipError_t launch_rope_scatter(bool f32, const void* QKV, int B, int m, int s0, int H, int Hkv, int dh,
                               const float2* rope, void* Kc, void* Vc, int cap, bool v_transposed, hipStream_t st,
                               const int* rmap, const int* ptab, int pld, const int* nlim) {
  if (B <= 0 || m <= 0) return hipSuccess;
  if (Hkv < 1 || H % Hkv || (ptab && !v_transposed)) return hipErrorInvalidValue;
  const KvPages pg{ptab, pld, nlim};
  dim3 grid((m + 63) / 64, Hkv, B);
  if (!f32 && v_transposed && s0 % 8 == 0 && cap % 8 == 0 && (dh == 64 || dh == 128)) {
    if (dh == 64)
      hipLaunchKernelGGL(k_rope_scatter_v<64>, grid, dim3(256), 0, st, (const f16*)QKV, m, s0, H, Hkv, rope, (f16*)Kc,
                         (f16*)Vc, cap, rmap, pg);
    else
      hipLaunchKernelGGL(k_rope_scatter_v<128>, grid, dim3(256), 0, st, (const f16*)QKV, m, s0, H, Hkv, rope, (f16*)Kc,
                         (f16*)Vc, cap, rmap, pg);
    return hipGetLastError();
  }
  if (f32)
    hipLaunchKernelGGL(k_rope_scatter<float>, grid, dim3(256), 0, st, (const float*)QKV, m, s0, H, Hkv, dh, rope,
                       (float*)Kc, (float*)Vc, cap, (int)v_transposed, rmap, pg);
  else
    hipLaunchKernelGGL(k_rope_scatter<f16>, grid, dim3(256), 0, st, (const f16*)QKV, m, s0, H, Hkv, dh, rope,
                       (f16*)Kc, (f16*)Vc, cap, (int)v_transposed, rmap, pg);
  return hipGetLastError();
}

// ---------------------------------------------------------------- MFMA flash prefill (fp16)
// The query tiles of one (row, head) run on one XCD, consecutively and longest first, so that the
// row's keys and values come from that XCD's L2 after the first tile instead of from HBM.  Each
// 64-key tile of K ([key][dh]) and V^T ([dh][key]) is loaded once per workgroup with coalesced
// 16-byte loads into a double-buffered LDS stage (the next tile's loads are in flight while the
// current one is used) and read by all four waves.  S^T = K Q^T, so that the probabilities come out
// of the MFMA already in the operand layout of O^T = V^T P^T.  MFMA 16x16x32 layouts (lane l,
// g = l / 16):
//   A operand: row l % 16, k = 8g..8g+7;  B operand: column l % 16, same k;
//   result:    column l % 16, rows 4g..4g+3.
// MFMA flash prefill with QG 16-query groups per wave (32 queries at head width 64): each key and
// value fragment read from LDS serves every group, so the LDS traffic per MFMA drops by QG against
// 16 queries per wave, and the per-tile softmax bookkeeping (running maxima, rescaling) is amortised
// over QG times the scores.  grid ceil(n / (64 QG)) * H * B, 4 waves.  Further:
//  * values are stored in LDS with the keys of each 32-key slice permuted so that the 8 keys a lane
//    contributes to a P * V MFMA (keys 4g..4g+3 and 16+4g..16+4g+3 of the slice, the probabilities
//    it holds) are contiguous: one 16-byte LDS read per value fragment;
//  * the row sums come from an MFMA of a ones operand with the probabilities (no per-score adds);
//  * the score MFMAs start from minus a per-query offset (the running maximum as of the last
//    rescale), so no subtraction precedes the exp2, and the accumulators are rescaled only when a
//    score exceeds its offset by more than 2^8 (probabilities up to 256 in fp16), not whenever a
//    running maximum grows: the exp2 and the fp16 conversion are most of the per-score VALU work,
//    which bounds this kernel at head width 64;
//  * the per-lane maxima use the three-operand maximum (no quieting of the MFMA results);
//  * a wave skips the key tiles that lie entirely after its last query.
template <int DH, int QG>
__global__ __launch_bounds__(256) void k_flash_prefill2(const f16* __restrict__ QKV, int n, int H, int Hkv,
                                                        const float2* __restrict__ rope, const f16* __restrict__ Kc,
                                                        const f16* __restrict__ VTc, int cap, f16* __restrict__ ACT,
                                                        int ld_act, float scale_log2, const int* __restrict__ rmap,
                                                        KvPages pg) {
  constexpr int KS = DH / 32;   // 32-wide dh slices of q and k
  constexpr int MT = DH / 16;   // 16-row dh tiles of O^T
  constexpr int QT = 64 * QG;   // queries per workgroup (QG 16-query groups per wave)
  constexpr int KLD = DH + 8;   // LDS row strides (+16 B)
  constexpr int VLD = 64 + 8;
  constexpr int CK = 64 * DH / 8 / 256;  // 16-byte chunks per thread of a K tile
  constexpr int CV = DH * 64 / 8 / 256;  // ... and of a V^T tile
  __shared__ __attribute__((aligned(16))) f16 Ks[2][64 * KLD];
  __shared__ __attribute__((aligned(16))) f16 Vs[2][DH * VLD];

  const int nq = (n + QT - 1) / QT, lt = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int pair = lt / nq, qt = nq - 1 - lt % nq;  // longest (latest) query tiles first
  const int h = pair % H, b = pair / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int qw0 = qt * QT + wave * 16 * QG;  // first query of this wave
  const int cb = rmap ? rmap[b] : b, hk = h / (H / Hkv);
  if (pg.nlim && qt * QT >= pg.nlim[cb]) return;  // queries past the row's length: nothing reads them

  half8 rk[CK], rv[CV];
  auto gload = [&](int kb) {
    const f16* __restrict__ Kt = Kc + kv_key(pg, cb, hk, kb, Hkv, cap, DH);
    const f16* __restrict__ Vt = VTc + kv_val(pg, cb, hk, 0, kb, Hkv, cap, DH);
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256, r = c / (DH / 8), cc = c % (DH / 8);
      rk[i] = *(const half8*)(Kt + (size_t)r * DH + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int c = tid + i * 256, r = c % DH, cc = c / DH;
      rv[i] = *(const half8*)(Vt + ((size_t)cc * DH + r) * 8);
    }
  };
  // value chunk cc (keys 8cc..8cc+7 of dimension r): its first four keys go to LDS column base,
  // the last four to base + 8, base = 32 (cc / 4) + 16 (cc % 2) + 4 ((cc / 2) % 2)
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * 256, r = c / (DH / 8), cc = c % (DH / 8);
      *(half8*)&Ks[buf][r * KLD + cc * 8] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int c = tid + i * 256, r = c % DH, cc = c / DH;
      const int base = 32 * (cc >> 2) + 16 * (cc & 1) + 4 * ((cc >> 1) & 1);
      half4 lo4, hi4;
#pragma unroll
      for (int e = 0; e < 4; ++e) lo4[e] = rv[i][e], hi4[e] = rv[i][4 + e];
      *(half4*)&Vs[buf][r * VLD + base] = lo4;
      *(half4*)&Vs[buf][r * VLD + base + 8] = hi4;
    }
  };

  float4_ o[QG][MT];
#pragma unroll
  for (int grp = 0; grp < QG; ++grp)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[grp][mt] = float4_{0.f, 0.f, 0.f, 0.f};
  // Scores are taken relative to an offset mref per query: the exact running maximum as of the last
  // rescale (0 before the first tile).  The score MFMAs start from -mref, so they produce s - mref
  // directly, and a tile is rescaled only when one of its scores exceeds mref by more than
  // kSlackLog2 (or on the first tile, which sets mref exactly); otherwise its probabilities
  // exp2(s - mref) are at most 2^kSlackLog2, well inside fp16, and the running sums stay as they are.
  // The normalised output is the same softmax; only the common factor of each query's numerator and
  // denominator differs.  The row sums accumulate on the MFMA: a 16 x 32 operand of ones times P^T
  // gives, in every lane, the sum of its query's 32 probabilities of the slice (the same fp16 values
  // the P * V product uses).
  constexpr float kSlackLog2 = 8.f;
  float mref[QG];
  float4_ lacc[QG];
#pragma unroll
  for (int grp = 0; grp < QG; ++grp) mref[grp] = 0.f, lacc[grp] = float4_{0.f, 0.f, 0.f, 0.f};
  half8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (f16)1.0f;
  const int kmax = min(n, qt * QT + QT) - 1;                  // last key any query here needs
  const int ntiles = kmax / 64 + 1;
  const int wtiles = qw0 <= kmax ? min(qw0 + 16 * QG - 1, kmax) / 64 + 1 : 0;  // tiles this wave uses

  gload(0);  // the first key / value tile is in flight while the queries are prepared
  // q^T fragments (rotary and softmax scale folded in), one set per query group
  half8 qf[QG][KS];
#pragma unroll
  for (int grp = 0; grp < QG; ++grp) {
    const int qrow = min(qw0 + 16 * grp + c16, n - 1);
    float x[KS][8];
    const f16* qp = QKV + ((size_t)b * n + qrow) * (H + 2 * Hkv) * DH + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load8(qp + 32 * ks + 8 * g, x[ks]);
    const float2* rp = rope + (size_t)qrow * (DH / 2);
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = rp[32 * ks + 8 * g + e];
        const float x1 = x[ks][e], x2 = x[ks + KS / 2][e];
        qf[grp][ks][e] = to_f16_bounded((x1 * cs.x - x2 * cs.y) * scale_log2);
        qf[grp][ks + KS / 2][e] = to_f16_bounded((x2 * cs.x + x1 * cs.y) * scale_log2);
      }
  }

  sstore(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1, kb = t * 64;
    if (t + 1 < ntiles) gload(kb + 64);
    if (t < wtiles) {
      float4_ s[QG][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        half8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const half8*)&Ks[buf][(nt * 16 + c16) * KLD + 32 * ks + 8 * g];
#pragma unroll
        for (int grp = 0; grp < QG; ++grp) {
          s[grp][nt] = float4_{-mref[grp], -mref[grp], -mref[grp], -mref[grp]};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            s[grp][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], qf[grp][ks], s[grp][nt], 0, 0, 0);
        }
      }
      if (kb + 63 > qw0) {  // the tile reaches past the wave's first query: causal mask
#pragma unroll
        for (int grp = 0; grp < QG; ++grp)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              s[grp][nt][i] = kb + nt * 16 + 4 * g + i <= qw0 + 16 * grp + c16 ? s[grp][nt][i] : -INFINITY;
      }
#pragma unroll
      for (int grp = 0; grp < QG; ++grp) {
        // (elementwise maximum: three-operand instructions, no quieting of the MFMA results)
        float mx = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, s[grp][nt][0]),
                                             __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[grp][nt][1], s[grp][nt][2]),
                                                                           s[grp][nt][3]));
        if (t == 0 || __ballot(mx > kSlackLog2) != 0ull) {
          // every key tile of a wave holds a valid key for each of its queries, so the maximum is finite
          mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 16, 64));
          mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32, 64));
          const float d = t == 0 ? mx : fmaxf(mx, 0.f);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[grp][nt][i] -= d;
          if (t != 0 && __ballot(d > 0.f) != 0ull) {
            const float corr = __builtin_amdgcn_exp2f(-d);  // exactly 1 where d = 0
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) o[grp][mt] *= corr;
            lacc[grp] *= corr;
          }
          mref[grp] += d;
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[grp][nt][i] = __builtin_amdgcn_exp2f(s[grp][nt][i]);
      }
      // O^T += V^T P^T over two 32-key slices
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        half8 pf[QG];
#pragma unroll
        for (int grp = 0; grp < QG; ++grp)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pf[grp][e] = (f16)s[grp][2 * sl][e];
            pf[grp][4 + e] = (f16)s[grp][2 * sl + 1][e];
          }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const half8 vf = *(const half8*)&Vs[buf][(mt * 16 + c16) * VLD + 32 * sl + 8 * g];
#pragma unroll
          for (int grp = 0; grp < QG; ++grp)
            o[grp][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[grp], o[grp][mt], 0, 0, 0);
        }
#pragma unroll
        for (int grp = 0; grp < QG; ++grp)
          lacc[grp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[grp], lacc[grp], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int grp = 0; grp < QG; ++grp) {
    const int qi = qw0 + 16 * grp + c16;
    if (qi < n) {
      const float inv = 1.0f / lacc[grp][0];
      const int row = b * n + qi;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        store4_bounded(ACT, frag_off(row, h * DH + mt * 16 + 4 * g, ld_act), o[grp][mt][0] * inv,
                       o[grp][mt][1] * inv, o[grp][mt][2] * inv, o[grp][mt][3] * inv);
    }
  }
}

// ---------------------------------------------------------------- plain prefill attention (fp32)
// grid (n, H, B), one wave per query; scores staged in dynamic LDS.
template <typename T>
__global__ __launch_bounds__(64) void k_attn_naive(const T* __restrict__ QKV, int n, int H, int Hkv, int dh,
                                                   const float2* __restrict__ rope, const T* __restrict__ Kc,
                                                   const T* __restrict__ VTc, int cap, T* __restrict__ ACT,
                                                   int ld_act, float scale, const int* __restrict__ rmap,
                                                   KvPages pg) {
  extern __shared__ float sm[];
  float* q = sm;          // [dh]
  float* sc = sm + 128;   // [n]
  const int qi = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int cb = rmap ? rmap[b] : b, hk = h / (H / Hkv);
  if (pg.nlim && qi >= pg.nlim[cb]) return;
  const T* qp = QKV + ((size_t)b * n + qi) * (H + 2 * Hkv) * dh + h * dh;
  const int half = dh / 2;
  for (int c = lane; c < half; c += 64) {
    const float2 cs = rope[(size_t)qi * half + c];
    const float x1 = (float)qp[c], x2 = (float)qp[c + half];
    q[c] = x1 * cs.x - x2 * cs.y;
    q[c + half] = x2 * cs.x + x1 * cs.y;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = lane; j <= qi; j += 64) {
    const T* kp = Kc + kv_key(pg, cb, hk, j, Hkv, cap, dh);
    float d = 0.f;
    for (int e = 0; e < dh; ++e) d = fmaf(q[e], (float)kp[e], d);
    sc[j] = d * scale;
    mx = fmaxf(mx, d * scale);
  }
  mx = wave_max(mx);
  float l = 0.f;
  for (int j = lane; j <= qi; j += 64) {
    float p = expf(sc[j] - mx);
    sc[j] = p;
    l += p;
  }
  l = wave_sum(l);
  __syncthreads();
  for (int d = lane; d < dh; d += 64) {
    float o = 0.f;
    for (int j = 0; j <= qi; ++j) o = fmaf(sc[j], (float)VTc[kv_val(pg, cb, hk, d, j, Hkv, cap, dh)], o);
    ACT[opnd_idx(ACT, b * n + qi, h * dh + d, ld_act)] = round_t<T>(o / l);
  }
}

hipError_t launch_prefill_attention(bool f32, const void* QKV, int B, int n, int H, int Hkv, int dh,
                                    const float2* rope, const void* Kc, const void* Vc, int cap, void* ACT,
                                    int ld_act, hipStream_t st, const int* rmap, const int* ptab, int pld,
                                    const int* nlim) {
  if (B <= 0 || n <= 0) return hipSuccess;
  if (Hkv < 1 || H % Hkv) return hipErrorInvalidValue;
  const KvPages pg{ptab, pld, nlim};
  const float scale = 1.0f / sqrtf((float)dh);
  if (f32) {
    size_t lds = (128 + (size_t)n) * sizeof(float);
    hipLaunchKernelGGL(k_attn_naive<float>, dim3(n, H, B), dim3(64), lds, st, (const float*)QKV, n, H, Hkv, dh, rope,
                       (const float*)Kc, (const float*)Vc, cap, (float*)ACT, ld_act, scale, rmap, pg);
    return hipGetLastError();
  }
  // 32 queries per wave (measured faster than 16 at 512 and 8192 positions)
  if (dh == 64)
    hipLaunchKernelGGL((k_flash_prefill2<64, 2>), dim3((n + 127) / 128 * H * B), dim3(256), 0, st, (const f16*)QKV, n,
                       H, Hkv, rope, (const f16*)Kc, (const f16*)Vc, cap, (f16*)ACT, ld_act, scale * kLog2e, rmap, pg);
  else if (dh == 128)
    hipLaunchKernelGGL((k_flash_prefill2<128, 2>), dim3((n + 127) / 128 * H * B), dim3(256), 0, st, (const f16*)QKV, n,
                       H, Hkv, rope, (const f16*)Kc, (const f16*)Vc, cap, (f16*)ACT, ld_act, scale * kLog2e, rmap, pg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------- block-attention decode
// grid (nsplit, Hkv * nsub, B), 256 threads.  A workgroup serves gsz <= GM query heads of one KV
// head (the group of G = H / Hkv heads is cut into nsub runs of gsz), so that the KV head's keys
// and values are streamed from HBM once for all of them.  Keys [0, n) come from the cache, key n
// is the new one (rotated here, appended to the cache by split 0 of the group's first run, and
// used from LDS by the split that owns it).
constexpr int kMaxChunk = 4096;  // scores held in LDS per workgroup, over all its query heads
constexpr int kMaxSplit = 128;   // with GM = 4 (chunks of 1024 keys): the 131072-entry capacity limit

template <typename T, int DH, int GM, bool PAGED>
__global__ __launch_bounds__(256) void k_attn_decode(const T* __restrict__ QKV, const int* __restrict__ n_ptr, int H,
                                                     int Hkv, int gsz, const float2* __restrict__ rope,
                                                     T* __restrict__ Kc, T* __restrict__ VTc, int cap,
                                                     T* __restrict__ ACT, int ld_act, float* __restrict__ part,
                                                     int nsplit, int chunk, float scale_log2,
                                                     const int* __restrict__ ptab, int pld) {
  static_assert(GM >= 1 && GM <= 4, "one wave scores each head's new key");
  constexpr int LPK = DH / 8;      // lanes per key in the score pass (8 values each)
  constexpr int KPW = 64 / LPK;    // keys per wave per step
  constexpr int RPL = DH / 32;     // value rows per lane in the value pass
  constexpr int U = 8;             // key loads in flight per lane (score pass)
  constexpr int UV = (GM > 1 && DH == 128) ? 2 : 4;  // value-chunk loads in flight per lane and row
  __shared__ float qs[GM][DH], kn[DH], vn[DH];
  __shared__ __attribute__((aligned(16))) float sc[kMaxChunk + 8];  // [GM][chunk]
  __shared__ float red[GM][8];
  __shared__ int pgs[PAGED ? kMaxChunk / 64 : 1];  // pages of this split's keys (paged cache)
  const int s = blockIdx.x, b = blockIdx.z;
  const int G = H / Hkv, nsub = (G + gsz - 1) / gsz;
  const int hk = blockIdx.y / nsub, run = blockIdx.y % nsub;
  const int h0 = hk * G + run * gsz, gcnt = min(gsz, G - run * gsz);  // query heads [h0, h0 + gcnt)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // entries already cached in this row; the new one goes to slot n (the host keeps every row below
  // the capacity; the clamp only keeps a misused row inside its own cache)
  const int n = min(n_ptr[b], cap - 1);
  const size_t bk = (size_t)b * Hkv + hk;
  T* __restrict__ K = Kc + bk * cap * DH;  // (flat cache)
  T* __restrict__ VT = VTc + bk * DH * cap;
  const int j0 = s * chunk, j1 = min(n + 1, j0 + chunk);  // this split's keys [j0, j1)
  const int jc_end = min(j1, n);                           // of which cached: [j0, jc_end)
  const bool owns_new = (n >= j0 && n < j1);
  const bool appends = s == 0 && run == 0;
  // paged: key j at Kc[((page * Hkv + hk) * 64 + j % 64) * DH], value (d, j) at
  // VTc[(((page * Hkv + hk) * 8 + j % 64 / 8) * DH + d) * 8 + j % 8], page = pgs[(j - j0) / 64]
  // (j0 % 64 == 0)
  if (PAGED)
    for (int k = threadIdx.x; k < chunk / 64 && j0 / 64 + k < pld; k += 256) pgs[k] = ptab[(size_t)b * pld + j0 / 64 + k];
  auto kaddr = [&](int j) -> const T* {
    if (!PAGED) return K + (size_t)j * DH;
    return Kc + (((size_t)pgs[(j - j0) >> 6] * Hkv + hk) * 64 + (j & 63)) * DH;
  };
  auto vaddr = [&](int row, int j) -> const T* {  // 8 entries from j (j % 8 == 0)
    if (!PAGED) return VT + ((size_t)(j >> 3) * DH + row) * 8;
    return VTc + ((((size_t)pgs[(j - j0) >> 6] * Hkv + hk) * 8 + ((j & 63) >> 3)) * DH + row) * 8;
  };
  // the appended entry's place (its page comes from the table directly: LDS is not ready yet);
  // value dimension d at Vn[d * 8]
  size_t kn_off = (size_t)n * DH, vn_off = (size_t)(n >> 3) * DH * 8 + (n & 7);
  constexpr size_t vn_stride = 8;
  if (PAGED) {
    const size_t pn = (size_t)ptab[(size_t)b * pld + (n >> 6)] * Hkv + hk;
    kn_off = (pn * 64 + (n & 63)) * DH;
    vn_off = ((pn * 8 + ((n & 63) >> 3)) * DH) * 8 + (n & 7);
  }
  T* __restrict__ Kn = PAGED ? Kc + kn_off : K + kn_off;
  T* __restrict__ Vn = PAGED ? VTc + vn_off : VT + vn_off;

  const T* row = QKV + (size_t)b * (H + 2 * Hkv) * DH;
  for (int e = tid; e < GM * (DH / 2); e += 256) {
    // slots g >= gcnt repeat the last head; their results are never stored
    const int g = e / (DH / 2), c = e % (DH / 2), hq = h0 + min(g, gcnt - 1);
    const float2 cs = rope[(size_t)n * (DH / 2) + c];
    const float q1 = (float)row[hq * DH + c], q2 = (float)row[hq * DH + c + DH / 2];
    qs[g][c] = q1 * cs.x - q2 * cs.y;
    qs[g][c + DH / 2] = q2 * cs.x + q1 * cs.y;
  }
  if (tid < DH / 2) {
    const int c = tid;
    const float2 cs = rope[(size_t)n * (DH / 2) + c];
    const T* kr = row + (size_t)(H + hk) * DH;
    const float k1 = (float)kr[c], k2 = (float)kr[c + DH / 2];
    const T ka = round_t<T>(k1 * cs.x - k2 * cs.y), kb = round_t<T>(k2 * cs.x + k1 * cs.y);
    kn[c] = (float)ka;
    kn[c + DH / 2] = (float)kb;
    if (appends) {
      Kn[c] = ka;
      Kn[c + DH / 2] = kb;
    }
  } else if (tid >= 64 && tid < 64 + DH) {
    const int d = tid - 64;
    const T v = row[(size_t)(H + Hkv + hk) * DH + d];
    vn[d] = (float)v;
    if (appends) Vn[(size_t)d * vn_stride] = v;
  }
  __syncthreads();

  // ---- scores of the cached keys: each key is loaded once and scored against every head
  const int kl = lane / LPK, pp = lane % LPK;
  float qr[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[g][e] = qs[g][8 * pp + e];
  for (int jb = j0 + wave * KPW; jb < jc_end; jb += 4 * KPW * U) {
    float kv[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // clamped rather than guarded, so that the U loads are in flight together
      const int j = min(jb + u * 4 * KPW + kl, jc_end - 1);
      load8_nt(kaddr(j) + 8 * pp, kv[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d[GM];
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        d[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d[g] = fmaf(qr[g][e], kv[u][e], d[g]);
      }
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1)
#pragma unroll
        for (int g = 0; g < GM; ++g) d[g] += __shfl_xor(d[g], o, 64);
      const int j = jb + u * 4 * KPW + kl;
      if (pp == 0 && j < jc_end)
#pragma unroll
        for (int g = 0; g < GM; ++g) sc[g * chunk + j - j0] = d[g] * scale_log2;
    }
  }
  if (owns_new && wave < GM) {  // wave g scores the new key for head slot g
    float d = 0.f;
    for (int e = lane; e < DH; e += 64) d = fmaf(qs[wave][e], kn[e], d);
    d = wave_sum(d);
    if (lane == 0) sc[wave * chunk + n - j0] = d * scale_log2;
  }
  __syncthreads();

  // ---- softmax over [j0, j1), per head
  const int cnt = j1 - j0;
  float mx[GM], ls[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) mx[g] = -INFINITY;
  for (int j = tid; j < cnt; j += 256)
#pragma unroll
    for (int g = 0; g < GM; ++g) mx[g] = fmaxf(mx[g], sc[g * chunk + j]);
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    mx[g] = wave_max(mx[g]);
    if (lane == 0) red[g][wave] = mx[g];
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    mx[g] = fmaxf(fmaxf(red[g][0], red[g][1]), fmaxf(red[g][2], red[g][3]));
    ls[g] = 0.f;
  }
  for (int j = tid; j < cnt; j += 256)
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      const float p = __builtin_amdgcn_exp2f(sc[g * chunk + j] - mx[g]);
      sc[g * chunk + j] = p;
      ls[g] += p;
    }
#pragma unroll
  for (int g = 0; g < GM; ++g) ls[g] = wave_sum(ls[g]);
  __syncthreads();  // everyone has read red[] (max) before it is reused
  if (lane == 0)
#pragma unroll
    for (int g = 0; g < GM; ++g) red[g][4 + wave] = ls[g];
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GM; ++g) ls[g] = red[g][4] + red[g][5] + red[g][6] + red[g][7];

  // ---- values: lane (row lane rl, chunk lane cl) owns rows r*32 + wave*8 + rl, keys cl*8 + 64t
  const int cl = lane & 7, rl = lane >> 3;
  float acc[GM][RPL];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int r = 0; r < RPL; ++r) acc[g][r] = 0.f;
  for (int jb = j0 + cl * 8; jb < jc_end; jb += 64 * UV) {
    // UV chunks of 8 keys per row in flight; chunks past the cached keys are clamped to a valid
    // address and weighted by zero
    float v[UV][RPL][8];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int jc = jb + 64 * u < jc_end ? jb + 64 * u : jb;
#pragma unroll
      for (int r = 0; r < RPL; ++r) load8_nt(vaddr(r * 32 + wave * 8 + rl, jc), v[u][r]);
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int jc = jb + 64 * u;
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        // jc - j0 is a multiple of 8 and the row's 8 scores end within sc (chunk + 8 padding)
        const float4 s0 = *(const float4*)&sc[g * chunk + jc - j0];
        const float4 s1 = *(const float4*)&sc[g * chunk + jc - j0 + 4];
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = (jc + e < jc_end) ? sv[e] : 0.f;
#pragma unroll
          for (int r = 0; r < RPL; ++r) acc[g][r] = fmaf(p, v[u][r][e], acc[g][r]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) acc[g][r] += __shfl_xor(acc[g][r], o, 64);
  if (cl == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= gcnt) break;
      const int h = h0 + g;
      const float pn = owns_new ? sc[g * chunk + n - j0] : 0.f;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const int d = r * 32 + wave * 8 + rl;
        const float o = acc[g][r] + pn * vn[d];
        if (nsplit == 1) {
          ACT[opnd_idx(ACT, b, h * DH + d, ld_act)] = round_t<T>(o / ls[g]);
        } else {
          float* pp_ = part + (((size_t)b * H + h) * nsplit + s) * (DH + 2);
          pp_[2 + d] = o;
          if (d == 0) {
            pp_[0] = mx[g];
            pp_[1] = ls[g];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- block-attention decode, one wave per unit (fp16)
// Multi-head attention (one query head per KV head).  A unit is one (row b, head h, key split s);
// its cached keys [j0, jc_end) are taken in steps of KS = 8 NG keys (64 at d_h = 64, 32 at
// d_h = 128).  Lane (group kl, part pp) loads dims 8 pp .. 8 pp + 7 of keys kl*8 + u (u < 8) and
// value rows r * LPK + pp (r < 8) of the same 8 keys (one 16-byte load per row from their value
// group), so the probabilities a lane weighs its values with are the 8 scores its own lane group has
// just reduced:
// a step's keys and values are in flight together, and nothing passes through LDS.  Online softmax
// in registers across steps; the new entry (slot n: rotated here, appended by split 0 after its
// output is stored) joins at the end.  WPU = 4: the unit's steps are dealt round-robin to the 4 waves of a workgroup, merged
// through LDS (few units); WPU = 1: four units per workgroup, one per wave, no barrier.  Compared
// with the workgroup-per-unit kernel above, a short cache costs one round trip for the length and
// one for everything else, instead of five separated by barriers.
template <int DH, int WPU, bool PAGED>
__global__ __launch_bounds__(256) void k_attn_decode_wave(const f16* __restrict__ QKV, const int* __restrict__ n_ptr,
                                                          int B, int H, const float2* __restrict__ rope,
                                                          f16* __restrict__ Kc, f16* __restrict__ VTc, int cap,
                                                          f16* __restrict__ ACT, int ld_act, float* __restrict__ part,
                                                          int nsplit, int chunk, float scale_log2,
                                                          const int* __restrict__ ptab, int pld) {
  static_assert(DH == 64 || DH == 128, "head width");
  static_assert(WPU == 1 || WPU == 4, "waves per unit");
  constexpr int LPK = DH / 8, NG = 64 / LPK, KS = 8 * NG, HALF = DH / 2;
  __shared__ float mrg[4][DH + 2];  // per wave: (m, l, value rows)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = WPU == 1 ? blockIdx.x * 4 + wave : blockIdx.x;
  if (WPU == 1 && unit >= B * H * nsplit) return;  // idle waves of the last workgroup (no barrier in this mode)
  const int s = unit % nsplit, bh = unit / nsplit, h = bh % H, b = bh / H;
  const int w = WPU == 1 ? 0 : wave;  // this wave takes steps w, w + WPU, ...
  const int kl = lane / LPK, pp = lane % LPK;
  // entries already cached in this row; the new one goes to slot n (the host keeps every row below
  // the capacity; the clamp only keeps a misused row inside its own cache)
  const int n = min(n_ptr[b], cap - 1);
  const int j0 = s * chunk, j1 = min(n + 1, j0 + chunk), jc_end = min(j1, n);
  const bool owns_new = n >= j0 && n < j1;
  const int nsteps = jc_end > j0 ? (jc_end - j0 + KS - 1) / KS : 0;
  // 8-key group holding the last cached key: value loads of groups past the cached keys are
  // clamped into it (their weights are zero; every slot below the capacity is finite).  Loads of a
  // step past the unit's keys (the first step of a unit or wave without any) stay inside the
  // capacity, on page 0 for a paged cache, and their values are never used.
  const int jlast = min(max(j0, (jc_end - 1) & ~7), cap - 8);
  // paged: lane i holds the page of keys j0 + 64 i .. (chunk <= 4096 keys: at most 64 pages); a
  // step's keys lie in one page
  int pg = 0;
  if (PAGED && j0 / 64 + lane < pld && lane * 64 < chunk) pg = ptab[(size_t)b * pld + j0 / 64 + lane];
  const int pg_new = PAGED && s == 0 ? ptab[(size_t)b * pld + (n >> 6)] : 0;  // page of the appended entry

  // ---- query, new key and value of this head: lane pp holds dims 8 pp .. 8 pp + 7 and their
  // rotary partners (dims +- d_h / 2)
  const f16* row = QKV + (size_t)b * 3 * H * DH;
  const int dp = (8 * pp + HALF) % DH, c0 = (8 * pp) % HALF;
  const half8 q_own = *(const half8*)(row + h * DH + 8 * pp), q_par = *(const half8*)(row + h * DH + dp);
  const half8 k_own = *(const half8*)(row + (H + h) * DH + 8 * pp), k_par = *(const half8*)(row + (H + h) * DH + dp);
  const half8 v_new = *(const half8*)(row + (2 * H + h) * DH + 8 * pp);
  float4 cs4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cs4[i] = *(const float4*)(rope + (size_t)n * HALF + c0 + 2 * i);

  // ---- the first step's keys and values, issued before the query is rotated
  auto load_step = [&](int t, half8 (&kr)[8], half8 (&vr)[8]) {
    const int jb = j0 + t * KS;
    const int page = PAGED && t < nsteps ? __builtin_amdgcn_readlane(pg, (jb - j0) >> 6) : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = max(0, min(jb + kl * 8 + u, jc_end - 1));
      const f16* p = PAGED ? Kc + (((size_t)page * H + h) * 64 + (j & 63)) * DH : Kc + ((size_t)bh * cap + j) * DH;
      kr[u] = __builtin_nontemporal_load((const half8*)(p + 8 * pp));
    }
    // value rows r * LPK + pp of the group at jg: the LPK lanes of a lane group read one whole
    // 16 * LPK-byte run of the group per instruction
    const int jg = min(jb + kl * 8, jlast);
    const f16* vg = PAGED ? VTc + ((((size_t)page * H + h) * 8 + ((jg & 63) >> 3)) * DH) * 8
                          : VTc + (((size_t)bh * (cap >> 3) + (jg >> 3)) * DH) * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) vr[r] = __builtin_nontemporal_load((const half8*)(vg + (size_t)(r * LPK + pp) * 8));
  };
  half8 kr[8], vr[8];
  load_step(w, kr, vr);

  const bool lo = 8 * pp < HALF;
  float qr[8], kn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = e & 1 ? cs4[e >> 1].z : cs4[e >> 1].x, sn = e & 1 ? cs4[e >> 1].w : cs4[e >> 1].y;
    const float qa = (float)q_own[e], qb = (float)q_par[e], ka = (float)k_own[e], kb = (float)k_par[e];
    qr[e] = lo ? qa * c - qb * sn : qa * c + qb * sn;
    kn[e] = (float)to_f16(lo ? ka * c - kb * sn : ka * c + kb * sn);
  }
  float sn_new = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) sn_new = fmaf(qr[e], kn[e], sn_new);
  sn_new = sum_lanes<LPK>(sn_new) * scale_log2;

  // ---- cached keys, online softmax: m (running maximum, log2 units), l (this lane group's sum of
  // weights), acc[r] (value row 8 pp + r weighted by this lane group's keys)
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
  // (the next step's loads follow the exit test, so that they reuse the registers of this one)
  for (int t = w; t < nsteps;) {
    const int jb = j0 + t * KS;
    float sv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qr[e], (float)kr[u][e], d);
      d = sum_lanes<LPK>(d);
      sv[u] = jb + kl * 8 + u < jc_end ? d * scale_log2 : -INFINITY;
    }
    float cm = sv[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) cm = fmaxf(cm, sv[u]);
    cm = wave_max(cm);  // (the lanes of a lane group hold the same value)
    const float mn = fmaxf(m, cm);  // finite: every step holds a cached key
    const float al = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    l *= al;
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] *= al;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float p = __builtin_amdgcn_exp2f(sv[u] - mn);
      l += p;
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = fmaf(p, (float)vr[r][u], acc[r]);
    }
    // the weighting is finished here, before the next loads (left to itself the compiler sinks it
    // below them, which needs a second set of value registers)
#pragma unroll
    for (int r = 0; r < 8; ++r) asm volatile("" : "+v"(acc[r]));
    asm volatile("" : "+v"(l));
    t += WPU;
    if (t >= nsteps) break;
    load_step(t, kr, vr);
  }
  // sum over the lane groups (the lanes of one group hold the same l)
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] += __shfl_xor(acc[r], o, 64);
  }
  // lane pp of group 0 holds value rows r * LPK + pp; through LDS it takes rows 8 pp .. 8 pp + 7
  if (kl == 0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) mrg[wave][2 + r * LPK + pp] = acc[r];
    if (pp == 0) mrg[wave][0] = m, mrg[wave][1] = l;
  }
  if constexpr (WPU == 1) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = mrg[wave][2 + 8 * pp + r];  // same wave: LDS keeps its order
  } else {
    __syncthreads();
    if (wave != 0) return;
    float M = mrg[0][0];
#pragma unroll
    for (int i = 1; i < WPU; ++i) M = fmaxf(M, mrg[i][0]);
    l = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < WPU; ++i) {
      const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrg[i][0] - M);
      l = fmaf(f, mrg[i][1], l);
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = fmaf(f, mrg[i][2 + 8 * pp + r], acc[r]);
    }
    m = M;
  }
  if (owns_new) {
    const float mn = fmaxf(m, sn_new);
    const float al = __builtin_amdgcn_exp2f(m - mn), pn = __builtin_amdgcn_exp2f(sn_new - mn);
    l = fmaf(l, al, pn);
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = fmaf(acc[r], al, pn * (float)v_new[r]);
    m = mn;
  }
  if (kl != 0) return;
  if (nsplit == 1) {
    half8 o;
#pragma unroll
    for (int r = 0; r < 8; ++r) o[r] = to_f16_bounded(acc[r] / l);
    *(half8*)(ACT + frag_off(b, h * DH + 8 * pp, ld_act)) = o;
  } else {
    float* q = part + ((size_t)bh * nsplit + s) * (DH + 2);
#pragma unroll
    for (int r = 0; r < 8; r += 2) *(float2*)(q + 2 + 8 * pp + r) = make_float2(acc[r], acc[r + 1]);
    if (pp == 0) *(float2*)q = make_float2(m, l);
  }
  // split 0 appends the new entry (wave 0 of the unit, lane group 0).  Last: stores count in the
  // same in-order counter as loads, so an earlier append would hold up every later wait for data
  // until its scattered value-column writes are acknowledged.
  if (s == 0 && w == 0) {
    // value dimension d of the entry at voff + d * 8 (within its group of 8 entries)
    size_t koff = ((size_t)bh * cap + n) * DH, voff = ((size_t)bh * (cap >> 3) + (n >> 3)) * DH * 8 + (n & 7);
    if (PAGED) {
      const size_t pn = (size_t)pg_new * H + h;
      koff = (pn * 64 + (n & 63)) * DH;
      voff = ((pn * 8 + ((n & 63) >> 3)) * DH) * 8 + (n & 7);
    }
    half8 kh;
#pragma unroll
    for (int e = 0; e < 8; ++e) kh[e] = to_f16(kn[e]);
    *(half8*)(Kc + koff + 8 * pp) = kh;
#pragma unroll
    for (int r = 0; r < 8; ++r) VTc[voff + (size_t)(8 * pp + r) * 8] = v_new[r];
  }
}

// ---------------------------------------------------------------- block-attention decode, MFMA (fp16)
// A unit is one (row b, KV head hk, key split s) with all G = H / Hkv query heads of that KV head
// (G <= 16: grouped-query heads share the unit, so their keys and values stream once).  WPU waves
// serve a unit: with WPU = 4 they take its TK-key steps round-robin and merge through LDS at the
// end (few units); with WPU = 1 a wave serves a unit alone, four units per workgroup, no barrier.
// Per step a wave stages the step's keys and values in its own LDS region (whole 128-byte rows,
// 1 KB per load instruction, non-temporal), then computes S^T = K Q^T with
// v_mfma_f32_16x16x32_f16 (A = keys, B = Q^T with one column per query head), an online softmax
// per column in registers, and O^T += V^T P^T.  The keys are assigned to the rows of the S^T tiles
// so that lane group g ends up holding the probabilities of 8 consecutive keys of each 32-key
// slice -- exactly its B operand of the P V product -- and its V^T operand is one 16-byte read of
// the same 8 keys; the probabilities never leave registers.  Keys past the cached range get score -inf and value 0; the new entry (slot n, appended by
// split 0) joins the softmax at the end, from registers.  MFMA layouts as in k_flash_prefill2.
template <int DH, int WPU, bool PAGED>
__global__ __launch_bounds__(256) void k_attn_decode_mfma(const f16* __restrict__ QKV, const int* __restrict__ n_ptr,
                                                          int B, int H, int Hkv, const float2* __restrict__ rope,
                                                          f16* __restrict__ Kc, f16* __restrict__ VTc, int cap,
                                                          f16* __restrict__ ACT, int ld_act, float* __restrict__ part,
                                                          int nsplit, int chunk, float scale_log2,
                                                          const int* __restrict__ ptab, int pld) {
  constexpr int KS = DH / 32, MT = DH / 16;
  constexpr int KT = DH == 64 ? 4 : 2;  // 16-key S^T tiles per step
  constexpr int SL = KT / 2;            // 32-key slices per step
  constexpr int TK = 16 * KT;           // keys per step (a step never straddles a 64-entry page)
  __shared__ float so[WPU == 1 ? 1 : WPU][16][WPU == 1 ? 1 : DH + 1];
  __shared__ float sm[WPU][16], sl_[WPU][16];
  // per-wave staging of a step's keys [TK][DH] and values [DH][TK] (padded rows: conflict-free
  // fragment reads), so that the global loads are whole 128-byte rows, 1 KB per instruction
  constexpr int KLD = DH + 8, VLD = TK + 8;
  __shared__ __attribute__((aligned(16))) f16 stage[4][TK * KLD + DH * VLD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f16* const Ks = stage[wave];
  f16* const Vs = stage[wave] + TK * KLD;
  const int c = lane & 15, g = lane >> 4;  // query column (head of the group), lane group
  const int G = H / Hkv;
  const int unit = WPU == 1 ? blockIdx.x * 4 + wave : blockIdx.x;
  if (unit >= B * Hkv * nsplit) return;  // whole wave (WPU = 1) or whole workgroup (WPU = 4)
  const int s = unit % nsplit, bk = unit / nsplit, hk = bk % Hkv, b = bk / Hkv;
  const int n = min(n_ptr[b], cap - 1);
  const int j0 = s * chunk, j1 = min(n + 1, j0 + chunk), jc_end = min(j1, n);
  const bool owns_new = n >= j0 && n < j1;
  const bool colv = c < G;
  const int hq = hk * G + min(c, G - 1);  // columns past the group repeat its last head (never stored)
  const f16* row = QKV + (size_t)b * (H + 2 * Hkv) * DH;

  // q^T operand with the rotary embedding at position n; the new key (rotated, rounded as cached)
  // for the new entry's score; the lane's new values; the append by split 0
  half8 qf[KS];
  float sc_new, vn[MT][4];
  {
    float q[KS][8], k[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      load8(row + hq * DH + 32 * ks + 8 * g, q[ks]);
      load8(row + (size_t)(H + hk) * DH + 32 * ks + 8 * g, k[ks]);
    }
    const float2* rp = rope + (size_t)n * (DH / 2);
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = rp[32 * ks + 8 * g + e];
        const float q1 = q[ks][e], q2 = q[ks + KS / 2][e], k1 = k[ks][e], k2 = k[ks + KS / 2][e];
        q[ks][e] = q1 * cs.x - q2 * cs.y;
        q[ks + KS / 2][e] = q2 * cs.x + q1 * cs.y;
        k[ks][e] = (float)to_f16(k1 * cs.x - k2 * cs.y);
        k[ks + KS / 2][e] = (float)to_f16(k2 * cs.x + k1 * cs.y);
      }
    float dot = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[ks][e] = colv ? to_f16(q[ks][e]) : (f16)0.f;
        dot = fmaf(q[ks][e], k[ks][e], dot);
      }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    sc_new = dot * scale_log2;
    const f16* vr = row + (size_t)(H + Hkv + hk) * DH;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const half4 v4 = *(const half4*)(vr + 16 * mt + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) vn[mt][i] = (float)v4[i];
    }
    if (s == 0 && c == 0 && (WPU == 1 || wave == 0)) {
      // lanes 0, 16, 32, 48 hold dims 8g.. of every 32-dim slice of k and rows 4g.. of each v tile
      // value dimension d of the entry at vofs + d * 8 (its group of 8 entries, transposed)
      size_t kofs, vofs;
      constexpr size_t vstr = 8;
      if (PAGED) {
        const size_t pg = (size_t)ptab[(size_t)b * pld + (n >> 6)] * Hkv + hk;
        kofs = (pg * 64 + (n & 63)) * DH, vofs = ((pg * 8 + ((n & 63) >> 3)) * DH) * 8 + (n & 7);
      } else {
        kofs = (((size_t)b * Hkv + hk) * cap + n) * DH;
        vofs = (((size_t)b * Hkv + hk) * (cap >> 3) + (n >> 3)) * DH * 8 + (n & 7);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        half8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = to_f16(k[ks][e]);
        *(half8*)(Kc + kofs + 32 * ks + 8 * g) = w;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) VTc[vofs + (size_t)(16 * mt + 4 * g + i) * vstr] = to_f16_bounded(vn[mt][i]);
    }
  }

  float4_ o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = float4_{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const int w0 = WPU == 1 ? 0 : wave;
  for (int t = j0 + w0 * TK; t < jc_end; t += WPU * TK) {
    // vb: the step's first value group ([TK / 8][DH][8], contiguous; t % 8 == 0)
    const f16 *kb, *vb;
    if (PAGED) {
      const size_t pg = (size_t)ptab[(size_t)b * pld + (t >> 6)] * Hkv + hk;
      kb = Kc + (pg * 64 + (t & 63)) * DH, vb = VTc + ((pg * 8 + ((t & 63) >> 3)) * DH) * 8;
    } else {
      kb = Kc + (((size_t)b * Hkv + hk) * cap + t) * DH;
      vb = VTc + (((size_t)b * Hkv + hk) * (cap >> 3) + (t >> 3)) * DH * 8;
    }
    const int lim = jc_end - t;  // keys of this step that are cached: [0, lim)
    // stage the step: key rows (clamped to cached keys, masked below) and value rows, 8 lanes per
    // 128-byte row segment
    {
      constexpr int LPR = DH / 8, RK = 64 / LPR;  // lanes per key row, key rows per instruction
      half8 rk[TK / RK], rv[DH * TK / 8 / 64];
#pragma unroll
      for (int i = 0; i < TK / RK; ++i) {
        const int kr = min(i * RK + lane / LPR, lim - 1);
        rk[i] = __builtin_nontemporal_load((const half8*)(kb + (size_t)kr * DH + 8 * (lane % LPR)));
      }
      // value item (row, group q): 16 bytes at vb + (q * DH + row) * 8; an instruction takes RV
      // consecutive rows of LPV groups
      constexpr int LPV = TK / 8, RV = 64 / LPV;  // groups per step, rows per instruction
#pragma unroll
      for (int i = 0; i < DH / RV; ++i)
        rv[i] = __builtin_nontemporal_load((const half8*)(vb + ((size_t)(lane / RV) * DH + i * RV + lane % RV) * 8));
#pragma unroll
      for (int i = 0; i < TK / RK; ++i) *(half8*)&Ks[(i * RK + lane / LPR) * KLD + 8 * (lane % LPR)] = rk[i];
#pragma unroll
      for (int i = 0; i < DH / RV; ++i) *(half8*)&Vs[(i * RV + lane % RV) * VLD + 8 * (lane / RV)] = rv[i];
    }
    __builtin_amdgcn_wave_barrier();
    // K rows: tile nt, row c holds key 32 (nt / 2) + 8 (c / 4) + 4 (nt % 2) + c % 4
    half8 kf[KT][KS], vf[SL][MT];
#pragma unroll
    for (int nt = 0; nt < KT; ++nt) {
      const int kk = 32 * (nt / 2) + 8 * (c / 4) + 4 * (nt % 2) + (c % 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[nt][ks] = *(const half8*)&Ks[kk * KLD + 32 * ks + 8 * g];
    }
    // V^T rows 16 mt + c at the 8 keys 32 sl + 8 g ..
#pragma unroll
    for (int sl = 0; sl < SL; ++sl)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) vf[sl][mt] = *(const half8*)&Vs[(16 * mt + c) * VLD + 32 * sl + 8 * g];
    float4_ sv[KT];
#pragma unroll
    for (int nt = 0; nt < KT; ++nt) {
      sv[nt] = float4_{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[nt][ks], qf[ks], sv[nt], 0, 0, 0);
    }
    // lane (c, g) holds the scores of keys 32 (nt / 2) + 8 g + 4 (nt % 2) + i for column c
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < KT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 32 * (nt / 2) + 8 * g + 4 * (nt % 2) + i;
        const float x = kk < lim ? sv[nt][i] * scale_log2 : -INFINITY;
        sv[nt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);  // finite: every step has a cached key
    const float corr = __builtin_amdgcn_exp2f(m - mnew);
    float ls = 0.f;
#pragma unroll
    for (int nt = 0; nt < KT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sv[nt][i] - mnew);
        sv[nt][i] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l = l * corr + ls;
    m = mnew;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] *= corr;
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) {
      half8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = to_f16_bounded(sv[2 * sl][e]);
        pf[4 + e] = to_f16_bounded(sv[2 * sl + 1][e]);
      }
      const bool tail = 32 * sl + 8 * g + 8 > lim;  // values past the cached keys must be 0, not junk
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        half8 v = vf[sl][mt];
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 32 * sl + 8 * g + e < lim ? v[e] : (f16)0.f;
        }
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, pf, o[mt], 0, 0, 0);
      }
    }
  }
  if (owns_new && (WPU == 1 || wave == 0)) {
    const float mnew = fmaxf(m, sc_new);
    const float corr = __builtin_amdgcn_exp2f(m - mnew), pn = __builtin_amdgcn_exp2f(sc_new - mnew);
    l = l * corr + pn;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[mt][i] = o[mt][i] * corr + pn * vn[mt][i];
    m = mnew;
  }
  if (WPU > 1) {
    // merge the waves' partial softmaxes of each column (fixed order)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[wave][c][16 * mt + 4 * g + i] = o[mt][i];
    if (g == 0) sm[wave][c] = m, sl_[wave][c] = l;
    __syncthreads();
    for (int it = threadIdx.x; it < G * DH; it += 256) {
      const int cc = it / DH, d = it % DH, h = hk * G + cc;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WPU; ++w) M = fmaxf(M, sm[w][cc]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY)
#pragma unroll
        for (int w = 0; w < WPU; ++w) {
          const float f = __builtin_amdgcn_exp2f(sm[w][cc] - M);
          L += f * sl_[w][cc];
          O += f * so[w][cc][d];
        }
      if (nsplit == 1) {
        ACT[frag_off(b, h * DH + d, ld_act)] = to_f16_bounded(O / L);
      } else {
        float* pp = part + (((size_t)b * H + h) * nsplit + s) * (DH + 2);
        pp[2 + d] = O;
        if (d == 0) pp[0] = M, pp[1] = L;
      }
    }
    return;
  }
  if (!colv) return;
  if (nsplit == 1) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      store4_bounded(ACT, frag_off(b, hq * DH + 16 * mt + 4 * g, ld_act), o[mt][0] * inv, o[mt][1] * inv, o[mt][2] * inv,
             o[mt][3] * inv);
  } else {
    float* pp = part + (((size_t)b * H + hq) * nsplit + s) * (DH + 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pp[2 + 16 * mt + 4 * g + i] = o[mt][i];
    if (g == 0) pp[0] = m, pp[1] = l;
  }
}

// merge split partials: o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)
template <typename T, int DH>
__global__ void k_attn_combine(const float* __restrict__ part, int H, int nsplit, T* __restrict__ ACT, int ld_act) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const size_t bh = (size_t)b * H + h;
  const float* p = part + bh * nsplit * (DH + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p[s * (DH + 2)]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = __builtin_amdgcn_exp2f(p[s * (DH + 2)] - M);
    l += w * p[s * (DH + 2) + 1];
    o += w * p[s * (DH + 2) + 2 + d];
  }
  ACT[opnd_idx(ACT, b, h * DH + d, ld_act)] = round_t<T>(o / l);
}

// query heads per decode workgroup: all of a group up to 4 (runs of <= 4 for larger groups)
static int decode_group_max(int H, int Hkv) { return H == Hkv ? 1 : (H / Hkv == 2 ? 2 : 4); }

template <typename T, int DH, int GM>
static hipError_t launch_decode_t(const void* QKV, int B, const int* n_ptr, int H, int Hkv, const float2* rope,
                                  void* Kc, void* Vc, int cap, void* ACT, int ld_act, float* part, size_t part_bytes,
                                  int nsplit, hipStream_t st, const int* ptab, int pld) {
  // the split layout covers the whole capacity, so it does not depend on the current length n
  // (which is read on the device); splits past n + 1 produce empty partials
  int chunk = (cap + nsplit - 1) / nsplit;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk * GM > kMaxChunk) return hipErrorInvalidValue;
  if (nsplit > 1 && (size_t)B * H * nsplit * (DH + 2) * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  const int G = H / Hkv, nsub = (G + GM - 1) / GM, gsz = (G + nsub - 1) / nsub;
  const float sl2 = kLog2e / sqrtf((float)DH);
  if (ptab)
    hipLaunchKernelGGL((k_attn_decode<T, DH, GM, true>), dim3(nsplit, Hkv * nsub, B), dim3(256), 0, st, (const T*)QKV,
                       n_ptr, H, Hkv, gsz, rope, (T*)Kc, (T*)Vc, cap, (T*)ACT, ld_act, part, nsplit, chunk, sl2, ptab,
                       pld);
  else
    hipLaunchKernelGGL((k_attn_decode<T, DH, GM, false>), dim3(nsplit, Hkv * nsub, B), dim3(256), 0, st, (const T*)QKV,
                       n_ptr, H, Hkv, gsz, rope, (T*)Kc, (T*)Vc, cap, (T*)ACT, ld_act, part, nsplit, chunk, sl2, ptab,
                       pld);
  if (nsplit > 1)
    hipLaunchKernelGGL((k_attn_combine<T, DH>), dim3(H, B), dim3(DH), 0, st, (const float*)part, H, nsplit, (T*)ACT,
                       ld_act);
  return hipGetLastError();
}

int decode_splits(int B, int H, int Hkv, int cap) {
  const int gm = decode_group_max(H, Hkv);
  const int wgs = B * Hkv * ((H / Hkv + gm - 1) / gm);              // workgroups per split
  int s = (cap + kMaxChunk / gm - 1) / (kMaxChunk / gm);            // LDS holds at most kMaxChunk scores
  if (wgs < 512) s = std::max(s, std::min((1024 + wgs - 1) / wgs, (cap + 255) / 256));
  return std::max(1, std::min(s, kMaxSplit));
}

// fp16, groups of <= 16 query heads: the MFMA kernel, 4 waves per unit while units are few
template <int DH>
static hipError_t launch_decode_mfma(const void* QKV, int B, const int* n_ptr, int H, int Hkv, const float2* rope,
                                     void* Kc, void* Vc, int cap, void* ACT, int ld_act, float* part, size_t part_bytes,
                                     int nsplit, hipStream_t st, const int* ptab, int pld) {
  int chunk = (cap + nsplit - 1) / nsplit;
  chunk = (chunk + 63) / 64 * 64;
  if (nsplit > 1 && (size_t)B * H * nsplit * (DH + 2) * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  const float sl2 = kLog2e / sqrtf((float)DH);
  const long units = (long)B * Hkv * nsplit;
#define BT_DM(WPUV, GRID)                                                                                        \
  {                                                                                                              \
    if (ptab)                                                                                                    \
      hipLaunchKernelGGL((k_attn_decode_mfma<DH, WPUV, true>), dim3(GRID), dim3(256), 0, st, (const f16*)QKV,    \
                         n_ptr, B, H, Hkv, rope, (f16*)Kc, (f16*)Vc, cap, (f16*)ACT, ld_act, part, nsplit, chunk, \
                         sl2, ptab, pld);                                                                        \
    else                                                                                                         \
      hipLaunchKernelGGL((k_attn_decode_mfma<DH, WPUV, false>), dim3(GRID), dim3(256), 0, st, (const f16*)QKV,   \
                         n_ptr, B, H, Hkv, rope, (f16*)Kc, (f16*)Vc, cap, (f16*)ACT, ld_act, part, nsplit, chunk, \
                         sl2, ptab, pld);                                                                        \
  }
  if (units < 1024) BT_DM(4, units) else BT_DM(1, (units + 3) / 4)
#undef BT_DM
  if (nsplit > 1)
    hipLaunchKernelGGL((k_attn_combine<f16, DH>), dim3(H, B), dim3(DH), 0, st, (const float*)part, H, nsplit,
                       (f16*)ACT, ld_act);
  return hipGetLastError();
}

// fp16 multi-head attention: one wave per (row, head, split); four waves share a unit while units
// are few
template <int DH>
static hipError_t launch_decode_wave(const void* QKV, int B, const int* n_ptr, int H, const float2* rope, void* Kc,
                                     void* Vc, int cap, void* ACT, int ld_act, float* part, size_t part_bytes,
                                     int nsplit, hipStream_t st, const int* ptab, int pld) {
  int chunk = (cap + nsplit - 1) / nsplit;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk > 4096) return hipErrorInvalidValue;  // a paged split's pages are held one per lane
  if (nsplit > 1 && (size_t)B * H * nsplit * (DH + 2) * sizeof(float) > part_bytes) return hipErrorInvalidValue;
  const float sl2 = kLog2e / sqrtf((float)DH);
  const long units = (long)B * H * nsplit;
#define BT_DW(WPUV, GRID)                                                                                        \
  {                                                                                                              \
    if (ptab)                                                                                                    \
      hipLaunchKernelGGL((k_attn_decode_wave<DH, WPUV, true>), dim3(GRID), dim3(256), 0, st, (const f16*)QKV,    \
                         n_ptr, B, H, rope, (f16*)Kc, (f16*)Vc, cap, (f16*)ACT, ld_act, part, nsplit, chunk, sl2, \
                         ptab, pld);                                                                             \
    else                                                                                                         \
      hipLaunchKernelGGL((k_attn_decode_wave<DH, WPUV, false>), dim3(GRID), dim3(256), 0, st, (const f16*)QKV,   \
                         n_ptr, B, H, rope, (f16*)Kc, (f16*)Vc, cap, (f16*)ACT, ld_act, part, nsplit, chunk, sl2, \
                         ptab, pld);                                                                             \
  }
  if (units < 2048) BT_DW(4, units) else BT_DW(1, (units + 3) / 4)
#undef BT_DW
  if (nsplit > 1)
    hipLaunchKernelGGL((k_attn_combine<f16, DH>), dim3(H, B), dim3(DH), 0, st, (const float*)part, H, nsplit,
                       (f16*)ACT, ld_act);
  return hipGetLastError();
}

hipError_t launch_block_attn_decode(bool f32, const void* QKV, int B, const int* n_ptr, int H, int Hkv, int dh,
                                    const float2* rope, void* Kc, void* Vc, int cap, void* ACT, int ld_act, float* part,
                                    size_t part_bytes, int nsplit, hipStream_t st, const int* ptab, int pld) {
  if (B <= 0) return hipSuccess;
  if (Hkv < 1 || H % Hkv) return hipErrorInvalidValue;
  // the kernels read whole 8-key value chunks and clamp loads into [0, cap)
  if (cap < 64 || cap % 64) return hipErrorInvalidValue;
  // fp16 multi-head attention: one wave per (row, head, split), VALU dot products (with one query
  // head per KV head an MFMA column would be 1/16 used; the MFMA kernel measured 95 us at the
  // decode-heavy shape and 543 entries against 90 us for the workgroup kernel, which this one
  // replaces: 75 us there, and 17 us instead of 22 us at 32-64 entries)
  if (!f32 && H == Hkv && (dh == 64 || dh == 128)) {
    if (dh == 64)
      return launch_decode_wave<64>(QKV, B, n_ptr, H, rope, Kc, Vc, cap, ACT, ld_act, part, part_bytes, nsplit, st,
                                    ptab, pld);
    return launch_decode_wave<128>(QKV, B, n_ptr, H, rope, Kc, Vc, cap, ACT, ld_act, part, part_bytes, nsplit, st,
                                   ptab, pld);
  }
  // grouped-query heads (2..16 per KV head): one MFMA wave reads a KV head's keys and values once
  // for all of them
  if (!f32 && H / Hkv > 1 && H / Hkv <= 16) {
    if (dh == 64)
      return launch_decode_mfma<64>(QKV, B, n_ptr, H, Hkv, rope, Kc, Vc, cap, ACT, ld_act, part, part_bytes, nsplit,
                                    st, ptab, pld);
    if (dh == 128)
      return launch_decode_mfma<128>(QKV, B, n_ptr, H, Hkv, rope, Kc, Vc, cap, ACT, ld_act, part, part_bytes, nsplit,
                                     st, ptab, pld);
  }
  const int gm = decode_group_max(H, Hkv);
#define BT_DEC(T, DHV, GMV)                                                                                        \
  if (dh == DHV && gm == GMV)                                                                                      \
    return launch_decode_t<T, DHV, GMV>(QKV, B, n_ptr, H, Hkv, rope, Kc, Vc, cap, ACT, ld_act, part, part_bytes,   \
                                        nsplit, st, ptab, pld);
#define BT_DEC_G(T, DHV) BT_DEC(T, DHV, 1) BT_DEC(T, DHV, 2) BT_DEC(T, DHV, 4)
  if (f32) {
    BT_DEC_G(float, 32) BT_DEC_G(float, 64) BT_DEC_G(float, 128)
  } else {
    BT_DEC_G(f16, 64) BT_DEC_G(f16, 128)
  }
#undef BT_DEC_G
#undef BT_DEC
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- local attention (token decoder)
// grid (H, B), one wave.  New slots [s0, s0 + m) of row b come from QKV rows b*m + i; the first
// query head of each KV group writes them to the cache (the others read only slots < s0).
constexpr int kMaxLocal = 32;

template <typename T, int DH>
__global__ __launch_bounds__(64) void k_local_attn(const T* __restrict__ QKV, int ldq, int m, int s0, int H, int Hkv,
                                                   const float2* __restrict__ rope, T* __restrict__ Kc,
                                                   T* __restrict__ Vc, int cap, T* __restrict__ ACT, int ld_act,
                                                   float scale, const int* __restrict__ rmap) {
  __shared__ float ks[kMaxLocal][DH + 1], vs[kMaxLocal][DH + 1], qs[kMaxLocal][DH + 1];
  __shared__ float ps[64];
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int G = H / Hkv, hk = h / G;
  const bool writes = h % G == 0;
  const size_t qw = (size_t)ldq, koff = (size_t)(H + hk) * DH, voff = (size_t)(H + Hkv + hk) * DH;
  const size_t bh = (size_t)(rmap ? rmap[b] : b) * Hkv + hk;
  T* __restrict__ K = Kc + bh * cap * DH;
  T* __restrict__ V = Vc + bh * cap * DH;
  constexpr int HALF = DH / 2;
  for (int e = lane; e < s0 * DH; e += 64) {
    ks[e / DH][e % DH] = (float)K[e];
    vs[e / DH][e % DH] = (float)V[e];
  }
  for (int e = lane; e < m * HALF; e += 64) {
    const int i = e / HALF, c = e % HALF, slot = s0 + i;
    const T* r = QKV + ((size_t)b * m + i) * qw;
    const float2 cs = rope[(size_t)slot * HALF + c];
    const float q1 = (float)r[h * DH + c], q2 = (float)r[h * DH + c + HALF];
    qs[i][c] = q1 * cs.x - q2 * cs.y;
    qs[i][c + HALF] = q2 * cs.x + q1 * cs.y;
    const float k1 = (float)r[koff + c], k2 = (float)r[koff + c + HALF];
    const T ka = round_t<T>(k1 * cs.x - k2 * cs.y), kb = round_t<T>(k2 * cs.x + k1 * cs.y);
    ks[slot][c] = (float)ka;
    ks[slot][c + HALF] = (float)kb;
    if (writes) {
      K[(size_t)slot * DH + c] = ka;
      K[(size_t)slot * DH + c + HALF] = kb;
    }
  }
  for (int e = lane; e < m * DH; e += 64) {
    const int i = e / DH, d = e % DH, slot = s0 + i;
    const T v = QKV[((size_t)b * m + i) * qw + voff + d];
    vs[slot][d] = (float)v;
    if (writes) V[(size_t)slot * DH + d] = v;
  }
  __syncthreads();
  for (int i = 0; i < m; ++i) {
    const int nkeys = s0 + i + 1;
    float sj = -INFINITY;
    if (lane < nkeys) {
      float d = 0.f;
#pragma unroll 8
      for (int e = 0; e < DH; ++e) d = fmaf(qs[i][e], ks[lane][e], d);
      sj = d * scale;
    }
    const float mx = wave_max(sj);
    const float p = lane < nkeys ? expf(sj - mx) : 0.f;
    const float l = wave_sum(p);
    ps[lane] = p;
    __syncthreads();
    for (int d = lane; d < DH; d += 64) {
      float o = 0.f;
      for (int j = 0; j < nkeys; ++j) o = fmaf(ps[j], vs[j][d], o);
      ACT[opnd_idx(ACT, b * m + i, h * DH + d, ld_act)] = round_t<T>(o / l);
    }
    __syncthreads();
  }
}

// 8 consecutive elements from floats
__device__ __forceinline__ void store8(f16* p, const float* v) {
  half8 w;
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = to_f16(v[e]);
  *(half8*)p = w;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Token-decoder attention for ONE new slot s0 per row (a decode step).  One wave per (row, head);
// LPK = DH / 8 lanes per key hold 8 dimensions each, so a wave scores 64 / LPK keys per pass.  The
// new key (rotary applied, rounded to the cache type) and value are written to local slot s0 and
// used from registers (the first query head of each KV group writes them); the s0 cached entries
// are read with 16-byte loads.  Each key group keeps an
// online softmax (base 2) over its keys; the groups are merged with shuffles in a fixed order.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_local_attn_step(const T* __restrict__ QKV, int ldq, int B, int s0, int H,
                                                         int Hkv,
                                                         const float2* __restrict__ rope, T* __restrict__ Kc,
                                                         T* __restrict__ Vc, int cap, T* __restrict__ ACT, int ld_act,
                                                         float scale_log2, const int* __restrict__ rmap) {
  constexpr int LPK = DH / 8, KPP = 64 / LPK, HALF = DH / 2;
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= B * H) return;  // whole wave
  const int b = pair / H, h = pair % H;
  const int g = lane % LPK, kg = lane / LPK;  // dimensions [8g, 8g + 8), key group
  const int G = H / Hkv, hk = h / G;
  const size_t bh = (size_t)(rmap ? rmap[b] : b) * Hkv + hk;
  T* __restrict__ K = Kc + bh * cap * DH;
  T* __restrict__ V = Vc + bh * cap * DH;
  const T* row = QKV + (size_t)b * ldq + 8 * g;
  float q[8], kn[8], vn[8], kc[8], vc[8];
  load8(row + h * DH, q);
  load8(row + (H + hk) * DH, kn);
  load8(row + (H + Hkv + hk) * DH, vn);
  const int nkeys = s0 + 1;
  // first pass's cached entry of this key group (clamped; masked below)
  const int jc0 = min(kg, max(s0 - 1, 0));
  load8(K + (size_t)jc0 * DH + 8 * g, kc);
  load8(V + (size_t)jc0 * DH + 8 * g, vc);
  // rotary embedding at position s0: dimension d pairs with d +- DH/2, held by lane ^ (LPK / 2)
  const bool first = 8 * g < HALF;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float qp = __shfl_xor(q[e], LPK / 2, 64), kp = __shfl_xor(kn[e], LPK / 2, 64);
    const float2 cs = rope[(size_t)s0 * HALF + (8 * g + e) % HALF];
    if (first) {
      q[e] = q[e] * cs.x - qp * cs.y;
      kn[e] = (float)round_t<T>(kn[e] * cs.x - kp * cs.y);
    } else {
      q[e] = q[e] * cs.x + qp * cs.y;
      kn[e] = (float)round_t<T>(kn[e] * cs.x + kp * cs.y);
    }
  }
  if (kg == 0 && h % G == 0) {
    store8(K + (size_t)s0 * DH + 8 * g, kn);
    store8(V + (size_t)s0 * DH + 8 * g, vn);
  }
  float mrun = -INFINITY, lrun = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int j0 = 0; j0 < nkeys; j0 += KPP) {
    const int j = j0 + kg;
    if (j0 > 0) {  // later passes (long local windows)
      const int jc = min(j, max(s0 - 1, 0));
      load8(K + (size_t)jc * DH + 8 * g, kc);
      load8(V + (size_t)jc * DH + 8 * g, vc);
    }
    const bool isnew = j == s0;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(q[e], isnew ? kn[e] : kc[e], dot);
    dot = sum_lanes<LPK>(dot);
    const float sc = j < nkeys ? dot * scale_log2 : -INFINITY;
    const float mn = fmaxf(mrun, sc);
    const float corr = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float p = sc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc - mn);
    lrun = lrun * corr + p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * corr + p * (isnew ? vn[e] : (j < nkeys ? vc[e] : 0.f));
    mrun = mn;
  }
  // merge the key groups
#pragma unroll
  for (int w = LPK; w < 64; w <<= 1) {
    const float mo = __shfl_xor(mrun, w, 64), lo = __shfl_xor(lrun, w, 64);
    const float mn = fmaxf(mrun, mo);
    const float c1 = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float c2 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
    lrun = lrun * c1 + lo * c2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * c1 + __shfl_xor(o[e], w, 64) * c2;
    mrun = mn;
  }
  if (kg == 0) {
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    store8(ACT + opnd_idx(ACT, b, h * DH + 8 * g, ld_act), o);
  }
}

hipError_t launch_local_attention(bool f32, const void* QKV, int ldq, int B, int m, int s0, int H, int Hkv, int dh,
                                  const float2* rope, void* Kc, void* Vc, int cap, void* ACT, int ld_act,
                                  hipStream_t st, const int* rmap) {
  if (B <= 0 || m <= 0) return hipSuccess;
  if (Hkv < 1 || H % Hkv || ldq < (H + 2 * Hkv) * dh || ldq % 8) return hipErrorInvalidValue;
  if (s0 + m > kMaxLocal || s0 + m > cap) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)dh);
  if (m == 1) {
    // decode step: register-resident kernel, 4 (row, head) pairs per workgroup
    const dim3 g1((B * H + 3) / 4);
#define BT_STEP(T, DHV)                                                                                         \
  if (dh == DHV) {                                                                                              \
    hipLaunchKernelGGL((k_local_attn_step<T, DHV>), g1, dim3(256), 0, st, (const T*)QKV, ldq, B, s0, H, Hkv,     \
                       rope,                                                                                    \
                       (T*)Kc, (T*)Vc, cap, (T*)ACT, ld_act, scale * kLog2e, rmap);                              \
    return hipGetLastError();                                                                                   \
  }
    if (f32) {
      BT_STEP(float, 32) BT_STEP(float, 64) BT_STEP(float, 128)
    } else {
      BT_STEP(f16, 64) BT_STEP(f16, 128)
    }
#undef BT_STEP
    return hipErrorInvalidValue;
  }
  dim3 grid(H, B);
#define BT_LOC(T, DHV)                                                                                          \
  if (dh == DHV) {                                                                                              \
    hipLaunchKernelGGL((k_local_attn<T, DHV>), grid, dim3(64), 0, st, (const T*)QKV, ldq, m, s0, H, Hkv, rope,  \
                       (T*)Kc, (T*)Vc, cap, (T*)ACT, ld_act, scale, rmap);                                       \
    return hipGetLastError();                                                                                   \
  }
  if (f32) {
    BT_LOC(float, 32) BT_LOC(float, 64) BT_LOC(float, 128)
  } else {
    BT_LOC(f16, 64) BT_LOC(f16, 128)
  }
#undef BT_LOC
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------- cross-attention (token decoder)
// Context injection by cross-attention: query head h of row b (QKV row b, columns qoff + h*DH, no
// rotary embedding) attends to the P encoder states of row b, whose keys and values (fp32) sit in
// XKV rows b*P + p at columns koff + hk*DH and koff + Hkv*DH + hk*DH, hk = h / (H / Hkv).  One
// wave per (row, head) with the layout of the local-attention step: DH / 8 lanes per key holding 8
// dimensions each, an online softmax (base 2) per key group, groups merged with shuffles.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_cross_attn(const T* __restrict__ QKV, int ldq, int qoff, int B, int H,
                                                    int Hkv, const float* __restrict__ XKV, int ldx, int koff, int P,
                                                    T* __restrict__ ACT, int ld_act, int act_col, float scale_log2) {
  constexpr int LPK = DH / 8, KPP = 64 / LPK;
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= B * H) return;  // whole wave
  const int b = pair / H, h = pair % H, hk = h / (H / Hkv);
  const int g = lane % LPK, kg = lane / LPK;  // dimensions [8g, 8g + 8), key group
  float q[8];
  load8(QKV + (size_t)b * ldq + qoff + h * DH + 8 * g, q);
  const float* kb = XKV + (size_t)b * P * ldx + koff + hk * DH + 8 * g;
  const float* vb = kb + Hkv * DH;
  float mrun = -INFINITY, lrun = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int p0 = 0; p0 < P; p0 += KPP) {
    const int p = p0 + kg, pc = min(p, P - 1);
    float kc[8], vc[8];
    load8(kb + (size_t)pc * ldx, kc);
    load8(vb + (size_t)pc * ldx, vc);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(q[e], kc[e], dot);
    dot = sum_lanes<LPK>(dot);
    const float sc = p < P ? dot * scale_log2 : -INFINITY;
    const float mn = fmaxf(mrun, sc);
    const float corr = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float pr = sc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc - mn);
    lrun = lrun * corr + pr;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * corr + pr * vc[e];
    mrun = mn;
  }
#pragma unroll
  for (int w = LPK; w < 64; w <<= 1) {
    const float mo = __shfl_xor(mrun, w, 64), lo = __shfl_xor(lrun, w, 64);
    const float mn = fmaxf(mrun, mo);
    const float c1 = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
    const float c2 = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
    lrun = lrun * c1 + lo * c2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * c1 + __shfl_xor(o[e], w, 64) * c2;
    mrun = mn;
  }
  if (kg == 0) {
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    store8(ACT + opnd_idx(ACT, b, act_col + h * DH + 8 * g, ld_act), o);
  }
}

hipError_t launch_cross_attention(bool f32, const void* QKV, int ldq, int qoff, int B, int H, int Hkv, int dh,
                                  const float* XKV, int ldx, int koff, int P, void* ACT, int ld_act, int act_col,
                                  hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if (P < 1 || Hkv < 1 || H % Hkv || ldq % 8 || qoff % 8 || ldx % 8 || koff % 8 || act_col % 8)
    return hipErrorInvalidValue;
  const float sl2 = kLog2e / sqrtf((float)dh);
  const dim3 grid((B * H + 3) / 4);
#define BT_XA(T, DHV)                                                                                          \
  if (dh == DHV) {                                                                                             \
    hipLaunchKernelGGL((k_cross_attn<T, DHV>), grid, dim3(256), 0, st, (const T*)QKV, ldq, qoff, B, H, Hkv, XKV, \
                       ldx, koff, P, (T*)ACT, ld_act, act_col, sl2);                                            \
    return hipGetLastError();                                                                                  \
  }
  if (f32) {
    BT_XA(float, 32) BT_XA(float, 64) BT_XA(float, 128)
  } else {
    BT_XA(f16, 64) BT_XA(f16, 128)
  }
#undef BT_XA
  return hipErrorInvalidValue;
}

BT_DEFINE_CLAMP_FLAG_ACCESS(clamp_flag_attention)

}  // namespace bt
