// Weight repack, rotary table, embedders, LayerNorm and greedy-id kernels.
#include "bt_internal.h"
#include "device_common.h"

namespace bt {

// ---------------------------------------------------------------- repack

// dst[(row0 + n) * ld_dst + col0 + k] = scale * src[k * N + n]: a [K, N] matrix stored as its
// transpose, tiled through LDS so that both the reads and the writes are coalesced.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void k_transpose_convert(const Tin* __restrict__ src, int K, int N,
                                                           Tout* __restrict__ dst, int ld_dst, int row0,
                                                           int col0, float scale) {
  __shared__ float tile[32][33];
  const int k0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    int k = k0 + r, n = n0 + tx;
    tile[r][tx] = (k < K && n < N) ? load_f32(src + (size_t)k * N + n) : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    int n = n0 + r, k = k0 + tx;
    if (n < N && k < K) store_from_f32(dst + (size_t)(row0 + n) * ld_dst + col0 + k, tile[tx][r] * scale);
  }
}

hipError_t launch_transpose_convert(const void* src, bool src_bf16, int K, int N, void* dst, bool dst_f32,
                                    int ld_dst, int row0, int col0, float scale, hipStream_t st) {
  dim3 grid((N + 31) / 32, (K + 31) / 32);
  if (src_bf16) {
    if (dst_f32)
      hipLaunchKernelGGL((k_transpose_convert<bf16_t, float>), grid, dim3(256), 0, st, (const bf16_t*)src, K, N,
                         (float*)dst, ld_dst, row0, col0, scale);
    else
      hipLaunchKernelGGL((k_transpose_convert<bf16_t, f16>), grid, dim3(256), 0, st, (const bf16_t*)src, K, N,
                         (f16*)dst, ld_dst, row0, col0, scale);
  } else {
    if (dst_f32)
      hipLaunchKernelGGL((k_transpose_convert<float, float>), grid, dim3(256), 0, st, (const float*)src, K, N,
                         (float*)dst, ld_dst, row0, col0, scale);
    else
      hipLaunchKernelGGL((k_transpose_convert<float, f16>), grid, dim3(256), 0, st, (const float*)src, K, N,
                         (f16*)dst, ld_dst, row0, col0, scale);
  }
  return hipGetLastError();
}

// fp16 weights in fragment order (frag_off): rows [row0, row0 + N) and columns [col0, col0 + K)
// of a destination of width Ktot receive scale * (element (n, k) of the source, at
// src[n * sn + k * sk]); rows n >= n_valid are zero.  One thread writes 8 consecutive columns.
// With wflags (a weight matrix at bt_init): a scaled value beyond fp16's range or not finite sets
// wflags[0] to at most tensor_id; a value fp16 cannot hold exactly (a magnitude below its
// subnormal spacing) adds one to wflags[1].  Without it (an activation operand) values are
// clamped like every other fp16 activation.
template <typename Tin>
__global__ __launch_bounds__(256) void k_pack_frag(const Tin* __restrict__ src, size_t sn, size_t sk, int n_valid,
                                                   int N, int K, f16* __restrict__ dst, int Ktot, int row0, int col0,
                                                   float scale, int* __restrict__ wflags, int tensor_id) {
  const size_t total = (size_t)N * (K / 8);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int n = (int)(i % N), kc = (int)(i / N);
    half8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = n < n_valid ? load_f32(src + (size_t)n * sn + (size_t)(kc * 8 + e) * sk) * scale : 0.f;
      if (wflags) {
        const f16 hv = (f16)fminf(fmaxf(v, -65504.f), 65504.f);
        if (!(fabsf(v) <= 65504.f)) atomicMin(&wflags[0], tensor_id);
        else if ((float)hv != v) atomicAdd(&wflags[1], 1);
        w[e] = hv;
      } else {
        w[e] = to_f16(v);
      }
    }
    *(half8*)(dst + frag_off(row0 + n, col0 + kc * 8, Ktot)) = w;
  }
}

hipError_t launch_pack_frag(const void* src, bool src_bf16, size_t sn, size_t sk, int n_valid, int N, int K,
                            void* dst, int Ktot, int row0, int col0, float scale, hipStream_t st, int* wflags,
                            int tensor_id) {
  if (K % 8 || col0 % 8 || Ktot % 32 || row0 % 16) return hipErrorInvalidValue;
  const size_t total = (size_t)N * (K / 8);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  if (src_bf16)
    hipLaunchKernelGGL(k_pack_frag<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)src, sn, sk, n_valid, N, K,
                       (f16*)dst, Ktot, row0, col0, scale, wflags, tensor_id);
  else
    hipLaunchKernelGGL(k_pack_frag<float>, dim3(blocks), dim3(256), 0, st, (const float*)src, sn, sk, n_valid, N, K,
                       (f16*)dst, Ktot, row0, col0, scale, wflags, tensor_id);
  return hipGetLastError();
}

// dst[r][c] = scale * src[r][c] for r < rows, 0 for rows <= r < rows_pad
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void k_convert_rows(const Tin* __restrict__ src, int rows, int cols,
                                                      int rows_pad, Tout* __restrict__ dst, float scale) {
  size_t total = (size_t)rows_pad * cols;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    size_t r = i / cols;
    float v = r < (size_t)rows ? load_f32(src + i) * scale : 0.f;
    store_from_f32(dst + i, v);
  }
}

hipError_t launch_convert_rows(const void* src, bool src_bf16, int rows, int cols, int rows_pad, void* dst,
                               bool dst_f32, float scale, hipStream_t st) {
  size_t total = (size_t)rows_pad * cols;
  int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  if (src_bf16) {
    if (dst_f32)
      hipLaunchKernelGGL((k_convert_rows<bf16_t, float>), dim3(blocks), dim3(256), 0, st, (const bf16_t*)src, rows,
                         cols, rows_pad, (float*)dst, scale);
    else
      hipLaunchKernelGGL((k_convert_rows<bf16_t, f16>), dim3(blocks), dim3(256), 0, st, (const bf16_t*)src, rows,
                         cols, rows_pad, (f16*)dst, scale);
  } else {
    if (dst_f32)
      hipLaunchKernelGGL((k_convert_rows<float, float>), dim3(blocks), dim3(256), 0, st, (const float*)src, rows,
                         cols, rows_pad, (float*)dst, scale);
    else
      hipLaunchKernelGGL((k_convert_rows<float, f16>), dim3(blocks), dim3(256), 0, st, (const float*)src, rows,
                         cols, rows_pad, (f16*)dst, scale);
  }
  return hipGetLastError();
}

hipError_t launch_to_f32(const void* src, bool src_bf16, int n, float* dst, hipStream_t st) {
  return launch_convert_rows(src, src_bf16, 1, n, 1, dst, true, 1.0f, st);
}

__global__ void k_add_f32(float* dst, const float* a, int n) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] += a[i];
}
hipError_t launch_add_f32(float* dst, const float* a, int n, hipStream_t st) {
  hipLaunchKernelGGL(k_add_f32, dim3((n + 255) / 256), dim3(256), 0, st, dst, a, n);
  return hipGetLastError();
}

// X[b][:] = base[:] + add[b][:] (add optional): the start slot of a local sequence
__global__ void k_rows_init(float* __restrict__ X, int D, const float* __restrict__ base,
                            const float* __restrict__ add, int add_ld) {
  const int b = blockIdx.y, d = blockIdx.x * 256 + threadIdx.x;
  if (d < D) X[(size_t)b * D + d] = base[d] + (add ? add[(size_t)b * add_ld + d] : 0.f);
}
hipError_t launch_rows_init(float* X, int B, int D, const float* base, const float* add, int add_ld,
                            hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rows_init, dim3((D + 255) / 256, B), dim3(256), 0, st, X, D, base, add, add_ld);
  return hipGetLastError();
}

// Rotary table: tab[p][i] = (cos, sin)(p * base^(-2i/dh)), angles in double precision.
__global__ void k_rope_table(float2* tab, int npos, int dh, double base) {
  int half = dh / 2;
  int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= npos * half) return;
  int p = idx / half, i = idx % half;
  double inv = pow(base, -2.0 * (double)i / (double)dh);
  double a = (double)p * inv;
  tab[idx] = make_float2((float)cos(a), (float)sin(a));
}
hipError_t launch_rope_table(float2* tab, int npos, int dh, float base, hipStream_t st) {
  int n = npos * (dh / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((n + 255) / 256), dim3(256), 0, st, tab, npos, dh, (double)base);
  return hipGetLastError();
}

// ---------------------------------------------------------------- embedders
// Token ids outside [0, V) are clamped into range (never read out of bounds).

__device__ __forceinline__ int clamp_id(int t, int V) { return t < 0 ? 0 : (t >= V ? V - 1 : t); }

template <typename Tt>
__global__ __launch_bounds__(256) void k_embed_prompt(const int32_t* __restrict__ prompt,
                                                      const int32_t* __restrict__ lengths, int T, int Tp, int pad,
                                                      const Tt* __restrict__ E, int V, int De, int L,
                                                      float* __restrict__ X, int* __restrict__ n_state, int ragged,
                                                      const int* __restrict__ rmap, int* __restrict__ last) {
  const int n = Tp / L;        // blocks per row in the activation layout
  const int row = blockIdx.x;  // b * n + i
  const int b = row / n, i = row % n;
  const int D = De * L;
  const int len = lengths ? min(max(lengths[b], 1), T) : T;
  // blocks of this row: every row padded to Tp, or (ragged) to its own multiple of L, left-aligned
  const int nb = ragged ? (len + L - 1) / L : n;
  if (i == 0 && threadIdx.x == 0) {
    n_state[rmap ? rmap[b] : b] = nb;
    if (last) last[b] = nb - 1;
  }
  for (int c = threadIdx.x; c < D; c += 256) {
    int o = c / De, d = c % De;
    int p = i * L + o - (nb * L - len);  // position in the row's unpadded prompt
    int tok = (p < 0 || i >= nb) ? pad : prompt[(size_t)b * T + p];
    X[(size_t)row * D + c] = load_f32(E + (size_t)clamp_id(tok, V) * De + d);
  }
}

hipError_t launch_embed_prompt(const int32_t* prompt, const int32_t* lengths, int B, int T, int Tp, int pad,
                               const void* E, bool tab_bf16, int V, int De, int L, float* X, int* n_state,
                               bool ragged, const int* rmap, int* last, hipStream_t st) {
  dim3 grid(B * (Tp / L));
  if (tab_bf16)
    hipLaunchKernelGGL(k_embed_prompt<bf16_t>, grid, dim3(256), 0, st, prompt, lengths, T, Tp, pad, (const bf16_t*)E,
                       V, De, L, X, n_state, (int)ragged, rmap, last);
  else
    hipLaunchKernelGGL(k_embed_prompt<float>, grid, dim3(256), 0, st, prompt, lengths, T, Tp, pad, (const float*)E, V,
                       De, L, X, n_state, (int)ragged, rmap, last);
  return hipGetLastError();
}

// X row (b, n - 1) = X row (b, last[b]): the last real block of a ragged row where the prefill
// tail reads its context embedding
__global__ void k_gather_last(float* __restrict__ X, int n, int D, const int* __restrict__ last) {
  const int b = blockIdx.y, d = blockIdx.x * 256 + threadIdx.x;
  const int src = last[b];
  if (d < D && src != n - 1) X[((size_t)b * n + n - 1) * D + d] = X[((size_t)b * n + src) * D + d];
}
hipError_t launch_gather_last(float* X, int B, int n, int D, const int* last, hipStream_t st) {
  hipLaunchKernelGGL(k_gather_last, dim3((D + 255) / 256, B), dim3(256), 0, st, X, n, D, last);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LayerNorm
// TPR threads per row (one wave for the many-row prefill case, a whole workgroup for the few-row
// decode case), PER values per thread held in registers (D <= TPR * PER); biased variance from the
// centred values.  Optionally completes a pending split-K residual update first (see ResidPending).
template <int TPR>
__device__ __forceinline__ float row_sum(float v, float* red) {
  // red[4] is written once per call: a caller reducing twice passes two arrays, so no barrier is
  // needed before the writes
  v = wave_sum(v);
  if constexpr (TPR == 64) {
    return v;
  } else {
    const int w = (threadIdx.x >> 6) & (TPR / 64 - 1);
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < TPR / 64; ++i) t += red[i];
    return t;
  }
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// TPR threads per row (64: one wave, 256: the whole workgroup); thread t of a row holds the
// 4-column chunks t, t + TPR, ... (CPT of them).  MAXS > 0: fold up to MAXS split-K partials.
template <int TPR, int CPT, int MAXS, typename To>
__global__ __launch_bounds__(256) void k_layernorm(float* __restrict__ X, int rows, int D, int stride, int off,
                                                   const float* __restrict__ p1, To* __restrict__ o1,
                                                   const float* __restrict__ p2, To* __restrict__ o2, float eps,
                                                   ResidPending rp) {
  __shared__ float red[2][4];
  constexpr int RPB = 256 / TPR;  // rows per block
  const int t = threadIdx.x % TPR;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  if (TPR == 64 && r >= rows) return;  // (TPR == 256: one row per block, always valid)
  const int nch = D >> 2;
  const size_t xr = (size_t)r * stride + off;
  float* __restrict__ x = X + xr * D;
  // Every load is issued before any arithmetic and none sits behind a divergent branch (indices
  // are clamped and out-of-range values masked afterwards), so the row costs one memory round trip.
  float4 v[CPT], g1[CPT], b1[CPT], g2[CPT], b2[CPT];
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = t + TPR * j, cc = 4 * min(c, nch - 1);
    const float4 xv = *(const float4*)(x + cc);
    v[j] = c < nch ? xv : zero;
    g1[j] = *(const float4*)(p1 + cc);
    b1[j] = *(const float4*)(p1 + D + cc);
    if (o2) {
      g2[j] = *(const float4*)(p2 + cc);
      b2[j] = *(const float4*)(p2 + D + cc);
    }
  }
  if constexpr (MAXS > 0) {
    if (rp.nsplit > 0) {
      float4 add[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int cc = 4 * min(t + TPR * j, nch - 1);
        add[j] = f4add(*(const float4*)(rp.bias_a + cc), *(const float4*)(rp.bias_b + cc));
      }
      // every partial in flight at once, then the sums (in split order)
      float4 pv[MAXS][CPT];
#pragma unroll
      for (int q = 0; q < MAXS; ++q) {
        const int qq = min(q, rp.nsplit - 1);
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const int cc = 4 * min(t + TPR * j, nch - 1);
          pv[q][j] = *(const float4*)(rp.part + ((size_t)qq * rp.part_rows + xr) * D + cc);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < MAXS; ++q)
#pragma unroll
        for (int j = 0; j < CPT; ++j) add[j] = f4add(add[j], q < rp.nsplit ? pv[q][j] : zero);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = t + TPR * j;
        if (c < nch) {
          v[j] = f4add(v[j], add[j]);
          *(float4*)(x + 4 * c) = v[j];
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  s = row_sum<TPR>(s, red[0]);
  const float mean = s / (float)D;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (t + TPR * j < nch) {
      const float d0 = v[j].x - mean, d1 = v[j].y - mean, d2 = v[j].z - mean, d3 = v[j].w - mean;
      q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
  }
  q = row_sum<TPR>(q, red[1]);
  const float rstd = 1.0f / sqrtf(q / (float)D + eps);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = t + TPR * j;
    if (c < nch) {
      const float y0 = (v[j].x - mean) * rstd, y1 = (v[j].y - mean) * rstd;
      const float y2 = (v[j].z - mean) * rstd, y3 = (v[j].w - mean) * rstd;
      store4(o1, opnd_idx(o1, r, 4 * c, D), y0 * g1[j].x + b1[j].x, y1 * g1[j].y + b1[j].y, y2 * g1[j].z + b1[j].z,
             y3 * g1[j].w + b1[j].w);
      if (o2)
        store4(o2, opnd_idx(o2, r, 4 * c, D), y0 * g2[j].x + b2[j].x, y1 * g2[j].y + b2[j].y,
               y2 * g2[j].z + b2[j].z, y3 * g2[j].w + b2[j].w);
    }
  }
}

template <int TPR, int CPT, int MAXS>
static void launch_ln_cfg(int rows, float* X, int D, int stride, int off, const float* p1, void* out1,
                          const float* p2, void* out2, bool out_f32, float eps, const ResidPending& rp,
                          hipStream_t st) {
  const int blocks = (rows + 256 / TPR - 1) / (256 / TPR);
  if (out_f32)
    hipLaunchKernelGGL((k_layernorm<TPR, CPT, MAXS, float>), dim3(blocks), dim3(256), 0, st, X, rows, D, stride, off,
                       p1, (float*)out1, p2, (float*)out2, eps, rp);
  else
    hipLaunchKernelGGL((k_layernorm<TPR, CPT, MAXS, f16>), dim3(blocks), dim3(256), 0, st, X, rows, D, stride, off,
                       p1, (f16*)out1, p2, (f16*)out2, eps, rp);
}

template <int CPT>
static void launch_ln_small(int rows, float* X, int D, int stride, int off, const float* p1, void* out1,
                            const float* p2, void* out2, bool out_f32, float eps, const ResidPending& rp,
                            hipStream_t st) {
  if (rp.nsplit <= 0)
    launch_ln_cfg<256, CPT, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
  else if (rp.nsplit <= 8)
    launch_ln_cfg<256, CPT, 8>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
  else if (rp.nsplit <= 10)  // (the fused local attention + [out|down] launch of a 12-head model)
    launch_ln_cfg<256, CPT, 10>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
  else if (rp.nsplit <= 12)
    launch_ln_cfg<256, CPT, 12>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
  else
    launch_ln_cfg<256, CPT, 16>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
}

// Many rows (prefill), fp16 outputs in fragment order: a workgroup normalises one 16-row group,
// each wave 4 rows with all their loads in flight (one wave per row, as above: the same sums in
// the same order), assembles the group's fragment tiles in LDS and writes them out as one
// contiguous range with 16-byte stores (the tiles of a 16-row group are contiguous in fragment
// order; per-row stores would scatter 8-byte pieces 256 bytes apart).  D <= 256 CPT, D % 32 == 0.
// Rows of the last group past `rows` repeat the last row (padding rows no consumer reads).
template <int CPT>
__global__ __launch_bounds__(256) void k_layernorm_g16(const float* __restrict__ X, int rows, int D,
                                                       const float* __restrict__ p1, f16* __restrict__ o1,
                                                       const float* __restrict__ p2, f16* __restrict__ o2,
                                                       float eps) {
  __shared__ __attribute__((aligned(16))) f16 tiles[2][16 * 256 * CPT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, grp = blockIdx.x;
  const int nch = D >> 2;
  float4 g1[CPT], b1[CPT], g2[CPT], b2[CPT], v[4][CPT];
  uint32_t trk = 0u;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int cc = 4 * min(lane + 64 * j, nch - 1);
    g1[j] = *(const float4*)(p1 + cc);
    b1[j] = *(const float4*)(p1 + D + cc);
    if (o2) {
      g2[j] = *(const float4*)(p2 + cc);
      b2[j] = *(const float4*)(p2 + D + cc);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = min(16 * grp + 4 * wave + rr, rows - 1);
#pragma unroll
    for (int j = 0; j < CPT; ++j) v[rr][j] = *(const float4*)(X + (size_t)row * D + 4 * min(lane + 64 * j, nch - 1));
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * wave + rr;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      if (lane + 64 * j < nch) s += (v[rr][j].x + v[rr][j].y) + (v[rr][j].z + v[rr][j].w);
    s = wave_sum(s);
    const float mean = s / (float)D;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (lane + 64 * j < nch) {
        const float d0 = v[rr][j].x - mean, d1 = v[rr][j].y - mean, d2 = v[rr][j].z - mean, d3 = v[rr][j].w - mean;
        q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
      }
    }
    q = wave_sum(q);
    const float rstd = 1.0f / sqrtf(q / (float)D + eps);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) {
        const float y0 = (v[rr][j].x - mean) * rstd, y1 = (v[rr][j].y - mean) * rstd;
        const float y2 = (v[rr][j].z - mean) * rstd, y3 = (v[rr][j].w - mean) * rstd;
        const size_t o = frag_off(r, 4 * c, D);
        store4(tiles[0], o, y0 * g1[j].x + b1[j].x, y1 * g1[j].y + b1[j].y, y2 * g1[j].z + b1[j].z,
               y3 * g1[j].w + b1[j].w, trk);
        if (o2)
          store4(tiles[1], o, y0 * g2[j].x + b2[j].x, y1 * g2[j].y + b2[j].y, y2 * g2[j].z + b2[j].z,
                 y3 * g2[j].w + b2[j].w, trk);
      }
    }
  }
  clamp_note(trk);
  __syncthreads();
  const size_t base = (size_t)grp * 16 * D;
  for (int i = threadIdx.x; i < 2 * D; i += 256) {  // 16 D halves = 2 D chunks of 16 bytes
    *(half8*)(o1 + base + 8 * i) = *(const half8*)(tiles[0] + 8 * i);
    if (o2) *(half8*)(o2 + base + 8 * i) = *(const half8*)(tiles[1] + 8 * i);
  }
}

// Many rows of a wide model (D > 768), fp16 outputs in fragment order: lane l of a wave owns the
// column octets l, l + 64, ... (C8 of them), so each output write is one 16-byte operand piece, and
// the 4 consecutive rows of a wave put their pieces of an octet side by side (64 contiguous bytes
// of a fragment tile), with no LDS staging.  Sums as in the kernels above (per row, centred
// variance).  Rows of the last 16-row group past `rows` repeat the last row.  D % 32 == 0,
// D <= 512 C8.
template <int C8, int RPW>
__global__ __launch_bounds__(256) void k_layernorm_o8(const float* __restrict__ X, int rows, int D,
                                                      const float* __restrict__ p1, f16* __restrict__ o1,
                                                      const float* __restrict__ p2, f16* __restrict__ o2,
                                                      float eps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = 4 * RPW * blockIdx.x + RPW * wave, noct = D >> 3;
  float4 v[RPW][C8][2];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const float* __restrict__ x = X + (size_t)min(r0 + rr, rows - 1) * D;
#pragma unroll
    for (int j = 0; j < C8; ++j) {
      const int c = 8 * min(lane + 64 * j, noct - 1);
      v[rr][j][0] = *(const float4*)(x + c);
      v[rr][j][1] = *(const float4*)(x + c + 4);
    }
  }
  float mean[RPW], rstd[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < C8; ++j)
      if (lane + 64 * j < noct)
        s += ((v[rr][j][0].x + v[rr][j][0].y) + (v[rr][j][0].z + v[rr][j][0].w)) +
             ((v[rr][j][1].x + v[rr][j][1].y) + (v[rr][j][1].z + v[rr][j][1].w));
    mean[rr] = wave_sum(s) / (float)D;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < C8; ++j) {
      if (lane + 64 * j < noct) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float d0 = v[rr][j][h].x - mean[rr], d1 = v[rr][j][h].y - mean[rr];
          const float d2 = v[rr][j][h].z - mean[rr], d3 = v[rr][j][h].w - mean[rr];
          q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
        }
      }
    }
    rstd[rr] = 1.0f / sqrtf(wave_sum(q) / (float)D + eps);
  }
  uint32_t trk = 0u;
#pragma unroll
  for (int j = 0; j < C8; ++j) {
    const int oc = lane + 64 * j;
    if (oc >= noct) continue;
    const int c = 8 * oc;
    float g[8], b[8], g2[8], b2[8];
    {
      const float4 a0 = *(const float4*)(p1 + c), a1 = *(const float4*)(p1 + c + 4);
      const float4 c0 = *(const float4*)(p1 + D + c), c1 = *(const float4*)(p1 + D + c + 4);
      g[0] = a0.x, g[1] = a0.y, g[2] = a0.z, g[3] = a0.w, g[4] = a1.x, g[5] = a1.y, g[6] = a1.z, g[7] = a1.w;
      b[0] = c0.x, b[1] = c0.y, b[2] = c0.z, b[3] = c0.w, b[4] = c1.x, b[5] = c1.y, b[6] = c1.z, b[7] = c1.w;
    }
    if (o2) {
      const float4 a0 = *(const float4*)(p2 + c), a1 = *(const float4*)(p2 + c + 4);
      const float4 c0 = *(const float4*)(p2 + D + c), c1 = *(const float4*)(p2 + D + c + 4);
      g2[0] = a0.x, g2[1] = a0.y, g2[2] = a0.z, g2[3] = a0.w, g2[4] = a1.x, g2[5] = a1.y, g2[6] = a1.z, g2[7] = a1.w;
      b2[0] = c0.x, b2[1] = c0.y, b2[2] = c0.z, b2[3] = c0.w, b2[4] = c1.x, b2[5] = c1.y, b2[6] = c1.z, b2[7] = c1.w;
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const float y[8] = {v[rr][j][0].x, v[rr][j][0].y, v[rr][j][0].z, v[rr][j][0].w,
                          v[rr][j][1].x, v[rr][j][1].y, v[rr][j][1].z, v[rr][j][1].w};
      const size_t o = frag_off(r0 + rr, c, D);
      half8 w1, w2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float n = (y[e] - mean[rr]) * rstd[rr];
        w1[e] = to_f16_trk(n * g[e] + b[e], trk);
        if (o2) w2[e] = to_f16_trk(n * g2[e] + b2[e], trk);
      }
      *(half8*)(o1 + o) = w1;
      if (o2) *(half8*)(o2 + o) = w2;
    }
  }
  clamp_note(trk);
}

hipError_t launch_layernorm(float* X, int rows, int D, int stride, int off, const float* p1, void* out1,
                            const float* p2, void* out2, bool out_f32, float eps, const ResidPending* resid,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (D % 4) return hipErrorInvalidValue;
  ResidPending rp{};
  if (resid) rp = *resid;
  if (rp.nsplit > 16) return hipErrorInvalidValue;
  const int nch = D / 4;
  if (rows <= 1024) {
    // few rows (decode): one workgroup per row
    const int per = (nch + 255) / 256;
    if (per <= 1)
      launch_ln_small<1>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 2)
      launch_ln_small<2>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 4)
      launch_ln_small<4>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else
      return hipErrorInvalidValue;
  } else {
    // one wave per row; split-K partials are only produced for at most 1024 rows
    if (rp.nsplit > 0) return hipErrorInvalidValue;
    const int per = (nch + 63) / 64;
    if (!out_f32 && stride == 1 && off == 0 && D % 32 == 0 && per <= 3) {
      const dim3 grid((rows + 15) / 16);
      if (per == 1)
        hipLaunchKernelGGL(k_layernorm_g16<1>, grid, dim3(256), 0, st, X, rows, D, p1, (f16*)out1, p2, (f16*)out2, eps);
      else if (per == 2)
        hipLaunchKernelGGL(k_layernorm_g16<2>, grid, dim3(256), 0, st, X, rows, D, p1, (f16*)out1, p2, (f16*)out2, eps);
      else
        hipLaunchKernelGGL(k_layernorm_g16<3>, grid, dim3(256), 0, st, X, rows, D, p1, (f16*)out1, p2, (f16*)out2, eps);
      return hipGetLastError();
    }
    // wider rows: 16-byte operand pieces straight from registers (measured at D = 2048, 65 536
    // rows: 328 instead of 498 us on the kernel below; 2 or 1 rows a wave, for more waves per
    // SIMD, were no faster)
    const int per8 = (D / 8 + 63) / 64;
    if (!out_f32 && stride == 1 && off == 0 && D % 32 == 0 && per8 <= 4) {
      constexpr int kRpw = 4;
      const dim3 grid((rows + 15) / 16 * (4 / kRpw));  // whole 16-row groups, padding rows included
      if (per8 <= 2)
        hipLaunchKernelGGL((k_layernorm_o8<2, kRpw>), grid, dim3(256), 0, st, X, rows, D, p1, (f16*)out1, p2, (f16*)out2, eps);
      else
        hipLaunchKernelGGL((k_layernorm_o8<4, kRpw>), grid, dim3(256), 0, st, X, rows, D, p1, (f16*)out1, p2, (f16*)out2, eps);
      return hipGetLastError();
    }
    if (per <= 1)
      launch_ln_cfg<64, 1, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 2)
      launch_ln_cfg<64, 2, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 3)
      launch_ln_cfg<64, 3, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 4)
      launch_ln_cfg<64, 4, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 8)
      launch_ln_cfg<64, 8, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 16)
      launch_ln_cfg<64, 16, 0>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- greedy ids (+ next step's input)
// One workgroup per row reduces the classifier's partial maxima (packed value/id keys) in a fixed
// order; the largest key is the largest logit with the lowest id among equals.  The same workgroup
// then prepares the next decode step's input row: the embedding of the token just chosen (token
// step) or of the block it completes (block step), and the first layer's LN1/LN2 of that row.
struct NextStep {
  int mode;              // 0: nothing, 1: token step (E_tok row), 2: block step (concat of E_emb rows)
  const void* E;         // table of the next step's embedder
  int width;             // row width of that table (D for E_tok, D / L for E_emb)
  float* X;              // residual stream [B][D]
  const float* lnp;      // first layer's LayerNorm parameters [4][D]
  void* ln1;
  void* ln2;
  int D, V;
  float eps;
  const float* add;      // token step: fp32 [B][add_ld] added to the embedding row (or null)
  int add_ld;
};

template <int PER, typename Tt, typename To>
__global__ __launch_bounds__(256) void k_finalize(const unsigned long long* __restrict__ keys, int nparts, int ld,
                                                  int32_t* __restrict__ next, int32_t* __restrict__ cur, int L,
                                                  int j, int* __restrict__ n_state, int n_inc, NextStep ns,
                                                  const int* __restrict__ rmap, int from_cur) {
  __shared__ unsigned long long red[4];
  __shared__ float redf[2][4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int cb = rmap ? rmap[b] : b;  // the row's index in the caches and step state
  if (tid == 0 && n_inc) n_state[cb] += n_inc;
  int id;
  if (from_cur) {
    // only the next step's input, from the id already at offset j of the current block
    id = cur[(size_t)b * L + j];
  } else {
    // the row's keys are contiguous: 256 threads read 8 keys each per pass, all loads in flight
    // together (indices clamped into the row: a repeated key leaves the maximum unchanged)
    const unsigned long long* kr = keys + (size_t)b * ld;
    unsigned long long best = 0ull;
    for (int p0 = 0; p0 < nparts; p0 += 8 * 256) {
      unsigned long long k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) k[u] = kr[min(p0 + tid + 256 * u, nparts - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) best = k[u] > best ? k[u] : best;
    }
    best = wave_max_u64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    best = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) best = red[w] > best ? red[w] : best;
    id = (int)(0xFFFFFFFFu - (unsigned)(best & 0xFFFFFFFFull));
    if (tid == 0) {
      next[b] = id;
      cur[(size_t)cb * L + j] = id;
    }
  }
  if (ns.mode == 0) return;
  const int D = ns.D;
  const Tt* __restrict__ E = (const Tt*)ns.E;
  // token of each of this thread's columns (the block's ids for a block step), then every table
  // load at once: no load waits behind another
  int tok[PER], col[PER];
  if (ns.mode == 1) {
#pragma unroll
    for (int q = 0; q < PER; ++q) tok[q] = id, col[q] = min(tid + 256 * q, D - 1);
  } else {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int cc = min(tid + 256 * q, D - 1), o = cc / ns.width;
      const int cv = cur[(size_t)cb * L + o];
      tok[q] = o == j ? id : cv;
      col[q] = cc - o * ns.width;
    }
  }
  // every load first, through valid (clamped) addresses and behind no branch (the summand of a
  // summation context is read from the parameters when there is none), then the arithmetic
  float v[PER], ad[PER], g1[PER], b1[PER], g2[PER], b2[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int cc = min(tid + 256 * q, D - 1);
    const int t = tok[q] < 0 ? 0 : (tok[q] >= ns.V ? ns.V - 1 : tok[q]);
    v[q] = load_f32(E + (size_t)t * ns.width + col[q]);
    ad[q] = *(ns.add ? ns.add + (size_t)b * ns.add_ld + cc : ns.lnp + cc);
    g1[q] = ns.lnp[cc];
    b1[q] = ns.lnp[D + cc];
    g2[q] = ns.lnp[2 * D + cc];
    b2[q] = ns.lnp[3 * D + cc];
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const float e = ns.add ? v[q] + ad[q] : v[q];
    v[q] = tid + 256 * q < D ? e : 0.f;
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < PER; ++q) s += v[q];
  s = row_sum<256>(s, redf[0]);
  const float mean = s / (float)D;
  float var = 0.f;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = tid + 256 * q;
    const float d = c < D ? v[q] - mean : 0.f;
    var += d * d;
  }
  var = row_sum<256>(var, redf[1]);
  const float rstd = 1.0f / sqrtf(var / (float)D + ns.eps);
  To* o1 = (To*)ns.ln1;
  To* o2 = (To*)ns.ln2;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = tid + 256 * q;
    if (c < D) {
      ns.X[(size_t)b * D + c] = v[q];
      const float y = (v[q] - mean) * rstd;
      store_from_f32(o1 + opnd_idx(o1, b, c, D), y * g1[q] + b1[q]);
      store_from_f32(o2 + opnd_idx(o2, b, c, D), y * g2[q] + b2[q]);
    }
  }
}

template <int PER>
static void launch_fin_cfg(bool tab_bf16, bool out_f32, int B, const unsigned long long* keys, int nparts, int ld,
                           int32_t* next, int32_t* cur, int L, int j, int* n_state, int n_inc, const NextStep& ns,
                           const int* rmap, int from_cur, hipStream_t st) {
  if (tab_bf16) {
    if (out_f32)
      hipLaunchKernelGGL((k_finalize<PER, bf16_t, float>), dim3(B), dim3(256), 0, st, keys, nparts, ld, next, cur, L, j,
                         n_state, n_inc, ns, rmap, from_cur);
    else
      hipLaunchKernelGGL((k_finalize<PER, bf16_t, f16>), dim3(B), dim3(256), 0, st, keys, nparts, ld, next, cur, L, j,
                         n_state, n_inc, ns, rmap, from_cur);
  } else {
    if (out_f32)
      hipLaunchKernelGGL((k_finalize<PER, float, float>), dim3(B), dim3(256), 0, st, keys, nparts, ld, next, cur, L, j,
                         n_state, n_inc, ns, rmap, from_cur);
    else
      hipLaunchKernelGGL((k_finalize<PER, float, f16>), dim3(B), dim3(256), 0, st, keys, nparts, ld, next, cur, L, j,
                         n_state, n_inc, ns, rmap, from_cur);
  }
}

hipError_t launch_finalize(const unsigned long long* keys, int nparts, int ld, int B, int32_t* next, int32_t* cur,
                           int L, int j, int* n_state, int n_inc, const NextStepArgs& a, hipStream_t st,
                           const int* rmap, bool from_cur) {
  if (B <= 0) return hipSuccess;
  NextStep ns{a.mode, a.E, a.width, a.X, a.lnp, a.ln1, a.ln2, a.D, a.V, a.eps, a.add, a.add_ld};
  const int per = (a.D + 255) / 256;
  if (per <= 1)
    launch_fin_cfg<1>(a.tab_bf16, a.out_f32, B, keys, nparts, ld, next, cur, L, j, n_state, n_inc, ns, rmap, (int)from_cur, st);
  else if (per <= 3)
    launch_fin_cfg<3>(a.tab_bf16, a.out_f32, B, keys, nparts, ld, next, cur, L, j, n_state, n_inc, ns, rmap, (int)from_cur, st);
  else if (per <= 8)
    launch_fin_cfg<8>(a.tab_bf16, a.out_f32, B, keys, nparts, ld, next, cur, L, j, n_state, n_inc, ns, rmap, (int)from_cur, st);
  else if (per <= 16)
    launch_fin_cfg<16>(a.tab_bf16, a.out_f32, B, keys, nparts, ld, next, cur, L, j, n_state, n_inc, ns, rmap, (int)from_cur, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// A kernel that does nothing: its back-to-back launches time the fixed cost of one dependent launch
// on the stream (dispatch, workgroup launch, end-of-kernel release), the floor under every decode
// kernel's duration.
__global__ __launch_bounds__(256) void k_empty() {}

hipError_t launch_empty(int workgroups, hipStream_t st) {
  hipLaunchKernelGGL(k_empty, dim3(workgroups), dim3(256), 0, st);
  return hipGetLastError();
}

BT_DEFINE_CLAMP_FLAG_ACCESS(clamp_flag_misc)

}  // namespace bt
