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
__global__ __launch_bounds__(256) void k_embed_prompt(const int32_t* __restrict__ prompt, int T, int Tp, int pad,
                                                      const Tt* __restrict__ E, int V, int De, int L,
                                                      float* __restrict__ X, int* __restrict__ n_state) {
  const int n = Tp / L;
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_state = n;
  const int row = blockIdx.x;  // b * n + i
  const int b = row / n, i = row % n;
  const int D = De * L;
  for (int c = threadIdx.x; c < D; c += 256) {
    int o = c / De, d = c % De;
    int p = i * L + o - (Tp - T);  // position in the unpadded prompt
    int tok = p < 0 ? pad : prompt[(size_t)b * T + p];
    X[(size_t)row * D + c] = load_f32(E + (size_t)clamp_id(tok, V) * De + d);
  }
}

hipError_t launch_embed_prompt(const int32_t* prompt, int B, int T, int Tp, int pad, const void* E,
                               bool tab_bf16, int V, int De, int L, float* X, int* n_state, hipStream_t st) {
  dim3 grid(B * (Tp / L));
  if (tab_bf16)
    hipLaunchKernelGGL(k_embed_prompt<bf16_t>, grid, dim3(256), 0, st, prompt, T, Tp, pad, (const bf16_t*)E, V,
                       De, L, X, n_state);
  else
    hipLaunchKernelGGL(k_embed_prompt<float>, grid, dim3(256), 0, st, prompt, T, Tp, pad, (const float*)E, V, De,
                       L, X, n_state);
  return hipGetLastError();
}

template <typename Tt>
__global__ __launch_bounds__(256) void k_embed_rows(const int32_t* __restrict__ cur, int L, int j0, int nt,
                                                    const Tt* __restrict__ E, int V, int W,
                                                    float* __restrict__ X) {
  // row b: X[b][o*W + d] = E[cur[b*L + j0 + o]][d] for o < nt
  const int b = blockIdx.x;
  const int D = W * nt;
  for (int c = threadIdx.x; c < D; c += 256) {
    int o = c / W, d = c % W;
    int tok = clamp_id(cur[b * L + j0 + o], V);
    X[(size_t)b * D + c] = load_f32(E + (size_t)tok * W + d);
  }
}

hipError_t launch_embed_block(const int32_t* cur, int B, int L, const void* E, bool tab_bf16, int V, int De,
                              float* X, hipStream_t st) {
  if (tab_bf16)
    hipLaunchKernelGGL(k_embed_rows<bf16_t>, dim3(B), dim3(256), 0, st, cur, L, 0, L, (const bf16_t*)E, V, De, X);
  else
    hipLaunchKernelGGL(k_embed_rows<float>, dim3(B), dim3(256), 0, st, cur, L, 0, L, (const float*)E, V, De, X);
  return hipGetLastError();
}

hipError_t launch_embed_token(const int32_t* cur, int B, int L, int j, const void* E, bool tab_bf16, int V, int D,
                              float* X, hipStream_t st) {
  if (tab_bf16)
    hipLaunchKernelGGL(k_embed_rows<bf16_t>, dim3(B), dim3(256), 0, st, cur, L, j, 1, (const bf16_t*)E, V, D, X);
  else
    hipLaunchKernelGGL(k_embed_rows<float>, dim3(B), dim3(256), 0, st, cur, L, j, 1, (const float*)E, V, D, X);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LayerNorm
// TPR threads per row (one wave for the many-row prefill case, a whole workgroup for the few-row
// decode case), PER values per thread held in registers (D <= TPR * PER); biased variance from the
// centred values.  Optionally completes a pending split-K residual update first (see ResidPending).
template <int TPR>
__device__ __forceinline__ float row_sum(float v, float* red) {
  v = wave_sum(v);
  if constexpr (TPR == 64) {
    return v;
  } else {
    const int w = (threadIdx.x >> 6) & (TPR / 64 - 1);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < TPR / 64; ++i) t += red[i];
    return t;
  }
}

template <int TPR, int PER, typename To>
__global__ __launch_bounds__(256) void k_layernorm(float* __restrict__ X, int rows, int D, int stride, int off,
                                                   const float* __restrict__ p1, To* __restrict__ o1,
                                                   const float* __restrict__ p2, To* __restrict__ o2, float eps,
                                                   ResidPending rp) {
  __shared__ float red[4];
  constexpr int RPB = 256 / TPR;  // rows per block
  constexpr int MAXS = 16;        // split-K partials folded in (at most)
  const int t = threadIdx.x % TPR;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  if (TPR == 64 && r >= rows) return;  // (TPR == 256: one row per block, always valid)
  const size_t xr = (size_t)r * stride + off;
  float* __restrict__ x = X + xr * D;
  const float* __restrict__ part = rp.part;
  // Every load is issued before any arithmetic and none sits behind a divergent branch (indices
  // are clamped and out-of-range values masked afterwards), so the row costs one memory round trip.
  float v[PER], g1[PER], b1[PER], g2[PER], b2[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = t + TPR * j;
    const int cc = min(c, D - 1);
    const float xv = x[cc];
    v[j] = c < D ? xv : 0.f;
    g1[j] = p1[cc];
    b1[j] = p1[D + cc];
    if (o2) {
      g2[j] = p2[cc];
      b2[j] = p2[D + cc];
    }
  }
  if (rp.nsplit > 0) {
    float add[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int cc = min(t + TPR * j, D - 1);
      add[j] = rp.bias_a[cc] + rp.bias_b[cc];
    }
#pragma unroll
    for (int q = 0; q < MAXS; ++q) {
      const int qq = min(q, rp.nsplit - 1);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int cc = min(t + TPR * j, D - 1);
        const float pv = part[((size_t)qq * rp.part_rows + xr) * D + cc];
        add[j] += q < rp.nsplit ? pv : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = t + TPR * j;
      if (c < D) {
        v[j] += add[j];
        x[c] = v[j];
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) s += v[j];
  s = row_sum<TPR>(s, red);
  const float mean = s / (float)D;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = t + TPR * j;
    const float d = c < D ? v[j] - mean : 0.f;
    q += d * d;
  }
  q = row_sum<TPR>(q, red);
  const float rstd = 1.0f / sqrtf(q / (float)D + eps);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = t + TPR * j;
    if (c < D) {
      const float y = (v[j] - mean) * rstd;
      store_from_f32(o1 + (size_t)r * D + c, y * g1[j] + b1[j]);
      if (o2) store_from_f32(o2 + (size_t)r * D + c, y * g2[j] + b2[j]);
    }
  }
}

template <int TPR, int PER>
static void launch_ln_cfg(int rows, float* X, int D, int stride, int off, const float* p1, void* out1,
                          const float* p2, void* out2, bool out_f32, float eps, const ResidPending& rp,
                          hipStream_t st) {
  const int blocks = (rows + 256 / TPR - 1) / (256 / TPR);
  if (out_f32)
    hipLaunchKernelGGL((k_layernorm<TPR, PER, float>), dim3(blocks), dim3(256), 0, st, X, rows, D, stride, off, p1,
                       (float*)out1, p2, (float*)out2, eps, rp);
  else
    hipLaunchKernelGGL((k_layernorm<TPR, PER, f16>), dim3(blocks), dim3(256), 0, st, X, rows, D, stride, off, p1,
                       (f16*)out1, p2, (f16*)out2, eps, rp);
}

hipError_t launch_layernorm(float* X, int rows, int D, int stride, int off, const float* p1, void* out1,
                            const float* p2, void* out2, bool out_f32, float eps, const ResidPending* resid,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  ResidPending rp{};
  if (resid) rp = *resid;
  if (rows <= 1024) {
    // few rows: one workgroup per row
    const int per = (D + 255) / 256;
    if (per <= 1)
      launch_ln_cfg<256, 1>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 3)
      launch_ln_cfg<256, 3>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 8)
      launch_ln_cfg<256, 8>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 16)
      launch_ln_cfg<256, 16>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else
      return hipErrorInvalidValue;
  } else {
    const int per = (D + 63) / 64;
    if (per <= 2)
      launch_ln_cfg<64, 2>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 12)
      launch_ln_cfg<64, 12>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 32)
      launch_ln_cfg<64, 32>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else if (per <= 64)
      launch_ln_cfg<64, 64>(rows, X, D, stride, off, p1, out1, p2, out2, out_f32, eps, rp, st);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- greedy ids
// One workgroup per row reduces the classifier's partial maxima (packed value/id keys) in a fixed
// order; the largest key is the largest logit with the lowest id among equals.
__global__ __launch_bounds__(256) void k_finalize(const unsigned long long* __restrict__ keys, int nparts, int ld,
                                                  int32_t* __restrict__ next, int32_t* __restrict__ cur, int L,
                                                  int j, int* __restrict__ n_state, int n_inc) {
  __shared__ unsigned long long red[256];
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0 && n_inc) *n_state += n_inc;
  unsigned long long best = 0ull;
  for (int p = threadIdx.x; p < nparts; p += 256) {
    const unsigned long long k = keys[(size_t)p * ld + b];
    best = k > best ? k : best;
  }
  red[threadIdx.x] = best;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const unsigned long long k = red[threadIdx.x + o];
      if (k > red[threadIdx.x]) red[threadIdx.x] = k;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int id = (int)(0xFFFFFFFFu - (unsigned)(red[0] & 0xFFFFFFFFull));
    next[b] = id;
    cur[b * L + j] = id;
  }
}
hipError_t launch_finalize(const unsigned long long* keys, int nparts, int ld, int B, int32_t* next, int32_t* cur,
                           int L, int j, int* n_state, int n_inc, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3(B), dim3(256), 0, st, keys, nparts, ld, next, cur, L, j, n_state, n_inc);
  return hipGetLastError();
}

}  // namespace bt
