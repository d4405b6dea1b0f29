// Internal declarations of libbt: workspace layout and kernel launchers.
// Device code targets gfx950 (CDNA4): wave64, MFMA f32_16x16x32_f16, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "bt.h"

namespace bt {

typedef _Float16 f16;
typedef uint16_t bf16_bits;

// Pre-scale applied to fp16 weights so that every bf16 weight of magnitude
// >= 2^-22 converts to fp16 exactly (fp16 normals start at 2^-14); the GEMM
// epilogue multiplies the fp32 accumulator by the inverse (exact, power of 2).
constexpr float kWeightScale = 256.0f;
constexpr float kWeightUnscale = 1.0f / 256.0f;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct LayerOff {
  size_t ln;  // fp32 [4][D]: ln1.g, ln1.b, ln2.g, ln2.b
  size_t w1;  // T [N1 = QW + F][D]: rows = output features of q | k | v | up (fp32: K-contiguous;
              //   fp16: fragment order, see frag_off)
  size_t b1;  // fp32 [QW + F]
  size_t w2;  // T [D][D + F]: row n = output feature n of attn.out (k < D) and mlp.down (k >= D),
              //   same layout as w1
  size_t b2;  // fp32 [3][D]: attn.out.b (+ xattn.out.b), mlp.down.b, (xattn.out.b at init)
  int n1;     // q | k | v (| cross-attention q) columns of w1: QW, or QW + D in a token layer with
              //   cross-attention; the up rows follow
  int k2;     // width of the [attn | gelu(up) (| cross-attention)] operand of w2: D + F (+ D)
};

struct Layout {
  // model dimensions
  int V, D, H, dh, F, L, P, Nb, Nt, De;
  int Hkv;      // key/value heads (grouped-query attention: H / Hkv query heads per KV head)
  int QW;       // width of the fused q | k | v projection: D + 2 Hkv dh
  int mode;     // bt_context_mode
  int lead;     // local slots before a block's first token: P (prefix) or 1 (start slot)
  int NC;       // vectors of the context projection: P, or L_B for summation
  int maxN1, maxK2;  // largest LayerOff::n1 and ::k2 (QKV and ACT widths)
  int Bmax, max_tokens;
  int max_prompt;  // longest padded prompt the activations hold (a multiple of L)
  int ncap;     // block-KV entries per (layer, row, KV head), multiple of 64
  int pages;    // paged block KV: pages of 64 entries in the pool (0: one flat cache per row)
  size_t ptab;  // int32 [Bmax][ncap / 64] page table (paged)
  int lcap;     // local-KV entries per (layer, row, KV head) = P + L
  int npos;     // rows of the rotary table
  int Vpad;     // classifier rows padded to a multiple of 128
  int64_t Mmax; // activation rows
  int64_t Mpad; // activation rows rounded up to 16 (fragment-order operands)
  bool f32;     // BT_FP32 mode (fp32 everywhere) vs fp16 operands
  bool vanilla; // n_token_layers == 0: token-level transformer (block decoder + classifier)
  size_t elem;  // bytes per matrix / cache element (4 or 2)
  size_t tab_elem;  // bytes per embedding-table element (blob dtype)
  // workspace regions (byte offsets)
  size_t emb_block, emb_tok, head, lnf_blk, lnf_tok, prefix_w, prefix_b, rope;
  std::vector<LayerOff> blk, tok;
  size_t block_kv, local_kv;
  size_t X;     // fp32 [Mmax][D] residual stream
  size_t LN;    // T [2][Mpad][D] LayerNorm outputs (ln1, ln2); fp16: fragment order
  size_t QKV;   // T [Mmax][QW]
  size_t ACT;   // T [Mpad][D + F]: attention output | GELU(up); fp16: fragment order
  size_t part;  // fp32 split-KV partials of block-attention decode
  size_t part_bytes;
  size_t keys;  // u64 [nparts][Bmax] partial argmax keys of the classifier
  size_t pad_emb;  // fp32 [D] token embedding of pad_id (start slot of summation / cross-attention)
  size_t ctx;      // summation: fp32 [Bmax][L][D] projected summands of the current block
  size_t enc;      // cross-attention: fp32 [Bmax * P][D] encoder states of the current block
  size_t enc16;    // ... the same as an fp16 operand in fragment order (BT_BF16)
  size_t xkv_w;    // cross-attention: T [Nt * 2 Hkv dh][D] key|value projections of all token layers
  size_t xkv_b;    // fp32 [Nt * 2 Hkv dh]
  size_t xkv;      // fp32 [Bmax * P][Nt * 2 Hkv dh] keys and values of the encoder states
  int xkv_ld;      // Nt * 2 Hkv dh
  size_t rpart; // fp32 [16][rpart_rows][D] split-K partials of the [out|down] GEMM (decode)
  int rpart_rows;
  size_t cur;   // int32 [Bmax][L] ids of the block being generated
  size_t dstate;  // int32 [Bmax] device state: block-KV entries of each row (per layer)
  size_t rowmap;  // int32 [Bmax]: cache rows of the rows a join prefills
  size_t lastblk; // int32 [Bmax]: last real prompt block of each prefilled row
  size_t wflags;  // int32 [2]: weight-conversion flags of bt_init (see launch_pack_frag)
  size_t total;
  size_t block_kv_bytes, local_kv_bytes;
  // canonical blob offsets (bytes)
  struct BlobLayer {
    size_t ln1g, ln1b, qkvw, qkvb, outw, outb, ln2g, ln2b, upw, upb, downw, downb;
    size_t xqw = 0, xqb = 0, xkvw = 0, xkvb = 0, xow = 0, xob = 0;  // cross-attention (token layers)
  };
  size_t bl_emb_block, bl_lnf_blk_g, bl_lnf_blk_b, bl_prefix_w, bl_prefix_b, bl_emb_tok, bl_lnf_tok_g,
      bl_lnf_tok_b, bl_head, bl_total;
  std::vector<BlobLayer> bl_blk, bl_tok;
};

// Static scratch (scratch.hip): kStaticScratchBytes of device memory per GPU, for the partial
// results of bt_decode_step_static.  static_scratch() returns its address on the current device
// (looked up once per device with hipGetSymbolAddress).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** ptr);

// Fills `lo` for cfg; returns an empty string or the reason cfg is invalid.
std::string plan_layout(const bt_config& cfg, Layout& lo);

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `st` and return hipGetLastError().

// ---- weight repack (bt_init)
hipError_t launch_transpose_convert(const void* src, bool src_bf16, int K, int N, void* dst, bool dst_f32,
                                    int ld_dst, int row0, int col0, float scale, hipStream_t st);
hipError_t launch_convert_rows(const void* src, bool src_bf16, int rows, int cols, int rows_pad, void* dst,
                               bool dst_f32, float scale, hipStream_t st);
// fp16 weights in fragment order: destination rows [row0, row0 + N), columns [col0, col0 + K) of a
// matrix of width Ktot take scale * src[n * sn + k * sk] (zero for rows n >= n_valid).  wflags
// (weights at bt_init, else null): [0] = min(itself, tensor_id) if a scaled value is beyond fp16's
// range or not finite, [1] += values fp16 rounds (see k_pack_frag).
hipError_t launch_pack_frag(const void* src, bool src_bf16, size_t sn, size_t sk, int n_valid, int N, int K,
                            void* dst, int Ktot, int row0, int col0, float scale, hipStream_t st,
                            int* wflags = nullptr, int tensor_id = 0);
// Clamp flag of each kernel file (see to_f16): copied to *value (and cleared with reset) on st.
hipError_t clamp_flag_misc(unsigned int* value, bool reset, hipStream_t st);
hipError_t clamp_flag_gemm(unsigned int* value, bool reset, hipStream_t st);
hipError_t clamp_flag_gemm_decode(unsigned int* value, bool reset, hipStream_t st);
hipError_t clamp_flag_attention(unsigned int* value, bool reset, hipStream_t st);
hipError_t launch_empty(int workgroups, hipStream_t st);
hipError_t launch_to_f32(const void* src, bool src_bf16, int n, float* dst, hipStream_t st);
hipError_t launch_add_f32(float* dst, const float* a, int n, hipStream_t st);
// X[b][:] = base[:] (+ add[b * add_ld + :] when add is not null), rows b < B of width D
hipError_t launch_rows_init(float* X, int B, int D, const float* base, const float* add, int add_ld,
                            hipStream_t st);
hipError_t launch_rope_table(float2* tab, int npos, int dh, float base, hipStream_t st);

// ---- embedders
// prompt blocks: X[b*n + i][o*De + d] = E[tok(b, i*L + o)][d], n = Tp / L, tok from the left-padded
// prompt: row b holds len_b tokens at positions [0, len_b) (len_b = T without `lengths`, else
// lengths[b] clamped to [1, T]) and is padded on the left to Tp, or with `ragged` to its own
// n_b = ceil(len_b / L) blocks, left-aligned (blocks i >= n_b hold pad tokens).  Sets the row's
// block-KV length n_state[rmap ? rmap[b] : b] = n_b and, if `last` is given, last[b] = n_b - 1.
hipError_t launch_embed_prompt(const int32_t* prompt, const int32_t* lengths, int B, int T, int Tp, int pad, const void* E,
                               bool tab_bf16, int V, int De, int L, float* X, int* n_state, bool ragged,
                               const int* rmap, int* last, hipStream_t st);
// X row (b, n - 1) = X row (b, last[b]) for rows b < B of an activation laid out [B][n][D]
hipError_t launch_gather_last(float* X, int B, int n, int D, const int* last, hipStream_t st);
// ---- LayerNorm over rows r < rows of X[(r*stride + off)][:] -> out1 (params p1), out2 (p2, optional).
// With `resid` (split-K residual update pending), the row is first completed as
//   x = X + sum_{s < nsplit} part[s][row][:] + bias_a + bias_b   (fixed summation order)
// and written back to X.
struct ResidPending {
  const float* part;    // [nsplit][part_rows][D] fp32 partial products of the [out|down] GEMM
  int nsplit, part_rows;
  const float* bias_a;  // attn.out.b
  const float* bias_b;  // mlp.down.b
};
hipError_t launch_layernorm(float* X, int rows, int D, int stride, int off, const float* p1, void* out1,
                            const float* p2, void* out2, bool out_f32, float eps, const ResidPending* resid,
                            hipStream_t st);

// ---- GEMM: C[M][N] = A[M][K] * W[N][K]^T with an epilogue.  fp32: row-major operands (A with
// leading dimension lda).  fp16: both operands in fragment order with width K (lda unused); the
// GELU columns of EPI_QKV_GELU are written to out1 in fragment order (width ld1).
enum EpiMode { EPI_QKV_GELU = 0, EPI_RESID = 1, EPI_STORE = 2, EPI_ARGMAX = 3 };
struct Epi {
  float wscale;             // multiplies the accumulator
  const float* bias;        // [N] (QKV|up, STORE), attn.out.b (RESID); unused for ARGMAX
  const float* bias2;       // mlp.down.b (RESID)
  void* out0;               // QKV (T, ld0) | X (fp32, ld0) | Y (fp32, ld0) | logits (fp32, ld0, may be null)
  void* out1;               // ACT (T, width ld1; fp16: fragment order) for the GELU columns
  int ld0, ld1;
  int n_split;              // QKV_GELU: columns >= n_split take A2 and go through GELU into out1
  int act_col0;             // QKV_GELU: first ACT column of the GELU part
  int n_valid;              // ARGMAX: columns >= n_valid are padding
  unsigned long long* keys; // ARGMAX: packed (value, id) maxima, [M][keys_ld]: per row, one entry
                            // for every column group (entries [0, nparts) written by each launch)
  int keys_ld;              //   >= the number of column groups of any kernel (N / 4 + 64 suffices)
  int* nparts_out;          // ARGMAX: receives the number of column groups
  int splits;               // RESID: K is split over `splits` workgroups per tile (1 = no split)
  float* part;              // RESID with splits > 1: [splits][M][N] fp32 partial products (no bias)
};
// Number of K splits the [out|down] GEMM uses for M rows (1 for large M); also the partial count
// the next LayerNorm must reduce.
int resid_splits(int M, int N, int K);
// Decode-shape (M <= 256) fp16 GEMM (gemm_decode.hip): the configuration a shape runs, and its launch.
struct SkinnyPlan {
  bool ok;             // the shape runs on the skinny kernel
  int mg, mw, ng, kw;  // row groups per wave, waves along M, column groups per wave, waves along K
  int splits;          // K splits over workgroups (EPI_RESID)
  int rg = 1;          // workgroups along M (each 16 mg mw rows)
  int depth = 2;       // K steps in flight per wave
};
// row_groups = false: one workgroup covers all M rows (the fused local attention + [out|down] launch)
SkinnyPlan skinny_plan(int M, int N, int K, EpiMode mode, bool row_groups = true);
hipError_t launch_gemm_skinny(const SkinnyPlan& p, const void* A1, const void* A2, const void* W, int M, int N, int K,
                              EpiMode mode, const Epi& ep, hipStream_t st);
hipError_t launch_gemm(bool f32, const void* A1, const void* A2, int lda, const void* W, int M, int N,
                       int K, EpiMode mode, const Epi& ep, hipStream_t st);

// Decode step of a token-decoder layer with head width 64 (fp16): the local attention of the new
// slot fused into the [out|down] GEMM that consumes it (gemm_decode.hip).  ACT holds the GELU
// columns [D, D + F) of the operand (width K = D + F, fragment order); W is that GEMM's weight.
// Every product goes to ep.part as a split-K partial: attn_out_splits(M, N = D, K, H) of them
// (0: the shape does not run fused), folded with both biases by the next LayerNorm.
struct LocalStep {
  const f16* qkv;  // [M][ldq]: q (H x 64) | k (Hkv x 64) | v (Hkv x 64) of the new slot
  int ldq, H, Hkv, s0;  // s0: local slot of the new entry (= entries already cached)
  const float2* rope;   // [slot][32] (cos, sin)
  f16* kc;              // local keys [cache row][Hkv][cap][64]; the new key is written at slot s0
  f16* vc;              // local values, same layout
  int cap;
  const int* rmap;  // cache row of activation row b (null: b)
  float scale_log2;  // log2(e) / sqrt(64)
  // cross-attention context (xkv null: none): query head h of row b at qkv column xq_off + 64 h;
  // keys and values of its P encoder states (fp32) in xkv rows b P + p, columns xkv_off + 64 hk and
  // xkv_off + 64 (Hkv + hk); the output multiplies the W rows of K range [k_mlp, k_mlp + 64 H)
  const float* xkv;
  int xkv_ld, xkv_off, P, xq_off;
  int k_mlp;  // end of the GELU columns' K range (the whole K without cross-attention)
};
int attn_out_splits(int M, int N, int K, int H);
hipError_t launch_attn_out_decode(const void* ACT, const void* W, int M, int N, int K, const Epi& ep,
                                  const LocalStep& ls, hipStream_t st);

// ---- attention
// Attention launchers take H query heads and Hkv key/value heads of width dh (H % Hkv == 0); a
// QKV row is [q: H dh | k: Hkv dh | v: Hkv dh] and query head h reads KV head h / (H / Hkv).
// Caches are [row][KV head][...].
//
// rotary + scatter of K (row-major [slot][dh]) and V (block cache, v_transposed: groups of 8 slots,
// each transposed, [slot / 8][dh][8]; local cache: row-major) for rows (b, i) of QKV [B*m][QW] into
// cache slots s0 + i, at rotary positions s0 + i.
// (rmap: optional cache row of each activation row b, for a prefill into rows of a running batch;
// the same argument of the prefill and local attention launchers.  ptab / pld: page table of a
// paged block KV (pages of 64 entries, [page][Hkv][64][dh] keys, [page][Hkv][8][dh][8] values),
// nlim: with it, entries past each cache row's length nlim[row] are neither written nor read.)
hipError_t launch_rope_scatter(bool f32, const void* QKV, int B, int m, int s0, int H, int Hkv, int dh,
                               const float2* rope, void* Kc, void* Vc, int cap, bool v_transposed,
                               hipStream_t st, const int* rmap = nullptr, const int* ptab = nullptr, int pld = 0,
                               const int* nlim = nullptr);
// causal prefill attention of rows (b, i < n) at positions i over cache entries [0, i]
hipError_t launch_prefill_attention(bool f32, const void* QKV, int B, int n, int H, int Hkv, int dh,
                                    const float2* rope, const void* Kc, const void* Vc, int cap, void* ACT,
                                    int ld_act, hipStream_t st, const int* rmap = nullptr, const int* ptab = nullptr,
                                    int pld = 0, const int* nlim = nullptr);
// one new block-decoder position per row: n = n_ptr[b] (device state of row b) entries are cached;
// rotary at position n, append K/V at slot n, attend over [0, n].  nsplit = decode_splits(B, H, Hkv, cap)
// splits of the capacity (fixed for a batch size, so the launch does not depend on n).
int decode_splits(int B, int H, int Hkv, int cap);
hipError_t launch_block_attn_decode(bool f32, const void* QKV, int B, const int* n_ptr, int H, int Hkv, int dh,
                                    const float2* rope, void* Kc, void* Vc, int cap, void* ACT, int ld_act,
                                    float* part, size_t part_bytes, int nsplit, hipStream_t st,
                                    const int* ptab = nullptr, int pld = 0);
// local attention: new slots [s0, s0 + m) per row; rotary at slot, write to local cache, attend over [0, slot]
// (ldq = QKV row stride, >= (H + 2 Hkv) dh: token layers with cross-attention carry its queries too)
hipError_t launch_local_attention(bool f32, const void* QKV, int ldq, int B, int m, int s0, int H, int Hkv, int dh,
                                  const float2* rope, void* Kc, void* Vc, int cap, void* ACT, int ld_act,
                                  hipStream_t st, const int* rmap = nullptr);
// cross-attention of one slot per row: query head h of row b (QKV[b * ldq + qoff + h dh ..], no rotary)
// over the P encoder states of row b, keys and values (fp32) at XKV[(b P + p) * ldx + koff + ..]
// (keys of KV head hk at hk dh, values at Hkv dh + hk dh); output to ACT columns act_col + h dh.
hipError_t launch_cross_attention(bool f32, const void* QKV, int ldq, int qoff, int B, int H, int Hkv, int dh,
                                  const float* XKV, int ldx, int koff, int P, void* ACT, int ld_act, int act_col,
                                  hipStream_t st);

// ---- greedy ids from the classifier's partial maxima [B][ld] (nparts per row): next[b] = id,
// cur[b*L + j] = id.
// The step that completes a block also advances the device block-KV length (*n_state += n_inc).
// With next.mode != 0 the same kernel writes the next decode step's input row into X and that
// step's first-layer LN1/LN2 outputs (the next step then starts at its first GEMM).
struct NextStepArgs {
  int mode = 0;          // 0: none, 1: next step is a token step, 2: a block step
  const void* E = nullptr;
  int width = 0;         // table row width (D for the token table, D / L for the block embedder)
  bool tab_bf16 = false, out_f32 = false;
  float* X = nullptr;
  const float* lnp = nullptr;
  void* ln1 = nullptr;
  void* ln2 = nullptr;
  int D = 0, V = 0;
  float eps = 1e-5f;
  const float* add = nullptr;  // token step: fp32 [B][add_ld] added to the embedding (summation)
  int add_ld = 0;
};
// rmap: cache/state row of each row b (cur, n_state); from_cur: no argmax, the next step's input is
// prepared from the id already at cur[b][j] (next, cur and n_state untouched)
hipError_t launch_finalize(const unsigned long long* keys, int nparts, int ld, int B, int32_t* next, int32_t* cur,
                           int L, int j, int* n_state, int n_inc, const NextStepArgs& nxt, hipStream_t st,
                           const int* rmap = nullptr, bool from_cur = false);

}  // namespace bt
