/*
 * bt.h — C-ABI of the Block Transformer inference library (libbt.so, gfx950).
 *
 * The library runs batched inference of a Block Transformer as described on
 * the summary page "Block Transformer: Global-to-Local Language Modeling for
 * Fast Inference" (arXiv 2406.02657):
 *   - §3.2 "Big-Picture Architecture": embedder -> block decoder -> context
 *     embedding -> prefix -> token decoder -> output classifier;
 *   - §3.4 "The Inference Cost Model": inference is a prefill of the whole
 *     prompt followed by one generated token per decode step;
 *   - §3.4 "The Block Decoder": its KV cache holds one entry per block;
 *   - §3.4 "The Token Decoder": its KV cache holds at most prefix + one block
 *     and does not persist across blocks.
 * Generation is greedy (argmax, lowest id on ties).
 *
 * Memory: the caller allocates and owns every device buffer (weights blob,
 * workspace, prompt, outputs) and keeps them alive until bt_destroy.  The
 * library never allocates device memory; it owns only the host-side handle.
 * Calls enqueue work on the HIP stream given to bt_init and return without
 * synchronising; outputs are valid once the caller has synchronised that
 * stream.  A handle is not thread-safe: use it from one thread and stream.
 *
 * Errors: every call validates its arguments and the handle's state on the
 * host before launching anything; on failure it returns a negative bt_status
 * and bt_last_error() describes the cause.  After BT_ERR_HIP the handle is
 * unusable (only bt_destroy is valid).  No exception crosses the ABI.
 */
#ifndef BT_H_
#define BT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bt_handle bt_handle; /* opaque, host-side */

typedef enum {
  BT_OK = 0,
  BT_ERR_INVALID_ARG = -1, /* malformed config, NULL pointer, size mismatch   */
  BT_ERR_CAPACITY = -2,    /* batch or sequence beyond the configured capacity */
  BT_ERR_STATE = -3,       /* call out of order (decode before prefill, ...)   */
  BT_ERR_HIP = -4,         /* a HIP runtime call failed                        */
  BT_ERR_UNSUPPORTED = -5  /* valid config this build does not handle          */
} bt_status;

typedef enum {
  BT_FP32 = 0, /* weights, activations and caches in fp32                     */
  BT_BF16 = 1  /* bf16 weights blob; matrix operands and KV caches held as fp16,
                  fp32 accumulation, fp32 residual stream.  Weight matrices are
                  stored as fp16 after a 2^8 pre-scale: exact for every bf16
                  weight of magnitude in [2^-25, 256) and for every multiple
                  of 2^-32 below; other magnitudes below 2^-25 round to a
                  multiple of 2^-32 (counted, see bt_numerics_status); a
                  magnitude >= 256 or a non-finite value
                  makes bt_init fail.  Activations and cache entries beyond
                  fp16's range are clamped to +-65504 (flagged, same call).   */
} bt_dtype;

/* How the context embedding of the previous block reaches the token decoder (summary page §3.4
 * "The Token Decoder" and its comparison of prefix tokens with summation and cross-attention). */
typedef enum {
  BT_CTX_PREFIX = 0, /* P prefix vectors lead the local sequence (the method's own design)      */
  BT_CTX_SUM = 1,    /* the projection gives L_B vectors; u_i is added to local slot i, which
                        holds a start token (the pad token's embedding) at i = 0 and the block's
                        token i-1 after it; slot i predicts the block's token i                 */
  BT_CTX_XATTN = 2   /* the projection gives P encoder states; the same start-token local
                        sequence; every token-decoder layer adds a cross-attention branch
                        h + Attn(LN1 h) + XAttn(LN1 h) + MLP(LN2 h) (no rotary, no mask)        */
} bt_context_mode;

/* Model and capacity.  Constraints (checked by bt_init and the sizing calls):
 *   d_model % n_heads == 0, d_head = d_model / n_heads in {32, 64, 128};
 *   d_model % block_len == 0 (embedder width d_model / block_len, even);
 *   n_block_layers >= 1, n_token_layers >= 0, block_len >= 1, prefix_len >= 1;
 *   n_token_layers = 0 selects a token-level ("vanilla") transformer on the same kernels: it
 *   needs block_len = 1, and the classifier reads the block decoder's final LayerNorm output
 *   directly (no prefix projection, no token decoder, no local KV);
 *   BT_BF16 also needs d_model % 64 == 0 and d_mlp % 64 == 0;
 *   max_batch >= 1; max_tokens >= block_len (padded prompt + generated);
 *   0 <= max_prompt_tokens <= max_tokens;
 *   n_kv_heads = 0 (multi-head) or a divisor of n_heads (grouped-query; 1 = multi-query);
 *   context_mode a bt_context_mode, BT_CTX_PREFIX when n_token_layers = 0;
 *   0 <= kv_pages <= max_batch * cap / 64 (cap below, bt_workspace_region). */
typedef struct {
  int32_t vocab, d_model, n_heads, d_mlp;
  int32_t n_block_layers, n_token_layers;
  int32_t block_len;  /* L_B: tokens per block                              */
  int32_t prefix_len; /* P: prefix vectors projected from a context vector  */
  int32_t max_batch, max_tokens;
  int32_t dtype;      /* bt_dtype                                           */
  int32_t pad_id;     /* token used to left-pad prompts to whole blocks     */
  float ln_eps;       /* LayerNorm epsilon (1e-5)                           */
  float rope_base;    /* rotary frequency base (10000)                      */
  int32_t max_prompt_tokens; /* longest prompt bt_prefill accepts, after left padding; sizes the
                                prefill activations (one row per prompt block and batch row).
                                0 = max_tokens.  Must be <= max_tokens when set. */
  int32_t n_kv_heads; /* key/value heads of every attention layer (block and token decoder).
                         0 = n_heads.  With H_kv < n_heads, query heads are grouped in runs of
                         G = n_heads / H_kv consecutive heads and head i attends with key/value
                         head i / G (grouped-query attention; summary page §3.4 "The Block
                         Decoder" names it as compatible); the KV caches then hold H_kv heads. */
  int32_t context_mode; /* bt_context_mode (0 = prefix) */
  int32_t kv_pages;     /* 0: every row owns a block-KV cache of the full capacity.  > 0: paged
                           block KV (the PagedAttention idea): a pool of kv_pages pages of 64
                           entries (all block layers), given to rows as their caches grow, so
                           rows of different lengths share the pool.  Running out of pages is
                           BT_ERR_CAPACITY, reported before any work is queued. */
} bt_config;

/* Size in bytes of the canonical weights blob for this config.  The blob is
 * the concatenation, without padding, of these tensors in this order, each
 * row-major, elements of the config's dtype (bf16 or fp32):
 *   emb_block [V, D/L_B]
 *   per block layer l: ln1.g [D], ln1.b [D], attn.qkv.w [D, Q] (columns: q | k | v,
 *     head-major inside each; Q = D + 2 H_kv d_head, = 3D for multi-head attention),
 *     attn.qkv.b [Q], attn.out.w [D, D], attn.out.b [D],
 *     ln2.g [D], ln2.b [D], mlp.up.w [D, F], mlp.up.b [F], mlp.down.w [F, D], mlp.down.b [D]
 *   blk.lnf.g [D], blk.lnf.b [D]
 *   prefix.w [D, C*D], prefix.b [C*D]     (context projection; C = L_B for BT_CTX_SUM, else P)
 *   emb_token [V, D]
 *   per token layer: same twelve tensors as a block layer; with BT_CTX_XATTN followed by
 *     xattn.q.w [D, D], xattn.q.b [D], xattn.kv.w [D, 2 H_kv d_head] (columns: k | v),
 *     xattn.kv.b [2 H_kv d_head], xattn.out.w [D, D], xattn.out.b [D]
 *   tok.lnf.g [D], tok.lnf.b [D]
 *   head.w [V, D]                      (output classifier, no bias)
 * With n_token_layers = 0 the blob ends blk.lnf.g, blk.lnf.b, head.w (no prefix, token table,
 * token layers or tok.lnf).
 * Linear maps are y = x W + b with W stored [in, out].  Returns 0 for an
 * invalid config (see bt_last_error). */
size_t bt_weights_bytes(const bt_config* cfg);

/* Size in bytes of the device workspace bt_init needs: repacked weights,
 * rotary table, block-KV and local-KV caches, activations and step state.
 * Returns 0 for an invalid config. */
size_t bt_workspace_bytes(const bt_config* cfg);

/* Repack the canonical weights blob (device pointer, bt_weights_bytes long)
 * into the workspace (device pointer, ws_bytes >= bt_workspace_bytes, 256-byte
 * aligned) and create a handle bound to hip_stream (a hipStream_t; NULL = the
 * default stream).  Once the stream has synchronised, the caller may free the
 * weights blob; the workspace must outlive the handle.  BT_BF16: bt_init
 * synchronises the stream to check the converted weight matrices and returns
 * BT_ERR_UNSUPPORTED (no handle; bt_last_error names the tensor) if one holds a
 * magnitude >= 256 or a non-finite value, which the fp16 operands cannot hold. */
int bt_init(const bt_config* cfg, const void* d_weights, void* d_workspace, size_t ws_bytes,
            void* hip_stream, bt_handle** out);

/* Prefill (summary page §3.4 "The Inference Cost Model", prefill stage):
 * d_prompt is a device int32 [B, T] row-major array of token ids in [0, vocab);
 * every row has T tokens.  Rows are left padded with pad_id to T' = the next
 * multiple of L_B (at least L_B).  Runs the embedder and the block decoder over
 * all T'/L_B prompt blocks (filling the block-KV cache), then the token decoder
 * over the P prefix slots of the last context embedding (resetting the local
 * KV), and writes the first generated token of every row to d_next (device
 * int32 [B]).  If d_logits is not NULL, the fp32 logits [B, V] of that token
 * are written there too.  Requires 1 <= B <= max_batch, T >= 1, T' + 1 <= max_tokens and
 * T' <= max_prompt_tokens when that is set (else BT_ERR_CAPACITY). */
int bt_prefill(bt_handle* h, const int32_t* d_prompt, int32_t B, int32_t T, int32_t* d_next,
               float* d_logits);

/* Prefill with a prompt length per row (summary page §3.4 "The Embedder": sequences are left
 * padded so that every row is whole blocks).  Row b of d_prompt (device int32 [B, T]) holds its
 * lengths[b] tokens in columns [0, lengths[b]); the rest of the row is ignored.  Every row is left
 * padded with pad_id to the same T' as bt_prefill computes from T, so a row of length len gets
 * T' - len pad tokens; the result equals bt_prefill on that host-padded prompt.  d_lengths: device
 * int32 [B]; values outside [1, T] are clamped to it (they are not read on the host).  Other
 * arguments, capacities and errors as bt_prefill. */
int bt_prefill_lengths(bt_handle* h, const int32_t* d_prompt, const int32_t* d_lengths, int32_t B, int32_t T,
                       int32_t* d_next, float* d_logits);

/* Prefill in which every row is padded only to its own whole number of blocks (summary page §3.4
 * "The Embedder": left padding to a multiple of L_B): row b (device int32 [B, T], its lengths[b]
 * tokens in columns [0, lengths[b])) gets ceil(len_b / L_B) blocks, so rows keep block-KV lengths of
 * their own and each row's result equals a prefill of that row alone.  The activations are sized
 * for ceil(T / L_B) blocks per row (shorter rows leave the rest unused).  d_lengths: device int32
 * [B], clamped to [1, T].  Other arguments, capacities and errors as bt_prefill. */
int bt_prefill_ragged(bt_handle* h, const int32_t* d_prompt, const int32_t* d_lengths, int32_t B, int32_t T,
                      int32_t* d_next, float* d_logits);

/* Continuous batching: new sequences take over rows of the running batch while the other rows keep
 * decoding.  Rows rows[0..B_new) (host int32, distinct, each in [0, B) of the running batch) are
 * prefilled with the prompts of d_prompt / d_lengths exactly as bt_prefill_ragged would (each row
 * padded to its own whole blocks, block-KV length of its own); their first token goes to d_next
 * (device int32 [B_new]) and, if d_logits is not NULL, its logits to d_logits (fp32 [B_new, V]).
 * The other rows are untouched, and the next bt_decode_step advances every row by one token.
 * Rows join where a block starts, that is right after a call that emitted the first token of a
 * block (bt_prefill, or a decode step at in-block offset 0; any step when L_B = 1), so that every
 * row is at the same in-block offset: else BT_ERR_STATE.  BT_CTX_PREFIX only
 * (BT_ERR_UNSUPPORTED otherwise).  Capacities as bt_prefill for the new prompts; every row's
 * tokens stay bounded by max_tokens (bt_decode_step returns BT_ERR_CAPACITY before any row would
 * exceed it). */
int bt_prefill_rows(bt_handle* h, const int32_t* rows, int32_t B_new, const int32_t* d_prompt,
                    const int32_t* d_lengths, int32_t T, int32_t* d_next, float* d_logits);

/* Block-KV entries of each row of the running batch (host int32 [B]); synchronises the stream. */
int bt_block_lengths(bt_handle* h, int32_t* lengths);

/* Paged block KV: the page table, host int32 [max_batch][cap / 64] (page of each row's entries
 * 64 i .. 64 i + 63; entries past a row's length are unspecified).  BT_ERR_UNSUPPORTED without
 * kv_pages. */
int bt_page_table(bt_handle* h, int32_t* table);

/* One decode step (summary page §3.4, decode stage): feeds back the token the
 * previous call emitted and writes the next token of every row to d_next
 * (device int32 [B]; B is the prefill's batch), plus its fp32 logits [B, V] if
 * d_logits is not NULL.  When the previous L_B emitted tokens complete a block,
 * the step first embeds that block, runs one block-decoder position against
 * the block-KV cache, projects a new prefix and resets the local KV; otherwise
 * it runs one token-decoder position against the local KV.  BT_ERR_STATE
 * before a successful prefill; BT_ERR_CAPACITY once T' + generated tokens
 * would exceed max_tokens. */
int bt_decode_step(bt_handle* h, int32_t* d_next, float* d_logits);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): bt_decode_step with the same arguments, results and errors, bit for
 * bit, that allocates nothing and captures no graph of its own.  Its kernels are launched
 * individually on the handle's stream (so the caller may capture them), and the step's partial
 * results (split-K products, split-KV partials, the classifier's partial maxima) live in a static
 * device array of the library (64 MiB per GPU, held from the first bt_init on that GPU until the
 * process ends) instead of the workspace.  The handle's GPU must be the current device.  A batch
 * whose partial results exceed the array is refused with BT_ERR_CAPACITY before anything is
 * queued (the d = 768, V = 50304 model needs 9.2 MiB at batch 64 and 36.7 MiB at batch 256);
 * paged block KV is BT_ERR_UNSUPPORTED.  Every call on one GPU shares the array, which keeps the
 * last call's contents: calls that overlap on one GPU (other handles, other streams) race. */
int bt_decode_step_static(bt_handle* h, int32_t* d_next, float* d_logits);

/* Decode steps are replayed from HIP graphs captured on first use (one per position inside a
 * block; recaptured when the batch size changes) unless logits are requested or the stream is the
 * NULL stream.  enable = 0 launches every kernel individually instead (same results, bit for bit).
 * Default: enabled. */
int bt_set_graphs(bt_handle* h, int32_t enable);

/* Host mirror of the cache lengths after the last call: block-KV entries per
 * block-decoder layer (the largest over the rows after a ragged prefill or a join; see
 * bt_block_lengths) and local-KV entries per token-decoder layer. */
int bt_cache_lengths(const bt_handle* h, int32_t* block_kv_len, int32_t* local_kv_len);

/* Read-only introspection of the workspace layout, for tests and tools.
 * which = 0: block-KV cache [N_blk][2 (K, V)][max_batch][H_kv][cap * d_head] with
 *            cap = ceil(max_tokens / L_B) rounded up to a multiple of 64; per (layer,
 *            row, KV head) the keys are [cap][d_head] (after the rotary embedding) and the
 *            values are in groups of 8 entries, each group transposed: [cap / 8][d_head][8];
 *            with kv_pages > 0 the cache is a pool [N_blk][2][kv_pages][H_kv][64 * d_head]
 *            (keys [64][d_head], values [8][d_head][8] per page and head; capacity = 64), and
 *            entry j of row b is in page bt_page_table(h)[b][j / 64] at j % 64;
 * which = 1: local-KV cache [N_tok][2][max_batch][H_kv][S + L_B][d_head] (keys after
 *            the rotary embedding, values not transposed).
 * Elements are fp16 for BT_BF16 and fp32 for BT_FP32.  Writes the byte
 * offset from the workspace start, the byte size and the per-head capacity.  H_kv is
 * n_kv_heads, or n_heads when that is 0; S is P for BT_CTX_PREFIX, else 1 (the start slot). */
int bt_workspace_region(const bt_config* cfg, int32_t which, size_t* offset, size_t* bytes,
                        int32_t* capacity);

/* Range of the fp16 values of a BT_BF16 handle (for BT_FP32 both entries stay 0).
 * status[0]: weight elements bt_init rounded when converting them to fp16 (magnitudes below
 *            2^-25 that are not multiples of 2^-32; the rounding error is at most 2^-33 each);
 * status[1]: 1 if an activation or cache value was beyond fp16's range or not finite, and was
 *            clamped to +-65504, since the flag was last cleared; else 0.  The flag is kept per
 *            device and process and is shared by every handle on the device.
 * reset != 0 clears the flag after reading it.  Synchronises the handle's stream. */
int bt_numerics_status(bt_handle* h, int32_t reset, int64_t* status);

/* Free the host handle (no device memory is owned). */
int bt_destroy(bt_handle* h);

/* Message of the last failure on this thread ("" if none). */
const char* bt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BT_H_ */
