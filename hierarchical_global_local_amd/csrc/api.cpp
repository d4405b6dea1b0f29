// Host orchestrator and C-ABI of libbt: config validation, workspace layout, weight repack,
// and the per-call launch schedules of prefill and decode.
//
// The schedules follow "Block Transformer: Global-to-Local Language Modeling for Fast Inference"
// (summary page, §3.2 and §3.4): prefill embeds all prompt blocks and runs the block decoder over
// them (writing the block-KV cache), then runs the token decoder over the P prefix slots only;
// each decode step either runs one token-decoder position against the local KV, or — when the
// previous L_B tokens complete a block — embeds that block, runs one block-decoder position
// against the block-KV cache and restarts the token decoder from a fresh prefix.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "bt.h"
#include "bt_internal.h"
#include "bt_test.h"

namespace {
thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
}  // namespace

namespace bt {

std::string plan_layout(const bt_config& c, Layout& lo) {
  if (c.dtype != BT_FP32 && c.dtype != BT_BF16) return "dtype must be BT_FP32 or BT_BF16";
  if (c.vocab < 1 || c.d_model < 1 || c.n_heads < 1 || c.d_mlp < 1) return "vocab, d_model, n_heads, d_mlp must be >= 1";
  if (c.d_model % c.n_heads) return "d_model must be a multiple of n_heads";
  const int dh = c.d_model / c.n_heads;
  const bool f32 = c.dtype == BT_FP32;
  if (!(dh == 64 || dh == 128 || (f32 && dh == 32)))
    return f32 ? "d_head must be 32, 64 or 128" : "d_head must be 64 or 128 for BT_BF16";
  if (c.block_len < 1 || c.prefix_len < 1) return "block_len and prefix_len must be >= 1";
  if (c.d_model % c.block_len) return "d_model must be a multiple of block_len";
  if (c.prefix_len + c.block_len > 32) return "prefix_len + block_len must be <= 32";
  if (c.n_block_layers < 1 || c.n_token_layers < 0) return "n_block_layers must be >= 1, n_token_layers >= 0";
  if (c.n_token_layers == 0 && c.block_len != 1)
    return "n_token_layers = 0 (token-level transformer) needs block_len = 1";
  if (c.d_model > 4096) return "d_model must be <= 4096";
  if (!f32 && (c.d_model % 64 || c.d_mlp % 64)) return "BT_BF16 needs d_model and d_mlp multiples of 64";
  if (c.max_batch < 1 || c.max_batch > (1 << 20)) return "max_batch must be in [1, 1048576]";
  if (c.max_tokens < c.block_len + 1) return "max_tokens must be > block_len";
  if (!(c.ln_eps > 0.f) || !(c.rope_base > 0.f)) return "ln_eps and rope_base must be > 0";
  const int nblk = (c.max_tokens + c.block_len - 1) / c.block_len;
  if (nblk > 131072) return "max_tokens / block_len must be <= 131072";
  if (c.max_prompt_tokens < 0 || c.max_prompt_tokens > c.max_tokens)
    return "max_prompt_tokens must be in [0, max_tokens]";
  if (c.n_kv_heads < 0 || c.n_kv_heads > c.n_heads || (c.n_kv_heads > 0 && c.n_heads % c.n_kv_heads))
    return "n_kv_heads must be 0 or a divisor of n_heads";
  if (c.pad_id < 0 || c.pad_id >= c.vocab) return "pad_id must be in [0, vocab)";
  if (c.kv_pages < 0 || (int64_t)c.kv_pages > (int64_t)c.max_batch * ((nblk + 63) / 64))
    return "kv_pages must be in [0, max_batch * cap / 64]";
  if (c.context_mode < BT_CTX_PREFIX || c.context_mode > BT_CTX_XATTN)
    return "context_mode must be BT_CTX_PREFIX, BT_CTX_SUM or BT_CTX_XATTN";
  if (c.n_token_layers == 0 && c.context_mode != BT_CTX_PREFIX)
    return "context_mode needs a token decoder (n_token_layers >= 1)";
  const int max_prompt = c.max_prompt_tokens > 0 ? c.max_prompt_tokens : c.max_tokens;
  const int nblk_prompt = std::max(1, (max_prompt + c.block_len - 1) / c.block_len);

  lo.V = c.vocab;
  lo.D = c.d_model;
  lo.H = c.n_heads;
  lo.Hkv = c.n_kv_heads > 0 ? c.n_kv_heads : c.n_heads;
  lo.dh = dh;
  lo.QW = lo.D + 2 * lo.Hkv * dh;
  lo.F = c.d_mlp;
  lo.L = c.block_len;
  lo.P = c.prefix_len;
  lo.mode = c.context_mode;
  lo.lead = lo.mode == BT_CTX_PREFIX ? lo.P : 1;
  lo.NC = lo.mode == BT_CTX_SUM ? lo.L : lo.P;
  lo.Nb = c.n_block_layers;
  lo.Nt = c.n_token_layers;
  lo.De = c.d_model / c.block_len;
  lo.Bmax = c.max_batch;
  lo.max_tokens = c.max_tokens;
  lo.f32 = f32;
  lo.vanilla = c.n_token_layers == 0;
  lo.elem = f32 ? 4 : 2;
  lo.tab_elem = f32 ? 4 : 2;
  lo.ncap = (int)align_up((size_t)nblk, 64);
  lo.lcap = lo.lead + lo.L;
  lo.npos = std::max(lo.ncap, lo.lcap);
  lo.Vpad = (int)align_up((size_t)lo.V, 128);
  lo.max_prompt = nblk_prompt * lo.L;  // prompts up to this padded length fit the activations
  lo.Mmax = std::max<int64_t>((int64_t)lo.Bmax * nblk_prompt, (int64_t)lo.Bmax * lo.P);
  lo.Mpad = (int64_t)align_up((size_t)lo.Mmax, 16);

  const size_t D = lo.D, F = lo.F, V = lo.V, P = lo.P, E = lo.elem, TE = lo.tab_elem, QW = lo.QW;
  // ---- canonical blob
  size_t o = 0;
  auto take = [&](size_t n) { size_t r = o; o += n * TE; return r; };
  lo.bl_emb_block = take(V * lo.De);
  const bool xattn = lo.mode == BT_CTX_XATTN;
  const size_t KVW = (size_t)lo.Hkv * dh, NC = lo.NC;
  auto blob_layer = [&](bool with_xattn) {
    Layout::BlobLayer b;
    b.ln1g = take(D); b.ln1b = take(D); b.qkvw = take(D * QW); b.qkvb = take(QW);
    b.outw = take(D * D); b.outb = take(D); b.ln2g = take(D); b.ln2b = take(D);
    b.upw = take(D * F); b.upb = take(F); b.downw = take(F * D); b.downb = take(D);
    if (with_xattn) {
      b.xqw = take(D * D); b.xqb = take(D); b.xkvw = take(D * 2 * KVW); b.xkvb = take(2 * KVW);
      b.xow = take(D * D); b.xob = take(D);
    }
    return b;
  };
  lo.bl_blk.clear();
  lo.bl_tok.clear();
  for (int l = 0; l < lo.Nb; ++l) lo.bl_blk.push_back(blob_layer(false));
  lo.bl_lnf_blk_g = take(D);
  lo.bl_lnf_blk_b = take(D);
  if (!lo.vanilla) {  // a token-level transformer has no prefix projection and no token decoder
    lo.bl_prefix_w = take(D * NC * D);
    lo.bl_prefix_b = take(NC * D);
    lo.bl_emb_tok = take(V * D);
    for (int l = 0; l < lo.Nt; ++l) lo.bl_tok.push_back(blob_layer(xattn));
    lo.bl_lnf_tok_g = take(D);
    lo.bl_lnf_tok_b = take(D);
  }
  lo.bl_head = take(V * D);
  lo.bl_total = o;

  // ---- workspace
  size_t w = 0;
  auto region = [&](size_t bytes) { size_t r = w; w = align_up(w + bytes, 256); return r; };
  const size_t tokw = lo.vanilla ? 0 : 1;  // token-decoder side present
  lo.emb_block = region(V * lo.De * TE);
  lo.emb_tok = region(tokw * V * D * TE);
  lo.head = region((size_t)lo.Vpad * D * E);
  lo.lnf_blk = region(2 * D * 4);
  lo.lnf_tok = region(tokw * 2 * D * 4);
  lo.prefix_w = region(tokw * NC * D * D * E);
  lo.prefix_b = region(tokw * NC * D * 4);
  lo.rope = region((size_t)lo.npos * (lo.dh / 2) * sizeof(float2));
  auto layer = [&](bool with_xattn) {
    LayerOff L;
    L.n1 = (int)(QW + (with_xattn ? D : 0));
    L.k2 = (int)(D + F + (with_xattn ? D : 0));
    L.ln = region(4 * D * 4);
    L.w1 = region((L.n1 + F) * D * E);
    L.b1 = region((L.n1 + F) * 4);
    L.w2 = region(D * L.k2 * E);
    L.b2 = region(3 * D * 4);
    return L;
  };
  lo.blk.clear();
  lo.tok.clear();
  for (int l = 0; l < lo.Nb; ++l) lo.blk.push_back(layer(false));
  for (int l = 0; l < lo.Nt; ++l) lo.tok.push_back(layer(xattn));
  lo.maxN1 = (int)QW + (xattn ? lo.D : 0);
  lo.maxK2 = lo.D + lo.F + (xattn ? lo.D : 0);
  lo.pages = c.kv_pages;
  // flat: per layer and K/V, [Bmax][Hkv][ncap][dh]; paged: [pages][Hkv][64][dh] (the same bytes per entry)
  lo.block_kv_bytes = (size_t)lo.Nb * 2 * (lo.pages ? (size_t)lo.pages * 64 : (size_t)lo.Bmax * lo.ncap) * lo.Hkv *
                      lo.dh * E;
  lo.local_kv_bytes = (size_t)lo.Nt * 2 * lo.Bmax * lo.Hkv * lo.lcap * lo.dh * E;  // 0 for Nt = 0
  lo.block_kv = region(lo.block_kv_bytes);
  lo.local_kv = region(lo.local_kv_bytes);
  const size_t M = (size_t)lo.Mmax;
  lo.X = region(M * D * 4);
  lo.LN = region(2 * (size_t)lo.Mpad * D * E);
  lo.QKV = region(M * lo.maxN1 * E);
  lo.ACT = region((size_t)lo.Mpad * lo.maxK2 * E);
  // split-KV partials [B][H][nsplit][dh + 2] for the largest B * nsplit any batch size uses
  lo.part_bytes = 0;
  for (int b = 1; b <= lo.Bmax; ++b) {
    const int ns = decode_splits(b, lo.H, lo.Hkv, lo.ncap);
    if (ns > 1) lo.part_bytes = std::max(lo.part_bytes, (size_t)b * lo.H * ns * (lo.dh + 2) * 4);
  }
  lo.part = region(lo.part_bytes);
  lo.keys = region((size_t)lo.Bmax * (lo.Vpad / 4 + 64) * 8);
  const bool start_slot = !lo.vanilla && lo.mode != BT_CTX_PREFIX;
  const size_t encr = xattn ? (size_t)lo.Bmax * P : 0;  // encoder-state rows
  lo.xkv_ld = xattn ? (int)(lo.Nt * 2 * KVW) : 0;
  lo.pad_emb = region(start_slot ? D * 4 : 0);
  lo.ctx = region(lo.mode == BT_CTX_SUM ? (size_t)lo.Bmax * lo.L * D * 4 : 0);
  lo.enc = region(encr * D * 4);
  lo.enc16 = region(f32 ? 0 : align_up(encr, 16) * D * E);
  lo.xkv_w = region((size_t)lo.xkv_ld * D * E);
  lo.xkv_b = region((size_t)lo.xkv_ld * 4);
  lo.xkv = region(encr * lo.xkv_ld * 4);
  lo.rpart_rows = (int)std::min<int64_t>(lo.Mmax, 1024);
  lo.rpart = region((size_t)16 * lo.rpart_rows * D * 4);
  lo.cur = region((size_t)lo.Bmax * lo.L * 4);
  lo.dstate = region(std::max<size_t>(64, (size_t)lo.Bmax * 4));
  lo.rowmap = region((size_t)lo.Bmax * 4);
  lo.ptab = region(lo.pages ? (size_t)lo.Bmax * (lo.ncap / 64) * 4 : 0);
  lo.lastblk = region((size_t)lo.Bmax * 4);
  lo.wflags = region(2 * 4);
  lo.total = w;
  return "";
}

}  // namespace bt

using namespace bt;

struct bt_handle {
  bt_config cfg;
  Layout lo;
  char* ws = nullptr;
  hipStream_t st = nullptr;
  int B = 0, Tp = 0;
  int n_blocks = 0;   // block-KV entries per layer (the largest over the rows)
  int local_len = 0;  // local-KV entries per layer
  int g = 0;          // tokens emitted since the prefill
  std::vector<int64_t> row_tok;  // per row: padded prompt + emitted tokens, an upper bound
  const int* rmap = nullptr;     // during a join: device cache row of each prefilled row
  // paged block KV: the host allocates pages (a row's entries are known here exactly)
  std::vector<int> free_pages;              // stack of free page ids
  std::vector<std::vector<int>> row_pages;  // pages of each row, in entry order
  std::vector<int> row_n;                   // block-KV entries of each row
  int32_t* ptab_host = nullptr;             // pinned mirror of the page table [Bmax][ncap / 64]
  hipEvent_t ptab_ev = nullptr;             // completion of its last upload
  bool ready = false, broken = false;
  // optional per-kernel-class event timing
  bool prof = false;
  std::vector<hipEvent_t> ev_pool;
  struct Rec { int kind, ev; double bytes, flops; };
  std::vector<Rec> ev_used;
  size_t ev_next = 0;
  bool decode_phase = false;  // classes are split by phase: prefill, decode
  ResidPending pending{};     // split-K residual update not yet folded into X (nsplit = 0: none)
  int head_nparts = 0;        // column groups of the last classifier launch
  int dec_nsplit = 1;         // key splits of block-attention decode for this batch size
  int64_t weights_rounded = 0;  // weight elements bt_init could not convert to fp16 exactly
  // bt_decode_step_static: the step's partial results (split-K, split-KV, argmax keys) in the
  // library's static scratch instead of the workspace (null: the workspace regions)
  char* scr_rpart = nullptr;
  char* scr_part = nullptr;
  char* scr_keys = nullptr;
  size_t scr_part_bytes = 0;
  // decode steps replayed from HIP graphs, one per in-block offset j (0 = block step)
  bool use_graphs = true;
  // decode steps run the token decoder's local attention inside its [out|down] GEMM where the
  // shape allows (attn_out_splits); off: separate launches (test hook)
  bool fuse_local = true;
  int graph_B = -1;
  std::vector<hipGraphExec_t> graphs;
};

namespace {

enum ProfKind { PK_EMBED = 0, PK_LN, PK_GEMM_QKV, PK_GEMM_OUT, PK_GEMM_PREFIX, PK_GEMM_HEAD, PK_ATTN_PREFILL,
                PK_ROPE_SCATTER, PK_ATTN_DECODE, PK_ATTN_LOCAL, PK_FINALIZE, PK_ATTN_CROSS, PK_LOCAL_OUT, PK_COUNT };
static_assert(PK_COUNT == BT_PROFILE_KINDS, "profiler classes");

// Records a pair of events around one launch with its algorithmic bytes and flops (the minimal
// traffic and arithmetic of the operation, independent of how the kernel achieves it).
struct Prof {
  bt_handle* h;
  int kind;
  double bytes, flops;
  int idx = -1;
  Prof(bt_handle* h_, int k, double by = 0.0, double fl = 0.0)
      : h(h_), kind(k + (h_->decode_phase ? PK_COUNT : 0)), bytes(by), flops(fl) {
    if (!h->prof) return;
    if (h->ev_next + 2 > h->ev_pool.size()) {
      for (int i = 0; i < 256; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        h->ev_pool.push_back(e);
      }
    }
    idx = (int)h->ev_next;
    h->ev_next += 2;
    (void)hipEventRecord(h->ev_pool[idx], h->st);
  }
  ~Prof() {
    if (idx < 0) return;
    (void)hipEventRecord(h->ev_pool[idx + 1], h->st);
    h->ev_used.push_back({kind, idx, bytes, flops});
  }
};

inline char* P_(bt_handle* h, size_t off) { return h->ws + off; }

// Partial-result buffers of the current call: the workspace's, or the static scratch's during
// bt_decode_step_static.
float* rpart_buf(bt_handle* h) { return h->scr_rpart ? (float*)h->scr_rpart : (float*)P_(h, h->lo.rpart); }
float* part_buf(bt_handle* h) { return h->scr_part ? (float*)h->scr_part : (float*)P_(h, h->lo.part); }
size_t part_cap(bt_handle* h) { return h->scr_keys ? h->scr_part_bytes : h->lo.part_bytes; }
unsigned long long* keys_buf(bt_handle* h) {
  return (unsigned long long*)(h->scr_keys ? h->scr_keys : P_(h, h->lo.keys));
}
int keys_ld(const Layout& lo) { return lo.Vpad / 4 + 64; }

int hip_fail(bt_handle* h, hipError_t e, const char* what) {
  if (h) h->broken = true;
  return fail(BT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define BT_CHECK(h, expr, what)                    \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hip_fail(h, e_, what); \
  } while (0)

// bytes of one layer's keys (or values) in the block-KV region
size_t block_kv_per(const Layout& lo) {
  return (lo.pages ? (size_t)lo.pages * 64 : (size_t)lo.Bmax * lo.ncap) * lo.Hkv * lo.dh * lo.elem;
}
void* block_k(bt_handle* h, int l) { return P_(h, h->lo.block_kv + (size_t)(2 * l) * block_kv_per(h->lo)); }
void* block_v(bt_handle* h, int l) { return P_(h, h->lo.block_kv + (size_t)(2 * l + 1) * block_kv_per(h->lo)); }
void* local_k(bt_handle* h, int l) {
  const Layout& lo = h->lo;
  size_t per = (size_t)lo.Bmax * lo.Hkv * lo.lcap * lo.dh * lo.elem;
  return P_(h, lo.local_kv + (size_t)(2 * l) * per);
}
void* local_v(bt_handle* h, int l) {
  const Layout& lo = h->lo;
  size_t per = (size_t)lo.Bmax * lo.Hkv * lo.lcap * lo.dh * lo.elem;
  return P_(h, lo.local_kv + (size_t)(2 * l + 1) * per);
}
void* ln_buf(bt_handle* h, int which) {
  const Layout& lo = h->lo;
  return P_(h, lo.LN + (size_t)which * lo.Mpad * lo.D * lo.elem);
}

float wscale(const Layout& lo) { return lo.f32 ? 1.0f : kWeightUnscale; }

const ResidPending* pending(bt_handle* h) { return h->pending.nsplit > 0 ? &h->pending : nullptr; }

// ---- paged block KV
const int* page_table(bt_handle* h) { return h->lo.pages ? (const int*)P_(h, h->lo.ptab) : nullptr; }
// per-row entry counts (the device lengths) bound what a paged prefill writes and reads
const int* page_limits(bt_handle* h) { return h->lo.pages ? (const int*)P_(h, h->lo.dstate) : nullptr; }

// Waits until the previous upload of the pinned mirror has been consumed, so it may change.
int pages_wait(bt_handle* h) {
  BT_CHECK(h, hipEventSynchronize(h->ptab_ev), "page table");
  return BT_OK;
}
int pages_upload(bt_handle* h) {
  const Layout& lo = h->lo;
  BT_CHECK(h, hipMemcpyAsync(P_(h, lo.ptab), h->ptab_host, (size_t)lo.Bmax * (lo.ncap / 64) * 4,
                             hipMemcpyHostToDevice, h->st),
           "page table");
  BT_CHECK(h, hipEventRecord(h->ptab_ev, h->st), "page table");
  return BT_OK;
}
// Gives rows[i] pages for entries [0, entries[i]), releasing what they held first; nothing changes
// (BT_ERR_CAPACITY) if the pool is short.  Uploads the table.
int pages_assign(bt_handle* h, const std::vector<int>& rows, const std::vector<int>& entries) {
  const Layout& lo = h->lo;
  size_t held = 0, want = 0;
  for (size_t i = 0; i < rows.size(); ++i) {
    held += h->row_pages[rows[i]].size();
    want += (size_t)(entries[i] + 63) / 64;
  }
  if (h->free_pages.size() + held < want) return fail(BT_ERR_CAPACITY, "kv_pages exhausted");
  int r = pages_wait(h);
  if (r) return r;
  for (int row : rows) {
    for (int pg : h->row_pages[row]) h->free_pages.push_back(pg);
    h->row_pages[row].clear();
  }
  const int pld = lo.ncap / 64;
  for (size_t i = 0; i < rows.size(); ++i) {
    auto& mine = h->row_pages[rows[i]];
    for (int k = 0; k < (entries[i] + 63) / 64; ++k) {
      mine.push_back(h->free_pages.back());
      h->free_pages.pop_back();
      h->ptab_host[(size_t)rows[i] * pld + k] = mine.back();
    }
    h->row_n[rows[i]] = entries[i];
  }
  return pages_upload(h);
}
// Before a block step: a page for every row whose append slot starts one.
int pages_grow(bt_handle* h) {
  const Layout& lo = h->lo;
  size_t need = 0;
  for (int b = 0; b < h->B; ++b) need += h->row_n[b] % 64 == 0;
  if (!need) return BT_OK;
  if (h->free_pages.size() < need) return fail(BT_ERR_CAPACITY, "kv_pages exhausted");
  int r = pages_wait(h);
  if (r) return r;
  const int pld = lo.ncap / 64;
  for (int b = 0; b < h->B; ++b)
    if (h->row_n[b] % 64 == 0) {
      h->row_pages[b].push_back(h->free_pages.back());
      h->free_pages.pop_back();
      h->ptab_host[(size_t)b * pld + h->row_n[b] / 64] = h->row_pages[b].back();
    }
  return pages_upload(h);
}
// Exact entries of each row after a ragged prefill of B rows (reads the lengths back).
int ragged_entries(bt_handle* h, const int32_t* d_lengths, int B, int T, std::vector<int>& out) {
  std::vector<int32_t> len(B);
  BT_CHECK(h, hipMemcpyAsync(len.data(), d_lengths, (size_t)B * 4, hipMemcpyDeviceToHost, h->st), "lengths");
  BT_CHECK(h, hipStreamSynchronize(h->st), "lengths");
  out.resize(B);
  for (int b = 0; b < B; ++b) out[b] = (std::min(std::max(len[b], 1), T) + h->lo.L - 1) / h->lo.L;
  return BT_OK;
}

// Epilogue of the [q|k|v|up] GEMM: bias, q|k|v to the QKV buffer, GELU(up) to ACT.
Epi qkv_epi(bt_handle* h, const LayerOff& w) {
  const Layout& lo = h->lo;
  Epi ep{};
  ep.wscale = wscale(lo);
  ep.bias = (const float*)P_(h, w.b1);
  ep.out0 = P_(h, lo.QKV);
  ep.ld0 = w.n1;
  ep.out1 = P_(h, lo.ACT);
  ep.ld1 = w.k2;
  ep.n_split = w.n1;
  ep.act_col0 = lo.D;
  return ep;
}

// LN1/LN2 -> [q|k|v|up] GEMM with bias (+GELU on the up part).  With ln_done the LayerNorm
// outputs were already written (by the previous step's finalisation).
int run_ln_qkv(bt_handle* h, const LayerOff& w, int rows, bool ln_done = false) {
  const Layout& lo = h->lo;
  const float* lnp = (const float*)P_(h, w.ln);
  const double E = (double)lo.elem, D = lo.D, N1 = (double)w.n1 + lo.F;
  if (!ln_done) {
    Prof p(h, PK_LN, rows * D * (4.0 + 2.0 * E), 8.0 * rows * D);
    BT_CHECK(h, launch_layernorm((float*)P_(h, lo.X), rows, lo.D, 1, 0, lnp, ln_buf(h, 0), lnp + 2 * lo.D,
                                 ln_buf(h, 1), lo.f32, h->cfg.ln_eps, pending(h), h->st),
             "layernorm");
    h->pending.nsplit = 0;
  }
  const Epi ep = qkv_epi(h, w);
  Prof p(h, PK_GEMM_QKV, N1 * D * E + 2.0 * rows * D * E + rows * N1 * E + N1 * 4.0, 2.0 * rows * N1 * D);
  BT_CHECK(h, launch_gemm(lo.f32, ln_buf(h, 0), ln_buf(h, 1), lo.D, P_(h, w.w1), rows, w.n1 + lo.F, lo.D,
                          EPI_QKV_GELU, ep, h->st),
           "gemm qkv|up");
  return BT_OK;
}

// Epilogue of the [out|down] GEMM with `splits` K splits; with more than one the partial products
// are summed (with both biases) by the next LayerNorm.
Epi resid_epi(bt_handle* h, const LayerOff& w, int rows, int splits) {
  const Layout& lo = h->lo;
  Epi ep{};
  ep.wscale = wscale(lo);
  ep.bias = (const float*)P_(h, w.b2);
  ep.bias2 = (const float*)P_(h, w.b2) + lo.D;
  ep.out0 = P_(h, lo.X);
  ep.ld0 = lo.D;
  ep.splits = splits;
  ep.part = rpart_buf(h);
  if (ep.splits > 1) {
    h->pending.part = ep.part;
    h->pending.nsplit = ep.splits;
    h->pending.part_rows = rows;
    h->pending.bias_a = ep.bias;
    h->pending.bias_b = ep.bias2;
  }
  return ep;
}

// [attn | gelu(up) (| cross-attention)] x [W_o ; W_down (; W_xo)] + biases added into the residual stream
int run_out(bt_handle* h, const LayerOff& w, int rows) {
  const Layout& lo = h->lo;
  const Epi ep = resid_epi(h, w, rows, rows <= lo.rpart_rows ? resid_splits(rows, lo.D, w.k2) : 1);
  const double E = (double)lo.elem, D = lo.D, K2 = w.k2;
  Prof p(h, PK_GEMM_OUT, D * K2 * E + rows * K2 * E + 8.0 * rows * D + 8.0 * D, 2.0 * rows * D * K2);
  BT_CHECK(h, launch_gemm(lo.f32, P_(h, lo.ACT), nullptr, w.k2, P_(h, w.w2), rows, lo.D, w.k2,
                          EPI_RESID, ep, h->st),
           "gemm out|down");
  return BT_OK;
}

// Partial count of the token decoder's fused local attention (and cross-attention) + [out|down]
// launch for one new slot per row (attn_out_splits over the GELU columns' K range), 0 where it runs
// as separate launches: fp32, head width other than 64, or more rows than the partial buffer or the
// fused kernel take.
int fused_local_splits(bt_handle* h, int m) {
  const Layout& lo = h->lo;
  const int rows = h->B * m;
  if (m != 1 || !h->fuse_local || lo.f32 || lo.dh != 64 || rows > lo.rpart_rows || lo.Nt == 0) return 0;
  return attn_out_splits(rows, lo.D, lo.D + lo.F, lo.H);
}

// Token layer l, one new slot s0 per row: local attention inside the [out|down] GEMM; its
// `splits` partial products are folded by the next LayerNorm.
int run_fused_local_out(bt_handle* h, int l, int s0, int splits) {
  const Layout& lo = h->lo;
  const LayerOff& w = lo.tok[l];
  const int rows = h->B;
  LocalStep ls{};
  ls.qkv = (const f16*)P_(h, lo.QKV);
  ls.ldq = w.n1;
  ls.H = lo.H;
  ls.Hkv = lo.Hkv;
  ls.s0 = s0;
  ls.rope = (const float2*)P_(h, lo.rope);
  ls.kc = (f16*)local_k(h, l);
  ls.vc = (f16*)local_v(h, l);
  ls.cap = lo.lcap;
  ls.rmap = h->rmap;
  ls.scale_log2 = 1.4426950408889634f / sqrtf((float)lo.dh);
  ls.k_mlp = lo.D + lo.F;
  if (lo.mode == BT_CTX_XATTN) {
    // the cross-attention of this layer: its query columns follow q|k|v, its encoder keys and
    // values are the layer's slice of the per-block K|V projection
    ls.xkv = (const float*)P_(h, lo.xkv);
    ls.xkv_ld = lo.xkv_ld;
    ls.xkv_off = l * 2 * lo.Hkv * lo.dh;
    ls.P = lo.P;
    ls.xq_off = (int)lo.QW;
  }
  const Epi ep = resid_epi(h, w, rows, splits);
  const double E = (double)lo.elem, D = lo.D, Bd = h->B, KVW = (double)lo.Hkv * lo.dh, F = lo.F;
  // weights, the GELU columns, q|k|v, cached K/V read and the new K/V written, the residual
  // stream read and written (fp32) and both biases
  // (cross-attention: its query columns and the P encoder keys and values, fp32, per row)
  const double xa = lo.mode == BT_CTX_XATTN ? rows * (D * E + lo.P * 2.0 * KVW * 4.0) : 0.0;
  Prof p(h, PK_LOCAL_OUT,
         D * w.k2 * E + rows * F * E + (Bd * s0 * 2.0 * KVW + rows * (D + 4.0 * KVW)) * E + 8.0 * rows * D + 8.0 * D +
             xa,
         2.0 * rows * D * w.k2 + 4.0 * Bd * lo.H * lo.dh * (s0 + 1 + (lo.mode == BT_CTX_XATTN ? lo.P : 0)));
  BT_CHECK(h, launch_attn_out_decode(P_(h, lo.ACT), P_(h, w.w2), rows, lo.D, w.k2, ep, ls, h->st),
           "local attention + out|down");
  return BT_OK;
}

// token decoder over new local slots [s0, s0 + m) of every row (rows = B * m in X)
int run_token_decoder(bt_handle* h, int m, int s0, bool first_ln_done = false) {
  const Layout& lo = h->lo;
  const int rows = h->B * m;
  const int fused_splits = fused_local_splits(h, m);
  for (int l = 0; l < lo.Nt; ++l) {
    int r = run_ln_qkv(h, lo.tok[l], rows, l == 0 && first_ln_done);
    if (r) return r;
    if (fused_splits > 0) {
      r = run_fused_local_out(h, l, s0, fused_splits);
      if (r) return r;
      continue;
    }
    {
      const double E = (double)lo.elem, D = lo.D, Bd = h->B, KVW = (double)lo.Hkv * lo.dh;
      double pairs = 0;
      for (int i = 0; i < m; ++i) pairs += s0 + i + 1;
      // cached K/V read, q|k|v read, new K/V and the output written
      Prof p(h, PK_ATTN_LOCAL, (Bd * s0 * 2.0 * KVW + 2.0 * rows * (D + 2.0 * KVW)) * E,
             4.0 * Bd * lo.H * lo.dh * pairs);
      BT_CHECK(h, launch_local_attention(lo.f32, P_(h, lo.QKV), lo.tok[l].n1, h->B, m, s0, lo.H, lo.Hkv, lo.dh,
                                         (const float2*)P_(h, lo.rope), local_k(h, l), local_v(h, l), lo.lcap,
                                         P_(h, lo.ACT), lo.tok[l].k2, h->st, h->rmap),
               "local attention");
    }
    if (lo.mode == BT_CTX_XATTN) {
      // one local slot per row (the local sequence starts with a single start slot)
      if (m != 1) return fail(BT_ERR_INVALID_ARG, "cross-attention runs one local slot per row");
      const double E = (double)lo.elem, D = lo.D, Bd = h->B, KVW = (double)lo.Hkv * lo.dh;
      Prof p(h, PK_ATTN_CROSS, Bd * (lo.P * 2.0 * KVW * 4.0 + 2.0 * D * E), 4.0 * Bd * lo.H * lo.dh * lo.P);
      BT_CHECK(h, launch_cross_attention(lo.f32, P_(h, lo.QKV), lo.tok[l].n1, lo.QW, h->B, lo.H, lo.Hkv, lo.dh,
                                         (const float*)P_(h, lo.xkv), lo.xkv_ld, l * 2 * lo.Hkv * lo.dh, lo.P,
                                         P_(h, lo.ACT), lo.tok[l].k2, lo.D + lo.F, h->st),
               "cross attention");
    }
    r = run_out(h, lo.tok[l], rows);
    if (r) return r;
  }
  return BT_OK;
}

// final LN of the token decoder at rows (b, slot) of X [B][m][D], then classifier + partial argmax
int run_head(bt_handle* h, int m, int slot, float* d_logits) {
  const Layout& lo = h->lo;
  const double E = (double)lo.elem, D = lo.D, Bd = h->B, V = lo.V;
  {
    // a token-level transformer classifies the block decoder's (token-level) output directly
    const float* lnf = (const float*)P_(h, lo.vanilla ? lo.lnf_blk : lo.lnf_tok);
    Prof p(h, PK_LN, Bd * D * (4.0 + E), 8.0 * Bd * D);
    BT_CHECK(h, launch_layernorm((float*)P_(h, lo.X), h->B, lo.D, m, slot, lnf,
                                 ln_buf(h, 0), nullptr, nullptr, lo.f32, h->cfg.ln_eps, pending(h), h->st),
             "final layernorm");
    h->pending.nsplit = 0;
  }
  Epi ep{};
  ep.wscale = wscale(lo);
  ep.out0 = d_logits;
  ep.ld0 = lo.V;
  ep.n_valid = lo.V;
  ep.keys = keys_buf(h);
  ep.keys_ld = keys_ld(lo);
  ep.nparts_out = &h->head_nparts;
  Prof p(h, PK_GEMM_HEAD, V * D * E + Bd * D * E + (d_logits ? Bd * V * 4.0 : 0.0) + Bd * 8.0, 2.0 * Bd * V * D);
  BT_CHECK(h, launch_gemm(lo.f32, ln_buf(h, 0), nullptr, lo.D, P_(h, lo.head), h->B, lo.f32 ? lo.V : lo.Vpad, lo.D,
                          EPI_ARGMAX, ep, h->st),
           "classifier");
  return BT_OK;
}

// Input of the decode step that predicts token gn: the embedding row of the id just emitted (token
// step) or of the block it completes (block step), and the first layer's LN1/LN2 of that row.
NextStepArgs next_step_args(bt_handle* h, int gn) {
  const Layout& lo = h->lo;
  NextStepArgs nx;
  const bool next_is_block = gn % lo.L == 0;
  nx.mode = next_is_block ? 2 : 1;
  nx.E = next_is_block ? P_(h, lo.emb_block) : P_(h, lo.emb_tok);
  nx.width = next_is_block ? lo.De : lo.D;
  nx.tab_bf16 = !lo.f32;
  nx.out_f32 = lo.f32;
  nx.X = (float*)P_(h, lo.X);
  nx.lnp = (const float*)P_(h, next_is_block ? lo.blk[0].ln : lo.tok[0].ln);  // (vanilla: always a block step)
  nx.ln1 = ln_buf(h, 0);
  nx.ln2 = ln_buf(h, 1);
  nx.D = lo.D;
  nx.V = lo.V;
  nx.eps = h->cfg.ln_eps;
  if (lo.mode == BT_CTX_SUM && !next_is_block) {
    // summation: that slot, gn % L, also takes its projected summand
    nx.add = (const float*)P_(h, lo.ctx) + (size_t)(gn % lo.L) * lo.D;
    nx.add_ld = lo.L * lo.D;
  }
  return nx;
}

// Greedy ids of in-block offset j into d_next and the current-block buffer; a block step also
// advances the device block-KV lengths.  The same kernel prepares the input of decode step g + 1
// (g = the index of the token just chosen), except in a join (rows prefilled into a running batch:
// their inputs are prepared afterwards, with everyone else's).
int run_finalize(bt_handle* h, int j, int32_t* d_next, int n_inc) {
  const Layout& lo = h->lo;
  NextStepArgs nx = next_step_args(h, h->g + 1);
  if (h->rmap) nx.mode = 0;
  Prof p(h, PK_FINALIZE, (double)h->B * (16.0 + lo.D * (lo.tab_elem + 4.0 + 2.0 * lo.elem)), 0.0);
  BT_CHECK(h, launch_finalize(keys_buf(h), h->head_nparts, keys_ld(lo), h->B, d_next,
                              (int32_t*)P_(h, lo.cur), lo.L, j, (int*)P_(h, lo.dstate), n_inc, nx, h->st, h->rmap),
           "finalize");
  return BT_OK;
}

// After a join: the input of the next decode step (which predicts token g) of every row, from the
// id each row emitted last (offset (g - 1) % L of its current block)
int run_prepare_inputs(bt_handle* h) {
  const Layout& lo = h->lo;
  NextStepArgs nx = next_step_args(h, h->g);
  Prof p(h, PK_FINALIZE, (double)h->B * (4.0 + lo.D * (lo.tab_elem + 4.0 + 2.0 * lo.elem)), 0.0);
  BT_CHECK(h, launch_finalize(nullptr, 0, 0, h->B, nullptr, (int32_t*)P_(h, lo.cur), lo.L, (h->g - 1) % lo.L,
                              (int*)P_(h, lo.dstate), 0, nx, h->st, nullptr, true),
           "next-step inputs");
  return BT_OK;
}

// Context embedding of rows (b, slot) of X [B][m][D] -> the token decoder's lead slots:
//   prefix: the P projected vectors become rows X [B][P][D];
//   summation: the L_B projected vectors go to CTX [B][L][D], and X [B][D] = pad embedding + u_0;
//   cross-attention: the P projected vectors go to ENC [B*P][D], their keys and values for every
//   token layer to XKV [B*P][Nt * 2 Hkv dh], and X [B][D] = pad embedding.
int run_prefix(bt_handle* h, int m, int slot) {
  const Layout& lo = h->lo;
  const double E = (double)lo.elem, D = lo.D, Bd = h->B, PD = (double)lo.NC * lo.D;
  {
    Prof p(h, PK_LN, Bd * D * (4.0 + E), 8.0 * Bd * D);
    BT_CHECK(h, launch_layernorm((float*)P_(h, lo.X), h->B, lo.D, m, slot, (const float*)P_(h, lo.lnf_blk),
                                 ln_buf(h, 0), nullptr, nullptr, lo.f32, h->cfg.ln_eps, pending(h), h->st),
             "context layernorm");
    h->pending.nsplit = 0;
  }
  Epi ep{};
  ep.wscale = wscale(lo);
  ep.bias = (const float*)P_(h, lo.prefix_b);
  ep.out0 = P_(h, lo.mode == BT_CTX_PREFIX ? lo.X : lo.mode == BT_CTX_SUM ? lo.ctx : lo.enc);
  ep.ld0 = lo.NC * lo.D;
  {
    Prof p(h, PK_GEMM_PREFIX, PD * D * E + Bd * D * E + Bd * PD * 4.0 + PD * 4.0, 2.0 * Bd * PD * D);
    BT_CHECK(h, launch_gemm(lo.f32, ln_buf(h, 0), nullptr, lo.D, P_(h, lo.prefix_w), h->B, lo.NC * lo.D, lo.D,
                            EPI_STORE, ep, h->st),
             "context projection");
  }
  if (lo.mode == BT_CTX_XATTN) {
    const int rows = h->B * lo.P;
    const double R = rows, N = lo.xkv_ld;
    Prof p(h, PK_GEMM_PREFIX, N * D * E + R * D * (4.0 + E) + R * N * 4.0 + N * 4.0, 2.0 * R * N * D);
    const void* A = P_(h, lo.enc);
    if (!lo.f32) {
      // encoder states as an fp16 operand in fragment order (rows padded to 16 with zeros)
      BT_CHECK(h, launch_pack_frag(P_(h, lo.enc), false, lo.D, 1, rows, (int)align_up(rows, 16), lo.D,
                                   P_(h, lo.enc16), lo.D, 0, 0, 1.0f, h->st),
               "encoder states");
      A = P_(h, lo.enc16);
    }
    Epi ex{};
    ex.wscale = wscale(lo);
    ex.bias = (const float*)P_(h, lo.xkv_b);
    ex.out0 = P_(h, lo.xkv);
    ex.ld0 = lo.xkv_ld;
    BT_CHECK(h, launch_gemm(lo.f32, A, nullptr, lo.D, P_(h, lo.xkv_w), rows, lo.xkv_ld, lo.D, EPI_STORE, ex, h->st),
             "cross-attention keys and values");
  }
  if (lo.mode != BT_CTX_PREFIX) {
    Prof p(h, PK_EMBED, Bd * D * (lo.mode == BT_CTX_SUM ? 12.0 : 8.0), 0.0);
    BT_CHECK(h, launch_rows_init((float*)P_(h, lo.X), h->B, lo.D, (const float*)P_(h, lo.pad_emb),
                                 lo.mode == BT_CTX_SUM ? (const float*)P_(h, lo.ctx) : nullptr, lo.L * lo.D, h->st),
             "start slot");
  }
  return BT_OK;
}


void drop_graphs(bt_handle* h) {
  for (hipGraphExec_t g : h->graphs)
    if (g) (void)hipGraphExecDestroy(g);
  h->graphs.clear();
  h->graph_B = -1;
}

// host mirror of what a decode step at in-block offset j does to the caches
void advance_host_state(bt_handle* h, int j) {
  if (j == 0) {
    h->n_blocks += 1;
    h->local_len = h->lo.vanilla ? 0 : h->lo.lead;
  } else {
    h->local_len = h->lo.lead + j;
  }
  h->pending.nsplit = 0;
}

// Enqueues one decode step up to and including the classifier (the greedy ids are finalised
// separately).  Kernel arguments depend only on (batch, j); the block-KV length is read on the
// device, so the same launch sequence is valid for every step with this j.
int enqueue_decode(bt_handle* h, int j, float* d_logits) {
  const Layout& lo = h->lo;
  const int lead = lo.lead;
  const double E = (double)lo.elem, Dd = lo.D, Bd = h->B, KVW = (double)lo.Hkv * lo.dh;
  int r;
  if (j == 0) {
    // the previous L_B emitted tokens complete a block: one block-decoder step (its input block
    // embedding and first LayerNorms were written by the previous finalisation)
    const int n = h->n_blocks;  // host mirror, for the profiler's byte count only
    for (int l = 0; l < lo.Nb; ++l) {
      if ((r = run_ln_qkv(h, lo.blk[l], h->B, l == 0))) return r;
      {
        // keys and values of entries [0, n) read once per KV head, q|k|v read, the new entry and
        // the output written
        Prof p(h, PK_ATTN_DECODE, Bd * (double)n * KVW * 2.0 * E + Bd * (2.0 * Dd + 4.0 * KVW) * E,
               4.0 * Bd * lo.H * lo.dh * (double)(n + 1));
        BT_CHECK(h, launch_block_attn_decode(lo.f32, P_(h, lo.QKV), h->B, (const int*)P_(h, lo.dstate), lo.H,
                                             lo.Hkv, lo.dh, (const float2*)P_(h, lo.rope), block_k(h, l), block_v(h, l),
                                             lo.ncap, P_(h, lo.ACT), lo.blk[l].k2, part_buf(h),
                                             part_cap(h), h->dec_nsplit, h->st, page_table(h), lo.ncap / 64),
                 "block attention decode");
      }
      if ((r = run_out(h, lo.blk[l], h->B))) return r;
    }
    if (lo.vanilla) {
      if ((r = run_head(h, 1, 0, d_logits))) return r;
    } else {
      if ((r = run_prefix(h, 1, 0))) return r;
      if ((r = run_token_decoder(h, lead, 0))) return r;
      if ((r = run_head(h, lead, lead - 1, d_logits))) return r;
    }
  } else {
    // one token-decoder position at local slot lead + j - 1 (input row and first LayerNorms written
    // by the previous finalisation)
    if ((r = run_token_decoder(h, 1, lead + j - 1, true))) return r;
    if ((r = run_head(h, 1, 0, d_logits))) return r;
  }
  advance_host_state(h, j);
  return BT_OK;
}

}  // namespace

extern "C" {

const char* bt_last_error(void) { return g_last_error.c_str(); }

size_t bt_weights_bytes(const bt_config* cfg) {
  if (!cfg) return (size_t)fail(0, "cfg is NULL");
  Layout lo;
  std::string e = plan_layout(*cfg, lo);
  if (!e.empty()) return (size_t)fail(0, e);
  return lo.bl_total;
}

size_t bt_workspace_bytes(const bt_config* cfg) {
  if (!cfg) return (size_t)fail(0, "cfg is NULL");
  Layout lo;
  std::string e = plan_layout(*cfg, lo);
  if (!e.empty()) return (size_t)fail(0, e);
  return lo.total;
}

int bt_workspace_region(const bt_config* cfg, int32_t which, size_t* offset, size_t* bytes, int32_t* capacity) {
  if (!cfg || !offset || !bytes || !capacity) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  Layout lo;
  std::string e = plan_layout(*cfg, lo);
  if (!e.empty()) return fail(BT_ERR_INVALID_ARG, e);
  if (which == 0) {
    *offset = lo.block_kv;
    *bytes = lo.block_kv_bytes;
    *capacity = lo.pages ? 64 : lo.ncap;
  } else if (which == 1) {
    *offset = lo.local_kv;
    *bytes = lo.local_kv_bytes;
    *capacity = lo.lcap;
  } else {
    return fail(BT_ERR_INVALID_ARG, "which must be 0 (block KV) or 1 (local KV)");
  }
  return BT_OK;
}

int bt_init(const bt_config* cfg, const void* d_weights, void* d_workspace, size_t ws_bytes, void* hip_stream,
            bt_handle** out) {
  if (!cfg || !d_weights || !d_workspace || !out) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  *out = nullptr;
  Layout lo;
  std::string e = plan_layout(*cfg, lo);
  if (!e.empty()) return fail(BT_ERR_INVALID_ARG, e);
  if (ws_bytes < lo.total) return fail(BT_ERR_INVALID_ARG, "workspace smaller than bt_workspace_bytes");
  if ((uintptr_t)d_workspace % 256) return fail(BT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if ((uintptr_t)d_weights % 16) return fail(BT_ERR_INVALID_ARG, "weights blob must be 16-byte aligned");
  bt_handle* h = new (std::nothrow) bt_handle();
  if (!h) return fail(BT_ERR_INVALID_ARG, "out of host memory");
  h->cfg = *cfg;
  h->lo = lo;
  h->ws = (char*)d_workspace;
  h->st = (hipStream_t)hip_stream;
  const char* wb = (const char*)d_weights;
  const bool bf = !lo.f32;
  const bool f32 = lo.f32;
  const float sc = f32 ? 1.0f : kWeightScale;
  const int D = lo.D, F = lo.F, QW = lo.QW;
  auto fin = [&](hipError_t err, const char* what) -> int {
    if (err == hipSuccess) return 0;
    bt_destroy(h);
    return fail(BT_ERR_HIP, std::string("bt_init ") + what + ": " + hipGetErrorString(err));
  };
#define INIT_CHECK(expr, what) \
  if (int r_ = fin((expr), what)) return r_;
  // caches and step state start at zero: every value ever read from them is then finite
  INIT_CHECK(hipMemsetAsync(h->ws + lo.block_kv, 0, lo.block_kv_bytes, h->st), "memset");
  INIT_CHECK(hipMemsetAsync(h->ws + lo.local_kv, 0, lo.local_kv_bytes, h->st), "memset");
  INIT_CHECK(hipMemsetAsync(h->ws + lo.cur, 0, (size_t)lo.Bmax * lo.L * 4, h->st), "memset");
  // weight-conversion flags: [0] = first out-of-range tensor (none: 0x7f7f7f7f), [1] = rounded count
  int* wflags = (int*)(h->ws + lo.wflags);
  INIT_CHECK(hipMemsetAsync(wflags, 0x7f, 4, h->st), "memset");
  INIT_CHECK(hipMemsetAsync(wflags + 1, 0, 4, h->st), "memset");
  std::vector<std::string> tensor_names;  // index = the tensor id the conversion reports
  INIT_CHECK(hipMemcpyAsync(h->ws + lo.emb_block, wb + lo.bl_emb_block, (size_t)lo.V * lo.De * lo.tab_elem,
                            hipMemcpyDeviceToDevice, h->st),
             "copy");
  if (!lo.vanilla)
    INIT_CHECK(hipMemcpyAsync(h->ws + lo.emb_tok, wb + lo.bl_emb_tok, (size_t)lo.V * D * lo.tab_elem,
                              hipMemcpyDeviceToDevice, h->st),
               "copy");
  // one [in, out] canonical matrix into rows [row0, row0 + N) and columns [col0, col0 + K) of a
  // repacked [rows][Ktot] weight (element (n = out, k = in) at src[k * N + n])
  auto name_id = [&](const std::string& name) {
    tensor_names.push_back(name);
    return (int)tensor_names.size() - 1;
  };
  auto put = [&](const std::string& name, size_t src, int K, int N, size_t dst, int Ktot, int row0,
                 int col0) -> hipError_t {
    if (f32) return launch_transpose_convert(wb + src, bf, K, N, h->ws + dst, f32, Ktot, row0, col0, sc, h->st);
    return launch_pack_frag(wb + src, bf, 1, N, N, N, K, h->ws + dst, Ktot, row0, col0, sc, h->st, wflags,
                            name_id(name));
  };
  // xl: index of a token layer with a cross-attention branch, else -1; pf: the layer's tensor-name prefix
  auto repack_layer = [&](const Layout::BlobLayer& s, const LayerOff& d, int xl, const std::string& pf) -> hipError_t {
    hipError_t err;
    float* ln = (float*)(h->ws + d.ln);
    if ((err = launch_to_f32(wb + s.ln1g, bf, D, ln, h->st))) return err;
    if ((err = launch_to_f32(wb + s.ln1b, bf, D, ln + D, h->st))) return err;
    if ((err = launch_to_f32(wb + s.ln2g, bf, D, ln + 2 * D, h->st))) return err;
    if ((err = launch_to_f32(wb + s.ln2b, bf, D, ln + 3 * D, h->st))) return err;
    // w1 rows: q | k | v (| cross-attention q) | up
    if ((err = put(pf + ".attn.qkv.w", s.qkvw, D, QW, d.w1, D, 0, 0))) return err;
    if (xl >= 0 && (err = put(pf + ".xattn.q.w", s.xqw, D, D, d.w1, D, QW, 0))) return err;
    if ((err = put(pf + ".mlp.up.w", s.upw, D, F, d.w1, D, d.n1, 0))) return err;
    float* b1 = (float*)(h->ws + d.b1);
    if ((err = launch_to_f32(wb + s.qkvb, bf, QW, b1, h->st))) return err;
    if (xl >= 0 && (err = launch_to_f32(wb + s.xqb, bf, D, b1 + QW, h->st))) return err;
    if ((err = launch_to_f32(wb + s.upb, bf, F, b1 + d.n1, h->st))) return err;
    // w2 columns: attn.out | mlp.down (| cross-attention out)
    if ((err = put(pf + ".attn.out.w", s.outw, D, D, d.w2, d.k2, 0, 0))) return err;
    if ((err = put(pf + ".mlp.down.w", s.downw, F, D, d.w2, d.k2, 0, D))) return err;
    if (xl >= 0 && (err = put(pf + ".xattn.out.w", s.xow, D, D, d.w2, d.k2, 0, D + F))) return err;
    float* b2 = (float*)(h->ws + d.b2);
    if ((err = launch_to_f32(wb + s.outb, bf, D, b2, h->st))) return err;
    if ((err = launch_to_f32(wb + s.downb, bf, D, b2 + D, h->st))) return err;
    if (xl < 0) return hipSuccess;
    // the branch's output bias joins attn.out.b; its key|value projection joins those of all layers
    if ((err = launch_to_f32(wb + s.xob, bf, D, b2 + 2 * D, h->st))) return err;
    if ((err = launch_add_f32(b2, b2 + 2 * D, D, h->st))) return err;
    const int xw = 2 * lo.Hkv * lo.dh;
    if ((err = put(pf + ".xattn.kv.w", s.xkvw, D, xw, lo.xkv_w, D, xl * xw, 0))) return err;
    return launch_to_f32(wb + s.xkvb, bf, xw, (float*)(h->ws + lo.xkv_b) + (size_t)xl * xw, h->st);
  };
  for (int l = 0; l < lo.Nb; ++l)
    INIT_CHECK(repack_layer(lo.bl_blk[l], lo.blk[l], -1, "blk." + std::to_string(l)), "repack block layer");
  for (int l = 0; l < lo.Nt; ++l)
    INIT_CHECK(repack_layer(lo.bl_tok[l], lo.tok[l], lo.mode == BT_CTX_XATTN ? l : -1, "tok." + std::to_string(l)),
               "repack token layer");
  if (!lo.vanilla && lo.mode != BT_CTX_PREFIX)
    INIT_CHECK(launch_to_f32(wb + lo.bl_emb_tok + (size_t)cfg->pad_id * D * lo.tab_elem, bf, D,
                             (float*)(h->ws + lo.pad_emb), h->st),
               "pad embedding");
  float* lnf = (float*)(h->ws + lo.lnf_blk);
  INIT_CHECK(launch_to_f32(wb + lo.bl_lnf_blk_g, bf, D, lnf, h->st), "repack");
  INIT_CHECK(launch_to_f32(wb + lo.bl_lnf_blk_b, bf, D, lnf + D, h->st), "repack");
  if (!lo.vanilla) {
    lnf = (float*)(h->ws + lo.lnf_tok);
    INIT_CHECK(launch_to_f32(wb + lo.bl_lnf_tok_g, bf, D, lnf, h->st), "repack");
    INIT_CHECK(launch_to_f32(wb + lo.bl_lnf_tok_b, bf, D, lnf + D, h->st), "repack");
    if (f32) {
      INIT_CHECK(launch_transpose_convert(wb + lo.bl_prefix_w, bf, D, lo.NC * D, h->ws + lo.prefix_w, f32, D, 0, 0, sc,
                                          h->st),
                 "repack prefix");
    } else {
      INIT_CHECK(launch_pack_frag(wb + lo.bl_prefix_w, bf, 1, (size_t)lo.NC * D, lo.NC * D, lo.NC * D, D,
                                  h->ws + lo.prefix_w, D, 0, 0, sc, h->st, wflags, name_id("prefix.w")),
                 "repack prefix");
    }
    INIT_CHECK(launch_to_f32(wb + lo.bl_prefix_b, bf, lo.NC * D, (float*)(h->ws + lo.prefix_b), h->st), "repack");
  }
  // classifier table [V, D]: element (n = id, k) at src[n * D + k]; rows up to Vpad are zero
  if (f32) {
    INIT_CHECK(launch_convert_rows(wb + lo.bl_head, bf, lo.V, D, lo.Vpad, h->ws + lo.head, f32, sc, h->st),
               "repack head");
  } else {
    INIT_CHECK(launch_pack_frag(wb + lo.bl_head, bf, D, 1, lo.V, lo.Vpad, D, h->ws + lo.head, D, 0, 0, sc, h->st,
                                wflags, name_id("head.w")),
               "repack head");
  }
  INIT_CHECK(launch_rope_table((float2*)(h->ws + lo.rope), lo.npos, lo.dh, cfg->rope_base, h->st), "rope table");
  if (lo.pages) {
    // every table entry starts at page 0, so no entry ever names memory outside the pool
    const size_t tab = (size_t)lo.Bmax * (lo.ncap / 64) * 4;
    INIT_CHECK(hipHostMalloc((void**)&h->ptab_host, tab), "page table");
    memset(h->ptab_host, 0, tab);
    INIT_CHECK(hipEventCreateWithFlags(&h->ptab_ev, hipEventDisableTiming), "page table");
    INIT_CHECK(hipMemcpyAsync(h->ws + lo.ptab, h->ptab_host, tab, hipMemcpyHostToDevice, h->st), "page table");
    INIT_CHECK(hipEventRecord(h->ptab_ev, h->st), "page table");
  }
  {
    // set-up of the static scratch of bt_decode_step_static on this device (once per device)
    void* scr = nullptr;
    INIT_CHECK(static_scratch(&scr), "static scratch");
  }
  if (!f32) {
    // every weight matrix must fit fp16 after the pre-scale: read the conversion flags back
    int32_t fl[2] = {0, 0};
    INIT_CHECK(hipMemcpyAsync(fl, wflags, sizeof(fl), hipMemcpyDeviceToHost, h->st), "weight check");
    INIT_CHECK(hipStreamSynchronize(h->st), "weight check");
    if (fl[0] != 0x7f7f7f7f) {
      const std::string name = fl[0] >= 0 && fl[0] < (int)tensor_names.size() ? tensor_names[fl[0]] : "?";
      bt_destroy(h);
      return fail(BT_ERR_UNSUPPORTED, "weight tensor " + name +
                                          " holds a value of magnitude >= 256 or a non-finite value: BT_BF16 "
                                          "keeps weight matrices as fp16 scaled by 2^8, which cannot hold it");
    }
    h->weights_rounded = fl[1];
  }
#undef INIT_CHECK
  *out = h;
  return BT_OK;
}

// Prefill of h->B rows (a join: into the cache rows h->rmap of a running batch): the block decoder
// over their Tp / L prompt blocks, the prefill tail and the first generated token.  ragged: every
// row padded only to its own multiple of L (its blocks left-aligned; the rest of the Tp / L rows
// are pad blocks whose results nothing reads).
static int prefill_core(bt_handle* h, const int32_t* d_prompt, const int32_t* d_lengths, int32_t T, int Tp,
                        bool ragged, int32_t* d_next, float* d_logits) {
  const Layout& lo = h->lo;
  const int L = lo.L, B = h->B;
  const int n0 = Tp / L;
  const int M = B * n0;
  h->pending.nsplit = 0;
  h->decode_phase = false;
  const double E = (double)lo.elem, Dd = lo.D, Md = M, KVW = (double)lo.Hkv * lo.dh;
  {
    Prof p(h, PK_EMBED, Md * Dd * (lo.tab_elem + 4.0) + (double)B * T * 4.0, 0.0);
    BT_CHECK(h, launch_embed_prompt(d_prompt, d_lengths, B, T, Tp, h->cfg.pad_id, P_(h, lo.emb_block), !lo.f32, lo.V,
                                    lo.De, L, (float*)P_(h, lo.X), (int*)P_(h, lo.dstate), ragged, h->rmap,
                                    ragged ? (int*)P_(h, lo.lastblk) : nullptr, h->st),
             "embed prompt");
  }
  for (int l = 0; l < lo.Nb; ++l) {
    int r = run_ln_qkv(h, lo.blk[l], M);
    if (r) return r;
    {
      Prof p(h, PK_ROPE_SCATTER, Md * 4.0 * KVW * E, 3.0 * Md * KVW);
      BT_CHECK(h, launch_rope_scatter(lo.f32, P_(h, lo.QKV), B, n0, 0, lo.H, lo.Hkv, lo.dh,
                                      (const float2*)P_(h, lo.rope), block_k(h, l), block_v(h, l), lo.ncap, true,
                                      h->st, h->rmap, page_table(h), lo.ncap / 64, page_limits(h)),
               "rope scatter");
    }
    {
      Prof p(h, PK_ATTN_PREFILL, Md * (2.0 * Dd + 2.0 * KVW) * E,
             4.0 * B * lo.H * lo.dh * (double)n0 * (n0 + 1) / 2.0);
      BT_CHECK(h, launch_prefill_attention(lo.f32, P_(h, lo.QKV), B, n0, lo.H, lo.Hkv, lo.dh,
                                           (const float2*)P_(h, lo.rope), block_k(h, l), block_v(h, l), lo.ncap,
                                           P_(h, lo.ACT), lo.blk[l].k2, h->st, h->rmap, page_table(h), lo.ncap / 64,
                                           page_limits(h)),
               "prefill attention");
    }
    r = run_out(h, lo.blk[l], M);
    if (r) return r;
  }
  int r;
  if (ragged && n0 > 1) {
    // the context of each row is its last real block: move it to the row's last activation slot
    if (h->pending.nsplit) {
      // the last layer's split-K residual is normally folded in by the LayerNorm that reads the
      // context row, after this move: fold it into every row first (its outputs are scratch)
      Prof p(h, PK_LN, Md * Dd * (4.0 + E), 8.0 * Md * Dd);
      BT_CHECK(h, launch_layernorm((float*)P_(h, lo.X), M, lo.D, 1, 0, (const float*)P_(h, lo.lnf_blk),
                                   ln_buf(h, 0), nullptr, nullptr, lo.f32, h->cfg.ln_eps, pending(h), h->st),
               "fold residual");
      h->pending.nsplit = 0;
    }
    Prof p(h, PK_EMBED, (double)B * Dd * 8.0, 0.0);
    BT_CHECK(h, launch_gather_last((float*)P_(h, lo.X), B, n0, lo.D, (const int*)P_(h, lo.lastblk), h->st),
             "last prompt blocks");
  }
  if (lo.vanilla) {
    if ((r = run_head(h, n0, n0 - 1, d_logits))) return r;
  } else {
    if ((r = run_prefix(h, n0, n0 - 1))) return r;
    if ((r = run_token_decoder(h, lo.lead, 0))) return r;
    if ((r = run_head(h, lo.lead, lo.lead - 1, d_logits))) return r;
  }
  return run_finalize(h, 0, d_next, 0);
}

static int prefill_impl(bt_handle* h, const int32_t* d_prompt, const int32_t* d_lengths, int32_t B, int32_t T,
                        int32_t* d_next, float* d_logits, bool ragged) {
  if (!h || !d_prompt || !d_next) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (h->broken) return fail(BT_ERR_STATE, "handle unusable after a HIP error");
  const Layout& lo = h->lo;
  if (B < 1 || T < 1) return fail(BT_ERR_INVALID_ARG, "B and T must be >= 1");
  if (B > lo.Bmax) return fail(BT_ERR_CAPACITY, "B exceeds max_batch");
  const int L = lo.L;
  const int Tp = std::max(L, (T + L - 1) / L * L);
  if ((int64_t)Tp + 1 > lo.max_tokens) return fail(BT_ERR_CAPACITY, "padded prompt + 1 exceeds max_tokens");
  if (Tp > lo.max_prompt) return fail(BT_ERR_CAPACITY, "padded prompt exceeds max_prompt_tokens");
  h->ready = false;
  h->g = 0;  // index of the token the prefill emits
  if (B != h->graph_B) drop_graphs(h);
  h->B = B;
  h->Tp = Tp;
  h->rmap = nullptr;
  h->dec_nsplit = decode_splits(B, lo.H, lo.Hkv, lo.ncap);
  if (lo.pages) {
    // a new batch: every page back in the pool, then each row's prompt blocks
    std::vector<int> rows(B), entries(B, Tp / L);
    for (int b = 0; b < B; ++b) rows[b] = b;
    if (ragged) {
      int e = ragged_entries(h, d_lengths, B, T, entries);
      if (e) return e;
    }
    size_t want = 0;
    for (int n : entries) want += (size_t)(n + 63) / 64;
    if (want > (size_t)lo.pages) return fail(BT_ERR_CAPACITY, "kv_pages exhausted");
    h->free_pages.clear();
    for (int pg = lo.pages - 1; pg >= 0; --pg) h->free_pages.push_back(pg);
    h->row_pages.assign(lo.Bmax, {});
    h->row_n.assign(lo.Bmax, 0);
    int e = pages_assign(h, rows, entries);
    if (e) return e;
  }
  int r = prefill_core(h, d_prompt, d_lengths, T, Tp, ragged, d_next, d_logits);
  if (r) return r;
  h->n_blocks = Tp / L;
  h->local_len = lo.vanilla ? 0 : lo.lead;
  h->row_tok.assign(B, (int64_t)Tp + 1);
  h->g = 1;
  h->ready = true;
  return BT_OK;
}

int bt_prefill(bt_handle* h, const int32_t* d_prompt, int32_t B, int32_t T, int32_t* d_next, float* d_logits) {
  return prefill_impl(h, d_prompt, nullptr, B, T, d_next, d_logits, false);
}

int bt_prefill_lengths(bt_handle* h, const int32_t* d_prompt, const int32_t* d_lengths, int32_t B, int32_t T,
                       int32_t* d_next, float* d_logits) {
  if (!d_lengths) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  return prefill_impl(h, d_prompt, d_lengths, B, T, d_next, d_logits, false);
}

int bt_prefill_ragged(bt_handle* h, const int32_t* d_prompt, const int32_t* d_lengths, int32_t B, int32_t T,
                      int32_t* d_next, float* d_logits) {
  if (!d_lengths) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  return prefill_impl(h, d_prompt, d_lengths, B, T, d_next, d_logits, true);
}

int bt_prefill_rows(bt_handle* h, const int32_t* rows, int32_t B_new, const int32_t* d_prompt,
                    const int32_t* d_lengths, int32_t T, int32_t* d_next, float* d_logits) {
  if (!h || !rows || !d_prompt || !d_lengths || !d_next) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (h->broken) return fail(BT_ERR_STATE, "handle unusable after a HIP error");
  if (!h->ready) return fail(BT_ERR_STATE, "bt_prefill_rows before bt_prefill");
  const Layout& lo = h->lo;
  if (lo.mode != BT_CTX_PREFIX) return fail(BT_ERR_UNSUPPORTED, "rows join only with BT_CTX_PREFIX");
  if (B_new < 1 || B_new > h->B || T < 1) return fail(BT_ERR_INVALID_ARG, "B_new must be in [1, B], T >= 1");
  std::vector<char> seen(h->B, 0);
  for (int i = 0; i < B_new; ++i) {
    if (rows[i] < 0 || rows[i] >= h->B || seen[rows[i]]) return fail(BT_ERR_INVALID_ARG, "rows must be distinct, in [0, B)");
    seen[rows[i]] = 1;
  }
  const int L = lo.L;
  if (h->g % L != 1 % L)
    return fail(BT_ERR_STATE, "rows join only where a block starts (after a step that emitted a block's first token)");
  const int Tp = std::max(L, (T + L - 1) / L * L);
  if ((int64_t)Tp + 1 > lo.max_tokens) return fail(BT_ERR_CAPACITY, "padded prompt + 1 exceeds max_tokens");
  if (Tp > lo.max_prompt) return fail(BT_ERR_CAPACITY, "padded prompt exceeds max_prompt_tokens");
  if (lo.pages) {
    // the joining rows give back their pages and take what their prompts need
    std::vector<int> rv(rows, rows + B_new), entries;
    int e = ragged_entries(h, d_lengths, B_new, T, entries);
    if (!e) e = pages_assign(h, rv, entries);
    if (e) return e;
  }
  BT_CHECK(h, hipMemcpyAsync(P_(h, lo.rowmap), rows, (size_t)B_new * 4, hipMemcpyHostToDevice, h->st), "row map");
  // the join runs its own classifier at B_new rows; the running batch's (possibly replayed from a
  // graph, which does not record it) column-group count must survive for its finalisations
  const int running_B = h->B, running_nparts = h->head_nparts;
  h->B = B_new;
  h->rmap = (const int*)P_(h, lo.rowmap);
  int r = prefill_core(h, d_prompt, d_lengths, T, Tp, true, d_next, d_logits);
  h->B = running_B;
  h->head_nparts = running_nparts;
  h->rmap = nullptr;
  h->pending.nsplit = 0;
  if (r) {
    h->ready = false;  // some rows may be half written
    return r;
  }
  // the prefill used the activation rows that held every row's next-step input: rebuild them
  if ((r = run_prepare_inputs(h))) {
    h->ready = false;
    return r;
  }
  for (int i = 0; i < B_new; ++i) h->row_tok[rows[i]] = (int64_t)Tp + 1;
  h->n_blocks = std::max(h->n_blocks, Tp / L);
  return BT_OK;
}

namespace {

// Checks shared by the decode-step entry points.
int decode_precheck(bt_handle* h, int32_t* d_next) {
  if (!h || !d_next) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (h->broken) return fail(BT_ERR_STATE, "handle unusable after a HIP error");
  if (!h->ready) return fail(BT_ERR_STATE, "bt_decode_step before bt_prefill");
  int64_t most = 0;
  for (int64_t t : h->row_tok) most = std::max(most, t);
  if (most + 1 > h->lo.max_tokens) return fail(BT_ERR_CAPACITY, "max_tokens reached");
  return BT_OK;
}

// Host bookkeeping after a decode step was enqueued.
void decode_done(bt_handle* h, int j) {
  h->g += 1;
  for (int64_t& t : h->row_tok) t += 1;
  if (h->lo.pages && j == 0)
    for (int b = 0; b < h->B; ++b) h->row_n[b] += 1;
}

}  // namespace

int bt_decode_step(bt_handle* h, int32_t* d_next, float* d_logits) {
  int r = decode_precheck(h, d_next);
  if (r) return r;
  const Layout& lo = h->lo;
  const int j = h->g % lo.L;
  h->decode_phase = true;
  if (lo.pages && j == 0 && (r = pages_grow(h))) return r;
  // graphs replay everything up to the classifier; the logits variant and profiling run eagerly
  if (h->use_graphs && !d_logits && !h->prof && h->st != nullptr) {
    if (h->graph_B != h->B) {
      drop_graphs(h);
      h->graphs.assign(lo.L, nullptr);
      h->graph_B = h->B;
    }
    if (!h->graphs[j]) {
      hipError_t e = hipStreamBeginCapture(h->st, hipStreamCaptureModeRelaxed);
      if (e != hipSuccess) return hip_fail(h, e, "graph capture");
      r = enqueue_decode(h, j, nullptr);
      hipGraph_t graph = nullptr;
      hipError_t e2 = hipStreamEndCapture(h->st, &graph);
      if (r) {
        if (graph) (void)hipGraphDestroy(graph);
        return r;
      }
      if (e2 != hipSuccess) return hip_fail(h, e2, "graph capture");
      hipGraphExec_t exec = nullptr;
      e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      if (e != hipSuccess) return hip_fail(h, e, "graph instantiate");
      h->graphs[j] = exec;
    } else {
      advance_host_state(h, j);
    }
    BT_CHECK(h, hipGraphLaunch(h->graphs[j], h->st), "graph launch");
  } else {
    r = enqueue_decode(h, j, d_logits);
    if (r) return r;
  }
  r = run_finalize(h, j, d_next, j == 0 ? 1 : 0);
  if (r) return r;
  decode_done(h, j);
  return BT_OK;
}

int bt_decode_step_static(bt_handle* h, int32_t* d_next, float* d_logits) {
  int r = decode_precheck(h, d_next);
  if (r) return r;
  const Layout& lo = h->lo;
  if (lo.pages) return fail(BT_ERR_UNSUPPORTED, "bt_decode_step_static does not run a paged block KV");
  // the step's partial results: split-K products of the [out|down] GEMMs (at most 16 per launch,
  // for up to B * lead rows), split-KV partials of the block attention, the classifier's keys
  const int rows = (int)std::min<int64_t>((int64_t)h->B * std::max(1, lo.lead), lo.rpart_rows);
  const size_t rpart = align_up((size_t)16 * rows * lo.D * 4, 256);
  const size_t part = align_up(h->dec_nsplit > 1 ? (size_t)h->B * lo.H * h->dec_nsplit * (lo.dh + 2) * 4 : 0, 256);
  const size_t keys = align_up((size_t)h->B * keys_ld(lo) * 8, 256);
  if (rpart + part + keys > kStaticScratchBytes)
    return fail(BT_ERR_CAPACITY, "bt_decode_step_static needs " + std::to_string(rpart + part + keys) +
                                     " bytes of static scratch at this batch; the maximum is " +
                                     std::to_string(kStaticScratchBytes));
  void* scr = nullptr;
  BT_CHECK(h, static_scratch(&scr), "static scratch");
  h->scr_rpart = (char*)scr;
  h->scr_part = (char*)scr + rpart;
  h->scr_part_bytes = part;
  h->scr_keys = (char*)scr + rpart + part;
  // eager launches only: no graph is captured or replayed and no profiling event is created
  const bool prof = h->prof;
  h->prof = false;
  const int j = h->g % lo.L;
  h->decode_phase = true;
  r = enqueue_decode(h, j, d_logits);
  if (!r) r = run_finalize(h, j, d_next, j == 0 ? 1 : 0);
  h->prof = prof;
  h->scr_rpart = h->scr_part = h->scr_keys = nullptr;
  h->scr_part_bytes = 0;
  if (r) return r;
  decode_done(h, j);
  return BT_OK;
}

int bt_page_table(bt_handle* h, int32_t* table) {
  if (!h || !table) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (!h->lo.pages) return fail(BT_ERR_UNSUPPORTED, "the block KV is not paged (kv_pages = 0)");
  BT_CHECK(h, hipStreamSynchronize(h->st), "synchronize");
  BT_CHECK(h, hipMemcpy(table, P_(h, h->lo.ptab), (size_t)h->lo.Bmax * (h->lo.ncap / 64) * 4,
                        hipMemcpyDeviceToHost),
           "copy");
  return BT_OK;
}

int bt_block_lengths(bt_handle* h, int32_t* lengths) {
  if (!h || !lengths) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (!h->ready) return fail(BT_ERR_STATE, "bt_block_lengths before bt_prefill");
  BT_CHECK(h, hipStreamSynchronize(h->st), "synchronize");
  BT_CHECK(h, hipMemcpy(lengths, P_(h, h->lo.dstate), (size_t)h->B * 4, hipMemcpyDeviceToHost), "copy");
  return BT_OK;
}

int bt_test_fuse_local(bt_handle* h, int32_t enable) {
  if (!h) return fail(BT_ERR_INVALID_ARG, "NULL handle");
  if (h->fuse_local != (enable != 0)) drop_graphs(h);
  h->fuse_local = enable != 0;
  return BT_OK;
}

int bt_set_graphs(bt_handle* h, int32_t enable) {
  if (!h) return fail(BT_ERR_INVALID_ARG, "NULL handle");
  h->use_graphs = enable != 0;
  if (!h->use_graphs) drop_graphs(h);
  return BT_OK;
}

int bt_cache_lengths(const bt_handle* h, int32_t* block_kv_len, int32_t* local_kv_len) {
  if (!h || !block_kv_len || !local_kv_len) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  *block_kv_len = h->ready ? h->n_blocks : 0;
  *local_kv_len = h->ready ? h->local_len : 0;
  return BT_OK;
}

int bt_numerics_status(bt_handle* h, int32_t reset, int64_t* status) {
  if (!h || !status) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (h->broken) return fail(BT_ERR_STATE, "handle unusable after a HIP error");
  unsigned int f[4] = {0u, 0u, 0u, 0u};
  BT_CHECK(h, clamp_flag_misc(&f[0], reset != 0, h->st), "clamp flag");
  BT_CHECK(h, clamp_flag_gemm(&f[1], reset != 0, h->st), "clamp flag");
  BT_CHECK(h, clamp_flag_gemm_decode(&f[2], reset != 0, h->st), "clamp flag");
  BT_CHECK(h, clamp_flag_attention(&f[3], reset != 0, h->st), "clamp flag");
  BT_CHECK(h, hipStreamSynchronize(h->st), "clamp flag");
  status[0] = h->weights_rounded;
  status[1] = (f[0] | f[1] | f[2] | f[3]) ? 1 : 0;
  return BT_OK;
}

int bt_destroy(bt_handle* h) {
  if (!h) return fail(BT_ERR_INVALID_ARG, "NULL handle");
  drop_graphs(h);
  for (hipEvent_t e : h->ev_pool) (void)hipEventDestroy(e);
  if (h->ptab_ev) (void)hipEventDestroy(h->ptab_ev);
  if (h->ptab_host) (void)hipHostFree(h->ptab_host);
  delete h;
  return BT_OK;
}

// ---------------------------------------------------------------- profiling and test entry points

int bt_profile_enable(bt_handle* h, int32_t on) {
  if (!h) return fail(BT_ERR_INVALID_ARG, "NULL handle");
  h->prof = on != 0;
  h->ev_used.clear();
  h->ev_next = 0;
  return BT_OK;
}

int bt_profile_read(bt_handle* h, int32_t n_kinds, double* total_ms, int64_t* launches, double* bytes,
                    double* flops) {
  if (!h || !total_ms || !launches || !bytes || !flops || n_kinds < 2 * PK_COUNT)
    return fail(BT_ERR_INVALID_ARG, "bad argument");
  for (int k = 0; k < n_kinds; ++k) {
    total_ms[k] = bytes[k] = flops[k] = 0.0;
    launches[k] = 0;
  }
  hipError_t e = hipStreamSynchronize(h->st);
  if (e != hipSuccess) return hip_fail(h, e, "profile sync");
  for (auto& u : h->ev_used) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, h->ev_pool[u.ev], h->ev_pool[u.ev + 1]) == hipSuccess) {
      total_ms[u.kind] += ms;
      launches[u.kind] += 1;
      bytes[u.kind] += u.bytes;
      flops[u.kind] += u.flops;
    }
  }
  h->ev_used.clear();
  h->ev_next = 0;
  return BT_OK;
}

int bt_test_replay(bt_handle* h, int32_t kind, int32_t reps) {
  if (!h || reps < 1) return fail(BT_ERR_INVALID_ARG, "bad argument");
  if (h->broken) return fail(BT_ERR_STATE, "handle unusable after a HIP error");
  if (h->B <= 0) return fail(BT_ERR_STATE, "bt_test_replay before bt_prefill");
  const Layout& lo = h->lo;
  // the attention appends at slot n (the device length, equal to the host mirror between calls)
  if (kind == PK_ATTN_DECODE && h->n_blocks >= lo.ncap) return fail(BT_ERR_CAPACITY, "block-KV cache full");
  if (kind == PK_ATTN_DECODE && lo.pages)
    return fail(BT_ERR_UNSUPPORTED, "no replay of the block attention on a paged cache (its append slot may have no page)");
  int r = BT_OK;
  for (int i = 0; i < reps && r == BT_OK; ++i) {
    if (kind == PK_GEMM_QKV) {
      // the decode step's [q|k|v|up] GEMM, cycling over the layers of both decoders (as many
      // distinct weights as a decode step streams between two uses of one layer) and over up to 64
      // distinct row ranges of the LayerNorm outputs (prefill-sized buffers), so that neither operand
      // is resident in a cache from the previous launch, as inside a decode step
      const int nl = lo.Nb + lo.Nt, l = i % nl;
      const LayerOff& w = l < lo.Nt ? lo.tok[l] : lo.blk[l - lo.Nt];
      const Epi ep = qkv_epi(h, w);
      const int64_t rows16 = (int64_t)align_up((size_t)h->B, 16);
      const int64_t na = std::max<int64_t>(1, std::min<int64_t>(64, lo.Mpad / rows16));
      const size_t off = (size_t)((i / nl) % na) * rows16 * lo.D * lo.elem;
      hipError_t e = launch_gemm(lo.f32, (char*)ln_buf(h, 0) + off, (char*)ln_buf(h, 1) + off, lo.D, P_(h, w.w1), h->B,
                                 w.n1 + lo.F, lo.D, EPI_QKV_GELU, ep, h->st);
      if (e != hipSuccess) r = hip_fail(h, e, "replay gemm");
    } else if (kind == PK_LOCAL_OUT) {
      // the token decoder's fused local attention + [out|down] launch at the next local slot (not
      // yet valid; the next token step writes it again), cycling over the token layers; its
      // products only go to the split-K partials, which nothing folds
      const int fs = fused_local_splits(h, 1);
      if (fs == 0) return fail(BT_ERR_UNSUPPORTED, "no fused [out|down] launch at this shape to replay");
      const ResidPending keep = h->pending;
      r = run_fused_local_out(h, i % lo.Nt, std::min(h->local_len, lo.lcap - 1), fs);
      h->pending = keep;
    } else if (kind == PK_ATTN_DECODE) {
      const int l = i % lo.Nb;
      hipError_t e = launch_block_attn_decode(lo.f32, P_(h, lo.QKV), h->B, (const int*)P_(h, lo.dstate), lo.H,
                                              lo.Hkv, lo.dh, (const float2*)P_(h, lo.rope), block_k(h, l),
                                              block_v(h, l), lo.ncap, P_(h, lo.ACT), lo.blk[l].k2, part_buf(h),
                                              part_cap(h), h->dec_nsplit, h->st, page_table(h), lo.ncap / 64);
      if (e != hipSuccess) r = hip_fail(h, e, "replay attention");
    } else if (kind == -1) {
      hipError_t e = launch_empty(256, h->st);
      if (e != hipSuccess) r = hip_fail(h, e, "replay empty kernel");
    } else {
      r = fail(BT_ERR_INVALID_ARG, "kind not replayable");
    }
  }
  return r;
}

int bt_test_gemm(int32_t dtype, const void* d_a, const void* d_w, float* d_c, int32_t M, int32_t N, int32_t K,
                 float scale, void* stream) {
  if (!d_a || !d_w || !d_c) return fail(BT_ERR_INVALID_ARG, "NULL argument");
  if (M < 1 || N < 1 || K < 1) return fail(BT_ERR_INVALID_ARG, "M, N, K must be >= 1");
  const bool f32 = dtype == BT_FP32;
  if (!f32 && (K % 64 || N % 32)) return fail(BT_ERR_INVALID_ARG, "fp16 GEMM needs K % 64 == 0 and N % 32 == 0");
  Epi ep{};
  ep.wscale = scale;
  ep.out0 = d_c;
  ep.ld0 = N;
  hipError_t e = launch_gemm(f32, d_a, nullptr, K, d_w, M, N, K, EPI_STORE, ep, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BT_ERR_HIP, std::string("gemm: ") + hipGetErrorString(e));
  return BT_OK;
}

}  // extern "C"
