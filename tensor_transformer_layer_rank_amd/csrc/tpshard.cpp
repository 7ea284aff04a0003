// C ABI of libtpshard: argument validation, per-rank sizes, workspace
// layout and the launch sequence of each entry point.  See tpshard.h.
//
// Per-rank sizes follow "8. How several ranks share one ledger" ("Weights
// are cut by name": even chunks along dim 0 / dim 1, one whole kv head per
// rank when there are fewer kv heads than ranks, vocab rows in ceil(V/n)
// blocks) and "Tensor parallelism from scratch" ("KV heads and the limit on
// TP": head counts that do not divide are rejected).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <string>
#include <vector>

#include "../../include/tpshard.h"
#include "common.h"

using namespace tps;

// Per-kernel timing marks (tp_kernel_marks): per host thread, the caller's
// events and the names of the kernels marked so far.
namespace {
struct KernelMarks {
  std::vector<hipEvent_t> events;
  std::vector<std::string> names;
};
thread_local KernelMarks g_marks;
}  // namespace

namespace tps {
bool kmarks_armed() { return g_marks.names.size() < g_marks.events.size(); }
void kmark(hipStream_t s, const char* name) {
  if (!kmarks_armed()) return;
  (void)hipEventRecord(g_marks.events[g_marks.names.size()], s);
  g_marks.names.emplace_back(name);
}
}  // namespace tps

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_cfg(const tp_cfg* c, tp_local* L) {
  if (!c) return TP_ERR_NULL;
  if (c->tp_size < 1 || c->tp_rank < 0 || c->tp_rank >= c->tp_size) return TP_ERR_RANK;
  if (c->dtype != TP_F32 && c->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (c->hidden <= 0 || c->intermediate < 0 || c->n_q_heads < 0 || c->n_kv_heads < 0 || c->vocab < 0 ||
      c->head_dim < 0)
    return TP_ERR_SHAPE;
  const int n = c->tp_size, r = c->tp_rank;
  if (c->n_q_heads % n || c->intermediate % n) return TP_ERR_SHAPE;
  tp_local o{};
  o.lq = c->n_q_heads / n;
  if (c->n_q_heads == 0 && c->n_kv_heads == 0) {
    o.lkv = 0;
    o.kv_head0 = 0;
  } else {
    if (c->n_q_heads == 0 || c->n_kv_heads == 0 || c->head_dim <= 0) return TP_ERR_SHAPE;
    if (c->n_q_heads % c->n_kv_heads) return TP_ERR_SHAPE;   // GQA groups must be whole
    if (c->n_kv_heads >= n) {
      if (c->n_kv_heads % n) return TP_ERR_SHAPE;
      o.lkv = c->n_kv_heads / n;
      o.kv_head0 = r * o.lkv;
    } else {
      if (n % c->n_kv_heads) return TP_ERR_SHAPE;
      o.lkv = 1;                                             // replicated kv head
      o.kv_head0 = (int32_t)((int64_t)r * c->n_kv_heads / n);
    }
  }
  o.li = c->intermediate / n;
  o.n_qkv = (int64_t)(o.lq + 2 * o.lkv) * c->head_dim;
  const int64_t per = (c->vocab + n - 1) / n;
  o.vocab_start = (int64_t)r * per < c->vocab ? (int64_t)r * per : c->vocab;
  o.vocab_end = (int64_t)(r + 1) * per < c->vocab ? (int64_t)(r + 1) * per : c->vocab;
  if (L) *L = o;
  return TP_OK;
}

int esize_of(const tp_cfg* c) { return c->dtype == TP_BF16 ? 2 : 4; }

// workspace layout of tp_qkv_attn (each region 256-byte aligned)
struct AttnWs {
  size_t q, attn, scratch, scratch_bytes, total;
};
AttnWs attn_ws(const tp_cfg* c, const tp_local& L, int64_t B, int64_t T, int64_t past) {
  const int64_t M = B * T;
  AttnWs w{};
  w.q = 0;
  w.attn = w.q + align_up((size_t)(M * L.lq * 128) * 2);
  w.scratch = w.attn + align_up((size_t)(M * L.lq * 128) * 2);
  size_t sb = gemm_scratch_bytes(M, L.n_qkv, c->hidden, EPI_QKV);
  const size_t so = gemm_scratch_bytes(M, c->hidden, (int64_t)L.lq * 128, EPI_BF16);
  if (so > sb) sb = so;
  w.scratch_bytes = align_up(sb);
  w.total = w.scratch + w.scratch_bytes;
  return w;
}

struct MlpWs {
  size_t h, scratch, scratch_bytes, total;
};
MlpWs mlp_ws(const tp_cfg* c, const tp_local& L, int64_t M) {
  MlpWs w{};
  w.h = 0;
  w.scratch = align_up((size_t)(M * L.li) * esize_of(c));
  size_t sb = 0;
  if (c->dtype == TP_BF16) {
    sb = gemm_scratch_bytes(M, 2 * (int64_t)L.li, c->hidden, EPI_SILU_BF16);
    const size_t sd = gemm_scratch_bytes(M, c->hidden, L.li, EPI_BF16);
    if (sd > sb) sb = sd;
  }
  w.scratch_bytes = align_up(sb);
  w.total = w.scratch + w.scratch_bytes;
  return w;
}

// workspace of tp_lm_head_argmax: one 8-byte candidate per row and N tile
// of the logits GEMM, or per row and workgroup of the resident-rows kernel
struct LmWs {
  bool resident;
  int64_t tiles_n;
  size_t total;
};
LmWs lm_ws(const tp_cfg* c, const tp_local& L, int64_t M) {
  LmWs w{};
  const int64_t N = L.vocab_end - L.vocab_start;
  w.resident = argmax_resident_ok(M, N, c->hidden);
  w.tiles_n = w.resident ? argmax_resident_groups() : gemm_argmax_tiles_n(M, N, c->hidden);
  w.total = align_up((size_t)(M * w.tiles_n) * 8);
  return w;
}

int launched(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_LAUNCH; }

// the optional row list of the heads: rows_opt NULL (x rows 0..M-1) or an
// int32 list into x's x_rows rows, read through one 31-bit descriptor range
int check_head_rows(const tp_cfg* cfg, int64_t M, const int32_t* rows, int64_t x_rows) {
  if (!rows) return TP_OK;
  if (x_rows < 1) return TP_ERR_RANGE;
  if ((uintptr_t)rows & 3) return TP_ERR_ALIGN;
  if (x_rows * cfg->hidden * 2 >= ((int64_t)1 << 31)) return TP_ERR_SHAPE;
  (void)M;
  return TP_OK;
}

// the decode head's launches: per-shard candidates into `cand` (w.total
// bytes), then their reduction to one (value, id) per row
hipError_t lm_head_argmax_launch(const tp_cfg* cfg, const tp_local& L, const void* x, int64_t M, const int32_t* rows,
                                 int64_t x_rows, const void* vocab_local, float* out_val, int32_t* out_idx,
                                 const LmWs& w, void* cand, hipStream_t s) {
  const int64_t N = L.vocab_end - L.vocab_start, H = cfg->hidden;
  if (w.resident) {
    // few rows, short hidden size: rows resident on chip, the vocab slice
    // streamed once
    const hipError_t e = argmax_resident(x, M, rows, x_rows, vocab_local, N, H, cand, s);
    if (e != hipSuccess) return e;
  } else if (N > 0) {
    // logits GEMM whose epilogue leaves one candidate per row and N tile
    GemmProblem g{static_cast<const bf16*>(x), static_cast<const bf16*>(vocab_local), cand, M, N, H, H, H,
                  w.tiles_n, 0};
    g.a_rows = rows;
    g.a_total = x_rows;
    const hipError_t e = gemm_bf16(g, EPI_ARGMAX, nullptr, 0, s);
    if (e != hipSuccess) return e;
  }
  return argmax_candidates(cand, M, w.tiles_n, L.vocab_start, out_val, out_idx, s);
}

// The kernels read through buffer descriptors whose byte range is 32-bit.
// A GEMM tile's descriptor starts at the tile's first row and its loads
// reach at most 256 rows of the operand, so a row length (K, in elements)
// below 2^22 keeps every offset under 2^31; an attention descriptor covers
// one (sequence, kv head) slab of 256-byte cache rows, so positions stay
// below 2^24.
constexpr int64_t kMaxRowElems = int64_t(1) << 22;
constexpr int64_t kMaxPositions = int64_t(1) << 24;
bool row_ok(int64_t k) { return k > 0 && k < kMaxRowElems; }

}  // namespace

extern "C" {

int tp_local_dims(const tp_cfg* cfg, tp_local* out) {
  if (!out) return TP_ERR_NULL;
  return check_cfg(cfg, out);
}

int tp_kernel_marks(void* const* events, int32_t n_events) {
  if (n_events < 0) return TP_ERR_RANGE;
  if (n_events > 0 && !events) return TP_ERR_NULL;
  g_marks.events.assign(reinterpret_cast<const hipEvent_t*>(events),
                        reinterpret_cast<const hipEvent_t*>(events) + n_events);
  g_marks.names.clear();
  return TP_OK;
}

int32_t tp_kernel_marks_used(void) { return (int32_t)g_marks.names.size(); }

const char* tp_kernel_mark_name(int32_t i) {
  return i >= 0 && (size_t)i < g_marks.names.size() ? g_marks.names[i].c_str() : "";
}

const char* tp_status_str(int s) {
  switch (s) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "null pointer";
    case TP_ERR_RANK: return "tp_rank outside [0, tp_size)";
    case TP_ERR_SHAPE: return "shape not splittable across ranks or not supported";
    case TP_ERR_DTYPE: return "dtype not supported";
    case TP_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TP_ERR_WORKSPACE: return "workspace too small";
    case TP_ERR_RANGE: return "size out of range (negative, or past_len + T > S_max)";
    case TP_ERR_LAUNCH: return "kernel launch failed";
    case TP_ERR_KIND: return "unknown weight kind or op";
    default: return "unknown status";
  }
}

int tp_workspace_bytes(const tp_cfg* cfg, int op, int64_t B, int64_t T, int64_t past_len, size_t* out_bytes) {
  if (!out_bytes) return TP_ERR_NULL;
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (B < 0 || T < 0 || past_len < 0) return TP_ERR_RANGE;
  if (op == TP_OP_ATTN) {
    if (L.lq == 0) return TP_ERR_SHAPE;
    *out_bytes = attn_ws(cfg, L, B, T, past_len).total;
  } else if (op == TP_OP_MLP) {
    *out_bytes = mlp_ws(cfg, L, B * T).total;
  } else if (op == TP_OP_LM_ARGMAX) {
    *out_bytes = lm_ws(cfg, L, B * T).total;
  } else {
    return TP_ERR_KIND;
  }
  return TP_OK;
}

int tp_shard_weights(const tp_cfg* cfg, int kind, const void* full, void* dst, void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (kind < TP_W_Q || kind > TP_W_VOCAB) return TP_ERR_KIND;
  if (!full || !dst) return TP_ERR_NULL;
  if (!aligned16(full) || !aligned16(dst)) return TP_ERR_ALIGN;
  const int es = esize_of(cfg);
  const int64_t H = cfg->hidden, d = cfg->head_dim, r = cfg->tp_rank;
  const bool heads = L.lq > 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* dp = static_cast<char*>(dst);
  hipError_t e = hipSuccess;
  switch (kind) {
    case TP_W_Q:
      if (!heads) return TP_ERR_SHAPE;
      e = copy2d(full, H, r * L.lq * d, 0, dp, H, L.lq * d, H, es, s);
      break;
    case TP_W_K:
      if (!heads) return TP_ERR_SHAPE;
      e = copy2d(full, H, (int64_t)L.kv_head0 * d, 0, dp + (L.lq * d * H) * es, H, L.lkv * d, H, es, s);
      break;
    case TP_W_V:
      if (!heads) return TP_ERR_SHAPE;
      e = copy2d(full, H, (int64_t)L.kv_head0 * d, 0, dp + ((L.lq + L.lkv) * d * H) * es, H, L.lkv * d, H, es, s);
      break;
    case TP_W_O:
      if (!heads) return TP_ERR_SHAPE;
      e = copy2d(full, (int64_t)cfg->n_q_heads * d, 0, r * L.lq * d, dp, L.lq * d, H, L.lq * d, es, s);
      break;
    case TP_W_GATE:
      if (L.li == 0) return TP_ERR_SHAPE;
      e = copy2d(full, H, r * L.li, 0, dp, H, L.li, H, es, s);
      break;
    case TP_W_UP:
      if (L.li == 0) return TP_ERR_SHAPE;
      e = copy2d(full, H, r * L.li, 0, dp + ((int64_t)L.li * H) * es, H, L.li, H, es, s);
      break;
    case TP_W_DOWN:
      if (L.li == 0) return TP_ERR_SHAPE;
      e = copy2d(full, cfg->intermediate, 0, r * L.li, dp, L.li, H, L.li, es, s);
      break;
    case TP_W_VOCAB:
      if (cfg->vocab == 0) return TP_ERR_SHAPE;
      e = copy2d(full, H, L.vocab_start, 0, dp, H, L.vocab_end - L.vocab_start, H, es, s);
      break;
  }
  return launched(e);
}

int tp_embed_vocab(const tp_cfg* cfg, const int32_t* ids, int64_t n_tokens, const void* vocab_local, void* out,
                   void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (n_tokens < 0) return TP_ERR_RANGE;
  if (!ids || !vocab_local || !out) return TP_ERR_NULL;
  if (!aligned16(ids) || !aligned16(vocab_local) || !aligned16(out)) return TP_ERR_ALIGN;
  if (((int64_t)cfg->hidden * esize_of(cfg)) % 16) return TP_ERR_SHAPE;
  if (n_tokens == 0) return TP_OK;
  return launched(embed_masked(ids, n_tokens, vocab_local, L.vocab_start, L.vocab_end, cfg->hidden,
                               esize_of(cfg), out, static_cast<hipStream_t>(stream)));
}

int tp_qkv_attn(const tp_cfg* cfg, const void* x, int32_t B, int32_t T, int32_t past_len, const void* w_qkv,
                const void* q_norm_w, const void* k_norm_w, const void* w_o, void* k_cache, void* v_cache,
                int32_t S_max, void* q_out_opt, void* attn_out_opt, void* out_partial, void* workspace,
                size_t ws_bytes, void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (L.lq == 0 || cfg->head_dim != 128 || cfg->hidden % 8) return TP_ERR_SHAPE;
  if (!row_ok(cfg->hidden) || !row_ok((int64_t)L.lq * 128) || S_max >= kMaxPositions) return TP_ERR_SHAPE;
  const int rep = L.lq / L.lkv;
  if (L.lq % L.lkv || (rep != 1 && rep != 2 && rep != 4 && rep != 8 && rep != 16)) return TP_ERR_SHAPE;
  if (B < 0 || T < 0 || past_len < 0 || S_max < 0) return TP_ERR_RANGE;
  if ((int64_t)past_len + T > S_max) return TP_ERR_RANGE;
  if (!x || !w_qkv || !q_norm_w || !k_norm_w || !w_o || !k_cache || !v_cache || !out_partial)
    return TP_ERR_NULL;
  const void* ptrs[] = {x, w_qkv, q_norm_w, k_norm_w, w_o, k_cache, v_cache, out_partial};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TP_ERR_ALIGN;
  if ((q_out_opt && !aligned16(q_out_opt)) || (attn_out_opt && !aligned16(attn_out_opt))) return TP_ERR_ALIGN;
  if ((int64_t)B * T == 0) return TP_OK;
  const AttnWs w = attn_ws(cfg, L, B, T, past_len);
  if (!workspace) return TP_ERR_NULL;
  if (!aligned16(workspace)) return TP_ERR_ALIGN;
  if (ws_bytes < w.total) return TP_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t M = (int64_t)B * T, H = cfg->hidden, lqd = (int64_t)L.lq * 128;
  bf16* q = q_out_opt ? static_cast<bf16*>(q_out_opt) : reinterpret_cast<bf16*>(ws + w.q);
  bf16* attn = attn_out_opt ? static_cast<bf16*>(attn_out_opt) : reinterpret_cast<bf16*>(ws + w.attn);
  void* scratch = ws + w.scratch;

  // 1. merged column-parallel projection, finished per head in the epilogue:
  //    QK-norm, RoPE, q to its buffer, k and v appended to the caches
  GemmProblem g{static_cast<const bf16*>(x), static_cast<const bf16*>(w_qkv), nullptr, M, L.n_qkv, H, H, H, 0, 0};
  g.qkv = QkvArgs{static_cast<const bf16*>(q_norm_w), static_cast<const bf16*>(k_norm_w), q,
                  static_cast<bf16*>(k_cache), static_cast<bf16*>(v_cache), B, T, past_len, S_max, L.lq, L.lkv,
                  cfg->rms_eps, cfg->rope_theta};
  //    (decode with a split-K plan: only the partials; the attention kernel
  //    finishes them, which saves the reduction launch)
  int qkv_splits = 0;
  hipError_t e = gemm_qkv(g, scratch, w.scratch_bytes, T == 1, &qkv_splits, s);
  if (e != hipSuccess) return TP_ERR_LAUNCH;
  // 2. attention over the local heads
  AttnArgs aa{q, static_cast<const bf16*>(k_cache), static_cast<const bf16*>(v_cache), attn,
              B, T, past_len, S_max, L.lq, L.lkv};
  if (qkv_splits > 0) {
    aa.qkv_part = static_cast<const float*>(scratch);
    aa.qkv_splits = qkv_splits;
    aa.q_norm_w = static_cast<const bf16*>(q_norm_w);
    aa.k_norm_w = static_cast<const bf16*>(k_norm_w);
    aa.eps = cfg->rms_eps;
    aa.theta = cfg->rope_theta;
    aa.q_store = q_out_opt ? q : nullptr;
  }
  e = T > 1 && attn_prefill_fills(B, T, L.lq, L.lkv) ? attn_prefill(aa, s) : attn_flash(aa, s);
  if (e != hipSuccess) return TP_ERR_LAUNCH;
  // 3. row-parallel o_proj -> partial sum
  GemmProblem go{attn, static_cast<const bf16*>(w_o), out_partial, M, H, lqd, lqd, lqd, H, 0};
  return launched(gemm_bf16(go, EPI_BF16, scratch, w.scratch_bytes, s));
}

int tp_mlp(const tp_cfg* cfg, const void* x, int64_t M, const void* w_gate_up, const void* w_down, void* h_opt,
           void* out_partial, void* workspace, size_t ws_bytes, void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (L.li == 0 || cfg->hidden % 8 || L.li % 8) return TP_ERR_SHAPE;
  if (!row_ok(cfg->hidden) || !row_ok(L.li)) return TP_ERR_SHAPE;
  if (M < 0) return TP_ERR_RANGE;
  if (!x || !w_gate_up || !w_down || !out_partial) return TP_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(out_partial) ||
      (h_opt && !aligned16(h_opt)))
    return TP_ERR_ALIGN;
  if (M == 0) return TP_OK;
  const MlpWs w = mlp_ws(cfg, L, M);
  if (!h_opt || w.scratch_bytes) {
    if (!workspace) return TP_ERR_NULL;
    if (!aligned16(workspace)) return TP_ERR_ALIGN;
    if (ws_bytes < w.total) return TP_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t H = cfg->hidden, li = L.li;
  void* h = h_opt ? h_opt : ws + w.h;
  if (cfg->dtype == TP_F32) {
    hipError_t e = gemm_f32(static_cast<const float*>(x), static_cast<const float*>(w_gate_up),
                            static_cast<float*>(h), M, 2 * li, H, (int)li, s);
    if (e != hipSuccess) return TP_ERR_LAUNCH;
    return launched(gemm_f32(static_cast<const float*>(h), static_cast<const float*>(w_down),
                             static_cast<float*>(out_partial), M, H, li, 0, s));
  }
  void* scratch = ws ? ws + w.scratch : nullptr;
  // gate_up column-parallel GEMM with silu(gate) * up fused
  GemmProblem g{static_cast<const bf16*>(x), static_cast<const bf16*>(w_gate_up), h, M, 2 * li, H, H, H, li, li};
  hipError_t e = gemm_bf16(g, EPI_SILU_BF16, scratch, w.scratch_bytes, s);
  if (e != hipSuccess) return TP_ERR_LAUNCH;
  // down row-parallel GEMM -> partial sum
  GemmProblem gd{static_cast<const bf16*>(h), static_cast<const bf16*>(w_down), out_partial, M, H, li, li, li, H, 0};
  return launched(gemm_bf16(gd, EPI_BF16, scratch, w.scratch_bytes, s));
}

int tp_lm_head(const tp_cfg* cfg, const void* x, int64_t M, const int32_t* rows_opt, int64_t x_rows,
               const void* vocab_local, void* logits_local, void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (cfg->vocab == 0 || cfg->hidden % 8 || !row_ok(cfg->hidden)) return TP_ERR_SHAPE;
  if (M < 0) return TP_ERR_RANGE;
  if (!x || !vocab_local || !logits_local) return TP_ERR_NULL;
  if (!aligned16(x) || !aligned16(vocab_local) || !aligned16(logits_local)) return TP_ERR_ALIGN;
  if ((st = check_head_rows(cfg, M, rows_opt, x_rows))) return st;
  if (rows_opt && cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  const int64_t N = L.vocab_end - L.vocab_start, H = cfg->hidden;
  if (M == 0 || N == 0) return TP_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg->dtype == TP_F32)
    return launched(gemm_f32(static_cast<const float*>(x), static_cast<const float*>(vocab_local),
                             static_cast<float*>(logits_local), M, N, H, 0, s));
  GemmProblem g{static_cast<const bf16*>(x), static_cast<const bf16*>(vocab_local), logits_local, M, N, H, H, H, N, 0};
  g.a_rows = rows_opt;
  g.a_total = x_rows;
  return launched(gemm_bf16(g, EPI_BF16, nullptr, 0, s));
}

int tp_lm_head_argmax(const tp_cfg* cfg, const void* x, int64_t M, const int32_t* rows_opt, int64_t x_rows,
                      const void* vocab_local, float* out_val, int32_t* out_idx, void* workspace, size_t ws_bytes,
                      void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (cfg->vocab == 0 || cfg->hidden % 8 || !row_ok(cfg->hidden)) return TP_ERR_SHAPE;
  if (M < 0) return TP_ERR_RANGE;
  if (!x || !vocab_local || !out_val || !out_idx) return TP_ERR_NULL;
  if (!aligned16(x) || !aligned16(vocab_local) || ((uintptr_t)out_val & 3) || ((uintptr_t)out_idx & 3))
    return TP_ERR_ALIGN;
  if ((st = check_head_rows(cfg, M, rows_opt, x_rows))) return st;
  if (M == 0) return TP_OK;
  const LmWs w = lm_ws(cfg, L, M);
  if (w.total > 0) {
    if (!workspace) return TP_ERR_NULL;
    if (!aligned16(workspace)) return TP_ERR_ALIGN;
    if (ws_bytes < w.total) return TP_ERR_WORKSPACE;
  }
  return launched(lm_head_argmax_launch(cfg, L, x, M, rows_opt, x_rows, vocab_local, out_val, out_idx, w, workspace,
                                        static_cast<hipStream_t>(stream)));
}

int tp_lm_head_argmax_noalloc(const tp_cfg* cfg, const void* x, int64_t M, const int32_t* rows_opt, int64_t x_rows,
                              const void* vocab_local, float* out_val, int32_t* out_idx, void* stream) {
  tp_local L;
  int st = check_cfg(cfg, &L);
  if (st) return st;
  if (cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (cfg->vocab == 0 || cfg->hidden % 8 || !row_ok(cfg->hidden)) return TP_ERR_SHAPE;
  if (M < 0) return TP_ERR_RANGE;
  if (!x || !vocab_local || !out_val || !out_idx) return TP_ERR_NULL;
  if (!aligned16(x) || !aligned16(vocab_local) || ((uintptr_t)out_val & 3) || ((uintptr_t)out_idx & 3))
    return TP_ERR_ALIGN;
  if ((st = check_head_rows(cfg, M, rows_opt, x_rows))) return st;
  if (M == 0) return TP_OK;
  const LmWs w = lm_ws(cfg, L, M);
  if (w.total > kNoAllocScratchBytes) return TP_ERR_WORKSPACE;   // candidates exceed the static array
  void* cand = nullptr;
  if (noalloc_scratch(&cand) != hipSuccess) return TP_ERR_LAUNCH;
  return launched(lm_head_argmax_launch(cfg, L, x, M, rows_opt, x_rows, vocab_local, out_val, out_idx, w, cand,
                                        static_cast<hipStream_t>(stream)));
}

int tp_argmax_combine(const float* vals, const int32_t* idx, int32_t n_shards, int64_t M, int32_t* out_idx,
                      float* out_val_opt, void* stream) {
  if (n_shards < 1 || M < 0) return TP_ERR_RANGE;
  if (!vals || !idx || !out_idx) return TP_ERR_NULL;
  if (((uintptr_t)vals & 3) || ((uintptr_t)idx & 3) || ((uintptr_t)out_idx & 3) || ((uintptr_t)out_val_opt & 3))
    return TP_ERR_ALIGN;
  if (M == 0) return TP_OK;
  return launched(argmax_combine(vals, idx, n_shards, M, out_idx, out_val_opt, static_cast<hipStream_t>(stream)));
}

int tp_residual_rmsnorm(const tp_cfg* cfg, const void* partials, int32_t n_partials, int64_t M, const void* residual,
                        const void* norm_w, void* h_out, void* y_out, void* stream) {
  int st = check_cfg(cfg, nullptr);
  if (st) return st;
  if (cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (cfg->hidden % 8 || cfg->hidden > 8192) return TP_ERR_SHAPE;
  if (n_partials < 0 || M < 0) return TP_ERR_RANGE;
  if ((n_partials > 0 && (!partials || !h_out)) || !residual || !norm_w || !y_out) return TP_ERR_NULL;
  const void* ptrs[] = {partials, residual, norm_w, h_out, y_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TP_ERR_ALIGN;
  if (M == 0) return TP_OK;
  NormArgs a{static_cast<const bf16*>(partials), n_partials, M * cfg->hidden, M, cfg->hidden,
             static_cast<const bf16*>(residual), static_cast<const bf16*>(norm_w), cfg->rms_eps,
             static_cast<bf16*>(h_out), static_cast<bf16*>(y_out), nullptr, M};
  return launched(residual_rmsnorm(a, static_cast<hipStream_t>(stream)));
}

int tp_rmsnorm_rows(const tp_cfg* cfg, const void* x, int64_t x_rows, const int32_t* rows, int64_t n_rows,
                    const void* norm_w, void* y_out, void* stream) {
  int st = check_cfg(cfg, nullptr);
  if (st) return st;
  if (cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (cfg->hidden % 8 || cfg->hidden > 8192) return TP_ERR_SHAPE;
  if (x_rows < 0 || n_rows < 0 || (!rows && n_rows > x_rows) || (rows && n_rows > 0 && x_rows < 1)) return TP_ERR_RANGE;
  if (n_rows == 0) return TP_OK;
  if (!x || !norm_w || !y_out) return TP_ERR_NULL;
  if (!aligned16(x) || !aligned16(norm_w) || !aligned16(y_out) || ((uintptr_t)rows & 3)) return TP_ERR_ALIGN;
  NormArgs a{nullptr, 0, 0, n_rows, cfg->hidden, static_cast<const bf16*>(x), static_cast<const bf16*>(norm_w),
             cfg->rms_eps, nullptr, static_cast<bf16*>(y_out), rows, rows ? x_rows : n_rows};
  return launched(residual_rmsnorm(a, static_cast<hipStream_t>(stream)));
}

int tp_last_token_rows(const int32_t* seq_lens, int32_t n_seqs, int32_t* rows_out) {
  if (n_seqs < 0) return TP_ERR_RANGE;
  if (n_seqs > 0 && (!seq_lens || !rows_out)) return TP_ERR_NULL;
  int64_t end = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    if (seq_lens[b] < 1) return TP_ERR_RANGE;
    end += seq_lens[b];
    if (end - 1 > INT32_MAX) return TP_ERR_SHAPE;
  }
  end = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    end += seq_lens[b];
    rows_out[b] = (int32_t)(end - 1);
  }
  return TP_OK;
}

int tp_sp_rows(const tp_cfg* cfg, int64_t M, int64_t* row0, int64_t* row1) {
  int st = check_cfg(cfg, nullptr);
  if (st) return st;
  if (!row0 || !row1) return TP_ERR_NULL;
  if (M < 0) return TP_ERR_RANGE;
  const int64_t per = (M + cfg->tp_size - 1) / cfg->tp_size;
  *row0 = std::min<int64_t>((int64_t)cfg->tp_rank * per, M);
  *row1 = std::min<int64_t>((int64_t)(cfg->tp_rank + 1) * per, M);
  return TP_OK;
}

int tp_sp_residual_rmsnorm(const tp_cfg* cfg, const void* partials, int64_t M, const void* residual_slice,
                           const void* norm_w, void* h_slice_out, void* y_gathered, void* stream) {
  int64_t r0 = 0, r1 = 0;
  int st = tp_sp_rows(cfg, M, &r0, &r1);
  if (st) return st;
  if (cfg->dtype != TP_BF16) return TP_ERR_DTYPE;
  if (cfg->hidden % 8 || cfg->hidden > 8192) return TP_ERR_SHAPE;
  if (r1 == r0) return TP_OK;   // no token on this rank: nothing to read or write
  if (!partials || !residual_slice || !norm_w || !h_slice_out || !y_gathered) return TP_ERR_NULL;
  const void* ptrs[] = {partials, residual_slice, norm_w, h_slice_out, y_gathered};
  for (const void* p : ptrs)
    if (!aligned16(p)) return TP_ERR_ALIGN;
  const int64_t H = cfg->hidden;
  NormArgs a{static_cast<const bf16*>(partials) + r0 * H, cfg->tp_size, M * H, r1 - r0, cfg->hidden,
             static_cast<const bf16*>(residual_slice), static_cast<const bf16*>(norm_w), cfg->rms_eps,
             static_cast<bf16*>(h_slice_out), static_cast<bf16*>(y_gathered) + r0 * H, nullptr, r1 - r0};
  return launched(residual_rmsnorm(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
