/*
 * tpshard.h -- C ABI of the tensor-parallel rank shard library (libtpshard.so).
 *
 * One tensor-parallel rank's shard of a Qwen3-style decoder layer on one
 * MI355X (gfx950):
 *   - the merged column-parallel QKV and gate_up projections,
 *   - SiLU(gate) * up,
 *   - the row-parallel o_proj / down_proj, which leave partial sums,
 *   - GQA attention over the rank's local heads (kv heads replicated when the
 *     tensor-parallel size exceeds the kv-head count),
 *   - the vocab-parallel masked embedding and the lm_head vocab slice,
 *   - the greedy decode head: per-shard (max, first id) candidates computed
 *     without storing the logits, and their combine across shards,
 *   - the residual add of the summed row-parallel partials with the next
 *     RMSNorm, and its sequence-parallel form on the rank's token slice.
 *
 * Sources (web pages; the section that defines each operation is cited at
 * each entry point):
 *   [TPS]    "Tensor parallelism from scratch" (ai-infra-handbooks):
 *            "Two ways to split", "Implementation", "KV heads and the limit
 *            on TP", "The cost of communication", "Exercises".
 *   [LEDGER] "8. How several ranks share one ledger" (mini-SGLang series):
 *            "Weights are cut by name".
 *   [CH9]    "Chapter 9 Multi-process and Tensor Parallelism"
 *            (zero-to-sglang): 3.3 "Loading Weights and Model State".
 *
 * Conventions for every entry point
 *   - All tensors are caller-owned, contiguous, row-major device memory
 *     (allocated with hipMalloc or by PyTorch).  The library allocates
 *     nothing; its only state is the per-thread timing marks of
 *     tp_kernel_marks (off unless armed); calls are re-entrant.
 *   - Weights use the [out, in] layout of a linear layer (the input dimension
 *     is contiguous).  Element type is cfg->dtype: TP_BF16 (bfloat16 bits)
 *     or TP_F32.
 *   - Every pointer argument must be 16-byte aligned (TP_ERR_ALIGN).
 *   - Arguments are validated on the host before anything is launched; on a
 *     non-zero return nothing has been written.  Row lengths of GEMM operands
 *     (hidden, the local intermediate, lq * head_dim) must be below 2^22
 *     elements and S_max below 2^24 (TP_ERR_SHAPE): the kernels address a
 *     tile or a cache slab through 32-bit buffer descriptors.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and runs
 *     asynchronously; TP_ERR_LAUNCH reports a failed launch.
 *   - Collectives are not part of the library: a row-parallel call returns
 *     the rank's partial sum, a column-parallel call the rank's slice.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = -1,      /* a required pointer is NULL                        */
  TP_ERR_RANK = -2,      /* tp_rank outside [0, tp_size) or tp_size < 1       */
  TP_ERR_SHAPE = -3,     /* heads / intermediate / vocab not splittable, or a
                            size the kernels do not support                   */
  TP_ERR_DTYPE = -4,     /* dtype not supported by this entry point           */
  TP_ERR_ALIGN = -5,     /* pointer not 16-byte aligned                       */
  TP_ERR_WORKSPACE = -6, /* workspace smaller than tp_workspace_bytes()       */
  TP_ERR_RANGE = -7,     /* negative size, or past_len + T > S_max            */
  TP_ERR_LAUNCH = -8,    /* a kernel launch failed                            */
  TP_ERR_KIND = -9       /* unknown tp_weight_kind / tp_op                    */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Weight names of the shard rule table ([LEDGER] "Weights are cut by name"). */
typedef enum {
  TP_W_Q = 0, TP_W_K = 1, TP_W_V = 2, TP_W_O = 3,
  TP_W_GATE = 4, TP_W_UP = 5, TP_W_DOWN = 6, TP_W_VOCAB = 7
} tp_weight_kind;

typedef enum { TP_OP_ATTN = 0, TP_OP_MLP = 1, TP_OP_LM_ARGMAX = 2 } tp_op;

/* Model shape and this rank's place in the group ([TPS] "Implementation":
 * every layer is built from the rank and the group size).  48 bytes. */
typedef struct {
  int32_t hidden;        /* H                                                 */
  int32_t intermediate;  /* I (full, unsharded)                               */
  int32_t n_q_heads;     /* full q-head count                                 */
  int32_t n_kv_heads;    /* full kv-head count                                */
  int32_t head_dim;      /* d                                                 */
  int32_t tp_size;       /* n                                                 */
  int32_t tp_rank;       /* r                                                 */
  int32_t dtype;         /* tp_dtype                                          */
  int64_t vocab;         /* V (full)                                          */
  float rms_eps;         /* QK-norm epsilon (Qwen3: 1e-6)                     */
  float rope_theta;      /* RoPE base (Qwen3: 1e6)                            */
} tp_cfg;

/* Per-rank sizes ([LEDGER] "Weights are cut by name"; [TPS] "KV heads and
 * the limit on TP"). */
typedef struct {
  int32_t lq;            /* local q heads = n_q_heads / n                     */
  int32_t lkv;           /* local kv heads = n_kv_heads / n, or 1 when
                            n_kv_heads < n (replicated)                        */
  int32_t kv_head0;      /* global index of the first local kv head:
                            r * lkv, or r * n_kv_heads / n when replicated     */
  int32_t li;            /* local intermediate = I / n                        */
  int64_t n_qkv;         /* rows of the merged local qkv weight (lq+2lkv)*d  */
  int64_t vocab_start;   /* local vocab rows [vocab_start, vocab_end):        */
  int64_t vocab_end;     /* per = ceil(V/n), [min(r*per,V), min((r+1)*per,V)) */
} tp_local;

/* ------------------------------------------------------------------------
 * Host-only helpers: no HIP calls, usable on a machine without a GPU.
 * ---------------------------------------------------------------------- */

/* Validates cfg and fills *out.  Rejected ([TPS] "KV heads and the limit on
 * TP": a head count that does not divide is an error):
 *   tp_rank outside [0, tp_size)                      -> TP_ERR_RANK
 *   n_q_heads % n, intermediate % n                   -> TP_ERR_SHAPE
 *   n_kv_heads >= n and n_kv_heads % n                -> TP_ERR_SHAPE
 *   n_kv_heads <  n and n % n_kv_heads                -> TP_ERR_SHAPE
 *   negative sizes, dtype not TP_F32/TP_BF16          -> TP_ERR_SHAPE / DTYPE
 * A shape with no heads (n_q_heads = n_kv_heads = 0) is valid for the MLP,
 * embedding and lm_head entry points. */
int tp_local_dims(const tp_cfg* cfg, tp_local* out);

/* Bytes of device workspace that tp_qkv_attn (op = TP_OP_ATTN), tp_mlp
 * (op = TP_OP_MLP) or tp_lm_head_argmax (op = TP_OP_LM_ARGMAX) needs for B
 * sequences of T new tokens after past_len cached ones (tp_mlp and
 * tp_lm_head_argmax: M = B * T rows; past_len ignored). */
int tp_workspace_bytes(const tp_cfg* cfg, int op, int64_t B, int64_t T, int64_t past_len,
                       size_t* out_bytes);

/* Static description of a status code. */
const char* tp_status_str(int status);

/* ------------------------------------------------------------------------
 * Per-kernel timing marks (instrumentation; host thread-local state)
 * ---------------------------------------------------------------------- */

/* tp_kernel_marks -- arms the calling host thread: the device entry points it
 * calls next record events[i] on the call's stream right after launching
 * their i-th kernel (counting across calls), for i < n_events; later kernels
 * are not marked.  events are hipEvent_t handles created by the caller (with
 * timing enabled) and must stay valid while armed; the array itself is
 * copied.  The time from an event the caller records before the first call
 * to mark 0, and from mark i-1 to mark i, is the stream time of each kernel
 * (launch gaps included).  events = NULL with n_events = 0 disarms.  Errors:
 * n_events < 0 -> TP_ERR_RANGE; events NULL with n_events > 0 -> TP_ERR_NULL. */
int tp_kernel_marks(void* const* events, int32_t n_events);

/* Marks recorded since the last tp_kernel_marks call on this thread. */
int32_t tp_kernel_marks_used(void);

/* Name of the kernel launched just before mark i on this thread, e.g.
 * "gemm_tile<256,256,2>/silu[4096x24576x5120]" (GEMM family: tile, stages,
 * epilogue and the launched M x N x K, N counting the rows of B) or
 * "attn_flash/decode"; "" when i is out of range.  Valid until the next
 * tp_kernel_marks call on this thread. */
const char* tp_kernel_mark_name(int32_t i);

/* ------------------------------------------------------------------------
 * Device entry points
 * ---------------------------------------------------------------------- */

/* tp_shard_weights -- copy rank r's shard of one full weight into its place
 * in the rank's local (merged) weight ([LEDGER] "Weights are cut by name":
 * the shard rule table; [CH9] 3.3: shard first, then merge q/k/v into
 * qkv_proj and gate/up into gate_up_proj).  A bit-exact copy.
 *   kind     full (unsharded, [out, in])   dst and the rows this call writes
 *   TP_W_Q     [nq*d,  H]  rows r*lq*d..    qkv [n_qkv, H], rows [0, lq*d)
 *   TP_W_K     [nkv*d, H]  kv heads         qkv, rows [lq*d, (lq+lkv)*d)
 *   TP_W_V     [nkv*d, H]  kv_head0..+lkv   qkv, rows [(lq+lkv)*d, n_qkv)
 *   TP_W_GATE  [I, H]      rows r*li..      gate_up [2*li, H], rows [0, li)
 *   TP_W_UP    [I, H]      rows r*li..      gate_up, rows [li, 2*li)
 *   TP_W_O     [H, nq*d]   cols r*lq*d..    o_local [H, lq*d] (whole)
 *   TP_W_DOWN  [H, I]      cols r*li..      down_local [H, li] (whole)
 *   TP_W_VOCAB [V, H]      rows vocab_start.. vocab_local [vocab_end-vocab_start, H]
 * When n_kv_heads < n the K/V shard is the single head kv_head0 (replica).
 * Elements are 2 (TP_BF16) or 4 (TP_F32) bytes. */
int tp_shard_weights(const tp_cfg* cfg, int kind, const void* full, void* dst, void* stream);

/* tp_embed_vocab -- vocab-parallel embedding lookup before its all-reduce
 * ([TPS] "Implementation", VocabParallelEmbedding; [CH9] 3.3 vocab layers):
 *   out[t, :] = vocab_local[ids[t] - vocab_start, :]  if vocab_start <= ids[t] < vocab_end
 *             = +0.0                                  otherwise (any id, incl. negative)
 * ids: int32 [n_tokens]; vocab_local: [vocab_end - vocab_start, H];
 * out: [n_tokens, H].  Bit-exact copy.  n_tokens = 0 is a no-op. */
int tp_embed_vocab(const tp_cfg* cfg, const int32_t* ids, int64_t n_tokens,
                   const void* vocab_local, void* out, void* stream);

/* tp_qkv_attn -- the attention half of the layer shard ([TPS]
 * "Implementation", TPAttention.forward; "Two ways to split"):
 *   qkv = x @ w_qkv^T            merged column-parallel projection
 *   q, k, v = split into lq, lkv, lkv heads of d
 *   q, k = RMSNorm_d(q) * q_norm_w, RMSNorm_d(k) * k_norm_w   (QK-norm)
 *   q, k = RoPE(q, pos), RoPE(k, pos)   rotate-half, pos = past_len + t
 *   cache[b, h, past_len + t, :] = k, v
 *   attn = softmax(q k^T / sqrt(d) + causal) v, q head i reads kv head i/rep
 *   out_partial = attn @ w_o^T   row-parallel partial (before its all-reduce)
 * Arguments:
 *   x          bf16 [B*T, H], the normed hidden states (row b*T + t)
 *   w_qkv      bf16 [n_qkv, H] merged local weight ([q; k; v])
 *   q_norm_w, k_norm_w  bf16 [d]
 *   w_o        bf16 [H, lq*d] local o_proj (column slice)
 *   k_cache, v_cache    bf16 [B, lkv, S_max, d]; positions < past_len are
 *              read, [past_len, past_len+T) written, the rest untouched
 *   q_out_opt  bf16 [B*T, lq*d] normed+rotated q, or NULL
 *   attn_out_opt bf16 [B*T, lq*d] attention output, or NULL
 *   out_partial  bf16 [B*T, H]
 *   workspace  >= tp_workspace_bytes(cfg, TP_OP_ATTN, B, T, past_len)
 * Requires dtype TP_BF16 (TP_ERR_DTYPE), head_dim == 128 and H % 8 == 0
 * (TP_ERR_SHAPE), past_len >= 0, past_len + T <= S_max (TP_ERR_RANGE).
 * B*T = 0 is a no-op. */
int tp_qkv_attn(const tp_cfg* cfg, const void* x, int32_t B, int32_t T, int32_t past_len,
                const void* w_qkv, const void* q_norm_w, const void* k_norm_w, const void* w_o,
                void* k_cache, void* v_cache, int32_t S_max,
                void* q_out_opt, void* attn_out_opt, void* out_partial,
                void* workspace, size_t ws_bytes, void* stream);

/* tp_mlp -- the MLP half of the layer shard ([TPS] "Implementation",
 * TPMLP.forward; "Two ways to split": gate/up column split, down row split):
 *   h = silu(x @ w_gate^T) * (x @ w_up^T),  silu(z) = z / (1 + exp(-z))
 *   out_partial = h @ w_down^T   (partial sum before the all-reduce)
 * x: [M, H]; w_gate_up: [2*li, H] merged ([gate; up]); w_down: [H, li];
 * h_opt: [M, li] or NULL; out_partial: [M, H].  TP_BF16 (fp32 accumulate,
 * bf16 stores) or TP_F32.  H and li must be multiples of 8 (TP_ERR_SHAPE).
 * workspace >= tp_workspace_bytes(cfg, TP_OP_MLP, M, 1, 0).  M = 0: no-op. */
int tp_mlp(const tp_cfg* cfg, const void* x, int64_t M, const void* w_gate_up,
           const void* w_down, void* h_opt, void* out_partial,
           void* workspace, size_t ws_bytes, void* stream);

/* tp_lm_head -- the rank's slice of the logits before the all-gather ([CH9]
 * 3.3 ParallelLMHead; [TPS] "Implementation", the vocab-split output layer,
 * tied to the embedding shard when the model ties them):
 *   logits_local[m] = x[row m] @ vocab_local^T,   m < M
 * Rows: with rows_opt NULL, row m of x (x: [M, H], x_rows ignored); with
 * rows_opt an int32 device array [M] of indices into x [x_rows, H], row
 * rows_opt[m] -- the head's last-token selection ([CH9] 3.3: in prefill
 * only each sequence's last row reaches the head; tp_last_token_rows gives
 * those indices).  An index outside [0, x_rows) reads as a zero row (its
 * logits are 0).  A row list needs TP_BF16 (TP_ERR_DTYPE), x_rows >= 1
 * (TP_ERR_RANGE), 4-byte alignment (TP_ERR_ALIGN) and x_rows * H * 2 < 2^31
 * (TP_ERR_SHAPE).  vocab_local: [vocab_end - vocab_start, H];
 * logits_local: [M, vocab_end - vocab_start].  M = 0: no-op. */
int tp_lm_head(const tp_cfg* cfg, const void* x, int64_t M, const int32_t* rows_opt, int64_t x_rows,
               const void* vocab_local, void* logits_local, void* stream);

/* tp_lm_head_argmax -- this rank's greedy candidate per row ([TPS]
 * "Implementation": decode takes the argmax of the last position's logits;
 * the vocab-split output layer gives each rank a slice of them).  Instead of
 * all-gathering V logits per row, the rank reduces its slice:
 *   logits = bf16(x @ vocab_local^T)            as tp_lm_head stores them
 *   out_val[m] = max_n logits[m, n]             (fp32 holding the bf16 value)
 *   out_idx[m] = vocab_start + first n attaining it (a global token id)
 * An empty vocab slice gives (-inf, -1).  The candidates of all ranks
 * (gathered into [n_shards, M]) combine with tp_argmax_combine.
 * x, rows_opt, x_rows: the rows of the head, as for tp_lm_head (x bf16).
 * vocab_local: bf16 [vocab_end - vocab_start, H];
 * out_val: float [M]; out_idx: int32 [M];
 * workspace >= tp_workspace_bytes(cfg, TP_OP_LM_ARGMAX, M, 1, 0), 16-byte
 * aligned: it holds 8-byte partial candidates (per row and logits tile, or per
 * row and workgroup when up to 64 rows with H <= 1024, H % 256 == 0 keep x
 * resident on chip); the logits themselves are never stored.  Requires
 * TP_BF16 (TP_ERR_DTYPE) and H % 8 == 0.  M = 0: no-op. */
int tp_lm_head_argmax(const tp_cfg* cfg, const void* x, int64_t M, const int32_t* rows_opt, int64_t x_rows,
                      const void* vocab_local, float* out_val, int32_t* out_idx, void* workspace, size_t ws_bytes,
                      void* stream);

/* tp_lm_head_argmax_noalloc -- tp_lm_head_argmax for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments and
 * results as tp_lm_head_argmax minus the workspace: the per-row partial
 * candidates go to a static device array of 4 MiB inside the library (one
 * per GPU, held until the process ends), so the call allocates nothing.
 * Limit: the candidates of M rows must fit it, i.e. the bytes
 * tp_workspace_bytes(cfg, TP_OP_LM_ARGMAX, M, 1, 0) reports must be at most
 * 4 MiB (TP_ERR_WORKSPACE otherwise; e.g. 64 rows on the on-chip path, or
 * 512 rows of a 75968-row vocab slice, fit).  The array is
 * looked up on the current device (hipGetDevice): `stream` must belong to
 * it.  Every call on one GPU shares that GPU's array, so calls that overlap
 * on one GPU (on different streams, or from several host threads) race;
 * calls on one stream are ordered and safe.  Nothing in the array needs
 * clearing: each call writes every slot it reads. */
int tp_lm_head_argmax_noalloc(const tp_cfg* cfg, const void* x, int64_t M, const int32_t* rows_opt, int64_t x_rows,
                              const void* vocab_local, float* out_val, int32_t* out_idx, void* stream);

/* tp_argmax_combine -- the cross-shard step of the greedy argmax: per row the
 * candidate with the largest value, ties to the smallest token id (the first
 * maximum of the concatenated logits, as argmax takes it); candidates with
 * idx < 0 (empty shards) never win.  vals: float [n_shards, M]; idx: int32
 * [n_shards, M] (each rank's tp_lm_head_argmax outputs, gathered); out_idx:
 * int32 [M]; out_val_opt: float [M] or NULL.  n_shards >= 1 (TP_ERR_RANGE).
 * Pointers 4-byte aligned (TP_ERR_ALIGN).  M = 0: no-op. */
int tp_argmax_combine(const float* vals, const int32_t* idx, int32_t n_shards, int64_t M,
                      int32_t* out_idx, float* out_val_opt, void* stream);

/* tp_residual_rmsnorm -- the replicated step after a row-parallel layer,
 * with its all-reduce ([TPS] "Implementation", TPTransformer.forward: the
 * residual add and the next RMSNorm; "The cost of communication": fusing the
 * all-reduce with the following RMSNorm):
 *   h = bf16(residual + sum_{r < n_partials} partials[r])   (fp32 sum in rank order)
 *   y = bf16(h / sqrt(mean(h^2) + rms_eps) * norm_w)
 * partials: bf16 [n_partials, M, H] (the ranks' tp_qkv_attn / tp_mlp
 * out_partial, stacked: on one GPU this stands in for the all-reduce);
 * residual, h_out, y_out: bf16 [M, H]; norm_w: bf16 [H].  h_out may be the
 * residual buffer (in-place update of the residual stream); y_out must not
 * overlap the inputs.  n_partials = 0 is the plain RMSNorm of the residual
 * (the final norm before the head; partials and h_out may then be NULL).
 * Requires TP_BF16 (TP_ERR_DTYPE), H % 8 == 0 and H <= 8192 (TP_ERR_SHAPE),
 * n_partials >= 0 (TP_ERR_RANGE).  M = 0: no-op. */
int tp_residual_rmsnorm(const tp_cfg* cfg, const void* partials, int32_t n_partials, int64_t M,
                        const void* residual, const void* norm_w, void* h_out, void* y_out, void* stream);

/* tp_rmsnorm_rows -- the final RMSNorm on selected rows before the head
 * ([TPS] "Implementation", TPTransformer.forward: norm(x[:, -1:]), each
 * sequence's last position):
 *   y[m] = bf16(x[i] / sqrt(mean(x[i]^2) + rms_eps) * norm_w),  m < n_rows,
 *   i = rows[m] (rows: int32 device array [n_rows]) or i = m (rows NULL,
 *   n_rows <= x_rows)
 * x: bf16 [x_rows, H]; norm_w: bf16 [H]; y_out: bf16 [n_rows, H].  An index
 * outside [0, x_rows) gives a zero row; a row list needs x_rows >= 1
 * (TP_ERR_RANGE).  Requires TP_BF16 (TP_ERR_DTYPE),
 * H % 8 == 0 and H <= 8192 (TP_ERR_SHAPE); rows 4-byte aligned.
 * n_rows = 0: no-op. */
int tp_rmsnorm_rows(const tp_cfg* cfg, const void* x, int64_t x_rows, const int32_t* rows, int64_t n_rows,
                    const void* norm_w, void* y_out, void* stream);

/* tp_last_token_rows -- host only, no HIP call: the row of each sequence's
 * last token in a batch of n_seqs sequences packed one after another
 * ([CH9] 3.3: the head keeps each sequence's last index; [TPS]
 * "Implementation": x[:, -1:]):  rows_out[b] = seq_lens[0] + ... +
 * seq_lens[b] - 1.  seq_lens, rows_out: host int32 arrays [n_seqs].  A
 * length < 1 or n_seqs < 0 -> TP_ERR_RANGE; a sum past 2^31 - 1 ->
 * TP_ERR_SHAPE. */
int tp_last_token_rows(const int32_t* seq_lens, int32_t n_seqs, int32_t* rows_out);

/* tp_sp_rows -- host only, no HIP call: rank tp_rank's token slice
 * [*row0, *row1) of M tokens under sequence parallelism ([TPS] "Exercises",
 * sequence parallelism: each rank keeps the full sum for 1/tp of the
 * tokens).  Contiguous blocks of ceil(M / tp_size) rows in rank order; the
 * last slices may be shorter or empty (the vocab split's rule; the pages do
 * not fix a token count that tp does not divide).  M < 0: TP_ERR_RANGE. */
int tp_sp_rows(const tp_cfg* cfg, int64_t M, int64_t* row0, int64_t* row1);

/* tp_sp_residual_rmsnorm -- the sequence-parallel form of
 * tp_residual_rmsnorm ([TPS] "Exercises", sequence parallelism: the
 * all-reduce after o_proj / down splits into a reduce-scatter over tokens,
 * the residual add and RMSNorm run on the rank's own tokens, and an
 * all-gather restores all tokens before the next column-split layer).  With
 * [row0, row1) = tp_sp_rows(cfg, M) and S = row1 - row0:
 *   reduce-scatter: rows [row0, row1) of sum_{r < tp_size} partials[r]
 *   h_slice = bf16(residual_slice + that)              (fp32, rank order)
 *   y       = bf16(h_slice / sqrt(mean(h^2) + rms_eps) * norm_w)
 *   all-gather: y is written to rows [row0, row1) of y_gathered.
 * partials: bf16 [tp_size, M, H], every rank's partial over all M tokens
 * (on one GPU this stands in for the reduce-scatter's inputs);
 * residual_slice, h_slice_out: bf16 [S, H] (this rank's rows of the residual
 * stream; h_slice_out may be residual_slice); norm_w: bf16 [H]; y_gathered:
 * bf16 [M, H], of which only this rank's rows are written (every rank
 * writing its rows into one buffer is the all-gather).  Requires TP_BF16
 * (TP_ERR_DTYPE), H % 8 == 0 and H <= 8192 (TP_ERR_SHAPE).  A rank whose
 * slice is empty returns TP_OK without reading or writing anything (its
 * pointers may then be NULL). */
int tp_sp_residual_rmsnorm(const tp_cfg* cfg, const void* partials, int64_t M, const void* residual_slice,
                           const void* norm_w, void* h_slice_out, void* y_gathered, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
