"""CPU oracle for one tensor-parallel rank's shard of a Qwen3-style decoder layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

Plain, slow, obviously-correct NumPy.  Arithmetic is float64 on the exact
values of the bf16 (or fp32) inputs; a tensor that the GPU path stores to
memory in bf16 is rounded to bf16 here at the same point (``store``), and
nowhere else.

Sources (web pages; sections named, not line numbers):
  [TPS]    "Tensor parallelism from scratch", ai-infra-handbooks (anrans):
           sections "Two ways to split", "Implementation" (tp.py: Column-/Row-
           ParallelLinear, VocabParallelEmbedding, TPAttention, TPMLP,
           TPTransformer), "KV heads and the limit on TP".
  [LEDGER] "8. How several ranks share one ledger", mini-SGLang code series
           (jaehun.me): section "Weights are cut by name" (_shard_tensor and
           the RowParallel forward).
  [CH9]    "Chapter 9 Multi-process and Tensor Parallelism", zero-to-sglang
           (datawhalechina): section 3.3 "Loading Weights and Model State"
           (shard-then-merge into qkv_proj / gate_up_proj, vocab layers).

Readings where the pages are silent (each also listed in the design notes):
  * RMSNorm is x / sqrt(mean(x^2) + eps) * w with eps = 1e-6 (the pages import
    RMSNorm without showing it).                        -- parity unpinned (eps)
  * RoPE is the rotate-half form: the pair (x[i], x[i + d/2]) is rotated by the
    angle pos * theta^(-2i/d); theta = 1e6.            -- parity unpinned (theta)
  * Attention scale is 1/sqrt(head_dim) (the SDPA default the pages rely on).
  * Merge order is qkv = [q; k; v] and gate_up = [gate; up] along dim 0.
  * A vocab shard whose start passes the vocab size is empty (start clamped).
  * Sequence parallelism cuts the tokens like the vocab: ceil(M / tp) rows per
    rank, in rank order, the last slices shorter or empty.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Weight kinds, in the order the shard rule table names them.
W_Q, W_K, W_V, W_O, W_GATE, W_UP, W_DOWN, W_VOCAB = range(8)


@dataclass(frozen=True)
class Cfg:
    """Model shape plus this rank's place in the tensor-parallel group."""
    hidden: int
    intermediate: int = 0
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 128
    vocab: int = 0
    tp_size: int = 1
    tp_rank: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6


@dataclass(frozen=True)
class Local:
    lq: int           # local q heads
    lkv: int          # local kv heads (1 when kv heads are replicated)
    kv_head0: int     # global index of the first local kv head
    li: int           # local intermediate size
    n_qkv: int        # rows of the merged local qkv weight
    vocab_start: int
    vocab_end: int


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def f32(x):
    """Round float64 values to the nearest float32 (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """Round to bfloat16 as a store does: to fp32 first, then round-to-
    nearest-even on the upper 16 bits of the fp32 pattern.  Returns float64."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    keep = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = (keep.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return out.astype(np.float64)


def bf16_bits(x):
    """The uint16 bit patterns of bf16(x)."""
    return (bf16(x).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# shard index maps   ([LEDGER] "Weights are cut by name"; [TPS] Implementation)
# --------------------------------------------------------------------------

def local_dims(c: Cfg) -> Local:
    """Per-rank sizes.  q heads and the intermediate size are cut evenly
    (a non-divisible head count is an error, [TPS] "KV heads and the limit on
    TP"); kv heads are cut evenly when there are at least as many as ranks,
    otherwise each rank keeps one whole kv head, head r*nkv//n ([LEDGER])."""
    n, r = c.tp_size, c.tp_rank
    if not (0 <= r < n):
        raise ValueError("rank out of range")
    if c.n_q_heads % n or c.intermediate % n:
        raise ValueError("heads / intermediate not divisible by tp")
    lq = c.n_q_heads // n
    if c.n_q_heads == 0 and c.n_kv_heads == 0:        # vocab-only / MLP-only shape
        lkv, kv0 = 0, 0
    elif c.n_kv_heads >= n:
        if c.n_kv_heads % n:
            raise ValueError("kv heads not divisible by tp")
        lkv, kv0 = c.n_kv_heads // n, r * (c.n_kv_heads // n)
    else:
        if c.n_kv_heads == 0 or n % c.n_kv_heads:
            raise ValueError("tp not a multiple of kv heads")
        lkv, kv0 = 1, r * c.n_kv_heads // n
    per = -(-c.vocab // n) if c.vocab else 0           # ceil(V / n)
    vs = min(r * per, c.vocab)
    ve = min((r + 1) * per, c.vocab)
    return Local(lq, lkv, kv0, c.intermediate // n, (lq + 2 * lkv) * c.head_dim, vs, ve)


def shard_rows(c: Cfg, kind: int):
    """(axis, start, stop) of the full [out, in] weight that rank r keeps."""
    L = local_dims(c)
    d, r = c.head_dim, c.tp_rank
    if kind == W_Q:
        return 0, r * L.lq * d, (r + 1) * L.lq * d
    if kind in (W_K, W_V):
        return 0, L.kv_head0 * d, (L.kv_head0 + L.lkv) * d
    if kind in (W_GATE, W_UP):
        return 0, r * L.li, (r + 1) * L.li
    if kind == W_O:
        return 1, r * L.lq * d, (r + 1) * L.lq * d
    if kind == W_DOWN:
        return 1, r * L.li, (r + 1) * L.li
    if kind == W_VOCAB:
        return 0, L.vocab_start, L.vocab_end
    raise ValueError(kind)


def shard(c: Cfg, kind: int, full):
    """Rank r's slice of one full weight (column split takes rows of the
    [out, in] matrix, row split takes columns)."""
    axis, a, b = shard_rows(c, kind)
    full = np.asarray(full)
    return full[a:b, :].copy() if axis == 0 else full[:, a:b].copy()


def merge_qkv(q, k, v):
    """Shard first, then merge: the rank's own q/k/v slices stacked."""
    return np.concatenate([q, k, v], axis=0)


def merge_gate_up(g, u):
    return np.concatenate([g, u], axis=0)


# --------------------------------------------------------------------------
# vocab-parallel embedding and lm head   ([TPS] Implementation; [CH9] 3.3)
# --------------------------------------------------------------------------

def embed_vocab(ids, table_local, vocab_start, vocab_end):
    """Rows of the local table for ids inside [start, end); +0.0 rows for
    every id outside it (including negative or >= vocab ids)."""
    ids = np.asarray(ids, dtype=np.int64)
    H = table_local.shape[1]
    out = np.zeros((ids.shape[0], H), dtype=table_local.dtype)
    for t, i in enumerate(ids):
        if vocab_start <= i < vocab_end:
            out[t] = table_local[i - vocab_start]
    return out


def lm_head(x, table_local, store=bf16, ft=np.float64):
    """Local slice of the logits: x @ table_local^T."""
    return store(np.asarray(x, ft) @ np.asarray(table_local, ft).T)


# Greedy decode over vocab-parallel logits ([TPS] Implementation: the next
# token is the argmax of the last position's logits after the all-gather of
# every rank's slice; argmax takes the first index of the maximum).  Per
# shard: the (max, first global index of it) of the local slice; the shards'
# candidates then combine to the max, ties going to the smaller global index,
# which is the first maximum of the concatenated logits.

def lm_head_argmax(x, table_local, vocab_start, store=bf16):
    """(values [M], global indices [M]) of this shard's local logits."""
    logits = lm_head(x, table_local, store)
    if logits.shape[1] == 0:
        return np.full(logits.shape[0], -np.inf), np.full(logits.shape[0], -1, np.int64)
    vals = np.empty(logits.shape[0])
    idx = np.empty(logits.shape[0], np.int64)
    for m in range(logits.shape[0]):
        best = 0
        for n in range(1, logits.shape[1]):
            if logits[m, n] > logits[m, best]:
                best = n
        vals[m], idx[m] = logits[m, best], vocab_start + best
    return vals, idx


# Last-token selection and the final norm before the head ([TPS]
# Implementation, TPTransformer.forward: the final RMSNorm runs on x[:, -1:],
# each sequence's last position; [CH9] 3.3, ParallelLMHead: in prefill only
# each sequence's last row reaches the vocab-split linear).  With sequences
# of different lengths packed one after another, sequence b's last row is
# the sum of the lengths up to and including b, minus one.

def last_token_rows(seq_lens):
    """Row of each sequence's last token in the packed [sum(lens), H] batch."""
    rows, end = [], 0
    for n in seq_lens:
        if n < 1:
            raise ValueError("a sequence has no token")
        end += int(n)
        rows.append(end - 1)
    return np.asarray(rows, np.int64)


def gather_rows(x, rows):
    """x[rows]; an index outside [0, len(x)) gives a zero row (the library
    reads such a row through a bounds-checked load as zeros)."""
    x = np.asarray(x)
    out = np.zeros((len(rows),) + x.shape[1:], x.dtype)
    for m, r in enumerate(rows):
        if 0 <= r < x.shape[0]:
            out[m] = x[r]
    return out


def rmsnorm_rows(x, rows, w, eps, store=bf16):
    """The final norm on the selected rows: store(rms_norm(x[rows]) * w)."""
    return store(rms_norm(gather_rows(x, rows), w, eps))


def argmax_combine(vals, idx):
    """vals, idx: [n_shards, M] candidates.  Per row the largest value; among
    equal values the smallest global index; shards with no vocabulary carry
    (-inf, -1) and never win."""
    vals = np.asarray(vals, np.float64)
    idx = np.asarray(idx, np.int64)
    out_v = np.empty(vals.shape[1])
    out_i = np.empty(vals.shape[1], np.int64)
    for m in range(vals.shape[1]):
        bv, bi = -np.inf, -1
        for r in range(vals.shape[0]):
            v, i = vals[r, m], idx[r, m]
            if i < 0:
                continue
            if bi < 0 or v > bv or (v == bv and i < bi):
                bv, bi = v, i
        out_v[m], out_i[m] = bv, bi
    return out_v, out_i


# --------------------------------------------------------------------------
# attention block pieces   ([TPS] Implementation, TPAttention.forward)
# --------------------------------------------------------------------------

def rms_norm(v, w, eps, ft=np.float64):
    """Normalise the last axis to unit RMS, then scale by w."""
    v = np.asarray(v, ft)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(w, ft)


def rope_angles(positions, head_dim, theta):
    """angle[p, i] = pos_p * theta^(-2i/d) for i < d/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]


def rope(v, positions, theta, ft=np.float64):
    """Rotate-half RoPE on the last axis; v is [rows, heads, d] and
    positions is [rows]."""
    v = np.asarray(v, ft)
    d = v.shape[-1]
    ang = rope_angles(positions, d, theta)[:, None, :]
    c, s = np.cos(ang).astype(ft), np.sin(ang).astype(ft)
    x1, x2 = v[..., : d // 2], v[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def q_heads(c: Cfg, x, w_qkv_local, q_norm_w, positions, store=bf16, ft=np.float64):
    """q part of the merged column-parallel projection: the rank's lq heads,
    QK-norm per head, then RoPE at each row's position; [rows, lq, d]."""
    L = local_dims(c)
    d = c.head_dim
    w = np.asarray(w_qkv_local, ft)[: L.lq * d]
    q = (np.asarray(x, ft) @ w.T).reshape(-1, L.lq, d)
    return store(rope(rms_norm(q, q_norm_w, c.rms_eps, ft), positions, c.rope_theta, ft))


def kv_heads(c: Cfg, x, w_qkv_local, k_norm_w, positions, store=bf16, ft=np.float64):
    """k and v parts of the merged projection: k gets QK-norm and RoPE, v
    neither; each [rows, lkv, d]."""
    L = local_dims(c)
    d = c.head_dim
    w = np.asarray(w_qkv_local, ft)
    x = np.asarray(x, ft)
    k = (x @ w[L.lq * d:(L.lq + L.lkv) * d].T).reshape(-1, L.lkv, d)
    v = (x @ w[(L.lq + L.lkv) * d:].T).reshape(-1, L.lkv, d)
    k = rope(rms_norm(k, k_norm_w, c.rms_eps, ft), positions, c.rope_theta, ft)
    return store(k), store(v)


def qkv_heads(c: Cfg, x, w_qkv_local, q_norm_w, k_norm_w, positions, store=bf16, ft=np.float64):
    """Merged column-parallel projection split into the rank's heads:
    stored (q, k, v) as [rows, heads, d]."""
    k, v = kv_heads(c, x, w_qkv_local, k_norm_w, positions, store, ft)
    return q_heads(c, x, w_qkv_local, q_norm_w, positions, store, ft), k, v


def attend(q_rows, q_pos, k_seq, v_seq, rep):
    """Causal GQA attention for a set of query rows of ONE sequence.

    q_rows [n, lq, d]; q_pos [n] absolute positions; k_seq/v_seq [lkv, S, d]
    hold the sequence's keys/values at positions 0..S-1.  Query head i reads
    kv head i // rep; query at position p sees keys 0..p.  Returns float64
    [n, lq, d] (unrounded)."""
    n, lq, d = q_rows.shape
    out = np.zeros((n, lq, d), q_rows.dtype)
    scale = 1.0 / math.sqrt(d)
    for a in range(n):
        p = int(q_pos[a])
        for i in range(lq):
            kk = k_seq[i // rep, : p + 1]
            vv = v_seq[i // rep, : p + 1]
            s = (kk @ q_rows[a, i]) * scale
            s = np.exp(s - s.max())
            out[a, i] = (s / s.sum()) @ vv
    return out


def qkv_attn(c: Cfg, x, B, T, past, w_qkv_local, q_norm_w, k_norm_w, w_o_local,
             k_cache, v_cache, store=bf16, ft=np.float64):
    """One call of the attention shard: B sequences with T new tokens each at
    positions past..past+T-1.  Writes k/v into copies of the caches
    [B, lkv, S_max, d] and returns dict(q, k_cache, v_cache, attn, partial),
    q/attn as [B*T, lq*d] and the row-parallel partial [B*T, H].
    ft: the arithmetic type (float64 for parity; float32 only to time the
    CPU baseline, whose store must then return float32 too)."""
    L = local_dims(c)
    d = c.head_dim
    rep = L.lq // L.lkv
    x = np.asarray(x, ft)
    pos = np.tile(np.arange(past, past + T), B)
    q, k, v = qkv_heads(c, x, w_qkv_local, q_norm_w, k_norm_w, pos, store, ft)
    kc = np.array(k_cache, dtype=ft, copy=True)
    vc = np.array(v_cache, dtype=ft, copy=True)
    attn = np.zeros((B * T, L.lq, d), ft)
    for b in range(B):
        rows = slice(b * T, (b + 1) * T)
        kc[b, :, past:past + T] = k[rows].transpose(1, 0, 2)
        vc[b, :, past:past + T] = v[rows].transpose(1, 0, 2)
        attn[rows] = attend(q[rows], pos[rows], kc[b, :, : past + T], vc[b, :, : past + T], rep)
    attn = store(attn.reshape(B * T, L.lq * d))
    partial = store(attn @ np.asarray(w_o_local, ft).T)
    return dict(q=q.reshape(B * T, L.lq * d), k_cache=kc, v_cache=vc, attn=attn, partial=partial)


# --------------------------------------------------------------------------
# residual add + RMSNorm after a row-parallel layer   ([TPS] Implementation,
# TPTransformer.forward: x = x + attn(input_layernorm(x)), then
# x = x + mlp(post_attention_layernorm(x)); each row-parallel output is the
# all-reduce (sum over ranks) of the ranks' partials; "The cost of
# communication": engines fuse that all-reduce with the following RMSNorm)
# --------------------------------------------------------------------------

def residual_rmsnorm(partials, residual, w, eps, store=bf16):
    """partials: [n, M, H] (one per rank), residual: [M, H], w: [H].
    h = store(residual + sum over ranks of partials)   the new residual stream
    y = store(rms_norm(h, w, eps))                     the next layer's input
    Returns (h, y)."""
    total = np.asarray(residual, np.float64).copy()
    for p in np.asarray(partials, np.float64):
        total = total + p
    h = store(total)
    return h, store(rms_norm(h, np.asarray(w, np.float64), eps))


# --------------------------------------------------------------------------
# sequence-parallel variant   ([TPS] "Exercises", the sequence-parallelism
# exercise: the all-reduce after o_proj / down becomes a reduce-scatter over
# tokens, so that each rank holds the full sum for its 1/tp of the tokens; the
# residual add and RMSNorm run on those rows only; an all-gather brings every
# token back before the next column-split layer)
# --------------------------------------------------------------------------

def sp_rows(M, n, r):
    """Rank r's token slice [start, end) of M rows: contiguous blocks of
    ceil(M / n) rows in rank order, the last ones shorter or empty (the pages
    do not say how a token count that tp does not divide is cut; this is the
    rule the vocab split uses)."""
    if not (0 <= r < n):
        raise ValueError("rank out of range")
    per = -(-M // n) if M else 0
    return min(r * per, M), min((r + 1) * per, M)


def reduce_scatter(partials, n, r):
    """Rank r's rows of the sum over ranks of the partials [n, M, H]."""
    partials = np.asarray(partials, np.float64)
    s, e = sp_rows(partials.shape[1], n, r)
    total = np.zeros((e - s,) + partials.shape[2:], np.float64)
    for p in partials:
        total = total + p[s:e]
    return total


def all_gather(slices):
    """The ranks' token slices, in rank order, back to all tokens."""
    return np.concatenate([np.asarray(t, np.float64) for t in slices], axis=0)


def sp_residual_rmsnorm(partials, residual_slice, w, eps, r, store=bf16):
    """partials: [n, M, H], every rank's partial over all M tokens (n = tp);
    residual_slice: rank r's rows of the residual stream, [end - start, H].
    h = store(residual_slice + reduce_scatter(partials))   this rank's rows
    y = store(rms_norm(h, w, eps))                          this rank's rows
    Returns (h, y); all_gather of every rank's y is the next layer's input."""
    partials = np.asarray(partials, np.float64)
    h = store(np.asarray(residual_slice, np.float64) + reduce_scatter(partials, partials.shape[0], r))
    return h, store(rms_norm(h, np.asarray(w, np.float64), eps))


# --------------------------------------------------------------------------
# MLP shard   ([TPS] Implementation, TPMLP.forward)
# --------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


def mlp(c: Cfg, x, w_gate_up_local, w_down_local, store=bf16, ft=np.float64):
    """h = silu(x Wg^T) * (x Wu^T) on the local intermediate slice, then the
    row-parallel partial h Wd^T.  Returns (h, partial), both stored."""
    li = local_dims(c).li
    x = np.asarray(x, ft)
    w = np.asarray(w_gate_up_local, ft)
    g = x @ w[:li].T
    u = x @ w[li:].T
    h = store(silu(g) * u)
    return h, store(h @ np.asarray(w_down_local, ft).T)


# --------------------------------------------------------------------------
# unsharded reference = the same maths at tp = 1
# --------------------------------------------------------------------------

def unsharded(c: Cfg) -> Cfg:
    return Cfg(c.hidden, c.intermediate, c.n_q_heads, c.n_kv_heads, c.head_dim, c.vocab,
               1, 0, c.rms_eps, c.rope_theta)


def with_rank(c: Cfg, r: int) -> Cfg:
    return Cfg(c.hidden, c.intermediate, c.n_q_heads, c.n_kv_heads, c.head_dim, c.vocab,
               c.tp_size, r, c.rms_eps, c.rope_theta)
