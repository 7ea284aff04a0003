"""Pins for the CPU oracle: each test ties it to something other than itself
(the pages' printed numbers, library routines, closed forms, brute force).
CPU only."""
import cmath
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _rand(seed, shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ---------------------------------------------------------------- bf16 store

def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 1e3)]).astype(np.float32)
    # exact ties and near-ties in the dropped half-word
    u = rng.integers(0x3000, 0x4F00, 2000).astype(np.uint32) << np.uint32(16)   # finite, |x| in ~[1e-10, 1e9]
    ties = np.concatenate([(u | 0x8000), (u | 0x7FFF), (u | 0x8001), (u | 0x18000)]).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0, 65504.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits(x), ref)
    assert np.array_equal(O.bf16(x), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- shard maps

QWEN06 = O.Cfg(hidden=1024, intermediate=3072, n_q_heads=16, n_kv_heads=8, head_dim=128,
               vocab=151936, tp_size=2)


def test_vocab_ranges_golden():
    for V, n, r, s, e in _golden_rows("vocab_ranges.txt"):
        L = O.local_dims(O.Cfg(hidden=8, vocab=int(V), tp_size=int(n), tp_rank=int(r)))
        assert (L.vocab_start, L.vocab_end) == (int(s), int(e)), (V, n, r)


def test_kv_replication_golden():
    for row in _golden_rows("kv_replication.txt"):
        nkv, n, heads = int(row[0]), int(row[1]), [int(h) for h in row[2:]]
        got = [O.local_dims(O.Cfg(hidden=8, n_q_heads=n, n_kv_heads=nkv, tp_size=n, tp_rank=r)).kv_head0
               for r in range(n)]
        assert got == heads


@pytest.mark.parametrize("n", [1, 2, 4])
def test_shard_matches_torch_chunk(n):
    """q/k/v/gate/up take dim-0 chunks, o/down take dim-1 chunks (the pages'
    chunk(n, dim)[r] rule when heads divide evenly)."""
    base = O.Cfg(hidden=32, intermediate=48, n_q_heads=8, n_kv_heads=4, head_dim=4, vocab=37, tp_size=n)
    full = {O.W_Q: (32, 32), O.W_K: (16, 32), O.W_V: (16, 32), O.W_O: (32, 32),
            O.W_GATE: (48, 32), O.W_UP: (48, 32), O.W_DOWN: (32, 48)}
    dim = {O.W_Q: 0, O.W_K: 0, O.W_V: 0, O.W_GATE: 0, O.W_UP: 0, O.W_O: 1, O.W_DOWN: 1}
    for kind, shape in full.items():
        w = torch.arange(shape[0] * shape[1], dtype=torch.float64).reshape(shape)
        for r in range(n):
            c = O.with_rank(base, r)
            ref = w.chunk(n, dim=dim[kind])[r].numpy()
            assert np.array_equal(O.shard(c, kind, w.numpy()), ref), (kind, r)


def test_replicated_kv_heads_are_gqa_consistent():
    """With fewer kv heads than ranks, the kv head a rank keeps is the one
    every one of its global q heads reads under GQA (q head h -> kv head
    h // (nq / nkv))."""
    for nq, nkv, n in [(64, 8, 16), (8, 2, 4), (4, 1, 4), (16, 8, 16)]:
        for r in range(n):
            c = O.Cfg(hidden=8, n_q_heads=nq, n_kv_heads=nkv, head_dim=4, tp_size=n, tp_rank=r)
            L = O.local_dims(c)
            for h in range(r * L.lq, (r + 1) * L.lq):
                assert h // (nq // nkv) == L.kv_head0 + (h - r * L.lq) // (L.lq // L.lkv)


def test_rejects_non_divisible():
    with pytest.raises(ValueError):
        O.local_dims(O.Cfg(hidden=8, n_q_heads=28, n_kv_heads=4, tp_size=8))   # 28 q heads, TP 8
    with pytest.raises(ValueError):
        O.local_dims(O.Cfg(hidden=8, n_q_heads=12, n_kv_heads=4, tp_size=6))   # 4 kv < 6 ranks, 6 % 4 != 0
    with pytest.raises(ValueError):
        O.local_dims(O.Cfg(hidden=8, intermediate=10, n_q_heads=4, n_kv_heads=4, tp_size=4))  # 10 % 4
    assert O.local_dims(O.Cfg(hidden=8, n_q_heads=12, n_kv_heads=3, tp_size=6)).lkv == 1  # legal replication
    with pytest.raises(ValueError):
        O.local_dims(O.Cfg(hidden=8, n_q_heads=16, n_kv_heads=6, tp_size=4))   # 6 % 4
    with pytest.raises(ValueError):
        O.local_dims(O.Cfg(hidden=8, n_q_heads=2, n_kv_heads=2, tp_size=2, tp_rank=2))


def test_pages_printed_parameter_counts():
    """Qwen3-0.6B at TP=2: per-rank and full parameter counts, kv heads per
    rank, all-reduces per prefill, as printed by the pages' run."""
    g = {k: int(v) for k, v in _golden_rows("pages_printed_numbers.txt")}
    layers = g["layers"]

    def count(c):
        L = O.local_dims(c)
        H, d = c.hidden, c.head_dim
        n = 0
        for kind, (rows, cols) in {O.W_Q: (c.n_q_heads * d, H), O.W_K: (c.n_kv_heads * d, H),
                                   O.W_V: (c.n_kv_heads * d, H), O.W_O: (H, c.n_q_heads * d),
                                   O.W_GATE: (c.intermediate, H), O.W_UP: (c.intermediate, H),
                                   O.W_DOWN: (H, c.intermediate)}.items():
            axis, a, b = O.shard_rows(c, kind)
            n += (b - a) * (cols if axis == 0 else rows)
        n += 2 * H + 2 * d                     # input/post-attn norms, q/k norms: replicated
        n = n * layers
        n += (L.vocab_end - L.vocab_start) * H  # tied embedding / lm head
        n += H                                 # final norm
        return n, L

    full, _ = count(O.unsharded(QWEN06))
    per, L = count(QWEN06)
    assert round(full / 1e6) == g["params_full_millions"]
    assert round(per / 1e6) == g["params_per_rank_millions"]
    assert L.lkv == g["kv_heads_per_rank"] and QWEN06.n_kv_heads == g["kv_heads_total"]
    assert 2 * layers + 1 == g["all_reduces_per_prefill"]


# ---------------------------------------------------------------- embedding

@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_vocab_sum_identity(n):
    V, H = 37, 8
    E = O.bf16(_rand(1, (V, H), 0.02))
    ids = np.concatenate([np.random.default_rng(2).integers(0, V, 50), [0, V - 1, V, V + 5, -1, -V]])
    total = np.zeros((len(ids), H))
    for r in range(n):
        c = O.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = O.local_dims(c)
        part = O.embed_vocab(ids, O.shard(c, O.W_VOCAB, E), L.vocab_start, L.vocab_end)
        # every in-vocab id is served by exactly one rank, and rows are copies
        total += part
    valid = (ids >= 0) & (ids < V)
    assert np.array_equal(total[valid], E[ids[valid]])
    assert np.all(total[~valid] == 0.0)
    assert np.array_equal(total[valid], torch.nn.functional.embedding(
        torch.from_numpy(ids[valid]), torch.from_numpy(E)).numpy())


# ---------------------------------------------------------------- RoPE / RMSNorm conventions

def test_rope_and_rmsnorm_match_qwen3_library():
    """Rotate-half RoPE with inv_freq = theta^(-2i/d) and RMSNorm as in the
    Qwen3 model code (the pages run Qwen3-0.6B but do not print either)."""
    from transformers.models.qwen3 import configuration_qwen3, modeling_qwen3 as m
    d, theta = 128, 1e6
    cfg = configuration_qwen3.Qwen3Config(head_dim=d, hidden_size=1024, num_attention_heads=8,
                                          rope_parameters={"rope_type": "default", "rope_theta": theta})
    emb = m.Qwen3RotaryEmbedding(cfg)
    pos = torch.tensor([[0, 1, 7, 100, 1023, 4095]])
    x = torch.from_numpy(_rand(3, (1, 2, 6, d))).float()
    cos, sin = emb(x, pos)
    ref, _ = m.apply_rotary_pos_emb(x, x, cos, sin)
    got = O.rope(x[0].permute(1, 0, 2).double().numpy(), pos[0].numpy(), theta)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).double().numpy(), atol=2e-3, rtol=0)
    norm = m.Qwen3RMSNorm(d, eps=1e-6)
    with torch.no_grad():
        norm.weight.copy_(torch.linspace(0.5, 1.5, d))
    got = O.rms_norm(x.double().numpy(), norm.weight.detach().double().numpy(), 1e-6)
    np.testing.assert_allclose(got, norm(x).detach().double().numpy(), rtol=1e-5, atol=1e-6)


def test_rope_special_cases():
    d = 16
    v = _rand(4, (3, 2, d))
    assert np.allclose(O.rope(v, np.zeros(3), 1e6), v, atol=0, rtol=1e-15)      # position 0: identity
    q, k = _rand(5, (1, 1, d)), _rand(6, (1, 1, d))
    dots = []
    for m_, n_ in [(3, 1), (10, 8), (1002, 1000)]:           # same offset m - n = 2
        a = O.rope(q, np.array([m_]), 1e4)[0, 0]
        b = O.rope(k, np.array([n_]), 1e4)[0, 0]
        dots.append(a @ b)
    assert np.allclose(dots, dots[0], rtol=1e-9)
    # norm preserved (a rotation)
    r = O.rope(v, np.array([5, 77, 3000]), 1e6)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-12)


def test_rmsnorm_unit_rms_and_silu():
    v = _rand(7, (5, 3, 64)) * 7.0
    y = O.rms_norm(v, np.ones(64), 1e-12)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-9)
    z = torch.from_numpy(_rand(8, (1000,)) * 5)
    assert np.allclose(O.silu(z.numpy()), torch.nn.functional.silu(z).numpy(), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- attention special cases

def test_attention_special_cases():
    d = 8
    q = _rand(9, (1, 2, d))
    k = _rand(10, (1, 1, d))
    v = _rand(11, (1, 1, d))
    # one key: output is that key's value
    out = O.attend(q, np.array([0]), k, v, rep=2)
    assert np.allclose(out[0, 0], v[0, 0]) and np.allclose(out[0, 1], v[0, 0])
    # all keys equal: output is the mean of the values
    S = 6
    kk = np.repeat(_rand(12, (1, 1, d)), S, axis=1)
    vv = _rand(13, (1, S, d))
    out = O.attend(q, np.array([S - 1]), kk, vv, rep=2)
    assert np.allclose(out[0, 0], vv[0].mean(axis=0), rtol=1e-12)
    # causal: a query at position p ignores keys after p
    vv2 = vv.copy()
    vv2[0, 3:] = 1e6
    assert np.allclose(O.attend(q, np.array([2]), kk, vv2, 2), O.attend(q, np.array([2]), kk, vv, 2))


def test_attention_matches_torch_sdpa_with_pages_mask():
    """torch's SDPA (CPU, fp64) with the pages' mask ones(T,S).tril(S-T) and
    kv heads expanded by repeat_interleave."""
    B, lq, lkv, d, past, T = 2, 4, 2, 16, 5, 3
    S = past + T
    q = _rand(14, (B * T, lq, d))
    kc = _rand(15, (B, lkv, S, d))
    vc = _rand(16, (B, lkv, S, d))
    pos = np.tile(np.arange(past, S), B)
    mask = torch.ones(T, S, dtype=torch.bool).tril(diagonal=S - T)
    for b in range(B):
        got = O.attend(q[b * T:(b + 1) * T], pos[b * T:(b + 1) * T], kc[b], vc[b], lq // lkv)
        tq = torch.from_numpy(q[b * T:(b + 1) * T]).permute(1, 0, 2)[None]
        tk = torch.from_numpy(kc[b])[None].repeat_interleave(lq // lkv, dim=1)
        tv = torch.from_numpy(vc[b])[None].repeat_interleave(lq // lkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- tp identities

TINY = O.Cfg(hidden=64, intermediate=96, n_q_heads=8, n_kv_heads=4, head_dim=16, vocab=0,
             rms_eps=1e-6, rope_theta=1e4)


def _tiny_full(seed=20, c=TINY):
    d, H = c.head_dim, c.hidden
    return dict(q=O.bf16(_rand(seed, (c.n_q_heads * d, H), 0.1)),
                k=O.bf16(_rand(seed + 1, (c.n_kv_heads * d, H), 0.1)),
                v=O.bf16(_rand(seed + 2, (c.n_kv_heads * d, H), 0.1)),
                o=O.bf16(_rand(seed + 3, (H, c.n_q_heads * d), 0.1)),
                gate=O.bf16(_rand(seed + 4, (c.intermediate, H), 0.1)),
                up=O.bf16(_rand(seed + 5, (c.intermediate, H), 0.1)),
                down=O.bf16(_rand(seed + 6, (H, c.intermediate), 0.1)),
                qn=O.bf16(np.random.default_rng(seed + 7).uniform(0.5, 1.5, d)),
                kn=O.bf16(np.random.default_rng(seed + 8).uniform(0.5, 1.5, d)))


def _rank_weights(c, W):
    qkv = O.merge_qkv(O.shard(c, O.W_Q, W["q"]), O.shard(c, O.W_K, W["k"]), O.shard(c, O.W_V, W["v"]))
    gu = O.merge_gate_up(O.shard(c, O.W_GATE, W["gate"]), O.shard(c, O.W_UP, W["up"]))
    return qkv, O.shard(c, O.W_O, W["o"]), gu, O.shard(c, O.W_DOWN, W["down"])


def _run_attn(c, W, x, B, T, past, prior_k, prior_v, store):
    """prior_k / prior_v: [B, n_kv_heads(global), past, d] cache contents."""
    L = O.local_dims(c)
    qkv, wo, _, _ = _rank_weights(c, W)
    S_max = past + T + 2
    kc = np.zeros((B, L.lkv, S_max, c.head_dim))
    vc = np.zeros_like(kc)
    kc[:, :, :past] = prior_k[:, L.kv_head0:L.kv_head0 + L.lkv]
    vc[:, :, :past] = prior_v[:, L.kv_head0:L.kv_head0 + L.lkv]
    return O.qkv_attn(c, x, B, T, past, qkv, W["qn"], W["kn"], wo, kc, vc, store=store)


def _ident(v):
    return np.asarray(v, np.float64)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_column_concat_and_row_sum_identities(n):
    """Column shards concatenate to the unsharded output; row-parallel
    partials sum to it ("Two ways to split").  n = 8 > 4 kv heads exercises
    replication."""
    c1 = TINY
    W = _tiny_full()
    B, T, past = 2, 3, 4
    x = O.bf16(_rand(30, (B * T, c1.hidden)))
    pk = O.bf16(_rand(31, (B, c1.n_kv_heads, past, c1.head_dim)))
    pv = O.bf16(_rand(32, (B, c1.n_kv_heads, past, c1.head_dim)))
    full = _run_attn(c1, W, x, B, T, past, pk, pv, _ident)
    _, _, gu1, wd1 = _rank_weights(c1, W)
    h1, p1 = O.mlp(c1, x, gu1, wd1, store=_ident)
    psum = np.zeros_like(full["partial"])
    msum = np.zeros_like(p1)
    hs, qs, attn = [], [], []
    cn = O.Cfg(**{**c1.__dict__, "tp_size": n})
    for r in range(n):
        c = O.with_rank(cn, r)
        L = O.local_dims(c)
        res = _run_attn(c, W, x, B, T, past, pk, pv, _ident)
        psum += res["partial"]
        qs.append(res["q"])
        attn.append(res["attn"])
        # the rank's cache holds exactly the unsharded cache's kv heads
        assert np.allclose(res["k_cache"], full["k_cache"][:, L.kv_head0:L.kv_head0 + L.lkv], rtol=1e-12, atol=1e-13)
        _, _, gu, wd = _rank_weights(c, W)
        h, p = O.mlp(c, x, gu, wd, store=_ident)
        hs.append(h)
        msum += p
    np.testing.assert_allclose(np.concatenate(qs, 1), full["q"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(attn, 1), full["attn"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(hs, 1), h1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(psum, full["partial"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(msum, p1, rtol=1e-10, atol=1e-12)


def test_replica_ranks_bit_identical():
    """Ranks sharing one replicated kv head write bit-identical caches."""
    W = _tiny_full()
    B, T, past = 1, 4, 2
    x = O.bf16(_rand(40, (B * T, TINY.hidden)))
    pk = O.bf16(_rand(41, (B, TINY.n_kv_heads, past, TINY.head_dim)))
    pv = O.bf16(_rand(42, (B, TINY.n_kv_heads, past, TINY.head_dim)))
    cn = O.Cfg(**{**TINY.__dict__, "tp_size": 8})   # 4 kv heads over 8 ranks
    res = [_run_attn(O.with_rank(cn, r), W, x, B, T, past, pk, pv, O.bf16) for r in range(8)]
    for j in range(4):
        a, b = res[2 * j], res[2 * j + 1]
        assert np.array_equal(a["k_cache"], b["k_cache"]) and np.array_equal(a["v_cache"], b["v_cache"])
    assert not np.array_equal(res[0]["k_cache"], res[2]["k_cache"])


# ---------------------------------------------------------------- brute force

def _bf_layer(c, W, x, B, T, past, pk, pv):
    """Unsharded attention block + MLP written with scalar Python loops;
    RoPE via complex rotation of the pair (x_i, x_{i+d/2})."""
    H, d, nq, nkv, I = c.hidden, c.head_dim, c.n_q_heads, c.n_kv_heads, c.intermediate
    rows = B * T

    def lin(vec, w):
        return [sum(vec[k] * w[o][k] for k in range(len(vec))) for o in range(len(w))]

    def norm_rope(vec, wn, p):
        ss = sum(t * t for t in vec) / d
        inv = 1.0 / math.sqrt(ss + c.rms_eps)
        vec = [vec[i] * inv * wn[i] for i in range(d)]
        out = [0.0] * d
        for i in range(d // 2):
            z = complex(vec[i], vec[i + d // 2]) * cmath.exp(1j * p * c.rope_theta ** (-2 * i / d))
            out[i], out[i + d // 2] = z.real, z.imag
        return out

    Wq, Wk, Wv, Wo = W["q"].tolist(), W["k"].tolist(), W["v"].tolist(), W["o"].tolist()
    qn, kn = W["qn"].tolist(), W["kn"].tolist()
    keys = [[[list(pk[b, h, s]) for s in range(past)] for h in range(nkv)] for b in range(B)]
    vals = [[[list(pv[b, h, s]) for s in range(past)] for h in range(nkv)] for b in range(B)]
    qrows = []
    for rrow in range(rows):
        b, t = divmod(rrow, T)
        xr = list(x[rrow])
        qf, kf, vf = lin(xr, Wq), lin(xr, Wk), lin(xr, Wv)
        qrows.append([norm_rope(qf[h * d:(h + 1) * d], qn, past + t) for h in range(nq)])
        for h in range(nkv):
            keys[b][h].append(norm_rope(kf[h * d:(h + 1) * d], kn, past + t))
            vals[b][h].append(vf[h * d:(h + 1) * d])
    attn_out, partial = [], []
    for rrow in range(rows):
        b, t = divmod(rrow, T)
        cat = []
        for h in range(nq):
            g = h // (nq // nkv)
            sc = [sum(qrows[rrow][h][i] * keys[b][g][s][i] for i in range(d)) / math.sqrt(d)
                  for s in range(past + t + 1)]
            m = max(sc)
            e = [math.exp(v - m) for v in sc]
            z = sum(e)
            cat += [sum(e[s] / z * vals[b][g][s][i] for s in range(len(e))) for i in range(d)]
        attn_out.append(cat)
        partial.append(lin(cat, Wo))
    Wg, Wu, Wd = W["gate"].tolist(), W["up"].tolist(), W["down"].tolist()
    mlp_out = []
    for rrow in range(rows):
        xr = list(x[rrow])
        g, u = lin(xr, Wg), lin(xr, Wu)
        h = [g[j] / (1 + math.exp(-g[j])) * u[j] for j in range(I)]
        mlp_out.append(lin(h, Wd))
    return np.array(attn_out), np.array(partial), np.array(mlp_out)


def test_brute_force_tiny_layer():
    """The sharded oracle at tp 1, 2, 4 (4 replicates kv heads when
    n_kv = 2) against scalar loops of the unsharded layer."""
    c1 = O.Cfg(hidden=24, intermediate=16, n_q_heads=4, n_kv_heads=2, head_dim=8, rms_eps=1e-6, rope_theta=1e4)
    W = _tiny_full(50, c1)
    B, T, past = 1, 5, 3
    x = O.bf16(_rand(60, (B * T, c1.hidden)))
    pk = O.bf16(_rand(61, (B, 2, past, 8)))
    pv = O.bf16(_rand(62, (B, 2, past, 8)))
    a_bf, p_bf, m_bf = _bf_layer(c1, W, x, B, T, past, pk, pv)
    for n in (1, 2, 4):
        cn = O.Cfg(**{**c1.__dict__, "tp_size": n})
        attn, psum, msum = [], 0.0, 0.0
        for r in range(n):
            c = O.with_rank(cn, r)
            res = _run_attn(c, W, x, B, T, past, pk, pv, _ident)
            attn.append(res["attn"])
            psum = psum + res["partial"]
            _, _, gu, wd = _rank_weights(c, W)
            msum = msum + O.mlp(c, x, gu, wd, store=_ident)[1]
        np.testing.assert_allclose(np.concatenate(attn, 1), a_bf, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(psum, p_bf, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(msum, m_bf, rtol=1e-10, atol=1e-12)


def test_lm_head_matches_linear_and_concats():
    V, H, n = 29, 16, 3
    E = O.bf16(_rand(70, (V, H), 0.02))
    x = O.bf16(_rand(71, (5, H)))
    parts = []
    for r in range(n):
        c = O.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        parts.append(O.lm_head(x, O.shard(c, O.W_VOCAB, E), store=_ident))
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(E)).numpy()
    np.testing.assert_allclose(np.concatenate(parts, 1), ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------ greedy argmax over shards

def _sharded_argmax(x, E, V, H, n):
    vals, idx = [], []
    for r in range(n):
        c = O.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = O.local_dims(c)
        v, i = O.lm_head_argmax(x, O.shard(c, O.W_VOCAB, E), L.vocab_start)
        vals.append(v)
        idx.append(i)
    return O.argmax_combine(np.stack(vals), np.stack(idx))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_sharded_argmax_equals_torch_argmax_of_gathered_logits(n):
    """Per-shard (max, first index) plus the combine equals torch.argmax over
    the all-gathered, bf16-stored logits (uneven last shard at n = 3, 8)."""
    V, H, M = 1000, 64, 12
    E = O.bf16(_rand(80, (V, H), 0.02))
    x = O.bf16(_rand(81, (M, H)))
    v, i = _sharded_argmax(x, E, V, H, n)
    full = torch.from_numpy(O.bf16(x @ E.T))
    ref_v, ref_i = full.max(dim=1)
    assert np.array_equal(i, torch.argmax(full, dim=1).numpy())
    assert np.array_equal(i, ref_i.numpy())
    np.testing.assert_array_equal(v, ref_v.numpy())


@pytest.mark.parametrize("n", [2, 4])
def test_sharded_argmax_ties_go_to_the_first_index(n):
    """Planted ties across and inside shards: the winner is the smallest
    global index holding the maximum (torch.argmax and a plain scan agree)."""
    V, H, M = 40, 8, 6
    rng = np.random.default_rng(82)
    E = O.bf16(rng.standard_normal((V, H)) * 0.1)
    for dup in (3, 17, 18, 31, 39):       # identical rows in several shards
        E[dup] = E[25]
    x = O.bf16(rng.standard_normal((M, H)))
    x[0] = 0.0                            # every logit 0: index 0 wins
    E[:, :] = np.where(np.arange(V)[:, None] == 7, E[25], E)    # one more copy
    v, i = _sharded_argmax(x, E, V, H, n)
    logits = O.bf16(x @ E.T)
    for m in range(M):
        best = 0
        for k in range(V):
            if logits[m, k] > logits[m, best]:
                best = k
        assert i[m] == best and v[m] == logits[m, best]
    assert i[0] == 0
    assert np.array_equal(i, torch.argmax(torch.from_numpy(logits), dim=1).numpy())


def test_argmax_combine_skips_empty_shards():
    """V = 5 over 4 ranks leaves the last shard empty; it never wins."""
    V, H, n = 5, 4, 4
    E = O.bf16(_rand(83, (V, H)))
    x = O.bf16(_rand(84, (3, H)))
    v, i = _sharded_argmax(x, E, V, H, n)
    assert np.array_equal(i, np.argmax(O.bf16(x @ E.T), axis=1))


# ------------------------------------------- residual + RMSNorm after the sum

def test_residual_rmsnorm_matches_torch_sum_and_rms_norm():
    """The fused step equals: sum the ranks' partials (the all-reduce), add
    the residual, store bf16, then torch's rms_norm with the weight."""
    n, M, H, eps = 3, 5, 96, 1e-6
    P = O.bf16(_rand(90, (n, M, H)))
    res = O.bf16(_rand(91, (M, H)))
    w = O.bf16(np.random.default_rng(92).uniform(0.5, 1.5, H))
    h, y = O.residual_rmsnorm(P, res, w, eps)
    ht = (torch.from_numpy(res) + torch.from_numpy(P).sum(0)).to(torch.bfloat16)
    yt = torch.nn.functional.rms_norm(ht.double(), (H,), torch.from_numpy(w), eps).to(torch.bfloat16)
    np.testing.assert_array_equal(h, ht.double().numpy())
    np.testing.assert_array_equal(y, yt.double().numpy())


def test_residual_rmsnorm_special_cases():
    """One rank with a zero partial is plain RMSNorm of the residual; with
    unit weights every output row has unit RMS (before the bf16 store)."""
    M, H, eps = 4, 64, 1e-6
    res = O.bf16(_rand(93, (M, H)))
    w = np.ones(H)
    h, y = O.residual_rmsnorm(np.zeros((1, M, H)), res, w, eps, store=lambda v: np.asarray(v, np.float64))
    np.testing.assert_array_equal(h, res)
    np.testing.assert_allclose(np.sqrt((y * y).mean(1)), 1.0, rtol=1e-6)
    np.testing.assert_allclose(y, res / np.sqrt((res * res).mean(1, keepdims=True) + eps), rtol=1e-12)


@pytest.mark.parametrize("M,n", [(0, 2), (1, 2), (7, 2), (8, 4), (9, 4), (5, 8), (4096, 2), (1023, 16)])
def test_sp_rows_match_torch_chunk(M, n):
    """The token slices are torch.chunk's pieces in rank order (ranks past the
    pieces torch returns get empty slices): contiguous, disjoint, covering."""
    rows = torch.arange(M)
    pieces = torch.chunk(rows, n) if M else ()
    end = 0
    for r in range(n):
        s, e = O.sp_rows(M, n, r)
        assert s == end and s <= e
        got = rows[s:e]
        want = pieces[r] if r < len(pieces) else rows[:0]
        assert torch.equal(got, want), (M, n, r)
        end = e
    assert end == M


def test_reduce_scatter_then_all_gather_is_all_reduce():
    """Reduce-scatter + all-gather equals the all-reduce (torch's sum over
    ranks), for a token count that tp does not divide."""
    n, M, H = 3, 10, 24
    P = _rand(94, (n, M, H))
    got = O.all_gather([O.reduce_scatter(P, n, r) for r in range(n)])
    np.testing.assert_array_equal(got, torch.from_numpy(P).sum(0).numpy())
    s, e = O.sp_rows(M, n, 1)
    assert O.reduce_scatter(P, n, 1).shape == (e - s, H)


@pytest.mark.parametrize("M,n", [(6, 2), (7, 4), (3, 4)])
def test_sp_residual_rmsnorm_gathers_to_torch(M, n):
    """Every rank normalises only its own rows; the gathered result equals
    torch's sum + rms_norm over all tokens (and the non-sequence-parallel
    fused step), including ranks that own no token."""
    H, eps = 64, 1e-6
    P = O.bf16(_rand(95, (n, M, H)))
    res = O.bf16(_rand(96, (M, H)))
    w = O.bf16(np.random.default_rng(97).uniform(0.5, 1.5, H))
    hs, ys = [], []
    for r in range(n):
        s, e = O.sp_rows(M, n, r)
        h, y = O.sp_residual_rmsnorm(P, res[s:e], w, eps, r)
        assert h.shape == y.shape == (e - s, H)
        hs.append(h)
        ys.append(y)
    ht = (torch.from_numpy(res) + torch.from_numpy(P).sum(0)).to(torch.bfloat16)
    yt = torch.nn.functional.rms_norm(ht.double(), (H,), torch.from_numpy(w), eps).to(torch.bfloat16)
    np.testing.assert_array_equal(O.all_gather(hs), ht.double().numpy())
    np.testing.assert_array_equal(O.all_gather(ys), yt.double().numpy())
    h_full, y_full = O.residual_rmsnorm(P, res, w, eps)
    np.testing.assert_array_equal(O.all_gather(ys), y_full)


def test_float32_variant_tracks_float64():
    """The float32 variant (used only to time the CPU baseline) computes the
    same maths: without storage rounding it stays within float32 rounding of
    the float64 oracle, and with bf16 stores within one bf16 step."""
    c = O.Cfg(**{**TINY.__dict__, "tp_size": 2, "tp_rank": 1})
    W = _tiny_full()
    L = O.local_dims(c)
    B, T, past = 2, 3, 4
    x = O.bf16(_rand(40, (B * T, c.hidden)))
    pk = O.bf16(_rand(41, (B, c.n_kv_heads, past, c.head_dim)))
    pv = O.bf16(_rand(42, (B, c.n_kv_heads, past, c.head_dim)))
    qkv, wo, gu, wd = _rank_weights(c, W)
    S_max = past + T + 2
    kc = np.zeros((B, L.lkv, S_max, c.head_dim))
    vc = np.zeros_like(kc)
    kc[:, :, :past] = pk[:, L.kv_head0:L.kv_head0 + L.lkv]
    vc[:, :, :past] = pv[:, L.kv_head0:L.kv_head0 + L.lkv]
    f32 = np.float32
    for store64, store32, tol in ((_ident, lambda v: np.asarray(v, f32), 1e-5),
                                  (O.bf16, lambda v: O.bf16(v).astype(f32), 2 ** -7)):
        r64 = O.qkv_attn(c, x, B, T, past, qkv, W["qn"], W["kn"], wo, kc, vc, store=store64)
        r32 = O.qkv_attn(c, x.astype(f32), B, T, past, qkv.astype(f32), W["qn"].astype(f32),
                         W["kn"].astype(f32), wo.astype(f32), kc.astype(f32), vc.astype(f32),
                         store=store32, ft=f32)
        assert r32["partial"].dtype == f32
        for k in ("q", "attn", "partial"):
            rel = np.max(np.abs(r32[k] - r64[k])) / np.max(np.abs(r64[k]))
            assert rel <= tol, (k, rel)
        h64, p64 = O.mlp(c, x, gu, wd, store=store64)
        h32, p32 = O.mlp(c, x.astype(f32), gu.astype(f32), wd.astype(f32), store=store32, ft=f32)
        assert p32.dtype == f32
        assert np.max(np.abs(p32 - p64)) / np.max(np.abs(p64)) <= tol


# ---- last-token selection and the final norm before the head ----------------

def test_last_token_rows_match_torch_indexing():
    """Equal lengths: the rows x.view(B, T, H)[:, -1] picks ([TPS]
    TPTransformer.forward, x[:, -1:]); ragged lengths: the last row of each
    piece that torch.split cuts the packed batch into."""
    B, T = 4, 5
    idx = torch.arange(B * T).view(B, T)[:, -1]
    assert np.array_equal(O.last_token_rows([T] * B), idx.numpy())
    lens = [3, 1, 7, 2]
    pieces = torch.split(torch.arange(sum(lens)), lens)
    assert np.array_equal(O.last_token_rows(lens), np.array([p[-1].item() for p in pieces]))
    with pytest.raises(ValueError):
        O.last_token_rows([2, 0])


def test_rmsnorm_rows_commutes_with_selection():
    """Norm after selection ([TPS] order) equals selection after norm over
    all rows ([CH9] order), and equals torch's rms_norm on the selected rows;
    an index outside the batch gives a zero row."""
    rng = np.random.default_rng(50)
    x = O.bf16(rng.standard_normal((9, 48)))
    w = O.bf16(rng.uniform(0.5, 1.5, 48))
    rows = np.array([8, 2, 2, 5])
    y = O.rmsnorm_rows(x, rows, w, 1e-6, store=_ident)
    y_all = O.rms_norm(x, w, 1e-6)
    assert np.allclose(y, y_all[rows], rtol=0, atol=1e-12)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x)[torch.from_numpy(rows)], (48,),
                                       torch.from_numpy(w), eps=1e-6).numpy()
    assert np.allclose(y, ref, rtol=0, atol=1e-12)
    z = O.rmsnorm_rows(x, np.array([0, 9, -1]), w, 1e-6, store=_ident)
    assert np.array_equal(z[1:], np.zeros((2, 48))) and np.allclose(z[0], y_all[0])


@pytest.mark.parametrize("n", [1, 2, 4])
def test_decode_head_on_last_tokens_equals_torch(n):
    """Greedy next token of each sequence from the last rows, normed, over n
    vocab shards equals torch.argmax of F.linear(rms_norm(x[:, -1:]), E)."""
    rng = np.random.default_rng(51 + n)
    B, T, H, V = 3, 4, 32, 50
    x = O.bf16(rng.standard_normal((B * T, H)))
    w = O.bf16(rng.uniform(0.5, 1.5, H))
    E = O.bf16(rng.standard_normal((V, H)) * 0.3)
    rows = O.last_token_rows([T] * B)
    y = O.rmsnorm_rows(x, rows, w, 1e-6)
    vals, idx = [], []
    for r in range(n):
        c = O.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = O.local_dims(c)
        v, i = O.lm_head_argmax(y, O.shard(c, O.W_VOCAB, E), L.vocab_start)
        vals.append(v)
        idx.append(i)
    _, tok = O.argmax_combine(np.stack(vals), np.stack(idx))
    xt = torch.from_numpy(x).view(B, T, H)[:, -1:]
    yt = torch.nn.functional.rms_norm(xt, (H,), torch.from_numpy(w), eps=1e-6)
    yt = torch.from_numpy(O.bf16(yt.numpy()))
    logits = torch.from_numpy(O.bf16(torch.nn.functional.linear(yt, torch.from_numpy(E)).numpy()))
    assert np.array_equal(tok, torch.argmax(logits[:, -1], dim=-1).numpy())
