"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: shard maps and the masked embedding bit-exact; numerics
max|gpu - oracle| / max|oracle| <= 1e-2 per tensor for bf16 (fp32 accumulate)
and <= 1e-5 for the fp32 workload.  Mid-size cases (several tiles plus ragged
tails in M, N and K) are compared element by element; the five full-size
workloads are compared on sampled rows that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_transformer_layer_rank_amd as tp

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 1e-2
TOL_F32 = 1e-5


def relerr(gpu, ref):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    den = np.max(np.abs(ref)) if ref.size else 1.0
    return float(np.max(np.abs(gpu - ref)) / max(den, 1e-30)) if ref.size else 0.0


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits16(t):
    return t.detach().cpu().view(torch.int16).numpy()


def tcfg(w, r, n=None, dtype=tp.TP_BF16):
    return tp.Cfg(hidden=w["hidden"], intermediate=w["intermediate"], n_q_heads=w["n_q_heads"],
                  n_kv_heads=w["n_kv_heads"], head_dim=w["head_dim"], tp_size=n or w["tp"], tp_rank=r,
                  dtype=dtype, vocab=w.get("vocab", 0))


def ocfg(w, r, n=None):
    return O.Cfg(hidden=w["hidden"], intermediate=w["intermediate"], n_q_heads=w["n_q_heads"],
                 n_kv_heads=w["n_kv_heads"], head_dim=w["head_dim"], vocab=w.get("vocab", 0),
                 tp_size=n or w["tp"], tp_rank=r)


# mid-size shapes: several tiles and ragged tails; each exercises one GQA shape
MID = {
    "rep2": dict(hidden=520, intermediate=1568, n_q_heads=8, n_kv_heads=4, head_dim=128, vocab=1000, tp=2),
    "rep4-replicated": dict(hidden=256, intermediate=512, n_q_heads=8, n_kv_heads=2, head_dim=128, vocab=300, tp=4),
    "rep8": dict(hidden=512, intermediate=1024, n_q_heads=16, n_kv_heads=2, head_dim=128, vocab=777, tp=2),
    "rep1": dict(hidden=264, intermediate=528, n_q_heads=4, n_kv_heads=4, head_dim=128, vocab=64, tp=2),
    "rep16": dict(hidden=384, intermediate=768, n_q_heads=32, n_kv_heads=2, head_dim=128, vocab=100, tp=2),
    "rep4": dict(hidden=320, intermediate=640, n_q_heads=16, n_kv_heads=4, head_dim=128, vocab=200, tp=2),
}
MID_WID = {k: 100 + i for i, k in enumerate(MID)}


class Rank:
    """One rank's local weights, sharded on the device by tp_shard_weights
    from the full weights."""

    def __init__(self, w, r, W, n=None):
        self.c = tcfg(w, r, n)
        self.L = tp.tp_local_dims(self.c)
        L, H = self.L, w["hidden"]
        dt = torch.bfloat16
        self.qkv = torch.empty(L.n_qkv, H, dtype=dt, device=DEV)
        self.gu = torch.empty(2 * L.li, H, dtype=dt, device=DEV)
        self.o = torch.empty(H, L.lq * 128, dtype=dt, device=DEV)
        self.down = torch.empty(H, L.li, dtype=dt, device=DEV)
        for kind, name, dst in ((tp.TP_W_Q, "q", self.qkv), (tp.TP_W_K, "k", self.qkv), (tp.TP_W_V, "v", self.qkv),
                                (tp.TP_W_GATE, "gate", self.gu), (tp.TP_W_UP, "up", self.gu),
                                (tp.TP_W_O, "o", self.o), (tp.TP_W_DOWN, "down", self.down)):
            tp.tp_shard_weights(self.c, kind, W[name], dst)
        self.qn, self.kn = W["q_norm"], W["k_norm"]


def gpu_weights(w, wid):
    return {k: v.to(DEV) for k, v in synth.full_weights(wid, w).items()}


def shard64(oc, kind, Wt):
    """Oracle shard of a full bf16 weight, taken on its bit patterns, then
    widened to float64 (cheaper than widening the full matrix)."""
    b = O.shard(oc, kind, Wt.view(torch.int16).numpy())
    return synth.to_f64(torch.from_numpy(np.ascontiguousarray(b)).view(torch.bfloat16))


def oracle_rank_weights(oc, Wc):
    """The oracle's own shard + merge of the CPU copies of the full weights."""
    qkv = O.merge_qkv(O.shard(oc, O.W_Q, Wc["q"]), O.shard(oc, O.W_K, Wc["k"]), O.shard(oc, O.W_V, Wc["v"]))
    gu = O.merge_gate_up(O.shard(oc, O.W_GATE, Wc["gate"]), O.shard(oc, O.W_UP, Wc["up"]))
    return qkv, gu, O.shard(oc, O.W_O, Wc["o"]), O.shard(oc, O.W_DOWN, Wc["down"])


def run_attn(rk, x, B, T, past, kc, vc, S_max):
    L = rk.L
    M = B * T
    H = x.shape[1]
    ws = torch.empty(tp.tp_workspace_bytes(rk.c, tp.TP_OP_ATTN, B, T, past), dtype=torch.uint8, device=DEV)
    q = torch.empty(M, L.lq * 128, dtype=torch.bfloat16, device=DEV)
    a = torch.empty_like(q)
    part = torch.empty(M, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_qkv_attn(rk.c, x, B, T, past, rk.qkv, rk.qn, rk.kn, rk.o, kc, vc, S_max, part, ws, q_out=q, attn_out=a)
    return q, a, part


def run_mlp(rk, x, M):
    ws = torch.empty(tp.tp_workspace_bytes(rk.c, tp.TP_OP_MLP, M, 1), dtype=torch.uint8, device=DEV)
    h = torch.empty(M, rk.L.li, dtype=x.dtype, device=DEV)
    part = torch.empty(M, x.shape[1], dtype=x.dtype, device=DEV)
    tp.tp_mlp(rk.c, x, M, rk.gu, rk.down, part, ws, h_out=h)
    return h, part


# ------------------------------------------------------------------ shards and embedding

@pytest.mark.parametrize("name", list(MID) + ["w2", "w4", "w5"])
def test_shard_weights_bit_exact(name):
    """Every weight kind, merged, bit for bit against the oracle's shard +
    merge.  w4 (32B tp=2: 42 MB q / o shards, 131 MB gate / up / down shards)
    takes the copy kernel's grid-stride path, which strides 32 MB a pass."""
    if name in MID:
        w, wid = MID[name], MID_WID[name]
    else:
        wid = int(name[1])
        w = synth.WORKLOADS[wid]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    Wb = {k: v.view(torch.int16).numpy() for k, v in W.items()}
    n = w["tp"]
    ranks = range(n) if n <= 4 else [0, 1, 2, n - 1]
    for r in ranks:
        rk = Rank(w, r, Wg)
        qkv, gu, o, down = oracle_rank_weights(ocfg(w, r), Wb)
        assert np.array_equal(bits16(rk.qkv), qkv), (name, r, "qkv")
        assert np.array_equal(bits16(rk.gu), gu), (name, r, "gate_up")
        assert np.array_equal(bits16(rk.o), o), (name, r, "o")
        assert np.array_equal(bits16(rk.down), down), (name, r, "down")


@pytest.mark.parametrize("H", [1024, 5120])
def test_vocab_shard_whole_slice_bit_exact(H):
    """The whole vocab slice of both ranks (151936 rows over 2: 155.6 MB at
    hidden 1024, 777.9 MB at 5120, several grid-stride passes of the copy)
    bit for bit against the oracle's rows."""
    V = 151936
    E = _big_vocab(V, H)
    Eg = E.to(DEV)
    Eb = E.view(torch.int16).numpy()
    for r in range(2):
        c = tp.Cfg(hidden=H, vocab=V, tp_size=2, tp_rank=r)
        L = tp.tp_local_dims(c)
        dst = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, Eg, dst)
        ref = O.shard(O.Cfg(hidden=H, vocab=V, tp_size=2, tp_rank=r), O.W_VOCAB, Eb)
        assert np.array_equal(bits16(dst), ref), (H, r)
        del dst


def test_shard_weights_fp32_and_vocab():
    w = synth.WORKLOADS[1]
    W = synth.mlp_weights(1, w, torch.float32)
    for r in range(2):
        c = tcfg(w, r, dtype=tp.TP_F32)
        L = tp.tp_local_dims(c)
        gu = torch.empty(2 * L.li, w["hidden"], device=DEV)
        down = torch.empty(w["hidden"], L.li, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_GATE, W["gate"].to(DEV), gu)
        tp.tp_shard_weights(c, tp.TP_W_UP, W["up"].to(DEV), gu)
        tp.tp_shard_weights(c, tp.TP_W_DOWN, W["down"].to(DEV), down)
        oc = ocfg(w, r)
        ref = O.merge_gate_up(O.shard(oc, O.W_GATE, W["gate"].numpy()), O.shard(oc, O.W_UP, W["up"].numpy()))
        assert np.array_equal(gu.cpu().numpy().view(np.int32), ref.view(np.int32))
        assert np.array_equal(down.cpu().numpy().view(np.int32), O.shard(oc, O.W_DOWN, W["down"].numpy()).view(np.int32))
    # vocab rows, uneven last shard (V = 1000 over 3 ranks: 334, 334, 332)
    V, H = 1000, 136
    E = synth.embedding(7, V, H)
    for r in range(3):
        c = tp.Cfg(hidden=H, vocab=V, tp_size=3, tp_rank=r)
        L = tp.tp_local_dims(c)
        dst = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, E.to(DEV), dst)
        ref = O.shard(O.Cfg(hidden=H, vocab=V, tp_size=3, tp_rank=r), O.W_VOCAB, E.view(torch.int16).numpy())
        assert np.array_equal(bits16(dst), ref)


@pytest.mark.parametrize("case", ["w3", "w4-32b-tp2", "w5-32b-tp16", "ragged"])
def test_embed_vocab_bit_exact_and_vocab_sum(case):
    """Masked embedding on every rank, bit-exact, and the ranks' outputs sum
    to the full table's rows.  w3 and the 32B cases are the bench's embed
    shapes at full size (4096 or 1024 ids over the 151936-row vocabulary)."""
    if case == "w3":
        w = synth.WORKLOADS[3]
        V, H, n, n_ids = w["vocab"], w["hidden"], w["tp"], w["n_ids"]
        E = synth.embedding(3, V, H)
        ids = synth.token_ids(3, n_ids, V)
    elif case in ("w4-32b-tp2", "w5-32b-tp16"):
        wid = 4 if case.startswith("w4") else 5
        w = synth.WORKLOADS[wid]
        V, H, n = w["vocab"], w["hidden"], w["tp"]
        E = _big_vocab(V, H)
        ids = synth.token_ids(wid, 4096 if wid == 4 else 1024, V)
    else:
        V, H, n = 1001, 72, 3
        E = synth.embedding(9, V, H)
        ids = synth.token_ids(9, 37, V)
    # out-of-vocab and negative ids give zero rows on every rank
    ids = torch.cat([ids, torch.tensor([0, V - 1, V, V + 17, -1, -V], dtype=torch.int32)])
    Eg, idg = E.to(DEV), ids.to(DEV)
    Eb = E.view(torch.int16).numpy()
    total = torch.zeros(ids.numel(), H, dtype=torch.float32, device=DEV)
    for r in range(n):
        c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = tp.tp_local_dims(c)
        shard = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, Eg, shard)
        out = torch.full((ids.numel(), H), 7.0, dtype=torch.bfloat16, device=DEV)
        tp.tp_embed_vocab(c, idg, shard, out)
        oc = O.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        ref = O.embed_vocab(ids.numpy(), O.shard(oc, O.W_VOCAB, Eb), L.vocab_start, L.vocab_end)
        assert np.array_equal(bits16(out), ref), r
        total += out.float()
    valid = (ids >= 0) & (ids < V)
    assert torch.equal(total.cpu()[valid], E[ids[valid].long()].float())
    assert torch.count_nonzero(total.cpu()[~valid]) == 0


# ------------------------------------------------------------------ lm_head

@pytest.mark.parametrize("case", ["w3", "w4-32b-tp2", "w5-32b-tp16", "mid", "many-ragged", "persistent-ragged"])
def test_lm_head(case):
    """Logits of a vocab shard.  w3 and the 32B cases are the bench's lm_head
    shapes at full size (4096 rows at tp=2 and 1024 rows at tp=16 of the 32B
    hidden size 5120), sampled rows against the oracle; the ragged cases also
    check from the kernel marks which GEMM kernel ran."""
    kernel = None
    if case == "w3":
        w = synth.WORKLOADS[3]
        V, H, n, M = w["vocab"], w["hidden"], w["tp"], w["n_ids"]
        E = synth.embedding(3, V, H)
        x = synth.activations(3, M, H)
        rows = np.unique(np.concatenate([[0, 1, M - 1], np.random.default_rng(3).integers(0, M, 13)]))
        ranks = [0, 1]
    elif case in ("w4-32b-tp2", "w5-32b-tp16"):
        wid = 4 if case.startswith("w4") else 5
        w = synth.WORKLOADS[wid]
        V, H, n, M = w["vocab"], w["hidden"], w["tp"], 4096 if wid == 4 else 1024
        E = _big_vocab(V, H)
        x = synth.activations(wid, M, H)
        rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(wid).integers(0, M, 8)]))
        ranks = [0]
    elif case == "many-ragged":
        # 11.4 rounds of 256 x 320 tiles (33 K blocks), with ragged M, N and
        # K tails
        V, H, n, M = 116400, 2104, 2, 3996
        E = synth.embedding(12, V, H)
        x = synth.activations(12, M, H)
        rows = np.unique(np.concatenate([[0, 255, 256, 1279, 1280, 2047, 2048, 3839, 3840, M - 1],
                                         np.random.default_rng(12).integers(0, M, 8)]))
        ranks = [1]
        kernel = "gemm_tile<256,320,2>/bf16"
    elif case == "persistent-ragged":
        # eight rounds of 256 x 256 tiles (the persistent kernel), with ragged
        # M, N and K tails
        V, H, n, M = 65462, 1000, 2, 3996
        E = synth.embedding(13, V, H)
        x = synth.activations(13, M, H)
        rows = np.unique(np.concatenate([[0, 255, 256, 2047, 2048, 3839, 3840, M - 1],
                                         np.random.default_rng(13).integers(0, M, 8)]))
        ranks = [0]
        kernel = "gemm_persist<256,256,2>/bf16"
    else:
        V, H, n, M = 777, 520, 2, 300
        E = synth.embedding(11, V, H)
        x = synth.activations(11, M, H)
        rows = np.arange(M)
        ranks = [0, 1]
    Eg, xg = E.to(DEV), x.to(DEV)
    for r in ranks:
        c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = tp.tp_local_dims(c)
        shard = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, Eg, shard)
        logits = torch.empty(M, L.vocab_end - L.vocab_start, dtype=torch.bfloat16, device=DEV)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        tp.tp_kernel_marks(ev)
        try:
            tp.tp_lm_head(c, xg, M, shard, logits)
            torch.cuda.synchronize()
            names = tp.tp_kernel_mark_names()
        finally:
            tp.tp_kernel_marks([])
        if kernel:
            assert any(nm.startswith(kernel) for nm in names), (case, names)
        ref = O.lm_head(synth.to_f64(x)[rows], synth.to_f64(E[L.vocab_start:L.vocab_end]))
        err = relerr(f64(logits)[rows], ref)
        assert err <= TOL_BF16, (case, r, err)


# ------------------------------------------------------------------ MLP

def test_mlp_fp32_tiny_both_ranks_and_row_sum():
    w = synth.WORKLOADS[1]
    W = synth.mlp_weights(1, w, torch.float32)
    x = synth.activations(1, w["mlp_tokens"], w["hidden"], torch.float32)
    xc = synth.to_f64(x)
    Wc = {k: synth.to_f64(v) for k, v in W.items()}
    psum = torch.zeros(x.shape, dtype=torch.float64)
    for r in range(w["tp"]):
        c = tcfg(w, r, dtype=tp.TP_F32)
        L = tp.tp_local_dims(c)
        gu = torch.empty(2 * L.li, w["hidden"], device=DEV)
        down = torch.empty(w["hidden"], L.li, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_GATE, W["gate"].to(DEV), gu)
        tp.tp_shard_weights(c, tp.TP_W_UP, W["up"].to(DEV), gu)
        tp.tp_shard_weights(c, tp.TP_W_DOWN, W["down"].to(DEV), down)
        ws = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_MLP, x.shape[0], 1) + 1, dtype=torch.uint8, device=DEV)
        h = torch.empty(x.shape[0], L.li, device=DEV)
        part = torch.empty(x.shape, device=DEV)
        tp.tp_mlp(c, x.to(DEV), x.shape[0], gu, down, part, ws, h_out=h)
        oc = ocfg(w, r)
        gu_o = O.merge_gate_up(O.shard(oc, O.W_GATE, Wc["gate"]), O.shard(oc, O.W_UP, Wc["up"]))
        h_ref, p_ref = O.mlp(oc, xc, gu_o, O.shard(oc, O.W_DOWN, Wc["down"]), store=O.f32)
        assert relerr(f64(h), h_ref) <= TOL_F32
        assert relerr(f64(part), p_ref) <= TOL_F32
        psum += part.double().cpu()
    # summed row-parallel partials == the unsharded MLP
    oc1 = O.unsharded(ocfg(w, 0))
    _, full = O.mlp(oc1, xc, O.merge_gate_up(Wc["gate"], Wc["up"]), Wc["down"], store=O.f32)
    assert relerr(psum.numpy(), full) <= TOL_F32


@pytest.mark.parametrize("name", list(MID))
def test_mlp_mid_all_ranks(name):
    w, wid = MID[name], MID_WID[name]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    Wc = {k: synth.to_f64(v) for k, v in W.items()}
    for M in (300, 7):
        x = synth.activations(wid, M, w["hidden"], tid=synth.T_X + 20 * M)
        xc = synth.to_f64(x)
        psum = torch.zeros(M, w["hidden"], dtype=torch.float64)
        for r in range(w["tp"]):
            rk = Rank(w, r, Wg)
            h, part = run_mlp(rk, x.to(DEV), M)
            oc = ocfg(w, r)
            _, gu, _, down = oracle_rank_weights(oc, Wc)
            h_ref, p_ref = O.mlp(oc, xc, gu, down)
            assert relerr(f64(h), h_ref) <= TOL_BF16, (name, M, r, "h")
            assert relerr(f64(part), p_ref) <= TOL_BF16, (name, M, r, "partial")
            psum += part.double().cpu()
        _, full = O.mlp(O.unsharded(ocfg(w, 0)), xc, O.merge_gate_up(Wc["gate"], Wc["up"]), Wc["down"],
                        store=lambda v: np.asarray(v, np.float64))
        assert relerr(psum.numpy(), full) <= TOL_BF16, (name, M, "row-sum")


@pytest.mark.parametrize("wid", [2, 4, 5])
def test_mlp_full_size_sampled(wid):
    w = synth.WORKLOADS[wid]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    rk = Rank(w, 0, Wg)
    oc = ocfg(w, 0)
    gu = O.merge_gate_up(shard64(oc, O.W_GATE, W["gate"]), shard64(oc, O.W_UP, W["up"]))
    down = shard64(oc, O.W_DOWN, W["down"])
    for M in (w["prefill_T"], w["decode_B"]):
        x = synth.activations(wid, M, w["hidden"])
        h, part = run_mlp(rk, x.to(DEV), M)
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).integers(0, M, 10)]))
        h_ref, p_ref = O.mlp(oc, synth.to_f64(x)[rows], gu, down)
        assert relerr(f64(h)[rows], h_ref) <= TOL_BF16, (wid, M, "h")
        assert relerr(f64(part)[rows], p_ref) <= TOL_BF16, (wid, M, "partial")


def test_mlp_wide_tile_ragged():
    """The row-parallel down projection on its 320-column tiles, element by
    element: hidden 4904 is 15 tiles and a 104-column tail, the 3900 rows 15
    tiles and a 60-row tail (the last wave rows of a tile are written in a
    second staging pass).  The kernel marks confirm the tile shape ran."""
    w = dict(hidden=4904, intermediate=1280, n_q_heads=2, n_kv_heads=2, head_dim=128, vocab=0, tp=2)
    wid, M = 120, 3900
    W = synth.full_weights(wid, w)
    rk = Rank(w, 1, {k: v.to(DEV) for k, v in W.items()})
    oc = ocfg(w, 1)
    gu = O.merge_gate_up(shard64(oc, O.W_GATE, W["gate"]), shard64(oc, O.W_UP, W["up"]))
    down = shard64(oc, O.W_DOWN, W["down"])
    x = synth.activations(wid, M, w["hidden"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    tp.tp_kernel_marks(ev)
    try:
        h, part = run_mlp(rk, x.to(DEV), M)
        torch.cuda.synchronize()
        names = tp.tp_kernel_mark_names()
    finally:
        tp.tp_kernel_marks([])
    assert any(n.startswith("gemm_tile<256,320,2>/bf16[3900x4904x640]") for n in names), names
    h_ref, p_ref = O.mlp(oc, synth.to_f64(x), gu, down)
    assert relerr(f64(h), h_ref) <= TOL_BF16
    assert relerr(f64(part), p_ref) <= TOL_BF16


def test_mlp_wide_tile_silu_ragged():
    """The gate_up + SiLU GEMM on 320-row weight tiles (160 outputs each, 16
    gate rows beside their 16 up rows in every 32-row block), element by
    element: 2504 local intermediate columns are 15 tiles and a 104-column
    tail, 3900 rows 15 tiles and a 60-row tail, and hidden 1000 ends inside a
    64-wide K block.  The kernel marks confirm the tile shape ran."""
    w = dict(hidden=1000, intermediate=5008, n_q_heads=2, n_kv_heads=2, head_dim=128, vocab=0, tp=2)
    wid, M = 121, 3900
    W = synth.full_weights(wid, w)
    rk = Rank(w, 1, {k: v.to(DEV) for k, v in W.items()})
    oc = ocfg(w, 1)
    gu = O.merge_gate_up(shard64(oc, O.W_GATE, W["gate"]), shard64(oc, O.W_UP, W["up"]))
    down = shard64(oc, O.W_DOWN, W["down"])
    x = synth.activations(wid, M, w["hidden"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    tp.tp_kernel_marks(ev)
    try:
        h, part = run_mlp(rk, x.to(DEV), M)
        torch.cuda.synchronize()
        names = tp.tp_kernel_mark_names()
    finally:
        tp.tp_kernel_marks([])
    assert any(n.startswith("gemm_tile<256,320,2>/silu[3900x5008x1000]") for n in names), names
    h_ref, p_ref = O.mlp(oc, synth.to_f64(x), gu, down)
    assert relerr(f64(h), h_ref) <= TOL_BF16
    assert relerr(f64(part), p_ref) <= TOL_BF16


def test_mlp_wide_tile_silu_two_rounds_sampled():
    """The gate_up + SiLU GEMM on two rounds of 320-row weight tiles (512
    tiles; 33 K blocks, the last ragged), then a down projection on 256 x 128
    tiles with a split-K tail: sampled rows against the oracle, element by
    element.  The kernel marks confirm the tile shape ran."""
    w = dict(hidden=2104, intermediate=10000, n_q_heads=2, n_kv_heads=2, head_dim=128, vocab=0, tp=2)
    wid, M = 122, 3900
    W = synth.full_weights(wid, w)
    rk = Rank(w, 0, {k: v.to(DEV) for k, v in W.items()})
    oc = ocfg(w, 0)
    gu = O.merge_gate_up(shard64(oc, O.W_GATE, W["gate"]), shard64(oc, O.W_UP, W["up"]))
    down = shard64(oc, O.W_DOWN, W["down"])
    x = synth.activations(wid, M, w["hidden"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    tp.tp_kernel_marks(ev)
    try:
        h, part = run_mlp(rk, x.to(DEV), M)
        torch.cuda.synchronize()
        names = tp.tp_kernel_mark_names()
    finally:
        tp.tp_kernel_marks([])
    assert any(n.startswith("gemm_tile<256,320,2>/silu[3900x10000x2104]") for n in names), names
    rows = np.unique(np.concatenate([[0, 255, 256, 3839, 3840, M - 1], np.random.default_rng(M).integers(0, M, 10)]))
    h_ref, p_ref = O.mlp(oc, synth.to_f64(x)[rows], gu, down)
    assert relerr(f64(h)[rows], h_ref) <= TOL_BF16
    assert relerr(f64(part)[rows], p_ref) <= TOL_BF16


# ------------------------------------------------------------------ attention

def make_cache(w, wid, rk, B, S_max, past, n_global_kv):
    """Rank-local caches [B, lkv, S_max, d] holding the synthetic prior
    entries (drawn per global kv head) at positions < past; the rest is NaN
    so that a read outside the written range shows up."""
    L = rk.L
    kc = torch.full((B, L.lkv, S_max, 128), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    pk = pv = None
    if past > 0:
        pk = synth.prior_cache(wid, synth.T_KC, B, n_global_kv, past, 128)
        pv = synth.prior_cache(wid, synth.T_VC, B, n_global_kv, past, 128)
        kc[:, :, :past] = pk[:, L.kv_head0:L.kv_head0 + L.lkv]
        vc[:, :, :past] = pv[:, L.kv_head0:L.kv_head0 + L.lkv]
    return kc.to(DEV), vc.to(DEV), pk, pv


def check_attn(w, wid, r, B, T, past, S_max, rows=None, Wg=None, W=None, tol=TOL_BF16):
    """Runs tp_qkv_attn for rank r and compares q, the new cache entries, the
    attention output and the partial with the oracle (on `rows`, or all)."""
    W = W if W is not None else synth.full_weights(wid, w)
    Wg = Wg if Wg is not None else {k: v.to(DEV) for k, v in W.items()}
    rk = Rank(w, r, Wg)
    L, H, d = rk.L, w["hidden"], 128
    M = B * T
    x = synth.activations(wid, M, H, tid=synth.T_X + 7 * T + B)
    kc, vc, pk, pv = make_cache(w, wid, rk, B, S_max, past, w["n_kv_heads"])
    q, a, part = run_attn(rk, x.to(DEV), B, T, past, kc, vc, S_max)
    torch.cuda.synchronize()

    oc = ocfg(w, r)
    qkv_o = O.merge_qkv(shard64(oc, O.W_Q, W["q"]), shard64(oc, O.W_K, W["k"]), shard64(oc, O.W_V, W["v"]))
    wo = shard64(oc, O.W_O, W["o"])
    qn, kn = synth.to_f64(W["q_norm"]), synth.to_f64(W["k_norm"])
    xc = synth.to_f64(x)
    pos = np.tile(np.arange(past, past + T), B)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    # k, v of every new token (oracle), q of the checked rows
    k_new, v_new = O.kv_heads(oc, xc, qkv_o, kn, pos)
    q_ref = O.q_heads(oc, xc[rows], qkv_o, qn, pos[rows])
    rep = L.lq // L.lkv
    kc_g, vc_g = f64(kc), f64(vc)
    errs = {}
    errs["q"] = relerr(f64(q)[rows], q_ref.reshape(len(rows), -1))
    errs["k_cache"] = relerr(kc_g[:, :, past:past + T].transpose(0, 2, 1, 3).reshape(M, L.lkv, d), k_new)
    errs["v_cache"] = relerr(vc_g[:, :, past:past + T].transpose(0, 2, 1, 3).reshape(M, L.lkv, d), v_new)
    if past > 0:   # prior entries untouched
        assert np.array_equal(bits16(kc.cpu()[:, :, :past]), bits16(pk[:, L.kv_head0:L.kv_head0 + L.lkv]))
    assert torch.isnan(kc[:, :, past + T:].float()).all() if past + T < S_max else True
    attn_ref = np.zeros((len(rows), L.lq, d))
    for b in range(B):
        sel = np.nonzero(rows // T == b)[0]
        if len(sel) == 0:
            continue
        kseq = np.zeros((L.lkv, past + T, d))
        vseq = np.zeros_like(kseq)
        if past > 0:
            kseq[:, :past] = synth.to_f64(pk[b, L.kv_head0:L.kv_head0 + L.lkv])
            vseq[:, :past] = synth.to_f64(pv[b, L.kv_head0:L.kv_head0 + L.lkv])
        kseq[:, past:] = k_new[b * T:(b + 1) * T].transpose(1, 0, 2)
        vseq[:, past:] = v_new[b * T:(b + 1) * T].transpose(1, 0, 2)
        attn_ref[sel] = O.attend(q_ref[sel], pos[rows[sel]], kseq, vseq, rep)
    attn_ref = O.bf16(attn_ref.reshape(len(rows), -1))
    errs["attn"] = relerr(f64(a)[rows], attn_ref)
    errs["partial"] = relerr(f64(part)[rows], O.bf16(attn_ref @ wo.T))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (w, r, B, T, past, errs)
    return rk, kc, vc, part


def test_qkv_attn_wide_prefill_sampled():
    """A prefill whose (kv head, row block) workgroups fill the GPU by
    themselves runs the GQA-sharing prefill kernel: 17 sequences of 1000
    tokens (ragged last row block), sampled rows of every sequence."""
    w, wid = MID["rep2"], MID_WID["rep2"]
    B, T = 17, 1000
    rows = np.unique(np.concatenate([[0, 127, 128, T - 1, T, B * T - 1],
                                     np.random.default_rng(5).integers(0, B * T, 24)]))
    for r in range(w["tp"]):
        check_attn(w, wid, r, B, T, 0, T + 8, rows=rows)


@pytest.mark.parametrize("name", list(MID))
@pytest.mark.parametrize("phase", ["prefill", "prefill-after-past", "prefill-tiny", "prefill-few-tiles", "decode",
                                   "decode-ctx1", "decode-long"])
def test_qkv_attn_mid(name, phase):
    """prefill: 2 sequences of 300 tokens; prefill-after-past: 77 new tokens
    after 150 cached ones; prefill-tiny: 3 sequences of 2 tokens (one key
    tile: three of a block's four waves have none); prefill-few-tiles: 40
    tokens after 60 cached ones (0 to 2 tiles per wave, the pipelined loop's
    short cases); decode: 8 sequences; decode-ctx1: 3 sequences, one key;
    decode-long: 2 sequences at context 3000 (the key range split among a
    block's waves and merged).  These grids are small, so the one-pass flash
    kernel runs every phase."""
    w, wid = MID[name], MID_WID[name]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    B, T, past, S_max = {"prefill": (2, 300, 0, 320), "prefill-after-past": (2, 77, 150, 240),
                         "prefill-tiny": (3, 2, 0, 4), "prefill-few-tiles": (2, 40, 60, 128),
                         "decode": (8, 1, 299, 310), "decode-ctx1": (3, 1, 0, 4),
                         "decode-long": (2, 1, 2999, 3000)}[phase]
    for r in range(w["tp"]):
        check_attn(w, wid, r, B, T, past, S_max, Wg=Wg, W=W)


@pytest.mark.parametrize("name", ["rep1", "rep2", "rep4-replicated", "rep4", "rep8", "rep16"])
@pytest.mark.parametrize("past", [0, 37])
def test_qkv_attn_gqa_prefill_kernel(name, past):
    """Prefills wide enough that the GQA-sharing prefill kernel runs (its
    (kv head, row block) workgroups alone fill the GPU), at every group size
    (local rep 1, 2, 2 with a replicated kv head, 4, 8, 16), from an empty cache and
    after 37 cached positions (the causal offset of its row blocks).  The
    kernel marks confirm which attention kernel ran."""
    w, wid = MID[name], MID_WID[name]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    # (kv head, row block) workgroups: B * lkv * head groups * ceil(T / rows)
    # >= 256 with 333 tokens (rows = 32 * 8 / min(rep, 8): 256-row blocks for
    # rep 1, 128 for rep 2, 64 for rep 4, 32 for 8 and 16)
    B = {"rep1": 64, "rep2": 48, "rep4-replicated": 96, "rep4": 24, "rep8": 24, "rep16": 24}[name]
    T = 333
    S_max = past + T + 3
    rows = np.unique(np.concatenate([[0, 31, 32, T - 1, T, B * T - 1],
                                     np.random.default_rng(past + len(name)).integers(0, B * T, 24)]))
    for r in range(w["tp"]):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(32)]
        tp.tp_kernel_marks(ev)
        try:
            check_attn(w, wid, r, B, T, past, S_max, rows=rows, Wg=Wg, W=W)
            names = tp.tp_kernel_mark_names()
        finally:
            tp.tp_kernel_marks([])
        assert "attn_prefill" in names, names


def test_qkv_attn_row_sum_and_head_concat():
    """Summed o_proj partials over all ranks match the unsharded oracle, and
    concatenated per-rank attention outputs match the unsharded attention."""
    w, wid = MID["rep4-replicated"], MID_WID["rep4-replicated"]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    B, T, past, S_max = 2, 40, 0, 48
    x = synth.activations(wid, B * T, w["hidden"], tid=synth.T_X + 7 * T + B)
    psum = torch.zeros(B * T, w["hidden"], dtype=torch.float64)
    attn = []
    for r in range(w["tp"]):
        rk = Rank(w, r, Wg)
        kc, vc, _, _ = make_cache(w, wid, rk, B, S_max, past, w["n_kv_heads"])
        _, a, part = run_attn(rk, x.to(DEV), B, T, past, kc, vc, S_max)
        psum += part.double().cpu()
        attn.append(f64(a))
    oc1 = O.unsharded(ocfg(w, 0))
    Wc = {k: synth.to_f64(v) for k, v in W.items()}
    kc1 = np.zeros((B, w["n_kv_heads"], S_max, 128))
    ref = O.qkv_attn(oc1, synth.to_f64(x), B, T, past, O.merge_qkv(Wc["q"], Wc["k"], Wc["v"]), Wc["q_norm"],
                     Wc["k_norm"], Wc["o"], kc1, kc1.copy(), store=lambda v: np.asarray(v, np.float64))
    assert relerr(np.concatenate(attn, 1), ref["attn"]) <= TOL_BF16
    assert relerr(psum.numpy(), ref["partial"]) <= TOL_BF16


@pytest.mark.parametrize("wid", [2, 4, 5])
@pytest.mark.parametrize("phase", ["prefill", "decode"])
def test_qkv_attn_full_size_sampled(wid, phase):
    w = synth.WORKLOADS[wid]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    if phase == "prefill":
        B, T, past = 1, w["prefill_T"], 0
        S_max = T
        rows = np.unique(np.concatenate([[0, 1, 63, 64, T - 1], np.random.default_rng(T).integers(0, T, 11)]))
    else:
        B, T, past = w["decode_B"], 1, w["decode_ctx"] - 1
        S_max = w["decode_ctx"]
        rows = np.unique(np.concatenate([[0, B - 1], np.random.default_rng(B).integers(0, B, 6)]))
    ranks = [0, 1]
    out = {}
    for r in ranks:
        rk, kc, vc, part = check_attn(w, wid, r, B, T, past, S_max, rows=rows, Wg=Wg, W=W)
        out[r] = (rk.L.kv_head0, kc.cpu(), vc.cpu())
    if wid == 5:   # ranks 0 and 1 hold replicas of kv head 0: bit-identical caches
        assert out[0][0] == out[1][0] == 0
        assert torch.equal(out[0][1].view(torch.int16), out[1][1].view(torch.int16))
        assert torch.equal(out[0][2].view(torch.int16), out[1][2].view(torch.int16))


def test_deterministic_reruns():
    w, wid = MID["rep2"], MID_WID["rep2"]
    W = synth.full_weights(wid, w)
    Wg = {k: v.to(DEV) for k, v in W.items()}
    rk = Rank(w, 1, Wg)
    x = synth.activations(wid, 130, w["hidden"]).to(DEV)
    outs = []
    for _ in range(2):
        kc, vc, _, _ = make_cache(w, wid, rk, 2, 80, 10, w["n_kv_heads"])
        q, a, part = run_attn(rk, x, 2, 65, 10, kc, vc, 80)
        h, mp = run_mlp(rk, x, 130)
        outs.append([t.clone() for t in (q, a, part, kc, vc, h, mp)])
    for t1, t2 in zip(*outs):
        assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))


# ------------------------------------------------------------------ greedy argmax

def _argmax_case(V, H, n, M, wid, ties=False):
    E = synth.embedding(wid, V, H)
    x = synth.activations(wid, M, H)
    if ties:
        # copies of one row in several shards, and rows of x along it, so
        # that the copies tie exactly at the maximum: the smallest id wins
        k = V // 3
        for j in (3, V // 2 + 1, V - 2):
            E[j] = E[k]
        for m in range(0, M, 4):
            x[m] = (E[k].float() * 40.0).to(torch.bfloat16)
    Eg, xg = E.to(DEV), x.to(DEV)
    xc, Ec = synth.to_f64(x), synth.to_f64(E)
    vals = torch.empty(n, M, dtype=torch.float32, device=DEV)
    idx = torch.empty(n, M, dtype=torch.int32, device=DEV)
    ov, oi = [], []
    for r in range(n):
        c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = tp.tp_local_dims(c)
        shard = torch.empty(max(L.vocab_end - L.vocab_start, 1), H, dtype=torch.bfloat16, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, Eg, shard)
        ws = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, M, 1), dtype=torch.uint8, device=DEV)
        tp.tp_lm_head_argmax(c, xg, M, shard, vals[r], idx[r], ws)
        v, i = O.lm_head_argmax(xc, Ec[L.vocab_start:L.vocab_end], L.vocab_start)
        ov.append(v)
        oi.append(i)
    out_i = torch.empty(M, dtype=torch.int32, device=DEV)
    out_v = torch.empty(M, dtype=torch.float32, device=DEV)
    tp.tp_argmax_combine(vals, idx, n, M, out_i, out_v)
    torch.cuda.synchronize()
    ref_v, ref_i = O.argmax_combine(np.stack(ov), np.stack(oi))
    return (vals.cpu().numpy(), idx.cpu().numpy(), out_v.cpu().numpy(), out_i.cpu().numpy(),
            np.stack(ov), np.stack(oi), ref_v, ref_i, xc, Ec)


def _check_argmax(gv, gi, rv, ri, xc, Ec):
    """Token ids equal the oracle's, except where the oracle's top two logits
    lie within one bf16 step of each other (then any of them is a correct
    greedy token: fp32 and fp64 accumulation may round either way); values
    are the bf16 logits of the chosen ids."""
    for m in range(len(ri)):
        if gi[m] == ri[m]:
            assert gv[m] == rv[m], (m, gv[m], rv[m])
            continue
        logit = O.bf16(xc[m] @ Ec[gi[m]])
        assert abs(logit - rv[m]) <= 2.0 ** -7 * abs(rv[m]), (m, gi[m], ri[m], logit, rv[m])


def test_lm_head_argmax_decode_full_vocab():
    """The 0.6B vocabulary (151936 over 2 ranks), 64 decode rows: per-rank
    candidates and the combined greedy token against the oracle, and the
    combined token against argmax over the concatenated oracle logits."""
    w = synth.WORKLOADS[3]
    gvr, gir, gv, gi, ov, oi, rv, ri, xc, Ec = _argmax_case(w["vocab"], w["hidden"], w["tp"], 64, 3)
    for r in range(w["tp"]):
        _check_argmax(gvr[r], gir[r], ov[r], oi[r], xc, Ec)
    _check_argmax(gv, gi, rv, ri, xc, Ec)
    full = O.bf16(xc @ Ec.T)
    assert np.array_equal(ri, np.argmax(full, axis=1))


_BIG_VOCAB = {}


def _big_vocab(V, H):
    """One synthetic full vocabulary [V, H] (bf16, N(0, 0.02)) shared by the
    full-size decode-head cases."""
    if (V, H) not in _BIG_VOCAB:
        _BIG_VOCAB.clear()
        _BIG_VOCAB[(V, H)] = synth.embedding(4, V, H)
    return _BIG_VOCAB[(V, H)]


@pytest.mark.parametrize("wid", [4, 5])
def test_lm_head_argmax_full_size_sampled(wid):
    """The 32B decode heads at full size in the bench's launch configuration
    (hidden 5120: the logits-GEMM path with the argmax epilogue; 128 decode
    rows over 2 ranks, 256 over 16): every rank's shard runs, the ranks'
    candidates are combined on the GPU, and sampled rows are checked against
    the oracle over each rank's whole vocab slice and over the whole
    vocabulary."""
    w = synth.WORKLOADS[wid]
    V, H, n, M = w["vocab"], w["hidden"], w["tp"], w["decode_B"]
    E = _big_vocab(V, H)
    x = synth.activations(wid, M, H)
    Eg, xg = E.to(DEV), x.to(DEV)
    vals = torch.empty(n, M, dtype=torch.float32, device=DEV)
    idx = torch.empty(n, M, dtype=torch.int32, device=DEV)
    ranges = []
    for r in range(n):
        c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = tp.tp_local_dims(c)
        ranges.append((L.vocab_start, L.vocab_end))
        shard = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, Eg, shard)
        ws = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, M, 1), dtype=torch.uint8, device=DEV)
        tp.tp_lm_head_argmax(c, xg, M, shard, vals[r], idx[r], ws)
        del shard
    out_i = torch.empty(M, dtype=torch.int32, device=DEV)
    out_v = torch.empty(M, dtype=torch.float32, device=DEV)
    tp.tp_argmax_combine(vals, idx, n, M, out_i, out_v)
    torch.cuda.synchronize()
    del Eg
    gvr, gir = vals.cpu().numpy(), idx.cpu().numpy()
    gv, gi = out_v.cpu().numpy(), out_i.cpu().numpy()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M + wid).integers(0, M, 4)]))
    xc = synth.to_f64(x)[rows]
    ov, oi = [], []
    for r, (a, b) in enumerate(ranges):
        v, i = O.lm_head_argmax(xc, synth.to_f64(E[a:b]), a)
        ov.append(v)
        oi.append(i)
    rv, ri = O.argmax_combine(np.stack(ov), np.stack(oi))

    def check(got_v, got_i, ref_v, ref_i):
        # as _check_argmax, with the chosen id's logit taken from E directly
        for k, m in enumerate(rows):
            if got_i[m] == ref_i[k]:
                assert got_v[m] == ref_v[k], (wid, m, got_v[m], ref_v[k])
                continue
            logit = O.bf16(xc[k] @ synth.to_f64(E[int(got_i[m])]))
            assert abs(logit - ref_v[k]) <= 2.0 ** -7 * abs(ref_v[k]), (wid, m, got_i[m], ref_i[k])

    for r in range(n):
        check(gvr[r], gir[r], ov[r], oi[r])
    check(gv, gi, rv, ri)


@pytest.mark.parametrize("M", [128, 256, 100, 64])
def test_lm_head_argmax_matches_logits_argmax(M):
    """Every row of the 32B tp=2 decode head (hidden 5120, rank 1's 75968-row
    vocab slice): the argmax-epilogue GEMM, whose schedule may split the
    columns into a main launch and a tail (128 and 256 rows here), returns
    for each row exactly the first maximum of the logits that tp_lm_head
    computes on the GPU (no split-K in either, so both round the same fp32
    sums), with ids from the whole slice."""
    w = synth.WORKLOADS[4]
    V, H, n = w["vocab"], w["hidden"], w["tp"]
    c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=1)
    L = tp.tp_local_dims(c)
    nv = L.vocab_end - L.vocab_start
    E = _big_vocab(V, H)
    x = synth.activations(40 + M, M, H).to(DEV)
    shard = torch.empty(nv, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_shard_weights(c, tp.TP_W_VOCAB, E.to(DEV), shard)
    ws = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, M, 1), dtype=torch.uint8, device=DEV)
    v = torch.empty(M, dtype=torch.float32, device=DEV)
    i = torch.empty(M, dtype=torch.int32, device=DEV)
    tp.tp_lm_head_argmax(c, x, M, shard, v, i, ws)
    lg = torch.empty(M, nv, dtype=torch.bfloat16, device=DEV)
    tp.tp_lm_head(c, x, M, shard, lg)
    torch.cuda.synchronize()
    lgf = lg.float().cpu().numpy()
    ref_i = np.argmax(lgf, axis=1)
    assert np.array_equal(i.cpu().numpy(), ref_i + L.vocab_start)
    assert np.array_equal(v.cpu().numpy(), lgf[np.arange(M), ref_i])


@pytest.mark.parametrize("case", ["ragged-ties", "empty-shard", "resident-ties", "resident-empty-shard",
                                  "resident-one-row", "resident-h256", "resident-m20", "resident-h768"])
def test_lm_head_argmax_ragged(case):
    """Odd local vocab sizes (row stride not a multiple of 16 bytes), uneven
    shards, planted exact ties across shards (the smallest id must win), and
    an empty last shard that must never win.  The resident cases take the
    kernel that keeps the rows on chip (up to 64 rows, hidden 256, 512, 768
    or 1024, in its 16-, 32- and 64-row forms): fewer vocab rows than
    workgroups (most get none), one row, 20 rows, 50 rows, 64 rows."""
    if case in ("ragged-ties", "resident-ties"):
        V, H, n, M = (1001, 520, 3, 37) if case == "ragged-ties" else (701, 256, 2, 37)
        out = _argmax_case(V, H, n, M, 13 if case == "ragged-ties" else 15, ties=True)
        assert (out[7][0::4] == 3).all()           # the oracle's winner is the first copy
    else:
        V, H, n, M, wid = {"empty-shard": (5, 64, 4, 9, 14), "resident-empty-shard": (5, 256, 4, 9, 18),
                           "resident-one-row": (151936, 1024, 2, 1, 16),
                           "resident-h256": (5003, 256, 3, 64, 17),
                           "resident-m20": (30011, 512, 2, 20, 19),
                           "resident-h768": (40009, 768, 2, 50, 20)}[case]
        out = _argmax_case(V, H, n, M, wid)
    gvr, gir, gv, gi, ov, oi, rv, ri, xc, Ec = out
    for r in range(n):
        if oi[r][0] < 0:
            assert (gir[r] == -1).all() and np.isneginf(gvr[r]).all()
        else:
            _check_argmax(gvr[r], gir[r], ov[r], oi[r], xc, Ec)
    _check_argmax(gv, gi, rv, ri, xc, Ec)
    assert np.array_equal(gi, ri)


def bf16_ulp(a):
    """One bf16 unit in the last place at |a| (fp32 spacing scaled by 2^16)."""
    a = np.abs(np.asarray(a, np.float64)).astype(np.float32)
    return np.spacing(np.maximum(a, np.float32(2.0 ** -100))).astype(np.float64) * 65536.0


NORM_CASES = {
    # name: (workload id, partials n, rows M, hidden H, rows the oracle checks or None for all)
    "0.6b-tp2-prefill": (2, 2, 2048, 1024, None),
    "32b-tp16-decode": (5, 16, 256, 5120, None),
    "32b-tp2-prefill-sampled": (4, 2, 4096, 5120, [0, 1, 2, 3, 511, 2048, 3333, 4092, 4093, 4094, 4095]),
    "ragged-h520": (20, 3, 7, 520, None),
    "two-wave-rows-h2056": (24, 5, 11, 2056, None),
    "max-h8192": (21, 1, 5, 8192, None),
    "h8192-many-rows": (27, 2, 600, 8192, None),
    "h8": (22, 2, 9, 8, None),
}


def _run_norm(wid, n, M, H, inplace=False):
    P, R, Wn = synth.norm_inputs(wid, n, M, H)
    c = tp.Cfg(hidden=H, tp_size=n)
    Pg, Rg, Wg = P.to(DEV), R.to(DEV), Wn.to(DEV)
    hg = Rg if inplace else torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    yg = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    tp.tp_residual_rmsnorm(c, Pg, n, M, Rg, Wg, hg, yg)
    torch.cuda.synchronize()
    return P, R, Wn, c, hg, yg


def _check_norm(P, R, Wn, eps, hg, yg, rows):
    Pc, Rc, Wc = synth.to_f64(P), synth.to_f64(R), synth.to_f64(Wn)
    if rows is not None:
        Pc, Rc = Pc[:, rows], Rc[rows]
        hg, yg = hg[rows], yg[rows]
    h_ref, y_ref = O.residual_rmsnorm(Pc, Rc, Wc, eps)
    h, y = f64(hg), f64(yg)
    assert relerr(h, h_ref) <= TOL_BF16 and relerr(y, y_ref) <= TOL_BF16
    # fp32 against fp64 sums of bf16 terms: at most one rounding step apart
    assert (np.abs(h - h_ref) <= bf16_ulp(np.maximum(np.abs(h), np.abs(h_ref)))).all()
    assert (np.abs(y - y_ref) <= 2 * bf16_ulp(np.maximum(np.abs(y), np.abs(y_ref)))).all()


@pytest.mark.parametrize("case", list(NORM_CASES))
def test_residual_rmsnorm(case):
    """Residual add of the summed row-parallel partials and the next RMSNorm
    against the oracle: the 0.6B tp2 prefill rows and the 32B tp16 decode
    batch element by element, the 32B tp2 prefill on sampled rows (first,
    last, ragged last workgroup), a hidden size that leaves one lane of a
    second chunk (520), two-wave rows with a partial count that is not a
    multiple of the load group (2056, 5 partials), the largest supported
    hidden size and the smallest."""
    wid, n, M, H, rows = NORM_CASES[case]
    P, R, Wn, c, hg, yg = _run_norm(wid, n, M, H)
    _check_norm(P, R, Wn, c.rms_eps, hg, yg, rows)


def test_residual_rmsnorm_inplace_and_empty():
    """The residual buffer updated in place gives the same h and y; M = 0
    writes nothing."""
    P, R, Wn, c, hg, yg = _run_norm(23, 2, 33, 1024, inplace=True)
    _check_norm(P, R, Wn, c.rms_eps, hg, yg, None)
    _, _, _, c, h0, y0 = _run_norm(23, 2, 33, 1024)
    assert torch.equal(h0.view(torch.int16), hg.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), yg.view(torch.int16))
    y = torch.full((4, 1024), 7.0, dtype=torch.bfloat16, device=DEV)
    tp.tp_residual_rmsnorm(c, y, 2, 0, y, y[0], y, y)
    torch.cuda.synchronize()
    assert (y == 7.0).all()


SP_CASES = {
    # name: (workload id, tp, tokens M, hidden H, rows the oracle checks or None for all)
    "0.6b-tp2-prefill": (2, 2, 2048, 1024, None),
    "32b-tp16-prefill": (5, 16, 1024, 5120, [0, 1, 63, 64, 65, 511, 512, 1022, 1023]),
    "ragged-empty-rank": (25, 4, 9, 520, None),
    "ragged-short-last": (26, 3, 7, 2056, None),
}


@pytest.mark.parametrize("case", list(SP_CASES))
def test_sp_residual_rmsnorm(case):
    """Sequence parallelism: every rank in turn sums its token slice of the
    ranks' partials into its slice of the residual stream, normalises it and
    writes its rows of the gathered output.  Each rank's rows against the
    oracle; the gathered residual bit-equal to the non-sequence-parallel
    fused step's and the gathered normed rows within one bf16 step of it; a
    rank's call leaves the other rows of the gathered buffer untouched; a
    rank with no token writes nothing."""
    wid, n, M, H, rows = SP_CASES[case]
    P, R, Wn = synth.norm_inputs(wid, n, M, H)
    Pg, Rg, Wg = P.to(DEV), R.to(DEV), Wn.to(DEV)
    Wc = synth.to_f64(Wn)
    if rows is None:
        Pc, Rc = synth.to_f64(P), synth.to_f64(R)
    else:   # sampled rows: the oracle's fused step on those rows alone
        Pc, Rc = synth.to_f64(P[:, rows]), synth.to_f64(R[rows])
        h_smp, y_smp = O.residual_rmsnorm(Pc, Rc, Wc, 1e-6)
    nan = float("nan")
    y_all = torch.full((M, H), nan, dtype=torch.bfloat16, device=DEV)
    hs = []
    for r in range(n):
        c = tp.Cfg(hidden=H, tp_size=n, tp_rank=r)
        s, e = tp.tp_sp_rows(c, M)
        assert (s, e) == O.sp_rows(M, n, r)
        h = torch.full((e - s, H), nan, dtype=torch.bfloat16, device=DEV)
        y_one = torch.full((M, H), nan, dtype=torch.bfloat16, device=DEV)
        tp.tp_sp_residual_rmsnorm(c, Pg, M, Rg[s:e], Wg, h, y_one)
        tp.tp_sp_residual_rmsnorm(c, Pg, M, Rg[s:e], Wg, h, y_all)
        torch.cuda.synchronize()
        outside = torch.ones(M, dtype=torch.bool)
        outside[s:e] = False
        assert torch.isnan(y_one.float().cpu()[outside]).all()
        hs.append(h)
        if rows is None:
            if e == s:
                continue
            h_ref, y_ref = O.sp_residual_rmsnorm(Pc, Rc[s:e], Wc, c.rms_eps, r)
            hg, yg = f64(h), f64(y_one[s:e])
        else:
            pick = [i for i, m in enumerate(rows) if s <= m < e]
            if not pick:
                continue
            h_ref, y_ref = h_smp[pick], y_smp[pick]
            hg, yg = f64(h[[rows[i] - s for i in pick]]), f64(y_one[[rows[i] for i in pick]])
        assert relerr(hg, h_ref) <= TOL_BF16 and relerr(yg, y_ref) <= TOL_BF16
        assert (np.abs(hg - h_ref) <= bf16_ulp(np.maximum(np.abs(hg), np.abs(h_ref)))).all()
        assert (np.abs(yg - y_ref) <= 2 * bf16_ulp(np.maximum(np.abs(yg), np.abs(y_ref)))).all()
    h_full = torch.empty(M, H, dtype=torch.bfloat16, device=DEV)
    y_full = torch.empty(M, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_residual_rmsnorm(tp.Cfg(hidden=H, tp_size=n), Pg, n, M, Rg, Wg, h_full, y_full)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(hs).view(torch.int16), h_full.view(torch.int16))
    # y: the sum of squares is reduced in an order that follows the launch
    # shape, which depends on the row count; at most one bf16 step apart
    ya, yf = f64(y_all), f64(y_full)
    assert (np.abs(ya - yf) <= bf16_ulp(np.maximum(np.abs(ya), np.abs(yf)))).all()
