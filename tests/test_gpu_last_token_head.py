"""GPU parity of the decode head on each sequence's last token: the
last-token selection and the final RMSNorm inside the library ("Tensor
parallelism from scratch", "Implementation", TPTransformer.forward: the final
norm on x[:, -1:], then the vocab-split output layer; "Chapter 9
Multi-process and Tensor Parallelism", 3.3: ParallelLMHead keeps each
sequence's last row).

Two orders that give the same rows: select then norm (tp_rmsnorm_rows with
the last-token rows, then the head on the compact rows) and norm then select
(tp_residual_rmsnorm with no partials over every token, then the head with
the row list).  Greedy ids are compared with the oracle exactly, except where
the oracle's top two logits lie within one bf16 step (then either id is a
correct greedy token); the normed rows and the logits within the bf16
tolerance."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import tensor_transformer_layer_rank_amd as tp

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 1e-2


def relerr(gpu, ref):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_ids(gv, gi, rv, ri, y, E):
    for m in range(len(ri)):
        if gi[m] == ri[m]:
            assert gv[m] == rv[m], (m, gv[m], rv[m])
            continue
        logit = O.bf16(y[m] @ E[gi[m]])
        assert abs(logit - rv[m]) <= 2.0 ** -7 * abs(rv[m]), (m, gi[m], ri[m], logit, rv[m])


CASES = {
    # name: (vocab, hidden, tp, sequence lengths, workload id); the first
    # three take the head kernel that keeps the rows on chip (<= 64 rows,
    # hidden <= 1024), the others the logits GEMM with the argmax epilogue
    "0.6b-4x37": (151936, 1024, 2, [37] * 4, 60),
    "0.6b-ragged": (151936, 1024, 2, [3, 1, 70, 2, 33], 61),
    "h256-64seqs": (5003, 256, 3, [2] * 64, 62),
    "32b-tp2-4x37": (151936, 5120, 2, [37] * 4, 63),
    "32b-ragged-100seqs": (20011, 5120, 2, list(np.random.default_rng(64).integers(1, 9, 100)), 64),
}


@pytest.mark.parametrize("case", list(CASES))
def test_last_token_head(case):
    V, H, n, lens, wid = CASES[case]
    lens = [int(v) for v in lens]
    rows = tp.tp_last_token_rows(lens)
    assert rows == list(O.last_token_rows(lens))
    Mx, B = sum(lens), len(lens)
    x = synth.activations(wid, Mx, H)
    w = synth.uniform(wid, synth.T_LNW, (H,), 0.5, 1.5)
    E = synth.embedding(wid, V, H)
    xg, wg, Eg = x.to(DEV), w.to(DEV), E.to(DEV)
    rows_g = torch.tensor(rows, dtype=torch.int32, device=DEV)
    c0 = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=0)
    # select then norm
    y = torch.empty(B, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_rmsnorm_rows(c0, xg, rows_g, B, wg, y)
    # norm then select
    y_all = torch.empty(Mx, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_residual_rmsnorm(c0, None, 0, Mx, xg, wg, None, y_all)
    ids = {}
    for order in ("select-norm", "norm-select"):
        vals = torch.empty(n, B, dtype=torch.float32, device=DEV)
        idx = torch.empty(n, B, dtype=torch.int32, device=DEV)
        for r in range(n):
            c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
            L = tp.tp_local_dims(c)
            shard = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
            tp.tp_shard_weights(c, tp.TP_W_VOCAB, Eg, shard)
            ws = torch.empty(max(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, B, 1), 256), dtype=torch.uint8,
                             device=DEV)
            if order == "select-norm":
                tp.tp_lm_head_argmax(c, y, B, shard, vals[r], idx[r], ws)
            else:
                tp.tp_lm_head_argmax(c, y_all, B, shard, vals[r], idx[r], ws, rows=rows_g)
            if r == 0 and order == "norm-select":
                # the logits of rank 0's slice through the row list
                lg = torch.empty(B, L.vocab_end - L.vocab_start, dtype=torch.bfloat16, device=DEV)
                tp.tp_lm_head(c, y_all, B, shard, lg, rows=rows_g)
                logits0 = f64(lg)
        out_i = torch.empty(B, dtype=torch.int32, device=DEV)
        out_v = torch.empty(B, dtype=torch.float32, device=DEV)
        tp.tp_argmax_combine(vals, idx, n, B, out_i, out_v)
        torch.cuda.synchronize()
        ids[order] = (out_v.cpu().numpy(), out_i.cpu().numpy())

    xc, wc, Ec = synth.to_f64(x), synth.to_f64(w), synth.to_f64(E)
    y_ref = O.rmsnorm_rows(xc, np.asarray(rows), wc, c0.rms_eps)
    assert relerr(f64(y), y_ref) <= TOL_BF16
    assert relerr(f64(y_all)[rows], y_ref) <= TOL_BF16
    # the oracle's head on its own normed rows
    ov, oi = [], []
    for r in range(n):
        oc = O.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
        L = O.local_dims(oc)
        v, i = O.lm_head_argmax(y_ref, Ec[L.vocab_start:L.vocab_end], L.vocab_start)
        ov.append(v)
        oi.append(i)
        if r == 0:
            assert relerr(logits0, O.lm_head(y_ref, Ec[L.vocab_start:L.vocab_end])) <= TOL_BF16
    rv, ri = O.argmax_combine(np.stack(ov), np.stack(oi))
    for order, (gv, gi) in ids.items():
        _check_ids(gv, gi, rv, ri, y_ref, Ec)


def test_head_row_list_out_of_range_reads_zero():
    """An index outside x reads as a zero row: its logits are exactly 0 and
    its greedy id is the shard's first (every logit ties at 0)."""
    V, H, n = 3001, 1024, 2
    x = synth.activations(70, 10, H).to(DEV)
    E = synth.embedding(70, V, H).to(DEV)
    rows = torch.tensor([9, -1, 10, 0], dtype=torch.int32, device=DEV)
    c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=1)
    L = tp.tp_local_dims(c)
    shard = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_shard_weights(c, tp.TP_W_VOCAB, E, shard)
    lg = torch.empty(4, L.vocab_end - L.vocab_start, dtype=torch.bfloat16, device=DEV)
    tp.tp_lm_head(c, x, 4, shard, lg, rows=rows)
    ws = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, 4, 1), dtype=torch.uint8, device=DEV)
    v = torch.empty(4, dtype=torch.float32, device=DEV)
    i = torch.empty(4, dtype=torch.int32, device=DEV)
    tp.tp_lm_head_argmax(c, x, 4, shard, v, i, ws, rows=rows)
    y = torch.empty(4, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_rmsnorm_rows(c, x, rows, 4, torch.ones(H, dtype=torch.bfloat16, device=DEV), y)
    torch.cuda.synchronize()
    lg, v, i, y = f64(lg), v.cpu().numpy(), i.cpu().numpy(), f64(y)
    assert (lg[1] == 0).all() and (lg[2] == 0).all()
    assert v[1] == 0 and v[2] == 0 and i[1] == L.vocab_start and i[2] == L.vocab_start
    assert (y[1] == 0).all() and (y[2] == 0).all()
    Ec = f64(E)[L.vocab_start:L.vocab_end]
    xc = f64(x)
    ref = O.lm_head(xc[[9, 0]], Ec)
    assert relerr(lg[[0, 3]], ref) <= TOL_BF16
