"""The allocation-free decode head (tp_lm_head_argmax_noalloc) against the
workspace entry point (tp_lm_head_argmax): the same kernels, so the same
bits.  Two calls in a row share the library's static candidate array; the
second has fewer rows, so a stale slot of the first call would show up."""
import pytest
import torch

import synth
import tensor_transformer_layer_rank_amd as tp

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_pair(c, x, M, shard, rows=None):
    ws = torch.empty(max(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, M, 1), 256), dtype=torch.uint8, device=DEV)
    v1 = torch.empty(M, dtype=torch.float32, device=DEV)
    i1 = torch.empty(M, dtype=torch.int32, device=DEV)
    tp.tp_lm_head_argmax(c, x, M, shard, v1, i1, ws, rows=rows)
    v2 = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    i2 = torch.full((M,), -7, dtype=torch.int32, device=DEV)
    tp.tp_lm_head_argmax_noalloc(c, x, M, shard, v2, i2, rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(v1.view(torch.int32), v2.view(torch.int32))
    assert torch.equal(i1, i2)
    return i2


@pytest.mark.parametrize("H,V,n,r,M1,M2", [
    (1024, 151936, 2, 1, 64, 16),      # rows kept on chip
    (5120, 151936, 2, 0, 256, 100),    # logits GEMM with the argmax epilogue
])
def test_noalloc_head_matches_workspace_head(H, V, n, r, M1, M2):
    c = tp.Cfg(hidden=H, vocab=V, tp_size=n, tp_rank=r)
    L = tp.tp_local_dims(c)
    E = synth.embedding(80, V, H).to(DEV)
    shard = torch.empty(L.vocab_end - L.vocab_start, H, dtype=torch.bfloat16, device=DEV)
    tp.tp_shard_weights(c, tp.TP_W_VOCAB, E, shard)
    del E
    x1 = synth.activations(81, M1, H).to(DEV)
    _run_pair(c, x1, M1, shard)
    # the second call: fewer rows, a row list into a different x
    x2 = synth.activations(82, 3 * M2, H).to(DEV)
    rows = torch.arange(3 * M2 - 1, -1, -3, dtype=torch.int32, device=DEV)
    _run_pair(c, x2, M2, shard, rows=rows)


def test_noalloc_head_rejects_more_candidates_than_the_array():
    c = tp.Cfg(hidden=5120, vocab=151936, tp_size=2)
    assert tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, 2000, 1) > 4 << 20
    x = torch.zeros(2000, 5120, dtype=torch.bfloat16, device=DEV)
    L = tp.tp_local_dims(c)
    shard = torch.zeros(L.vocab_end - L.vocab_start, 5120, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(2000, dtype=torch.float32, device=DEV)
    i = torch.empty(2000, dtype=torch.int32, device=DEV)
    with pytest.raises(tp.TpError) as e:
        tp.tp_lm_head_argmax_noalloc(c, x, 2000, shard, v, i)
    assert e.value.status == -6
