"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  This module holds shapes and random draws only -- none of the
method's arithmetic.  bf16 inputs are produced by torch's own fp32->bf16
conversion so that both sides see identical bits.

Tensor ids (second seed word): 0 x, 1 q, 2 k, 3 v, 4 o, 5 gate, 6 up, 7 down,
8 q_norm, 9 k_norm, 10 prior K cache, 11 prior V cache, 12 ids, 13 embedding,
14 row-parallel partials, 15 residual stream, 16 layer-norm weight.
Generator: numpy.random.default_rng([workload_id, tensor_id]).
"""
from __future__ import annotations

import numpy as np
import torch

(T_X, T_Q, T_K, T_V, T_O, T_GATE, T_UP, T_DOWN, T_QN, T_KN, T_KC, T_VC, T_IDS, T_EMB,
 T_PART, T_RES, T_LNW) = range(17)

# The five workloads: model shapes (Qwen3-0.6B / Qwen3-32B) and per-rank sizes.
WORKLOADS = {
    1: dict(name="tiny-swiglu-mlp-fp32-tp2", dtype="f32", hidden=64, intermediate=192,
            n_q_heads=2, n_kv_heads=2, head_dim=128, vocab=0, tp=2, mlp_tokens=8),
    2: dict(name="qwen3-0.6b-layer-shard-tp2", dtype="bf16", hidden=1024, intermediate=3072,
            n_q_heads=16, n_kv_heads=8, head_dim=128, vocab=151936, tp=2,
            prefill_T=2048, decode_B=64, decode_ctx=1024),
    3: dict(name="vocab-embed-lmhead-tp2", dtype="bf16", hidden=1024, intermediate=3072,
            n_q_heads=16, n_kv_heads=8, head_dim=128, vocab=151936, tp=2, n_ids=4096),
    4: dict(name="qwen3-32b-layer-shard-tp2", dtype="bf16", hidden=5120, intermediate=25600,
            n_q_heads=64, n_kv_heads=8, head_dim=128, vocab=151936, tp=2,
            prefill_T=4096, decode_B=128, decode_ctx=2048),
    5: dict(name="qwen3-32b-layer-shard-tp16-kv-replicated", dtype="bf16", hidden=5120,
            intermediate=25600, n_q_heads=64, n_kv_heads=8, head_dim=128, vocab=151936, tp=16,
            prefill_T=1024, decode_B=256, decode_ctx=4096),
}


def rng(wid: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([wid, tid])


def normal(wid: int, tid: int, shape, std: float = 1.0, dtype=torch.bfloat16) -> torch.Tensor:
    a = rng(wid, tid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return torch.from_numpy(a).to(dtype)


def uniform(wid: int, tid: int, shape, lo: float, hi: float, dtype=torch.bfloat16) -> torch.Tensor:
    a = rng(wid, tid).uniform(lo, hi, size=shape).astype(np.float32)
    return torch.from_numpy(a).to(dtype)


def token_ids(wid: int, n: int, vocab: int, tid: int = T_IDS) -> torch.Tensor:
    return torch.from_numpy(rng(wid, tid).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32))


def full_weights(wid: int, w: dict, dtype=torch.bfloat16) -> dict:
    """Unsharded [out, in] layer weights ~ N(0, 0.02); norm weights ~ U(0.5, 1.5)."""
    H, I, d = w["hidden"], w["intermediate"], w["head_dim"]
    nq, nkv = w["n_q_heads"], w["n_kv_heads"]
    s = 0.02
    return dict(
        q=normal(wid, T_Q, (nq * d, H), s, dtype), k=normal(wid, T_K, (nkv * d, H), s, dtype),
        v=normal(wid, T_V, (nkv * d, H), s, dtype), o=normal(wid, T_O, (H, nq * d), s, dtype),
        gate=normal(wid, T_GATE, (I, H), s, dtype), up=normal(wid, T_UP, (I, H), s, dtype),
        down=normal(wid, T_DOWN, (H, I), s, dtype),
        q_norm=uniform(wid, T_QN, (d,), 0.5, 1.5, dtype), k_norm=uniform(wid, T_KN, (d,), 0.5, 1.5, dtype))


def mlp_weights(wid: int, w: dict, dtype) -> dict:
    H, I = w["hidden"], w["intermediate"]
    return dict(gate=normal(wid, T_GATE, (I, H), 0.02, dtype), up=normal(wid, T_UP, (I, H), 0.02, dtype),
                down=normal(wid, T_DOWN, (H, I), 0.02, dtype))


def embedding(wid: int, vocab: int, hidden: int, dtype=torch.bfloat16) -> torch.Tensor:
    return normal(wid, T_EMB, (vocab, hidden), 0.02, dtype)


def activations(wid: int, rows: int, hidden: int, dtype=torch.bfloat16, tid: int = T_X) -> torch.Tensor:
    return normal(wid, tid, (rows, hidden), 1.0, dtype)


def prior_cache(wid: int, tid: int, B: int, n_kv_heads: int, S: int, d: int) -> torch.Tensor:
    """Cache contents for positions already written, per GLOBAL kv head:
    [B, n_kv_heads, S, d] ~ N(0,1); a rank copies its own heads out of it."""
    return normal(wid, tid, (B, n_kv_heads, S, d), 1.0)


def norm_inputs(wid: int, n: int, rows: int, hidden: int, dtype=torch.bfloat16):
    """Inputs of the residual add + RMSNorm after a row-parallel layer:
    n stacked rank partials [n, rows, hidden] ~ N(0, 0.5), the residual
    stream [rows, hidden] ~ N(0, 1) and the norm weight ~ U(0.5, 1.5)."""
    return (normal(wid, T_PART, (n, rows, hidden), 0.5, dtype), normal(wid, T_RES, (rows, hidden), 1.0, dtype),
            uniform(wid, T_LNW, (hidden,), 0.5, 1.5, dtype))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 view of a bf16/fp32 CPU tensor (for the oracle)."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)
