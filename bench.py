#!/usr/bin/env python3
"""Benchmark of one tensor-parallel rank's shard of a Qwen3-style decoder
layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step runs every row of the hot path once, on rank 0, in this order:
  shard   tp_shard_weights for q, k, v, o, gate, up, down and the vocab rows
  embed   tp_embed_vocab over the workload's token ids
  prefill tp_qkv_attn (B=1, T tokens, empty cache) + tp_mlp (T rows)
  lm_head tp_lm_head over the id rows (the vocab slice of the logits)
  decode  tp_qkv_attn (B sequences, 1 token, context c) + tp_mlp (B rows)
  decode_argmax  tp_lm_head_argmax over the B decode rows (this rank's greedy
          candidates over its vocab slice)
  residual_norm  tp_residual_rmsnorm over the T prefill rows: the tp ranks'
          partials summed into the residual stream, then the next RMSNorm
  sp_norm tp_sp_residual_rmsnorm, the sequence-parallel form: rank 0's
          ceil(T / tp) token rows only, written into the gathered output
HIP events on the launch stream bracket each phase.  `value` is the layer's
prefill throughput (TFLOP/s of the prefill phase); decode GB/s, the lm_head
TFLOP/s and the other phases are reported beside it.  Inputs are synthetic,
seeded, resident in HBM before timing; buffer sets are rotated so that the
working set between two uses of a buffer exceeds the 256 MB Infinity Cache.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
MALL_BYTES = 256 << 20

WORKLOADS = {
    # configs of the same model share the vocab; each names its hidden size
    "qwen3-0.6b-tp2": dict(layer=2, vocab_from=3, n_ids=4096),
    "qwen3-32b-tp2": dict(layer=4, vocab_from=None, n_ids=4096),
    "qwen3-32b-tp16": dict(layer=5, vocab_from=None, n_ids=1024),
}


def flops_prefill(w, L, T):
    H, d = w["hidden"], w["head_dim"]
    return {"qkv": 2 * T * L.n_qkv * H, "attn": 4 * d * L.lq * T * (T + 1) // 2,
            "o_proj": 2 * T * H * L.lq * d, "gate_up": 2 * T * 2 * L.li * H, "down": 2 * T * H * L.li}


def bytes_decode(w, L, B, ctx):
    H, d = w["hidden"], w["head_dim"]
    lqd = L.lq * d
    weights = 2 * (L.n_qkv * H + H * lqd + 2 * L.li * H + H * L.li)
    kv = B * ctx * L.lkv * d * 2 * 2
    act = 2 * B * (H + L.n_qkv) + 2 * B * 2 * lqd + 2 * B * (lqd + H) + 2 * B * (H + L.li) + 2 * B * (L.li + H)
    return {"weights": weights, "kv": kv, "activations": act}


def src_sha(name):
    p = os.path.join(ROOT, "tensor_transformer_layer_rank_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profile(kernel_file):
    """HBM bytes per launch of the lm_head GEMM from the committed rocprofv3
    counter summary, or None if it is missing or was taken on another
    version of the kernel source."""
    p = os.path.join(ROOT, "profiles", "lm_head_gemm_qwen3-0.6b-tp2_hbm_traffic.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha") != src_sha(kernel_file):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Set:
    """One buffer set: full weights, the rank's local weights, caches,
    activations and outputs."""

    def __init__(self, src, w, L, c, T, B, ctx, n_ids, V, H):
        import torch
        dev, bf = "cuda", torch.bfloat16
        self.full = {k: v.clone() for k, v in src["full"].items()}
        self.emb = src["emb"].clone()
        self.ids = src["ids"].clone()
        self.x_pre = src["x_pre"].clone()
        self.x_dec = src["x_dec"].clone()
        self.x_lm = src["x_lm"].clone()
        self.kc_dec = src["kc_dec"].clone()
        self.vc_dec = src["vc_dec"].clone()
        self.kc_pre = torch.zeros(1, L.lkv, T, 128, dtype=bf, device=dev)
        self.vc_pre = torch.zeros_like(self.kc_pre)
        self.qkv = torch.empty(L.n_qkv, H, dtype=bf, device=dev)
        self.gu = torch.empty(2 * L.li, H, dtype=bf, device=dev)
        self.o = torch.empty(H, L.lq * 128, dtype=bf, device=dev)
        self.down = torch.empty(H, L.li, dtype=bf, device=dev)
        self.vocab = torch.empty(L.vocab_end - L.vocab_start, H, dtype=bf, device=dev)
        self.emb_out = torch.empty(n_ids, H, dtype=bf, device=dev)
        self.p_attn = torch.empty(T, H, dtype=bf, device=dev)
        self.p_mlp = torch.empty(T, H, dtype=bf, device=dev)
        self.d_attn = torch.empty(B, H, dtype=bf, device=dev)
        self.d_mlp = torch.empty(B, H, dtype=bf, device=dev)
        self.logits = torch.empty(n_ids, L.vocab_end - L.vocab_start, dtype=bf, device=dev)
        self.tok_val = torch.empty(B, dtype=torch.float32, device=dev)
        self.tok_idx = torch.empty(B, dtype=torch.int32, device=dev)
        self.parts = src["parts"].clone()
        self.resid = src["resid"].clone()
        self.ln_w = src["ln_w"].clone()
        self.h_res = torch.empty(T, H, dtype=bf, device=dev)
        self.y_norm = torch.empty(T, H, dtype=bf, device=dev)

    def nbytes(self):
        import torch
        return sum(t.numel() * t.element_size() for t in vars(self).values() if isinstance(t, torch.Tensor)) + \
            sum(t.numel() * t.element_size() for t in self.full.values())


def run_bench(args):
    import torch

    import synth
    import tensor_transformer_layer_rank_amd as tp

    spec = WORKLOADS[args.workload]
    w = dict(synth.WORKLOADS[spec["layer"]])
    H, V, n = w["hidden"], w["vocab"], w["tp"]
    T, B, ctx, n_ids = w["prefill_T"], w["decode_B"], w["decode_ctx"], spec["n_ids"]
    c = tp.Cfg(hidden=H, intermediate=w["intermediate"], n_q_heads=w["n_q_heads"], n_kv_heads=w["n_kv_heads"],
               head_dim=128, tp_size=n, tp_rank=0, vocab=V)
    L = tp.tp_local_dims(c)
    dev = "cuda"
    torch.cuda.set_device(0)
    wid = spec["layer"]
    vid = spec["vocab_from"] or wid

    # --- inputs (seeded, synthetic), resident in HBM --------------------------------
    full = {k: v.to(dev) for k, v in synth.full_weights(wid, w).items()}
    src = dict(full=full, emb=synth.embedding(vid, V, H).to(dev), ids=synth.token_ids(vid, n_ids, V).to(dev),
               x_pre=synth.activations(wid, T, H).to(dev), x_dec=synth.activations(wid, B, H, tid=40).to(dev),
               x_lm=synth.activations(vid, n_ids, H, tid=41).to(dev))
    kc = torch.empty(B, L.lkv, ctx, 128, dtype=torch.bfloat16)
    vc = torch.empty_like(kc)
    pk = synth.prior_cache(wid, synth.T_KC, B, w["n_kv_heads"], ctx - 1, 128)
    kc[:, :, :ctx - 1] = pk[:, L.kv_head0:L.kv_head0 + L.lkv]
    del pk
    pv = synth.prior_cache(wid, synth.T_VC, B, w["n_kv_heads"], ctx - 1, 128)
    vc[:, :, :ctx - 1] = pv[:, L.kv_head0:L.kv_head0 + L.lkv]
    del pv
    src["kc_dec"], src["vc_dec"] = kc.to(dev), vc.to(dev)
    src["parts"], src["resid"], src["ln_w"] = (t.to(dev) for t in synth.norm_inputs(wid, n, T, H))
    sets = [Set(src, w, L, c, T, B, ctx, n_ids, V, H)]
    per_set = sets[0].nbytes()
    n_sets = max(2, -(-2 * MALL_BYTES // per_set) + 1)
    while len(sets) < n_sets:
        sets.append(Set(src, w, L, c, T, B, ctx, n_ids, V, H))
    del src, full
    ws_attn_p = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_ATTN, 1, T, 0), dtype=torch.uint8, device=dev)
    ws_attn_d = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_ATTN, B, 1, ctx - 1), dtype=torch.uint8, device=dev)
    ws_mlp = torch.empty(max(tp.tp_workspace_bytes(c, tp.TP_OP_MLP, T, 1), tp.tp_workspace_bytes(c, tp.TP_OP_MLP, B, 1)),
                         dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, B, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    kinds = ((tp.TP_W_Q, "q", "qkv"), (tp.TP_W_K, "k", "qkv"), (tp.TP_W_V, "v", "qkv"), (tp.TP_W_O, "o", "o"),
             (tp.TP_W_GATE, "gate", "gu"), (tp.TP_W_UP, "up", "gu"), (tp.TP_W_DOWN, "down", "down"))
    phases = ["shard", "embed", "prefill", "lm_head", "decode", "decode_argmax", "residual_norm", "sp_norm"]
    sp0, sp1 = tp.tp_sp_rows(c, T)

    def step(s: Set, ev=None):
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        for kind, name, dst in kinds:
            tp.tp_shard_weights(c, kind, s.full[name], getattr(s, dst))
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, s.emb, s.vocab)
        rec(1)
        tp.tp_embed_vocab(c, s.ids, s.vocab, s.emb_out)
        rec(2)
        tp.tp_qkv_attn(c, s.x_pre, 1, T, 0, s.qkv, s.full["q_norm"], s.full["k_norm"], s.o, s.kc_pre, s.vc_pre, T,
                       s.p_attn, ws_attn_p)
        tp.tp_mlp(c, s.x_pre, T, s.gu, s.down, s.p_mlp, ws_mlp)
        rec(3)
        tp.tp_lm_head(c, s.x_lm, n_ids, s.vocab, s.logits)
        rec(4)
        tp.tp_qkv_attn(c, s.x_dec, B, 1, ctx - 1, s.qkv, s.full["q_norm"], s.full["k_norm"], s.o, s.kc_dec,
                       s.vc_dec, ctx, s.d_attn, ws_attn_d)
        tp.tp_mlp(c, s.x_dec, B, s.gu, s.down, s.d_mlp, ws_mlp)
        rec(5)
        tp.tp_lm_head_argmax(c, s.x_dec, B, s.vocab, s.tok_val, s.tok_idx, ws_lm)
        rec(6)
        tp.tp_residual_rmsnorm(c, s.parts, n, T, s.resid, s.ln_w, s.h_res, s.y_norm)
        rec(7)
        tp.tp_sp_residual_rmsnorm(c, s.parts, T, s.resid[sp0:sp1], s.ln_w, s.h_res[sp0:sp1], s.y_norm)
        rec(8)

    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % n_sets], events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ph = {p: 0.0 for p in phases}
    for ev in events:
        for j, p in enumerate(phases):
            ph[p] += ev[j].elapsed_time(ev[j + 1]) * 1e-3
    ph = {p: v / args.steps for p, v in ph.items()}   # seconds per step

    fp = flops_prefill(w, L, T)
    prefill_flops = sum(fp.values())
    lm_flops = 2 * n_ids * (L.vocab_end - L.vocab_start) * H
    db = bytes_decode(w, L, B, ctx)
    dec_bytes = sum(db.values())
    nv = L.vocab_end - L.vocab_start
    in_shard = int(((src_ids := sets[0].ids.cpu()) >= L.vocab_start).logical_and(src_ids < L.vocab_end).sum())
    emb_bytes = 4 * n_ids + 2 * H * in_shard + 2 * H * n_ids
    # greedy decode head: the vocab slice and the decode rows are read once;
    # one (value, id) pair per row is written
    argmax_bytes = 2 * nv * H + 2 * B * H + 8 * B
    # residual + RMSNorm: n partials and the residual read, h and y written
    norm_bytes = 2 * (n + 1) * T * H + 2 * 2 * T * H + 2 * H
    sp_rows = sp1 - sp0
    sp_bytes = 2 * (n + 1) * sp_rows * H + 2 * 2 * sp_rows * H + 2 * H
    shard_bytes = 2 * 2 * (L.n_qkv * H + H * L.lq * 128 + 2 * L.li * H + H * L.li + nv * H)

    prefill_tflops = prefill_flops / ph["prefill"] / 1e12
    lm_tflops = lm_flops / ph["lm_head"] / 1e12
    dec_gbps = dec_bytes / ph["decode"] / 1e9
    traffic = traffic_from_profile("gemm.hip")
    out = {
        "metric": "TP-shard layer prefill TFLOP/s + decode GB/s on 1 MI355X, % of roofline",
        "value": round(prefill_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} rank 0: layer prefill T={T} (B=1, empty cache), decode B={B} "
                               f"at KV context {ctx}, vocab-parallel embed + lm_head over {n_ids} ids "
                               f"(vocab {V}, local {nv} rows)",
                   "hidden": H, "intermediate_local": L.li, "q_heads_local": L.lq, "kv_heads_local": L.lkv,
                   "head_dim": 128, "tp": n, "buffer_sets": n_sets},
        "prefill_pct_mfma_peak": round(100 * prefill_tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "decode_GBps": round(dec_gbps, 1),
        "decode_pct_hbm_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
        "lm_head_TFLOPs": round(lm_tflops, 1),
        "lm_head_pct_mfma_peak": round(100 * lm_tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "decode_argmax_GBps": round(argmax_bytes / ph["decode_argmax"] / 1e9, 1),
        "decode_argmax_pct_hbm_peak": round(100 * argmax_bytes / ph["decode_argmax"] / 1e9 / HBM_PEAK_GBPS, 2),
        "residual_norm_GBps": round(norm_bytes / ph["residual_norm"] / 1e9, 1),
        "residual_norm_pct_hbm_peak": round(100 * norm_bytes / ph["residual_norm"] / 1e9 / HBM_PEAK_GBPS, 2),
        "sp_norm_GBps": round(sp_bytes / ph["sp_norm"] / 1e9, 1),
        "sp_norm_pct_hbm_peak": round(100 * sp_bytes / ph["sp_norm"] / 1e9 / HBM_PEAK_GBPS, 2),
        "embed_GBps": round(emb_bytes / ph["embed"] / 1e9, 1),
        "shard_GBps": round(shard_bytes / ph["shard"] / 1e9, 1),
        "phase_us": {p: round(v * 1e6, 2) for p, v in ph.items()},
        "work": {"prefill_GFLOP": round(prefill_flops / 1e9, 2), "lm_head_GFLOP": round(lm_flops / 1e9, 2),
                 "decode_MB": round(dec_bytes / 1e6, 2), "decode_KV_MB": round(db["kv"] / 1e6, 2)},
        "roofline": {"kernel": "gemm_persist_kernel (tp_lm_head, one launch per step)", "bound": "mfma",
                     "achieved": round(lm_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(lm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_bytes_per_launch": 2 * (n_ids * H + nv * H + n_ids * nv),
                     "traffic": traffic},
    }
    return out, (w, L, c)


def cpu_baseline(w, seconds_hint=20.0):
    """The oracle, as it stands, on a bounded sample of the prefill workload:
    rank 0's attention block and MLP over the first T_s tokens."""
    import numpy as np
    import torch

    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    oc = O.Cfg(hidden=w["hidden"], intermediate=w["intermediate"], n_q_heads=w["n_q_heads"],
               n_kv_heads=w["n_kv_heads"], head_dim=128, vocab=w["vocab"], tp_size=w["tp"], tp_rank=0)
    L = O.local_dims(oc)
    wid = [k for k, v in synth.WORKLOADS.items() if v["hidden"] == w["hidden"] and v["tp"] == w["tp"]][0]
    W = synth.full_weights(wid, w)
    f = lambda t: synth.to_f64(t)
    bits = lambda t: t.view(torch.int16).numpy()
    sh = lambda kind, name: f(torch.from_numpy(np.ascontiguousarray(O.shard(oc, kind, bits(W[name])))).view(torch.bfloat16))
    qkv = O.merge_qkv(sh(O.W_Q, "q"), sh(O.W_K, "k"), sh(O.W_V, "v"))
    gu = O.merge_gate_up(sh(O.W_GATE, "gate"), sh(O.W_UP, "up"))
    wo, wd = sh(O.W_O, "o"), sh(O.W_DOWN, "down")
    # grow the prompt up to the workload's T while one pass stays short, then
    # repeat whole passes until about `seconds_hint` of CPU time is spent
    T_s = 128
    reps, total_flops, total_t = 0, 0.0, 0.0
    while True:
        x = f(synth.activations(wid, T_s, w["hidden"]))
        fl = (2 * T_s * L.n_qkv * w["hidden"] + 4 * 128 * L.lq * T_s * (T_s + 1) // 2 +
              2 * T_s * w["hidden"] * L.lq * 128 + 2 * T_s * 3 * L.li * w["hidden"])
        kc = np.zeros((1, L.lkv, T_s, 128))
        t0 = time.perf_counter()
        O.qkv_attn(oc, x, 1, T_s, 0, qkv, f(W["q_norm"]), f(W["k_norm"]), wo, kc, kc.copy())
        O.mlp(oc, x, gu, wd)
        dt = time.perf_counter() - t0
        if T_s < w["prefill_T"] and dt * 4 < seconds_hint:
            T_s *= 2
            continue
        reps, total_flops, total_t = reps + 1, total_flops + fl, total_t + dt
        if total_t >= seconds_hint / 2:
            break
    return {"value": round(total_flops / total_t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x prefill of {T_s} tokens (B=1, empty cache) through rank 0's attention block "
                      f"and MLP, float64 NumPy oracle, {total_t:.1f} s timed"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-0.6b-tp2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the shard of one tensor-parallel rank runs on a single MI355X; "
              "collectives across GPUs are not part of this library.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    out, (w, L, c) = run_bench(args)
    out["cpu_baseline"] = None if args.no_cpu else cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
