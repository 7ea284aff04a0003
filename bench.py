#!/usr/bin/env python3
"""Benchmark of one tensor-parallel rank's shard of a Qwen3-style decoder
layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-extra]
                    [--only kv_stream|vocab]

The timed step (default workload qwen3-32b-tp2: Qwen3-32B at tp=2, rank 0)
runs every row of the hot path once, in this order:
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
`value` is the prefill phase's throughput (TFLOP/s); decode GB/s and the
other phases are reported beside it.  After the timed steps, two more
measurements run on their own buffers (not part of ms_per_step): the decode
layer of Qwen3-32B at tp=16 (batch 256 at KV context 4096, one replicated kv
head: the KV stream) and the vocab-parallel embedding + lm_head of
Qwen3-0.6B at tp=2 (4096 ids, vocab 151936).

Timing: HIP events on the launch stream (torch's current stream, which the
binding passes to every call) bracket each phase of the K timed steps; then
K more steps run with the library's per-kernel marks (tp_kernel_marks), an
event after every kernel, which gives each kernel's average duration (the
marks add an event-record gap of a few microseconds at each kernel
boundary, so the phase times come from the unmarked steps).  Inputs are synthetic,
seeded and resident in HBM before timing; buffer sets are rotated so that
the working set between two uses of a buffer exceeds the 256 MB Infinity
Cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
MALL_BYTES = 256 << 20

FULL_PHASES = ["shard", "embed", "prefill", "lm_head", "decode", "decode_argmax", "residual_norm", "sp_norm"]

WORKLOADS = {
    # layer: synth workload of the layer shapes; vocab_from: workload whose
    # vocab inputs are used (None: the layer's own); n_ids: embed / lm_head rows
    "qwen3-32b-tp2": dict(layer=4, vocab_from=None, n_ids=4096),
    "qwen3-0.6b-tp2": dict(layer=2, vocab_from=3, n_ids=4096),
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


def traffic_from_profile(summary, kernel_file):
    """HBM bytes per launch of one kernel from a committed rocprofv3 counter
    summary under profiles/, or None if it is missing or was taken on
    another version of the kernel's source file."""
    p = os.path.join(ROOT, "profiles", summary)
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


class Problem:
    """Shapes, config and source tensors (on the GPU) of one workload."""

    def __init__(self, tp, synth, name, need):
        import torch
        spec = WORKLOADS[name]
        self.name, self.need = name, need
        w = dict(synth.WORKLOADS[spec["layer"]])
        self.w = w
        self.H, self.V, self.n = w["hidden"], w["vocab"], w["tp"]
        self.T, self.B, self.ctx, self.n_ids = w["prefill_T"], w["decode_B"], w["decode_ctx"], spec["n_ids"]
        self.c = tp.Cfg(hidden=self.H, intermediate=w["intermediate"], n_q_heads=w["n_q_heads"],
                        n_kv_heads=w["n_kv_heads"], head_dim=128, tp_size=self.n, tp_rank=0, vocab=self.V)
        self.L = L = tp.tp_local_dims(self.c)
        self.nv = L.vocab_end - L.vocab_start
        wid = spec["layer"]
        vid = spec["vocab_from"] or wid
        dev = "cuda"
        H, T, B, ctx = self.H, self.T, self.B, self.ctx
        src = {}
        if need & {"shard", "prefill", "decode"}:
            src["full"] = {k: v.to(dev) for k, v in synth.full_weights(wid, w).items()}
        if need & {"shard", "embed", "lm_head", "decode_argmax"}:
            src["emb"] = synth.embedding(vid, self.V, H).to(dev)
        if "embed" in need:
            src["ids"] = synth.token_ids(vid, self.n_ids, self.V).to(dev)
        if "prefill" in need:
            src["x_pre"] = synth.activations(wid, T, H).to(dev)
        if need & {"decode", "decode_argmax"}:
            src["x_dec"] = synth.activations(wid, B, H, tid=40).to(dev)
        if "lm_head" in need:
            src["x_lm"] = synth.activations(vid, self.n_ids, H, tid=41).to(dev)
        if "decode" in need:
            kc = torch.empty(B, L.lkv, ctx, 128, dtype=torch.bfloat16)
            vc = torch.empty_like(kc)
            pk = synth.prior_cache(wid, synth.T_KC, B, w["n_kv_heads"], ctx - 1, 128)
            kc[:, :, :ctx - 1] = pk[:, L.kv_head0:L.kv_head0 + L.lkv]
            del pk
            pv = synth.prior_cache(wid, synth.T_VC, B, w["n_kv_heads"], ctx - 1, 128)
            vc[:, :, :ctx - 1] = pv[:, L.kv_head0:L.kv_head0 + L.lkv]
            del pv
            src["kc_dec"], src["vc_dec"] = kc.to(dev), vc.to(dev)
        if need & {"residual_norm", "sp_norm"}:
            src["parts"], src["resid"], src["ln_w"] = (t.to(dev) for t in synth.norm_inputs(wid, self.n, T, H))
        self.src = src
        c = self.c
        self.ws = {}
        if "prefill" in need:
            self.ws["attn_p"] = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_ATTN, 1, T, 0), dtype=torch.uint8,
                                            device=dev)
        if "decode" in need:
            self.ws["attn_d"] = torch.empty(tp.tp_workspace_bytes(c, tp.TP_OP_ATTN, B, 1, ctx - 1),
                                            dtype=torch.uint8, device=dev)
        if need & {"prefill", "decode"}:
            self.ws["mlp"] = torch.empty(max(tp.tp_workspace_bytes(c, tp.TP_OP_MLP, T, 1),
                                             tp.tp_workspace_bytes(c, tp.TP_OP_MLP, B, 1)), dtype=torch.uint8,
                                         device=dev)
        if "decode_argmax" in need:
            self.ws["lm"] = torch.empty(max(tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, B, 1), 256),
                                        dtype=torch.uint8, device=dev)

    def sets(self):
        """Buffer sets, enough that reuse distance exceeds twice the MALL."""
        first = Set(self)
        per = first.nbytes()
        n_sets = max(2, -(-2 * MALL_BYTES // per) + 1)
        return [first] + [Set(self) for _ in range(n_sets - 1)]


class Set:
    """One buffer set of a Problem: its own copies of every input, the rank's
    local weights, caches and outputs."""

    def __init__(self, P):
        import torch
        dev, bf = "cuda", torch.bfloat16
        L, H, T, B = P.L, P.H, P.T, P.B
        need, src = P.need, P.src
        self.t = {}
        t = self.t
        if "full" in src:
            self.full = {k: v.clone() for k, v in src["full"].items()}
        for k in ("emb", "ids", "x_pre", "x_dec", "x_lm", "kc_dec", "vc_dec", "parts", "resid", "ln_w"):
            if k in src:
                t[k] = src[k].clone()
        if need & {"shard", "prefill", "decode"}:
            t["qkv"] = torch.empty(L.n_qkv, H, dtype=bf, device=dev)
            t["gu"] = torch.empty(2 * L.li, H, dtype=bf, device=dev)
            t["o"] = torch.empty(H, L.lq * 128, dtype=bf, device=dev)
            t["down"] = torch.empty(H, L.li, dtype=bf, device=dev)
            if "shard" not in need:      # local weights sharded once, outside the timed steps
                self._shard_layer(P)
        if need & {"shard", "embed", "lm_head", "decode_argmax"}:
            t["vocab"] = torch.empty(P.nv, H, dtype=bf, device=dev)
            if "shard" not in need:
                import tensor_transformer_layer_rank_amd as tp
                tp.tp_shard_weights(P.c, tp.TP_W_VOCAB, t["emb"], t["vocab"])
        if "embed" in need:
            t["emb_out"] = torch.empty(P.n_ids, H, dtype=bf, device=dev)
        if "prefill" in need:
            t["kc_pre"] = torch.zeros(1, L.lkv, T, 128, dtype=bf, device=dev)
            t["vc_pre"] = torch.zeros_like(t["kc_pre"])
            t["p_attn"] = torch.empty(T, H, dtype=bf, device=dev)
            t["p_mlp"] = torch.empty(T, H, dtype=bf, device=dev)
        if "decode" in need:
            t["d_attn"] = torch.empty(B, H, dtype=bf, device=dev)
            t["d_mlp"] = torch.empty(B, H, dtype=bf, device=dev)
        if "lm_head" in need:
            t["logits"] = torch.empty(P.n_ids, P.nv, dtype=bf, device=dev)
        if "decode_argmax" in need:
            t["tok_val"] = torch.empty(B, dtype=torch.float32, device=dev)
            t["tok_idx"] = torch.empty(B, dtype=torch.int32, device=dev)
        if need & {"residual_norm", "sp_norm"}:
            t["h_res"] = torch.empty(T, H, dtype=bf, device=dev)
            t["y_norm"] = torch.empty(T, H, dtype=bf, device=dev)

    def _shard_layer(self, P):
        import tensor_transformer_layer_rank_amd as tp
        for kind, name, dst in KINDS:
            tp.tp_shard_weights(P.c, kind, self.full[name], self.t[dst])

    def nbytes(self):
        n = sum(v.numel() * v.element_size() for v in self.t.values())
        if hasattr(self, "full"):
            n += sum(v.numel() * v.element_size() for v in self.full.values())
        return n


KINDS = ()


def run_phase(tp, P, s, phase):
    """Enqueue one phase of the step on buffer set s."""
    c, t, L = P.c, s.t, P.L
    if phase == "shard":
        for kind, name, dst in KINDS:
            tp.tp_shard_weights(c, kind, s.full[name], t[dst])
        tp.tp_shard_weights(c, tp.TP_W_VOCAB, t["emb"], t["vocab"])
    elif phase == "embed":
        tp.tp_embed_vocab(c, t["ids"], t["vocab"], t["emb_out"])
    elif phase == "prefill":
        tp.tp_qkv_attn(c, t["x_pre"], 1, P.T, 0, t["qkv"], s.full["q_norm"], s.full["k_norm"], t["o"], t["kc_pre"],
                       t["vc_pre"], P.T, t["p_attn"], P.ws["attn_p"])
        tp.tp_mlp(c, t["x_pre"], P.T, t["gu"], t["down"], t["p_mlp"], P.ws["mlp"])
    elif phase == "lm_head":
        tp.tp_lm_head(c, t["x_lm"], P.n_ids, t["vocab"], t["logits"])
    elif phase == "decode":
        tp.tp_qkv_attn(c, t["x_dec"], P.B, 1, P.ctx - 1, t["qkv"], s.full["q_norm"], s.full["k_norm"], t["o"],
                       t["kc_dec"], t["vc_dec"], P.ctx, t["d_attn"], P.ws["attn_d"])
        tp.tp_mlp(c, t["x_dec"], P.B, t["gu"], t["down"], t["d_mlp"], P.ws["mlp"])
    elif phase == "decode_argmax":
        tp.tp_lm_head_argmax(c, t["x_dec"], P.B, t["vocab"], t["tok_val"], t["tok_idx"], P.ws["lm"])
    elif phase == "residual_norm":
        tp.tp_residual_rmsnorm(c, t["parts"], P.n, P.T, t["resid"], t["ln_w"], t["h_res"], t["y_norm"])
    elif phase == "sp_norm":
        sp0, sp1 = tp.tp_sp_rows(c, P.T)
        tp.tp_sp_residual_rmsnorm(c, t["parts"], P.T, t["resid"][sp0:sp1], t["ln_w"], t["h_res"][sp0:sp1],
                                  t["y_norm"])
    else:
        raise ValueError(phase)


MAX_MARKS = 64


def time_steps(tp, P, sets, phases, steps, warmup):
    """Runs warmup steps, then `steps` timed steps with HIP events at the
    phase boundaries only, then `steps` more with the library's per-kernel
    marks armed (an event after every kernel).  The marks add a small gap
    at each kernel boundary (an event record, a few microseconds), so the
    phase times and the step time come from the first pass and the
    per-kernel times from the second.  Returns (wall seconds of the first
    pass, seconds per phase per step, [(phase, kernel name, average seconds)]
    in launch order)."""
    import torch
    for i in range(warmup):
        for ph in phases:
            run_phase(tp, P, sets[i % len(sets)], ph)
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)
    pev = [[mk() for _ in range(len(phases) + 1)] for _ in range(steps)]
    kev = [[mk() for _ in range(MAX_MARKS)] for _ in range(steps)]
    k0 = [mk() for _ in range(steps)]
    # torch creates an event at its first record; do that now, outside the
    # timed region, so that the library can be handed the handles
    for e in sum(pev + kev, []) + k0:
        e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s = sets[i % len(sets)]
        pev[i][0].record()
        for j, ph in enumerate(phases):
            run_phase(tp, P, s, ph)
            pev[i][j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # second pass: per-kernel marks
    ph_marks, names = [], None
    for i in range(steps):
        s = sets[i % len(sets)]
        tp.tp_kernel_marks(kev[i])
        bounds = [0]
        k0[i].record()
        for ph in phases:
            run_phase(tp, P, s, ph)
            bounds.append(tp.tp_kernel_marks_used())
        if names is None:
            names = tp.tp_kernel_mark_names()
        tp.tp_kernel_marks([])
        ph_marks.append(bounds)
    torch.cuda.synchronize()
    ph_t = {p: 0.0 for p in phases}
    n_k = ph_marks[0][-1]
    if n_k >= MAX_MARKS:
        raise RuntimeError("more kernels per step than timing marks")
    k_t = [0.0] * n_k
    for i in range(steps):
        for j, p in enumerate(phases):
            ph_t[p] += pev[i][j].elapsed_time(pev[i][j + 1]) * 1e-3
        for k in range(n_k):
            prev = k0[i] if k == 0 else kev[i][k - 1]
            k_t[k] += prev.elapsed_time(kev[i][k]) * 1e-3
    ph_t = {p: v / steps for p, v in ph_t.items()}
    bounds = ph_marks[0]
    kernels = []
    for j, p in enumerate(phases):
        for k in range(bounds[j], bounds[j + 1]):
            kernels.append((p, names[k], k_t[k] / steps))
    return wall, ph_t, kernels


def find_kernel(kernels, phase, pred):
    for p, name, t in kernels:
        if p == phase and pred(name):
            return name, t
    return None, None


def gemm_dims(name):
    """(M, N, K) of a GEMM-family mark name, e.g. gemm_tile<256,256,2>/silu[4096x24576x5120]."""
    m = re.search(r"\[(\d+)x(\d+)x(\d+)\]$", name)
    return tuple(int(v) for v in m.groups())


def kernel_table(kernels):
    out, seen = {}, {}
    for p, name, t in kernels:
        key = f"{p}:{name}"
        seen[key] = seen.get(key, 0) + 1
        if seen[key] > 1:
            key += f"#{seen[key]}"
        out[key] = round(t * 1e6, 2)
    return out


def run_bench(args):
    import torch

    import synth
    import tensor_transformer_layer_rank_amd as tp

    global KINDS
    KINDS = ((tp.TP_W_Q, "q", "qkv"), (tp.TP_W_K, "k", "qkv"), (tp.TP_W_V, "v", "qkv"), (tp.TP_W_O, "o", "o"),
             (tp.TP_W_GATE, "gate", "gu"), (tp.TP_W_UP, "up", "gu"), (tp.TP_W_DOWN, "down", "down"))
    torch.cuda.set_device(0)

    if args.only == "kv_stream":
        return extra_kv_stream(tp, synth, args, {}), None
    if args.only == "vocab":
        return extra_vocab(tp, synth, args, {}), None
    # ---- the timed step: every row of the path on the main workload -------------
    P = Problem(tp, synth, args.workload, set(FULL_PHASES))
    sets = P.sets()
    torch.cuda.synchronize()
    wall, ph, kernels = time_steps(tp, P, sets, FULL_PHASES, args.steps, args.warmup)
    w, L, H, T, B, ctx, n_ids, nv, n = P.w, P.L, P.H, P.T, P.B, P.ctx, P.n_ids, P.nv, P.n
    n_sets = len(sets)
    in_shard = int(((ids := sets[0].t["ids"].cpu()) >= L.vocab_start).logical_and(ids < L.vocab_end).sum())
    del sets

    fp = flops_prefill(w, L, T)
    prefill_flops = sum(fp.values())
    lm_flops = 2 * n_ids * nv * H
    db = bytes_decode(w, L, B, ctx)
    dec_bytes = sum(db.values())
    emb_bytes = 4 * n_ids + 2 * H * in_shard + 2 * H * n_ids
    argmax_bytes = 2 * nv * H + 2 * B * H + 8 * B
    norm_bytes = 2 * (n + 1) * T * H + 2 * 2 * T * H + 2 * H
    sp0, sp1 = tp.tp_sp_rows(P.c, T)
    sp_rows = sp1 - sp0
    sp_bytes = 2 * (n + 1) * sp_rows * H + 2 * 2 * sp_rows * H + 2 * H
    shard_bytes = 2 * 2 * (L.n_qkv * H + H * L.lq * 128 + 2 * L.li * H + H * L.li + nv * H)
    prefill_tflops = prefill_flops / ph["prefill"] / 1e12
    lm_tflops = lm_flops / ph["lm_head"] / 1e12
    dec_gbps = dec_bytes / ph["decode"] / 1e9

    # dominant kernel: the prefill gate_up GEMM with its SiLU epilogue
    # (the first SiLU launch: under a tail schedule it covers the leading
    # columns only, so its work is read from the launched M x N x K)
    gu_name, gu_t = find_kernel(kernels, "prefill", lambda s: "/silu[" in s and s.startswith("gemm_tile"))
    gm, gn, gk = gemm_dims(gu_name) if gu_name else (T, 2 * L.li, H)
    gu_flops = 2 * gm * gn * gk
    gu_bytes = 2 * (gm * gk + gn * gk + gm * gn // 2)
    gu_traffic = traffic_from_profile(f"gate_up_gemm_{args.workload}_hbm_traffic.txt", "gemm.hip")
    gu_tflops = gu_flops / gu_t / 1e12 if gu_t else None
    cover = (f"one launch over all {L.li} output columns" if gn // 2 >= L.li
             else f"the launch over output columns [0, {gn // 2}) of {L.li}")
    roofline = {"kernel": f"{gu_name} (tp_mlp gate_up + SiLU*up of prefill {T} x {2 * L.li} x {H}: {cover})",
                "bound": "mfma", "achieved": round(gu_tflops, 1) if gu_tflops else None,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tflops / MFMA_BF16_PEAK_TFLOPS, 4) if gu_tflops else None,
                "avg_launch_us": round(gu_t * 1e6, 2) if gu_t else None,
                "algorithmic_bytes_per_launch": gu_bytes, "traffic": gu_traffic}
    # decode attention of the main workload
    da_name, da_t = find_kernel(kernels, "decode", lambda s: s.startswith("attn_flash/decode"))
    da_bytes = db["kv"] + 2 * B * L.lq * 128 * 2
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
                               f"(vocab {P.V}, local {nv} rows)",
                   "hidden": H, "intermediate_local": L.li, "q_heads_local": L.lq, "kv_heads_local": L.lkv,
                   "head_dim": 128, "tp": n, "buffer_sets": n_sets},
        "prefill_pct_mfma_peak": round(100 * prefill_tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "decode_GBps": round(dec_gbps, 1),
        "decode_pct_hbm_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
        "decode_attention_GBps": round(da_bytes / da_t / 1e9, 1) if da_t else None,
        "lm_head_TFLOPs": round(lm_tflops, 1),
        "lm_head_pct_mfma_peak": round(100 * lm_tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "decode_argmax_GBps": round(argmax_bytes / ph["decode_argmax"] / 1e9, 1),
        "residual_norm_GBps": round(norm_bytes / ph["residual_norm"] / 1e9, 1),
        "sp_norm_GBps": round(sp_bytes / ph["sp_norm"] / 1e9, 1),
        "embed_GBps": round(emb_bytes / ph["embed"] / 1e9, 1),
        "shard_GBps": round(shard_bytes / ph["shard"] / 1e9, 1),
        "phase_us": {p: round(v * 1e6, 2) for p, v in ph.items()},
        "kernel_us": kernel_table(kernels),
        "work": {"prefill_GFLOP": round(prefill_flops / 1e9, 2), "lm_head_GFLOP": round(lm_flops / 1e9, 2),
                 "decode_MB": round(dec_bytes / 1e6, 2), "decode_KV_MB": round(db["kv"] / 1e6, 2)},
        "roofline": roofline,
    }

    # ---- beside the step: the KV stream (32B tp=16 decode) and the 0.6B lm_head -
    if not args.no_extra and args.workload == "qwen3-32b-tp2" and args.only is None:
        extra_kv_stream(tp, synth, args, out)
        extra_vocab(tp, synth, args, out)
    return out, P


def extra_kv_stream(tp, synth, args, out):
    """The decode layer of Qwen3-32B at tp=16 (rank 0): B=256 at KV context
    4096 over one replicated kv head; the attention kernel is the KV stream."""
    import torch
    PK = Problem(tp, synth, "qwen3-32b-tp16", {"decode"})
    ks = PK.sets()
    torch.cuda.synchronize()
    _, kph, kk = time_steps(tp, PK, ks, ["decode"], args.steps, args.warmup)
    del ks
    kdb = bytes_decode(PK.w, PK.L, PK.B, PK.ctx)
    ka_name, ka_t = find_kernel(kk, "decode", lambda s: s.startswith("attn_flash/decode"))
    ka_bytes = kdb["kv"] + 2 * PK.B * PK.L.lq * 128 * 2
    ka_gbps = ka_bytes / ka_t / 1e9
    w_t = sum(t for p, nm, t in kk if not nm.startswith("attn_flash"))
    out["kv_stream"] = {
        "workload": f"qwen3-32b-tp16 rank 0 decode: B={PK.B} at KV context {PK.ctx}, 1 replicated kv head "
                    f"(4 local q heads)",
        "decode_GBps": round(sum(kdb.values()) / kph["decode"] / 1e9, 1),
        "decode_us": round(kph["decode"] * 1e6, 2),
        "attention_GBps": round(ka_gbps, 1), "attention_us": round(ka_t * 1e6, 2),
        "attention_pct_hbm_peak": round(100 * ka_gbps / HBM_PEAK_GBPS, 2),
        "weight_stream_us": round(w_t * 1e6, 2),
        "weight_stream_GBps": round(kdb["weights"] / w_t / 1e9, 1),
        "kernel_us": kernel_table(kk)}
    out["roofline_hbm"] = {
        "kernel": f"{ka_name} (tp_qkv_attn decode attention, KV stream B={PK.B} x ctx {PK.ctx})",
        "bound": "hbm", "achieved": round(ka_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(ka_gbps / HBM_PEAK_GBPS, 4), "avg_launch_us": round(ka_t * 1e6, 2),
        "algorithmic_bytes_per_launch": ka_bytes,
        "traffic": traffic_from_profile("decode_attention_qwen3-32b-tp16_hbm_traffic.txt", "attn_flash.hip")}
    del PK
    return out


def extra_vocab(tp, synth, args, out):
    """The vocab-parallel embedding + lm_head of Qwen3-0.6B at tp=2 (rank 0)."""
    import torch
    PL = Problem(tp, synth, "qwen3-0.6b-tp2", {"embed", "lm_head"})
    ls = PL.sets()
    torch.cuda.synchronize()
    _, lph, lk = time_steps(tp, PL, ls, ["embed", "lm_head"], args.steps, args.warmup)
    del ls
    l_flops = 2 * PL.n_ids * PL.nv * PL.H
    out["vocab_0.6b"] = {
        "workload": f"qwen3-0.6b-tp2 rank 0: embed + lm_head over {PL.n_ids} ids, hidden {PL.H}, "
                    f"local vocab {PL.nv}",
        "lm_head_TFLOPs": round(l_flops / lph["lm_head"] / 1e12, 1),
        "lm_head_pct_mfma_peak": round(100 * l_flops / lph["lm_head"] / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
        "embed_us": round(lph["embed"] * 1e6, 2), "kernel_us": kernel_table(lk)}
    del PL
    return out


def cpu_baseline(w, seconds_hint=20.0):
    """The oracle, as it stands, in its float32 variant, on a bounded sample
    of the prefill workload: rank 0's attention block and MLP over the first
    T_s tokens."""
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
    ft = np.float32
    f = lambda t: t.float().numpy()
    store = lambda x: O.bf16(x).astype(ft)
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
        kc = np.zeros((1, L.lkv, T_s, 128), ft)
        t0 = time.perf_counter()
        O.qkv_attn(oc, x, 1, T_s, 0, qkv, f(W["q_norm"]), f(W["k_norm"]), wo, kc, kc.copy(), store=store, ft=ft)
        O.mlp(oc, x, gu, wd, store=store, ft=ft)
        dt = time.perf_counter() - t0
        if T_s < w["prefill_T"] and dt * 4 < seconds_hint:
            T_s *= 2
            continue
        reps, total_flops, total_t = reps + 1, total_flops + fl, total_t + dt
        if total_t >= seconds_hint / 2:
            break
    return {"value": round(total_flops / total_t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x prefill of {T_s} tokens (B=1, empty cache) through rank 0's attention block "
                      f"and MLP at the workload's shapes, float32 variant of the NumPy oracle, "
                      f"{total_t:.1f} s timed"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-32b-tp2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the KV-stream and 0.6B lm_head measurements")
    ap.add_argument("--only", choices=["kv_stream", "vocab"], default=None,
                    help="run only one of the measurements beside the step (for profiling); prints its object")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the shard of one tensor-parallel rank runs on a single MI355X; "
              "collectives across GPUs are not part of this library.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    out, P = run_bench(args)
    if P is not None:
        out["cpu_baseline"] = None if args.no_cpu else cpu_baseline(P.w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
