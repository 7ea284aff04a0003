"""Python binding of libtpshard (one tensor-parallel rank's shard of a
Qwen3-style decoder layer on MI355X).  Argument marshalling only: every step
of the computation runs in the HIP kernels behind the C ABI (include/tpshard.h).

Tensors are torch tensors on the GPU (device memory and streams only); each
call is enqueued on torch's current stream.  A non-zero status from the
library raises TpError.  If the shared library is not built, importing the
binding works but every call raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")

TP_F32, TP_BF16 = 0, 1
TP_W_Q, TP_W_K, TP_W_V, TP_W_O, TP_W_GATE, TP_W_UP, TP_W_DOWN, TP_W_VOCAB = range(8)
TP_OP_ATTN, TP_OP_MLP, TP_OP_LM_ARGMAX = 0, 1, 2

EXPORTS = ("tp_local_dims", "tp_workspace_bytes", "tp_status_str", "tp_kernel_marks", "tp_kernel_marks_used",
           "tp_kernel_mark_name", "tp_shard_weights", "tp_embed_vocab", "tp_qkv_attn", "tp_mlp", "tp_lm_head",
           "tp_lm_head_argmax", "tp_lm_head_argmax_noalloc", "tp_argmax_combine", "tp_residual_rmsnorm",
           "tp_rmsnorm_rows", "tp_last_token_rows", "tp_sp_rows", "tp_sp_residual_rmsnorm")


class TpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class tp_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("tp_size", ctypes.c_int32),
                ("tp_rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("vocab", ctypes.c_int64),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class tp_local(ctypes.Structure):
    _fields_ = [("lq", ctypes.c_int32), ("lkv", ctypes.c_int32), ("kv_head0", ctypes.c_int32),
                ("li", ctypes.c_int32), ("n_qkv", ctypes.c_int64), ("vocab_start", ctypes.c_int64),
                ("vocab_end", ctypes.c_int64)]


@dataclass
class Cfg:
    """Model shape and rank (mirrors tp_cfg)."""
    hidden: int
    intermediate: int = 0
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 128
    tp_size: int = 1
    tp_rank: int = 0
    dtype: int = TP_BF16
    vocab: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    def c(self) -> tp_cfg:
        return tp_cfg(self.hidden, self.intermediate, self.n_q_heads, self.n_kv_heads, self.head_dim,
                      self.tp_size, self.tp_rank, self.dtype, self.vocab, self.rms_eps, self.rope_theta)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m tensor_transformer_layer_rank_amd.build")
        # The tensors handed to the library belong to torch's HIP runtime, so
        # the library must bind to that same runtime: torch is loaded first,
        # and its libamdhip64 (soname libamdhip64.so.7) then satisfies the
        # library's dependency.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        _check_single_hip_runtime()
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        C = ctypes.POINTER(tp_cfg)
        L.tp_local_dims.argtypes = [C, ctypes.POINTER(tp_local)]
        L.tp_workspace_bytes.argtypes = [C, ctypes.c_int, I64, I64, I64, ctypes.POINTER(SZ)]
        L.tp_status_str.argtypes = [ctypes.c_int]
        L.tp_status_str.restype = ctypes.c_char_p
        L.tp_kernel_marks.argtypes = [ctypes.POINTER(ctypes.c_void_p), I32]
        L.tp_kernel_marks_used.argtypes = []
        L.tp_kernel_mark_name.argtypes = [I32]
        L.tp_kernel_mark_name.restype = ctypes.c_char_p
        L.tp_shard_weights.argtypes = [C, ctypes.c_int, P, P, P]
        L.tp_embed_vocab.argtypes = [C, P, I64, P, P, P]
        L.tp_qkv_attn.argtypes = [C, P, I32, I32, I32, P, P, P, P, P, P, I32, P, P, P, P, SZ, P]
        L.tp_mlp.argtypes = [C, P, I64, P, P, P, P, P, SZ, P]
        L.tp_lm_head.argtypes = [C, P, I64, P, I64, P, P, P]
        L.tp_lm_head_argmax.argtypes = [C, P, I64, P, I64, P, P, P, P, SZ, P]
        L.tp_lm_head_argmax_noalloc.argtypes = [C, P, I64, P, I64, P, P, P, P]
        L.tp_argmax_combine.argtypes = [P, P, I32, I64, P, P, P]
        L.tp_residual_rmsnorm.argtypes = [C, P, I32, I64, P, P, P, P, P]
        L.tp_rmsnorm_rows.argtypes = [C, P, I64, P, I64, P, P, P]
        L.tp_last_token_rows.argtypes = [ctypes.POINTER(I32), I32, ctypes.POINTER(I32)]
        L.tp_sp_rows.argtypes = [C, I64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.tp_sp_residual_rmsnorm.argtypes = [C, P, I64, P, P, P, P, P]
        for name in EXPORTS:
            if name not in ("tp_status_str", "tp_kernel_mark_name"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check_single_hip_runtime():
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return
    paths = {os.path.realpath(l.split()[-1]) for l in maps if "libamdhip64" in l and "/" in l}
    if len(paths) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded ({sorted(paths)}); import torch before loading libtpshard")


def _check(st: int):
    if st != 0:
        raise TpError(st, lib().tp_status_str(st).decode())


def _ptr(t):
    """Device pointer of a tensor, or NULL for None (no copies, no checks:
    shapes and dtypes are the caller's contract, see tpshard.h)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def tp_local_dims(cfg: Cfg) -> tp_local:
    out = tp_local()
    _check(lib().tp_local_dims(ctypes.byref(cfg.c()), ctypes.byref(out)))
    return out


def tp_workspace_bytes(cfg: Cfg, op: int, B: int, T: int, past_len: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tp_workspace_bytes(ctypes.byref(cfg.c()), op, B, T, past_len, ctypes.byref(n)))
    return n.value


def tp_status_str(status: int) -> str:
    return lib().tp_status_str(status).decode()


def tp_kernel_marks(events):
    """Arms per-kernel timing marks on this thread: `events` are
    torch.cuda.Event(enable_timing=True) objects, recorded in order after each
    kernel that the following calls launch.  An empty list disarms."""
    import torch
    handles = []
    for e in events:
        if e.cuda_event == 0:          # torch creates the event at its first record
            e.record(torch.cuda.current_stream())
        handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * max(len(handles), 1))(*handles)
    _check(lib().tp_kernel_marks(arr if handles else None, len(handles)))


def tp_kernel_marks_used() -> int:
    return lib().tp_kernel_marks_used()


def tp_kernel_mark_names() -> list:
    """Names of the kernels marked since the last tp_kernel_marks call."""
    L = lib()
    return [L.tp_kernel_mark_name(i).decode() for i in range(L.tp_kernel_marks_used())]


def tp_shard_weights(cfg: Cfg, kind: int, full, dst, stream=None):
    _check(lib().tp_shard_weights(ctypes.byref(cfg.c()), kind, _ptr(full), _ptr(dst), _stream(stream)))


def tp_embed_vocab(cfg: Cfg, ids, vocab_local, out, stream=None):
    _check(lib().tp_embed_vocab(ctypes.byref(cfg.c()), _ptr(ids), ids.numel(), _ptr(vocab_local), _ptr(out),
                                _stream(stream)))


def tp_qkv_attn(cfg: Cfg, x, B: int, T: int, past_len: int, w_qkv, q_norm_w, k_norm_w, w_o, k_cache, v_cache,
                S_max: int, out_partial, workspace, q_out=None, attn_out=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tp_qkv_attn(ctypes.byref(cfg.c()), _ptr(x), B, T, past_len, _ptr(w_qkv), _ptr(q_norm_w),
                             _ptr(k_norm_w), _ptr(w_o), _ptr(k_cache), _ptr(v_cache), S_max, _ptr(q_out),
                             _ptr(attn_out), _ptr(out_partial), _ptr(workspace), ws_bytes, _stream(stream)))


def tp_mlp(cfg: Cfg, x, M: int, w_gate_up, w_down, out_partial, workspace, h_out=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tp_mlp(ctypes.byref(cfg.c()), _ptr(x), M, _ptr(w_gate_up), _ptr(w_down), _ptr(h_out),
                        _ptr(out_partial), _ptr(workspace), ws_bytes, _stream(stream)))


def _x_rows(x, rows):
    return 0 if rows is None else x.shape[0]


def tp_lm_head(cfg: Cfg, x, M: int, vocab_local, logits_local, stream=None, rows=None):
    """rows: optional int32 device tensor [M] of row indices into x."""
    _check(lib().tp_lm_head(ctypes.byref(cfg.c()), _ptr(x), M, _ptr(rows), _x_rows(x, rows), _ptr(vocab_local),
                            _ptr(logits_local), _stream(stream)))


def tp_lm_head_argmax(cfg: Cfg, x, M: int, vocab_local, out_val, out_idx, workspace, stream=None, rows=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tp_lm_head_argmax(ctypes.byref(cfg.c()), _ptr(x), M, _ptr(rows), _x_rows(x, rows), _ptr(vocab_local),
                                   _ptr(out_val), _ptr(out_idx), _ptr(workspace), ws_bytes, _stream(stream)))


def tp_lm_head_argmax_noalloc(cfg: Cfg, x, M: int, vocab_local, out_val, out_idx, stream=None, rows=None):
    """tp_lm_head_argmax with its candidates in the library's static device
    array: no workspace, no allocation."""
    _check(lib().tp_lm_head_argmax_noalloc(ctypes.byref(cfg.c()), _ptr(x), M, _ptr(rows), _x_rows(x, rows),
                                           _ptr(vocab_local), _ptr(out_val), _ptr(out_idx), _stream(stream)))


def tp_argmax_combine(vals, idx, n_shards: int, M: int, out_idx, out_val=None, stream=None):
    _check(lib().tp_argmax_combine(_ptr(vals), _ptr(idx), n_shards, M, _ptr(out_idx), _ptr(out_val), _stream(stream)))


def tp_residual_rmsnorm(cfg: Cfg, partials, n_partials: int, M: int, residual, norm_w, h_out, y_out, stream=None):
    _check(lib().tp_residual_rmsnorm(ctypes.byref(cfg.c()), _ptr(partials), n_partials, M, _ptr(residual),
                                     _ptr(norm_w), _ptr(h_out), _ptr(y_out), _stream(stream)))


def tp_rmsnorm_rows(cfg: Cfg, x, rows, n_rows: int, norm_w, y_out, stream=None):
    """y_out[m] = RMSNorm(x[rows[m]]) * norm_w; rows None: x rows 0..n_rows-1."""
    _check(lib().tp_rmsnorm_rows(ctypes.byref(cfg.c()), _ptr(x), 0 if x is None else x.shape[0], _ptr(rows), n_rows,
                                 _ptr(norm_w), _ptr(y_out), _stream(stream)))


def tp_last_token_rows(seq_lens):
    """Row of each sequence's last token in the packed batch (a list)."""
    n = len(seq_lens)
    lens = (ctypes.c_int32 * max(n, 1))(*seq_lens)
    out = (ctypes.c_int32 * max(n, 1))()
    _check(lib().tp_last_token_rows(lens, n, out))
    return list(out)[:n]


def tp_sp_rows(cfg: Cfg, M: int):
    """Rank cfg.tp_rank's token slice (row0, row1) of M tokens."""
    r0, r1 = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().tp_sp_rows(ctypes.byref(cfg.c()), M, ctypes.byref(r0), ctypes.byref(r1)))
    return r0.value, r1.value


def tp_sp_residual_rmsnorm(cfg: Cfg, partials, M: int, residual_slice, norm_w, h_slice_out, y_gathered,
                           stream=None):
    _check(lib().tp_sp_residual_rmsnorm(ctypes.byref(cfg.c()), _ptr(partials), M, _ptr(residual_slice),
                                        _ptr(norm_w), _ptr(h_slice_out), _ptr(y_gathered), _stream(stream)))
