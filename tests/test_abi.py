"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and validates arguments before any launch.  No GPU work:
every device entry point here is called with arguments that validation
rejects (or with an empty size), so nothing is enqueued.  Those calls pass
fake device addresses, so they run only where no GPU is visible: on a GPU
host a regression in the validation order would launch a kernel on an
unmapped address instead of failing an assertion."""
import ctypes
import os
import re

import pytest

import oracle as O
import tensor_transformer_layer_rank_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

OK, E_NULL, E_RANK, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_RANGE, E_LAUNCH, E_KIND = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|const char\*|size_t)\s+(tp_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(tp.EXPORTS)
    L = tp.lib()
    for n in names:
        assert hasattr(L, n), n


def test_struct_layouts():
    assert ctypes.sizeof(tp.tp_cfg) == 48
    assert ctypes.sizeof(tp.tp_local) == 40


def _ocfg(c: tp.Cfg):
    return O.Cfg(hidden=c.hidden, intermediate=c.intermediate, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
                 head_dim=c.head_dim, vocab=c.vocab, tp_size=c.tp_size, tp_rank=c.tp_rank)


SHAPES = [
    dict(hidden=1024, intermediate=3072, n_q_heads=16, n_kv_heads=8, vocab=151936),    # Qwen3-0.6B
    dict(hidden=5120, intermediate=25600, n_q_heads=64, n_kv_heads=8, vocab=151936),   # Qwen3-32B
    dict(hidden=64, intermediate=192, n_q_heads=4, n_kv_heads=1, vocab=37),
    dict(hidden=64, intermediate=192, n_q_heads=12, n_kv_heads=3, vocab=10),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 6, 8, 16])
def test_local_dims_match_oracle(shape, n):
    for r in range(n):
        c = tp.Cfg(**shape, tp_size=n, tp_rank=r)
        try:
            ref = O.local_dims(_ocfg(c))
        except ValueError:
            with pytest.raises(tp.TpError) as ei:
                tp.tp_local_dims(c)
            assert ei.value.status == E_SHAPE
            continue
        got = tp.tp_local_dims(c)
        assert (got.lq, got.lkv, got.kv_head0, got.li, got.n_qkv, got.vocab_start, got.vocab_end) == \
               (ref.lq, ref.lkv, ref.kv_head0, ref.li, ref.n_qkv, ref.vocab_start, ref.vocab_end)


def _status(fn, *args):
    try:
        fn(*args)
    except tp.TpError as e:
        return e.status
    return OK


def test_config_errors():
    base = dict(hidden=64, intermediate=192, n_q_heads=4, n_kv_heads=2, vocab=100)
    assert _status(tp.tp_local_dims, tp.Cfg(**base, tp_size=2, tp_rank=2)) == E_RANK
    assert _status(tp.tp_local_dims, tp.Cfg(**base, tp_size=0, tp_rank=0)) == E_RANK
    assert _status(tp.tp_local_dims, tp.Cfg(**base, tp_size=2, tp_rank=-1)) == E_RANK
    assert _status(tp.tp_local_dims, tp.Cfg(**{**base, "n_q_heads": 6}, tp_size=4)) == E_SHAPE
    assert _status(tp.tp_local_dims, tp.Cfg(**{**base, "intermediate": 190}, tp_size=4)) == E_SHAPE
    assert _status(tp.tp_local_dims, tp.Cfg(**{**base, "n_q_heads": 12, "n_kv_heads": 4}, tp_size=6)) == E_SHAPE
    assert _status(tp.tp_local_dims, tp.Cfg(**base, tp_size=2, dtype=7)) == E_DTYPE
    assert _status(tp.tp_local_dims, tp.Cfg(**{**base, "hidden": 0}, tp_size=2)) == E_SHAPE
    assert tp.tp_status_str(E_WS) == "workspace too small"


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# device entry points called with fake addresses: host-only
host_only = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses are only passed where no GPU is visible")


class Fake:
    """A stand-in 'tensor' with a fake device address; used only where the
    library must reject the call before launching anything."""

    def __init__(self, addr, numel=0, esize=1):
        self.addr, self.n, self.es = addr, numel, esize

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return self.es

    @property
    def shape(self):
        return (self.n,)


class NullStream:
    cuda_stream = 0


A = Fake(1 << 40)           # 16-byte aligned
MIS = Fake((1 << 40) + 8)   # misaligned


@host_only
def test_shard_and_embed_validation():
    c = tp.Cfg(hidden=64, intermediate=192, n_q_heads=4, n_kv_heads=2, vocab=100, tp_size=2)
    s = NullStream()
    assert _status(tp.tp_shard_weights, c, 99, A, A, s) == E_KIND
    assert _status(tp.tp_shard_weights, c, tp.TP_W_Q, None, A, s) == E_NULL
    assert _status(tp.tp_shard_weights, c, tp.TP_W_Q, A, MIS, s) == E_ALIGN
    cm = tp.Cfg(hidden=64, intermediate=192, tp_size=2)          # MLP-only shape
    assert _status(tp.tp_shard_weights, cm, tp.TP_W_K, A, A, s) == E_SHAPE
    assert _status(tp.tp_shard_weights, cm, tp.TP_W_VOCAB, A, A, s) == E_SHAPE
    ids = Fake(1 << 40, numel=0)
    assert _status(tp.tp_embed_vocab, c, ids, A, A, s) == OK           # empty: no-op
    assert _status(tp.tp_embed_vocab, c, Fake((1 << 40) + 4, 5), A, A, s) == E_ALIGN
    assert _status(tp.tp_embed_vocab, c, Fake(1 << 40, 5), None, A, s) == E_NULL


@host_only
def test_attn_validation():
    c = tp.Cfg(hidden=256, intermediate=512, n_q_heads=4, n_kv_heads=2, head_dim=128, tp_size=2)
    s = NullStream()
    args = lambda **kw: dict(dict(cfg=c, x=A, B=2, T=3, past_len=4, w_qkv=A, q_norm_w=A, k_norm_w=A, w_o=A,
                                  k_cache=A, v_cache=A, S_max=16, out_partial=A, workspace=Fake(1 << 40, 16, 1),
                                  stream=s), **kw)

    def st(**kw):
        try:
            tp.tp_qkv_attn(**args(**kw))
        except tp.TpError as e:
            return e.status
        return OK

    assert st(workspace=Fake(1 << 40, 16, 1)) == E_WS
    assert st(past_len=14) == E_RANGE                     # 14 + 3 > 16
    assert st(T=-1) == E_RANGE
    assert st(x=None) == E_NULL
    assert st(k_cache=MIS) == E_ALIGN
    assert st(attn_out=MIS) == E_ALIGN
    assert st(workspace=None) == E_NULL
    assert st(B=0) == OK                                  # empty: no-op
    assert st(cfg=tp.Cfg(**{**c.__dict__, "dtype": tp.TP_F32})) == E_DTYPE
    assert st(cfg=tp.Cfg(**{**c.__dict__, "head_dim": 64})) == E_SHAPE
    assert st(cfg=tp.Cfg(**{**c.__dict__, "hidden": 260})) == E_SHAPE
    need = tp.tp_workspace_bytes(c, tp.TP_OP_ATTN, 2, 3, 4)
    assert need >= 2 * (2 * 3) * 2 * 128 * 2           # at least the q and attention-output buffers


@host_only
def test_mlp_and_lm_head_validation():
    c = tp.Cfg(hidden=256, intermediate=512, tp_size=2)
    s = NullStream()
    assert _status(tp.tp_mlp, c, A, 0, A, A, A, None, None, s) == OK        # M = 0
    assert _status(tp.tp_mlp, c, A, -1, A, A, A, None, None, s) == E_RANGE
    assert _status(tp.tp_mlp, c, A, 4, A, A, A, None, None, s) == E_NULL     # no workspace
    assert _status(tp.tp_mlp, c, A, 4, A, A, A, Fake(1 << 40, 8, 1), None, s) == E_WS
    assert _status(tp.tp_mlp, tp.Cfg(hidden=256, intermediate=20, tp_size=2), A, 4, A, A, A,
                   Fake(1 << 40, 1 << 20, 1), None, s) == E_SHAPE              # li = 10
    assert tp.tp_workspace_bytes(c, tp.TP_OP_MLP, 4, 1) >= 4 * 256 * 2
    cv = tp.Cfg(hidden=256, vocab=1000, tp_size=4, tp_rank=3)
    assert _status(tp.tp_lm_head, cv, A, 0, A, A, s) == OK
    assert _status(tp.tp_lm_head, cv, A, 4, MIS, A, s) == E_ALIGN
    assert _status(tp.tp_lm_head, tp.Cfg(hidden=256, tp_size=1), A, 4, A, A, s) == E_SHAPE


@host_only
def test_lm_head_argmax_and_combine_validation():
    s = NullStream()
    cv = tp.Cfg(hidden=256, vocab=1000, tp_size=4, tp_rank=3)
    need = tp.tp_workspace_bytes(cv, tp.TP_OP_LM_ARGMAX, 5, 1)
    assert need >= 5 * 8                                          # a candidate per row
    ws = Fake(1 << 40, need, 1)
    assert _status(tp.tp_lm_head_argmax, cv, A, 0, A, A, A, ws, s) == OK          # M = 0
    assert _status(tp.tp_lm_head_argmax, cv, A, -1, A, A, A, ws, s) == E_RANGE
    assert _status(tp.tp_lm_head_argmax, cv, A, 5, A, None, A, ws, s) == E_NULL
    assert _status(tp.tp_lm_head_argmax, cv, A, 5, A, A, A, None, s) == E_NULL    # no workspace
    assert _status(tp.tp_lm_head_argmax, cv, A, 5, A, A, A, Fake(1 << 40, need - 1, 1), s) == E_WS
    assert _status(tp.tp_lm_head_argmax, cv, MIS, 5, A, A, A, ws, s) == E_ALIGN
    assert _status(tp.tp_lm_head_argmax, tp.Cfg(hidden=256, vocab=1000, tp_size=4, dtype=tp.TP_F32),
                   A, 5, A, A, A, ws, s) == E_DTYPE
    assert _status(tp.tp_lm_head_argmax, tp.Cfg(hidden=256, tp_size=1), A, 5, A, A, A, ws, s) == E_SHAPE
    assert _status(tp.tp_argmax_combine, A, A, 0, 5, A, None, s) == E_RANGE       # no shards
    assert _status(tp.tp_argmax_combine, A, A, 2, 0, A, None, s) == OK            # M = 0
    assert _status(tp.tp_argmax_combine, None, A, 2, 5, A, None, s) == E_NULL
    assert _status(tp.tp_argmax_combine, A, Fake((1 << 40) + 2, 5), 2, 5, A, None, s) == E_ALIGN


def test_lm_head_argmax_workspace_paths():
    """The decode head's workspace holds 8-byte candidates: one per row and
    workgroup (256 of them) when up to 64 rows with a hidden size of at most
    1024 (a multiple of 256) keep the activations on chip, else one per row
    and logits tile.  Host logic only."""
    c = tp.Cfg(hidden=1024, vocab=151936, tp_size=2)
    for M in (1, 16, 33, 64):
        assert tp.tp_workspace_bytes(c, tp.TP_OP_LM_ARGMAX, M, 1) == M * 256 * 8
    for cfg, M in ((c, 65), (tp.Cfg(hidden=520, vocab=151936, tp_size=2), 8),
                   (tp.Cfg(hidden=5120, vocab=151936, tp_size=2), 8)):
        need = tp.tp_workspace_bytes(cfg, tp.TP_OP_LM_ARGMAX, M, 1)
        assert need >= M * 8 and need % 16 == 0
        assert need != M * 256 * 8                                  # the logits-GEMM path


@host_only
def test_residual_rmsnorm_validation():
    s = NullStream()
    c = tp.Cfg(hidden=256, tp_size=2)
    assert _status(tp.tp_residual_rmsnorm, c, A, 2, 0, A, A, A, A, s) == OK             # M = 0
    assert _status(tp.tp_residual_rmsnorm, c, A, 2, -1, A, A, A, A, s) == E_RANGE
    assert _status(tp.tp_residual_rmsnorm, c, A, -1, 5, A, A, A, A, s) == E_RANGE       # negative count
    assert _status(tp.tp_residual_rmsnorm, c, None, 0, 0, A, A, None, A, s) == OK       # plain norm, M = 0
    assert _status(tp.tp_residual_rmsnorm, c, None, 1, 5, A, A, A, A, s) == E_NULL      # partials needed
    assert _status(tp.tp_residual_rmsnorm, c, A, 1, 5, A, A, None, A, s) == E_NULL      # h_out needed
    assert _status(tp.tp_residual_rmsnorm, c, None, 0, 5, A, A, None, None, s) == E_NULL
    assert _status(tp.tp_residual_rmsnorm, c, A, 2, 5, None, A, A, A, s) == E_NULL
    assert _status(tp.tp_residual_rmsnorm, c, A, 2, 5, A, A, A, None, s) == E_NULL
    assert _status(tp.tp_residual_rmsnorm, c, A, 2, 5, A, A, MIS, A, s) == E_ALIGN
    assert _status(tp.tp_residual_rmsnorm, tp.Cfg(hidden=250, tp_size=2), A, 2, 5, A, A, A, A, s) == E_SHAPE
    assert _status(tp.tp_residual_rmsnorm, tp.Cfg(hidden=8200, tp_size=2), A, 2, 5, A, A, A, A, s) == E_SHAPE
    assert _status(tp.tp_residual_rmsnorm, tp.Cfg(hidden=256, tp_size=2, dtype=tp.TP_F32),
                   A, 2, 5, A, A, A, A, s) == E_DTYPE


@pytest.mark.parametrize("M,n", [(0, 2), (7, 2), (9, 4), (5, 8), (4096, 2), (1023, 16)])
def test_sp_rows_match_oracle(M, n):
    for r in range(n):
        assert tp.tp_sp_rows(tp.Cfg(hidden=64, tp_size=n, tp_rank=r), M) == O.sp_rows(M, n, r)


@host_only
def test_sp_residual_rmsnorm_validation():
    s = NullStream()
    c = tp.Cfg(hidden=256, tp_size=4, tp_rank=3)
    assert _status(tp.tp_sp_rows, c, -1) == E_RANGE
    assert _status(tp.tp_sp_rows, tp.Cfg(hidden=256, tp_size=4, tp_rank=4), 8) == E_RANK
    assert _status(tp.tp_sp_residual_rmsnorm, c, A, 6, A, A, A, A, s) == OK      # rank 3 owns no row of 6
    assert _status(tp.tp_sp_residual_rmsnorm, c, A, 6, None, A, None, A, s) == OK
    assert _status(tp.tp_sp_residual_rmsnorm, c, A, -1, A, A, A, A, s) == E_RANGE
    assert _status(tp.tp_sp_residual_rmsnorm, c, A, 8, A, A, None, A, s) == E_NULL
    assert _status(tp.tp_sp_residual_rmsnorm, c, A, 8, A, A, A, MIS, s) == E_ALIGN
    assert _status(tp.tp_sp_residual_rmsnorm, tp.Cfg(hidden=260, tp_size=4), A, 8, A, A, A, A, s) == E_SHAPE
    assert _status(tp.tp_sp_residual_rmsnorm, tp.Cfg(hidden=256, tp_size=4, dtype=tp.TP_F32),
                   A, 8, A, A, A, A, s) == E_DTYPE


def test_kernel_marks_host_logic():
    """Arming and disarming the per-kernel timing marks is host-only state:
    no event is recorded until a device entry point launches a kernel."""
    L = tp.lib()
    assert L.tp_kernel_marks(None, 0) == OK
    assert L.tp_kernel_marks(None, -1) == E_RANGE
    assert L.tp_kernel_marks(None, 3) == E_NULL
    assert L.tp_kernel_marks_used() == 0
    assert L.tp_kernel_mark_name(0) == b""
    assert L.tp_kernel_mark_name(-1) == b""


@host_only
def test_descriptor_range_limits():
    """Buffer-descriptor byte ranges are 32-bit: the kernels address a tile's
    rows (at most 256 of them) and a cache slab's positions relative to one
    base, so a row length of 2^22 elements or more, or an S_max of 2^24 or
    more, is rejected on the host."""
    s = NullStream()
    big = 1 << 22
    c = tp.Cfg(hidden=256, intermediate=512, n_q_heads=4, n_kv_heads=2, head_dim=128, tp_size=2)
    ws = Fake(1 << 40, 1 << 30, 1)
    assert _status(tp.tp_qkv_attn, c, A, 1, 1, 0, A, A, A, A, A, A, 1 << 24, A, ws, None, None, s) == E_SHAPE
    cb = tp.Cfg(hidden=big, intermediate=512, n_q_heads=4, n_kv_heads=2, head_dim=128, tp_size=2)
    assert _status(tp.tp_qkv_attn, cb, A, 1, 1, 0, A, A, A, A, A, A, 8, A, ws, None, None, s) == E_SHAPE
    assert _status(tp.tp_mlp, tp.Cfg(hidden=big, intermediate=512, tp_size=2), A, 4, A, A, A, ws, None, s) == E_SHAPE
    assert _status(tp.tp_mlp, tp.Cfg(hidden=256, intermediate=2 * big, tp_size=2), A, 4, A, A, A, ws, None,
                   s) == E_SHAPE
    cv = tp.Cfg(hidden=big, vocab=1000, tp_size=2)
    assert _status(tp.tp_lm_head, cv, A, 4, A, A, s) == E_SHAPE
    assert _status(tp.tp_lm_head_argmax, cv, A, 4, A, A, A, ws, s) == E_SHAPE


@host_only
def test_rmsnorm_rows_and_head_rows_validation():
    s = NullStream()
    c = tp.Cfg(hidden=256, tp_size=2)
    assert _status(tp.tp_rmsnorm_rows, c, A, A, 0, A, A, s) == OK                 # n_rows = 0
    assert _status(tp.tp_rmsnorm_rows, c, A, A, -1, A, A, s) == E_RANGE
    assert _status(tp.tp_rmsnorm_rows, c, Fake(1 << 40), None, 5, A, A, s) == E_RANGE    # 5 rows of a 0-row x
    assert _status(tp.tp_rmsnorm_rows, c, Fake(1 << 40, 9), Fake((1 << 40) + 2), 5, A, A, s) == E_ALIGN
    assert _status(tp.tp_rmsnorm_rows, c, A, A, 5, A, A, s) == E_RANGE                  # row list, 0-row x
    assert _status(tp.tp_rmsnorm_rows, c, Fake(1 << 40, 9), A, 5, A, None, s) == E_NULL
    assert _status(tp.tp_rmsnorm_rows, tp.Cfg(hidden=260, tp_size=2), A, A, 5, A, A, s) == E_SHAPE
    assert _status(tp.tp_rmsnorm_rows, tp.Cfg(hidden=256, tp_size=2, dtype=tp.TP_F32), A, A, 5, A, A, s) == E_DTYPE
    cv = tp.Cfg(hidden=256, vocab=1000, tp_size=4, tp_rank=1)
    ws = Fake(1 << 40, 1 << 20, 1)
    lib = tp.lib()
    assert lib.tp_lm_head(cv.c(), A.addr, 4, (1 << 40) + 2, 8, A.addr, A.addr, None) == E_ALIGN
    assert lib.tp_lm_head(cv.c(), A.addr, 4, 1 << 40, 0, A.addr, A.addr, None) == E_RANGE
    assert lib.tp_lm_head(cv.c(), A.addr, 4, 1 << 40, 1 << 22, A.addr, A.addr, None) == E_SHAPE   # 2 GiB of rows
    assert lib.tp_lm_head_argmax(cv.c(), A.addr, 4, 1 << 40, 0, A.addr, A.addr, A.addr, ws.addr, ws.n, None) == E_RANGE
    cf = tp.Cfg(hidden=256, vocab=1000, tp_size=4, dtype=tp.TP_F32)
    assert lib.tp_lm_head(cf.c(), A.addr, 4, 1 << 40, 8, A.addr, A.addr, None) == E_DTYPE


def test_last_token_rows():
    assert tp.tp_last_token_rows([5, 5, 5]) == list(O.last_token_rows([5, 5, 5]))
    assert tp.tp_last_token_rows([3, 1, 7, 2]) == list(O.last_token_rows([3, 1, 7, 2]))
    assert tp.tp_last_token_rows([]) == []
    assert _status(tp.tp_last_token_rows, [2, 0]) == E_RANGE
    assert _status(tp.tp_last_token_rows, [1 << 30, 1 << 30, 1 << 30]) == E_SHAPE
