"""ctypes binding of libtplayer.so: the C-ABI entry points under the same
names, taking torch tensors (device memory) and marshalling them to pointers.

No computation happens here. If the library is missing the import of this
module succeeds but every call raises, telling how to build it; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# TPL_LIBRARY selects another build of the same library (the AddressSanitizer
# build of the host code, libtplayer_asan.so, for the CPU tests of the C ABI)
LIB_PATH = os.environ.get("TPL_LIBRARY") or os.path.join(HERE, "libtplayer.so")

TPL_OK, TPL_ERR_INVALID_ARG, TPL_ERR_UNSUPPORTED, TPL_ERR_HIP = 0, 1, 2, 3
TPL_F32, TPL_BF16 = 0, 1
TPL_BLOCK_ATTN, TPL_BLOCK_MLP = 0, 1
TPL_BWD_SHARD, TPL_BWD_REPLICATED, TPL_BWD_SHARD_RECOMPUTE = 0, 1, 2
TPL_XENT_LOCAL, TPL_XENT_FINISH = 0, 1


class TplDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("tp", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("seq", ctypes.c_int32), ("micro_batch", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class TplBlockParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln_g", "ln_b", "w_in", "b_in", "w_out")]


class TplBlockGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("d_w_in", "d_b_in", "d_w_out", "d_ln_g", "d_ln_b", "d_b_out")]


class TplError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


_lib = None
_VP, _I32, _I64, _F32P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


def library_available() -> bool:
    return os.path.exists(LIB_PATH)


def lib() -> ctypes.CDLL:
    """Load libtplayer.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tensor_transformer_layer_03_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.tp_layer_saved_bytes.restype = ctypes.c_size_t
        L.tp_layer_saved_bytes.argtypes = [P(TplDesc), ctypes.c_int]
        L.vocab_parallel_xent_stats_bytes.restype = ctypes.c_size_t
        L.vocab_parallel_xent_stats_bytes.argtypes = [P(TplDesc)]
        L.vocab_parallel_embedding_ws_bytes.restype = ctypes.c_size_t
        L.vocab_parallel_embedding_ws_bytes.argtypes = [P(TplDesc)]
        L.vocab_parallel_embedding_fwd.argtypes = [P(TplDesc), _VP, _VP, _VP, _VP]
        L.vocab_parallel_embedding_bwd.argtypes = [P(TplDesc), _VP, _VP, _VP, _VP, _VP]
        L.vocab_parallel_embedding_bwd_noalloc.argtypes = [P(TplDesc), _VP, _VP, _VP, _VP]
        L.tp_layer_shard_fwd.argtypes = [P(TplDesc), ctypes.c_int, _VP, P(TplBlockParams), _VP, _VP, _VP]
        L.shard_partial_sum.argtypes = [P(TplDesc), P(ctypes.c_void_p), _I32, _VP, _VP, _VP, _I64, _I32, _VP]
        L.tp_layer_shard_bwd.argtypes = [P(TplDesc), ctypes.c_int, ctypes.c_int, _VP, _VP, _VP,
                                         P(TplBlockParams), _VP, _VP, _VP, P(TplBlockGrads), _VP]
        L.vocab_parallel_xent_fwd.argtypes = [P(TplDesc), ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _VP,
                                              P(ctypes.c_void_p), _VP, _VP, _VP, _VP]
        L.vocab_parallel_xent_bwd.argtypes = [P(TplDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float,
                                              _VP, _VP, _VP]
        L.tpl_gemm.argtypes = [_I32, _I32, _I32, _I64, _I64, _I64, _VP, _I64, _VP, _I64, _VP, _VP, _I64, _I32, _VP]
        L.tpl_rows_gather.argtypes = [_VP, ctypes.c_int64, _VP, ctypes.c_int64, ctypes.c_int64, _VP, _VP]
        L.tpl_rows_gather.restype = _I32
        L.tpl_rows_expand.argtypes = [_VP, ctypes.c_int64, _VP, ctypes.c_int64, ctypes.c_int64, _VP, _VP]
        L.tpl_rows_expand.restype = _I32
        L.tpl_trace_enable.argtypes = [_I32]
        L.tpl_trace_enable.restype = _I32
        L.tpl_trace_read.argtypes = [P(ctypes.c_int32), P(ctypes.c_float), P(ctypes.c_double), _I32]
        L.tpl_trace_read.restype = _I32
        L.tpl_trace_kernel_name.argtypes = [_I32]
        L.tpl_trace_kernel_name.restype = ctypes.c_char_p
        L.tpl_status_string.argtypes = [ctypes.c_int]
        L.tpl_status_string.restype = ctypes.c_char_p
        for fn in ("tp_layer_shard_fwd", "shard_partial_sum", "tp_layer_shard_bwd", "vocab_parallel_xent_fwd",
                   "vocab_parallel_xent_bwd", "tpl_gemm"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


EXPORTED = ("tp_layer_saved_bytes", "tp_layer_shard_fwd", "shard_partial_sum", "tp_layer_shard_bwd",
            "vocab_parallel_xent_stats_bytes", "vocab_parallel_xent_fwd",
            "vocab_parallel_embedding_ws_bytes", "vocab_parallel_embedding_fwd", "vocab_parallel_embedding_bwd",
            "vocab_parallel_embedding_bwd_noalloc", "vocab_parallel_xent_bwd", "tpl_rows_gather", "tpl_rows_expand", "tpl_gemm", "tpl_trace_enable",
            "tpl_trace_read", "tpl_trace_kernel_name", "tpl_status_string")


def status_string(status: int) -> str:
    try:
        return lib().tpl_status_string(status).decode()
    except Exception:  # library not loadable: still report the code
        return f"status {status}"


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(fn: str, status: int):
    if status != TPL_OK:
        raise TplError(fn, status)


def make_desc(hidden, heads, head_dim, ffn, tp, rank, seq, micro_batch, vocab, causal, dtype, ln_eps=1e-5):
    return TplDesc(hidden, heads, head_dim, ffn, tp, rank, seq, micro_batch, vocab, int(causal),
                   TPL_BF16 if dtype in ("bf16", TPL_BF16, torch.bfloat16) else TPL_F32, ln_eps)


def block_params(ln_g, ln_b, w_in, b_in, w_out) -> TplBlockParams:
    return TplBlockParams(_ptr(ln_g), _ptr(ln_b), _ptr(w_in), _ptr(b_in), _ptr(w_out))


def block_grads(d_w_in=None, d_b_in=None, d_w_out=None, d_ln_g=None, d_ln_b=None, d_b_out=None) -> TplBlockGrads:
    return TplBlockGrads(*(_ptr(t) for t in (d_w_in, d_b_in, d_w_out, d_ln_g, d_ln_b, d_b_out)))


# ------------------------------------------------------------------ entry points

def tp_layer_saved_bytes(desc: TplDesc, block: int) -> int:
    return int(lib().tp_layer_saved_bytes(ctypes.byref(desc), block))


def vocab_parallel_xent_stats_bytes(desc: TplDesc) -> int:
    return int(lib().vocab_parallel_xent_stats_bytes(ctypes.byref(desc)))


def vocab_parallel_embedding_ws_bytes(desc: TplDesc) -> int:
    return int(lib().vocab_parallel_embedding_ws_bytes(ctypes.byref(desc)))


def vocab_parallel_embedding_fwd(desc, tokens, emb_in, x_partial, stream=None):
    _check("vocab_parallel_embedding_fwd", lib().vocab_parallel_embedding_fwd(
        ctypes.byref(desc), _ptr(tokens), _ptr(emb_in), _ptr(x_partial), _stream(stream)))


def vocab_parallel_embedding_bwd(desc, tokens, d_out, d_emb_in, workspace, stream=None):
    _check("vocab_parallel_embedding_bwd", lib().vocab_parallel_embedding_bwd(
        ctypes.byref(desc), _ptr(tokens), _ptr(d_out), _ptr(d_emb_in), _ptr(workspace), _stream(stream)))


def vocab_parallel_embedding_bwd_noalloc(desc, tokens, d_out, d_emb_in, stream=None):
    _check("vocab_parallel_embedding_bwd_noalloc", lib().vocab_parallel_embedding_bwd_noalloc(
        ctypes.byref(desc), _ptr(tokens), _ptr(d_out), _ptr(d_emb_in), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 4 << 20   # TPL_NOALLOC_SCRATCH_BYTES of include/tp_layer.h


def tp_layer_shard_fwd(desc, block, x, params: TplBlockParams, partial, saved, stream=None):
    _check("tp_layer_shard_fwd", lib().tp_layer_shard_fwd(
        ctypes.byref(desc), block, _ptr(x), ctypes.byref(params), _ptr(partial), _ptr(saved), _stream(stream)))


def shard_partial_sum(desc, partials: Sequence, bias, residual, out, rows: int, cols: int, stream=None):
    arr = (ctypes.c_void_p * len(partials))(*[_ptr(p) for p in partials])
    _check("shard_partial_sum", lib().shard_partial_sum(
        ctypes.byref(desc), arr, len(partials), _ptr(bias), _ptr(residual), _ptr(out), rows, cols,
        _stream(stream)))


def tp_layer_shard_bwd(desc, block, phase, dy, d_ln_sum, x, params: TplBlockParams, saved, d_ln_partial, dx,
                       grads: TplBlockGrads, stream=None):
    _check("tp_layer_shard_bwd", lib().tp_layer_shard_bwd(
        ctypes.byref(desc), block, phase, _ptr(dy), _ptr(d_ln_sum), _ptr(x), ctypes.byref(params), _ptr(saved),
        _ptr(d_ln_partial), _ptr(dx), ctypes.byref(grads), _stream(stream)))


def vocab_parallel_xent_fwd(desc, phase, hidden=None, emb=None, targets=None, loss_mask=None, logits=None,
                            stats=None, all_stats: Sequence | None = None, lse=None, loss_rows=None, loss=None,
                            stream=None):
    arr = None
    if all_stats is not None:
        arr = (ctypes.c_void_p * len(all_stats))(*[_ptr(p) for p in all_stats])
    _check("vocab_parallel_xent_fwd", lib().vocab_parallel_xent_fwd(
        ctypes.byref(desc), phase, _ptr(hidden), _ptr(emb), _ptr(targets), _ptr(loss_mask), _ptr(logits),
        _ptr(stats), arr, _ptr(lse), _ptr(loss_rows), _ptr(loss), _stream(stream)))


def vocab_parallel_xent_bwd(desc, hidden, emb, targets, loss_mask, logits, lse, loss, dloss: float,
                            d_hidden_partial, d_emb, stream=None):
    _check("vocab_parallel_xent_bwd", lib().vocab_parallel_xent_bwd(
        ctypes.byref(desc), _ptr(hidden), _ptr(emb), _ptr(targets), _ptr(loss_mask), _ptr(logits), _ptr(lse),
        _ptr(loss), float(dloss), _ptr(d_hidden_partial), _ptr(d_emb), _stream(stream)))


def tpl_rows_gather(src, n_src, rows, n, row_bytes, dst, stream=None):
    _check("tpl_rows_gather", lib().tpl_rows_gather(_ptr(src), n_src, _ptr(rows), n, row_bytes, _ptr(dst),
                                                    _stream(stream)))


def tpl_rows_expand(src, n_src, pos, n_dst, row_bytes, dst, stream=None):
    _check("tpl_rows_expand", lib().tpl_rows_expand(_ptr(src), n_src, _ptr(pos), n_dst, row_bytes, _ptr(dst),
                                                    _stream(stream)))


def tpl_gemm(dtype, a_kmajor, b_kmajor, M, N, K, A, lda, B, ldb, bias, C, ldc, c_f32, stream=None):
    _check("tpl_gemm", lib().tpl_gemm(
        dtype, int(a_kmajor), int(b_kmajor), M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(bias), _ptr(C), ldc,
        int(c_f32), _stream(stream)))


def tpl_trace_enable(capacity: int) -> int:
    return int(lib().tpl_trace_enable(capacity))


def tpl_trace_read(max_n: int = 1 << 16) -> list[tuple[str, float, float]]:
    """[(kernel name, milliseconds, algorithmic work)] of the traced launches."""
    ids = (ctypes.c_int32 * max_n)()
    ms = (ctypes.c_float * max_n)()
    work = (ctypes.c_double * max_n)()
    n = lib().tpl_trace_read(ids, ms, work, max_n)
    if n < 0:
        raise RuntimeError("tpl_trace_read failed")
    return [(lib().tpl_trace_kernel_name(ids[i]).decode(), float(ms[i]), float(work[i])) for i in range(n)]
