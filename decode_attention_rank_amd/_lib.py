"""ctypes binding of libkvlr.so (include/kvlr.h).

Argument marshalling only: every function here converts tensors to device
pointers, calls the C entry point of the same name on the current HIP stream
and raises KvlrError on a non-zero status. Loading fails loudly when the
library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.environ.get("KVLR_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libkvlr.so")

KVLR_OK = 0
KVLR_ERR_INVALID_ARGUMENT = 1
KVLR_ERR_UNSUPPORTED = 2
KVLR_ERR_WORKSPACE_TOO_SMALL = 3
KVLR_ERR_HIP = 4

KVLR_DTYPE_BF16 = 0
KVLR_DTYPE_F32 = 1
KVLR_KEYS_LATENT = 0
KVLR_KEYS_EXACT = 1

EXPORTED = (
    "kvlr_append_encode", "kvlr_project_queries", "kvlr_qproj_width", "kvlr_route_pages",
    "kvlr_decode_attn", "kvlr_decode_attn_upproject", "kvlr_upproject", "kvlr_workspace_bytes",
    "kvlr_workspace_init", "kvlr_fold_output_weights", "kvlr_output_projection",
    "kvlr_status_string", "kvlr_version",
)


class KvlrError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


class kvlr_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_q_heads", "num_kv_heads", "head_dim", "page_size", "rank_v", "rank_k",
        "dtype", "key_mode", "num_phys_pages")]


class kvlr_cache(ctypes.Structure):
    _fields_ = [("v_lat", ctypes.c_void_p), ("k_lat", ctypes.c_void_p), ("k_exact", ctypes.c_void_p)]


class kvlr_factors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("A_v", "B_v", "A_k", "B_k", "W_pred")]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIG = {
    "kvlr_append_encode": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors),
                            ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _P, _I, _I, _I, _P], _I),
    "kvlr_project_queries": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _P, _I, _P], _I),
    "kvlr_qproj_width": ([ctypes.POINTER(kvlr_shape)], _I),
    "kvlr_route_pages": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_cache), _P, _P, _P, _I, _I,
                          _I, _I, _P, _P, _P, _P, ctypes.c_size_t, _I, _P], _I),
    "kvlr_decode_attn": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _I,
                          _P, _P, _I, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _I, _P], _I),
    "kvlr_decode_attn_upproject": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors),
                                    ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _I, _P, _P, _I,
                                    ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _I, _P], _I),
    "kvlr_upproject": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _P, _I, _P], _I),
    "kvlr_workspace_bytes": ([ctypes.POINTER(kvlr_shape), _I, _I], ctypes.c_size_t),
    "kvlr_fold_output_weights": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _I,
                                  _P, _P], _I),
    "kvlr_output_projection": ([ctypes.POINTER(kvlr_shape), _P, _P, _I, _P, _I, _P], _I),
    "kvlr_workspace_init": ([_P, ctypes.c_size_t, _P], _I),
    "kvlr_status_string": ([_I], ctypes.c_char_p),
    "kvlr_version": ([], _I),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m decode_attention_rank_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIG.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn: str, status: int):
    if status != KVLR_OK:
        raise KvlrError(fn, status, lib().kvlr_status_string(status).decode())


def make_shape(*, num_q_heads, num_kv_heads, head_dim, page_size, rank_v, rank_k, dtype, key_mode,
               num_phys_pages) -> kvlr_shape:
    return kvlr_shape(num_q_heads, num_kv_heads, head_dim, page_size, rank_v, rank_k, dtype,
                      key_mode, num_phys_pages)


def make_cache(v_lat=None, k_lat=None, k_exact=None) -> kvlr_cache:
    return kvlr_cache(_ptr(v_lat), _ptr(k_lat), _ptr(k_exact))


def make_factors(A_v=None, B_v=None, A_k=None, B_k=None, W_pred=None) -> kvlr_factors:
    return kvlr_factors(_ptr(A_v), _ptr(B_v), _ptr(A_k), _ptr(B_k), _ptr(W_pred))


def kvlr_version() -> int:
    return lib().kvlr_version()


def kvlr_status_string(status: int) -> str:
    return lib().kvlr_status_string(status).decode()


def kvlr_qproj_width(shape: kvlr_shape) -> int:
    return lib().kvlr_qproj_width(ctypes.byref(shape))


def kvlr_workspace_bytes(shape: kvlr_shape, batch: int, max_pages_per_seq: int) -> int:
    return lib().kvlr_workspace_bytes(ctypes.byref(shape), batch, max_pages_per_seq)


def kvlr_workspace_init(workspace, ws_bytes: int, stream=None):
    _check("kvlr_workspace_init", lib().kvlr_workspace_init(_ptr(workspace), ws_bytes, _stream(stream)))


def kvlr_append_encode(shape, factors, cache, k_new, v_new, cu_new, seq_lens_before, page_table,
                       max_pages_per_seq, batch, total_new, stream=None):
    _check("kvlr_append_encode", lib().kvlr_append_encode(
        ctypes.byref(shape), ctypes.byref(factors), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
        _ptr(cu_new), _ptr(seq_lens_before), _ptr(page_table), max_pages_per_seq, batch, total_new,
        _stream(stream)))


def kvlr_project_queries(shape, factors, q, q_proj, batch, stream=None):
    _check("kvlr_project_queries", lib().kvlr_project_queries(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(q), _ptr(q_proj), batch, _stream(stream)))


def kvlr_route_pages(shape, cache, q_proj, seq_lens, page_table, max_pages_per_seq, topk_num,
                     topk_den, k_max, sel_pages, sel_counts, page_scores, workspace, ws_bytes,
                     batch, stream=None):
    _check("kvlr_route_pages", lib().kvlr_route_pages(
        ctypes.byref(shape), ctypes.byref(cache), _ptr(q_proj), _ptr(seq_lens), _ptr(page_table),
        max_pages_per_seq, topk_num, topk_den, k_max, _ptr(sel_pages), _ptr(sel_counts),
        _ptr(page_scores), _ptr(workspace), ws_bytes, batch, _stream(stream)))


def kvlr_decode_attn(shape, cache, q, q_proj, seq_lens, page_table, max_pages_per_seq, sel_pages,
                     sel_counts, k_max, softmax_scale, z_out, lse_out, workspace, ws_bytes, batch,
                     stream=None):
    _check("kvlr_decode_attn", lib().kvlr_decode_attn(
        ctypes.byref(shape), ctypes.byref(cache), _ptr(q), _ptr(q_proj), _ptr(seq_lens),
        _ptr(page_table), max_pages_per_seq, _ptr(sel_pages), _ptr(sel_counts), k_max,
        float(softmax_scale), _ptr(z_out), _ptr(lse_out), _ptr(workspace), ws_bytes, batch,
        _stream(stream)))


def kvlr_decode_attn_upproject(shape, factors, cache, q, q_proj, seq_lens, page_table,
                               max_pages_per_seq, sel_pages, sel_counts, k_max, softmax_scale,
                               z_out, lse_out, o_out, workspace, ws_bytes, batch, stream=None):
    _check("kvlr_decode_attn_upproject", lib().kvlr_decode_attn_upproject(
        ctypes.byref(shape), ctypes.byref(factors), ctypes.byref(cache), _ptr(q), _ptr(q_proj),
        _ptr(seq_lens), _ptr(page_table), max_pages_per_seq, _ptr(sel_pages), _ptr(sel_counts),
        k_max, float(softmax_scale), _ptr(z_out), _ptr(lse_out), _ptr(o_out), _ptr(workspace),
        ws_bytes, batch, _stream(stream)))


def kvlr_upproject(shape, factors, z, o_out, batch, stream=None):
    _check("kvlr_upproject", lib().kvlr_upproject(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(z), _ptr(o_out), batch, _stream(stream)))


def kvlr_fold_output_weights(shape, factors, W_o, hidden, F_out, stream=None):
    _check("kvlr_fold_output_weights", lib().kvlr_fold_output_weights(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(W_o), hidden, _ptr(F_out), _stream(stream)))


def kvlr_output_projection(shape, F, z, hidden, out, batch, stream=None):
    _check("kvlr_output_projection", lib().kvlr_output_projection(
        ctypes.byref(shape), _ptr(F), _ptr(z), hidden, _ptr(out), batch, _stream(stream)))
