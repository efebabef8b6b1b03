"""ctypes binding of libkvlr.so (include/kvlr.h).

Argument marshalling only: every function here converts tensors to device
pointers, calls the C entry point of the same name on the current HIP stream
and raises KvlrError on a non-zero status. Loading fails loudly when the
library has not been built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.environ.get("KVLR_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libkvlr.so")

KVLR_OK = 0
KVLR_ERR_INVALID_ARGUMENT = 1
KVLR_ERR_UNSUPPORTED = 2
KVLR_ERR_WORKSPACE_TOO_SMALL = 3
KVLR_ERR_HIP = 4
KVLR_ERR_NUMERICAL = 5

KVLR_DTYPE_BF16 = 0
KVLR_DTYPE_F32 = 1
KVLR_DTYPE_BF16_FP8 = 2
KVLR_KEYS_LATENT = 0
KVLR_KEYS_EXACT = 1

EXPORTED = (
    "kvlr_append_encode", "kvlr_append_encode_project", "kvlr_project_queries", "kvlr_qproj_width", "kvlr_route_pages",
    "kvlr_decode_attn", "kvlr_decode_attn_upproject", "kvlr_upproject", "kvlr_workspace_bytes",
    "kvlr_workspace_init", "kvlr_fold_output_weights", "kvlr_output_projection",
    "kvlr_status_string", "kvlr_version", "kvlr_fit_workspace_bytes", "kvlr_fit_moments",
    "kvlr_fit_solve", "kvlr_fit_factors", "kvlr_choose_residual_ranks",
    "kvlr_decode_attn_upproject_noalloc", "kvlr_noalloc_scratch_bytes",
    "kvlr_fit_joint_workspace_bytes", "kvlr_fit_joint_moments", "kvlr_fit_joint_solve",
    "kvlr_fold_joint_decoder", "kvlr_fit_joint", "kvlr_residual_prep_bytes", "kvlr_prepare_residual",
    "kvlr_check_page_tables", "kvlr_score_pages", "kvlr_select_pages",
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
    _fields_ = [("v_lat", ctypes.c_void_p), ("k_lat", ctypes.c_void_p), ("k_exact", ctypes.c_void_p),
                ("k_lat_ranks", ctypes.POINTER(ctypes.c_int32))]


class kvlr_factors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("A_v", "B_v", "A_k", "B_k", "W_pred", "residual_prep")]


class kvlr_factor_buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("A_v", "B_v", "A_k", "B_k", "W_pred")]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIG = {
    "kvlr_append_encode": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors),
                            ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _P, _I, _I, _I, _P], _I),
    "kvlr_append_encode_project": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors),
                                    ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _P, _I, _I, _I, _P,
                                    _P, _P], _I),
    "kvlr_project_queries": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _P, _I, _P], _I),
    "kvlr_qproj_width": ([ctypes.POINTER(kvlr_shape)], _I),
    "kvlr_route_pages": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_cache), _P, _P, _P, _I, _I,
                          _I, _P, _I, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _P], _I),
    "kvlr_score_pages": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_cache), _P, _P, _P, _I, _P,
                          _I, _P], _I),
    "kvlr_select_pages": ([ctypes.POINTER(kvlr_shape), _P, _P, _I, _P, _I, _I, _P, _I, _P, _P, _P, _I,
                           _P], _I),
    "kvlr_decode_attn": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _I,
                          _P, _P, _P, _I, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _I, _P], _I),
    "kvlr_decode_attn_upproject": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors),
                                    ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _I, _P, _P, _P, _I,
                                    ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _I, _P], _I),
    "kvlr_decode_attn_upproject_noalloc": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors),
                                            ctypes.POINTER(kvlr_cache), _P, _P, _P, _P, _I, _P, _P, _P,
                                            _I, ctypes.c_float, _P, _P, _P, _I, _P], _I),
    "kvlr_noalloc_scratch_bytes": ([], ctypes.c_size_t),
    "kvlr_residual_prep_bytes": ([ctypes.POINTER(kvlr_shape)], ctypes.c_size_t),
    "kvlr_check_page_tables": ([ctypes.POINTER(kvlr_shape), _P, _P, _I, _I, _P, _P], _I),
    "kvlr_prepare_residual": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P,
                               ctypes.c_size_t, _P], _I),
    "kvlr_fit_joint_workspace_bytes": ([ctypes.POINTER(kvlr_shape), _I], ctypes.c_size_t),
    "kvlr_fit_joint_moments": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _I, _P,
                                _P, _I, _P, ctypes.c_size_t, _P], _I),
    "kvlr_fit_joint_solve": ([ctypes.POINTER(kvlr_shape), _P, _P, _P], _I),
    "kvlr_fold_joint_decoder": ([ctypes.POINTER(kvlr_shape), _P, _I, _P, _P, _P], _I),
    "kvlr_fit_joint": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _I, _P, _I, _P,
                        _P, _P, ctypes.c_size_t, _P], _I),
    "kvlr_upproject": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _P, _I, _P], _I),
    "kvlr_workspace_bytes": ([ctypes.POINTER(kvlr_shape), _I, _I], ctypes.c_size_t),
    "kvlr_fold_output_weights": ([ctypes.POINTER(kvlr_shape), ctypes.POINTER(kvlr_factors), _P, _I,
                                  _P, _P], _I),
    "kvlr_output_projection": ([ctypes.POINTER(kvlr_shape), _P, _P, _I, _P, _I, _P], _I),
    "kvlr_workspace_init": ([_P, ctypes.c_size_t, _P], _I),
    "kvlr_status_string": ([_I], ctypes.c_char_p),
    "kvlr_version": ([], _I),
    "kvlr_fit_workspace_bytes": ([ctypes.POINTER(kvlr_shape), _I], ctypes.c_size_t),
    "kvlr_fit_moments": ([ctypes.POINTER(kvlr_shape), _P, _P, _I, _P, _I, _P, ctypes.c_size_t, _P], _I),
    "kvlr_fit_solve": ([ctypes.POINTER(kvlr_shape), _P, _P, _P, _P, _P, _P], _I),
    "kvlr_fit_factors": ([ctypes.POINTER(kvlr_shape), _P, _P, _I, ctypes.POINTER(kvlr_factor_buffers),
                          _P, _P, _P, ctypes.c_size_t, _P], _I),
    "kvlr_choose_residual_ranks": ([ctypes.POINTER(kvlr_shape), _P, ctypes.c_double, _P], _I),
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
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return int(x)


def _host_f64(x, name):
    """A host float64 C-contiguous array (numpy or CPU tensor), or None."""
    if x is None:
        return None
    ok = (isinstance(x, np.ndarray) and x.dtype == np.float64 and x.flags["C_CONTIGUOUS"]) or (
        isinstance(x, torch.Tensor) and x.device.type == "cpu" and x.dtype == torch.float64
        and x.is_contiguous())
    if not ok:
        raise TypeError(f"{name} must be a C-contiguous host float64 array")
    return x


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


def make_cache(v_lat=None, k_lat=None, k_exact=None, k_lat_ranks=None) -> kvlr_cache:
    """k_lat_ranks: per-KV-head residual ranks (a sequence of ints) or None."""
    ranks = None
    if k_lat_ranks is not None:
        ranks = (ctypes.c_int32 * len(k_lat_ranks))(*[int(r) for r in k_lat_ranks])
    c = kvlr_cache(_ptr(v_lat), _ptr(k_lat), _ptr(k_exact),
                   ctypes.cast(ranks, ctypes.POINTER(ctypes.c_int32)) if ranks is not None else None)
    c._ranks = ranks  # keep the host array alive as long as the struct
    return c


def make_factors(A_v=None, B_v=None, A_k=None, B_k=None, W_pred=None,
                 residual_prep=None) -> kvlr_factors:
    return kvlr_factors(_ptr(A_v), _ptr(B_v), _ptr(A_k), _ptr(B_k), _ptr(W_pred), _ptr(residual_prep))


def kvlr_residual_prep_bytes(shape: kvlr_shape) -> int:
    return lib().kvlr_residual_prep_bytes(ctypes.byref(shape))


KVLR_TABLE_ERR_PAGE = 1
KVLR_TABLE_ERR_LENGTH = 2


def kvlr_check_page_tables(shape, seq_lens, page_table, max_pages_per_seq, batch, errors, stream=None):
    _check("kvlr_check_page_tables", lib().kvlr_check_page_tables(
        ctypes.byref(shape), _ptr(seq_lens), _ptr(page_table), max_pages_per_seq, batch, _ptr(errors),
        _stream(stream)))


def kvlr_prepare_residual(shape, factors, prep, prep_bytes, stream=None):
    _check("kvlr_prepare_residual", lib().kvlr_prepare_residual(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(prep), prep_bytes, _stream(stream)))


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


def kvlr_append_encode_project(shape, factors, cache, k_new, v_new, cu_new, seq_lens_before,
                               page_table, max_pages_per_seq, batch, total_new, q, q_proj,
                               stream=None):
    _check("kvlr_append_encode_project", lib().kvlr_append_encode_project(
        ctypes.byref(shape), ctypes.byref(factors), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
        _ptr(cu_new), _ptr(seq_lens_before), _ptr(page_table), max_pages_per_seq, batch, total_new,
        _ptr(q), _ptr(q_proj), _stream(stream)))


def kvlr_project_queries(shape, factors, q, q_proj, batch, stream=None):
    _check("kvlr_project_queries", lib().kvlr_project_queries(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(q), _ptr(q_proj), batch, _stream(stream)))


def kvlr_route_pages(shape, cache, q_proj, seq_lens, page_table, max_pages_per_seq, topk_num,
                     topk_den, k_pages, k_max, sel_pages, sel_counts, sel_phys, page_scores,
                     workspace, ws_bytes, batch, stream=None):
    _check("kvlr_route_pages", lib().kvlr_route_pages(
        ctypes.byref(shape), ctypes.byref(cache), _ptr(q_proj), _ptr(seq_lens), _ptr(page_table),
        max_pages_per_seq, topk_num, topk_den, _ptr(k_pages), k_max, _ptr(sel_pages),
        _ptr(sel_counts), _ptr(sel_phys), _ptr(page_scores), _ptr(workspace), ws_bytes, batch,
        _stream(stream)))


def kvlr_score_pages(shape, cache, q_proj, seq_lens, page_table, max_pages_per_seq, page_scores,
                     batch, stream=None):
    _check("kvlr_score_pages", lib().kvlr_score_pages(
        ctypes.byref(shape), ctypes.byref(cache), _ptr(q_proj), _ptr(seq_lens), _ptr(page_table),
        max_pages_per_seq, _ptr(page_scores), batch, _stream(stream)))


def kvlr_select_pages(shape, seq_lens, page_table, max_pages_per_seq, page_scores, topk_num,
                      topk_den, k_pages, k_max, sel_pages, sel_counts, sel_phys, batch, stream=None):
    _check("kvlr_select_pages", lib().kvlr_select_pages(
        ctypes.byref(shape), _ptr(seq_lens), _ptr(page_table), max_pages_per_seq, _ptr(page_scores),
        topk_num, topk_den, _ptr(k_pages), k_max, _ptr(sel_pages), _ptr(sel_counts), _ptr(sel_phys),
        batch, _stream(stream)))


def kvlr_decode_attn(shape, cache, q, q_proj, seq_lens, page_table, max_pages_per_seq, sel_pages,
                     sel_phys, sel_counts, k_max, softmax_scale, z_out, lse_out, workspace,
                     ws_bytes, batch, stream=None):
    _check("kvlr_decode_attn", lib().kvlr_decode_attn(
        ctypes.byref(shape), ctypes.byref(cache), _ptr(q), _ptr(q_proj), _ptr(seq_lens),
        _ptr(page_table), max_pages_per_seq, _ptr(sel_pages), _ptr(sel_phys), _ptr(sel_counts),
        k_max, float(softmax_scale), _ptr(z_out), _ptr(lse_out), _ptr(workspace), ws_bytes, batch,
        _stream(stream)))


def kvlr_decode_attn_upproject(shape, factors, cache, q, q_proj, seq_lens, page_table,
                               max_pages_per_seq, sel_pages, sel_phys, sel_counts, k_max,
                               softmax_scale, z_out, lse_out, o_out, workspace, ws_bytes, batch,
                               stream=None):
    _check("kvlr_decode_attn_upproject", lib().kvlr_decode_attn_upproject(
        ctypes.byref(shape), ctypes.byref(factors), ctypes.byref(cache), _ptr(q), _ptr(q_proj),
        _ptr(seq_lens), _ptr(page_table), max_pages_per_seq, _ptr(sel_pages), _ptr(sel_phys),
        _ptr(sel_counts), k_max, float(softmax_scale), _ptr(z_out), _ptr(lse_out), _ptr(o_out),
        _ptr(workspace), ws_bytes, batch, _stream(stream)))


def kvlr_decode_attn_upproject_noalloc(shape, factors, cache, q, q_proj, seq_lens, page_table,
                                       max_pages_per_seq, sel_pages, sel_phys, sel_counts, k_max,
                                       softmax_scale, z_out, lse_out, o_out, batch, stream=None):
    _check("kvlr_decode_attn_upproject_noalloc", lib().kvlr_decode_attn_upproject_noalloc(
        ctypes.byref(shape), ctypes.byref(factors), ctypes.byref(cache), _ptr(q), _ptr(q_proj),
        _ptr(seq_lens), _ptr(page_table), max_pages_per_seq, _ptr(sel_pages), _ptr(sel_phys),
        _ptr(sel_counts), k_max, float(softmax_scale), _ptr(z_out), _ptr(lse_out), _ptr(o_out),
        batch, _stream(stream)))


def kvlr_noalloc_scratch_bytes() -> int:
    return int(lib().kvlr_noalloc_scratch_bytes())


def kvlr_upproject(shape, factors, z, o_out, batch, stream=None):
    _check("kvlr_upproject", lib().kvlr_upproject(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(z), _ptr(o_out), batch, _stream(stream)))


def kvlr_fold_output_weights(shape, factors, W_o, hidden, F_out, stream=None):
    _check("kvlr_fold_output_weights", lib().kvlr_fold_output_weights(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(W_o), hidden, _ptr(F_out), _stream(stream)))


def kvlr_output_projection(shape, F, z, hidden, out, batch, stream=None):
    _check("kvlr_output_projection", lib().kvlr_output_projection(
        ctypes.byref(shape), _ptr(F), _ptr(z), hidden, _ptr(out), batch, _stream(stream)))


def make_factor_buffers(A_v=None, B_v=None, A_k=None, B_k=None, W_pred=None) -> kvlr_factor_buffers:
    return kvlr_factor_buffers(_ptr(A_v), _ptr(B_v), _ptr(A_k), _ptr(B_k), _ptr(W_pred))


def kvlr_fit_workspace_bytes(shape, n) -> int:
    return lib().kvlr_fit_workspace_bytes(ctypes.byref(shape), n)


def kvlr_fit_moments(shape, k, v, n, moments, accumulate, workspace, ws_bytes, stream=None):
    _check("kvlr_fit_moments", lib().kvlr_fit_moments(
        ctypes.byref(shape), _ptr(k), _ptr(v), n, _ptr(moments), int(accumulate), _ptr(workspace),
        ws_bytes, _stream(stream)))


def kvlr_fit_solve(shape, moments, A_v, A_k, W_pred=None, lam_v=None, lam_k=None):
    """Host call: every array is a host float64 array (numpy or CPU tensor)."""
    args = [_host_f64(x, nm) for x, nm in ((moments, "moments"), (A_v, "A_v"), (A_k, "A_k"),
                                          (W_pred, "W_pred"), (lam_v, "lam_v"), (lam_k, "lam_k"))]
    _check("kvlr_fit_solve", lib().kvlr_fit_solve(ctypes.byref(shape), *[_ptr(x) for x in args]))


def kvlr_fit_factors(shape, k, v, n, out, lam_v, lam_k, workspace, ws_bytes, stream=None):
    lam_v = _host_f64(lam_v, "lam_v")
    lam_k = _host_f64(lam_k, "lam_k")
    _check("kvlr_fit_factors", lib().kvlr_fit_factors(
        ctypes.byref(shape), _ptr(k), _ptr(v), n, ctypes.byref(out), _ptr(lam_v), _ptr(lam_k),
        _ptr(workspace), ws_bytes, _stream(stream)))


def kvlr_choose_residual_ranks(shape, lam_k, energy_frac) -> list:
    """Host call: per-head residual ranks from the fit's residual eigenvalues
    (lam_k host float64 [H_kv][rank_k])."""
    lam_k = _host_f64(lam_k, "lam_k")
    out = (ctypes.c_int32 * shape.num_kv_heads)()
    _check("kvlr_choose_residual_ranks", lib().kvlr_choose_residual_ranks(
        ctypes.byref(shape), _ptr(lam_k), float(energy_frac), ctypes.cast(out, ctypes.c_void_p)))
    return list(out)


def kvlr_fit_joint_workspace_bytes(shape, n) -> int:
    return int(lib().kvlr_fit_joint_workspace_bytes(ctypes.byref(shape), n))


def kvlr_fit_joint_moments(shape, factors, x, n, zz, zx, accumulate, workspace, ws_bytes,
                           stream=None):
    _check("kvlr_fit_joint_moments", lib().kvlr_fit_joint_moments(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(x), n, _ptr(zz), _ptr(zx), accumulate,
        _ptr(workspace), ws_bytes, _stream(stream)))


def kvlr_fit_joint_solve(shape, zz, zx):
    """Host solve; zz, zx host float64 arrays. Returns D (float64 numpy)."""
    zz = _host_f64(zz, "zz")
    zx = _host_f64(zx, "zx")
    zz = zz.numpy() if isinstance(zz, torch.Tensor) else zz
    zx = zx.numpy() if isinstance(zx, torch.Tensor) else zx
    D = np.empty(zx.shape, dtype=np.float64)
    _check("kvlr_fit_joint_solve", lib().kvlr_fit_joint_solve(
        ctypes.byref(shape), zz.ctypes.data_as(ctypes.c_void_p), zx.ctypes.data_as(ctypes.c_void_p),
        D.ctypes.data_as(ctypes.c_void_p)))
    return D


def kvlr_fold_joint_decoder(shape, W_o, hidden, D, F_out, stream=None):
    _check("kvlr_fold_joint_decoder", lib().kvlr_fold_joint_decoder(
        ctypes.byref(shape), _ptr(W_o), hidden, _ptr(D), _ptr(F_out), _stream(stream)))


def kvlr_fit_joint(shape, factors, x, n, W_o, hidden, F_out, workspace, ws_bytes, want_D=False,
                   stream=None):
    """The synchronous joint fit; returns the float64 decoder when asked."""
    D = None
    if want_D:
        nl = shape.num_q_heads * shape.rank_v
        nx = shape.num_q_heads * shape.head_dim
        D = np.empty((nl, nx), dtype=np.float64)
    _check("kvlr_fit_joint", lib().kvlr_fit_joint(
        ctypes.byref(shape), ctypes.byref(factors), _ptr(x), n, _ptr(W_o), hidden, _ptr(F_out),
        None if D is None else D.ctypes.data_as(ctypes.c_void_p), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return D
