"""Thin ctypes binding of libqsa (include/qsa.h), with the same entry-point names.

Argument marshalling only: every step of the QSA path runs in the HIP
kernels of libqsa.so.  Tensors are torch tensors (device memory and streams
are torch's); pointers, strides and the current HIP stream are passed
through.  A missing library raises at first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqsa.so")

QSA_OK = 0
STATUS = {0: "QSA_OK", 1: "QSA_ERR_INVALID_ARG", 2: "QSA_ERR_UNSUPPORTED",
          3: "QSA_ERR_WORKSPACE_TOO_SMALL", 4: "QSA_ERR_LAUNCH_FAILED", 5: "QSA_ERR_INTERNAL"}

BLOCK, IDX_HEADS, IDX_DIM, Q_HEADS, KV_HEADS, HEAD_DIM, ROPE_DIM, MAX_BUDGET = 4, 4, 128, 24, 2, 256, 64, 512
SOFTMAX_SCALE = 1.0 / 16.0

_c_void_p, _i32, _i64, _size = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/qsa.h
SIGNATURES = {
    "qsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qsa_abi_version": (ctypes.c_int, []),
    "qsa_pool_block_keys": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _i64, _c_void_p, _c_void_p,
                                           _i32, _i32, _c_void_p, _i64, _i32, _c_void_p]),
    "qsa_rope_apply": (ctypes.c_int, [_c_void_p, _i64, _i64, _i32, _c_void_p, _i32, _i32, _c_void_p,
                                      _c_void_p]),
    "qsa_yarn_rope": (ctypes.c_int, [ctypes.c_double] * 5 + [_c_void_p, _c_void_p]),
    "qsa_pool_block_keys_normed": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _i64, _c_void_p,
                                                  _c_void_p, _i32, _i32, _c_void_p, ctypes.c_double,
                                                  _c_void_p, _c_void_p, _i64, _i32, _c_void_p]),
    "qsa_index_query_transform": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                                 _i32, _i32, _c_void_p, ctypes.c_double, _c_void_p,
                                                 _c_void_p]),
    "qsa_index_select_workspace": (_size, [_i32, _i32, _i32]),
    "qsa_index_select": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                        _i32, _c_void_p, _i64, _i32, _c_void_p, _c_void_p, _c_void_p,
                                        _size, _c_void_p, _i64, _i32, _c_void_p]),
    "qsa_attend_prefill": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p,
                                          _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i32, _c_void_p,
                                          _c_void_p, _c_void_p, ctypes.c_float, _c_void_p, _i64,
                                          _i32, _c_void_p]),
    "qsa_attend_decode_workspace": (_size, [_i32]),
    "qsa_attend_decode": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _i64, _i64,
                                         _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p,
                                         _size, _c_void_p, ctypes.c_float, _c_void_p, _i64, _i32,
                                         _c_void_p]),
    "qsa_attend_decode_noalloc": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p,
                                                 _i64, _i64, _c_void_p, _c_void_p, _i32, _c_void_p,
                                                 _c_void_p, _c_void_p, ctypes.c_float, _c_void_p,
                                                 _i64, _i32, _c_void_p]),
    "qsa_attend_decode_multi_workspace": (_size, [_i32]),
    "qsa_attend_decode_multi": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _c_void_p,
                                               _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i32,
                                               _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p,
                                               ctypes.c_float, _c_void_p, _i64, _i32, _c_void_p]),
}

_lib = None


class QSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libqsa.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != QSA_OK:
        raise QSAError(fn, status)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("QSA tensors must be on the GPU")


def _host_f64(a):
    """(pointer, keep-alive) for an optional host float64 array of 32 frequencies."""
    if a is None:
        return None, None
    if len(a) != 32:
        raise ValueError("inv_freq holds 32 float64 frequencies")
    buf = (ctypes.c_double * 32)(*[float(v) for v in a])
    return ctypes.cast(buf, ctypes.c_void_p), buf


def _pages(pages):
    """(table pointer, table_stride, page_tokens) for pages = None (contiguous
    caches) or (block_table int32 [n_seq][stride] on the GPU, page_tokens)."""
    if pages is None:
        return None, 0, 0
    table, page_tokens = pages
    _dev(table)
    if table.dtype != torch.int32 or table.dim() != 2 or table.stride(1) != 1:
        raise ValueError("block_table must be a row-major int32 [n_seq][stride] tensor")
    return _p(table), table.stride(0), int(page_tokens)


def _kv_strides(k_cache, pages):
    """(kv_seq_stride, kv_head_stride): k_cache [n_seq][2][cap][256], or with
    pages the pool [2][n_pages * page_tokens][256]."""
    if pages is None:
        return k_cache.stride(0), k_cache.stride(1)
    return 0, k_cache.stride(0)


def status_string(status: int) -> str:
    return lib().qsa_status_string(status).decode()


def abi_version() -> int:
    return lib().qsa_abi_version()


def pool_block_keys(idx_k, block_keys, blk_begin, blk_end, max_span, pages=None, stream=None):
    """idx_k bf16 [n_seq][cap][128] -> block_keys bf16 [n_seq][cap/4][128] for blk_begin..blk_end
    (or the paged pools, pages = (block_table, page_tokens))."""
    _dev(idx_k, block_keys, blk_begin, blk_end)
    st = lib().qsa_pool_block_keys(_p(idx_k), idx_k.stride(0), _p(block_keys), block_keys.stride(0),
                                   _p(blk_begin), _p(blk_end), blk_begin.numel(), int(max_span),
                                   *_pages(pages), _stream(stream))
    _check("qsa_pool_block_keys", st)


def rope_apply(x, row_stride, head_stride, n_heads, n_rows, pos=None, pos0=0, inv_freq=None,
               stream=None):
    """Rotate dims 0..63 of n_rows x n_heads bf16 vectors of x in place."""
    _dev(x, pos)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_rope_apply(_p(x), int(row_stride), int(head_stride), int(n_heads), _p(pos),
                              int(pos0), int(n_rows), fp, _stream(stream))
    _check("qsa_rope_apply", st)


def yarn_rope(base=1.0e7, factor=4.0, orig_ctx=262144, alpha=1.0, beta=32.0):
    """(32 YaRN rotary frequencies, softmax scale) from the library's host helper."""
    buf = (ctypes.c_double * 32)()
    sc = ctypes.c_float()
    st = lib().qsa_yarn_rope(float(base), float(factor), float(orig_ctx), float(alpha), float(beta),
                             ctypes.cast(buf, ctypes.c_void_p), ctypes.cast(ctypes.pointer(sc),
                                                                             ctypes.c_void_p))
    _check("qsa_yarn_rope", st)
    return list(buf), sc.value


def pool_block_keys_normed(idx_k, block_keys, blk_begin, blk_end, max_span, gamma=None, eps=1e-6,
                           inv_freq=None, pages=None, stream=None):
    """Pool, RMS-normalise and rotate blocks blk_begin..blk_end (the pages' indexer keys)."""
    _dev(idx_k, block_keys, blk_begin, blk_end, gamma)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_pool_block_keys_normed(_p(idx_k), idx_k.stride(0), _p(block_keys),
                                          block_keys.stride(0), _p(blk_begin), _p(blk_end),
                                          blk_begin.numel(), int(max_span), _p(gamma), float(eps),
                                          fp, *_pages(pages), _stream(stream))
    _check("qsa_pool_block_keys_normed", st)


def index_query_transform(q_raw, q_out, cu_q, seq_len, max_q_len, gamma=None, eps=1e-6,
                          inv_freq=None, stream=None):
    """RMS-normalise and rotate the indexer query heads (bf16 [n_q][4][128]) at their positions."""
    _dev(q_raw, q_out, cu_q, seq_len, gamma)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_index_query_transform(_p(q_raw), _p(q_out), _p(cu_q), _p(seq_len),
                                         seq_len.numel(), q_raw.shape[0], int(max_q_len),
                                         _p(gamma), float(eps), fp, _stream(stream))
    _check("qsa_index_query_transform", st)


def index_select_workspace(n_q, max_q_len, max_blocks) -> int:
    return int(lib().qsa_index_select_workspace(int(n_q), int(max_q_len), int(max_blocks)))


def index_select(idx_q, w, cu_q, seq_len, max_q_len, max_blocks, block_keys, budget, sel,
                 sel_count, workspace, pages=None, stream=None):
    _dev(idx_q, w, cu_q, seq_len, block_keys, sel, sel_count, workspace)
    st = lib().qsa_index_select(_p(idx_q), _p(w), _p(cu_q), _p(seq_len), seq_len.numel(),
                                idx_q.shape[0], int(max_q_len), int(max_blocks), _p(block_keys),
                                block_keys.stride(0), int(budget), _p(sel), _p(sel_count),
                                _p(workspace), workspace.numel() * workspace.element_size(),
                                *_pages(pages), _stream(stream))
    _check("qsa_index_select", st)


def attend_prefill(q, cu_q, seq_len, max_q_len, k_cache, v_cache, sel, sel_count, budget, out,
                   lse=None, inv_freq=None, softmax_scale=SOFTMAX_SCALE, pages=None, stream=None):
    _dev(q, cu_q, seq_len, k_cache, v_cache, sel, sel_count, out, lse)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_attend_prefill(_p(q), _p(cu_q), _p(seq_len), seq_len.numel(), q.shape[0],
                                  int(max_q_len), _p(k_cache), _p(v_cache),
                                  *_kv_strides(k_cache, pages), _p(sel), _p(sel_count), int(budget),
                                  _p(out), _p(lse), fp, float(softmax_scale), *_pages(pages),
                                  _stream(stream))
    _check("qsa_attend_prefill", st)


def attend_decode_workspace(n_seq) -> int:
    return int(lib().qsa_attend_decode_workspace(int(n_seq)))


def attend_decode(q, seq_len, k_cache, v_cache, sel, sel_count, budget, out, lse, workspace,
                  inv_freq=None, softmax_scale=SOFTMAX_SCALE, pages=None, stream=None):
    _dev(q, seq_len, k_cache, v_cache, sel, sel_count, out, lse, workspace)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_attend_decode(_p(q), _p(seq_len), seq_len.numel(), _p(k_cache), _p(v_cache),
                                 *_kv_strides(k_cache, pages), _p(sel), _p(sel_count),
                                 int(budget), _p(out), _p(lse), _p(workspace),
                                 workspace.numel() * workspace.element_size(), fp,
                                 float(softmax_scale), *_pages(pages), _stream(stream))
    _check("qsa_attend_decode", st)


NOALLOC_MAX_SEQ = 128


def attend_decode_noalloc(q, seq_len, k_cache, v_cache, sel, sel_count, budget, out, lse,
                          inv_freq=None, softmax_scale=SOFTMAX_SCALE, pages=None, stream=None):
    """qsa_attend_decode without a workspace (the library's own per-GPU buffer,
    at most NOALLOC_MAX_SEQ sequences; overlapping calls on one GPU race)."""
    _dev(q, seq_len, k_cache, v_cache, sel, sel_count, out, lse)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_attend_decode_noalloc(_p(q), _p(seq_len), seq_len.numel(), _p(k_cache),
                                         _p(v_cache), *_kv_strides(k_cache, pages), _p(sel),
                                         _p(sel_count), int(budget), _p(out), _p(lse), fp,
                                         float(softmax_scale), *_pages(pages), _stream(stream))
    _check("qsa_attend_decode_noalloc", st)


def attend_decode_multi_workspace(n_q) -> int:
    return int(lib().qsa_attend_decode_multi_workspace(int(n_q)))


def attend_decode_multi(q, cu_q, seq_len, k_cache, v_cache, sel, sel_count, budget, out, lse,
                        workspace, inv_freq=None, softmax_scale=SOFTMAX_SCALE, pages=None,
                        stream=None):
    _dev(q, cu_q, seq_len, k_cache, v_cache, sel, sel_count, out, lse, workspace)
    fp, _keep = _host_f64(inv_freq)
    st = lib().qsa_attend_decode_multi(_p(q), _p(cu_q), _p(seq_len), seq_len.numel(), q.shape[0],
                                       _p(k_cache), _p(v_cache), *_kv_strides(k_cache, pages),
                                       _p(sel), _p(sel_count), int(budget),
                                       _p(out), _p(lse), _p(workspace),
                                       workspace.numel() * workspace.element_size(), fp,
                                       float(softmax_scale), *_pages(pages), _stream(stream))
    _check("qsa_attend_decode_multi", st)
