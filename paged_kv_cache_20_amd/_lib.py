"""ctypes binding of libpagedattn.so -- argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors where the C side takes device pointers (numpy arrays for host
pointers), checks nothing the library checks itself, and raises
``AttnError`` carrying the library's message when a call returns an error.
All arithmetic runs in the library's HIP kernels; there is no other path.
If the shared library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
VERIFY_ROWS = 8
PAGE_SIZE = 16

ATTN_OK = 0
ATTN_E_ARG = -1
ATTN_E_SHAPE = -2
ATTN_E_UNSUPPORTED = -3
ATTN_PREFILL_FP8_QK = 1
ATTN_PREFILL_FP8_PV = 2
ATTN_E_WORKSPACE = -4
ATTN_E_RANGE = -5
ATTN_E_DEVICE = -6

EXPORTS = [
    "attn_paged_decode", "attn_paged_decode_noalloc", "attn_paged_verify",
    "attn_paged_verify_width",
    "attn_paged_verify_tree", "attn_paged_prefill", "attn_paged_prefill_fp8",
    "attn_paged_mixed", "attn_paged_decode_window", "attn_paged_prefill_window",
    "attn_kv_append", "attn_block_table_build", "attn_paged_workspace_bytes", "attn_caps",
    "attn_check_lengths_host", "attn_check_block_table_host", "attn_check_device",
    "attn_last_error",
    "attn_set_kernel_timer", "attn_set_max_workgroups",
]


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError("libpagedattn.so is not built (%s); run "
                      "`python -m paged_kv_cache_20_amd.build`" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SPLIT_ARGS = [_P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32,
               _P, _P, _SZ, _P]
_lib.attn_paged_decode.argtypes = _SPLIT_ARGS
_lib.attn_paged_decode.restype = ctypes.c_int
_lib.attn_paged_decode_noalloc.argtypes = _SPLIT_ARGS[:-3] + [_P]
_lib.attn_paged_decode_noalloc.restype = ctypes.c_int
_lib.attn_paged_verify.argtypes = _SPLIT_ARGS
_lib.attn_paged_verify.restype = ctypes.c_int
_lib.attn_paged_verify_width.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32,
                                         _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]
_lib.attn_paged_verify_width.restype = ctypes.c_int
_lib.attn_paged_verify_tree.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _P,
                                        _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]
_lib.attn_paged_verify_tree.restype = ctypes.c_int
_lib.attn_paged_prefill.argtypes = [_P, _I32, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32, _I32,
                                    _I32, _I32, _I32, _P, _P, _SZ, _P]
_lib.attn_paged_prefill.restype = ctypes.c_int
_lib.attn_paged_prefill_fp8.argtypes = [_P, _I32, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                        _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]
_lib.attn_paged_prefill_fp8.restype = ctypes.c_int
_lib.attn_paged_mixed.argtypes = [_P, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _P, _I64, _P, _I32,
                                  _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]
_lib.attn_paged_mixed.restype = ctypes.c_int
_lib.attn_paged_decode_window.argtypes = [_P, _I32, _P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                          _I32, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ,
                                          _P]
_lib.attn_paged_decode_window.restype = ctypes.c_int
_lib.attn_paged_prefill_window.argtypes = [_P, _I32, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]
_lib.attn_paged_prefill_window.restype = ctypes.c_int
_lib.attn_kv_append.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32,
                                _P]
_lib.attn_kv_append.restype = ctypes.c_int
_lib.attn_block_table_build.argtypes = [_I32, _P, _I32, _I64, ctypes.c_uint64, _I32, _P, _P]
_lib.attn_block_table_build.restype = ctypes.c_int
_lib.attn_paged_workspace_bytes.argtypes = [ctypes.c_int, _I32, _I32, _I32, _I32]
_lib.attn_paged_workspace_bytes.restype = _SZ
_lib.attn_caps.argtypes = [_I32, _I32, _I32]
_lib.attn_caps.restype = ctypes.c_int
_lib.attn_check_lengths_host.argtypes = [_P, _I32, _I32, _I32, _I32]
_lib.attn_check_lengths_host.restype = ctypes.c_int
_lib.attn_check_block_table_host.argtypes = [_P, _P, _I32, _I32, _I32, _I64]
_lib.attn_check_block_table_host.restype = ctypes.c_int
_lib.attn_check_device.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I64, _P, _P]
_lib.attn_check_device.restype = ctypes.c_int
_lib.attn_last_error.argtypes = []
_lib.attn_last_error.restype = ctypes.c_char_p
_lib.attn_set_kernel_timer.argtypes = [_P, _P]
_lib.attn_set_kernel_timer.restype = None
_lib.attn_set_max_workgroups.argtypes = [_I32]
_lib.attn_set_max_workgroups.restype = None


def lib() -> ctypes.CDLL:
    return _lib


def attn_last_error() -> str:
    return (_lib.attn_last_error() or b"").decode()


def _check(rc: int) -> int:
    if rc != ATTN_OK:
        raise AttnError(rc, attn_last_error())
    return rc


def _dp(t) -> Optional[int]:
    """Device pointer of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def attn_paged_workspace_bytes(op: int, n_seq: int, max_pages_per_seq: int, n_head: int,
                               head_dim: int) -> int:
    return int(_lib.attn_paged_workspace_bytes(op, n_seq, max_pages_per_seq, n_head, head_dim))


def attn_caps(head_dim: int, page_size: int, kv_dtype: int) -> int:
    return int(_lib.attn_caps(head_dim, page_size, kv_dtype))


def _split(fn, q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table, max_pages_per_seq,
           ctx_lens, n_seq, n_head, n_head_kv, head_dim, page_size, kv_dtype, out, workspace,
           workspace_bytes, stream):
    return _check(fn(_dp(q), _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages,
                     _dp(block_table), max_pages_per_seq, _dp(ctx_lens), n_seq, n_head, n_head_kv,
                     head_dim, page_size, kv_dtype, _dp(out), _dp(workspace), workspace_bytes,
                     _stream(stream)))


def attn_paged_decode(q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                      max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim, page_size,
                      kv_dtype, out, workspace, workspace_bytes, stream=None):
    return _split(_lib.attn_paged_decode, q, k_pool, v_pool, k_scale, v_scale, n_pages,
                  block_table, max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim,
                  page_size, kv_dtype, out, workspace, workspace_bytes, stream)


def attn_paged_decode_noalloc(q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                              max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim,
                              page_size, kv_dtype, out, stream=None):
    return _check(_lib.attn_paged_decode_noalloc(
        _dp(q), _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages,
        _dp(block_table), max_pages_per_seq, _dp(ctx_lens), n_seq, n_head, n_head_kv, head_dim,
        page_size, kv_dtype, _dp(out), _stream(stream)))


def attn_paged_verify(q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                      max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim, page_size,
                      kv_dtype, out, workspace, workspace_bytes, stream=None):
    return _split(_lib.attn_paged_verify, q, k_pool, v_pool, k_scale, v_scale, n_pages,
                  block_table, max_pages_per_seq, ctx_lens, n_seq, n_head, n_head_kv, head_dim,
                  page_size, kv_dtype, out, workspace, workspace_bytes, stream)


def attn_paged_verify_width(q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                            max_pages_per_seq, ctx_lens, n_seq, width, n_head, n_head_kv,
                            head_dim, page_size, kv_dtype, out, workspace=None,
                            workspace_bytes=0, stream=None):
    return _check(_lib.attn_paged_verify_width(
        _dp(q), _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages, _dp(block_table),
        max_pages_per_seq, _dp(ctx_lens), n_seq, width, n_head, n_head_kv, head_dim, page_size,
        kv_dtype, _dp(out), _dp(workspace), workspace_bytes, _stream(stream)))


def attn_paged_decode_window(q, rows, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                             max_pages_per_seq, ctx_lens, n_seq, window, kv_floor, n_head,
                             n_head_kv, head_dim, page_size, kv_dtype, out, workspace=None,
                             workspace_bytes=0, stream=None):
    return _check(_lib.attn_paged_decode_window(
        _dp(q), rows, _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages,
        _dp(block_table), max_pages_per_seq, _dp(ctx_lens), n_seq, window, _dp(kv_floor), n_head,
        n_head_kv, head_dim, page_size, kv_dtype, _dp(out), _dp(workspace), workspace_bytes,
        _stream(stream)))


def attn_paged_prefill_window(q, n_rows, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                              max_pages_per_seq, ctx_len, window, kv_floor, n_head, n_head_kv,
                              head_dim, page_size, kv_dtype, out, workspace=None,
                              workspace_bytes=0, stream=None):
    return _check(_lib.attn_paged_prefill_window(
        _dp(q), n_rows, _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages,
        _dp(block_table), max_pages_per_seq, ctx_len, window, kv_floor, n_head, n_head_kv,
        head_dim, page_size, kv_dtype, _dp(out), _dp(workspace), workspace_bytes,
        _stream(stream)))


def attn_check_device(block_table, ctx_lens, kv_floor, window, n_seq, rows, max_pages_per_seq,
                      page_size, n_pages, err_word, stream=None):
    return _check(_lib.attn_check_device(
        _dp(block_table), _dp(ctx_lens), _dp(kv_floor), window, n_seq, rows, max_pages_per_seq,
        page_size, n_pages, _dp(err_word), _stream(stream)))


def attn_paged_verify_tree(q, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                           max_pages_per_seq, ctx_lens, n_seq, width, tree_mask, scratch_pages,
                           n_head, n_head_kv, head_dim, page_size, kv_dtype, out, workspace=None,
                           workspace_bytes=0, stream=None):
    return _check(_lib.attn_paged_verify_tree(
        _dp(q), _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages, _dp(block_table),
        max_pages_per_seq, _dp(ctx_lens), n_seq, width, _dp(tree_mask), _dp(scratch_pages),
        n_head, n_head_kv, head_dim, page_size, kv_dtype, _dp(out), _dp(workspace),
        workspace_bytes, _stream(stream)))


def attn_paged_mixed(q, n_tok, cu_seqlens, n_seq, n_seq_decode, max_q_len, k_pool, v_pool,
                     k_scale, v_scale, n_pages, block_table, max_pages_per_seq, ctx_lens, n_head,
                     n_head_kv, head_dim, page_size, kv_dtype, out, workspace=None,
                     workspace_bytes=0, stream=None):
    return _check(_lib.attn_paged_mixed(
        _dp(q), n_tok, _dp(cu_seqlens), n_seq, n_seq_decode, max_q_len, _dp(k_pool), _dp(v_pool),
        _dp(k_scale), _dp(v_scale), n_pages, _dp(block_table), max_pages_per_seq, _dp(ctx_lens),
        n_head, n_head_kv, head_dim, page_size, kv_dtype, _dp(out), _dp(workspace),
        workspace_bytes, _stream(stream)))


def attn_paged_prefill(q, n_rows, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                       max_pages_per_seq, ctx_len, n_head, n_head_kv, head_dim, page_size,
                       kv_dtype, out, workspace=None, workspace_bytes=0, stream=None):
    return _check(_lib.attn_paged_prefill(
        _dp(q), n_rows, _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages,
        _dp(block_table), max_pages_per_seq, ctx_len, n_head, n_head_kv, head_dim, page_size,
        kv_dtype, _dp(out), _dp(workspace), workspace_bytes, _stream(stream)))


def attn_paged_prefill_fp8(q, n_rows, k_pool, v_pool, k_scale, v_scale, n_pages, block_table,
                           max_pages_per_seq, ctx_len, n_head, n_head_kv, head_dim, page_size,
                           kv_dtype, prefill_fp8, out, workspace=None, workspace_bytes=0,
                           stream=None):
    return _check(_lib.attn_paged_prefill_fp8(
        _dp(q), n_rows, _dp(k_pool), _dp(v_pool), _dp(k_scale), _dp(v_scale), n_pages,
        _dp(block_table), max_pages_per_seq, ctx_len, n_head, n_head_kv, head_dim, page_size,
        kv_dtype, prefill_fp8, _dp(out), _dp(workspace), workspace_bytes, _stream(stream)))


def attn_kv_append(k_new, v_new, slot_mapping, n_tok, k_pool, v_pool, k_scale, v_scale, n_pages,
                   n_head_kv, head_dim, page_size, kv_dtype, stream=None):
    return _check(_lib.attn_kv_append(
        _dp(k_new), _dp(v_new), _dp(slot_mapping), n_tok, _dp(k_pool), _dp(v_pool),
        _dp(k_scale), _dp(v_scale), n_pages, n_head_kv, head_dim, page_size, kv_dtype,
        _stream(stream)))


def attn_block_table_build(ctx_lens_host, page_size: int, pool_pages: int, seed: int,
                           max_pages_per_seq: int, want_slots: bool = False):
    """Host builder; returns the int32 table (and the slot mapping)."""
    cl = np.ascontiguousarray(ctx_lens_host, dtype=np.int32)
    n_seq = cl.shape[0]
    table = np.empty((n_seq, max_pages_per_seq), dtype=np.int32)
    slots = np.empty(int(cl.astype(np.int64).sum()), dtype=np.int32) if want_slots else None
    rc = _lib.attn_block_table_build(
        n_seq, cl.ctypes.data_as(_P), page_size, pool_pages, seed & ((1 << 64) - 1),
        max_pages_per_seq, table.ctypes.data_as(_P),
        None if slots is None else slots.ctypes.data_as(_P))
    _check(rc)
    return (table, slots) if want_slots else table


def attn_check_lengths_host(ctx_lens_host, rows: int, max_pages_per_seq: int,
                            page_size: int) -> int:
    cl = np.ascontiguousarray(ctx_lens_host, dtype=np.int32)
    return _check(_lib.attn_check_lengths_host(cl.ctypes.data_as(_P), cl.shape[0], rows,
                                               max_pages_per_seq, page_size))


def attn_check_block_table_host(block_table_host, ctx_lens_host, max_pages_per_seq: int,
                                page_size: int, n_pages: int) -> int:
    bt = np.ascontiguousarray(block_table_host, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_lens_host, dtype=np.int32)
    return _check(_lib.attn_check_block_table_host(bt.ctypes.data_as(_P), cl.ctypes.data_as(_P),
                                                   cl.shape[0], max_pages_per_seq, page_size,
                                                   n_pages))


def attn_set_kernel_timer(start_event, stop_event) -> None:
    """Time the next attention call's main kernel with two torch.cuda.Events
    (or raw hipEvent_t handles); None cancels."""
    def h(e):
        if e is None:
            return None
        if isinstance(e, int):
            return e
        return e.cuda_event if hasattr(e, "cuda_event") else e.event_id
    _lib.attn_set_kernel_timer(h(start_event), h(stop_event))


def attn_set_max_workgroups(n: int) -> None:
    """Bound the decode/verify kernel's grid for later calls (0 = fill the
    device); results do not depend on it."""
    _lib.attn_set_max_workgroups(int(n))
