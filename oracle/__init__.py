"""CPU oracle for paged grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and the
two share no code: the attention and quantisation arithmetic lives in
``attn_oracle.c`` (plain fp64 loops, OpenMP over rows), the block-table
builder reference in ``block_table.py``.

Every function here takes numpy arrays that hold the *storage* bit patterns
(bf16 as uint16, fp8 codes as uint8, scales as float32), exactly as they sit
in device memory, and returns fp64 results or updates the arrays in place.

Pins (the checks that tie this oracle to something other than itself) live in
``tests/test_oracle_*.py``; no function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from .block_table import build_block_table  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KV_BF16 = 0
KV_FP8 = 1


def build(force: bool = False) -> str:
    """Compile liboracle.so with the host C compiler (IEEE arithmetic, no
    fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_paged_attention.argtypes = [
            P, i32, i32, P, P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, P, P, i32]
        lib.oracle_paged_attention.restype = ctypes.c_int
        lib.oracle_round_q_e4m3.argtypes = [P, i64, i32, P, P]
        lib.oracle_round_q_e4m3.restype = ctypes.c_int
        lib.oracle_paged_attention_window.argtypes = [
            P, i32, i32, P, P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, i32, P, P, P, i32]
        lib.oracle_paged_attention_window.restype = ctypes.c_int
        lib.oracle_kv_append.argtypes = [P, P, P, i32, P, P, P, P, i64, i32, i32, i32, i32]
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_tree_view.argtypes = [
            P, P, P, P, i64, P, i32, i32, i32, ctypes.c_uint32, i32, i32, i32, i32, i32,
            P, P, P, P, i32]
        lib.oracle_tree_view.restype = ctypes.c_int
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def paged_attention(q, k_pool, v_pool, block_table, ctx_lens, *, n_head, n_head_kv, head_dim,
                    page_size, kv_dtype=KV_BF16, k_scale=None, v_scale=None, row_mask=None,
                    window=0, kv_floor=None, q_fp8=False, threads=None) -> np.ndarray:
    """fp64 attention of every row of ``q`` (uint16 bf16 bits, shape
    [n_seq, rows, n_head, head_dim]) over the paged pools.

    Row r of sequence s sits at position p = ctx_lens[s]-rows+r and attends
    to key positions max(kv_floor[s], p-window+1) .. p (window 0: no window;
    kv_floor None: floor 0).  ``row_mask`` ([n_seq, rows], nonzero =
    compute) limits the work; skipped rows come back as NaN.  ``q_fp8``:
    every query vector is first rounded by ``round_q_e4m3`` (the fp8
    prefill's QK^T), the rest is unchanged.
    """
    lib = _load()
    q = _c(q, np.uint16)
    if q_fp8:
        q = round_q_e4m3(q)
    assert q.ndim == 4 and q.shape[2] == n_head and q.shape[3] == head_dim
    n_seq, rows = q.shape[0], q.shape[1]
    bt = _c(block_table, np.int32)
    cl = _c(ctx_lens, np.int32)
    assert bt.ndim == 2 and bt.shape[0] == n_seq and cl.shape == (n_seq,)
    el = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    kp, vp = _c(k_pool, el), _c(v_pool, el)
    assert kp.shape == vp.shape and kp.ndim == 4
    n_pages = kp.shape[0]
    assert kp.shape[1:] == (n_head_kv, page_size, head_dim)
    ks = _c(k_scale, np.float32)
    vs = _c(v_scale, np.float32)
    if kv_dtype == KV_FP8:
        assert ks is not None and vs is not None and ks.shape == (n_pages, n_head_kv)
    mask = None if row_mask is None else _c(np.asarray(row_mask).reshape(n_seq * rows) != 0,
                                            np.uint8)
    fl = None if kv_floor is None else _c(kv_floor, np.int32)
    assert fl is None or fl.shape == (n_seq,)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    rc = lib.oracle_paged_attention_window(
        _ptr(q), n_seq, rows, _ptr(kp), _ptr(vp), _ptr(ks), _ptr(vs), n_pages, _ptr(bt),
        bt.shape[1], _ptr(cl), n_head, n_head_kv, head_dim, page_size, kv_dtype, int(window),
        _ptr(fl), _ptr(mask), _ptr(out), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_paged_attention failed with %d" % rc)
    return out


def kv_append(k_new, v_new, slot_mapping, k_pool, v_pool, k_scale=None, v_scale=None, *,
              n_head_kv, head_dim, page_size, kv_dtype=KV_BF16) -> None:
    """Write rows into their slots, updating the numpy pools (and, for fp8,
    the scales) in place.  See ``oracle_kv_append`` in attn_oracle.c."""
    lib = _load()
    kn, vn = _c(k_new, np.uint16), _c(v_new, np.uint16)
    sm = _c(slot_mapping, np.int32)
    n_tok = sm.shape[0]
    assert kn.shape == (n_tok, n_head_kv, head_dim) and vn.shape == kn.shape
    for a in (k_pool, v_pool) + ((k_scale, v_scale) if kv_dtype == KV_FP8 else ()):
        assert a.flags.c_contiguous
    el = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    assert k_pool.dtype == el and v_pool.dtype == el
    rc = lib.oracle_kv_append(_ptr(kn), _ptr(vn), _ptr(sm), n_tok, _ptr(k_pool), _ptr(v_pool),
                              _ptr(k_scale), _ptr(v_scale), k_pool.shape[0], n_head_kv, head_dim,
                              page_size, kv_dtype)
    if rc != 0:
        raise ValueError("oracle_kv_append failed with %d" % rc)


def tree_view(k_pool, v_pool, k_scale, v_scale, table_row, ctx_len, rows, mask, r, *,
              n_head_kv, head_dim, page_size, kv_dtype=KV_BF16):
    """The cache row ``r`` of a tree-shaped round attends: its branch laid out
    as a plain sequence in ``ceil(L / page_size)`` private pages (identity
    block table).  Returns ``(k, v, k_scale, v_scale, L)`` (scales None for
    bf16).  See ``oracle_tree_view`` in attn_oracle.c for the rule."""
    lib = _load()
    tab = _c(table_row, np.int32)
    for a in (k_pool, v_pool) + ((k_scale, v_scale) if kv_dtype == KV_FP8 else ()):
        assert a.flags.c_contiguous
    el = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    assert k_pool.dtype == el and v_pool.dtype == el
    n_rows = ctx_len - rows + bin(int(mask) & ((1 << rows) - 1)).count("1")
    npg = max(1, -(-n_rows // page_size))
    shape = (npg, n_head_kv, page_size, head_dim)
    k2, v2 = np.zeros(shape, el), np.zeros(shape, el)
    ks2 = vs2 = None
    if kv_dtype == KV_FP8:
        ks2 = np.zeros((npg, n_head_kv), np.float32)
        vs2 = np.zeros((npg, n_head_kv), np.float32)
    rc = lib.oracle_tree_view(_ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                              k_pool.shape[0], _ptr(tab), tab.shape[0], int(ctx_len), int(rows),
                              int(mask) & 0xFFFFFFFF, int(r), n_head_kv, head_dim, page_size,
                              kv_dtype, _ptr(k2), _ptr(v2), _ptr(ks2), _ptr(vs2), npg)
    if rc < 0:
        raise ValueError("oracle_tree_view failed with %d" % rc)
    return k2, v2, ks2, vs2, rc


def round_q_e4m3(q, return_exps=False):
    """Query vectors rounded to E4M3 at a power-of-two scale per vector (the
    last axis), returned as bf16 bits of the same shape; see
    ``oracle_round_q_e4m3`` in attn_oracle.c for the rule."""
    lib = _load()
    qq = _c(q, np.uint16)
    d = qq.shape[-1]
    n = qq.size // d
    out = np.empty_like(qq)
    exps = np.empty(n, np.int32)
    rc = lib.oracle_round_q_e4m3(_ptr(qq), n, d, _ptr(out), _ptr(exps))
    if rc != 0:
        raise ValueError("oracle_round_q_e4m3 failed with %d" % rc)
    return (out, exps.reshape(qq.shape[:-1])) if return_exps else out


def e4m3_value(codes) -> np.ndarray:
    """fp64 value of each OCP E4M3 code."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_value(int(x)) for x in c.reshape(-1)],
                    dtype=np.float64).reshape(c.shape)


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value (ties to even, saturating)."""
    lib = _load()
    a = np.asarray(y, dtype=np.float32)
    return np.array([lib.oracle_e4m3_encode(float(x)) for x in a.reshape(-1)],
                    dtype=np.uint8).reshape(a.shape)


def bf16_bits_to_f64(a) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
