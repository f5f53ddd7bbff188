"""Oracle for the paged-KV hot path. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. It shares no code with the HIP library: its index metadata is built here in
plain Python and its store/attention arithmetic lives in ``oracle.c`` (double precision),
loaded through ctypes.

Pins (tests/test_oracle_*.py): the worked examples the pages print for slot mapping, packing
and decode metadata; fp64 brute force with a dense causal mask on tiny inputs; closed forms
(all-zero keys give the mean of the visible values, one key gives that value); invariants
(physical block permutation, decode equals the last prefill row, chunked or prefix-cached
prefill equals uncached prefill, GQA equals MHA with repeated kv heads, weights sum to one).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .meta import prepare_block_tables, prepare_decode, prepare_prefill  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (OpenMP on). No fast-math: sums keep their written order."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        L.oracle_store_kvcache.argtypes = [p, i64, p, i64, p, p, p, i64, i64]
        L.oracle_store_kvcache.restype = i64
        L.oracle_attend_row.argtypes = [p, p, p, i64, i64, ctypes.c_double, p, p]
        L.oracle_attend_row.restype = None
        L.oracle_attn_prefill.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                          ctypes.c_double, p]
        L.oracle_attn_prefill.restype = None
        L.oracle_attn_decode.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                         ctypes.c_double, p]
        L.oracle_attn_decode.restype = None
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _rows(a: np.ndarray, width: int):
    """(pointer, row stride in elements) of a 2-D uint16 view whose rows are contiguous."""
    assert a.dtype == np.uint16 and a.ndim == 2 and a.shape[1] == width
    assert a.strides[1] == 2 and a.strides[0] % 2 == 0
    return _ptr(a), a.strides[0] // 2


def store_kvcache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  slot_mapping: np.ndarray) -> int:
    """Bit copy of token rows into pool rows (in place). key/value: [N, D] uint16 views (rows
    contiguous, any row stride); caches: [num_slots, D] uint16 contiguous."""
    n, D = key.shape
    kp, ks = _rows(key, D)
    vp, vs = _rows(value, D)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.shape[1] == D and v_cache.shape[1] == D
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    assert sm.shape == (n,)
    return int(lib().oracle_store_kvcache(kp, ks, vp, vs, _ptr(k_cache), _ptr(v_cache), _ptr(sm),
                                          n, D))


def attend_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one query over contiguous keys: returns (out[d], weights[n])."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    n, d = K.shape
    out = np.zeros(d, dtype=np.float64)
    w = np.zeros(max(n, 1), dtype=np.float64)
    lib().oracle_attend_row(_ptr(q), _ptr(K), _ptr(V), n, d, float(scale), _ptr(out), _ptr(w))
    return out, w[:n]


def attn_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, cu_seqlens_q,
                 cu_seqlens_k, block_tables: np.ndarray, num_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, scale: float) -> np.ndarray:
    """q: [total_q, Hq, d] uint16 bf16 bits; caches [num_slots, Hkv*d] uint16. Returns float64
    [total_q, Hq, d]."""
    assert head_dim <= 512 and num_heads % num_kv_heads == 0
    q = np.ascontiguousarray(q, dtype=np.uint16)
    cq = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    batch = len(cq) - 1
    assert bt.ndim == 2 and bt.shape[0] == batch
    out = np.zeros((int(cq[-1]), num_heads, head_dim), dtype=np.float64)
    lib().oracle_attn_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cq), _ptr(ck), _ptr(bt),
                              bt.shape[1], batch, num_heads, num_kv_heads, head_dim, block_size,
                              float(scale), _ptr(out))
    return out


def attn_prefill_packed(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_q, cu_seqlens_k,
                        num_heads: int, num_kv_heads: int, head_dim: int,
                        scale: float) -> np.ndarray:
    """Prefill with no cached context over packed fresh K/V ("Nano-vLLM Field Guide", Step
    10.3: attention over the freshly projected q, k, v with cu_seqlens describing the packed
    sequences). k, v: [total_k, Hkv*d] uint16 bf16 bits; key j of sequence b is row
    cu_seqlens_k[b] + j. This is the paged computation with blocks of one token and a table
    naming those rows, so it runs through the same code. Returns float64 [total_q, Hq, d]."""
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    lens = ck[1:] - ck[:-1]
    width = max(1, int(lens.max()) if len(lens) else 1)
    table = np.full((len(lens), width), -1, dtype=np.int32)
    for b, (start, n) in enumerate(zip(ck[:-1], lens)):
        table[b, :n] = np.arange(start, start + n, dtype=np.int32)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    return attn_prefill(q, k, v, cu_seqlens_q, cu_seqlens_k, table, num_heads, num_kv_heads,
                        head_dim, 1, scale)


def attn_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, context_lens,
                block_tables: np.ndarray, num_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, scale: float) -> np.ndarray:
    """q: [B, Hq, d] uint16 bf16 bits. Returns float64 [B, Hq, d]."""
    assert head_dim <= 512 and num_heads % num_kv_heads == 0
    q = np.ascontiguousarray(q, dtype=np.uint16)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    batch = len(cl)
    assert bt.ndim == 2 and bt.shape[0] == batch
    out = np.zeros((batch, num_heads, head_dim), dtype=np.float64)
    lib().oracle_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cl), _ptr(bt),
                             bt.shape[1], batch, num_heads, num_kv_heads, head_dim, block_size,
                             float(scale), _ptr(out))
    return out
