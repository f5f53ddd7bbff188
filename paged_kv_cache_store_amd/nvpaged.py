"""Python binding of libnvpaged.so (the C ABI in include/nv_paged.h).

Argument marshalling only: tensors are checked for dtype, device and layout, then their data
pointers, sizes and the current HIP stream are passed to the C entry points of the same
names. Every step of the computation runs in the library's kernels; there is no fallback. If
the library has not been built this module raises ImportError on import.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvpaged.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py build` "
                      "(or paged_kv_cache_store_amd/build.py) before using the HIP path")

EXPORTS = ("nv_status_string", "nv_store_kvcache", "nv_paged_attn_prefill",
           "nv_attn_prefill_packed", "nv_qk_norm_rope_store",
           "nv_paged_attn_decode_workspace_size", "nv_paged_attn_decode",
           "nv_paged_attn_decode_split_keys", "nv_paged_attn_decode_store",
           "nv_paged_attn_decode_noalloc",
           "nv_prepare_prefill", "nv_prepare_decode",
           "nv_check_indices")

_p, _i32, _i64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_size_t)


def _bind(path: str) -> ctypes.CDLL:
    """Loads a build of the library and declares the C signatures of its entry points."""
    L = ctypes.CDLL(path)
    L.nv_status_string.argtypes = [ctypes.c_int]
    L.nv_status_string.restype = ctypes.c_char_p
    L.nv_store_kvcache.argtypes = [_p, _i64, _p, _i64, _p, _p, _p, _i64, _i32, _i32, _i64, _p]
    L.nv_store_kvcache.restype = ctypes.c_int
    L.nv_paged_attn_prefill.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _p, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _f32, _p, _p]
    L.nv_paged_attn_prefill.restype = ctypes.c_int
    L.nv_attn_prefill_packed.argtypes = [_p, _p, _i64, _p, _i64, _p, _p, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _f32, _p, _p]
    L.nv_attn_prefill_packed.restype = ctypes.c_int
    L.nv_qk_norm_rope_store.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _f32, _p, _p, _p, _p,
                                        _p, _i64, _i32, _i32, _i32, _i64, _p]
    L.nv_qk_norm_rope_store.restype = ctypes.c_int
    L.nv_paged_attn_decode_workspace_size.argtypes = [_i32] * 6
    L.nv_paged_attn_decode_workspace_size.restype = _sz
    L.nv_paged_attn_decode_split_keys.argtypes = [_i32] * 4
    L.nv_paged_attn_decode_split_keys.restype = _i32
    L.nv_paged_attn_decode.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _f32, _p, _sz, _p, _p]
    L.nv_paged_attn_decode.restype = ctypes.c_int
    L.nv_paged_attn_decode_noalloc.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _f32, _p, _p]
    L.nv_paged_attn_decode_noalloc.restype = ctypes.c_int
    L.nv_paged_attn_decode_store.argtypes = [_p, _p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _p,
                                             _i32, _i32, _i32, _i32, _i32, _i32, _f32, _p, _sz,
                                             _p, _i64, _p, _p]
    L.nv_paged_attn_decode_store.restype = ctypes.c_int
    L.nv_prepare_prefill.argtypes = [_p, _p, _p, _p, _i32, _i32, _p, _p, _p, _p, _p, _p, _i32,
                                     _p]
    L.nv_prepare_prefill.restype = ctypes.c_int
    L.nv_prepare_decode.argtypes = [_p, _p, _p, _p, _i32, _i32, _p, _p, _p, _i32]
    L.nv_prepare_decode.restype = ctypes.c_int
    L.nv_check_indices.argtypes = [_p, _i64, _i64, _p, _p, _i32, _i32, _i32, _i64, _p]
    L.nv_check_indices.restype = ctypes.c_int
    return L


_lib = _bind(LIB_PATH)

NV_OK, NV_ERR_INVALID_ARG, NV_ERR_UNSUPPORTED, NV_ERR_LAUNCH, NV_ERR_WORKSPACE, NV_ERR_SCRATCH = \
    0, -1, -2, -3, -4, -5
NV_DECODE_SCRATCH_BYTES = 32 << 20  # the static workspace of nv_paged_attn_decode_noalloc


class NvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {nv_status_string(status)}")


def nv_status_string(status: int) -> str:
    return _lib.nv_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != NV_OK:
        raise NvError(status, where)


def lib() -> ctypes.CDLL:
    return _lib


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _pool_rows(cache: torch.Tensor, name: str, row_elems: int) -> int:
    _dev(cache, name, torch.bfloat16)
    if not cache.is_contiguous() or cache.numel() % row_elems:
        raise ValueError(f"{name} must be a contiguous pool of rows of {row_elems} values")
    return cache.numel() // row_elems


# ---------------------------------------------------------------- device calls

def nv_store_kvcache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """key/value [N, Hkv, d] bf16 (last two dims contiguous, any row stride); caches of
    [num_slots, Hkv*d] (or [num_blocks, block_size, Hkv, d]) bf16; slot_mapping int32 [N]."""
    _dev(key, "key", torch.bfloat16)
    _dev(value, "value", torch.bfloat16)
    _dev(slot_mapping, "slot_mapping", torch.int32)
    if key.dim() != 3 or value.shape != key.shape:
        raise ValueError("key and value must both be [N, num_kv_heads, head_dim]")
    n, hkv, d = key.shape
    for t, nm in ((key, "key"), (value, "value")):
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{nm}: last dim must be contiguous and heads head_dim apart")
    if slot_mapping.numel() != n or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous with one entry per token")
    D = hkv * d
    ns = _pool_rows(k_cache, "k_cache", D)
    if _pool_rows(v_cache, "v_cache", D) != ns:
        raise ValueError("k_cache and v_cache differ in size")
    _check(_lib.nv_store_kvcache(key.data_ptr(), key.stride(0), value.data_ptr(), value.stride(0),
                                 k_cache.data_ptr(), v_cache.data_ptr(), slot_mapping.data_ptr(),
                                 n, hkv, d, ns, _stream(stream)), "nv_store_kvcache")


def _cu_seqlens(cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor) -> int:
    for t, nm in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _dev(t, nm, torch.int32)
        if t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous 1-D tensor")
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    return batch


def _q_out(q: torch.Tensor, out: torch.Tensor | None) -> torch.Tensor:
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, num_heads, head_dim] tensor")
    if out is None:
        return torch.empty_like(q)
    _dev(out, "out", torch.bfloat16)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous and shaped like q")
    return out


def nv_attn_prefill_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                           max_seqlen_q: int, max_seqlen_k: int, softmax_scale: float,
                           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal varlen attention over packed fresh K/V: k, v [total_k, Hkv, d] bf16 (last two
    dims contiguous, any row stride, e.g. views into a fused QKV output); sequence b's keys are
    rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]. q [total_q, Hq, d] -> out, bottom-right mask."""
    out = _q_out(q, out)
    _, hq, d = q.shape
    for t, nm in ((k, "k"), (v, "v")):
        _dev(t, nm, torch.bfloat16)
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != d or t.shape[2] != d:
            raise ValueError(f"{nm}: [total_k, num_kv_heads, head_dim] with the last two dims "
                             "contiguous")
    if v.shape != k.shape:
        raise ValueError("k and v differ in shape")
    batch = _cu_seqlens(cu_seqlens_q, cu_seqlens_k)
    _check(_lib.nv_attn_prefill_packed(q.data_ptr(), k.data_ptr(), k.stride(0), v.data_ptr(),
                                       v.stride(0), cu_seqlens_q.data_ptr(),
                                       cu_seqlens_k.data_ptr(), int(max_seqlen_q),
                                       int(max_seqlen_k), batch, hq, k.shape[1], d,
                                       float(softmax_scale), out.data_ptr(), _stream(stream)),
           "nv_attn_prefill_packed")
    return out


def rope_cos_sin_cache(max_position: int, head_dim: int, base: float, device) -> torch.Tensor:
    """The engine's rotary table, fp32 [max_position, head_dim]: row p = cos(p theta_i) for
    i < head_dim/2, then sin(p theta_i), theta_i = base^(-2i/head_dim), computed in fp32 as the
    engine does ("Nano-vLLM Field Guide", Step 10.5, rotary_embedding.py). This init-time table
    is an input of the fused call, like the norm weights, not a step of the hot path."""
    inv_freq = 1.0 / (base ** (torch.arange(0, head_dim, 2, dtype=torch.float) / head_dim))
    t = torch.arange(max_position, dtype=torch.float)
    freqs = torch.outer(t, inv_freq)
    return torch.cat((freqs.cos(), freqs.sin()), dim=-1).to(device)


def nv_qk_norm_rope_store(qkv: torch.Tensor, positions: torch.Tensor, q_norm_weight: torch.Tensor,
                          k_norm_weight: torch.Tensor, cos_sin_cache: torch.Tensor, eps: float,
                          k_cache: torch.Tensor, v_cache: torch.Tensor,
                          slot_mapping: torch.Tensor, num_heads: int, num_kv_heads: int,
                          q_out: torch.Tensor | None = None, want_k: bool = False,
                          stream=None):
    """qkv [N, (Hq + 2 Hkv) d] bf16 (last dim contiguous, any row stride): per-head RMSNorm and
    rotary embedding of q and k, store of k and v at slot_mapping. Returns (q_out [N, Hq, d],
    k_out [N, Hkv, d] or None)."""
    _dev(qkv, "qkv", torch.bfloat16)
    _dev(positions, "positions", torch.int64)
    _dev(slot_mapping, "slot_mapping", torch.int32)
    _dev(cos_sin_cache, "cos_sin_cache", torch.float32)
    for t, nm in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        _dev(t, nm, torch.bfloat16)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if qkv.dim() != 2 or qkv.stride(1) != 1:
        raise ValueError("qkv must be [num_tokens, width] with a contiguous last dim")
    n = qkv.shape[0]
    d = cos_sin_cache.shape[1]
    if cos_sin_cache.dim() != 2 or not cos_sin_cache.is_contiguous():
        raise ValueError("cos_sin_cache must be a contiguous [max_position, head_dim] tensor")
    if qkv.shape[1] != (num_heads + 2 * num_kv_heads) * d:
        raise ValueError("qkv width must be (num_heads + 2 num_kv_heads) * head_dim")
    if positions.numel() != n or slot_mapping.numel() != n:
        raise ValueError("positions and slot_mapping need one entry per token")
    ns = _pool_rows(k_cache, "k_cache", num_kv_heads * d)
    if _pool_rows(v_cache, "v_cache", num_kv_heads * d) != ns:
        raise ValueError("k_cache and v_cache differ in size")
    if q_out is None:
        q_out = torch.empty(n, num_heads, d, dtype=torch.bfloat16, device=qkv.device)
    k_out = (torch.empty(n, num_kv_heads, d, dtype=torch.bfloat16, device=qkv.device)
             if want_k else None)
    _check(_lib.nv_qk_norm_rope_store(qkv.data_ptr(), qkv.stride(0), positions.data_ptr(),
                                      q_norm_weight.data_ptr(), k_norm_weight.data_ptr(),
                                      cos_sin_cache.data_ptr(), cos_sin_cache.shape[0],
                                      float(eps), q_out.data_ptr(),
                                      k_out.data_ptr() if k_out is not None else None,
                                      k_cache.data_ptr(), v_cache.data_ptr(),
                                      slot_mapping.data_ptr(), n, int(num_heads),
                                      int(num_kv_heads), d, ns, _stream(stream)),
           "nv_qk_norm_rope_store")
    return q_out, k_out


def nv_paged_attn_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                          max_seqlen_q: int, max_seqlen_k: int, block_tables: torch.Tensor,
                          num_kv_heads: int, block_size: int, softmax_scale: float,
                          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [total_q, Hq, d] bf16 contiguous -> out [total_q, Hq, d] bf16 (causal, bottom-right).
    block_tables None: k_cache/v_cache are contiguous packed fresh K/V [total_k, Hkv, d]."""
    out = _q_out(q, out)
    _, hq, d = q.shape
    _pool_rows(k_cache, "k_cache", num_kv_heads * d)
    _pool_rows(v_cache, "v_cache", num_kv_heads * d)
    batch = _cu_seqlens(cu_seqlens_q, cu_seqlens_k)
    bt_ptr, width = 0, 0
    if block_tables is not None:
        _dev(block_tables, "block_tables", torch.int32)
        if block_tables.dim() != 2 or block_tables.shape[0] != batch or \
                not block_tables.is_contiguous():
            raise ValueError("block_tables must be a contiguous [batch, max_blocks] tensor")
        bt_ptr, width = block_tables.data_ptr(), block_tables.shape[1]
    _check(_lib.nv_paged_attn_prefill(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                      cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                      int(max_seqlen_q), int(max_seqlen_k), bt_ptr, width, batch,
                                      hq, int(num_kv_heads), d, int(block_size),
                                      float(softmax_scale), out.data_ptr(), _stream(stream)),
           "nv_paged_attn_prefill")
    return out


def nv_paged_attn_decode_workspace_size(batch: int, num_heads: int, num_kv_heads: int,
                                        head_dim: int, max_blocks_per_seq: int,
                                        block_size: int) -> int:
    return int(_lib.nv_paged_attn_decode_workspace_size(batch, num_heads, num_kv_heads, head_dim,
                                                        max_blocks_per_seq, block_size))


def nv_paged_attn_decode_split_keys(batch: int, num_kv_heads: int, max_blocks_per_seq: int,
                                    block_size: int) -> int:
    return int(_lib.nv_paged_attn_decode_split_keys(batch, num_kv_heads, max_blocks_per_seq,
                                                    block_size))


def decode_workspace(q: torch.Tensor, num_kv_heads: int, block_tables: torch.Tensor,
                     block_size: int) -> torch.Tensor:
    """Allocates (with torch) a workspace of the size the decode call needs."""
    b, hq, d = q.shape
    nbytes = nv_paged_attn_decode_workspace_size(b, hq, num_kv_heads, d, block_tables.shape[1],
                                                 block_size)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)


def nv_paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         context_lens: torch.Tensor, block_tables: torch.Tensor,
                         num_kv_heads: int, block_size: int, softmax_scale: float,
                         workspace: torch.Tensor | None = None,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [B, Hq, d] bf16 contiguous -> out [B, Hq, d] bf16."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_heads, head_dim] tensor")
    b, hq, d = q.shape
    _pool_rows(k_cache, "k_cache", num_kv_heads * d)
    _pool_rows(v_cache, "v_cache", num_kv_heads * d)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(block_tables, "block_tables", torch.int32)
    if context_lens.numel() != b or not context_lens.is_contiguous():
        raise ValueError("context_lens must have one entry per row")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [batch, max_blocks] tensor")
    if workspace is None:
        workspace = decode_workspace(q, num_kv_heads, block_tables, block_size)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out must be contiguous and shaped like q")
    _check(_lib.nv_paged_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                     context_lens.data_ptr(), block_tables.data_ptr(),
                                     block_tables.shape[1], b, hq, int(num_kv_heads), d,
                                     int(block_size), float(softmax_scale), workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), out.data_ptr(),
                                     _stream(stream)), "nv_paged_attn_decode")
    return out


def nv_paged_attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 context_lens: torch.Tensor, block_tables: torch.Tensor,
                                 num_kv_heads: int, block_size: int, softmax_scale: float,
                                 out: torch.Tensor, stream=None) -> torch.Tensor:
    """nv_paged_attn_decode with the library's static workspace: the C call allocates nothing
    (and neither does this wrapper: ``out`` is the caller's). q, out [B, Hq, d] bf16."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_heads, head_dim] tensor")
    b, hq, d = q.shape
    _pool_rows(k_cache, "k_cache", num_kv_heads * d)
    _pool_rows(v_cache, "v_cache", num_kv_heads * d)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(block_tables, "block_tables", torch.int32)
    if context_lens.numel() != b or not context_lens.is_contiguous():
        raise ValueError("context_lens must have one entry per row")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [batch, max_blocks] tensor")
    _dev(out, "out", torch.bfloat16)
    if out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous and shaped like q")
    _check(_lib.nv_paged_attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                             context_lens.data_ptr(), block_tables.data_ptr(),
                                             block_tables.shape[1], b, hq, int(num_kv_heads), d,
                                             int(block_size), float(softmax_scale),
                                             out.data_ptr(), _stream(stream)),
           "nv_paged_attn_decode_noalloc")
    return out


def nv_paged_attn_decode_store(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                               slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                               v_cache: torch.Tensor, context_lens: torch.Tensor,
                               block_tables: torch.Tensor, num_kv_heads: int, block_size: int,
                               softmax_scale: float, workspace: torch.Tensor | None = None,
                               out: torch.Tensor | None = None,
                               counters: torch.Tensor | None = None,
                               stream=None) -> torch.Tensor:
    """Store of the decode rows' key/value [B, Hkv, d] at slot_mapping [B], then decode
    attention of q [B, Hq, d], in one launch; returns out [B, Hq, d] bf16.

    ``counters``: optional int32 device tensor of at least B * Hkv entries, all zero (e.g. from
    ``decode_counters``); given, split rows are merged inside the same launch (no merge
    kernel), and the call leaves the entries zero again."""
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [batch, num_heads, head_dim] tensor")
    b, hq, d = q.shape
    for t, nm in ((key, "key"), (value, "value")):
        _dev(t, nm, torch.bfloat16)
        if t.dim() != 3 or t.shape != (b, num_kv_heads, d) or t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{nm} must be [batch, num_kv_heads, head_dim] with contiguous heads")
    _dev(slot_mapping, "slot_mapping", torch.int32)
    if slot_mapping.numel() != b or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous with one entry per row")
    ns = _pool_rows(k_cache, "k_cache", num_kv_heads * d)
    if _pool_rows(v_cache, "v_cache", num_kv_heads * d) != ns:
        raise ValueError("k_cache and v_cache differ in size")
    _dev(context_lens, "context_lens", torch.int32)
    _dev(block_tables, "block_tables", torch.int32)
    if context_lens.numel() != b or not context_lens.is_contiguous():
        raise ValueError("context_lens must have one entry per row")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous [batch, max_blocks] tensor")
    if workspace is None:
        workspace = decode_workspace(q, num_kv_heads, block_tables, block_size)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out must be contiguous and shaped like q")
    cptr, ncnt = 0, 0
    if counters is not None:
        _dev(counters, "counters", torch.int32)
        if not counters.is_contiguous() or counters.numel() < b * num_kv_heads:
            raise ValueError("counters must be contiguous with at least batch * num_kv_heads entries")
        cptr, ncnt = counters.data_ptr(), counters.numel()
    _check(_lib.nv_paged_attn_decode_store(
        q.data_ptr(), key.data_ptr(), key.stride(0), value.data_ptr(), value.stride(0),
        slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ns,
        context_lens.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], b, hq,
        int(num_kv_heads), d, int(block_size), float(softmax_scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), cptr, ncnt, out.data_ptr(),
        _stream(stream)),
        "nv_paged_attn_decode_store")
    return out


def decode_counters(max_batch: int, num_kv_heads: int, device) -> torch.Tensor:
    """Zeroed arrival counters for ``nv_paged_attn_decode_store`` (one per row and kv head, for
    batches up to max_batch); every call leaves them zero, so they are allocated once."""
    return torch.zeros(max(1, max_batch * num_kv_heads), dtype=torch.int32, device=device)


# ---------------------------------------------------------------- host metadata

def _ragged(seqs):
    lens = [len(s.block_table) for s in seqs]
    offsets = np.zeros(len(seqs) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(lens, dtype=np.int64)
    ids = np.array([i for s in seqs for i in s.block_table], dtype=np.int32)
    if ids.size == 0:
        ids = np.zeros(1, dtype=np.int32)
    cached = np.array([s.num_cached for s in seqs], dtype=np.int32)
    new = np.array([s.num_new for s in seqs], dtype=np.int32)
    return cached, new, offsets, ids, max(lens, default=0)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def nv_prepare_prefill(seqs, block_size: int) -> dict:
    """Host metadata of a packed prefill batch (numpy int32 arrays + host ints)."""
    cached, new, offsets, ids, width = _ragged(seqs)
    batch = len(seqs)
    slots = np.zeros(max(int(new.sum()), 1), dtype=np.int32)
    cu_q = np.zeros(batch + 1, dtype=np.int32)
    cu_k = np.zeros(batch + 1, dtype=np.int32)
    bt = np.zeros((batch, max(width, 1)), dtype=np.int32)
    mq, mk, has = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.nv_prepare_prefill(_ptr(cached), _ptr(new), _ptr(offsets), _ptr(ids), batch,
                                   block_size, _ptr(slots), _ptr(cu_q), _ptr(cu_k),
                                   ctypes.addressof(mq), ctypes.addressof(mk), _ptr(bt),
                                   bt.shape[1], ctypes.addressof(has)), "nv_prepare_prefill")
    return dict(slot_mapping=slots[:int(new.sum())], cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                max_seqlen_q=mq.value, max_seqlen_k=mk.value, block_tables=bt,
                has_cached_context=bool(has.value))


def nv_prepare_decode(seqs, block_size: int) -> dict:
    """Host metadata of a decode batch (numpy int32 arrays)."""
    cached, new, offsets, ids, width = _ragged(seqs)
    batch = len(seqs)
    slots = np.zeros(batch, dtype=np.int32)
    ctx = np.zeros(batch, dtype=np.int32)
    bt = np.zeros((batch, max(width, 1)), dtype=np.int32)
    _check(_lib.nv_prepare_decode(_ptr(cached), _ptr(new), _ptr(offsets), _ptr(ids), batch,
                                  block_size, _ptr(slots), _ptr(ctx), _ptr(bt), bt.shape[1]),
           "nv_prepare_decode")
    return dict(slot_mapping=slots, context_lens=ctx, block_tables=bt)


def nv_check_indices(slot_mapping: np.ndarray, num_slots: int, block_tables: np.ndarray,
                     lens: np.ndarray, block_size: int, num_blocks: int):
    """Host check of index preconditions; returns (ok, first_bad_index)."""
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ln = np.ascontiguousarray(lens, dtype=np.int32)
    bad = ctypes.c_int64(-1)
    st = _lib.nv_check_indices(_ptr(sm), sm.size, num_slots, _ptr(bt), _ptr(ln), ln.size,
                               bt.shape[1] if bt.ndim == 2 else 0, block_size, num_blocks,
                               ctypes.addressof(bad))
    if st not in (NV_OK, NV_ERR_INVALID_ARG):
        _check(st, "nv_check_indices")
    return st == NV_OK, int(bad.value)

