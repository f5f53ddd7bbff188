"""Test-side helpers: bf16 bit views and an fp64 brute-force attention used to pin the oracle.

The brute force is deliberately built differently from the oracle: K/V are gathered block by
block into dense per-sequence arrays, kv heads are expanded with numpy.repeat, and attention
is one dense matrix product per head with an explicit mask matrix. It is only used on tiny
inputs.
"""
import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (a copy on the host; views keep their strides)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_kv(cache_bits: np.ndarray, table, n_keys: int, shape) -> np.ndarray:
    """[n_keys, Hkv, d] float64 of one sequence, copied block by block."""
    bs, hkv, d = shape.block_size, shape.num_kv_heads, shape.head_dim
    pool = bf16_bits_to_f64(cache_bits).reshape(-1, bs, hkv, d)
    parts = []
    for lb in range(-(-n_keys // bs)):
        take = min(bs, n_keys - lb * bs)
        parts.append(pool[table[lb], :take])
    if not parts:
        return np.zeros((0, hkv, d))
    return np.concatenate(parts, axis=0)


def brute_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    offset: int, head_map="contiguous", align="bottom_right",
                    drop_scale=False) -> np.ndarray:
    """q [Lq, Hq, d] float64; K/V [Lk, Hkv, d] float64. Row i sees keys j <= offset + i.

    The keyword arguments plant known mistakes for sensitivity checks: a head map of
    ``h % Hkv`` instead of ``h // G``, a top-left causal alignment, or a missing scale."""
    Lq, Hq, d = q.shape
    Lk, Hkv, _ = K.shape
    G = Hq // Hkv
    if head_map == "contiguous":
        Kx, Vx = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    else:
        Kx, Vx = np.tile(K, (1, G, 1)), np.tile(V, (1, G, 1))
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    off = offset if align == "bottom_right" else 0
    mask = np.where(j <= off + i, 0.0, -np.inf)
    out = np.zeros((Lq, Hq, d))
    sc = 1.0 if drop_scale else scale
    for h in range(Hq):
        S = (q[:, h, :] @ Kx[:, h, :].T) * sc + mask
        with np.errstate(invalid="ignore"):
            S = S - S.max(axis=1, keepdims=True)
            W = np.exp(S)
            W = W / W.sum(axis=1, keepdims=True)
        W = np.nan_to_num(W)
        out[:, h, :] = W @ Vx[:, h, :]
    return out
