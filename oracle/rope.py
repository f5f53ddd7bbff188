"""Oracle for the per-head RMSNorm + rotary embedding applied to q and k before the K/V store.

Test infrastructure (like the rest of oracle/): only tests/, smoke() and the CPU-baseline leg
of bench.py use it; the HIP path never does.

What is computed ("Nano-vLLM Field Guide", Step 9.5, Qwen3Attention.forward: q_norm and k_norm
on every head, then rotary_emb on q and k, then the store; Step 10.4, layernorm.py, for
RMSNorm; Step 10.5, rotary_embedding.py, for the table and the rotation):

  RMSNorm of one head x (d values):  n = round_bf16(x / sqrt(mean(x^2) + eps)),
                                     y = round_bf16(n * w)   (w the bf16 weight of length d)
  rotary embedding at position p:    with x1, x2 the first and second halves of y and
                                     c_i = cos(p * theta_i), s_i = sin(p * theta_i),
                                     theta_i = base^(-2 i / d), i < d/2:
                                     z1 = round_bf16(x1 * c - x2 * s)
                                     z2 = round_bf16(x2 * c + x1 * s)

The pages compute in fp32 with bf16 results; here every value between two roundings is
carried in float64 and rounded to bf16 (nearest even) exactly where the pages round, so the
result is the pages' definition up to the fp32 rounding of their intermediates. v is not
transformed. Everything is plain numpy, vectorised over tokens and heads.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32) \
        .astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); returns float64 values that
    are bf16-representable. Finite, normal-range inputs (as in these computations)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    m, e = np.frexp(x[nz])              # x = m * 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0)              # 8 significant bits; numpy rounds half to even
    out[nz] = np.ldexp(q / 256.0, e)
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable float64 values to their bf16 bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)  # exact for bf16 values
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def rope_table_f64(max_position: int, head_dim: int, base: float) -> np.ndarray:
    """[max_position, head_dim] float64: cos(p theta_i) for i < d/2, then sin(p theta_i),
    theta_i = base^(-2 i / d) (the rotary table's definition, evaluated in float64)."""
    i = np.arange(0, head_dim, 2, dtype=np.float64)
    theta = base ** (-i / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float, rounded: bool = True) -> np.ndarray:
    """x [..., d] float64 (bf16 values), w [d] float64 (bf16 values). With rounded=False the
    two bf16 roundings are skipped (for the invariants of the exact formula)."""
    var = np.mean(x * x, axis=-1, keepdims=True)
    n = x / np.sqrt(var + eps)
    if rounded:
        n = round_bf16(n)
    y = n * w
    return round_bf16(y) if rounded else y


def rope(x: np.ndarray, positions: np.ndarray, table: np.ndarray,
         rounded: bool = True) -> np.ndarray:
    """x [N, H, d] float64; positions [N]; table [max_position, d] (cos half, then sin half).
    Rotates the pair (x[i], x[i + d/2]) by the angle of frequency i at the token's position."""
    d = x.shape[-1]
    h = d // 2
    cs = table[np.asarray(positions, dtype=np.int64)]        # [N, d]
    c = cs[:, None, :h]
    s = cs[:, None, h:]
    x1, x2 = x[..., :h], x[..., h:]
    z = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return round_bf16(z) if rounded else z


def qk_norm_rope(qkv_bits: np.ndarray, positions, q_weight_bits, k_weight_bits, table,
                 num_heads: int, num_kv_heads: int, head_dim: int, eps: float):
    """qkv_bits [N, (Hq + 2 Hkv) d] uint16: the fused projection rows (q heads, k heads, v
    heads). Returns (q_out, k_out, v) as uint16 bf16 bits, [N, H, d] each: normalised and
    rotated q and k, v unchanged."""
    qkv_bits = np.asarray(qkv_bits, dtype=np.uint16)
    n = qkv_bits.shape[0]
    d, hq, hkv = head_dim, num_heads, num_kv_heads
    q = bf16_to_f64(qkv_bits[:, :hq * d]).reshape(n, hq, d)
    k = bf16_to_f64(qkv_bits[:, hq * d:(hq + hkv) * d]).reshape(n, hkv, d)
    v = qkv_bits[:, (hq + hkv) * d:(hq + 2 * hkv) * d].reshape(n, hkv, d)
    qw = bf16_to_f64(q_weight_bits)
    kw = bf16_to_f64(k_weight_bits)
    q_out = rope(rms_norm(q, qw, eps), positions, table)
    k_out = rope(rms_norm(k, kw, eps), positions, table)
    return f64_to_bf16_bits(q_out), f64_to_bf16_bits(k_out), v.copy()
