"""Pins of the QK-norm + rotary-embedding oracle (oracle/rope.py) against closed forms,
invariants and a library routine. No GPU.

Each pin is chosen so that a plausible slip fails at least one test: rotating interleaved
pairs (2i, 2i+1) instead of the two halves, the opposite rotation sign, a dropped eps, the
mean taken over the wrong axis, rounding to bf16 by truncation instead of to nearest even.
"""
import math

import numpy as np
import pytest
import torch

from oracle import rope as R

D = 128
BASE = 1e6


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_round_bf16_matches_torch_and_ties_to_even():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4096, generator=g) * torch.exp(torch.randn(4096, generator=g) * 4)
    ours = R.round_bf16(x.double().numpy())
    ref = x.bfloat16().double().numpy()
    np.testing.assert_array_equal(ours, ref)
    # exact halfway cases: 1 + 2^-8 lies between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3 * 2^-8 lies between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6); in [2, 4) the
    # spacing is 2^-6: 3 + 2^-7 -> 3 (even), 3 + 3 * 2^-7 -> 3 + 2^-5 (even)
    halfway = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3 + 2 ** -7,
                        3 + 3 * 2 ** -7])
    np.testing.assert_array_equal(R.round_bf16(halfway),
                                  [1.0, 1 + 2 ** -6, -1.0, 3.0, 3 + 2 ** -5])
    np.testing.assert_array_equal(R.round_bf16(halfway),
                                  torch.from_numpy(halfway).float().bfloat16().double().numpy())


def test_rope_unit_vectors_closed_form():
    """e_i (first half) at position p turns into cos(p theta_i) e_i + sin(p theta_i) e_{i+d/2};
    e_{i+d/2} into -sin e_i + cos e_{i+d/2}, theta_i = base^(-2i/d)."""
    h = D // 2
    table = R.rope_table_f64(64, D, BASE)
    for p in (1, 7, 63):
        for i in (0, 1, 17, h - 1):
            th = math.pow(BASE, -2.0 * i / D)
            c, s = math.cos(p * th), math.sin(p * th)
            x = np.zeros((1, 1, D))
            x[0, 0, i] = 1.0
            z = R.rope(x, [p], table, rounded=False)[0, 0]
            expect = np.zeros(D)
            expect[i], expect[i + h] = c, s
            np.testing.assert_allclose(z, expect, atol=1e-15)
            x = np.zeros((1, 1, D))
            x[0, 0, i + h] = 1.0
            z = R.rope(x, [p], table, rounded=False)[0, 0]
            expect = np.zeros(D)
            expect[i], expect[i + h] = -s, c
            np.testing.assert_allclose(z, expect, atol=1e-15)


def test_rope_table_entries():
    t = R.rope_table_f64(5000, D, BASE)
    assert t.shape == (5000, D)
    np.testing.assert_allclose(t[1, 0], math.cos(1.0), rtol=0, atol=1e-16)
    np.testing.assert_allclose(t[1, D // 2], math.sin(1.0), rtol=0, atol=1e-16)
    th = BASE ** (-(D - 2) / D)
    np.testing.assert_allclose(t[4321, D // 2 - 1], math.cos(4321 * th), atol=1e-14)
    np.testing.assert_allclose(t[4321, D - 1], math.sin(4321 * th), atol=1e-14)
    np.testing.assert_array_equal(t[0, :D // 2], 1.0)
    np.testing.assert_array_equal(t[0, D // 2:], 0.0)


def test_rope_position_zero_is_identity_and_rotation_invariants():
    rng = np.random.default_rng(4)
    table = R.rope_table_f64(4096, D, BASE)
    x = R.round_bf16(rng.standard_normal((6, 3, D)))
    np.testing.assert_array_equal(R.rope(x, np.zeros(6, np.int64), table), x)
    pos = rng.integers(0, 4000, size=6)
    z = R.rope(x, pos, table, rounded=False)
    h = D // 2
    np.testing.assert_allclose(z[..., :h] ** 2 + z[..., h:] ** 2,
                               x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-12)
    # q . k after rotation depends only on the position difference
    q, k = x[:1, :1], x[1:2, :1]
    for m, n, t in ((5, 3, 90), (1000, 17, 6), (0, 2000, 1500)):
        a = np.sum(R.rope(q, [m], table, False) * R.rope(k, [n], table, False))
        b = np.sum(R.rope(q, [m + t], table, False) * R.rope(k, [n + t], table, False))
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_rms_norm_closed_forms():
    w = np.ones(D)
    # constant vector c: c / sqrt(c^2 + eps); with c = 1e-3, eps = 1e-6 this is 1/sqrt(2)
    x = np.full((1, D), 1e-3)
    np.testing.assert_allclose(R.rms_norm(x, w, 1e-6, rounded=False), 1 / math.sqrt(2),
                               rtol=1e-12)
    np.testing.assert_array_equal(R.rms_norm(x, w, 1e-6), R.round_bf16(np.full((1, D),
                                                                               1 / math.sqrt(2))))
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 7, D))
    y = R.rms_norm(x, w, 0.0, rounded=False)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(R.rms_norm(3.5 * x, w, 0.0, rounded=False), y, rtol=1e-12)
    # the weight multiplies per dimension
    wv = rng.standard_normal(D)
    np.testing.assert_allclose(R.rms_norm(x, wv, 0.0, rounded=False), y * wv, rtol=1e-12)


def test_qk_norm_rope_splits_heads_and_leaves_v():
    g = torch.Generator().manual_seed(6)
    hq, hkv, n = 4, 2, 5
    qkv = torch.randn(n, (hq + 2 * hkv) * D, generator=g).bfloat16()
    wq = (1 + 0.1 * torch.randn(D, generator=g)).bfloat16()
    wk = (1 + 0.1 * torch.randn(D, generator=g)).bfloat16()
    pos = np.array([0, 1, 2, 300, 4000])
    table = R.rope_table_f64(4096, D, BASE)
    qo, ko, vo = R.qk_norm_rope(_bits(qkv), pos, _bits(wq), _bits(wk), table, hq, hkv, D, 1e-6)
    raw = _bits(qkv)
    np.testing.assert_array_equal(vo.reshape(n, -1), raw[:, (hq + hkv) * D:])
    # head 1 of token 3 by hand from the two formulas
    x = R.bf16_to_f64(raw[3, D:2 * D])
    nrm = R.round_bf16(x / np.sqrt(np.mean(x * x) + 1e-6))
    y = R.round_bf16(nrm * R.bf16_to_f64(_bits(wq)))
    h = D // 2
    c, s = table[300, :h], table[300, h:]
    z = R.round_bf16(np.concatenate([y[:h] * c - y[h:] * s, y[h:] * c + y[:h] * s]))
    np.testing.assert_array_equal(R.bf16_to_f64(qo[3, 1]), z)
    # k heads use the k weight: token 4, kv head 0
    x = R.bf16_to_f64(raw[4, hq * D:(hq + 1) * D])
    nrm = R.round_bf16(x / np.sqrt(np.mean(x * x) + 1e-6))
    y = R.round_bf16(nrm * R.bf16_to_f64(_bits(wk)))
    c, s = table[4000, :h], table[4000, h:]
    z = R.round_bf16(np.concatenate([y[:h] * c - y[h:] * s, y[h:] * c + y[:h] * s]))
    np.testing.assert_array_equal(R.bf16_to_f64(ko[4, 0]), z)


def test_pins_catch_planted_mistakes(monkeypatch):
    """Variants of the oracle with a planted slip fail the closed-form pins above."""
    def rope_interleaved(x, positions, table, rounded=True):
        h = x.shape[-1] // 2
        cs = table[np.asarray(positions)]
        c, s = cs[:, None, :h], cs[:, None, h:]
        x1, x2 = x[..., 0::2], x[..., 1::2]
        z = np.empty_like(x)
        z[..., 0::2], z[..., 1::2] = x1 * c - x2 * s, x2 * c + x1 * s
        return R.round_bf16(z) if rounded else z

    def rope_sign(x, positions, table, rounded=True):
        h = x.shape[-1] // 2
        cs = table[np.asarray(positions)]
        c, s = cs[:, None, :h], cs[:, None, h:]
        x1, x2 = x[..., :h], x[..., h:]
        z = np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)
        return R.round_bf16(z) if rounded else z

    def norm_no_eps(x, w, eps, rounded=True):
        y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * w
        return R.round_bf16(y) if rounded else y

    def truncating_round(x):
        x = np.asarray(x, np.float64)
        m, e = np.frexp(x)
        return np.ldexp(np.trunc(m * 256) / 256, e)

    for name, fn, test in (("rope", rope_interleaved, test_rope_unit_vectors_closed_form),
                           ("rope", rope_sign, test_rope_unit_vectors_closed_form),
                           ("rms_norm", norm_no_eps, test_rms_norm_closed_forms),
                           ("round_bf16", truncating_round,
                            test_round_bf16_matches_torch_and_ties_to_even)):
        with monkeypatch.context() as mp:
            mp.setattr(R, name, fn)
            with pytest.raises(AssertionError):
                test()
