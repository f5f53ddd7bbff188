"""GPU parity of the fused per-head QK RMSNorm + rotary embedding + K/V store against the oracle
(oracle/rope.py, float64 between the pages' bf16 roundings).

Bound: the kernel computes in fp32, the oracle in float64, each rounding to bf16 at the same
points. They agree bit for bit except where an fp32 value falls on the other side of a bf16
rounding boundary: a flipped rounding of the normalised value or of its product with the
weight moves y by at most 2^-6 |y|, so a rotated output differs by at most
2^-6 (|y_i| + |y_(i+d/2)|) + one bf16 ulp of the output. Nearly all elements must match
exactly; V rows are bit copies; slots of -1 and every other pool row stay untouched.
"""
import numpy as np
import pytest
import torch

from oracle import rope as R
from paged_kv_cache_store_amd import nvpaged, workloads
from helpers import bits

pytestmark = pytest.mark.gpu

EPS = 1e-6
BASE = 1e6
MAX_POS = 4096
D = 128


def _ulp(x):
    mag = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(mag)) - 7)


def _check_rotated(gpu_bits, ref_bits, y, what):
    g = R.bf16_to_f64(gpu_bits)
    r = R.bf16_to_f64(ref_bits)
    h = D // 2
    pair = np.abs(y[..., :h]) + np.abs(y[..., h:])
    pair = np.concatenate([pair, pair], axis=-1)
    bound = 2.0 ** -6 * pair + _ulp(r)
    err = np.abs(g - r)
    assert np.isfinite(g).all(), f"{what}: non-finite"
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} over the bound, first at "
                           f"{tuple(np.argwhere(bad)[0])}")
    exact = float(np.mean(gpu_bits == ref_bits))
    assert exact >= 0.995, f"{what}: only {exact:.4f} bit-exact"
    return exact


def _run(shape, n, seed, pad_cols=64, frac_pad=0.1):
    dev = torch.device("cuda")
    g = torch.Generator(device="cpu").manual_seed(seed)
    rng = np.random.default_rng(seed)
    hq, hkv = shape.num_heads, shape.num_kv_heads
    width = (hq + 2 * hkv) * D
    base = torch.randn(n, width + pad_cols, generator=g).bfloat16()
    qkv_host = base[:, :width]                       # rows with a stride past their width
    wq = (1 + 0.1 * torch.randn(D, generator=g)).bfloat16()
    wk = (1 + 0.1 * torch.randn(D, generator=g)).bfloat16()
    pos = rng.integers(0, MAX_POS, size=n).astype(np.int64)
    pos[:3] = [0, 1, MAX_POS - 1]
    n_slots = 2 * n + 16
    slots = rng.permutation(n_slots)[:n].astype(np.int32)
    slots[rng.random(n) < frac_pad] = -1
    table = nvpaged.rope_cos_sin_cache(MAX_POS, D, BASE, dev)
    kc = torch.randn(n_slots, hkv * D, generator=g).bfloat16()
    vc = torch.randn(n_slots, hkv * D, generator=g).bfloat16()
    kc0, vc0 = bits(kc).copy(), bits(vc).copy()
    base_d = base.to(dev)
    kc_d, vc_d = kc.to(dev), vc.to(dev)
    print(f"[norm-rope] {shape} n={n} seed={seed}", flush=True)
    q_out, k_out = nvpaged.nv_qk_norm_rope_store(
        base_d[:, :width], torch.from_numpy(pos).to(dev), wq.to(dev), wk.to(dev), table, EPS,
        kc_d, vc_d, torch.from_numpy(slots).to(dev), hq, hkv, want_k=True)
    torch.cuda.synchronize()
    # Oracle, on the same inputs (the fp32 table's values as given).
    tab = table.double().cpu().numpy()
    raw = bits(qkv_host)
    qo, ko, vo = R.qk_norm_rope(raw, pos, bits(wq), bits(wk), tab, hq, hkv, D, EPS)
    yq = R.rms_norm(R.bf16_to_f64(raw[:, :hq * D]).reshape(n, hq, D), R.bf16_to_f64(bits(wq)), EPS)
    yk = R.rms_norm(R.bf16_to_f64(raw[:, hq * D:(hq + hkv) * D]).reshape(n, hkv, D),
                    R.bf16_to_f64(bits(wk)), EPS)
    eq = _check_rotated(bits(q_out), qo, yq, f"q {shape}")
    ek = _check_rotated(bits(k_out), ko, yk, f"k {shape}")
    # Pools: rows at the slots hold k_out / v exactly, all other rows unchanged.
    kc1, vc1 = bits(kc_d), bits(vc_d)
    live = slots >= 0
    np.testing.assert_array_equal(kc1[slots[live]], bits(k_out).reshape(n, -1)[live])
    np.testing.assert_array_equal(vc1[slots[live]], vo.reshape(n, -1)[live])
    other = np.ones(n_slots, bool)
    other[slots[live]] = False
    np.testing.assert_array_equal(kc1[other], kc0[other])
    np.testing.assert_array_equal(vc1[other], vc0[other])
    return dict(q_exact=eq, k_exact=ek)


SHAPES = [workloads.QWEN3_0_6B, workloads.QWEN3_8B, workloads.AttnShape(12, 4),
          workloads.AttnShape(8, 8), workloads.AttnShape(2, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s.num_heads}q{s.num_kv_heads}kv")
def test_norm_rope_store_random(shape):
    print(_run(shape, 333, seed=shape.num_heads + 10 * shape.num_kv_heads))


def test_norm_rope_store_full_mixed_step_rows():
    """The row count and shape of the Qwen3-8B mixed step (4096 prefill + 512 decode tokens)."""
    print(_run(workloads.QWEN3_8B, 4608, seed=1005, pad_cols=0, frac_pad=0.0))
