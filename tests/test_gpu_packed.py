"""GPU parity of packed fresh-K/V prefill (no block table) against the oracle.

K/V are read straight from packed [total_k, Hkv, d] tensors (V as a strided view into a fused
QKV buffer, as the engine hands it over). Bounds as for the paged tests: max abs error <= 1e-2
plus half a bf16 ulp of the result, mean abs error <= 1e-3. The packed and paged paths
perform the same arithmetic, so on the same keys their outputs must be bitwise equal.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_store_amd import nvpaged, workloads
from gpu_common import assert_attn_close
from helpers import bits

pytestmark = pytest.mark.gpu


def _make(shape, lq, extra, seed):
    """Packed inputs: q contiguous, k contiguous, v a view with the fused-QKV row stride."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    lq = np.asarray(lq)
    lk = lq + np.asarray(extra)
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    hq, hkv, d = shape.num_heads, shape.num_kv_heads, shape.head_dim
    q = torch.randn(int(cq[-1]), hq, d, generator=g).bfloat16()
    fused = torch.randn(int(ck[-1]), (hq + 2 * hkv) * d, generator=g).bfloat16()
    k = fused[:, hq * d:(hq + hkv) * d].contiguous().view(-1, hkv, d)
    v = fused[:, (hq + hkv) * d:].view(-1, hkv, d)  # strided view
    return q, k, v, fused, cq, ck


def _gpu_packed(q, k, v, fused, cq, ck, scale):
    dev = torch.device("cuda")
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    fused_d = fused.to(dev)
    v_d = fused_d[:, (hq + hkv) * d:].view(-1, hkv, d)
    out = nvpaged.nv_attn_prefill_packed(
        q.to(dev), k.to(dev), v_d, torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev),
        int((cq[1:] - cq[:-1]).max()), int((ck[1:] - ck[:-1]).max()), scale)
    torch.cuda.synchronize()
    return out


def _oracle(q, k, v, cq, ck, shape, scale, rows=None):
    D = shape.num_kv_heads * shape.head_dim
    qb = bits(q)
    kb = bits(k.reshape(-1, D))
    vb = bits(v.reshape(-1, D).contiguous())
    out = oracle.attn_prefill_packed(qb, kb, vb, cq, ck, shape.num_heads, shape.num_kv_heads,
                                     shape.head_dim, scale)
    return out if rows is None else out[rows]


SHAPES = [workloads.AttnShape(16, 8, 128, 1), workloads.AttnShape(32, 8, 128, 1),
          workloads.AttnShape(12, 4, 128, 1), workloads.AttnShape(8, 8, 128, 1),
          workloads.AttnShape(16, 2, 128, 1), workloads.AttnShape(10, 2, 128, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s.num_heads}q{s.num_kv_heads}kv")
def test_packed_ragged_lengths(shape):
    """Fresh prompts (cu_seqlens_k == cu_seqlens_q) with lengths around tile edges, plus two
    sequences with extra leading keys."""
    lq = [1, 63, 64, 65, 127, 129, 300, 40]
    extra = [0, 0, 0, 0, 0, 0, 7, 90]
    q, k, v, fused, cq, ck = _make(shape, lq, extra, seed=shape.num_heads * 7 + shape.num_kv_heads)
    scale = shape.head_dim ** -0.5
    print(f"[packed] {shape} lq={lq} extra={extra}", flush=True)
    out = _gpu_packed(q, k, v, fused, cq, ck, scale)
    ref = _oracle(q, k, v, cq, ck, shape, scale)
    print(assert_attn_close(out, ref, f"packed {shape}"))


@pytest.mark.parametrize("shape", SHAPES[:3], ids=lambda s: f"{s.num_heads}q{s.num_kv_heads}kv")
def test_packed_long_context(shape):
    """Keys at least twice the new rows: the launch takes the 8-wave workgroups."""
    lq, extra = [100, 37, 64], [900, 400, 128]
    q, k, v, fused, cq, ck = _make(shape, lq, extra, seed=5 + shape.num_heads)
    scale = shape.head_dim ** -0.5
    print(f"[packed long] {shape}", flush=True)
    out = _gpu_packed(q, k, v, fused, cq, ck, scale)
    ref = _oracle(q, k, v, cq, ck, shape, scale)
    print(assert_attn_close(out, ref, f"packed long {shape}"))


@pytest.mark.parametrize("bs", [256, 16, 48])
def test_packed_equals_paged_bitwise(bs):
    """The same keys stored in a permuted pool and read through block tables give the same bits,
    and nv_paged_attn_prefill with no block table is the packed call."""
    shape = workloads.QWEN3_0_6B
    lq, extra = [700, 65, 300, 1], [0, 0, 200, 0]
    q, k, v, fused, cq, ck = _make(shape, lq, extra, seed=bs)
    scale = shape.head_dim ** -0.5
    print(f"[packed vs paged] bs={bs}", flush=True)
    dev = torch.device("cuda")
    out_packed = _gpu_packed(q, k, v, fused, cq, ck, scale)
    lk = ck[1:] - ck[:-1]
    nblk = [-(-int(n) // bs) for n in lk]
    rng = np.random.default_rng(bs)
    perm = rng.permutation(sum(nblk) + 5).astype(np.int32)
    D = shape.num_kv_heads * shape.head_dim
    kc = torch.zeros(len(perm) * bs, D, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    table = np.full((len(lk), max(nblk)), -1, np.int32)
    nxt = 0
    kf, vf = k.reshape(-1, D), v.reshape(-1, D)
    for b in range(len(lk)):
        table[b, :nblk[b]] = perm[nxt:nxt + nblk[b]]
        nxt += nblk[b]
        j = np.arange(lk[b])
        slots = torch.from_numpy(table[b, j // bs].astype(np.int64) * bs + j % bs)
        kc[slots] = kf[ck[b]:ck[b + 1]]
        vc[slots] = vf[ck[b]:ck[b + 1]]
    cq_d, ck_d = torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev)
    out_paged = nvpaged.nv_paged_attn_prefill(
        q.to(dev), kc.to(dev), vc.to(dev), cq_d, ck_d, int(max(lq)), int(lk.max()),
        torch.from_numpy(table).to(dev), shape.num_kv_heads, bs, scale)
    out_null = nvpaged.nv_paged_attn_prefill(
        q.to(dev), kf.to(dev), vf.contiguous().to(dev), cq_d, ck_d, int(max(lq)), int(lk.max()),
        None, shape.num_kv_heads, bs, scale)
    torch.cuda.synchronize()
    assert torch.equal(out_packed.view(torch.int16), out_paged.view(torch.int16))
    assert torch.equal(out_packed.view(torch.int16), out_null.view(torch.int16))


@pytest.mark.parametrize("which", ["prefill_varlen", "mixed_8b"])
def test_packed_full_size_fresh_prompts(which):
    """The fresh prompts of the varlen and mixed workloads (their lengths and shapes) in packed
    mode; every output finite, sampled sequences against the oracle."""
    w = workloads.CONFIGS[which]()
    st = next(s for s in w.steps if s.prefill)
    lq = [s.num_new for s in st.prefill]
    extra = [s.num_cached for s in st.prefill]
    q, k, v, fused, cq, ck = _make(w.shape, lq, extra, seed=w.seed)
    scale = w.shape.head_dim ** -0.5
    print(f"[packed full] {which} lq={lq}", flush=True)
    out = _gpu_packed(q, k, v, fused, cq, ck, scale)
    assert torch.isfinite(out.float()).all()
    pick = [0, len(lq) - 1] if which == "mixed_8b" else list(range(len(lq)))
    rows = np.concatenate([np.arange(cq[b], cq[b + 1]) for b in pick])
    sub_q = q[torch.from_numpy(rows)]
    sub_cq = np.concatenate([[0], np.cumsum([lq[b] for b in pick])]).astype(np.int32)
    kparts = [k[ck[b]:ck[b + 1]] for b in pick]
    vparts = [v[ck[b]:ck[b + 1]] for b in pick]
    sub_ck = np.concatenate([[0], np.cumsum([len(x) for x in kparts])]).astype(np.int32)
    ref = _oracle(sub_q, torch.cat(kparts), torch.cat(vparts), sub_cq, sub_ck, w.shape, scale)
    print(assert_attn_close(out[torch.from_numpy(rows).cuda()], ref, f"packed {which}"))


def test_step_packed_path_matches_paged_path():
    """The step glue's packed prefill (the step's own fresh K/V rows, no table) gives the same
    bits as the store + paged prefill of the same step."""
    from paged_kv_cache_store_amd import step as gstep
    from gpu_common import Run
    w = workloads.random_workload(77, workloads.QWEN3_8B, n_prefill=5, n_decode=3, max_len=900,
                                  max_cached=0)
    run = Run(w)
    ds = run.gpu_step(0)
    assert not ds.host["prefill"]["has_cached_context"]
    paged = ds.out_prefill.clone()
    gstep.run_prefill_packed(ds, run.scale)
    torch.cuda.synchronize()
    assert torch.equal(paged.view(torch.int16), ds.out_prefill.view(torch.int16))
