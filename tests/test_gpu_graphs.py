"""Decode steps replayed from HIP graphs (one graph per batch bucket) against eager launches of
the same padded inputs (bitwise), against the oracle (attention bound) and against the host
copy of the pool (bit-exact store; padding rows store nothing and output zeros). Replays are
interleaved with unrelated eager work and synchronisations, and every replay is checked."""
import numpy as np
import pytest
import torch

import oracle
from oracle import meta
from paged_kv_cache_store_amd import graphs, nvpaged, workloads
from gpu_common import assert_attn_close
from helpers import bits

pytestmark = pytest.mark.gpu


def _decode_batch(rng, pool, bs, max_ctx, block_size):
    seqs = []
    for _ in range(bs):
        L = int(rng.integers(1, max_ctx + 1))
        seqs.append(workloads.Seq(pool.take(-(-L // block_size)), L - 1, 1))
    return seqs


@pytest.mark.parametrize("fused", [False, True], ids=["two_call", "fused"])
@pytest.mark.parametrize("shape", [workloads.QWEN3_0_6B, workloads.QWEN3_8B],
                         ids=lambda s: f"{s.num_heads}q{s.num_kv_heads}kv")
def test_graph_replay_matches_eager_and_oracle(shape, fused):
    """fused: one store+decode launch per layer, split rows merged in the same launch through
    arrival counters shared by every bucket (contexts up to 700 split into 128-key pieces)."""
    dev = torch.device("cuda")
    bsz = shape.block_size
    max_bs, max_ctx = 48, 700
    max_blocks = -(-max_ctx // bsz)
    batches = [3, 1, 17, 48, 5, 33, 2]
    rng = np.random.default_rng(11)
    num_blocks = sum(batches) * max_blocks + 8
    pool = workloads._Pool(num_blocks, rng)
    gen = torch.Generator(device="cpu").manual_seed(12)
    D = shape.num_kv_heads * shape.head_dim
    k_cache = torch.randn(num_blocks * bsz, D, generator=gen).bfloat16().to(dev)
    v_cache = torch.randn(num_blocks * bsz, D, generator=gen).bfloat16().to(dev)
    k_host, v_host = bits(k_cache).copy(), bits(v_cache).copy()
    scale = shape.head_dim ** -0.5
    print(f"[graphs] {shape}: capturing buckets {graphs.buckets(max_bs)}", flush=True)
    dg = graphs.DecodeGraphs(shape, k_cache, v_cache, max_bs, max_blocks, scale, fused=fused)
    scratch = torch.randn(512, 512, device=dev)
    for step, bs in enumerate(batches):
        seqs = _decode_batch(rng, pool, bs, max_ctx, bsz)
        m = nvpaged.nv_prepare_decode(seqs, bsz)
        q = torch.randn(bs, shape.num_heads, shape.head_dim, generator=gen).bfloat16()
        kv = torch.randn(bs, 2, shape.num_kv_heads, shape.head_dim, generator=gen).bfloat16()
        args = (q.to(dev), kv[:, 0].contiguous().to(dev), kv[:, 1].contiguous().to(dev),
                torch.from_numpy(m["slot_mapping"]).to(dev),
                torch.from_numpy(m["context_lens"]).to(dev),
                torch.from_numpy(m["block_tables"]).to(dev))
        print(f"[graphs] step {step}: batch {bs} -> bucket {dg.bucket_for(bs)}", flush=True)
        out_g = dg.run(*args).clone()
        pad = dg.out[0, bs:dg.bucket_for(bs)].clone()
        scratch = scratch @ scratch.T / 512.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        out_e = dg.run_eager(*args).clone()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"step {step}"
        assert torch.count_nonzero(pad).item() == 0, "padding rows must output zeros"
        # The plain decode (merge kernel) over the pool the replay stored into: same bits.
        out_p = nvpaged.nv_paged_attn_decode(args[0], k_cache, v_cache, args[4], args[5],
                                             shape.num_kv_heads, bsz, scale)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_p.view(torch.int16)), f"step {step}"
        if dg.counters is not None:
            assert int(dg.counters.abs().sum()) == 0, "arrival counters must return to zero"
        # Oracle: its own metadata, its own store into the host pool, fp64 attention.
        om = meta.prepare_decode(seqs, bsz)
        oracle.store_kvcache(bits(kv[:, 0]).reshape(bs, D), bits(kv[:, 1]).reshape(bs, D),
                             k_host, v_host, om["slot_mapping"])
        rows = torch.from_numpy(om["slot_mapping"].astype(np.int64)).to(dev)
        assert np.array_equal(bits(k_cache[rows]), k_host[om["slot_mapping"]])
        assert np.array_equal(bits(v_cache[rows]), v_host[om["slot_mapping"]])
        ref = oracle.attn_decode(bits(q), k_host, v_host, om["context_lens"], om["block_tables"],
                                 shape.num_heads, shape.num_kv_heads, shape.head_dim, bsz, scale)
        print(assert_attn_close(out_g, ref, f"graph step {step}"))
    # Nothing else in either pool changed (padding rows stored nothing).
    assert np.array_equal(bits(k_cache), k_host) and np.array_equal(bits(v_cache), v_host)


@pytest.mark.parametrize("fused", [False, True], ids=["two_call", "fused"])
def test_graph_over_layer_stack(fused):
    """Three layers, each with its own pool, in one graph: every layer stores the step's rows
    into its own pool and attends over it; replay equals eager bitwise, each layer's output
    equals a single-layer eager call on that layer's pool."""
    dev = torch.device("cuda")
    shape = workloads.QWEN3_0_6B
    bsz, max_blocks, L = shape.block_size, 3, 3
    rng = np.random.default_rng(21)
    pool = workloads._Pool(40, rng)
    gen = torch.Generator(device="cpu").manual_seed(22)
    D = shape.num_kv_heads * shape.head_dim
    ks = [torch.randn(40 * bsz, D, generator=gen).bfloat16().to(dev) for _ in range(L)]
    vs = [torch.randn(40 * bsz, D, generator=gen).bfloat16().to(dev) for _ in range(L)]
    dg = graphs.DecodeGraphs(shape, ks, vs, max_bs=16, max_blocks=max_blocks, fused=fused)
    seqs = _decode_batch(rng, pool, 6, 700, bsz)
    m = nvpaged.nv_prepare_decode(seqs, bsz)
    q = torch.randn(6, shape.num_heads, shape.head_dim, generator=gen).bfloat16().to(dev)
    kv = torch.randn(6, 2, shape.num_kv_heads, shape.head_dim, generator=gen).bfloat16().to(dev)
    args = (q, kv[:, 0].contiguous(), kv[:, 1].contiguous(),
            torch.from_numpy(m["slot_mapping"]).to(dev), torch.from_numpy(m["context_lens"]).to(dev),
            torch.from_numpy(m["block_tables"]).to(dev))
    for rep in range(3):
        out_g = dg.run(*args).clone()
        torch.cuda.synchronize()
        out_e = dg.run_eager(*args).clone()
        torch.cuda.synchronize()
        assert out_g.shape == (L, 6, shape.num_heads, shape.head_dim)
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}"
    for layer in range(L):
        one = nvpaged.nv_paged_attn_decode(q, ks[layer], vs[layer], args[4], args[5],
                                           shape.num_kv_heads, bsz, shape.head_dim ** -0.5)
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16), out_g[layer].view(torch.int16))
