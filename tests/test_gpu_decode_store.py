"""GPU parity of the one-launch store + decode (nv_paged_attn_decode_store).

It must equal nv_store_kvcache followed by nv_paged_attn_decode bit for bit (pools and
outputs), for split and unsplit launches, padding rows and several shapes and block sizes,
with split rows merged by the merge kernel or inside the launch (arrival counters, which
every call must leave zero); and, on its own, match the oracle's store (bit-exact pools) and
decode (attention bound).
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_store_amd import graphs, nvpaged, workloads
from paged_kv_cache_store_amd import step as gstep
from gpu_common import Run, assert_attn_close, check_pools_bit_exact
from helpers import bits

pytestmark = pytest.mark.gpu

CASES = [  # shape, decode rows, max context, padding rows
    (workloads.QWEN3_0_6B, 4, 600, 2),        # small batch: 128-key splits, merge kernel
    (workloads.QWEN3_8B, 9, 3000, 1),
    (workloads.AttnShape(12, 4, 128, 16), 7, 900, 2),
    (workloads.AttnShape(32, 4, 128, 48), 5, 700, 0),
    (workloads.AttnShape(24, 4, 128, 256), 6, 2000, 1),   # G = 6
    (workloads.AttnShape(12, 2, 128, 32), 11, 1200, 2),   # G = 6, block size 32
    (workloads.AttnShape(16, 8, 128, 256), 508, 1500, 4),  # 4096 pairs: unsplit, no merge
]


@pytest.mark.parametrize("merge", ["merge_kernel", "in_kernel"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0].num_heads}q{c[0].num_kv_heads}kv_bs{c[0].block_size}_B{c[1]}")
def test_fused_equals_store_then_decode(case, merge):
    shape, n, max_len, pad = case
    w = workloads.random_workload(60 + n, shape, 0, n, max_len=max_len, pad_rows=pad)
    print(f"[decode_store] {shape} rows={n}+{pad}", flush=True)
    run_a = Run(w)
    run_b = Run(w)
    scale = run_a.scale
    ds_a = gstep.prepare_step(shape, w.steps[0], run_a.tensors[0], "cuda")
    ds_b = gstep.prepare_step(shape, w.steps[0], run_b.tensors[0], "cuda")
    # reference composition
    gstep.run_store(ds_a, run_a.k_cache, run_a.v_cache)
    gstep.run_decode(ds_a, run_a.k_cache, run_a.v_cache, scale)
    # fused, into an output that starts as NaN
    t = ds_b.tensors
    out = torch.full_like(t.q_decode, float("nan"))
    cnt = (nvpaged.decode_counters(t.q_decode.shape[0], shape.num_kv_heads, "cuda")
           if merge == "in_kernel" else None)
    nvpaged.nv_paged_attn_decode_store(t.q_decode, t.key, t.value, ds_b.slot_mapping,
                                       run_b.k_cache, run_b.v_cache, ds_b.context_lens,
                                       ds_b.decode_tables, shape.num_kv_heads, shape.block_size,
                                       scale, out=out, counters=cnt)
    torch.cuda.synchronize()
    if cnt is not None:
        assert int(cnt.abs().sum()) == 0, "arrival counters not returned to zero"
    assert np.array_equal(bits(run_a.k_cache), bits(run_b.k_cache))
    assert np.array_equal(bits(run_a.v_cache), bits(run_b.v_cache))
    assert np.array_equal(bits(ds_a.out_decode), bits(out)), "outputs differ"
    # and against the oracle
    run_b.oracle_store(0)
    check_pools_bit_exact(run_b, "fused store")
    ids, ref = run_b.oracle_decode(0)
    print(assert_attn_close(out[ids], ref, "fused decode"))


def test_in_kernel_merge_reuses_counters():
    """One zeroed counter array serves a run of calls of different batches and split counts
    (contexts up to 4000 keys in 128-key splits: up to 32 partials per row), each call
    bitwise equal to the same call with the merge kernel, the counters zero after each."""
    shape = workloads.QWEN3_0_6B
    cnt = nvpaged.decode_counters(64, shape.num_kv_heads, "cuda")
    for i, (n, max_len) in enumerate([(2, 4000), (7, 3000), (1, 4000), (40, 2500), (3, 600),
                                      (2, 4000)] * 2):
        w = workloads.random_workload(300 + i, shape, 0, n, max_len=max_len, pad_rows=1)
        print(f"[decode_store counters] call {i} rows={n}+1 max_len={max_len}", flush=True)
        outs = []
        for c in (None, cnt):
            run = Run(w)
            ds = gstep.prepare_step(shape, w.steps[0], run.tensors[0], "cuda")
            t = ds.tensors
            o = nvpaged.nv_paged_attn_decode_store(t.q_decode, t.key, t.value, ds.slot_mapping,
                                                   run.k_cache, run.v_cache, ds.context_lens,
                                                   ds.decode_tables, shape.num_kv_heads,
                                                   shape.block_size, run.scale, counters=c)
            torch.cuda.synchronize()
            outs.append(bits(o).copy())
        assert np.array_equal(outs[0], outs[1]), f"call {i}: in-kernel merge differs"
        assert int(cnt.abs().sum()) == 0, f"call {i}: counters not returned to zero"


def test_in_kernel_merge_stress():
    """300 one-launch calls on one workload with up to 32 partials per row, each on a random
    prefix of its rows, sharing one counter array: every output equals the merge-kernel
    result of the same call bit for bit (the split length depends on the batch, so the
    reference is taken per call), and the counters end at zero."""
    shape = workloads.QWEN3_8B
    w = workloads.random_workload(777, shape, 0, 24, max_len=4000, pad_rows=2)
    run = Run(w)
    ds = gstep.prepare_step(shape, w.steps[0], run.tensors[0], "cuda")
    t = ds.tensors
    n_all = t.q_decode.shape[0]
    args = lambda n: (t.q_decode[:n], t.key[:n], t.value[:n], ds.slot_mapping[:n], run.k_cache,
                      run.v_cache, ds.context_lens[:n], ds.decode_tables[:n], shape.num_kv_heads,
                      shape.block_size, run.scale)
    cnt = nvpaged.decode_counters(n_all, shape.num_kv_heads, "cuda")
    rng = np.random.default_rng(5)
    print(f"[decode_store stress] rows {n_all}, 300 calls", flush=True)
    for i in range(300):
        n = int(rng.integers(1, n_all + 1))
        ref = nvpaged.nv_paged_attn_decode_store(*args(n))  # merge kernel
        o = nvpaged.nv_paged_attn_decode_store(*args(n), counters=cnt)
        assert np.array_equal(bits(o), bits(ref)), f"call {i} (rows {n}) differs"
    torch.cuda.synchronize()
    assert int(cnt.abs().sum()) == 0


def test_fused_full_size_decode_large():
    """The 0.6B decode of 256 sequences (contexts U[512, 4096], a 4608-block pool) at full size:
    the one-launch call with arrival counters (two splits per long row, merged in the launch;
    a large grid, so pairs are numbered sequence fastest) leaves the pools and the output equal,
    bit for bit, to store then decode on a copy of the same pools."""
    w = workloads.config_decode_large()
    dev = torch.device("cuda")
    kc, vc, tens = workloads.materialize(w, dev)
    kc2, vc2 = kc.clone(), vc.clone()
    scale = w.shape.head_dim ** -0.5
    ds = gstep.prepare_step(w.shape, w.steps[0], tens[0], dev)
    print(f"[decode_store full size] {w.name}", flush=True)
    gstep.run_store(ds, kc, vc)
    gstep.run_decode(ds, kc, vc, scale)
    ref = ds.out_decode.clone()
    ds.out_decode.fill_(float("nan"))
    gstep.run_decode_store(ds, kc2, vc2, scale)
    torch.cuda.synchronize()
    assert torch.equal(ds.out_decode.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
    assert int(ds.counters.abs().sum()) == 0


def test_fused_unaligned_rows_fall_back():
    """A value view whose rows are not 16-byte aligned takes the two-call path, same result."""
    shape = workloads.AttnShape(8, 2, 128, 64)
    w = workloads.random_workload(71, shape, 0, 5, max_len=300, pad_rows=1)
    run_a, run_b = Run(w), Run(w)
    ds_a = gstep.prepare_step(shape, w.steps[0], run_a.tensors[0], "cuda")
    ds_b = gstep.prepare_step(shape, w.steps[0], run_b.tensors[0], "cuda")
    gstep.run_store(ds_a, run_a.k_cache, run_a.v_cache)
    gstep.run_decode(ds_a, run_a.k_cache, run_a.v_cache, run_a.scale)
    t = ds_b.tensors
    # copy the value rows into a buffer offset by one element: row pointers lose 16-B alignment
    n = t.value.shape[0]
    raw = torch.empty(n * 264 + 8, dtype=torch.bfloat16, device="cuda")
    val = raw[1:1 + n * 264].view(n, 264)[:, :256].view(n, 2, 128)
    val.copy_(t.value)
    assert val.data_ptr() % 16 != 0
    out = nvpaged.nv_paged_attn_decode_store(t.q_decode, t.key, val, ds_b.slot_mapping,
                                             run_b.k_cache, run_b.v_cache, ds_b.context_lens,
                                             ds_b.decode_tables, 2, 64, run_b.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(run_a.v_cache), bits(run_b.v_cache))
    assert np.array_equal(bits(ds_a.out_decode), bits(out))


def test_fused_graph_replay_matches_two_call_graph():
    """Decode graphs recorded with the fused call replay to the same outputs and pools as the
    two-call graphs, over several steps of a small batch."""
    shape = workloads.QWEN3_0_6B
    w = workloads.config_decode_small()
    res = []
    for fused, in_kernel in ((False, False), (True, False), (True, True)):
        run = Run(w)
        ds = gstep.prepare_step(shape, w.steps[0], run.tensors[0], "cuda")
        dg = graphs.DecodeGraphs(shape, run.k_cache, run.v_cache, max_bs=8,
                                 max_blocks=ds.decode_tables.shape[1], scale=run.scale,
                                 fused=fused, merge_in_kernel=in_kernel)
        t = ds.tensors
        outs = []
        for _ in range(3):
            o = dg.run(t.q_decode, t.key, t.value, ds.slot_mapping, ds.context_lens,
                       ds.decode_tables)
            torch.cuda.synchronize()
            outs.append(bits(o).copy())
        if dg.counters is not None:
            assert int(dg.counters.abs().sum()) == 0
        res.append((outs, bits(run.k_cache).copy(), bits(run.v_cache).copy()))
    o0, k0, v0 = res[0]
    for o1, k1, v1 in res[1:]:
        for a, b in zip(o0, o1):
            assert np.array_equal(a, b)
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
