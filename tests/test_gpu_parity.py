"""GPU parity: the HIP library against the oracle on the same seeded inputs.

Store and indexing: bit-exact over the whole pool (untouched rows included). Attention: max
abs error <= 1e-2 plus half a bf16 ulp of the result for the output's rounding
(gpu_common.attn_bound) and mean abs error <= 1e-3. Unowned blocks hold NaN, so a read outside a sequence's table fails loudly.
Every configuration, the full-size ones included, is compared on every output row.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_store_amd import workloads
from gpu_common import Run, assert_attn_close, check_metadata, check_pools_bit_exact

pytestmark = pytest.mark.gpu


def _full_check(w, label):
    run = Run(w)
    stats = {}
    for i, st in enumerate(w.steps):
        print(f"[{label}] step {i}: {len(st.prefill)} prefill seqs, {len(st.decode)} decode rows",
              flush=True)
        ds = run.gpu_step(i)
        om = run.oracle_store(i)
        check_metadata(ds, om)
        check_pools_bit_exact(run, f"{label} step {i}")
        if st.prefill:
            rows, ref = run.oracle_prefill(i, om)
            stats[f"prefill{i}"] = assert_attn_close(ds.out_prefill[rows], ref,
                                                     f"{label} prefill step {i}")
        if st.decode:
            ids, ref = run.oracle_decode(i)
            stats[f"decode{i}"] = assert_attn_close(ds.out_decode[ids], ref,
                                                    f"{label} decode step {i}")
    return stats


def test_config_decode_small():
    print(_full_check(workloads.config_decode_small(), "decode_small"))


def test_config_prefill_varlen():
    print(_full_check(workloads.config_prefill_varlen(), "prefill_varlen"))


SHAPES = [workloads.AttnShape(16, 8, 128, 256), workloads.AttnShape(32, 8, 128, 256),
          workloads.AttnShape(8, 8, 128, 64), workloads.AttnShape(12, 4, 128, 48),
          workloads.AttnShape(16, 2, 128, 16), workloads.AttnShape(8, 4, 128, 512),
          workloads.AttnShape(10, 2, 128, 128),
          # decode grid: kv heads of a (sequence, split) go to an XCD gcd(Hkv, G) at a time;
          # these split each pair's heads into 3 units of 2 (G = 4) and 3 units of 1 (G = 7)
          workloads.AttnShape(24, 6, 128, 32), workloads.AttnShape(21, 3, 128, 64),
          # six query heads per kv head: decode_split_kernel<6, *> and two-head prefill groups
          workloads.AttnShape(24, 4, 128, 256), workloads.AttnShape(12, 2, 128, 32),
          # one-key blocks: every key its own table entry (decode splits capped by the table
          # slice staged in LDS)
          workloads.AttnShape(16, 8, 128, 1)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s.num_heads}q{s.num_kv_heads}kv_bs{s.block_size}")
@pytest.mark.parametrize("seed", [0, 1])
def test_random_mixed(shape, seed):
    w = workloads.random_workload(100 + seed, shape, n_prefill=4, n_decode=9, max_len=700,
                                  max_cached=600, pad_rows=2, share_prefix=seed == 1)
    print(_full_check(w, f"random {shape} seed {seed}"))


def test_edge_lengths():
    """Lengths around tile and block edges: 1, 63, 64, 65, 255, 256, 257 new tokens and
    single-key decode rows."""
    shape = workloads.AttnShape(16, 8, 128, 256)
    lens = [1, 63, 64, 65, 255, 256, 257, 129]
    cached = [0, 1, 64, 191, 0, 256, 255, 1]
    rng = np.random.default_rng(9)
    need = sum(-(-(c + n) // 256) for c, n in zip(cached, lens)) + 4 + 2
    pool = workloads._Pool(need, rng)
    pre = [workloads.Seq(pool.take(-(-(c + n) // 256)), c, n) for c, n in zip(cached, lens)]
    dec = [workloads.Seq(pool.take(1), 0, 1), workloads.Seq(pool.take(1), 255, 1),
           workloads.Seq(pool.take(2), 256, 1), workloads.Seq([], 0, 0)]
    w = workloads.Workload("edges", shape, need, pool.owned,
                           [workloads.Step(prefill=pre, decode=dec)], 9)
    print(_full_check(w, "edges"))


def test_all_padding_decode_rows():
    shape = workloads.AttnShape(16, 8, 128, 256)
    w = workloads.Workload("pad", shape, 2, np.zeros(2, bool),
                           [workloads.Step(decode=[workloads.Seq([], 0, 0)] * 3)], 5)
    run = Run(w)
    ds = run.gpu_step(0)
    assert torch.count_nonzero(ds.out_decode).item() == 0
    om = run.oracle_store(0)
    check_pools_bit_exact(run, "padding rows store nothing")


def test_unsplit_decode_with_padding_rows():
    """A batch large enough that every row runs as one split (no merge kernel): the padding
    rows' zeros come from the split kernel, over an output buffer that starts as NaN."""
    from paged_kv_cache_store_amd import nvpaged, step as gstep
    shape = workloads.AttnShape(16, 8, 128, 256)
    w = workloads.random_workload(31, shape, 0, 506, max_len=1500, pad_rows=6)
    assert nvpaged.nv_paged_attn_decode_split_keys(512, 8, 6, 256) >= 1536
    run = Run(w)
    ds = gstep.prepare_step(shape, w.steps[0], run.tensors[0], "cuda")
    assert ds.decode_tables.shape[1] * 256 <= nvpaged.nv_paged_attn_decode_split_keys(
        512, 8, ds.decode_tables.shape[1], 256)
    ds.out_decode.fill_(float("nan"))
    print("[unsplit] 506 rows + 6 padding rows", flush=True)
    gstep.run_step(ds, run.k_cache, run.v_cache, run.scale)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ds.out_decode[506:]).item() == 0
    assert torch.isfinite(ds.out_decode.float()).all()
    run.oracle_store(0)
    ids, ref = run.oracle_decode(0, list(range(0, 506, 11)))
    print(assert_attn_close(ds.out_decode[ids], ref, "unsplit decode"))


@pytest.mark.parametrize("bs", [256, 16])
def test_long_contexts_many_splits(bs):
    """Few long decode rows: the split falls to the 128-key minimum (bs 256: ~160 splits per
    row, all merged by the combine kernel) or is capped by the LDS table slice (bs 16), next to
    a one-key row; plus a prefill chunk whose cached prefix fills ~2000 of the 2048 staged
    table entries (bs 16)."""
    from paged_kv_cache_store_amd import nvpaged
    shape = workloads.AttnShape(16, 8, 128, bs)
    rng = np.random.default_rng(77 + bs)
    lens = [1, 20000, 9000]
    pre = [(31960, 40)] if bs == 16 else [(4000, 70)]
    need = sum(-(-L // bs) for L in lens) + sum(-(-(c + n) // bs) for c, n in pre) + 2
    pool = workloads._Pool(need, rng)
    prefill = [workloads.Seq(pool.take(-(-(c + n) // bs)), c, n) for c, n in pre]
    decode = [workloads.Seq(pool.take(-(-L // bs)), L - 1, 1) for L in lens]
    w = workloads.Workload(f"long contexts bs{bs}", shape, need, pool.owned,
                           [workloads.Step(prefill=prefill, decode=decode)], 77)
    width = -(-max(lens) // bs)
    split = nvpaged.nv_paged_attn_decode_split_keys(len(lens), 8, width, bs)
    print(f"[long] bs={bs}: decode split {split} keys, {-(-max(lens) // split)} splits", flush=True)
    assert -(-max(lens) // split) >= 5
    print(_full_check(w, f"long contexts bs{bs}"))


def test_config_prefix_chunked():
    """Both 512-token chunk steps of all 16 prompts (4 prefix groups), every output row."""
    print(_full_check(workloads.config_prefix_chunked(), "prefix_chunked"))


def test_config_decode_large():
    """All 256 decode rows (contexts 512..4096, two key splits per row, merge kernel)."""
    print(_full_check(workloads.config_decode_large(), "decode_large"))


def test_config_mixed_8b():
    """All 4 prompts (4096 prefill rows) and all 512 decode rows of the 8B mixed step."""
    print(_full_check(workloads.config_mixed_8b(), "mixed_8b"))


@pytest.mark.parametrize("shape", [workloads.AttnShape(16, 8, 128, 256), workloads.AttnShape(12, 4, 128, 16),
                                   workloads.AttnShape(32, 8, 128, 64), workloads.AttnShape(8, 8, 128, 48)],
                         ids=lambda s: f"{s.num_heads}q{s.num_kv_heads}kv_bs{s.block_size}")
def test_long_prefix_short_chunks(shape):
    """Chunks much shorter than their cached prefix: the launch takes the 8-wave workgroups
    (max_seqlen_k >= 2 max_seqlen_q), including ragged q tails and odd group sizes."""
    w = workloads.random_workload(300 + shape.num_heads, shape, n_prefill=5, n_decode=0,
                                  max_len=150, max_cached=1500, share_prefix=True)
    st = w.steps[0]
    assert max(s.num_cached + s.num_new for s in st.prefill) >= 2 * max(s.num_new for s in st.prefill)
    print(_full_check(w, f"long prefix {shape}"))


@pytest.mark.parametrize("tp", [2, 4, 8])
@pytest.mark.parametrize("base", ["0.6b", "8b"])
def test_tp_rank_shapes(tp, base):
    """One rank's heads under tensor parallelism (q and kv heads divided by tp): store, prefill
    with cached prefixes and decode at those shapes, full check against the oracle."""
    shape = workloads.QWEN3_0_6B if base == "0.6b" else workloads.QWEN3_8B
    w = workloads.random_workload(400 + tp, shape, n_prefill=3, n_decode=6, max_len=500,
                                  max_cached=400, pad_rows=1, share_prefix=True)
    w = workloads.tp_share(w, tp)
    assert w.shape.num_heads == shape.num_heads // tp
    print(_full_check(w, f"{base} tp={tp}"))


def test_large_grid_order_is_longest_first_permutation():
    """A decode grid too large for one go orders its sequences longest first into the tail of
    the workspace: a permutation of the rows whose bucketed lengths never increase. The rows'
    outputs are still checked against the oracle (the order changes none of them)."""
    from paged_kv_cache_store_amd import nvpaged, step as gstep
    shape = workloads.AttnShape(16, 8, 128, 16)
    w = workloads.random_workload(47, shape, 0, 700, max_len=2000, pad_rows=12)
    run = Run(w)
    ds = gstep.prepare_step(shape, w.steps[0], run.tensors[0], "cuda")
    B, width = ds.decode_tables.shape
    need = nvpaged.nv_paged_attn_decode_workspace_size(B, 16, 8, 128, width, 16)
    S = nvpaged.nv_paged_attn_decode_split_keys(B, 8, width, 16)
    splits = -(-width * 16 // S)
    rows = B * 16 * splits
    part = 0 if splits == 1 else -(-rows * 8 // 256) * 256 + -(-rows * 512 // 256) * 256
    assert need == part + -(-B * 4 // 256) * 256
    ds.workspace.fill_(0xFF)
    print(f"[order] {B} rows, {splits} splits, table width {width}", flush=True)
    gstep.run_step(ds, run.k_cache, run.v_cache, run.scale)
    torch.cuda.synchronize()
    perm = ds.workspace[part:part + 4 * B].view(torch.int32).cpu().numpy()
    assert sorted(perm.tolist()) == list(range(B))
    lens = ds.context_lens.cpu().numpy().astype(np.int64)
    max_ctx = width * 16
    bucket = np.clip(lens, 0, max_ctx) * 1024 // (max_ctx + 1)
    assert (np.diff(bucket[perm]) <= 0).all()
    run.oracle_store(0)
    ids, ref = run.oracle_decode(0, list(range(0, 700, 9)))
    print(assert_attn_close(ds.out_decode[ids], ref, "ordered decode"))
