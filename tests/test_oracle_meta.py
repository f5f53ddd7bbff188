"""Pins of the oracle's index metadata against the worked examples the pages print.

Every expected value comes from tests/golden/worked_examples.json, which cites its page and
section. Nothing here needs a GPU.
"""
import json
import os
from types import SimpleNamespace as NS

import numpy as np
import pytest

from oracle import meta
from paged_kv_cache_store_amd import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def test_slot_toy():
    g = GOLD["slot_toy"]
    bt, p, bs = g["block_table"], g["position"], g["block_size"]
    assert bt[p // bs] == g["block"]
    assert meta.slot_of(bt, p, bs) == g["slot"]


def test_decode_counters():
    g = GOLD["decode_counters"]
    n = g["num_tokens"]
    d = meta.prepare_decode([NS(block_table=g["block_table"], num_cached=n - 1, num_new=1)],
                            g["block_size"])
    assert d["positions"].tolist() == g["positions"]
    assert d["context_lens"].tolist() == g["context_lens"]
    assert d["slot_mapping"].tolist() == g["slot_mapping"]
    # The runner's own form of the same slot: last block's base plus the fill of the last
    # block minus one ("Nano-vLLM Field Guide", Step 07.6).
    bs = g["block_size"]
    last_fill = n - (len(g["block_table"]) - 1) * bs
    assert g["block_table"][-1] * bs + last_fill - 1 == g["slot_mapping"][0]


def test_prefill_packing_figure():
    g = GOLD["prefill_packing"]
    seqs = [NS(**{k: v for k, v in s.items() if k != "name"}) for s in g["seqs"]]
    d = meta.prepare_prefill(seqs, g["block_size"])
    assert d["positions"].tolist() == g["positions"]
    assert d["slot_mapping"].tolist() == g["slot_mapping"]
    assert d["cu_seqlens_q"].tolist() == g["cu_seqlens_q"]
    assert d["cu_seqlens_k"].tolist() == g["cu_seqlens_k"]
    assert d["max_seqlen_q"] == g["max_seqlen_q"]
    assert d["max_seqlen_k"] == g["max_seqlen_k"]
    assert (d["cu_seqlens_q"][1:] - 1).tolist() == g["last_rows"]
    assert d["has_cached_context"] == g["block_tables_passed"]
    assert d["block_tables"].tolist() == [[2, 5, 8], [0, 6, -1], [3, 4, -1]]


def test_prefill_two_prompts():
    g = GOLD["prefill_two_prompts"]
    bs = g["block_size"]
    blocks = [-(-L // bs) for L in g["prompt_lens"]]
    assert blocks == g["blocks_per_prompt"]
    tables, nxt = [], 0
    for nb in blocks:
        tables.append(list(range(nxt, nxt + nb)))
        nxt += nb
    seqs = [NS(block_table=t, num_cached=0, num_new=L) for t, L in zip(tables, g["prompt_lens"])]
    d = meta.prepare_prefill(seqs, bs)
    assert d["cu_seqlens_q"].tolist() == g["cu_seqlens_q"]
    assert d["cu_seqlens_k"].tolist() == g["cu_seqlens_k"]
    assert d["max_seqlen_q"] == g["max_seqlen_q"]
    assert len(d["slot_mapping"]) == g["num_slots"]
    assert (d["cu_seqlens_q"][1:] - 1).tolist() == g["last_rows"]
    assert d["has_cached_context"] == g["block_tables_passed"]


def test_decode_three_with_padding_row():
    g = GOLD["decode_three"]
    bs = g["block_size"]
    tables, nxt = [], 0
    for L in g["seq_lens"]:
        nb = -(-L // bs)
        tables.append(list(range(nxt, nxt + nb)))
        nxt += nb
    assert [len(t) for t in tables] == g["table_lens"]
    seqs = [NS(block_table=t, num_cached=L - 1, num_new=1) for t, L in zip(tables, g["seq_lens"])]
    d = meta.prepare_decode(seqs, bs)
    assert d["positions"].tolist() == g["positions"]
    assert d["context_lens"].tolist() == g["context_lens"]
    assert list(d["block_tables"].shape) == g["block_tables_shape"]
    assert (d["block_tables"] == -1).sum() == 3 * 4 - sum(g["table_lens"])
    padded = meta.prepare_decode(seqs + [NS(block_table=[], num_cached=0, num_new=0)] *
                                 (g["bucket"] - len(seqs)), bs)
    assert padded["slot_mapping"][-1] == g["pad_row_slot"]
    assert padded["context_lens"][-1] == g["pad_row_context_len"]


def test_seven_token_prompt_then_decode():
    g = GOLD["slots_seven_tokens"]
    bs, bt = g["block_size"], g["block_table"]
    d = meta.prepare_prefill([NS(block_table=bt, num_cached=0, num_new=g["prompt_len"])], bs)
    assert d["slot_mapping"].tolist() == g["slot_mapping"]
    n = g["decode_len"]
    dd = meta.prepare_decode([NS(block_table=bt, num_cached=n - 1, num_new=1)], bs)
    assert dd["slot_mapping"].tolist() == [g["decode_slot"]]
    read = [meta.slot_of(bt, j, bs) for j in range(int(dd["context_lens"][0]))]
    assert read == g["decode_reads_slots"]


def test_prefix_hit_packing():
    g = GOLD["prefix_hit_packing"]
    bs = g["block_size"]
    seqs = [NS(block_table=list(range(10)), num_cached=s["num_cached"], num_new=s["num_new"])
            for s in g["seqs"]]
    d = meta.prepare_prefill(seqs, bs)
    assert d["positions"].tolist() == g["positions"]
    assert d["cu_seqlens_q"].tolist() == g["cu_seqlens_q"]
    assert d["cu_seqlens_k"].tolist() == g["cu_seqlens_k"]


def test_append_table_matches_block_reservation():
    g = GOLD["append_table"]
    bs = g["block_size"]
    for length, pos, needs_new in g["rows"]:
        assert length - 1 == pos
        grows = workloads._blocks_for(length, bs) > workloads._blocks_for(length - 1, bs)
        assert grows == needs_new
        # The stored position opens a new block exactly when it sits at offset 0.
        assert (pos % bs == 0) == needs_new


def test_long_prompt_chunks():
    g = GOLD["long_prompt_chunks"]
    bs, L, budget = g["block_size"], g["prompt_len"], g["budget"]
    assert workloads._blocks_for(L, bs) == g["blocks"]
    table = list(range(g["blocks"]))[::-1]  # any distinct ids
    chunks, cached, all_slots = [], 0, []
    while cached < L:
        n = min(budget, L - cached)
        d = meta.prepare_prefill([NS(block_table=table, num_cached=cached, num_new=n)], bs)
        assert d["cu_seqlens_k"].tolist() == [0, cached + n]
        assert d["has_cached_context"] == (cached > 0)
        all_slots.append(d["slot_mapping"])
        chunks.append(n)
        cached += n
    assert chunks[:-1] == [budget] * g["full_chunks"] and chunks[-1] == g["last_chunk"]
    s = np.concatenate(all_slots)
    # Every position lands in its own slot of the reserved blocks, each exactly once.
    assert len(np.unique(s)) == L
    assert set((s // bs).tolist()) == set(table)


def test_block_bytes():
    g = GOLD["block_bytes"]
    shape = workloads.AttnShape(num_heads=16, num_kv_heads=g["kv_heads"], head_dim=g["head_dim"],
                                block_size=g["block_size"])
    per_token_layer = 2 * shape.row_elems * g["itemsize"]
    assert per_token_layer * g["layers"] == g["bytes_per_token"]
    assert per_token_layer * g["layers"] * g["block_size"] == g["block_bytes"]


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_config_workloads_are_consistent(name):
    w = workloads.CONFIGS[name]()
    bs = w.shape.block_size
    for st in w.steps:
        ids = []
        for s in st.prefill + st.decode:
            n = s.num_cached + s.num_new
            assert len(s.block_table) == workloads._blocks_for(n, bs) or \
                (n <= len(s.block_table) * bs)
            ids += s.block_table
        assert all(0 <= i < w.num_blocks for i in ids)
        assert all(w.owned[i] for i in ids)
        # New-token slots of one step never collide (each token owns its slot).
        pre = meta.prepare_prefill(st.prefill, bs)["slot_mapping"] if st.prefill else \
            np.zeros(0, np.int32)
        dec = meta.prepare_decode(st.decode, bs)["slot_mapping"] if st.decode else \
            np.zeros(0, np.int32)
        allslots = np.concatenate([pre, dec])
        valid = allslots[allslots != -1]
        assert len(np.unique(valid)) == len(valid)
