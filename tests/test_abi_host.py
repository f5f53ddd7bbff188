"""CPU tests of the C ABI: the library loads and exports what include/nv_paged.h declares, the
host metadata builder agrees bit for bit with the oracle's, and argument errors are reported
before anything is launched. No call here reaches a kernel launch."""
import ctypes
import json
import os
import re
from types import SimpleNamespace as NS

import numpy as np
import pytest

from oracle import meta
from paged_kv_cache_store_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "worked_examples.json")))


@pytest.fixture(scope="module")
def nv():
    from paged_kv_cache_store_amd import nvpaged
    return nvpaged


def _declared(header_name):
    header = open(os.path.join(ROOT, "include", header_name)).read()
    return set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(nv_\w+)\s*\(", header, re.M))


def test_exports_every_declared_symbol(nv):
    """libnvpaged.so exports exactly what nv_paged.h declares; the benchmark's probe library
    exports what nv_probe.h declares, and the path's library does not export it."""
    from paged_kv_cache_store_amd import probe
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        ["nv_paged.h", "nv_probe.h"]
    declared = _declared("nv_paged.h")
    assert declared == set(nv.EXPORTS)
    for name in declared:
        assert hasattr(nv.lib(), name), name
    assert _declared("nv_probe.h") == set(probe.EXPORTS)
    for name in probe.EXPORTS:
        assert hasattr(probe.lib(), name), name
        assert not hasattr(nv.lib(), name), name


def test_status_strings(nv):
    for code in (0, -1, -2, -3, -4, -5):
        assert nv.nv_status_string(code).startswith("NV_")
    assert nv.nv_status_string(7) == "unknown nv_status"


def _same_prefill(nv, seqs, bs):
    a = nv.nv_prepare_prefill(seqs, bs)
    b = meta.prepare_prefill(seqs, bs)
    for k in ("slot_mapping", "cu_seqlens_q", "cu_seqlens_k"):
        assert np.array_equal(a[k], b[k]), k
    assert a["max_seqlen_q"] == b["max_seqlen_q"] and a["max_seqlen_k"] == b["max_seqlen_k"]
    assert a["has_cached_context"] == b["has_cached_context"]
    w = b["block_tables"].shape[1]
    assert np.array_equal(a["block_tables"][:, :w], b["block_tables"])


def _same_decode(nv, seqs, bs):
    a = nv.nv_prepare_decode(seqs, bs)
    b = meta.prepare_decode(seqs, bs)
    for k in ("slot_mapping", "context_lens"):
        assert np.array_equal(a[k], b[k]), k
    w = b["block_tables"].shape[1]
    if w:
        assert np.array_equal(a["block_tables"][:, :w], b["block_tables"])
    else:
        assert np.all(a["block_tables"] == -1)


def test_metadata_worked_examples(nv):
    g = GOLD["prefill_packing"]
    seqs = [NS(**{k: v for k, v in s.items() if k != "name"}) for s in g["seqs"]]
    p = nv.nv_prepare_prefill(seqs, g["block_size"])
    assert p["slot_mapping"].tolist() == g["slot_mapping"]
    assert p["cu_seqlens_k"].tolist() == g["cu_seqlens_k"]
    assert p["has_cached_context"] is True
    g = GOLD["decode_counters"]
    d = nv.nv_prepare_decode([NS(block_table=g["block_table"], num_cached=g["num_tokens"] - 1,
                                 num_new=1)], g["block_size"])
    assert d["slot_mapping"].tolist() == g["slot_mapping"]
    assert d["context_lens"].tolist() == g["context_lens"]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bs", [4, 16, 48, 256])
def test_metadata_matches_oracle_random(nv, seed, bs):
    shape = workloads.AttnShape(4, 2, 128, bs)
    w = workloads.random_workload(seed, shape, n_prefill=5, n_decode=7, max_len=600,
                                  max_cached=500, pad_rows=2, share_prefix=seed % 2 == 1)
    st = w.steps[0]
    _same_prefill(nv, st.prefill, bs)
    _same_decode(nv, st.decode, bs)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_metadata_matches_oracle_configs(nv, name):
    w = workloads.CONFIGS[name]()
    for st in w.steps:
        if st.prefill:
            _same_prefill(nv, st.prefill, w.shape.block_size)
        if st.decode:
            _same_decode(nv, st.decode, w.shape.block_size)


def test_metadata_rejects_bad_tables(nv):
    with pytest.raises(nv.NvError):
        nv.nv_prepare_prefill([NS(block_table=[0], num_cached=0, num_new=5)], 4)
    with pytest.raises(nv.NvError):
        nv.nv_prepare_decode([NS(block_table=[0], num_cached=3, num_new=2)], 4)
    with pytest.raises(nv.NvError):  # table longer than the sequence needs
        nv.nv_prepare_decode([NS(block_table=[0, 1], num_cached=2, num_new=1)], 4)


def test_check_indices(nv):
    ok, _ = nv.nv_check_indices(np.array([3, -1, 7], np.int32), 8,
                                np.array([[0, 1], [1, -1]], np.int32), np.array([8, 3], np.int32),
                                4, 2)
    assert ok
    ok, bad = nv.nv_check_indices(np.array([3, 3], np.int32), 8, np.zeros((0, 0), np.int32),
                                  np.zeros(0, np.int32), 4, 2)
    assert not ok and bad == 1  # duplicate slot
    ok, bad = nv.nv_check_indices(np.array([9], np.int32), 8, np.zeros((0, 0), np.int32),
                                  np.zeros(0, np.int32), 4, 2)
    assert not ok and bad == 0  # slot outside the pool
    ok, bad = nv.nv_check_indices(np.zeros(0, np.int32), 8, np.array([[0, -1]], np.int32),
                                  np.array([5], np.int32), 4, 2)
    assert not ok and bad == 1  # padding entry inside the read range
    # negative pool sizes are argument errors, reported before any slot is looked at
    ok, bad = nv.nv_check_indices(np.array([3], np.int32), -1, np.zeros((0, 0), np.int32),
                                  np.zeros(0, np.int32), 4, 2)
    assert not ok and bad == -1
    ok, bad = nv.nv_check_indices(np.array([3], np.int32), 8, np.array([[0]], np.int32),
                                  np.array([2], np.int32), 4, -1)
    assert not ok and bad == -1


def test_device_calls_reject_bad_arguments_without_launch(nv):
    L = nv.lib()
    null = None
    # store: null pointers, short row stride
    assert L.nv_store_kvcache(null, 1024, null, 1024, null, null, null, 4, 8, 128, 16, null) == -1
    assert L.nv_store_kvcache(1, 512, 1, 1024, 1, 1, 1, 4, 8, 128, 16, null) == -1
    assert L.nv_store_kvcache(null, 1024, null, 1024, null, null, null, 0, 8, 128, 16, null) == 0
    # prefill: q heads not a multiple of kv heads; head_dim 64 unsupported; no block table
    args = [1, 1, 1, 1, 1, 8, 8, 1, 1, 1]
    assert L.nv_paged_attn_prefill(*args, 6, 4, 128, 256, 0.1, 1, null) == -1
    assert L.nv_paged_attn_prefill(*args, 8, 4, 64, 256, 0.1, 1, null) == -2
    # packed mode (no block table): row strides below one row or not a multiple of 8
    assert L.nv_attn_prefill_packed(1, 1, 256, 1, 512, 1, 1, 8, 8, 1, 8, 4, 128, 0.1, 1,
                                    null) == -1
    assert L.nv_attn_prefill_packed(1, 1, 516, 1, 512, 1, 1, 8, 8, 1, 8, 4, 128, 0.1, 1,
                                    null) == -1
    assert L.nv_attn_prefill_packed(1, 1, 512, 1, 512, 1, 1, 9, 8, 1, 8, 4, 128, 0.1, 1,
                                    null) == -1  # max_seqlen_q > max_seqlen_k
    assert L.nv_attn_prefill_packed(null, null, 512, null, 512, null, null, 8, 8, 0, 8, 4, 128,
                                    0.1, null, null) == 0  # empty batch
    assert L.nv_paged_attn_prefill(1, 1, 1, 1, 1, 8, 8, null, 0, 1, 8, 4, 64, 0, 0.1, 1,
                                   null) == -2  # packed mode, head_dim 64
    assert L.nv_paged_attn_prefill(1, 1, 1, 1, 1, 9, 8, 1, 1, 1, 8, 4, 128, 256, 0.1, 1,
                                   null) == -1  # max_seqlen_q > max_seqlen_k
    assert L.nv_paged_attn_prefill(1, 1, 1, 1, 1, 8, 300, 1, 1, 1, 8, 4, 128, 256, 0.1, 1,
                                   null) == -1  # keys beyond the table width
    assert L.nv_paged_attn_prefill(1, 1, 1, 1, 1, 8, 2049, 1, 3000, 1, 8, 4, 128, 1, 0.1, 1,
                                   null) == -2  # table prefix larger than the LDS staging area
    assert L.nv_paged_attn_prefill(*args, 8, 4, 128, 256, -0.1, 1, null) == -1  # scale <= 0
    assert L.nv_paged_attn_decode(1, 1, 1, 1, 1, 3, 4, 16, 8, 128, 256, 0.0, 256, 1 << 30, 1,
                                  null) == -1  # scale <= 0
    # decode: workspace too small
    need = nv.nv_paged_attn_decode_workspace_size(4, 16, 8, 128, 3, 256)
    assert need > 0
    assert L.nv_paged_attn_decode(1, 1, 1, 1, 1, 3, 4, 16, 8, 128, 256, 0.1, 256, need - 1, 1,
                                  null) == -4
    assert L.nv_paged_attn_decode(1, 1, 1, 1, 1, 3, 4, 16, 8, 128, 256, 0.1, null, need, 1,
                                  null) == -4
    assert L.nv_paged_attn_decode(1, 1, 1, 1, 1, 3, 4, 16, 8, 64, 256, 0.1, 256, need, 1,
                                  null) == -2
    assert L.nv_paged_attn_decode(1, 1, 1, 1, 1, 3, 4, 48, 4, 128, 256, 0.1, 256, need, 1,
                                  null) == -2  # group of 12 q heads per kv head
    assert L.nv_paged_attn_decode(null, 1, 1, 1, 1, 3, 0, 16, 8, 128, 256, 0.1, null, 0, null,
                                  null) == 0  # empty batch


def test_prefill_table_prefix_limit(nv):
    """The block-table prefix a paged prefill stages in LDS holds 2048 entries: one more is
    refused before anything is launched (stand-in addresses, never touched)."""
    L = nv.lib()
    A = 1 << 20
    for bs in (1, 8, 256):
        assert L.nv_paged_attn_prefill(A, A, A, A, A, 64, 2049 * bs, A, 2049, 1, 16, 8, 128, bs,
                                       0.088, A, None) == nv.NV_ERR_UNSUPPORTED


def test_decode_store_argument_errors(nv):
    """The one-launch store + decode rejects bad store arguments before launching anything."""
    L = nv.lib()
    null = None
    # key null, key row stride below Hkv * d, negative num_slots, null slot_mapping
    assert L.nv_paged_attn_decode_store(1, null, 1024, 1, 1024, 1, 1, 1, 100, 1, 1, 3, 4, 16, 8,
                                        128, 256, 0.1, 256, 1 << 20, null, 0, 1, null) == -1
    assert L.nv_paged_attn_decode_store(1, 1, 512, 1, 1024, 1, 1, 1, 100, 1, 1, 3, 4, 16, 8,
                                        128, 256, 0.1, 256, 1 << 20, null, 0, 1, null) == -1
    assert L.nv_paged_attn_decode_store(1, 1, 1024, 1, 1024, 1, 1, 1, -1, 1, 1, 3, 4, 16, 8,
                                        128, 256, 0.1, 256, 1 << 20, null, 0, 1, null) == -1
    assert L.nv_paged_attn_decode_store(1, 16, 1024, 16, 1024, null, 16, 16, 100, 1, 1, 3, 4,
                                        16, 8, 128, 256, 0.1, 256, 1 << 20, null, 0, 1, null) == -1
    # decode-side errors surface unchanged (16-byte aligned dummies: the fused path is taken)
    assert L.nv_paged_attn_decode_store(16, 16, 1024, 16, 1024, 16, 16, 16, 100, 16, 16, 3, 4,
                                        16, 8, 128, 256, 0.0, 256, 1 << 20, null, 0, 16, null) == -1
    assert L.nv_paged_attn_decode_store(16, 16, 1024, 16, 1024, 16, 16, 16, 100, 16, 16, 3, 4,
                                        16, 8, 64, 256, 0.1, 256, 1 << 20, null, 0, 16, null) == -2
    # empty batch: nothing to do
    assert L.nv_paged_attn_decode_store(null, null, 1024, null, 1024, null, null, null, 0, null,
                                        null, 3, 0, 16, 8, 128, 256, 0.1, null, 0, null, 0,
                                        null, null) == 0
    # arrival counters shorter than batch * num_kv_heads (4 * 8), or not 4-byte aligned
    assert L.nv_paged_attn_decode_store(16, 16, 1024, 16, 1024, 16, 16, 16, 100, 16, 16, 3, 4,
                                        16, 8, 128, 256, 0.1, 256, 1 << 20, 64, 31, 16,
                                        null) == -1
    assert L.nv_paged_attn_decode_store(16, 16, 1024, 16, 1024, 16, 16, 16, 100, 16, 16, 3, 4,
                                        16, 8, 128, 256, 0.1, 256, 1 << 20, 66, 32, 16,
                                        null) == -1


def test_decode_split_choice(nv):
    # Small batches get short splits so the chip fills; large ones get long splits (few
    # partial results): 4096 (sequence, kv head) pairs or more run unsplit up to 8192 keys.
    assert nv.nv_paged_attn_decode_split_keys(6, 8, 3, 256) == 128
    assert nv.nv_paged_attn_decode_split_keys(256, 8, 16, 256) == 2048  # 2048 pairs x 2
    assert nv.nv_paged_attn_decode_split_keys(512, 8, 16, 256) == 8192
    assert nv.nv_paged_attn_decode_split_keys(64, 8, 16, 256) == 512  # 512 pairs x 8 splits
    # Unsplit, but a grid that runs in waves: the workspace holds only the longest-first
    # sequence order, one int32 per sequence, padded to 256 bytes.
    assert nv.nv_paged_attn_decode_workspace_size(512, 32, 8, 128, 16, 256) == 2048
    prev = None
    for b in (1, 3, 17, 100, 600, 5000):
        s = nv.nv_paged_attn_decode_split_keys(b, 8, 16, 256)
        assert s % 64 == 0 and 128 <= s <= 8192
        assert prev is None or s >= prev  # never shorter for a larger batch
        prev = s
    # Tiny blocks cap the split so one split's table slice fits the kernel's staging area.
    assert nv.nv_paged_attn_decode_split_keys(4, 8, 4096, 1) <= 262
    # One split over a grid that fits the chip in one go: no workspace needed.
    assert nv.nv_paged_attn_decode_workspace_size(4, 16, 8, 128, 1, 128) == 0
    assert nv.nv_paged_attn_decode_workspace_size(4096, 16, 8, 128, 1, 256) == 16384
    # A split grid adds the order after the partial results.
    n = 64 * 16 * 8  # 64 sequences x 16 heads x 8 splits of 512 keys
    assert nv.nv_paged_attn_decode_workspace_size(64, 16, 8, 128, 16, 256) == (
        n * 2 * 4 + n * 128 * 4 + 256)


def test_tp_share_divides_heads_only():
    w = workloads.config_mixed_8b()
    r = workloads.tp_share(w, 4)
    assert (r.shape.num_heads, r.shape.num_kv_heads) == (8, 2)
    assert r.shape.head_dim == 128 and r.shape.block_size == w.shape.block_size
    assert r.steps is w.steps and r.num_blocks == w.num_blocks
    assert workloads.tp_share(w, 1) is w
    with pytest.raises(ValueError):
        workloads.tp_share(w, 3)


def test_norm_rope_store_rejects_bad_arguments_without_launch(nv):
    L = nv.lib()
    null = None
    W = (16 + 2 * 8) * 128
    base = [1, W, 1, 1, 1, 1, 4096, 1e-6, 1, null, 1, 1, 1, 4, 16, 8, 128, 64, null]
    assert L.nv_qk_norm_rope_store(*base[:13], 0, *base[14:]) == 0  # no tokens
    bad = list(base); bad[1] = W - 8
    assert L.nv_qk_norm_rope_store(*bad) == -1  # row stride below the width
    bad = list(base); bad[1] = W + 4
    assert L.nv_qk_norm_rope_store(*bad) == -1  # row stride not a multiple of 8
    bad = list(base); bad[16] = 64
    assert L.nv_qk_norm_rope_store(*bad) == -2  # head_dim 64
    bad = list(base); bad[7] = -1.0
    assert L.nv_qk_norm_rope_store(*bad) == -1  # eps < 0
    bad = list(base); bad[14], bad[15] = 6, 4
    assert L.nv_qk_norm_rope_store(*bad) == -1  # q heads not a multiple of kv heads
    bad = list(base); bad[6] = 0
    assert L.nv_qk_norm_rope_store(*bad) == -1  # empty table
    bad = list(base); bad[2] = null
    assert L.nv_qk_norm_rope_store(*bad) == -1  # no positions


def test_noalloc_decode_rejects_oversize_without_launch(nv):
    """The allocation-free decode refuses, before any device call, a request whose workspace
    exceeds its static array (here 2048 rows x 64 q heads in 16 key splits: ~1 GiB)."""
    L = nv.lib()
    A = 1 << 20  # stand-in addresses: the call fails before touching them
    need = nv.nv_paged_attn_decode_workspace_size(2048, 64, 8, 128, 4096, 1)
    assert need > nv.NV_DECODE_SCRATCH_BYTES
    assert L.nv_paged_attn_decode_noalloc(A, A, A, A, A, 4096, 2048, 64, 8, 128, 1, 0.088, A,
                                          None) == nv.NV_ERR_SCRATCH


def test_norm_rope_store_rejects_misaligned_buffers(nv):
    """Every buffer the kernel moves in 16-byte vectors must be 16-byte aligned; a misaligned
    one (e.g. a column-sliced qkv view) is an argument error, returned before any launch."""
    L = nv.lib()
    A = 1 << 20  # stand-in addresses: every call below fails before touching them
    W = (16 + 2 * 8) * 128
    base = [A, W, A, A, A, A, 4096, 1e-6, A, A, A, A, A, 4, 16, 8, 128, 64, None]
    for i, name in ((0, "qkv"), (3, "q_norm_weight"), (4, "k_norm_weight"),
                    (5, "cos_sin_cache"), (8, "q_out"), (9, "k_out"), (10, "k_cache"),
                    (11, "v_cache")):
        bad = list(base)
        bad[i] = A + 8
        assert L.nv_qk_norm_rope_store(*bad) == -1, name


def test_rope_table_follows_the_formula():
    """The fp32 rotary table the binding builds against the oracle's float64 evaluation of the
    same formula: differences come only from fp32 rounding of theta_i, of p * theta_i (at most
    p * 2^-23 radians) and of cos/sin."""
    from oracle import rope as R
    from paged_kv_cache_store_amd import nvpaged as nvp
    tab = nvp.rope_cos_sin_cache(4096, 128, 1e6, "cpu").double().numpy()
    ref = R.rope_table_f64(4096, 128, 1e6)
    p = np.arange(4096, dtype=np.float64)[:, None]
    bound = p * 2.0 ** -22 + 2.0 ** -22
    assert np.all(np.abs(tab - ref) <= bound)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_token_positions_match_oracle(name):
    from paged_kv_cache_store_amd import step as gstep
    w = workloads.CONFIGS[name]()
    for st in w.steps:
        parts = []
        if st.prefill:
            parts.append(meta.prepare_prefill(st.prefill, w.shape.block_size)["positions"])
        if st.decode:
            parts.append(meta.prepare_decode(st.decode, w.shape.block_size)["positions"])
        assert np.array_equal(gstep.token_positions(st), np.concatenate(parts))


def test_probe_argument_errors():
    """The streaming-read probe rejects bad arguments before launching anything."""
    from paged_kv_cache_store_amd import probe
    L = probe.lib()
    assert L.nv_probe_stream_read(None, 1024, 64, None) == -1
    assert L.nv_probe_stream_read(64, 1024, None, None) == -1
    assert L.nv_probe_stream_read(64, 1000, 64, None) == -1   # not a multiple of 16
    assert L.nv_probe_stream_read(64, 0, 64, None) == -1
    assert L.nv_probe_stream_read(72, 1024, 64, None) == -1   # src not 16-byte aligned
