"""Benchmark of the paged-KV hot path on one MI355X.

One step = the whole hot path over one batch: store every new K/V row, causal paged prefill,
paged decode. Workload: the Qwen3-8B attention shape (32 q heads, 8 kv heads, head_dim 128,
block size 256), 512 decode sequences with contexts uniform in 256..4096 plus a fresh 4 x
1024-token prefill, blocks randomly permuted, N(0, 1) bf16 values. Inputs are resident in HBM
before timing starts.

Prints one JSON line. `value` is the decode attention's algorithmic HBM throughput (each
visible K/V element once, plus q, out, tables and lengths) over its average event-timed
duration in the step loop; prefill TFLOP/s and store GB/s (at their median step) are reported
beside it, and the CPU oracle is timed on the host on the same step's decode and prefill (all
host threads and one thread, median of 3 runs each). Extra parts, timed apart from the step:
all five configurations (0.6B decode of 4 + 2 rows, 0.6B varlen prefill, 0.6B prefix-cached +
chunked prefill, 0.6B decode of 256 rows, and this step) call by call, >= 50 repetitions each,
cold and warm for the three small ones; the fresh prompts through the packed (no block table)
prefill; the fused QK-norm + rotary embedding + K/V store over the step's rows; a small decode
step through 28 layers launched eagerly vs replayed from HIP graphs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixed_8b] [--tp T]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published


def decode_bytes(shape, context_lens) -> int:
    L = np.asarray(context_lens, dtype=np.int64)
    kv = int(L.sum()) * shape.num_kv_heads * shape.head_dim * 2 * 2
    qo = 2 * len(L) * shape.num_heads * shape.head_dim * 2
    tables = int(np.sum((L + shape.block_size - 1) // shape.block_size)) * 4 + len(L) * 4
    return kv + qo + tables


def prefill_flops(shape, seqs) -> int:
    tot = 0
    for s in seqs:
        lq, p = s.num_new, s.num_cached
        tot += shape.num_heads * 4 * shape.head_dim * (lq * p + lq * (lq + 1) // 2)
    return tot


def store_bytes(shape, slot_mapping) -> int:
    sm = np.asarray(slot_mapping)
    return int((sm != -1).sum()) * 4 * shape.row_elems * 2 + sm.size * 4


def source_hash(path: str) -> str:
    """Hash of a source's code: comments and whitespace are removed first, so a comment edit
    does not invalidate counters taken on the same code."""
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_store_amd", "csrc", "decode.hip")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "decode_traffic.json")
CALIB_ELEMS = 1 << 28  # int32 elements of the counter-calibration op (1 GiB read, 1 GiB written)


def load_traffic():
    """HBM bytes per decode call (order, split and combine kernels) from the committed counter summary,
    if it was taken on the current kernel source; otherwise None."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON))
    if rec.get("source_sha256_16") != source_hash(DECODE_SRC):
        return None
    return rec.get("bytes_per_launch")


def traffic_from_counters(fetch_csv: str, write_csv: str, group: int) -> dict:
    """Calibrated HBM traffic of the decode call from two rocprofv3 counter runs of
    `bench.py --calibrate-copy --step-only` (one with --pmc FETCH_SIZE, one with --pmc
    WRITE_SIZE); `group` = q heads per kv head of the workload (the split kernel's first
    template argument; the second, false, selects the plain decode the step runs).

    Each counter (KiB per dispatch) is scaled by the ratio of the true bytes to what the same
    counter reports for the calibration op, a bitwise NOT over CALIB_ELEMS int32 values that
    reads and writes exactly 4 * CALIB_ELEMS bytes."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("calib" if "bitwise_not" in name else
                   "split" if f"decode_split_kernel<{group}, false>" in name else
                   "combine" if "decode_combine_kernel" in name else
                   "order" if "decode_order_kernel" in name else None)
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: statistics.median(v) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    true_bytes = 4.0 * CALIB_ELEMS
    ff, wf = true_bytes / f["calib"], true_bytes / w["calib"]
    fetch = ff * (f["split"] + f.get("combine", 0.0) + f.get("order", 0.0))
    write = wf * (w["split"] + w.get("combine", 0.0) + w.get("order", 0.0))
    return {"source_sha256_16": source_hash(DECODE_SRC), "fetch_factor": round(ff, 4),
            "write_factor": round(wf, 4), "fetch_bytes_per_launch": round(fetch),
            "write_bytes_per_launch": round(write), "bytes_per_launch": round(fetch + write)}


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_of(n: int, fn) -> tuple:
    """Median wall time (s) of n runs of fn() and the list of times."""
    ts = []
    for _ in range(n):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[n // 2], ts


def cpu_baseline(shape, ds, k_cache, v_cache, scale, runs: int = 3):
    """The oracle (as it stands, fp64 C with OpenMP) on the host cores: the step's whole decode
    and its whole prefill with every host thread, and a bounded sample of each on one thread;
    each timed as the median of `runs` runs. Input generation is excluded; the oracle's gather
    through the block table is included."""
    import oracle  # test infrastructure: the baseline leg only
    from oracle import meta
    kb = k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    qd = ds.tensors.q_decode.view(torch.int16).cpu().numpy().view(np.uint16)
    m = meta.prepare_decode(ds.step.decode, shape.block_size)
    cores = oracle.num_threads()

    def dec(n):
        return lambda: oracle.attn_decode(qd[:n], kb, vb, m["context_lens"][:n],
                                          m["block_tables"][:n], shape.num_heads,
                                          shape.num_kv_heads, shape.head_dim, shape.block_size,
                                          scale)

    B = len(m["context_lens"])
    n1 = min(32, B)
    t_all, _ = _median_of(runs, dec(B))
    oracle.set_num_threads(1)
    try:
        t_one, _ = _median_of(runs, dec(n1))
    finally:
        oracle.set_num_threads(cores)
    nbytes = decode_bytes(shape, m["context_lens"])
    nbytes1 = decode_bytes(shape, m["context_lens"][:n1])
    res = {"value": round(nbytes / t_all / 1e9, 3), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"whole decode step ({B} sequences, {nbytes / 1e9:.2f} GB of K/V) in fp64 "
                     f"C, median of {runs} runs ({t_all:.2f} s each)",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "single_core_value": round(nbytes1 / t_one / 1e9, 3),
           "single_core_sample": f"first {n1} sequences ({nbytes1 / 1e9:.2f} GB of K/V) on 1 "
                                 f"thread, median of {runs} runs ({t_one:.2f} s each)"}
    if ds.cu_seqlens_q is not None:
        qp = ds.tensors.q_prefill.view(torch.int16).cpu().numpy().view(np.uint16)
        pm = meta.prepare_prefill(ds.step.prefill, shape.block_size)
        args = (shape.num_heads, shape.num_kv_heads, shape.head_dim, shape.block_size, scale)
        flops = prefill_flops(shape, ds.step.prefill)
        t_pre, _ = _median_of(runs, lambda: oracle.attn_prefill(
            qp, kb, vb, pm["cu_seqlens_q"], pm["cu_seqlens_k"], pm["block_tables"], *args))
        # one thread: the first 512 new rows of the first prompt (a prompt's leading rows see
        # only keys up to their own position, as in the full prefill)
        s0 = ds.step.prefill[0]
        rows = min(512, s0.num_new)
        from paged_kv_cache_store_amd.workloads import Seq
        sub = [Seq(s0.block_table, s0.num_cached, rows)]
        pm1 = meta.prepare_prefill(sub, shape.block_size)
        flops1 = prefill_flops(shape, sub)
        oracle.set_num_threads(1)
        try:
            t_pre1, _ = _median_of(runs, lambda: oracle.attn_prefill(
                qp[:rows], kb, vb, pm1["cu_seqlens_q"], pm1["cu_seqlens_k"],
                pm1["block_tables"], *args))
        finally:
            oracle.set_num_threads(cores)
        res["prefill"] = {
            "value": round(flops / t_pre / 1e9, 2), "unit": "GFLOP/s", "cores": cores,
            "sample": f"whole prefill of the step ({len(ds.step.prefill)} prompts, "
                      f"{flops / 1e9:.1f} GFLOP) in fp64 C, median of {runs} runs "
                      f"({t_pre:.2f} s each)",
            "single_core_value": round(flops1 / t_pre1 / 1e9, 3),
            "single_core_sample": f"first {rows} rows of the first prompt ({flops1 / 1e9:.2f} "
                                  f"GFLOP) on 1 thread, median of {runs} runs "
                                  f"({t_pre1:.2f} s each)"}
    return res


def norm_rope_store_part(shape, dsteps, k_cache, v_cache, iters: int) -> dict:
    """The step's rows through the fused per-head QK RMSNorm + rotary embedding + K/V store
    (one launch per step), HIP events; algorithmic bytes: the projection rows read, q written,
    K and V rows stored, positions and slots read (the 2 MiB rotary table is cache-resident and
    not counted)."""
    import torch as _t
    from paged_kv_cache_store_amd import nvpaged
    from paged_kv_cache_store_amd import step as gstep
    dev = k_cache.device
    g = _t.Generator(device="cpu").manual_seed(7)
    wq = (1 + 0.1 * _t.randn(shape.head_dim, generator=g)).bfloat16().to(dev)
    wk = (1 + 0.1 * _t.randn(shape.head_dim, generator=g)).bfloat16().to(dev)
    table = nvpaged.rope_cos_sin_cache(40960, shape.head_dim, 1e6, dev)
    nbytes = 0
    for ds in dsteps:
        n = ds.tensors.qkv.shape[0]
        live = int((ds.host["slot_mapping"] != -1).sum())
        nbytes += n * shape.qkv_width * 2 + n * shape.num_heads * shape.head_dim * 2 \
            + live * 2 * shape.row_elems * 2 + n * 12
    for _ in range(3):
        for ds in dsteps:
            gstep.run_norm_rope_store(ds, k_cache, v_cache, wq, wk, table)
    _t.cuda.synchronize()
    evs = []
    for _ in range(iters):
        a = _t.cuda.Event(enable_timing=True)
        b = _t.cuda.Event(enable_timing=True)
        a.record()
        for ds in dsteps:
            gstep.run_norm_rope_store(ds, k_cache, v_cache, wq, wk, table)
        b.record()
        evs.append((a, b))
    _t.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / iters
    gbs = nbytes / (ms * 1e-3) / 1e9
    # The same calls queued back to back behind a sleep kernel (the kernel's own rate, without
    # the host-side gaps between calls).
    qts = []
    for _ in range(5):
        if hasattr(_t.cuda, "_sleep"):
            _t.cuda._sleep(2_000_000)
        a = _t.cuda.Event(enable_timing=True)
        b = _t.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            for ds in dsteps:
                gstep.run_norm_rope_store(ds, k_cache, v_cache, wq, wk, table)
        b.record()
        _t.cuda.synchronize()
        qts.append(a.elapsed_time(b) / 20)
    qms = sorted(qts)[len(qts) // 2]
    qgbs = nbytes / (qms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "queued_ms": round(qms, 4), "queued_GB/s": round(qgbs, 1),
            "queued_frac_hbm_peak": round(qgbs / HBM_PEAK_GBS, 4)}


def percentiles(times_ms) -> dict:
    """p10 / p50 / p90 of per-step times (ms); the means above give the rates."""
    s = sorted(times_ms)
    at = lambda p: s[min(len(s) - 1, int(round(p / 100 * (len(s) - 1))))]
    return {"ms_p10": round(at(10), 4), "ms_p50": round(at(50), 4), "ms_p90": round(at(90), 4)}


def copy_ceiling(dev, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """A plain device copy of `nbytes` (torch copy_ of a contiguous bf16 buffer): bytes read
    plus bytes written per second, the practical ceiling a streaming kernel on this HBM can
    reach, beside the published peak. Median over `reps` HIP-event-timed copies."""
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        y.copy_(x)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    t = sorted(ts)[len(ts) // 2]
    gbs = 2 * nbytes / (t * 1e-3) / 1e9
    del x, y
    return {"ms": round(t, 4), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_read": nbytes, "bytes_written": nbytes}


def read_ceiling(dev, nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """The streaming-read probe (nv_probe_stream_read, libnvprobe.so) over `nbytes`, far larger
    than the caches: the HBM read rate a plain kernel reaches, the practical ceiling for the
    decode (read-only traffic). Median over `reps` HIP-event-timed calls."""
    from paged_kv_cache_store_amd import probe
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        probe.nv_probe_stream_read(x, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        probe.nv_probe_stream_read(x, sink)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    t = sorted(ts)[len(ts) // 2]
    gbs = nbytes / (t * 1e-3) / 1e9
    del x, sink
    return {"ms": round(t, 4), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_read": nbytes}


def prefill_queued(dsteps, k_cache, v_cache, scale: float, flops: int, inner: int = 10,
                   reps: int = 5) -> dict:
    """The step's prefill calls launched back to back behind a sleep kernel (as for
    `store_queued`): the kernel's own rate, without the host time between the start event and
    the launch that a single call in the step loop can include."""
    from paged_kv_cache_store_amd import step as gstep

    def once():
        for ds in dsteps:
            gstep.run_prefill(ds, k_cache, v_cache, scale)

    for _ in range(3):
        once()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(2_000_000)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(inner):
            once()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / inner)
    us = sorted(ts)[len(ts) // 2]
    tf = flops / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "TFLOP/s": round(tf, 1), "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "calls_per_region": inner}


def prefill_context(dsteps, k_cache, v_cache, scale: float, flops: int, reps: int = 25) -> dict:
    """The step's prefill calls timed one at a time (queued behind a sleep kernel, so no host
    gap) after different predecessors: another prefill (its prompts' K/V and queries still in
    L2 / MALL), the step's own order (decode of the previous step, then the store), and idle.
    The kernel is the same; the difference is the cache state its first tiles meet."""
    from paged_kv_cache_store_amd import step as gstep
    pre = lambda: [gstep.run_prefill(ds, k_cache, v_cache, scale) for ds in dsteps]
    dec = lambda: [gstep.run_decode(ds, k_cache, v_cache, scale) for ds in dsteps]
    sto = lambda: [gstep.run_store(ds, k_cache, v_cache) for ds in dsteps]
    ctxs = {"after_prefill": [pre], "after_decode_and_store": [dec, sto], "after_idle": []}
    res = {k: [] for k in ctxs}
    for _ in range(reps):
        for name, before in ctxs.items():
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(2_000_000)
            for f in before:
                f()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            pre()
            b.record()
            torch.cuda.synchronize()
            res[name].append(a.elapsed_time(b) * 1e3)
    out = {}
    for name, v in res.items():
        us = sorted(v)[len(v) // 2]
        out[name] = {"us": round(us, 2), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1)}
    return out


def store_queued(dsteps, k_cache, v_cache, nbytes: int, inner: int = 20, reps: int = 5) -> dict:
    """The step's store calls launched back to back, `inner` per HIP-event-timed region, with
    the GPU held busy by a sleep kernel while they are queued: the store kernel's own rate,
    without the launch gap that the single event-timed call of the step loop includes (at
    this size the gap is a third of that figure). Storing the same rows again is
    idempotent."""
    from paged_kv_cache_store_amd import step as gstep

    def once():
        for ds in dsteps:
            gstep.run_store(ds, k_cache, v_cache)

    for _ in range(3):
        once()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(2_000_000)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(inner):
            once()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / inner)
    us = sorted(ts)[len(ts) // 2]
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "calls_per_region": inner}


def small_decode_latency(dev, iters: int, layers: int = 28) -> dict:
    """Time of one small decode step (4 sequences + 2 padding rows, Qwen3-0.6B shape) through
    `layers` attention layers, each with its own pool: store + decode launched eagerly per
    layer vs one HIP-graph replay of all layers (inputs staged into the graph's static buffers
    once per step), each both as two launches per layer and as the one fused store+decode
    launch. HIP events around each step; median."""
    from paged_kv_cache_store_amd import graphs
    from paged_kv_cache_store_amd import step as gstep
    from paged_kv_cache_store_amd import workloads
    w = workloads.CONFIGS["decode_small"]()
    kc, vc, tens = workloads.materialize(w, dev)
    ds = gstep.prepare_step(w.shape, w.steps[0], tens[0], dev)
    scale = w.shape.head_dim ** -0.5
    t = ds.tensors
    ks = [kc] + [kc.clone() for _ in range(layers - 1)]
    vs = [vc] + [vc.clone() for _ in range(layers - 1)]
    assert t.key.shape[0] == t.q_decode.shape[0]  # decode-only step: one new row per sequence
    dg = graphs.DecodeGraphs(w.shape, ks, vs, max_bs=8, max_blocks=ds.decode_tables.shape[1],
                             scale=scale, fused=False)
    dgf = graphs.DecodeGraphs(w.shape, ks, vs, max_bs=8, max_blocks=ds.decode_tables.shape[1],
                              scale=scale, fused=True)
    args = (t.q_decode, t.key, t.value, ds.slot_mapping, ds.context_lens, ds.decode_tables)

    def eager():
        for k_l, v_l in zip(ks, vs):
            gstep.run_store(ds, k_l, v_l)
            gstep.run_decode(ds, k_l, v_l, scale)

    def eager_fused():
        for k_l, v_l in zip(ks, vs):
            gstep.run_decode_store(ds, k_l, v_l, scale)

    def replay():
        dg.run(*args)

    def replay_fused():
        dgf.run(*args)

    res = {"layers": layers}
    for name, fn in (("eager_us", eager), ("graph_us", replay),
                     ("eager_fused_us", eager_fused), ("graph_fused_us", replay_fused)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(iters):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        times = sorted(a.elapsed_time(b) for a, b in evs)
        res[name] = round(times[len(times) // 2] * 1e3, 2)  # median, microseconds
    res["rows"] = int(t.q_decode.shape[0])
    res["bucket"] = dg.bucket_for(int(t.q_decode.shape[0]))
    del dg, dgf, ks, vs
    return res


FLUSH_BYTES = 512 << 20  # larger than L2 (4 MB per XCD) and the 256 MB MALL together


def time_calls(fn, reps: int, flush=None, sleep_cycles: int = 1_000_000) -> list:
    """Per-call HIP-event times (ms) of fn() over `reps` repetitions. Each repetition is queued
    behind a GPU sleep kernel, so the host has launched everything before the timed call starts
    and no launch gap falls inside it. Cold (flush given): the flush buffer is overwritten right
    before the timed call, evicting L2 and MALL. Warm: the same call runs once, untimed, right
    before the timed one."""
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(sleep_cycles)
        if flush is not None:
            flush.fill_(1)
        else:
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return times


def _rate(times_ms, work: int, kind: str) -> dict:
    """Median / p10 / p90 of per-call times and the rate at the median against its peak."""
    p = percentiles(times_ms)
    t = p["ms_p50"] * 1e-3
    if kind == "bytes":
        r = work / t / 1e9
        return {**p, "GB/s": round(r, 1), "frac_hbm_peak": round(r / HBM_PEAK_GBS, 4),
                "bytes": work, "reps": len(times_ms)}
    r = work / t / 1e12
    return {**p, "TFLOP/s": round(r, 1), "frac_bf16_peak": round(r / BF16_PEAK_TFLOPS, 4),
            "flops": work, "reps": len(times_ms)}


def oracle_config(w, dsteps, k_cache, v_cache, runs: int = 3) -> dict:
    """The oracle (fp64 C, all host threads) over one configuration's whole attention work: every
    step's prefill and decode on host copies of the pools, median of `runs` runs; input copies
    excluded, the oracle's gather through the tables included. Rates in the bench's units."""
    import oracle  # test infrastructure: the CPU-baseline leg only
    from oracle import meta
    shape = w.shape
    scale = shape.head_dim ** -0.5
    kb = k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    args = (shape.num_heads, shape.num_kv_heads, shape.head_dim, shape.block_size, scale)
    pre_calls, dec_calls, flops, nbytes = [], [], 0, 0
    for st, ds in zip(w.steps, dsteps):
        if st.prefill:
            qp = ds.tensors.q_prefill.view(torch.int16).cpu().numpy().view(np.uint16)
            pm = meta.prepare_prefill(st.prefill, shape.block_size)
            pre_calls.append(lambda qp=qp, pm=pm: oracle.attn_prefill(
                qp, kb, vb, pm["cu_seqlens_q"], pm["cu_seqlens_k"], pm["block_tables"], *args))
            flops += prefill_flops(shape, st.prefill)
        if st.decode:
            qd = ds.tensors.q_decode.view(torch.int16).cpu().numpy().view(np.uint16)
            dm = meta.prepare_decode(st.decode, shape.block_size)
            bt = dm["block_tables"] if dm["block_tables"].shape[1] else \
                np.full((len(st.decode), 1), -1, np.int32)
            dec_calls.append(lambda qd=qd, dm=dm, bt=bt: oracle.attn_decode(
                qd, kb, vb, dm["context_lens"], bt, *args))
            nbytes += decode_bytes(shape, dm["context_lens"])
    rec = {"cores": oracle.num_threads(), "runs": runs}
    if pre_calls:
        t, _ = _median_of(runs, lambda: [c() for c in pre_calls])
        rec["prefill_s"] = round(t, 4)
        rec["GFLOP/s"] = round(flops / t / 1e9, 2)
    if dec_calls:
        t, _ = _median_of(runs, lambda: [c() for c in dec_calls])
        rec["decode_s"] = round(t, 4)
        rec["GB/s"] = round(nbytes / t / 1e9, 3)
    return rec


def config_parts(dev, reps: int, mixed=None, with_oracle: bool = False) -> tuple:
    """Every configuration's store, prefill and decode calls under one protocol: per-call HIP
    events, `reps` repetitions, median / p10 / p90 and the rate at the median. The three small
    configurations (which fit in the 256 MB MALL) are timed cold (L2 and MALL evicted by a
    512 MiB write before each call) and warm (the same call just before); the two large ones
    warm only (their K/V is far larger than the caches). A prefill configuration with two
    steps reports each step and their sum. `mixed`: the 8B mixed step already resident (its
    workload, pools and device steps)."""
    from paged_kv_cache_store_amd import step as gstep
    from paged_kv_cache_store_amd import workloads
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    out, cpu = {}, {}
    for name in ("decode_small", "prefill_varlen", "prefix_chunked", "decode_large", "mixed_8b"):
        if name == "mixed_8b" and mixed is not None:
            w, k_cache, v_cache, dsteps = mixed
        else:
            w = workloads.CONFIGS[name]()
            k_cache, v_cache, tens = workloads.materialize(w, dev, poison=False)
            dsteps = [gstep.prepare_step(w.shape, st, t, dev) for st, t in zip(w.steps, tens)]
        shape = w.shape
        scale = shape.head_dim ** -0.5
        cold_too = name in ("decode_small", "prefill_varlen", "prefix_chunked")
        for ds in dsteps:  # every step's rows in the pool before any attention call
            gstep.run_store(ds, k_cache, v_cache)
        torch.cuda.synchronize()
        rec = {"workload": w.name}
        modes = ("cold", "warm") if cold_too else ("warm",)
        for mode in modes:
            fl = flush if mode == "cold" else None
            parts = {}
            pre_total, pre_flops = 0.0, 0
            for i, (st, ds) in enumerate(zip(w.steps, dsteps)):
                sfx = f"_step{i}" if len(dsteps) > 1 else ""
                parts["store" + sfx] = _rate(
                    time_calls(lambda: gstep.run_store(ds, k_cache, v_cache), reps, fl),
                    store_bytes(shape, ds.host["slot_mapping"]), "bytes")
                if st.prefill:
                    f = prefill_flops(shape, st.prefill)
                    r = _rate(time_calls(lambda: gstep.run_prefill(ds, k_cache, v_cache, scale),
                                         reps, fl), f, "flops")
                    parts["prefill" + sfx] = r
                    pre_total += r["ms_p50"]
                    pre_flops += f
                if st.decode:
                    parts["decode" + sfx] = _rate(
                        time_calls(lambda: gstep.run_decode(ds, k_cache, v_cache, scale), reps,
                                   fl), decode_bytes(shape, ds.host["decode"]["context_lens"]),
                        "bytes")
            if len(dsteps) > 1 and pre_flops:
                tf = pre_flops / (pre_total * 1e-3) / 1e12
                parts["prefill_all_steps"] = {"ms_p50_sum": round(pre_total, 4),
                                              "TFLOP/s": round(tf, 1),
                                              "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                                              "flops": pre_flops}
            rec[mode] = parts
        out[name] = rec
        if with_oracle:
            cpu[name] = oracle_config(w, dsteps, k_cache, v_cache)
        if name != "mixed_8b" or mixed is None:
            del k_cache, v_cache, dsteps
            torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return out, cpu


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed_8b")
    ap.add_argument("--tp", type=int, default=1,
                    help="run one rank's share of a tensor-parallel deployment of degree TP "
                         "(heads divided by TP) on this one GPU")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step (store, prefill, decode): no extra parts")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run the counter-calibration op (1 GiB bitwise NOT) before timing")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the decode call's calibrated HBM traffic from two rocprofv3 "
                         "--pmc runs of --calibrate-copy to profiles/decode_traffic.json, exit")
    args = ap.parse_args()
    if args.traffic:
        from paged_kv_cache_store_amd import workloads as _w
        s_ = _w.tp_share(_w.CONFIGS[args.workload](), args.tp).shape
        rec = traffic_from_counters(*args.traffic, s_.num_heads // s_.num_kv_heads)
        rec["workload"] = args.workload
        json.dump(rec, open(TRAFFIC_JSON, "w"), indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    global torch
    import torch
    from paged_kv_cache_store_amd import step as gstep
    from paged_kv_cache_store_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.tp_share(workloads.CONFIGS[args.workload](), args.tp)
    shape = w.shape
    scale = shape.head_dim ** -0.5
    k_cache, v_cache, tens = workloads.materialize(w, dev, poison=False)
    dsteps = []
    for st, t in zip(w.steps, tens):
        ds = gstep.prepare_step(shape, st, t, dev)
        ds.step = st
        dsteps.append(ds)
    torch.cuda.synchronize()

    # Algorithmic work per step.
    dec_bytes = sum(decode_bytes(shape, ds.host["decode"]["context_lens"])
                    for ds in dsteps if "decode" in ds.host)
    pre_flops = sum(prefill_flops(shape, st.prefill) for st in w.steps)
    sto_bytes = sum(store_bytes(shape, ds.host["slot_mapping"]) for ds in dsteps)

    if args.calibrate_copy:
        x = torch.zeros(CALIB_ELEMS, dtype=torch.int32, device=dev)
        y = torch.empty_like(x)
        torch.bitwise_not(x, out=y)
        torch.cuda.synchronize()
        del x, y

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for ds in dsteps:
            gstep.run_step(ds, k_cache, v_cache, scale)
    torch.cuda.synchronize()

    names = ("store", "prefill", "decode")
    ev = {n: [] for n in names}
    # No Python garbage collection inside the timed region: a collection pass between an
    # event's record and its launch would stall the GPU and land in that part's time.
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for ds in dsteps:
            for n, fn in (("store", lambda: gstep.run_store(ds, k_cache, v_cache)),
                          ("prefill", lambda: gstep.run_prefill(ds, k_cache, v_cache, scale)),
                          ("decode", lambda: gstep.run_decode(ds, k_cache, v_cache, scale))):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                ev[n].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / args.steps for n in names}
    # Per-step times (the step's calls of each part summed) for percentiles.
    k = len(dsteps)
    per_step = {n: [sum(a.elapsed_time(b) for a, b in ev[n][i * k:(i + 1) * k])
                    for i in range(args.steps)] for n in names}

    # The same fresh prompts through the packed (no block table) prefill path, timed apart.
    packed = [ds for ds in dsteps if ds.cu_seqlens_q is not None
              and not ds.host["prefill"]["has_cached_context"] and not args.step_only]
    packed_ms = None
    if packed:
        for ds in packed:
            gstep.run_prefill_packed(ds, scale)
        pev = []
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for ds in packed:
                gstep.run_prefill_packed(ds, scale)
            b.record(stream)
            pev.append((a, b))
        torch.cuda.synchronize()
        packed_ms = sum(a.elapsed_time(b) for a, b in pev) / args.steps
        packed_flops = sum(prefill_flops(shape, ds.step.prefill) for ds in packed)

    # The headline and the roofline use the decode's average duration per step (the
    # profiler's statistic); every part also reports its median step, at which store and
    # prefill rates are given (a single slow step, e.g. the first one's launch gap, moves the
    # mean of a 10 us call by far more than its median).
    med = {n: percentiles(per_step[n])["ms_p50"] for n in names}
    dec_gbs = dec_bytes / (ms["decode"] * 1e-3) / 1e9 if dec_bytes else 0.0
    pre_tflops = pre_flops / (med["prefill"] * 1e-3) / 1e12 if pre_flops else 0.0
    sto_gbs = sto_bytes / (med["store"] * 1e-3) / 1e9
    traffic = load_traffic()

    res = {
        "metric": "paged decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% bf16 MFMA)",
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 values, randomly permuted physical blocks)",
        "config": {"workload": w.name, "tp_share": args.tp, "num_heads": shape.num_heads,
                   "num_kv_heads": shape.num_kv_heads, "head_dim": shape.head_dim,
                   "block_size": shape.block_size, "decode_seqs": len(w.steps[0].decode),
                   "prefill_tokens": w.steps[0].num_prefill_tokens, "seed": w.seed},
        "parts": {
            "store": {"ms": round(med["store"], 4), "ms_mean": round(ms["store"], 4),
                      "GB/s": round(sto_gbs, 1),
                      "frac_hbm_peak": round(sto_gbs / HBM_PEAK_GBS, 4), "bytes": sto_bytes,
                      **percentiles(per_step["store"])},
            "prefill": {"ms": round(med["prefill"], 4), "ms_mean": round(ms["prefill"], 4),
                        "TFLOP/s": round(pre_tflops, 1),
                        "frac_bf16_peak": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                        "flops": pre_flops, **percentiles(per_step["prefill"])},
            "decode": {"ms": round(ms["decode"], 4), "ms_mean": round(ms["decode"], 4),
                       "GB/s": round(dec_gbs, 1),
                       "frac_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4), "bytes": dec_bytes,
                       **percentiles(per_step["decode"])},
        },
        "roofline": {"bound": "hbm", "kernel": "decode (order kernel + split kernel, + merge kernel when a row is split)",
                     "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": None,
    }
    if not args.step_only:
        res["parts"]["norm_rope_store"] = norm_rope_store_part(shape, dsteps, k_cache, v_cache,
                                                               args.steps)
        res["parts"]["decode_small_step"] = small_decode_latency(dev, max(20, args.steps))
        res["parts"]["store_queued"] = store_queued(dsteps, k_cache, v_cache, sto_bytes)
        if pre_flops:
            res["parts"]["prefill_queued"] = prefill_queued(dsteps, k_cache, v_cache, scale,
                                                            pre_flops)
            res["parts"]["prefill_context"] = prefill_context(dsteps, k_cache, v_cache, scale,
                                                              pre_flops)
        res["parts"]["copy_ceiling"] = copy_ceiling(dev)
        res["parts"]["read_ceiling"] = read_ceiling(dev)
        res["roofline"]["measured_read_ceiling_GB/s"] = res["parts"]["read_ceiling"]["GB/s"]
        res["roofline"]["frac_of_measured_ceiling"] = round(
            dec_gbs / res["parts"]["read_ceiling"]["GB/s"], 4)
    cpu_per_config = {}
    if not args.step_only and args.tp == 1 and args.workload == "mixed_8b":
        res["parts"]["configs"], cpu_per_config = config_parts(
            dev, max(50, args.steps), mixed=(w, k_cache, v_cache, dsteps),
            with_oracle=not args.no_cpu_baseline)
    if packed_ms:
        tf = packed_flops / (packed_ms * 1e-3) / 1e12
        res["parts"]["prefill_packed"] = {"ms": round(packed_ms, 4), "TFLOP/s": round(tf, 1),
                                          "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                                          "flops": packed_flops}
    if not args.no_cpu_baseline and dsteps[0].context_lens is not None:
        res["cpu_baseline"] = cpu_baseline(shape, dsteps[0], k_cache, v_cache, scale)
        if cpu_per_config:
            # each configuration's whole attention work (every step's prefill and decode)
            res["cpu_baseline"]["per_config"] = cpu_per_config
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
