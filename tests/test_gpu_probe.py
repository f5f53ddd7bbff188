"""The streaming-read probe (the benchmark's measurement helper, include/nv_probe.h, libnvprobe.so) runs and writes nothing
for data whose fold is not its sentinel."""
import pytest
import torch

from paged_kv_cache_store_amd import probe

pytestmark = pytest.mark.gpu


def test_probe_reads_without_writing():
    x = torch.ones(32 << 20, dtype=torch.bfloat16, device="cuda")  # 64 MiB: every fold is 0
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    probe.nv_probe_stream_read(x, sink)
    probe.nv_probe_stream_read(x[:8], sink)  # a tail shorter than one grid stride
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
