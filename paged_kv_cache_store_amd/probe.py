"""Python binding of libnvprobe.so (include/nv_probe.h): the benchmark's streaming-read probe.

A measurement helper only, built into its own library next to libnvpaged.so and not part of the
paged-KV path: it measures the HBM read rate a plain streaming kernel reaches, the practical
ceiling the decode is compared against beside the published peak.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .nvpaged import NvError, NV_OK, _dev, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvprobe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py build`")

EXPORTS = ("nv_probe_stream_read",)

_lib = ctypes.CDLL(LIB_PATH)
_lib.nv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_void_p]
_lib.nv_probe_stream_read.restype = ctypes.c_int


def lib() -> ctypes.CDLL:
    return _lib


def nv_probe_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Reads every byte of the contiguous device tensor ``src`` once; ``sink`` is a device int32
    tensor of at least one element that the probe may write. The caller times it."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    _dev(sink, "sink", torch.int32)
    st = _lib.nv_probe_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                   sink.data_ptr(), _stream(stream))
    if st != NV_OK:
        raise NvError(st, "nv_probe_stream_read")
