"""Builds libnvpaged.so, the gfx950 HIP library behind include/nv_paged.h (and the measurement
helper of include/nv_probe.h), in-tree.

Every source is compiled for gfx950 only, with packed-fp32 instruction selection disabled, then
linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libnvpaged.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["store.hip", "decode.hip", "prefill.hip", "norm_rope_store.hip", "probe_read.hip",
           "host_meta.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    subprocess.run([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj],
                   check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
