"""The host-side metadata code (csrc/host_meta.cpp: nv_prepare_prefill, nv_prepare_decode,
nv_check_indices) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

A small C++ driver calls the three functions on thousands of random batches (block sizes 1 to
256, tables that are exactly long enough, longer, or one block short, table widths below and
above the longest table, empty batches, padding rows) with every output buffer allocated at
exactly the size the header documents, so any write or read past a buffer aborts the run.
Host code only: built with g++, nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
#include <stdio.h>
#include <random>
#include <vector>
#include "nv_paged.h"

template <class T> static T *ptr(std::vector<T> &v) { return v.empty() ? nullptr : v.data(); }

int main() {
    std::mt19937 rng(20260);
    const int sizes[] = {1, 4, 16, 48, 256};
    long ok = 0, rejected = 0;
    for (int it = 0; it < 4000; ++it) {
        const int batch = rng() % 9;
        const int bs = sizes[rng() % 5];
        const bool decode = rng() % 2;
        std::vector<int32_t> nc(batch), nn(batch), off(batch + 1, 0), ids;
        long total_new = 0;
        int widest = 0, next_block = 0;
        for (int b = 0; b < batch; ++b) {
            if (decode) {
                const bool pad = rng() % 5 == 0;
                nc[b] = pad ? 0 : (int32_t)(rng() % 700);
                nn[b] = pad ? 0 : 1;
            } else {
                nc[b] = rng() % 300;
                nn[b] = 1 + rng() % 300;
            }
            const int len = nc[b] + nn[b];
            int nblk = (len + bs - 1) / bs;
            const int r = rng() % 8;
            if (r == 0) nblk += 1;                  // a longer table than needed
            if (r == 1 && nblk > 0) nblk -= 1;      // one block short: must be rejected
            for (int j = 0; j < nblk; ++j) ids.push_back(next_block++);
            off[b + 1] = off[b] + nblk;
            total_new += nn[b];
            if (nblk > widest) widest = nblk;
        }
        int width = widest + (int)(rng() % 3);
        if (rng() % 6 == 0 && width > 0) width -= 1;  // narrower than a table: rejected
        std::vector<int32_t> tables((size_t)batch * width);
        nv_status st;
        std::vector<int32_t> slots;
        std::vector<int32_t> lens(batch);
        for (int b = 0; b < batch; ++b) lens[b] = nc[b] + nn[b];
        if (decode) {
            slots.assign(batch, 0);
            std::vector<int32_t> ctx(batch);
            st = nv_prepare_decode(ptr(nc), ptr(nn), off.data(), ptr(ids), batch, bs, ptr(slots),
                                   ptr(ctx), ptr(tables), width);
        } else {
            slots.assign(total_new, 0);
            std::vector<int32_t> cuq(batch + 1), cuk(batch + 1);
            int32_t mq, mk, cached;
            st = nv_prepare_prefill(ptr(nc), ptr(nn), off.data(), ptr(ids), batch, bs, ptr(slots),
                                    cuq.data(), cuk.data(), &mq, &mk, ptr(tables), width,
                                    &cached);
        }
        if (st == NV_OK) {
            ++ok;
            int64_t bad = -2;
            const int64_t num_blocks = next_block > 0 ? next_block : 1;
            nv_check_indices(ptr(slots), (int64_t)slots.size(), num_blocks * bs, ptr(tables),
                             ptr(lens), batch, width, bs, num_blocks, &bad);
        } else {
            ++rejected;
        }
    }
    printf("ok %ld rejected %ld\n", ok, rejected);
    return ok > 0 && rejected > 0 ? 0 : 1;
}
"""


def test_host_metadata_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    drv = tmp_path / "driver.cpp"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include",
           os.path.join(ROOT, "paged_kv_cache_store_amd", "csrc", "host_meta.cpp"), str(drv),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitizer" in (build.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-500:], run.stderr[-3000:])
    assert run.stdout.startswith("ok ")
    print(run.stdout.strip())
