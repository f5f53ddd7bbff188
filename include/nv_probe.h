/*
 * nv_probe.h - BENCHMARK-ONLY measurement helper, built into its own library (libnvprobe.so),
 * not into the paged-KV library and not part of its path. It measures the HBM read rate that a
 * plain streaming kernel reaches on this GPU, the practical ceiling against which the
 * bandwidth-bound kernels of the path (the decode, which reads each K/V byte once) are compared
 * beside the published peak. It includes nv_paged.h for the status type only.
 */
#ifndef NV_PROBE_H
#define NV_PROBE_H

#include "nv_paged.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` once (16-byte non-temporal loads, grid-stride over up to 65536
 * workgroups, eight loads in flight per lane) and folds them into a value that is written to `sink` (one uint32) only if
 * it equals a fixed constant, so the reads cannot be dropped and nothing else is written.
 *
 *   src    device buffer of `bytes` bytes, 16-byte aligned; read only.
 *   bytes  > 0 and a multiple of 16.
 *   sink   device uint32, written at most once (its value carries no meaning).
 * Errors: NV_ERR_INVALID_ARG (null pointer, bytes not a positive multiple of 16, src not
 * 16-byte aligned), NV_ERR_LAUNCH. Asynchronous on `stream`; the caller times it.
 */
nv_status nv_probe_stream_read(const void *src, int64_t bytes, uint32_t *sink,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NV_PROBE_H */
