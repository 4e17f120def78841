/*
 * pkv_probe.h - measurement kernels that sit beside the paged KV cache
 * library (libpkv.so). They compute nothing of attention: they give the
 * memory-system reference points the attention kernel is judged against.
 *
 *   pkv_probe_read   streams a buffer once with 16-byte non-temporal loads
 *                    (the flavour the attention kernels use for K/V): the practical
 *                    HBM read ceiling for a kernel that only reads.
 *   pkv_probe_copy   copies a buffer with 16-byte loads (non-temporal, as
 *                    above) and plain stores: a
 *                    transfer of known size, used to scale hardware traffic
 *                    counters (bytes fetched / written per dispatch) into
 *                    bytes.
 *
 * Conventions are those of pkv.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t, NULL = null stream), a pkv_status
 * returned, nothing allocated.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of `src` (16-byte aligned; bytes a positive multiple of
 * 16) once, in 16-byte pieces, and write one 32-bit value per workgroup into
 * `sink` (the XOR of what that workgroup read, so that no load can be
 * elided). `sink` must hold pkv_probe_read_sink_words(bytes) uint32 values.
 */
PKV_API int pkv_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Number of uint32 values pkv_probe_read writes to `sink` (0 if bytes is invalid). */
PKV_API size_t pkv_probe_read_sink_words(size_t bytes);

/*
 * Copy `bytes` bytes (a positive multiple of 16) from `src` to `dst`
 * (16-byte aligned, not overlapping) with 16-byte loads and stores.
 */
PKV_API int pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
