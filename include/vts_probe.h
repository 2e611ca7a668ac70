/*
 * vts_probe.h -- measurement probes shipped beside the top-k library
 * (libvts_probe.so).  Not part of the selection path: they exist so that a
 * benchmark can quote the top-k kernels against plain streaming kernels on the
 * same device.  Both calls are asynchronous on `stream` (a hipStream_t as
 * void*, NULL = null stream) and return 0, -1 for a bad argument (null,
 * not 16-byte aligned, size not a multiple of 16) or -4 for a launch error.
 */
#ifndef VTS_PROBE_H
#define VTS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device address `buf` once with 16-byte loads.
 * `sink` (device, >= 4096 uint32) is written only in a practically impossible
 * case; it keeps the loads from being optimised away. */
int vts_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Copies `bytes` bytes from device `src` to device `dst` with 16-byte loads and
 * stores (the buffers must not overlap). */
int vts_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VTS_PROBE_H */
