/*
 * libmnb_probe -- measurement support for the libmnb benchmark (not part of
 * the GEMV path).  A read-only streaming kernel gives the HBM read bandwidth
 * the GEMV's roofline fraction is read against.  Device pointers are owned
 * by the caller; nothing is allocated.
 */
#ifndef MNB_PROBE_H
#define MNB_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` (a multiple of 16) from device buffer `buf` with 16-byte
 * loads, |unroll| (1, 2, 4 or 8) loads in flight per thread (negative:
 * the same with nontemporal loads), grid
 * `workgroups` x 256 threads, on `stream` (hipStream_t, NULL = default).
 * Each thread writes one 32-bit word of a xor of what it read to
 * sink[global thread id] (sink holds workgroups*256 words), so the loads
 * cannot be dropped.  Returns 0, -1 for bad arguments, or a hipError_t.
 */
int mnb_probe_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                   int unroll, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MNB_PROBE_H */
