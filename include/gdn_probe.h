/*
 * gdn_probe.h - measurement probes of libgdn.so (not part of the gated delta
 * rule's computation).
 *
 * Each probe enqueues one kernel on `stream` that exercises one hardware limit,
 * so that a caller timing it (HIP events around the call) obtains the peak this
 * particular GPU actually reaches, to set beside the published peak when the
 * library's kernels are priced against a roofline:
 *
 *  gdn_probe_mfma_bf16  dense bf16 matrix-core rate: every wave issues
 *                       `iters` rounds of 8 independent 16x16x32 bf16 MFMAs
 *                       (16384 flops each) with fp32 accumulation; `waves`
 *                       waves in workgroups of 4 (one per SIMD of a CU).
 *                       Flops per call = waves * iters * 8 * 16384. Each
 *                       thread stores one float to sink[64 * wave + lane]
 *                       (sink holds waves * 64 floats).
 *  gdn_probe_copy       HBM streaming copy of `bytes` (a multiple of 16) from
 *                       src to dst: bytes read + bytes written per call.
 *                       (copy, write and read: each of 8192 workgroups sweeps
 *                       one contiguous 1/8192 of the buffer, four 16-byte
 *                       accesses in flight per lane)
 *  gdn_probe_write      HBM streaming write of `bytes` (a multiple of 16) to
 *                       dst (a constant pattern; nothing is read).
 *  gdn_probe_read       HBM streaming read of `bytes` (a multiple of 16) from
 *                       src; each workgroup writes one float of its partial sum
 *                       to sink[workgroup] (sink holds at least 8192 floats).
 *
 * Pointers are device pointers owned by the caller; 16-byte aligned. Returns
 * GDN_EINVAL for NULL or misaligned pointers, sizes that are not positive (or
 * not a multiple of 16), a wave count that is not a multiple of 4; GDN_EHIP if
 * the launch fails.
 */
#ifndef GDN_PROBE_H
#define GDN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

gdn_status gdn_probe_mfma_bf16(float* sink, int waves, int iters, void* stream);
gdn_status gdn_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);
gdn_status gdn_probe_write(void* dst, int64_t bytes, void* stream);
gdn_status gdn_probe_read(const void* src, float* sink, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PROBE_H */
