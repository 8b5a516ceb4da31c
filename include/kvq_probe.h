/*
 * kvq_probe.h -- a measurement aid beside the C ABI of kvq.h (not part of the decode path).
 *
 * kvq_hbm_read_probe reads `bytes` of device memory once with a plain streaming kernel
 * (non-temporal 16-byte loads, each of `workgroups` 256-thread workgroups reading one
 * contiguous slice) and writes one XOR word per workgroup to `sink` (device, `workgroups`
 * words), so that timing it gives the read rate a simple kernel reaches on this GPU: the
 * measured ceiling that the attention kernels' byte rates are compared with, beside the
 * vendor's peak.  `buf` must be 16-byte aligned and `bytes` a multiple of workgroups * 32 KiB.
 * Enqueues on `stream`; returns 0, -1 for invalid arguments, -5 if the launch is refused.
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int kvq_hbm_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_PROBE_H */
