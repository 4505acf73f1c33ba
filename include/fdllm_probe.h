/*
 * fdllm_probe.h -- measurement probe exported by libfdllm beside the fused
 * step: the streaming-read rate this GPU sustains, the ceiling the attention
 * phase's bandwidth is set against (the pages frame the fused step as an
 * I/O problem: alanhou.org summary, "The Gap" and "Core Mechanism" item 1).
 */
#ifndef FDLLM_PROBE_H
#define FDLLM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, >= 16) of the caller's device buffer `buf`
 * once with `workgroups` workgroups of 256 threads (0: 1024), each reading
 * one contiguous slice, 16 B per lane and eight loads in flight per lane.  `sink` is a
 * caller-owned 16-byte device buffer the kernel may write (it does not on
 * ordinary data).  Both pointers 16-byte aligned.  Asynchronous on stream
 * (a hipStream_t, NULL = default); time it with events around the call.
 * Statuses (fdllm.h): FDLLM_ERR_ARG, FDLLM_ERR_ALIGN, FDLLM_ERR_HIP. */
int fdllm_probe_read(const void* buf, int64_t bytes, int32_t workgroups, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FDLLM_PROBE_H */
