/*
 * fdllm_probe.h -- measurement probes exported by libfdllm beside the fused
 * step: the streaming-read rate this GPU sustains, the ceiling the attention
 * phase's bandwidth is set against (the pages frame the fused step as an
 * I/O problem: alanhou.org summary, "The Gap" and "Core Mechanism" item 1),
 * and the rates of the two instructions the step's kernels are built on (the
 * bf16 matrix instruction and the LDS-DMA load), which bound their loops.
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

/* Issue rate of the bf16 matrix instruction both MFMA kernels use
 * (v_mfma_f32_16x16x32_bf16): `workgroups` workgroups (0: 256) of `waves`
 * waves (1..8), each wave running `iters` (>= 1) rounds of eight independent
 * accumulations.  Executed flops = workgroups * waves * iters * 8 * 16384.
 * `sink` as above (written only on an impossible sum).  Asynchronous on
 * stream; time it with events.  Statuses: FDLLM_ERR_ARG, FDLLM_ERR_ALIGN,
 * FDLLM_ERR_HIP. */
int fdllm_probe_mfma(int32_t workgroups, int32_t waves, int32_t iters, void* sink, void* stream);

/* Rate of the LDS-DMA loads (global_load_lds, 16 B per lane) the attention
 * and projection rings are fed with: `workgroups` workgroups (0: 256) of
 * `waves` waves (1..8), each wave issuing `iters` (>= 1) 1 KB loads into the
 * workgroup's 64 KB of LDS, at most 16 in flight, cycling over the caller's
 * device buffer `buf` of `bytes` (a multiple of 1024, >= 1024; keep it small
 * for an L2-resident rate).  Bytes moved = workgroups * waves * iters * 1024.
 * `buf` and `sink` 16-byte aligned.  Asynchronous on stream.  Statuses:
 * FDLLM_ERR_ARG, FDLLM_ERR_ALIGN, FDLLM_ERR_HIP. */
int fdllm_probe_lds_dma(const void* buf, int64_t bytes, int32_t workgroups, int32_t waves, int32_t iters,
                        void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FDLLM_PROBE_H */
