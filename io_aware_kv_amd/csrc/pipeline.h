// pipeline.h -- the producer/consumer LDS ring used by the HIP kernels.
//
// One producer wave per workgroup streams tiles from global memory straight
// into a ring of LDS stages with global_load_lds (16 B per lane, no register
// staging) and releases each stage with a barrier once its own vmcnt shows
// the stage has landed; the consumer waves only read LDS.  Keeping all DMA in
// one wave lets that wave count its outstanding loads exactly (the compiler's
// own tracking of LDS DMA would wait for all of them), so several stages
// stay in flight while the consumers work.
#pragma once

#include "fdllm_common.h"

namespace fdllm {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// 16 B per lane from `src` into LDS at `dst` + lane * 16 (dst wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* dst)
{
    __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)dst, 16, 0, 0);
}

// Producer side: wait until at most `outstanding` of this wave's loads are in
// flight (rounded down to a supported bound, which only waits longer), then
// join the barrier that hands the oldest stage to the consumers.
__device__ __forceinline__ void ring_producer_sync(int outstanding)
{
#define FDLLM_PSYNC(N) asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory")
    if (outstanding >= 63) FDLLM_PSYNC(63);
    else if (outstanding >= 48) FDLLM_PSYNC(48);
    else if (outstanding >= 32) FDLLM_PSYNC(32);
    else if (outstanding >= 24) FDLLM_PSYNC(24);
    else if (outstanding >= 16) FDLLM_PSYNC(16);
    else if (outstanding >= 8) FDLLM_PSYNC(8);
    else FDLLM_PSYNC(0);
#undef FDLLM_PSYNC
}

// Exact form for a ring whose stages each take DMAP of this wave's loads:
// stage t has landed once at most `younger` * DMAP loads are in flight (loads
// complete in order and the counter saturates at 63).  Y is the largest
// number of younger stages the ring can hold.
template <int N>
__device__ __forceinline__ void ring_release()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int DMAP, int Y>
__device__ __forceinline__ void ring_producer_wait(int younger)
{
    if constexpr (Y <= 0) {
        ring_release<0>();
    } else {
        if (younger >= Y) ring_release<(Y * DMAP > 63 ? 63 : Y * DMAP)>();
        else ring_producer_wait<DMAP, Y - 1>(younger);
    }
}

// Consumer side of the same barrier: its LDS reads of the previous stage have
// returned, so the producer may overwrite that stage after the barrier.
__device__ __forceinline__ void ring_consumer_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace fdllm
