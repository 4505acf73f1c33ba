// decide.hip -- the Flash-Verify decisions on the device: per-row prediction
// and confidence from the logits, the confident / exploratory split, and the
// sequential acceptance of the verification pass.
//
// The pages (jaehun.me review, "Flash-Verify: Cache-Based Draft-Verification
// Parallel Decoding" and "How It Works: A Concrete Example", Step 1: Draft /
// Step 1: Verification): a masked position's draft prediction is the argmax of
// its distribution and its confidence the largest probability; positions with
// confidence >= eps are accepted at once (the confident set D), the others
// (the exploratory set S) are verified by a [MASK] view, and S is accepted in
// decoding order while the mask view agrees with the draft and its own
// confidence is >= gamma, up to the first failure.
//
//  * confidence_kernel: one or more workgroups per row of logits, 16-byte
//    loads, an online (max, sum of 2^(x - max)) over the whole vocabulary
//    and the argmax over the non-[MASK] ids (ties to the lowest id); the
//    confidence is that token's probability under the softmax over every id.
//    With fewer rows than CUs a row is cut into up to eight id ranges on
//    separate workgroups (each round of loads is a memory round trip the
//    next round waits for); the last of them to finish merges the ranges'
//    partial results.
//  * accept_kernel: one lane per sequence walks its exploratory rows in
//    decoding order.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kConfThreads = 1024;   // threads of a workgroup that takes a whole row
constexpr int kConfRangeThreads = 512;  // ... and of one that takes a range (two per CU)
constexpr int kConfLoads = 4;        // 16-byte loads per thread per round
constexpr int kConfMaxSplit = 8;     // id ranges per row at most
constexpr int kConfSlots = 8192;     // rows of the per-device meeting table

constexpr float kLog2e = 1.4426950408889634f;

struct Best {
    float m, s;      // running max of the logits in log2 units and sum of 2^(x - m)
    float bl;        // best non-[MASK] logit (as given: the argmax compares raw values)
    int bi;          // its id (lowest among equal logits)
};

// Where the id ranges of a split row meet: a count of finished ranges per row
// slot (back to zero once the row is merged) and each range's partial result.
// A call takes rows' worth of consecutive slots from a host-side ticket, so
// calls in flight together on one device meet in separate slots unless they
// hold more than kConfSlots split rows between them.
__device__ unsigned conf_count[kConfSlots];
__device__ Best conf_part[kConfSlots * kConfMaxSplit];

__device__ __forceinline__ void take(Best& b, float raw, int id, int mask_id)
{
    const float x = raw * kLog2e;
    if (x > b.m) {
        b.s = b.s * __builtin_amdgcn_exp2f(b.m - x) + 1.f;   // 2^-inf = 0 on the first id
        b.m = x;
    } else if (x > -INFINITY) {
        b.s += __builtin_amdgcn_exp2f(x - b.m);
    }
    if (id != mask_id && (raw > b.bl || (raw == b.bl && id < b.bi))) {
        b.bl = raw;
        b.bi = id;
    }
}

__device__ __forceinline__ Best merge(const Best& a, const Best& b)
{
    Best r;
    r.m = fmaxf(a.m, b.m);
    const float sa = a.s > 0.f ? a.s * __builtin_amdgcn_exp2f(a.m - r.m) : 0.f;
    const float sb = b.s > 0.f ? b.s * __builtin_amdgcn_exp2f(b.m - r.m) : 0.f;
    r.s = sa + sb;
    const bool takeb = b.bl > a.bl || (b.bl == a.bl && b.bi < a.bi);
    r.bl = takeb ? b.bl : a.bl;
    r.bi = takeb ? b.bi : a.bi;
    return r;
}

// A lane's state over the vector rounds: the running max, four partial sums
// of 2^(x - m) (four independent add chains), the best non-[MASK] logit and
// the first id of the round that holds it.
struct Acc {
    float m, s[4], bl;
    int bround;
};

// One round of a lane: NL 16-byte chunks, chunk u holding ids id0 + u * US ...
// Per element only the raw max and one fused multiply-add + exp2 + add: the
// round's raw max gives the rescale (scaling by log2 e and rounding are
// monotonic, so it bounds every scaled logit of the round), and the lane keeps
// the raw data of the round that holds its best non-[MASK] logit, so the
// first id holding it is found once after the range (ids grow along a lane's
// walk).  FULL: every chunk lies below hi (no range checks).
template <typename T, int NL, int US, bool FULL>
__device__ __forceinline__ void take_round(Acc& a, u32x4 (&keep)[NL], const u32x4 (&raw)[NL], int id0, int hi,
                                           int mask_id)
{
    constexpr int PER = 16 / sizeof(T);
    float f[NL * PER];
    float rmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const bool in = FULL || id0 + u * US < hi;
        const T* e = (const T*)&raw[u];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            f[u * PER + k] = in ? to_f32(e[k]) : -INFINITY;
            rmax = fmaxf(rmax, f[u * PER + k]);
        }
    }
    // the [MASK] id is left out of the argmax only
    float amax = rmax;
    const int d = mask_id - id0;
    if (d >= 0 && d < NL * US && (d & (US - 1)) < PER) {
        amax = -INFINITY;
#pragma unroll
        for (int u = 0; u < NL; ++u)
#pragma unroll
            for (int k = 0; k < PER; ++k)
                if (id0 + u * US + k != mask_id) amax = fmaxf(amax, f[u * PER + k]);
    }
    // a round's first chunk is in range, so it holds a non-[MASK] id
    const bool better = amax > a.bl || a.bround < 0;
    if (better) {
        a.bl = amax;
        a.bround = id0;
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) keep[u] = better ? raw[u] : keep[u];
    if (rmax > -INFINITY) {
        const float rm = rmax * kLog2e;
        if (rm > a.m) {
            const float c = __builtin_amdgcn_exp2f(a.m - rm);
#pragma unroll
            for (int j = 0; j < 4; ++j) a.s[j] *= c;
            a.m = rm;
        }
        const float nm = -a.m;
#pragma unroll
        for (int k = 0; k < NL * PER; ++k) a.s[k & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(f[k], kLog2e, nm));
    }
}

// grid: rows x nsplit workgroups of NT threads; workgroup (row, sp) takes ids
// [sp * rlen, min(V, (sp + 1) * rlen)) of its row; rlen is a multiple of
// NT * NL * 16 / sizeof(T) ids unless nsplit == 1.
template <typename T, int NL, int NT>
__global__ void __launch_bounds__(NT) confidence_kernel(const T* __restrict__ logits, int V, int mask_id,
                                                                  float thr, int32_t* __restrict__ pred,
                                                                  float* __restrict__ conf, uint8_t* __restrict__ over,
                                                                  int nsplit, int rlen, unsigned slot0)
{
    const size_t row = blockIdx.x / nsplit;
    const int sp = blockIdx.x - (int)row * nsplit;
    const int lo = sp * rlen, hi = min(V, lo + rlen);
    const T* x = logits + row * (size_t)V;
    Best b{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    constexpr int PER = 16 / sizeof(T);                 // elements per 16-byte load
    constexpr int US = NT * PER;                        // id stride between a lane's loads
    constexpr int RSTEP = US * NL;                      // ids per round of the workgroup
    const int tid = threadIdx.x;
    if ((V % PER) == 0) {
        Acc a{-INFINITY, {0.f, 0.f, 0.f, 0.f}, -INFINITY, -1};
        u32x4 keep[NL];
        const int nfull = hi > lo ? (hi - lo) / RSTEP : 0;
        int v0 = lo + tid * PER;
        for (int r = 0; r < nfull; ++r, v0 += RSTEP) {
            u32x4 raw[NL];
#pragma unroll
            for (int u = 0; u < NL; ++u) raw[u] = *(const u32x4*)(x + v0 + u * US);
            take_round<T, NL, US, true>(a, keep, raw, v0, hi, mask_id);
        }
        if (v0 < hi) {
            u32x4 raw[NL];
#pragma unroll
            for (int u = 0; u < NL; ++u) raw[u] = *(const u32x4*)(x + min(v0 + u * US, hi - PER));
            take_round<T, NL, US, false>(a, keep, raw, v0, hi, mask_id);
        }
        b.m = a.m;
        b.s = (a.s[0] + a.s[1]) + (a.s[2] + a.s[3]);
        b.bl = a.bl;
        if (a.bround >= 0) {
            // the first in-range non-[MASK] id of that round holding the best
            // logit (the round holds one when the best is -inf too)
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const T* e = (const T*)&keep[u];
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int id = a.bround + u * US + k;
                    const float fv = to_f32(e[k]);
                    if (b.bi == 0x7fffffff && id < hi && id != mask_id && (fv == b.bl || b.bl == -INFINITY))
                        b.bi = id;
                }
            }
        }
    } else {
        for (int v = lo + tid; v < hi; v += NT) take(b, to_f32(x[v]), v, mask_id);
    }
    // workgroup merge: lanes, then waves through LDS
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Best o;
        o.m = __shfl_xor(b.m, off);
        o.s = __shfl_xor(b.s, off);
        o.bl = __shfl_xor(b.bl, off);
        o.bi = __shfl_xor(b.bi, off);
        b = merge(b, o);
    }
    constexpr int NW = NT / 64;
    __shared__ Best sb[NW];
    if ((tid & 63) == 0) sb[tid >> 6] = b;
    __syncthreads();
    if (tid >= 64) return;
    // wave 0 merges the waves' results over a fixed tree of lanes (lanes past
    // the wave count hold the empty result)
    const Best none{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    Best r = tid < NW ? sb[tid] : none;
#pragma unroll
    for (int off = NW / 2; off >= 1; off >>= 1) {
        Best o;
        o.m = __shfl_xor(r.m, off);
        o.s = __shfl_xor(r.s, off);
        o.bl = __shfl_xor(r.bl, off);
        o.bi = __shfl_xor(r.bi, off);
        r = merge(r, o);
    }
    if (nsplit > 1) {
        // Publish this range's result; the last range of the row to arrive
        // merges all of them over a fixed tree of lanes, so the result does
        // not depend on the arrival order.  The partials are written and read only as
        // agent-scope atomics (coherent across the XCDs' L2s, no cached copy
        // to write back or invalidate), and the count is taken once those
        // stores have completed (vmcnt 0): the ordering an agent-scope
        // release gives, without its write-back of the whole L2 (measured
        // 1-3 us slower as a plain acquire-release count).
        const unsigned slot = (slot0 + (unsigned)row) % kConfSlots;
        if (tid == 0) {
            float* mine = (float*)&conf_part[slot * kConfMaxSplit + sp];
            __hip_atomic_store(mine + 0, r.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + 1, r.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(mine + 2, r.bl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store((int*)mine + 3, r.bi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        unsigned done = 0;
        if (tid == 0) done = __hip_atomic_fetch_add(&conf_count[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = __shfl(done, 0);
        if (done != (unsigned)nsplit - 1) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // lane k takes range k's partial
        r = none;
        if (tid < nsplit) {
            const float* q = (const float*)&conf_part[slot * kConfMaxSplit + tid];
            r.m = __hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            r.s = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            r.bl = __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            r.bi = __hip_atomic_load((const int*)q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int off = kConfMaxSplit / 2; off >= 1; off >>= 1) {
            Best o;
            o.m = __shfl_xor(r.m, off);
            o.s = __shfl_xor(r.s, off);
            o.bl = __shfl_xor(r.bl, off);
            o.bi = __shfl_xor(r.bi, off);
            r = merge(r, o);
        }
        if (tid == 0) __hip_atomic_store(&conf_count[slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid != 0) return;
    // probability of the best non-[MASK] id under the softmax over all ids
    const float c = (r.bi == 0x7fffffff || !(r.s > 0.f)) ? 0.f : __builtin_amdgcn_exp2f(r.bl * kLog2e - r.m) / r.s;
    pred[row] = r.bi == 0x7fffffff ? -1 : r.bi;
    conf[row] = c;
    if (over) over[row] = c >= thr ? 1 : 0;
}

__global__ void __launch_bounds__(64) accept_kernel(const int32_t* __restrict__ x_hat, const int32_t* __restrict__ x_tilde,
                                                    const float* __restrict__ c_tilde, int B, int S, float gamma,
                                                    int32_t* __restrict__ n_accept)
{
    const int b = blockIdx.x * 64 + threadIdx.x;
    if (b >= B) return;
    int n = 0;
    for (; n < S; ++n) {
        const size_t i = (size_t)b * S + n;
        if (!(x_tilde[i] == x_hat[i] && c_tilde[i] >= gamma)) break;
    }
    n_accept[b] = n;
}

}  // namespace

hipError_t launch_confidence(const void* logits, int dtype, int64_t rows, int V, int mask_id, float thr,
                             int32_t* pred, float* conf, uint8_t* over, hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    // With fewer rows than CUs, cut each row into up to eight ranges of
    // whole rounds of 512-thread workgroups (two run per CU), so that up to
    // two row-ranges run per CU at once; the ranges of a row meet in slots
    // taken from a ticket.  Otherwise one 1024-thread workgroup per row.
    const int esz = dtype == 1 ? 2 : 4;
    const int round_ids = kConfRangeThreads * kConfLoads * (16 / esz);
    const int rounds = (V + round_ids - 1) / round_ids;
    int nsplit = 1;
    if (rows < 256)
        while (nsplit < kConfMaxSplit && rows * nsplit * 2 <= 512 && nsplit * 2 <= rounds) nsplit *= 2;
    const dim3 grid((unsigned)(rows * nsplit));
    if (nsplit == 1) {
        if (dtype == 1)
            hipLaunchKernelGGL((confidence_kernel<bf16, kConfLoads, kConfThreads>), grid, dim3(kConfThreads), 0, s,
                               (const bf16*)logits, V, mask_id, thr, pred, conf, over, 1, V, 0u);
        else
            hipLaunchKernelGGL((confidence_kernel<float, kConfLoads, kConfThreads>), grid, dim3(kConfThreads), 0, s,
                               (const float*)logits, V, mask_id, thr, pred, conf, over, 1, V, 0u);
        return hipGetLastError();
    }
    const int rlen = ((rounds + nsplit - 1) / nsplit) * round_ids;
    static std::atomic<unsigned> ticket{0};
    const unsigned slot0 = ticket.fetch_add((unsigned)rows) % kConfSlots;
    if (dtype == 1)
        hipLaunchKernelGGL((confidence_kernel<bf16, kConfLoads, kConfRangeThreads>), grid, dim3(kConfRangeThreads),
                           0, s, (const bf16*)logits, V, mask_id, thr, pred, conf, over, nsplit, rlen, slot0);
    else
        hipLaunchKernelGGL((confidence_kernel<float, kConfLoads, kConfRangeThreads>), grid, dim3(kConfRangeThreads),
                           0, s, (const float*)logits, V, mask_id, thr, pred, conf, over, nsplit, rlen, slot0);
    return hipGetLastError();
}

hipError_t launch_accept(const int32_t* x_hat, const int32_t* x_tilde, const float* c_tilde, int B, int S,
                         float gamma, int32_t* n_accept, hipStream_t s)
{
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(accept_kernel, dim3((B + 63) / 64), dim3(64), 0, s, x_hat, x_tilde, c_tilde, B, S, gamma,
                       n_accept);
    return hipGetLastError();
}

}  // namespace fdllm
