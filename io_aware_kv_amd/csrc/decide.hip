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
//  * confidence_kernel: one workgroup per row of logits, 16-byte loads, an
//    online (max, sum of 2^(x - max)) over the whole vocabulary and the
//    argmax over the non-[MASK] ids (ties to the lowest id); the confidence
//    is that token's probability under the softmax over every id.
//  * accept_kernel: one lane per sequence walks its exploratory rows in
//    decoding order.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kConfThreads = 1024;
constexpr int kConfLoads = 4;        // 16-byte loads per thread per round

constexpr float kLog2e = 1.4426950408889634f;

struct Best {
    float m, s;      // running max of the logits in log2 units and sum of 2^(x - m)
    float bl;        // best non-[MASK] logit (as given: the argmax compares raw values)
    int bi;          // its id (lowest among equal logits)
};

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

template <typename T, int NL>
__global__ void __launch_bounds__(kConfThreads) confidence_kernel(const T* __restrict__ logits, int V, int mask_id,
                                                                  float thr, int32_t* __restrict__ pred,
                                                                  float* __restrict__ conf, uint8_t* __restrict__ over)
{
    const size_t row = blockIdx.x;
    const T* x = logits + row * (size_t)V;
    Best b{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    constexpr int PER = 16 / sizeof(T);                 // elements per 16-byte load
    const bool vec = (V % PER) == 0;
    const int tid = threadIdx.x;
    if (vec) {
        // kConfLoads 16-byte loads in flight per thread per round.  Per
        // element only the raw max and the exp2 sum: the round's max of the
        // raw logits gives the rescale (scaling by log2 e and rounding are
        // monotonic, so it bounds every scaled logit of the round), and a
        // lane keeps its best non-[MASK] logit with the raw data of the round
        // that holds it; after the row the first id holding it is found in
        // that copy (ids grow along a lane's walk, so the lowest id wins
        // ties).  The [MASK] id is left out of the argmax only, by a check
        // per load.
        int bround = -1;                                // round of the lane's best logit
        u32x4 keep[NL];                                 // ... and its raw logits
        for (int v0 = tid * PER; v0 < V; v0 += kConfThreads * PER * NL) {
            u32x4 raw[NL];
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const int v = min(v0 + u * kConfThreads * PER, V - PER);
                raw[u] = *(const u32x4*)(x + v);
            }
            float f[NL * PER];
            float rmax = -INFINITY;
            bool has_mask = false;
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const int base = v0 + u * kConfThreads * PER;
                const bool in = base < V;
                has_mask = has_mask || (in && mask_id >= base && mask_id < base + PER);
                const T* e = (const T*)&raw[u];
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    f[u * PER + k] = in ? to_f32(e[k]) : -INFINITY;
                    rmax = fmaxf(rmax, f[u * PER + k]);
                }
            }
            float amax = rmax;                          // best non-[MASK] logit of the round
            if (has_mask) {
                amax = -INFINITY;
#pragma unroll
                for (int u = 0; u < NL; ++u)
#pragma unroll
                    for (int k = 0; k < PER; ++k)
                        if (v0 + u * kConfThreads * PER + k != mask_id) amax = fmaxf(amax, f[u * PER + k]);
            }
            // a new best for this lane: remember the round (its id is found
            // after the row, from one re-read of that round)
            // (a round's first load is in range, so it holds a non-[MASK] id)
            const bool better = amax > b.bl || bround < 0;
            if (better) {
                b.bl = amax;
                bround = v0;
            }
#pragma unroll
            for (int u = 0; u < NL; ++u) keep[u] = better ? raw[u] : keep[u];
            if (rmax > -INFINITY) {
                const float rm = rmax * kLog2e;
                if (rm > b.m) {
                    b.s *= __builtin_amdgcn_exp2f(b.m - rm);
                    b.m = rm;
                }
                const float nm = -b.m;
#pragma unroll
                for (int k = 0; k < NL * PER; ++k) b.s += __builtin_amdgcn_exp2f(__builtin_fmaf(f[k], kLog2e, nm));
            }
        }
        if (bround >= 0) {
            // the first in-range non-[MASK] id of that round holding the best
            // logit (the round holds one when the best is -inf too)
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const int base = bround + u * kConfThreads * PER;
                if (base >= V) break;
                const T* e = (const T*)&keep[u];
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int id = base + k;
                    const float fv = to_f32(e[k]);
                    if (b.bi == 0x7fffffff && id != mask_id && (fv == b.bl || b.bl == -INFINITY)) b.bi = id;
                }
            }
        }
    } else {
        for (int v = tid; v < V; v += kConfThreads) take(b, to_f32(x[v]), v, mask_id);
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
    __shared__ Best sb[kConfThreads / 64];
    if ((tid & 63) == 0) sb[tid >> 6] = b;
    __syncthreads();
    if (tid == 0) {
        Best r = sb[0];
        for (int w = 1; w < kConfThreads / 64; ++w) r = merge(r, sb[w]);
        // probability of the best non-[MASK] id under the softmax over all ids
        const float c = (r.bi == 0x7fffffff || !(r.s > 0.f)) ? 0.f : __builtin_amdgcn_exp2f(r.bl * kLog2e - r.m) / r.s;
        pred[row] = r.bi == 0x7fffffff ? -1 : r.bi;
        conf[row] = c;
        if (over) over[row] = c >= thr ? 1 : 0;
    }
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
    if (dtype == 1)
        hipLaunchKernelGGL((confidence_kernel<bf16, kConfLoads>), dim3((unsigned)rows), dim3(kConfThreads), 0, s,
                           (const bf16*)logits, V, mask_id, thr, pred, conf, over);
    else
        hipLaunchKernelGGL((confidence_kernel<float, kConfLoads>), dim3((unsigned)rows), dim3(kConfThreads), 0, s,
                           (const float*)logits, V, mask_id, thr, pred, conf, over);
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
