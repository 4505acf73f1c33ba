// generic_kernels.hip -- scalar (non-MFMA) kernels of the fused KV-cache step.
//
// They serve the fp32 layers (where the tensor path would not keep fp32
// accuracy) and any head width the tiled MFMA kernels do not cover.  One
// workgroup per projected (row, head) and one per attended (sequence, query
// row, head); all arithmetic in fp32.
//
// The step follows the Flash-dLLM pages (jaehun.me review, "How It Works: A
// Concrete Example", Step 1: Draft / Step 1: Verification): gather only the
// query rows, project to q/k/v, rotate q and k by position, write k/v into the
// flat cache, attend over the whole cache under the view-visibility mask.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kGenThreads = 64;

// Does row j of sequence b own the cache write of its position?  (The first
// row at a position in query order owns it; later rows at that position are
// extra keys kept in the side buffer.)
__device__ bool owns_position(const int32_t* pos_b, int j)
{
    const int p = pos_b[j];
    for (int jj = 0; jj < j; ++jj)
        if (pos_b[jj] == p) return false;
    return true;
}

template <typename T>
__global__ void __launch_bounds__(kGenThreads) proj_generic_kernel(ProjArgs a)
{
    const int m = blockIdx.x;
    const int b = m / a.rows_per_seq;
    const int j = m - b * a.rows_per_seq;
    const int head = a.prefill ? a.H + (int)blockIdx.y : (int)blockIdx.y;
    if (!a.prefill && a.nq_seq && j >= a.nq_seq[b]) {
        // a padding row of a shorter sequence: no cache write; its q staging
        // row is cleared so the attention reads defined values
        if (head < a.H) {
            const int g = head / a.G, hl = head - g * a.G;
            float* qz = a.qbuf + (((size_t)b * a.Hkv + g) * a.q_max * a.G + (size_t)j * a.G + hl) * a.dh;
            for (int c = threadIdx.x; c < a.dh; c += kGenThreads) qz[c] = 0.f;
        }
        return;
    }
    const int xrow = a.prefill ? j : a.Q_idx[m];
    const int pos = a.prefill ? j : a.pos_ids[m];

    __shared__ int s_first;
    if (threadIdx.x == 0)
        s_first = a.prefill ? 1 : owns_position(a.pos_ids + (size_t)b * a.rows_per_seq, j);
    __syncthreads();

    const T* x = (const T*)a.X + ((size_t)b * a.x_rows + xrow) * a.d;
    const T* W = (const T*)a.W + (size_t)head * a.dh * a.d;
    const int half = a.dh / 2;
    const bool rotate = head < a.H + a.Hkv;  // q and k heads are rotated, v is not

    T* dst = nullptr;
    float* qdst = nullptr;   // q stays fp32: it is consumed on chip, never stored as T
    if (head < a.H) {
        const int g = head / a.G, hl = head - g * a.G;
        qdst = a.qbuf + (((size_t)b * a.Hkv + g) * a.q_max * a.G + (size_t)j * a.G + hl) * a.dh;
    } else {
        const bool isk = head < a.H + a.Hkv;
        const int g = head - a.H - (isk ? 0 : a.Hkv);
        if (s_first)
            dst = (T*)(isk ? a.Kc : a.Vc) + cache_row(a.map, b, g, pos, a.Hkv, a.N) * a.dh;
        else
            dst = (T*)(isk ? a.sideK : a.sideV) + (((size_t)b * a.Hkv + g) * a.q_max + j) * a.dh;
    }

    for (int c = threadIdx.x; c < half; c += kGenThreads) {
        const T* w0 = W + (size_t)c * a.d;
        const T* w1 = W + (size_t)(c + half) * a.d;
        float y0 = 0.f, y1 = 0.f;
        for (int k = 0; k < a.d; ++k) {
            const float xv = to_f32(x[k]);
            y0 = fmaf(to_f32(w0[k]), xv, y0);
            y1 = fmaf(to_f32(w1[k]), xv, y1);
        }
        if (rotate) {
            const float2 cs = a.rope[(size_t)pos * half + c];
            const float r0 = y0 * cs.x - y1 * cs.y;
            const float r1 = y1 * cs.x + y0 * cs.y;
            y0 = r0;
            y1 = r1;
        }
        if (qdst) {
            qdst[c] = y0;
            qdst[c + half] = y1;
        } else {
            dst[c] = from_f32<T>(y0);
            dst[c + half] = from_f32<T>(y1);
        }
    }
}

__device__ __forceinline__ float block_max64(float v, float* red)
{
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float block_sum64(float v)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// One workgroup (one wave) per (sequence b, query row i, head h).  Keys are
// walked in chunks of 64: indices 0..N-1 are cache positions, N..N+nq-1 are
// the step's own rows (only rows that do not own their position are keys
// there; an owning row is reached through its cache position).
template <typename T>
__global__ void __launch_bounds__(kGenThreads) attn_generic_kernel(AttnArgs a)
{
    const int bid = blockIdx.x;
    const int h = bid % a.H;
    const int i = (bid / a.H) % a.nq;
    const int b = bid / (a.H * a.nq);
    const int g = h / a.G, hl = h - g * a.G;
    const int t = threadIdx.x;
    const int nqb = a.nq_seq ? a.nq_seq[b] : a.nq;     // rows of this sequence
    const int L = a.seq_len ? a.seq_len[b] : a.N;      // its valid cache positions
    if (i >= nqb) {
        // padding row: no keys, zero output
        T* oz = (T*)a.O + (((size_t)b * a.nq + i) * a.H + h) * a.dh;
        for (int e = t; e < a.dh; e += kGenThreads) oz[e] = from_f32<T>(0.f);
        if (t == 0) a.LSE[((size_t)b * a.nq + i) * a.H + h] = -INFINITY;
        return;
    }

    extern __shared__ float smem[];
    float* sq = smem;                       // [dh]
    float* sp = sq + a.dh;                  // [64] probabilities of the chunk
    int* skey = (int*)(sp + kGenThreads);   // [64] key source of each chunk slot
    int* spos = skey + kGenThreads;         // [nq] positions of this sequence
    int* sown = spos + a.nq;                // [nq] first row at that position

    const int32_t* pos_b = a.pos_ids + (size_t)b * a.nq;
    for (int jj = t; jj < nqb; jj += kGenThreads) spos[jj] = pos_b[jj];
    __syncthreads();
    for (int jj = t; jj < nqb; jj += kGenThreads) {
        int f = jj;
        for (int q = 0; q < jj; ++q)
            if (spos[q] == spos[jj]) { f = q; break; }
        sown[jj] = f;
    }
    const float* qrow = a.qbuf + (((size_t)b * a.Hkv + g) * a.q_max * a.G + (size_t)i * a.G + hl) * a.dh;
    for (int e = t; e < a.dh; e += kGenThreads) sq[e] = qrow[e];
    __syncthreads();

    const T* Kp = (const T*)a.Kc;
    const T* Vp = (const T*)a.Vc;
    const T* SKb = (const T*)a.sideK + ((size_t)b * a.Hkv + g) * a.q_max * a.dh;
    const T* SVb = (const T*)a.sideV + ((size_t)b * a.Hkv + g) * a.q_max * a.dh;
    const uint8_t* vis_i = a.vis ? a.vis + ((size_t)b * a.nq + i) * a.nq : nullptr;

    float m = -INFINITY, l = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};   // dh <= 256: dims t, t+64, t+128, t+192
    const int nkeys = L + nqb;
    for (int base = 0; base < nkeys; base += kGenThreads) {
        const int kk = base + t;
        float s = -INFINITY;
        int src = -1;   // >= 0: cache position; < -1: side row -(src+2)
        if (kk < L) {
            int owner = -1;
            for (int q = 0; q < nqb; ++q)
                if (spos[q] == kk) { owner = q; break; }
            if (owner < 0 || !vis_i || vis_i[owner]) src = kk;
        } else if (kk < nkeys) {
            const int jj = kk - L;
            if (sown[jj] != jj && (!vis_i || vis_i[jj])) src = -(jj + 2);
        }
        if (src != -1) {
            const T* krow = src >= 0 ? Kp + cache_row(a.map, b, g, src, a.Hkv, a.N) * a.dh
                                     : SKb + (size_t)(-(src + 2)) * a.dh;
            float d = 0.f;
            for (int e = 0; e < a.dh; ++e) d = fmaf(sq[e], to_f32(krow[e]), d);
            s = d * a.scale_log2;
        }
        const float mc = block_max64(s, nullptr);
        const float m_new = fmaxf(m, mc);
        const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
        const float p = (s == -INFINITY) ? 0.f : exp2f(s - m_new);
        l = l * alpha + block_sum64(p);
        m = m_new;
        __syncthreads();
        sp[t] = p;
        skey[t] = src;
        __syncthreads();
        for (int r = 0; r < 4; ++r) acc[r] *= alpha;
        for (int c = 0; c < kGenThreads; ++c) {
            const float pc = sp[c];
            if (pc == 0.f) continue;
            const int sc = skey[c];
            const T* vrow = sc >= 0 ? Vp + cache_row(a.map, b, g, sc, a.Hkv, a.N) * a.dh
                                    : SVb + (size_t)(-(sc + 2)) * a.dh;
            for (int r = 0; r < 4; ++r) {
                const int e = t + r * kGenThreads;
                if (e < a.dh) acc[r] = fmaf(pc, to_f32(vrow[e]), acc[r]);
            }
        }
    }
    T* o = (T*)a.O + (((size_t)b * a.nq + i) * a.H + h) * a.dh;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int r = 0; r < 4; ++r) {
        const int e = t + r * kGenThreads;
        if (e < a.dh) o[e] = from_f32<T>(acc[r] * inv);
    }
    if (t == 0)
        a.LSE[((size_t)b * a.nq + i) * a.H + h] =
            l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

hipError_t launch_proj_generic(const ProjArgs& a, int dtype, hipStream_t s)
{
    const int M = a.B * a.rows_per_seq;
    const int heads = a.prefill ? 2 * a.Hkv : a.H + 2 * a.Hkv;
    if (M == 0) return hipSuccess;
    dim3 grid(M, heads);
    if (dtype == 0)
        hipLaunchKernelGGL(proj_generic_kernel<float>, grid, dim3(kGenThreads), 0, s, a);
    else
        hipLaunchKernelGGL(proj_generic_kernel<bf16>, grid, dim3(kGenThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s)
{
    const int blocks = a.B * a.nq * a.H;
    if (blocks == 0) return hipSuccess;
    const size_t shm = sizeof(float) * (a.dh + kGenThreads) + sizeof(int) * (kGenThreads + 2 * a.nq);
    if (dtype == 0)
        hipLaunchKernelGGL(attn_generic_kernel<float>, dim3(blocks), dim3(kGenThreads), shm, s, a);
    else
        hipLaunchKernelGGL(attn_generic_kernel<bf16>, dim3(blocks), dim3(kGenThreads), shm, s, a);
    return hipGetLastError();
}

}  // namespace fdllm
