// generic_kernels.hip -- scalar (non-MFMA) kernels of the fused KV-cache step.
//
// They serve the fp32 layers (where the tensor path would not keep fp32
// accuracy) and any head width the tiled MFMA kernels do not cover.  One
// workgroup per projected (row, head) and one per attended (sequence, kv
// head, block of query rows), rows staged in LDS with coalesced loads; all
// arithmetic in fp32.
//
// The step follows the Flash-dLLM pages (jaehun.me review, "How It Works: A
// Concrete Example", Step 1: Draft / Step 1: Verification): gather only the
// query rows, project to q/k/v, rotate q and k by position, write k/v into the
// flat cache, attend over the whole cache under the view-visibility mask.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kGenThreads = 256;

// One workgroup per projected (row, head): the row's hidden state is staged
// in LDS, each wave forms the dot products of its head columns with the
// lanes across d_model (coalesced weight rows) and a wave reduction, and the
// rotate-half pairs are applied from LDS.
template <typename T>
__global__ void __launch_bounds__(kGenThreads) proj_generic_kernel(ProjArgs a)
{
    extern __shared__ float smem[];
    float* sx = smem;                   // [d] the row's hidden state
    float* sy = sx + a.d;               // [dh] the head's projected values
    const int m = blockIdx.x;
    const int b = m / a.rows_per_seq;
    const int j = m - b * a.rows_per_seq;
    const int head = a.prefill ? a.H + (int)blockIdx.y : (int)blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (!a.prefill && a.nq_seq && j >= a.nq_seq[b]) {
        // a padding row of a shorter sequence: no cache write; its q staging
        // row is cleared so the attention reads defined values
        if (head < a.H) {
            const int g = head / a.G, hl = head - g * a.G;
            float* qz = a.qbuf + (((size_t)b * a.Hkv + g) * a.q_max * a.G + (size_t)j * a.G + hl) * a.dh;
            for (int c = tid; c < a.dh; c += kGenThreads) qz[c] = 0.f;
        }
        return;
    }
    // the first two d_model steps of this wave's first eight head columns are
    // loaded before the row is staged (they do not depend on it), so the
    // weights and the row arrive in one memory round trip
    const T* W = (const T*)a.W + (size_t)head * a.dh * a.d;
    constexpr int kCols = 8;
    constexpr int kPre = 2;
    float wpre[kPre][kCols];
#pragma unroll
    for (int i = 0; i < kPre; ++i)
#pragma unroll
        for (int u = 0; u < kCols; ++u) {
            const int c = min(wave * kCols + u, a.dh - 1), k = min(lane + 64 * i, a.d - 1);
            wpre[i][u] = to_f32(W[(size_t)c * a.d + k]);
        }
    const int xrow = a.prefill ? j : a.Q_idx[m];
    const int pos = a.prefill ? j : a.pos_ids[m];
    // this thread's rotary pair of the row's position, also ahead of the row
    const bool rot = head < a.H + a.Hkv;
    const float2 cs0 = rot && tid < a.dh / 2 ? a.rope[(size_t)pos * (a.dh / 2) + tid] : make_float2(1.f, 0.f);

    const T* x = (const T*)a.X + ((size_t)b * a.x_rows + xrow) * a.d;
    for (int k = tid; k < a.d; k += kGenThreads) sx[k] = to_f32(x[k]);
    // the row owns the cache write of its position unless an earlier row of
    // its sequence has the same one (the earlier rows are searched by all
    // threads at once; the barrier also publishes the staged row)
    int hit = 0;
    if (!a.prefill) {
        const int32_t* pos_b = a.pos_ids + (size_t)b * a.rows_per_seq;
        for (int jj = tid; jj < j; jj += kGenThreads) hit |= pos_b[jj] == pos;
    }
    const bool s_first = !__syncthreads_or(hit);

    // each wave takes eight head columns at a time, so every step of its
    // d_model loop has eight independent weight loads in flight
    for (int c0 = wave * kCols; c0 < a.dh; c0 += (kGenThreads / 64) * kCols) {
        float y[kCols];
        const T* w[kCols];
#pragma unroll
        for (int u = 0; u < kCols; ++u) {
            y[u] = 0.f;
            w[u] = W + (size_t)min(c0 + u, a.dh - 1) * a.d;
        }
        const bool first = c0 == wave * kCols;
        for (int k = lane, i = 0; k < a.d; k += 64, ++i) {
            float wv[kCols];
            if (first && i < kPre) {
#pragma unroll
                for (int u = 0; u < kCols; ++u) wv[u] = i == 0 ? wpre[0][u] : wpre[1][u];
            } else {
#pragma unroll
                for (int u = 0; u < kCols; ++u) wv[u] = to_f32(w[u][k]);
            }
            const float xv = sx[k];
#pragma unroll
            for (int u = 0; u < kCols; ++u) y[u] = fmaf(wv[u], xv, y[u]);
        }
        // the eight columns' reduction steps interleaved, so each step waits
        // once for its eight cross-lane reads (same sums, same order per column)
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
#pragma unroll
            for (int u = 0; u < kCols; ++u) y[u] += __shfl_xor(y[u], o);
#pragma unroll
        for (int u = 0; u < kCols; ++u)
            if (lane == 0 && c0 + u < a.dh) sy[c0 + u] = y[u];
    }
    __syncthreads();

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
    for (int c = tid; c < half; c += kGenThreads) {
        float y0 = sy[c], y1 = sy[c + half];
        if (rotate) {
            const float2 cs = c == tid ? cs0 : a.rope[(size_t)pos * half + c];
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

// One workgroup per (sequence b, kv head g, block of kGR of its nq * G query
// rows).  Keys are walked in chunks of kGK: indices 0..L-1 are cache
// positions, L.. are the step's rows that do not own their position (their
// k/v are in the side buffer; an owning row is reached through its cache
// position).  Each chunk's K and V rows are staged in LDS with coalesced
// loads; 16 threads per query row form its scores, then its online-softmax
// state and its share of the output dims.
constexpr int kGR = 16;     // query rows per workgroup
constexpr int kGK = 32;     // keys per chunk

size_t attn_generic_lds(int dh, int nq)
{
    return sizeof(float) * ((size_t)kGR * dh + (size_t)kGK * (dh + 1) + (size_t)kGK * dh + kGR * kGK) +
           sizeof(int) * (3 * (size_t)nq + kGK + 1);
}

template <typename T, int DU>
__global__ void __launch_bounds__(kGenThreads) attn_generic_kernel(AttnArgs a)
{
    extern __shared__ float smem[];
    const int dh = a.dh, nq = a.nq, G = a.G;
    float* sq = smem;                          // [kGR][dh] the block's q rows
    float* sk = sq + kGR * dh;                 // [kGK][dh + 1] the chunk's K rows (padded rows)
    float* sv = sk + kGK * (dh + 1);           // [kGK][dh] the chunk's V rows
    float* sp = sv + kGK * dh;                 // [kGR][kGK] probabilities
    int* spos = (int*)(sp + kGR * kGK);        // [nq] positions of this sequence
    int* sown = spos + nq;                     // [nq] first row at that position
    int* sdup = sown + nq;                     // [nq] rows that do not own their position
    int* sslot = sdup + nq;                    // [kGK] row owning each chunk position, or -1
    int* sndup = sslot + kGK;                  // [1] number of such rows

    const int rblocks = (a.R + kGR - 1) / kGR;
    const int rb = blockIdx.x % rblocks;
    const int bg = blockIdx.x / rblocks;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int tid = threadIdx.x;
    const int nqb = a.nq_seq ? a.nq_seq[b] : nq;       // rows of this sequence
    const int L = a.seq_len ? a.seq_len[b] : a.N;      // its valid cache positions

    // thread roles: query row rr of the block, key pair kq / kq + 16 for the
    // scores, dims dq + 16 u for the output
    const int rr = tid >> 4, kq = tid & 15;
    const int r = rb * kGR + rr;
    const int jrow = r / G;
    const bool live = r < a.R && jrow < nqb;
    const uint8_t* vis_i = (a.vis && live) ? a.vis + ((size_t)b * nq + jrow) * nq : nullptr;
    const T* Kp = (const T*)a.Kc;
    const T* Vp = (const T*)a.Vc;
    const T* SKb = (const T*)a.sideK + ((size_t)b * a.Hkv + g) * a.q_max * dh;
    const T* SVb = (const T*)a.sideV + ((size_t)b * a.Hkv + g) * a.q_max * dh;

    float m = -1.0e30f, l = 0.f;
    // dims kq + 16 u, u < DU (16 * DU >= dh); lanes past dh run on a clamped
    // dim and are never stored, so the loops carry no per-dim branches
    float acc[DU];
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[u] = 0.f;
    // a chunk's K and V rows move as 16-byte units (kEPU elements; a row is
    // dh / kEPU units), at most kUPT per thread; the next chunk is fetched
    // into registers while this one is worked on.  The unit coordinates
    // advance by fixed steps (no division per unit).
    constexpr int kEPU = 16 / (int)sizeof(T);
    constexpr int kUPT = 8;                      // kGK * 256 / (4 * kGenThreads): dh <= 256 in fp32
    const int U = dh / kEPU;
    const int nunits = kGK * U;
    const int k_first = tid / U, c_first = tid - k_first * U;
    const int k_step = kGenThreads / U, c_step = kGenThreads - k_step * U;
    u32x4 pku[kUPT], pvu[kUPT];
    // keys past L are the side buffer's rows; their count is known after the
    // ownership pass below (until then no fetch reaches past L)
    int nkeys = L;
    auto fetch = [&](int base) {
        int k = k_first, c = c_first;
#pragma unroll
        for (int t = 0; t < kUPT; ++t) {
            const int key = base + k;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (tid + t * kGenThreads < nunits) {
                if (key < L) {
                    const size_t row = cache_row(a.map, b, g, key, a.Hkv, a.N) * dh + c * kEPU;
                    kv = *(const u32x4*)(Kp + row);
                    vv = *(const u32x4*)(Vp + row);
                } else if (key < nkeys) {
                    const size_t row = (size_t)sdup[key - L] * dh + c * kEPU;
                    kv = *(const u32x4*)(SKb + row);
                    vv = *(const u32x4*)(SVb + row);
                }
            }
            pku[t] = kv;
            pvu[t] = vv;
            k += k_step;
            c += c_step;
            if (c >= U) { c -= U; ++k; }
        }
    };
    // the elements of a 16-byte unit as fp32
    auto unpack = [](u32x4 w, float* out) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                out[2 * i] = __uint_as_float(w[i] << 16);
                out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    };
    // the first chunk's K and V rows (cache positions only) are fetched
    // before the q rows and positions are staged, so both take one memory
    // round trip
    if (L >= kGK) fetch(0);


    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    for (int jj = tid; jj < nqb; jj += kGenThreads) spos[jj] = pos_b[jj];
    const float* qb = a.qbuf + ((size_t)b * a.Hkv + g) * a.q_max * G * dh;
    for (int e = tid; e < kGR * dh; e += kGenThreads) {
        const int rr = e / dh, d = e - rr * dh;
        const int r = rb * kGR + rr;
        sq[e] = (r < a.R && r / G < nqb) ? qb[(size_t)r * dh + d] : 0.f;
    }
    __syncthreads();
    for (int jj = tid; jj < nqb; jj += kGenThreads) {
        int f = jj;
        for (int q = 0; q < jj; ++q)
            if (spos[q] == spos[jj]) { f = q; break; }
        sown[jj] = f;
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        for (int jj = 0; jj < nqb; ++jj)
            if (sown[jj] != jj) sdup[n++] = jj;
        sndup[0] = n;
    }
    __syncthreads();
    const int ndup = sndup[0];
    nkeys = L + ndup;
    if (L < kGK) fetch(0);   // the first chunk reaches the side buffer
    for (int base = 0; base < nkeys; base += kGK) {
        // written positions of the chunk and their owner rows
        if (tid < kGK) sslot[tid] = -1;
        __syncthreads();
        for (int jj = tid; jj < nqb; jj += kGenThreads) {
            const int p = spos[jj];
            if (sown[jj] == jj && p >= base && p < base + kGK && p < L) sslot[p - base] = jj;
        }
        {
            int k = k_first, c = c_first;
#pragma unroll
            for (int t = 0; t < kUPT; ++t) {
                if (tid + t * kGenThreads < nunits) {
                    float kf[kEPU], vf[kEPU];
                    unpack(pku[t], kf);
                    unpack(pvu[t], vf);
#pragma unroll
                    for (int i = 0; i < kEPU; ++i) {
                        sk[k * (dh + 1) + c * kEPU + i] = kf[i];
                        sv[k * dh + c * kEPU + i] = vf[i];
                    }
                }
                k += k_step;
                c += c_step;
                if (c >= U) { c -= U; ++k; }
            }
        }
        if (base + kGK < nkeys) fetch(base + kGK);
        __syncthreads();
        float s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kq + 16 * h;
            const int key = base + k;
            bool keep = live && key < nkeys;
            if (keep && vis_i) {
                const int owner = key < L ? sslot[k] : sdup[key - L];
                if (owner >= 0 && !vis_i[owner]) keep = false;
            }
            float d0 = 0.f;
            if (keep) {
                // four independent partial sums, so the LDS reads of one
                // group of four dims are in flight together
                const float* qr = sq + rr * dh;
                const float* kr = sk + k * (dh + 1);
                float d1 = 0.f, d2 = 0.f, d3 = 0.f;
                int d = 0;
#pragma unroll 2
                for (; d + 4 <= dh; d += 4) {
                    d0 = fmaf(qr[d], kr[d], d0);
                    d1 = fmaf(qr[d + 1], kr[d + 1], d1);
                    d2 = fmaf(qr[d + 2], kr[d + 2], d2);
                    d3 = fmaf(qr[d + 3], kr[d + 3], d3);
                }
                for (; d < dh; ++d) d0 = fmaf(qr[d], kr[d], d0);
                d0 = (d0 + d1) + (d2 + d3);
            }
            s[h] = keep ? d0 * a.scale_log2 : -INFINITY;
        }
        // the row's max and sum over the 16 threads that hold it
        float mx = fmaxf(s[0], s[1]);
        for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        const float p0 = __builtin_amdgcn_exp2f(s[0] - m_new), p1 = __builtin_amdgcn_exp2f(s[1] - m_new);
        float ps = p0 + p1;
        for (int o = 8; o > 0; o >>= 1) ps += __shfl_xor(ps, o, 16);
        l = l * alpha + ps;
        m = m_new;
        sp[rr * kGK + kq] = p0;
        sp[rr * kGK + kq + 16] = p1;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < DU; ++u) acc[u] *= alpha;
#pragma unroll 4
        for (int k = 0; k < kGK; ++k) {
            const float pk = sp[rr * kGK + k];
            const float* vr = sv + k * dh;
#pragma unroll
            for (int u = 0; u < DU; ++u) acc[u] = fmaf(pk, vr[min(kq + 16 * u, dh - 1)], acc[u]);
        }
        __syncthreads();
    }
    if (r >= a.R || jrow >= nq) return;
    const int hl = r - jrow * G;
    const size_t orow = ((size_t)b * nq + jrow) * a.H + g * G + hl;
    T* o = (T*)a.O + orow * dh;
    const float inv = (live && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) {
        const int d = kq + 16 * u;
        if (d < dh) o[d] = from_f32<T>(acc[u] * inv);
    }
    if (kq == 0) a.LSE[orow] = (live && l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

template <auto K>
struct KernelTag { static constexpr auto value = K; };

}  // namespace

hipError_t launch_proj_generic(const ProjArgs& a, int dtype, hipStream_t s)
{
    const int M = a.B * a.rows_per_seq;
    const int heads = a.prefill ? 2 * a.Hkv : a.H + 2 * a.Hkv;
    if (M == 0) return hipSuccess;
    const size_t shm = sizeof(float) * ((size_t)a.d + a.dh);
    if (shm > 64 * 1024) return hipErrorInvalidValue;
    dim3 grid(M, heads);
    if (dtype == 0)
        hipLaunchKernelGGL(proj_generic_kernel<float>, grid, dim3(kGenThreads), shm, s, a);
    else
        hipLaunchKernelGGL(proj_generic_kernel<bf16>, grid, dim3(kGenThreads), shm, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s)
{
    const int blocks = a.B * a.Hkv * ((a.R + kGR - 1) / kGR);
    if (blocks == 0) return hipSuccess;
    if (a.dh > 256) return hipErrorInvalidValue;
    const size_t shm = attn_generic_lds(a.dh, a.nq);
    if (shm > 160 * 1024) return hipErrorInvalidValue;
    const int du = a.dh <= 32 ? 2 : a.dh <= 64 ? 4 : a.dh <= 128 ? 8 : 16;
    auto go = [&](auto kern) {
        (void)allow_full_lds<decltype(kern)::value>();
        (void)hipGetLastError();
        hipLaunchKernelGGL(decltype(kern)::value, dim3(blocks), dim3(kGenThreads), shm, s, a);
    };
    if (dtype == 0) {
        if (du == 2) go(KernelTag<attn_generic_kernel<float, 2>>{});
        else if (du == 4) go(KernelTag<attn_generic_kernel<float, 4>>{});
        else if (du == 8) go(KernelTag<attn_generic_kernel<float, 8>>{});
        else go(KernelTag<attn_generic_kernel<float, 16>>{});
    } else {
        if (du == 2) go(KernelTag<attn_generic_kernel<bf16, 2>>{});
        else if (du == 4) go(KernelTag<attn_generic_kernel<bf16, 4>>{});
        else if (du == 8) go(KernelTag<attn_generic_kernel<bf16, 8>>{});
        else go(KernelTag<attn_generic_kernel<bf16, 16>>{});
    }
    return hipGetLastError();
}

}  // namespace fdllm
