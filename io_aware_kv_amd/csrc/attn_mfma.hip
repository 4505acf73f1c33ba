// attn_mfma.hip -- split-N online-softmax attention of the query rows over the
// whole flat KV cache, with the verification-view mask, on bf16 MFMA (gfx950,
// head width 128).
//
// Flash-dLLM attends the query set over the full cache on chip (jaehun.me
// review, "How It Works: A Concrete Example", Step 1: Draft; alanhou.org,
// "Core Mechanism" item 1), and in the verification pass the draft view and
// the [MASK] view share positions but cannot see each other (jaehun.me,
// "Flash-Verify", Fig. 2).  The pages' kernel targets the SRAM and tensor
// cores of another GPU; this one is laid out for CDNA4:
//
//  * one workgroup per (sequence, kv head, cache split): all nq * H/Hkv query
//    rows that share a kv head are packed as the MFMA N dimension, so every
//    K/V byte is read from HBM once per step;
//  * one producer wave streams K/V tiles straight into a ring of LDS stages
//    with global_load_lds (16 B per lane, no registers), keeping up to three
//    tiles (~96 KB) in flight per CU; it waits on its own vmcnt and releases
//    each stage with a barrier.  The consumer waves never issue global loads
//    in the loop, they only read LDS and run MFMAs;
//  * LDS rows are 256 B with their 16 B chunks XOR-swizzled by the row index,
//    which makes both fragment read patterns below bank-conflict free;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 leaves each lane with one query
//    row, so the row max needs two cross-lane steps and the rescale of the
//    output accumulators is lane-local; q enters as bf16 hi + lo parts so the
//    scores keep q's fp32 accumulation precision;
//  * O^T += V^T P^T takes V^T fragments from the row-major tile with
//    ds_read_b64_tr_b16 (gfx950 transpose read) and P^T from the score
//    registers, so P never goes through LDS;
//  * consumer waves split the query rows and the keys of a tile; key-split
//    waves merge their softmax states through LDS at the end;
//  * with several cache splits, each writes its (max, sum, output) partial
//    state and a small second kernel merges them into O and LSE (a kernel
//    boundary is far cheaper than a device-scope fence per workgroup).
//
// Key set of query row i (same definition as the CPU oracle): every cache
// position not written by this step, plus each new row j that i may see.  A
// position written by its first row j is reached through the cache (the
// projection kernel stored it there) and gated by vis[i][j]; later rows at a
// shared position live in the side buffer and are attended as extra tiles.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kDH = 128;
constexpr int kRowB = kDH * 2;   // bytes of one K or V row

typedef __bf16 bf16x4g __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16x4g lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

template <int RG, int NWR, int NWK>
struct AttnCfg {
    static constexpr int NC = NWR * NWK;            // consumer waves
    static constexpr int NT = (NC + 1) * 64;        // + one producer wave
    static constexpr int KW = 32;                   // keys per consumer wave per tile
    static constexpr int TK = KW * NWK;             // keys per tile
    static constexpr int STAGE = TK * 2 * kRowB;    // K rows then V rows
    static constexpr int NS = (128 * 1024) / STAGE; // ring of 128 KB
    static constexpr int DMA = STAGE / 1024;        // producer instructions per stage
    static constexpr int MERGE = (NWK / 2) * NWR * RG * 64 * (32 + 2) * 4;
    static constexpr int SCRATCH = NS * STAGE > MERGE ? NS * STAGE : MERGE;
    static_assert(NS >= 2 && NS * STAGE == 128 * 1024, "stage ring");
};

// Producer wait: stage `it` has landed once at most `younger` * DMA of this
// wave's loads are outstanding; then release the stage to the consumers.
template <int DMA>
__device__ __forceinline__ void producer_sync(int younger)
{
#define FDLLM_PSYNC(N) asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory")
    const int n = younger * DMA;
    if (n >= 63) FDLLM_PSYNC(63);
    else if (n >= 48) FDLLM_PSYNC(48);
    else if (n >= 32) FDLLM_PSYNC(32);
    else if (n >= 16) FDLLM_PSYNC(16);
    else FDLLM_PSYNC(0);
#undef FDLLM_PSYNC
}

// Consumer side of the same barrier: its LDS reads of the previous stage have
// returned (so the producer may overwrite that stage).
__device__ __forceinline__ void consumer_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 read_vt_frag(const unsigned char* p0, const unsigned char* p1)
{
    const bf16x4g a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4g b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// One stage of the ring: TK cache rows from `base` (or side-buffer rows
// sDup[base ...] for the duplicate tiles), K then V, as 1 KB DMA blocks of 4
// rows; chunk c of row r lands in slot c ^ (r & 15).
template <int TK, int DMA>
__device__ __forceinline__ void issue_stage(unsigned char* st, bool dup, int base, int k1, int ndup,
                                            const int* sDup, const unsigned char* Kg, const unsigned char* Vg,
                                            const unsigned char* SKg, const unsigned char* SVg, int lane)
{
    const int srow = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int i = 0; i < DMA / 2; ++i) {
        const int row = 4 * i + srow;
        const int chunk = slot ^ (row & 15);
        size_t src;
        if (!dup) {
            const int key = min(base + row, k1 - 1);   // rows past the split are masked later
            src = (size_t)key * kRowB + chunk * 16;
        } else {
            const int kk = base + row;
            const int j = kk < ndup ? sDup[kk] : sDup[0];
            src = (size_t)j * kRowB + chunk * 16;
        }
        __builtin_amdgcn_global_load_lds((glb_void*)((dup ? SKg : Kg) + src), (lds_void*)(st + i * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void*)((dup ? SVg : Vg) + src),
                                         (lds_void*)(st + TK * kRowB + i * 1024), 16, 0, 0);
    }
}

template <int RG, int NWR, int NWK>
__global__ void __launch_bounds__((NWR * NWK + 1) * 64)
attn_mfma_kernel(AttnArgs a)
{
    using C = AttnCfg<RG, NWR, NWK>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int kps = a.keys_per_split;
    const int nq = a.nq;
    const int VW = (nq + 31) >> 5;                  // 32-bit words per visibility row
    int16_t* sSlot = (int16_t*)(smem + C::SCRATCH); // [kps] owner row of written positions, -1
    uint32_t* sVis = (uint32_t*)(smem + C::SCRATCH + 2 * ((kps + 1) & ~1));   // [nq][VW]
    int* sPos = (int*)(sVis + (size_t)nq * VW);     // [nq]
    int* sOwn = sPos + nq;                          // [nq] 1 if the row owns its position
    int* sDup = sOwn + nq;                          // [nq] rows that do not own their position
    int* sMisc = sDup + nq;                         // [0] dup count, [2..] tile flags

    const int total = a.B * a.Hkv * a.splits;
    const int logical = xcd_remap(blockIdx.x, total);
    if (logical < 0) return;
    const int bg = logical / a.splits;
    const int split = logical - bg * a.splits;
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    const int k0 = split * kps;
    const int k1 = min(a.N, k0 + kps);
    const int nkeys = k1 - k0;
    const int n_main = (nkeys + C::TK - 1) / C::TK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform in an SGPR, so branches on it stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int G = a.G;
    int* sTileFlag = sMisc + 2;

    // ---- per-sequence bookkeeping: positions, ownership, duplicates, gating
    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    for (int j = tid; j < nq; j += C::NT) sPos[j] = pos_b[j];
    if (a.vis) {
        for (int k = tid; k < nkeys; k += C::NT) sSlot[k] = -1;
        for (int t = tid; t < n_main; t += C::NT) sTileFlag[t] = 0;
        const uint8_t* vb = a.vis + (size_t)b * nq * nq;
        for (int w = tid; w < nq * VW; w += C::NT) {
            const int i = w / VW, j0 = (w - i * VW) * 32;
            uint32_t bits = 0;
            for (int j = j0; j < min(nq, j0 + 32); ++j)
                bits |= (vb[(size_t)i * nq + j] ? 1u : 0u) << (j - j0);
            sVis[w] = bits;
        }
    }
    __syncthreads();
    for (int j = tid; j < nq; j += C::NT) {
        int own = 1;
        for (int q = 0; q < j; ++q)
            if (sPos[q] == sPos[j]) { own = 0; break; }
        sOwn[j] = own;
        const int p = sPos[j];
        if (own && a.vis && p >= k0 && p < k1) {
            sSlot[p - k0] = (int16_t)j;
            sTileFlag[(p - k0) / C::TK] = 1;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        for (int j = 0; j < nq; ++j)
            if (!sOwn[j]) sDup[n++] = j;
        sMisc[0] = n;
    }
    __syncthreads();
    const int ndup = (split == 0) ? sMisc[0] : 0;
    const int ntot = n_main + (ndup + C::TK - 1) / C::TK;

    const size_t cache_off = (size_t)bg * a.N * kDH;
    const unsigned char* Kg = (const unsigned char*)((const bf16*)a.Kc + cache_off);
    const unsigned char* Vg = (const unsigned char*)((const bf16*)a.Vc + cache_off);
    const unsigned char* SKg = (const unsigned char*)((const bf16*)a.sideK + (size_t)bg * a.q_max * kDH);
    const unsigned char* SVg = (const unsigned char*)((const bf16*)a.sideV + (size_t)bg * a.q_max * kDH);

    float m_run[RG], l_run[RG];
    f32x4 o[RG][8];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        m_run[rg] = -INFINITY;
        l_run[rg] = 0.f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int wk = wave % NWK, wr = wave / NWK;    // consumer coordinates

    if (wave == C::NC) {
        // ================= producer wave: K/V tiles -> LDS ring =================
        int issued = 0;
        for (; issued < min(C::NS - 1, ntot); ++issued) {
            const bool dup = issued >= n_main;
            issue_stage<C::TK, C::DMA>(smem + (issued % C::NS) * C::STAGE, dup,
                                       dup ? (issued - n_main) * C::TK : k0 + issued * C::TK, k1, ndup,
                                       sDup, Kg, Vg, SKg, SVg, lane);
        }
        for (int t = 0; t < ntot; ++t) {
            producer_sync<C::DMA>(issued - t - 1);
            if (issued < ntot) {
                const bool dup = issued >= n_main;
                issue_stage<C::TK, C::DMA>(smem + (issued % C::NS) * C::STAGE, dup,
                                           dup ? (issued - n_main) * C::TK : k0 + issued * C::TK, k1, ndup,
                                           sDup, Kg, Vg, SKg, SVg, lane);
                ++issued;
            }
        }
    } else {
        // ================= consumer waves =================
        // query fragments: lane holds row (wr*RG + rg)*16 + lr, dims 32c + 8lg .. +7,
        // split into bf16 hi + lo so the scores keep q's fp32 precision
        const float* qbase = a.qbuf + (size_t)bg * a.q_max * G * kDH;
        bf16x8 qh[RG][4], ql[RG][4];
        int qrow[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = (wr * RG + rg) * 16 + lr;
            qrow[rg] = row < a.R ? row / G : -1;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float x[8];
                if (row < a.R) {
                    // scores come out of the MFMA already in log2 units
                    const f32x4 u = *(const f32x4*)(qbase + (size_t)row * kDH + c * 32 + lg * 8) * a.scale_log2;
                    const f32x4 v = *(const f32x4*)(qbase + (size_t)row * kDH + c * 32 + lg * 8 + 4) * a.scale_log2;
                    x[0] = u[0]; x[1] = u[1]; x[2] = u[2]; x[3] = u[3];
                    x[4] = v[0]; x[5] = v[1]; x[6] = v[2]; x[7] = v[3];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bf16 hi = (bf16)x[e];
                    qh[rg][c][e] = hi;
                    ql[rg][c][e] = (bf16)(x[e] - (float)hi);
                }
            }
        }

        for (int it = 0; it < ntot; ++it) {
            consumer_sync();
            const unsigned char* st = smem + (it % C::NS) * C::STAGE;
            const unsigned char* sK = st;
            const unsigned char* sV = st + C::TK * kRowB;
            const bool dup = it >= n_main;

            // ---- S^T = K Q^T for this wave's 32 keys
            f32x4 sc[RG][2];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                sc[rg][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                sc[rg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // all K fragments of the wave's 32 keys first (their LDS reads overlap),
            // then the MFMAs; row groups past R run on zero q and are discarded
            bf16x8 kf[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = wk * C::KW + kb * 16 + lr;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kf[kb][c] = *(const bf16x8*)(sK + row * kRowB + (((c * 4 + lg) ^ lr) << 4));
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg) {
                        sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][c], qh[rg][c], sc[rg][kb], 0, 0, 0);
                        sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][c], ql[rg][c], sc[rg][kb], 0, 0, 0);
                    }

            // ---- scale, mask, online softmax (lane: row lr, keys kb*16 + 4lg + i)
            const int kl0 = wk * C::KW + lg * 4;                     // key within the tile
            const bool gate = dup || (a.vis && sTileFlag[it]);
            const int tbase = dup ? (it - n_main) * C::TK : k0 + it * C::TK;
            // keys past the split (or past the duplicate list) are masked; a
            // gated key (written this step, or a duplicate row) needs the
            // query's visibility bit for its owning row
            const int kend = dup ? ndup : k1;
            bool keep_k[2][4];
            int owner_k[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = tbase + kl0 + kb * 16 + i;
                    keep_k[kb][i] = key < kend;
                    owner_k[kb][i] = -1;
                }
            if (gate) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = tbase + kl0 + kb * 16 + i;
                        if (keep_k[kb][i]) owner_k[kb][i] = dup ? sDup[key] : sSlot[key - k0];
                        if (dup && !a.vis) owner_k[kb][i] = -1;
                    }
            }
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float s = sc[rg][kb][i];
                        bool keep = keep_k[kb][i];
                        if (gate) {
                            const int j = owner_k[kb][i];
                            const bool seen = qrow[rg] >= 0 &&
                                              ((sVis[qrow[rg] * VW + (max(j, 0) >> 5)] >> (max(j, 0) & 31)) & 1u);
                            keep = keep && (j < 0 || seen);
                        }
                        s = keep ? s : -INFINITY;
                        sc[rg][kb][i] = s;
                        mx = fmaxf(mx, s);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                // lazy rescale: a row's exponentials stay relative to a
                // reference max that only moves when the row's max exceeds it
                // by more than 2^8, so p <= 256 and the output accumulators are
                // rescaled only a few times per split.  The decision is per
                // row (each row's result depends on its own scores only); the
                // whole block is skipped when no row of the wave grows.
                const bool grow = mx > m_run[rg] + 8.f;
                if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                    if (grow) {
                        const float alpha = (m_run[rg] == -INFINITY) ? 0.f : exp2f(m_run[rg] - mx);
                        l_run[rg] *= alpha;
#pragma unroll
                        for (int db = 0; db < 8; ++db) o[rg][db] *= alpha;
                        m_run[rg] = mx;
                    }
                }
                const float msub = (m_run[rg] == -INFINITY) ? 0.f : m_run[rg];
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float p = exp2f(sc[rg][kb][i] - msub);   // exp2(-inf) = 0
                        sc[rg][kb][i] = p;
                        lsum += p;
                    }
                l_run[rg] += lsum;
            }

            // ---- O^T += V^T P^T over the wave's 32 keys
            bf16x8 pf[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pf[rg][i] = (bf16)sc[rg][0][i];
                    pf[rg][4 + i] = (bf16)sc[rg][1][i];
                }
            const int rowA = wk * C::KW + 4 * lg + (lr >> 2);
            const int rowB = rowA + 16;
            bf16x8 vf[8];
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const int chunk = 2 * db + ((lr & 3) >> 1);
                const int half = (lr & 1) << 3;
                const unsigned char* pA = sV + rowA * kRowB + ((chunk ^ (rowA & 15)) << 4) + half;
                const unsigned char* pB = sV + rowB * kRowB + ((chunk ^ (rowB & 15)) << 4) + half;
                vf[db] = read_vt_frag(pA, pB);
            }
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
                    o[rg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf[rg], o[rg][db], 0, 0, 0);
        }
        // per-lane sums -> row sums (row lr is spread over the 4 lane groups)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            l_run[rg] += __shfl_xor(l_run[rg], 16);
            l_run[rg] += __shfl_xor(l_run[rg], 32);
        }
    }
    __syncthreads();   // the LDS ring is free from here on

    // ---- merge the key-split consumer waves through LDS (tree over wk)
    const bool consumer = wave < C::NC;
    if (NWK > 1) {
        float* scr = (float*)smem;
        constexpr int SLOT = RG * 64 * (32 + 2);
#pragma unroll
        for (int stride = NWK / 2; stride >= 1; stride /= 2) {
            if (consumer && wk >= stride && wk < 2 * stride) {
                float* dst = scr + (size_t)(wr * (NWK / 2) + (wk - stride)) * SLOT;
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
                    for (int db = 0; db < 8; ++db)
                        *(f32x4*)(dst + ((rg * 8 + db) * 64 + lane) * 4) = o[rg][db];
                    dst[RG * 64 * 32 + (rg * 64 + lane) * 2 + 0] = m_run[rg];
                    dst[RG * 64 * 32 + (rg * 64 + lane) * 2 + 1] = l_run[rg];
                }
            }
            __syncthreads();
            if (consumer && wk < stride) {
                const float* src = scr + (size_t)(wr * (NWK / 2) + wk) * SLOT;
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    const float mb = src[RG * 64 * 32 + (rg * 64 + lane) * 2 + 0];
                    const float lb = src[RG * 64 * 32 + (rg * 64 + lane) * 2 + 1];
                    const float mn = fmaxf(m_run[rg], mb);
                    const float fa = (m_run[rg] == -INFINITY) ? 0.f : exp2f(m_run[rg] - mn);
                    const float fb = (mb == -INFINITY) ? 0.f : exp2f(mb - mn);
#pragma unroll
                    for (int db = 0; db < 8; ++db) {
                        const f32x4 ob = *(const f32x4*)(src + ((rg * 8 + db) * 64 + lane) * 4);
                        o[rg][db] = o[rg][db] * fa + ob * fb;
                    }
                    l_run[rg] = l_run[rg] * fa + lb * fb;
                    m_run[rg] = mn;
                }
            }
            __syncthreads();
        }
    }

    // ---- outputs: lane holds row (wr*RG + rg)*16 + lr, dims db*16 + 4lg + i
    const float kLn2 = 0.69314718055994531f;
    const bool writer = consumer && wk == 0;
    if (a.splits == 1) {
        if (writer) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const int row = (wr * RG + rg) * 16 + lr;
                if (row >= a.R) continue;
                const int j = row / G, hl = row - j * G;
                const size_t orow = ((size_t)b * nq + j) * a.H + g * G + hl;
                const float inv = l_run[rg] > 0.f ? 1.f / l_run[rg] : 0.f;
                bf16* op = (bf16*)a.O + orow * kDH;
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    bf16x4v v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[rg][db][i] * inv);
                    *(bf16x4v*)(op + db * 16 + lg * 4) = v;
                }
                if (lg == 0)
                    a.LSE[orow] = l_run[rg] > 0.f ? (m_run[rg] + log2f(l_run[rg])) * kLn2 : -INFINITY;
            }
        }
        return;
    }

    // publish this split's partial state (max in log2 units, sum, unnormalised
    // output); the combine kernel merges the splits after this launch ends
    if (writer) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = (wr * RG + rg) * 16 + lr;
            if (row >= a.R) continue;
            const size_t prow = ((size_t)bg * a.splits + split) * a.Rpad + row;
            float* pp = a.apart + prow * kDH;
#pragma unroll
            for (int db = 0; db < 8; ++db) *(f32x4*)(pp + db * 16 + lg * 4) = o[rg][db];
            if (lg == 0) {
                a.aml[prow * 2 + 0] = m_run[rg];
                a.aml[prow * 2 + 1] = l_run[rg];
            }
        }
    }
}

// Merge of the cache splits: O = sum_s 2^(m_s - M) acc_s / L and
// LSE = (M + log2 L) ln 2 with M = max_s m_s, L = sum_s 2^(m_s - M) l_s.
// One thread per (query row, 4 output dims); 8 rows per workgroup.
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a)
{
    const int rows_per_wg = 8;
    const int wgs_per_bg = (a.R + rows_per_wg - 1) / rows_per_wg;
    const int bg = blockIdx.x / wgs_per_bg;
    const int row = (blockIdx.x - bg * wgs_per_bg) * rows_per_wg + (threadIdx.x >> 5);
    const int d4 = threadIdx.x & 31;
    if (row >= a.R) return;
    const int S = a.splits;
    const size_t pbase = (size_t)bg * S * a.Rpad + row;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.aml[(pbase + (size_t)s * a.Rpad) * 2]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != -INFINITY) {
#pragma unroll 4
        for (int s = 0; s < S; ++s) {
            const size_t pr = pbase + (size_t)s * a.Rpad;
            const float ms = a.aml[pr * 2];
            const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);
            L += a.aml[pr * 2 + 1] * w;
            acc += *(const f32x4*)(a.apart + pr * kDH + d4 * 4) * w;
        }
    }
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int j = row / a.G, hl = row - j * a.G;
    const size_t orow = ((size_t)b * a.nq + j) * a.H + g * a.G + hl;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    bf16x4v v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[i] * inv);
    *(bf16x4v*)((bf16*)a.O + orow * kDH + d4 * 4) = v;
    if (d4 == 0) a.LSE[orow] = L > 0.f ? (mx + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

template <int RG, int NWR, int NWK>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s)
{
    using C = AttnCfg<RG, NWR, NWK>;
    const int VW = (a.nq + 31) / 32;
    const int tiles = (a.keys_per_split + C::TK - 1) / C::TK;
    const size_t book = 2 * (size_t)((a.keys_per_split + 1) & ~1) + 4 * (size_t)a.nq * VW +
                        4 * (3 * (size_t)a.nq + 2 + tiles + 2);
    if (C::SCRATCH + book > 160 * 1024) return hipErrorInvalidValue;
    const size_t shm = C::SCRATCH + book;
    const int total = a.B * a.Hkv * a.splits;
    const int grid = ((total + 7) / 8) * 8;
    auto kern = attn_mfma_kernel<RG, NWR, NWK>;
    // raise the dynamic LDS limit; a refusal shows up as a launch error below
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), shm, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const int cgrid = a.B * a.Hkv * ((a.R + 7) / 8);
    hipLaunchKernelGGL(attn_combine_kernel, dim3(cgrid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Keys per tile of the configuration chosen for R query rows per kv head.
int attn_mfma_tile_keys(int R)
{
    const int r16 = (R + 15) / 16;
    return r16 <= 9 ? 64 : 32;
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s)
{
    if (a.B * a.Hkv * a.splits == 0 || a.R == 0) return hipSuccess;
    const int r16 = (a.R + 15) / 16;
    if (r16 <= 1) return launch_cfg<1, 1, 2>(a, s);
    if (r16 <= 2) return launch_cfg<1, 2, 2>(a, s);
    if (r16 <= 4) return launch_cfg<1, 4, 2>(a, s);
    if (r16 <= 6) return launch_cfg<2, 3, 2>(a, s);
    if (r16 <= 9) return launch_cfg<3, 3, 2>(a, s);
    if (r16 <= 12) return launch_cfg<2, 6, 1>(a, s);
    if (r16 <= 14) return launch_cfg<2, 7, 1>(a, s);
    if (r16 <= 18) return launch_cfg<3, 6, 1>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace fdllm
