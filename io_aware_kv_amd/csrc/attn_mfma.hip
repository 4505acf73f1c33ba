// attn_mfma.hip -- split-N online-softmax attention of the query rows over the
// whole flat KV cache, with the verification-view mask, on bf16 MFMA (gfx950,
// head width 128).
//
// Flash-dLLM attends the query set over the full cache on chip (jaehun.me
// review, "How It Works: A Concrete Example", Step 1: Draft; alanhou.org,
// "Core Mechanism" item 1), and in the verification pass the draft view and
// the [MASK] view share positions but cannot see each other (jaehun.me,
// "Flash-Verify", Fig. 2).  The pages' kernel targets SRAM and tensor cores of
// another GPU; this one is laid out for CDNA4:
//
//  * one workgroup per (sequence, kv head, cache split): all nq * H/Hkv query
//    rows that share a kv head are packed as the MFMA N dimension, so every
//    K/V byte is read from HBM exactly once per step;
//  * K and V tiles are streamed with coalesced 16 B loads into registers
//    (prefetch of the next tile overlaps the current tile's math), then
//    stored row-major into padded LDS;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 leaves each lane with one query
//    row, so the row max needs two cross-lane steps and the rescale of the
//    output accumulators is lane-local;
//  * O^T += V^T P^T takes V^T fragments straight from the row-major LDS tile
//    with ds_read_b64_tr_b16 (gfx950 transpose read) and P^T from the score
//    registers, so P never touches LDS;
//  * waves split either the keys of a tile (few query rows; partial softmax
//    states are merged through LDS at the end) or the query rows (many rows);
//  * the last workgroup of a (sequence, kv head) to finish (atomic ticket)
//    merges the splits' (max, sum, output) partials into O and LSE.
//
// Key set of query row i (same definition as the CPU oracle): every cache
// position not written by this step, plus each new row j that i may see.
// A position written by its first row j is reached through the cache (the
// projection kernel stored it there) and gated by vis[i][j]; later rows at a
// shared position live in the side buffer and are attended as an extra tile.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kDH = 128;
constexpr int kRowPad = kDH + 8;     // LDS row of K/V tiles (bf16): 272 B

typedef __bf16 bf16x4g __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16x4g lds_bf16x4;

__device__ __forceinline__ bf16x8 read_vt_frag(const bf16* p0, const bf16* p1)
{
    const bf16x4g a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4g b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// RG row groups of 16 query rows per wave; NWR waves split the rows, NWK waves
// split the keys of a tile; KW keys per wave per tile.
template <int RG, int NWR, int NWK, int KW>
struct AttnCfg {
    static constexpr int NW = NWR * NWK;
    static constexpr int NT = NW * 64;
    static constexpr int TK = KW * NWK;         // keys per tile
    static constexpr int KB = KW / 16;          // 16-key blocks per wave
    static constexpr int CHUNKS = TK * 2 * (kDH / 8);   // 16 B chunks of K+V per tile
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;
    static constexpr int TILE_BYTES = 2 * TK * kRowPad * 2;
    static constexpr int MERGE_BYTES = (NWK / 2) * NWR * RG * 64 * (32 + 2) * 4;
    static constexpr int SCRATCH = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
    static_assert(KW % 32 == 0, "PV consumes 32 keys per MFMA");
};

struct StepInfo {
    int b, g, bg, s, k0, k1;
};

template <int RG, int NWR, int NWK, int KW>
__global__ void __launch_bounds__(NWR * NWK * 64)
attn_mfma_kernel(AttnArgs a)
{
    using C = AttnCfg<RG, NWR, NWK, KW>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bf16* sK = (bf16*)smem;                         // [TK][kRowPad]
    bf16* sV = sK + C::TK * kRowPad;                // [TK][kRowPad]
    int16_t* sSlot = (int16_t*)(smem + C::SCRATCH); // [keys_per_split] owner row of written positions
    int* sInt = (int*)(sSlot + ((a.keys_per_split + 1) & ~1));
    int* sPos = sInt;                               // [nq]
    int* sOwn = sPos + a.q_max;                     // [nq] 1 if the row owns its position
    int* sDup = sOwn + a.q_max;                     // [nq] rows that do not own their position
    int* sMisc = sDup + a.q_max;                    // [0] dup count, [1] last flag, [2..] tile flags

    const int total = a.B * a.Hkv * a.splits;
    const int logical = xcd_remap(blockIdx.x, total);
    if (logical < 0) return;
    StepInfo si;
    si.bg = logical / a.splits;
    si.s = logical - si.bg * a.splits;
    si.b = si.bg / a.Hkv;
    si.g = si.bg - si.b * a.Hkv;
    si.k0 = si.s * a.keys_per_split;
    si.k1 = min(a.N, si.k0 + a.keys_per_split);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wk = wave % NWK, wr = wave / NWK;
    const int lr = lane & 15, lg = lane >> 4;
    const int nq = a.nq;
    const int G = a.G;
    const int nkeys = si.k1 - si.k0;
    const int ntiles = (nkeys + C::TK - 1) / C::TK;
    int* sTileFlag = sMisc + 2;

    // --- per-sequence bookkeeping: positions, ownership, duplicates, gating slots
    const int32_t* pos_b = a.pos_ids + (size_t)si.b * nq;
    for (int j = tid; j < nq; j += C::NT) sPos[j] = pos_b[j];
    if (a.vis) {
        for (int k = tid; k < nkeys; k += C::NT) sSlot[k] = -1;
        for (int t = tid; t < ntiles; t += C::NT) sTileFlag[t] = 0;
    }
    __syncthreads();
    for (int j = tid; j < nq; j += C::NT) {
        int own = 1;
        for (int q = 0; q < j; ++q)
            if (sPos[q] == sPos[j]) { own = 0; break; }
        sOwn[j] = own;
        const int p = sPos[j];
        if (own && a.vis && p >= si.k0 && p < si.k1) {
            sSlot[p - si.k0] = (int16_t)j;
            sTileFlag[(p - si.k0) / C::TK] = 1;
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
    const int ndup = (si.s == 0) ? sMisc[0] : 0;

    // --- query fragments: lane holds row (wr*RG + rg)*16 + lr, dims 32c + 8lg .. +7.
    // q arrives in fp32 and is split into bf16 hi + lo parts (q = hi + lo to
    // 16 significant bits), so the scores keep q's accumulation precision.
    const float* qbase = a.qbuf + (size_t)si.bg * a.q_max * G * kDH;
    bf16x8 qf[RG][4], ql[RG][4];
    int qrow_query[RG];   // query index of the lane's row, -1 for padding rows
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = (wr * RG + rg) * 16 + lr;
        qrow_query[rg] = row < a.R ? row / G : -1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float x[8];
            if (row < a.R) {
                const float4 u = *(const float4*)(qbase + (size_t)row * kDH + c * 32 + lg * 8);
                const float4 v = *(const float4*)(qbase + (size_t)row * kDH + c * 32 + lg * 8 + 4);
                x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
                x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
            } else {
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bf16 hi = (bf16)x[e];
                qf[rg][c][e] = hi;
                ql[rg][c][e] = (bf16)(x[e] - (float)hi);
            }
        }
    }
    bool rg_live[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) rg_live[rg] = (wr * RG + rg) * 16 < a.R;

    float m_run[RG], l_run[RG];
    f32x4 o[RG][8];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        m_run[rg] = -INFINITY;
        l_run[rg] = 0.f;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t cache_off = (size_t)si.bg * a.N * kDH;
    const bf16* Kg = (const bf16*)a.Kc + cache_off;
    const bf16* Vg = (const bf16*)a.Vc + cache_off;
    const bf16* SKg = (const bf16*)a.sideK + (size_t)si.bg * a.q_max * kDH;
    const bf16* SVg = (const bf16*)a.sideV + (size_t)si.bg * a.q_max * kDH;
    const uint8_t* vis_b = a.vis ? a.vis + (size_t)si.b * nq * nq : nullptr;

    uint4 pre[C::CPT];
    // tile loader: cache rows [t0, t0+TK) (mode 0) or side rows sDup[t0 ...] (mode 1)
    auto load_tile = [&](int t0, int mode) {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            const int c = tid + i * C::NT;
            pre[i] = make_uint4(0, 0, 0, 0);
            if (c < C::CHUNKS) {
                const int isv = c >= C::TK * 16;
                const int rem = c - isv * C::TK * 16;
                const int row = rem >> 4, part = rem & 15;
                const int key = t0 + row;
                if (mode == 0) {
                    if (key < si.k1)
                        pre[i] = *(const uint4*)((isv ? Vg : Kg) + (size_t)key * kDH + part * 8);
                } else if (key < ndup) {
                    const int j = sDup[key];
                    pre[i] = *(const uint4*)((isv ? SVg : SKg) + (size_t)j * kDH + part * 8);
                }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::CPT; ++i) {
            const int c = tid + i * C::NT;
            if (c < C::CHUNKS) {
                const int isv = c >= C::TK * 16;
                const int rem = c - isv * C::TK * 16;
                const int row = rem >> 4, part = rem & 15;
                *(uint4*)((isv ? sV : sK) + row * kRowPad + part * 8) = pre[i];
            }
        }
    };

    // one tile of math for this wave: keys [wk*KW, wk*KW+KW) of the LDS tile
    auto compute_tile = [&](int t0, int mode) {
        f32x4 sc[RG][C::KB];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) sc[rg][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 kf = *(const bf16x8*)(sK + (wk * KW + kb * 16 + lr) * kRowPad + c * 32 + lg * 8);
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
                    if (rg_live[rg]) {
                        sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rg][c], sc[rg][kb], 0, 0, 0);
                        sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, ql[rg][c], sc[rg][kb], 0, 0, 0);
                    }
            }
        }
        // scale, mask, online softmax; lane: row lr of each group, keys kb*16 + 4lg + i
        const bool gate = (mode == 1) || (a.vis && sTileFlag[(t0 - si.k0) / C::TK]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            if (!rg_live[rg]) continue;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kl = wk * KW + kb * 16 + lg * 4 + i;   // key within the tile
                    float s = sc[rg][kb][i] * a.scale_log2;
                    if (mode == 0) {
                        const int key = t0 + kl;
                        if (key >= si.k1) s = -INFINITY;
                        else if (gate) {
                            const int slot = sSlot[key - si.k0];
                            if (slot >= 0 && (qrow_query[rg] < 0 || !vis_b[(size_t)qrow_query[rg] * nq + slot]))
                                s = -INFINITY;
                        }
                    } else {
                        const int key = t0 + kl;
                        if (key >= ndup) s = -INFINITY;
                        else if (vis_b) {
                            const int j = sDup[key];
                            if (qrow_query[rg] < 0 || !vis_b[(size_t)qrow_query[rg] * nq + j]) s = -INFINITY;
                        }
                    }
                    sc[rg][kb][i] = s;
                    mx = fmaxf(mx, s);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[rg], mx);
            const float alpha = (m_run[rg] == -INFINITY) ? 0.f : exp2f(m_run[rg] - m_new);
            const float msub = (m_new == -INFINITY) ? 0.f : m_new;
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = exp2f(sc[rg][kb][i] - msub);   // exp2(-inf) = 0
                    sc[rg][kb][i] = p;
                    lsum += p;
                }
            l_run[rg] = l_run[rg] * alpha + lsum;
            m_run[rg] = m_new;
#pragma unroll
            for (int db = 0; db < 8; ++db) o[rg][db] *= alpha;
        }
        // O^T += V^T P^T, 32 keys per MFMA
#pragma unroll
        for (int ch = 0; ch < KW / 32; ++ch) {
            bf16x8 pf[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pf[rg][i] = (bf16)sc[rg][2 * ch][i];
                    pf[rg][4 + i] = (bf16)sc[rg][2 * ch + 1][i];
                }
            const int kbase = wk * KW + ch * 32 + lg * 4 + (lr >> 2);
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const int col = db * 16 + (lr & 3) * 4;
                const bf16x8 vf = read_vt_frag(sV + kbase * kRowPad + col, sV + (kbase + 16) * kRowPad + col);
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
                    if (rg_live[rg])
                        o[rg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rg], o[rg][db], 0, 0, 0);
            }
        }
    };

    // --- main loop over the split's cache rows
    if (ntiles > 0) load_tile(si.k0, 0);
    for (int it = 0; it < ntiles; ++it) {
        __syncthreads();                 // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (it + 1 < ntiles) load_tile(si.k0 + (it + 1) * C::TK, 0);
        compute_tile(si.k0 + it * C::TK, 0);
    }
    // --- rows that share a position with an earlier row (first split only)
    for (int t0 = 0; t0 < ndup; t0 += C::TK) {
        load_tile(t0, 1);
        __syncthreads();
        store_tile();
        __syncthreads();
        compute_tile(t0, 1);
    }

    // --- finish per-lane sums (row lr is spread over the 4 lane groups)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        l_run[rg] += __shfl_xor(l_run[rg], 16);
        l_run[rg] += __shfl_xor(l_run[rg], 32);
    }

    // --- merge the key-split waves through LDS (tree over wk)
    if (NWK > 1) {
        float* scr = (float*)smem;
        constexpr int SLOT = RG * 64 * (32 + 2);   // floats per wave state
#pragma unroll
        for (int stride = NWK / 2; stride >= 1; stride /= 2) {
            __syncthreads();
            if (wk >= stride && wk < 2 * stride) {
                float* dst = scr + ((size_t)(wr * (NWK / 2) + (wk - stride))) * SLOT;
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
            if (wk < stride) {
                const float* src = scr + ((size_t)(wr * (NWK / 2) + wk)) * SLOT;
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
        }
    }

    // --- outputs: lane holds row (wr*RG + rg)*16 + lr, dims db*16 + 4lg + i
    const float kLn2 = 0.69314718055994531f;
    if (a.splits == 1) {
        if (wk == 0) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const int row = (wr * RG + rg) * 16 + lr;
                if (row >= a.R) continue;
                const int j = row / G, hl = row - j * G;
                const int h = si.g * G + hl;
                const size_t orow = ((size_t)si.b * nq + j) * a.H + h;
                const float inv = l_run[rg] > 0.f ? 1.f / l_run[rg] : 0.f;
                bf16* op = (bf16*)a.O + orow * kDH;
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    bf16x4v v;
                    for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[rg][db][i] * inv);
                    *(bf16x4v*)(op + db * 16 + lg * 4) = v;
                }
                if (lg == 0)
                    a.LSE[orow] = l_run[rg] > 0.f ? (m_run[rg] + log2f(l_run[rg])) * kLn2 : -INFINITY;
            }
        }
        return;
    }

    // publish this split's partial state, then the last split of the (b, g) merges
    if (wk == 0) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = (wr * RG + rg) * 16 + lr;
            if (row >= a.R) continue;
            const size_t prow = ((size_t)si.bg * a.splits + si.s) * a.Rpad + row;
            float* pp = a.apart + prow * kDH;
#pragma unroll
            for (int db = 0; db < 8; ++db) *(f32x4*)(pp + db * 16 + lg * 4) = o[rg][db];
            if (lg == 0) {
                a.aml[prow * 2 + 0] = m_run[rg];
                a.aml[prow * 2 + 1] = l_run[rg];
            }
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) sMisc[1] = (atomicAdd(&a.aticket[si.bg], 1u) == (unsigned)(a.splits - 1));
    __syncthreads();
    if (!sMisc[1]) return;
    __threadfence();
    // combine: one thread per (row, 4 dims)
    const size_t pbase = (size_t)si.bg * a.splits * a.Rpad;
    for (int w = tid; w < a.R * (kDH / 4); w += C::NT) {
        const int row = w / (kDH / 4), d4 = w - row * (kDH / 4);
        float mx = -INFINITY;
        for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.aml[(pbase + (size_t)s * a.Rpad + row) * 2]);
        float L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (mx != -INFINITY) {
            for (int s = 0; s < a.splits; ++s) {
                const size_t pr = pbase + (size_t)s * a.Rpad + row;
                const float ms = a.aml[pr * 2];
                if (ms == -INFINITY) continue;
                const float f = exp2f(ms - mx);
                L += a.aml[pr * 2 + 1] * f;
                acc += *(const f32x4*)(a.apart + pr * kDH + d4 * 4) * f;
            }
        }
        const int j = row / G, hl = row - j * G;
        const size_t orow = ((size_t)si.b * nq + j) * a.H + si.g * G + hl;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        bf16x4v v;
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[i] * inv);
        *(bf16x4v*)((bf16*)a.O + orow * kDH + d4 * 4) = v;
        if (d4 == 0) a.LSE[orow] = L > 0.f ? (mx + log2f(L)) * kLn2 : -INFINITY;
    }
    if (tid == 0) a.aticket[si.bg] = 0u;
}

template <int RG, int NWR, int NWK, int KW>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t s)
{
    using C = AttnCfg<RG, NWR, NWK, KW>;
    const size_t shm = C::SCRATCH + 2 * (size_t)((a.keys_per_split + 1) & ~1) +
                       sizeof(int) * (3 * (size_t)a.q_max + 2 + (a.keys_per_split + C::TK - 1) / C::TK + 2);
    const int total = a.B * a.Hkv * a.splits;
    const int grid = ((total + 7) / 8) * 8;
    auto kern = attn_mfma_kernel<RG, NWR, NWK, KW>;
    if (shm > 64 * 1024) {
        // raise the dynamic LDS limit; a refusal shows up as a launch error below
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        (void)hipGetLastError();
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), shm, s, a);
    return hipGetLastError();
}

}  // namespace

// Keys per tile of the configuration chosen for R query rows per kv head.
int attn_mfma_tile_keys(int R)
{
    const int r16 = (R + 15) / 16;
    return r16 <= 3 ? 128 : 64;
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s)
{
    if (a.B * a.Hkv * a.splits == 0 || a.R == 0) return hipSuccess;
    const int r16 = (a.R + 15) / 16;
    switch (r16) {
        case 1: return launch_cfg<1, 1, 4, 32>(a, s);
        case 2: return launch_cfg<2, 1, 4, 32>(a, s);
        case 3: return launch_cfg<3, 1, 4, 32>(a, s);
        case 4: return launch_cfg<2, 2, 2, 32>(a, s);
        case 5: case 6: return launch_cfg<2, 3, 1, 64>(a, s);
        case 7: case 8: return launch_cfg<2, 4, 1, 64>(a, s);
        case 9: case 10: return launch_cfg<2, 5, 1, 64>(a, s);
        case 11: case 12: return launch_cfg<2, 6, 1, 64>(a, s);
        case 13: case 14: return launch_cfg<2, 7, 1, 64>(a, s);
        case 15: case 16: return launch_cfg<2, 8, 1, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fdllm
