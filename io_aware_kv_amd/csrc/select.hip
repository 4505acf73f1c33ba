// select.hip -- tracked-set scores and top-k selection after the fused step
// (gfx950, head width 128).
//
// Flash-dLLM keeps, as the tracked set of the next step, the previously
// decoded tokens that the masked query rows attend to most (jaehun.me review,
// "How It Works: A Concrete Example", Step 1: Cache selection, and the
// paragraph on Fig. 1b: middle layers concentrate their attention on a few
// tokens).  The score of cache position p is the attention mass that the
// selected query rows put on it in this layer, summed over their query heads:
//     a_p = sum_{i selected} sum_h 2^(s2_{i,h,p} - L2_{i,h}),
// with s2 the step's score in log2 units and L2 the step's LSE in log2 units,
// over the keys row i may see (positions written this step are the owner
// row's key, gated by the visibility mask).
//
//  * key_mass_ring_kernel / key_mass_kernel: one workgroup per (sequence, kv
//    head, key split).  The selected rows' q (fp32 in the step's staging
//    buffer, as bf16 hi + lo parts) are the MFMA A operand, 16-key blocks of
//    K the B operand, so a lane ends with 4 query rows of one key: the
//    per-key sum is four in-lane adds and two row-swap permutes.  With at
//    most 48 possible (row, head) pairs K streams through an LDS ring (the
//    pass is bound by HBM); with more, each wave loads its key blocks
//    straight into MFMA fragments (the pass is bound by its MFMAs and
//    exponentials).  Each kv head's partial sums go to a workspace row.
//  * key_mass_sum_kernel: a_p = sum over kv heads in head order (a fixed
//    order, so repeated runs agree bit for bit).
//  * select_top_kernel: one workgroup per sequence ranks the candidates by
//    64-bit keys (order-preserving score bits, then the inverted position so
//    equal scores rank the lower position first): a radix select finds the
//    k-th largest score, and only the k selected keys are sorted in LDS.
#include <algorithm>

#include "pipeline.h"

namespace fdllm {

namespace {

constexpr int kDH = 128;
constexpr int kMassWaves = 4;                 // consumer waves (one 16-key block of a tile each)
constexpr int kMassTK = 16 * kMassWaves;      // keys per ring stage
constexpr int kMassStage = kMassTK * 256;     // bytes per stage (K rows of 256 B)
constexpr int kMassMinStages = 3;
constexpr int kMassUnroll = 4;                // direct form: 16-key blocks a wave loads before computing
constexpr int kRowsWaves = 4;                 // pair-split ring form: consumer waves
constexpr int kRowsBlocks = 4;                // ... and row blocks of 16 pairs each wave can hold

__device__ __forceinline__ float sum4x(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// LDS layout (dynamic): the K ring [ns stages of kMassTK rows], then sSel[nq]
// int, sOwner[kps] int, sVis[nq * VW] u32.  One producer wave streams K tiles
// of kMassTK keys into the ring with global_load_lds (16 B chunks of a row
// XOR-swizzled by the row, so the fragment reads below are conflict-free) and
// releases each stage with a barrier once its own vmcnt shows it landed; the
// consumer waves take one 16-key block of each tile each, against all the
// selected (row, head) pairs: three 16-row blocks of q in registers (the
// launcher takes this form only when at most 48 pairs can be selected).
__global__ void __launch_bounds__((kMassWaves + 1) * 64) key_mass_ring_kernel(MassArgs a, int ns)
{
    constexpr int kMassRowBlocks = 3;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int sNsel;
    const int nq = a.nq, G = a.G;
    const int VW = (nq + 31) >> 5;
    int* sSel = (int*)(smem + (size_t)ns * kMassStage);
    int* sOwner = sSel + nq;
    uint32_t* sVis = (uint32_t*)(sOwner + a.keys_per_split);

    const int split = blockIdx.x % a.splits;
    const int bg = blockIdx.x / a.splits;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int k0 = split * a.keys_per_split;
    const int k1 = min(a.N, k0 + a.keys_per_split);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave == kMassWaves;
    const int lr = lane & 15, lg = lane >> 4;
    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    const uint8_t* sel_b = a.sel + (size_t)b * nq;
    const uint8_t* vis_b = a.vis ? a.vis + (size_t)b * nq * nq : nullptr;

    // selected rows in Q order (wave 0, 64 rows per ballot)
    if (wave == 0) {
        int n = 0;
        for (int c = 0; c < nq; c += 64) {
            const int j = c + lane;
            const bool s = j < nq && sel_b[j] != 0;
            const uint64_t m = __builtin_amdgcn_ballot_w64(s);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (s) sSel[n + below] = j;
            n += __builtin_popcountll(m);
        }
        if (lane == 0) sNsel = n;
    }
    // owner row of each position of the split: the first row in Q order
    for (int k = tid; k < k1 - k0; k += (kMassWaves + 1) * 64) sOwner[k] = 0x7fffffff;
    __syncthreads();
    for (int j = tid; j < nq; j += (kMassWaves + 1) * 64) {
        const int p = pos_b[j];
        if (p >= k0 && p < k1) atomicMin(&sOwner[p - k0], j);
    }
    const int nsel = sNsel;
    // visibility bits of the selected rows (word w covers owner rows 32w..)
    if (vis_b) {
        for (int t = tid; t < nsel * VW; t += (kMassWaves + 1) * 64) {
            const int s = t / VW, w = t - s * VW;
            const uint8_t* row = vis_b + (size_t)sSel[s] * nq;
            uint32_t bits = 0u;
            for (int e = 0; e < 32 && 32 * w + e < nq; ++e) bits |= (row[32 * w + e] != 0 ? 1u : 0u) << e;
            sVis[t] = bits;
        }
    }
    __syncthreads();

    const int R = min(nsel * G, 16 * kMassRowBlocks); // (selected row, head) pairs
    const int ntile = (k1 - k0 + kMassTK - 1) / kMassTK;
    const int total = ntile;
    const unsigned char* Kg = (const unsigned char*)((const bf16*)a.Kc + (size_t)bg * a.N * kDH);

    if (producer) {
        // ================= producer wave: K tiles -> LDS ring =================
        const int srow = lane >> 4, slot = lane & 15;
        auto issue = [&](int t) {
            unsigned char* st = smem + (size_t)(t % ns) * kMassStage;
            const int kt = k0 + (t % ntile) * kMassTK;
#pragma unroll
            for (int i = 0; i < kMassTK / 4; ++i) {
                const int row = 4 * i + srow;
                const int key = min(kt + row, k1 - 1);       // rows past the split repeat its last key
                __builtin_amdgcn_global_load_lds((glb_void*)(Kg + (size_t)key * 256 + ((slot ^ (row & 15)) << 4)),
                                                 (lds_void*)(st + i * 1024), 16, 0, 0);
            }
        };
        int issued = 0;
        for (; issued < min(ns - 1, total); ++issued) issue(issued);
        for (int t = 0; t < total; ++t) {
            // stage t has landed once at most (issued - t - 1) younger stages
            // of kMassTK / 4 loads each are in flight
            ring_producer_sync((issued - t - 1) * (kMassTK / 4));
            if (issued < total && issued < t + ns) issue(issued++);
        }
        return;
    }

    // ================= consumer waves =================
    // row of selected slot s (clamped; with no selected row, row 0 stands in
    // and every score is dropped through L2 = +inf)
    auto selrow = [&](int s) { return nsel > 0 ? sSel[min(s, nsel - 1)] : 0; };
    const float* qbase = a.qbuf + (size_t)bg * a.q_max * G * kDH;
    float* part = a.part + (size_t)bg * a.N;
    const float kLog2e = 1.4426950408889634f;
    // this wave's 16 keys of a tile: row wave * 16 + lr, chunk c * 4 + lg
    const int krow = wave * 16 + lr;
    int kofs[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kofs[c] = krow * 256 + (((c * 4 + lg) ^ (krow & 15)) << 4);

    bf16x8 qh[kMassRowBlocks][4], ql[kMassRowBlocks][4];
    float l2[kMassRowBlocks][4];
    auto rowbase = [&](int j) { return j * 16; };
    // q fragments as bf16 hi + lo parts (rows past R: zero q, L2 = +inf)
#pragma unroll
    for (int j = 0; j < kMassRowBlocks; ++j) {
        const int row = rowbase(j) + lr;
        const bool ok = row < R;
        const int rr = ok ? row : 0;
        const int s = rr / G, hl = rr - s * G;
        const float* qp = qbase + ((size_t)selrow(s) * G + hl) * kDH;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 x0 = *(const f32x4*)(qp + 32 * c + 8 * lg);
            const f32x4 x1 = *(const f32x4*)(qp + 32 * c + 8 * lg + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = ok ? (e < 4 ? x0[e] : x1[e - 4]) * a.scale_log2 : 0.f;
                const bf16 hi = (bf16)x;
                qh[j][c][e] = hi;
                ql[j][c][e] = (bf16)(x - (float)hi);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rowi = rowbase(j) + 4 * lg + i;
            const bool oki = rowi < R;
            const int ri = oki ? rowi : 0;
            const int si = ri / G, hli = ri - si * G;
            const int qi = selrow(si);
            const float lse = a.LSE[((size_t)b * nq + qi) * a.H + g * G + hli];
            // an empty key set (-inf) or a padding row contributes nothing
            l2[j][i] = (oki && lse > -INFINITY) ? lse * kLog2e : INFINITY;
        }
    }

    // scores of this wave's 16 keys at LDS row krow of stage st against the
    // register row blocks, masked, as 2^(s - L2), summed over the rows
    auto colsum_of = [&](const unsigned char* st, int krow, int key) {
        bf16x8 kf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[c] = *(const bf16x8*)(st + krow * 256 + (((c * 4 + lg) ^ (krow & 15)) << 4));
        const int ow = sOwner[min(key, k1 - 1) - k0];
        const int owner = ow == 0x7fffffff ? -1 : ow;
        const bool gated = vis_b != nullptr && owner >= 0;
        float cs = 0.f;
#pragma unroll
        for (int j = 0; j < kMassRowBlocks; ++j) {
            const int rb0 = rowbase(j);
            if (rb0 >= R && j > 0) break;                  // (uniform: no selected pair left)
            f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[j][c], kf[c], sc, 0, 0, 0);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[j][c], kf[c], sc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bool keep = key < k1;
                if (gated) {
                    // selected slot of the lane's row (past R: slot 0, whose
                    // term is zero through L2 anyway)
                    const int rowi = rb0 + 4 * lg + i;
                    const int sr = rowi < R ? rowi / G : 0;
                    keep = keep && ((sVis[sr * VW + (owner >> 5)] >> (owner & 31)) & 1u);
                }
                const float pv = __builtin_amdgcn_exp2f(sc[i] - l2[j][i]);   // 2^-inf = 0
                cs += keep ? pv : 0.f;
            }
        }
        return sum4x(cs);
    };

    for (int t = 0; t < total; ++t) {
        ring_consumer_sync();
        const unsigned char* st = smem + (size_t)(t % ns) * kMassStage;
        const int kt = k0 + (t % ntile) * kMassTK;
        const int key = kt + wave * 16 + lr;
        const float cs = colsum_of(st, wave * 16 + lr, key);
        if (lg == 0 && key < k1) part[key] = cs;
    }
}

// Ring form with the (selected row, head) pairs split across the consumer
// waves, for up to NW * RBW * 16 pairs: the producer wave streams 64-key K
// tiles into the LDS ring as in key_mass_ring_kernel; consumer wave w holds
// its share of the pairs' row blocks (at most RBW of 16 pairs) in registers
// and scores every key of each tile against them, so each K row is read
// from HBM once and from LDS once per wave.  A wave's per-key sums stay in
// LDS for the whole split and are added in wave order at the end (the same
// bits on every run).
template <int NW, int RBW>
__global__ void __launch_bounds__((NW + 1) * 64) key_mass_rows_kernel(MassArgs a, int ns)
{
    constexpr int NT = (NW + 1) * 64;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int sNsel;
    const int nq = a.nq, G = a.G;
    const int VW = (nq + 31) >> 5;
    const int kps = a.keys_per_split;
    int* sSel = (int*)(smem + (size_t)ns * kMassStage);
    int* sOwner = sSel + nq;
    uint32_t* sVis = (uint32_t*)(sOwner + kps);
    float* sAcc = (float*)(sVis + (size_t)nq * VW);   // [NW][kps] per-wave key sums

    const int split = blockIdx.x % a.splits;
    const int bg = blockIdx.x / a.splits;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int k0 = split * kps;
    const int k1 = min(a.N, k0 + kps);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave == NW;
    const int lr = lane & 15, lg = lane >> 4;
    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    const uint8_t* sel_b = a.sel + (size_t)b * nq;
    const uint8_t* vis_b = a.vis ? a.vis + (size_t)b * nq * nq : nullptr;

    // selected rows in Q order (wave 0, 64 rows per ballot)
    if (wave == 0) {
        int n = 0;
        for (int c = 0; c < nq; c += 64) {
            const int j = c + lane;
            const bool sl = j < nq && sel_b[j] != 0;
            const uint64_t m = __builtin_amdgcn_ballot_w64(sl);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (sl) sSel[n + below] = j;
            n += __builtin_popcountll(m);
        }
        if (lane == 0) sNsel = n;
    }
    // owner row of each position of the split: the first row in Q order
    for (int k = tid; k < k1 - k0; k += NT) sOwner[k] = 0x7fffffff;
    __syncthreads();
    for (int j = tid; j < nq; j += NT) {
        const int p = pos_b[j];
        if (p >= k0 && p < k1) atomicMin(&sOwner[p - k0], j);
    }
    const int nsel = sNsel;
    if (vis_b) {
        for (int t = tid; t < nsel * VW; t += NT) {
            const int sr = t / VW, w = t - sr * VW;
            const uint8_t* row = vis_b + (size_t)sSel[sr] * nq;
            uint32_t bits = 0u;
            for (int e = 0; e < 32 && 32 * w + e < nq; ++e) bits |= (row[32 * w + e] != 0 ? 1u : 0u) << e;
            sVis[t] = bits;
        }
    }
    __syncthreads();

    const int R = nsel * G;                       // selected (row, head) pairs (<= NW * RBW * 16)
    const int nrb = (R + 15) >> 4;
    const int per = (nrb + NW - 1) / NW;          // row blocks per consumer wave
    const int ntile = (k1 - k0 + kMassTK - 1) / kMassTK;
    const unsigned char* Kg = (const unsigned char*)((const bf16*)a.Kc + (size_t)bg * a.N * kDH);

    if (producer) {
        const int srow = lane >> 4, slot = lane & 15;
        auto issue = [&](int t) {
            unsigned char* st = smem + (size_t)(t % ns) * kMassStage;
            const int kt = k0 + t * kMassTK;
#pragma unroll
            for (int i = 0; i < kMassTK / 4; ++i) {
                const int row = 4 * i + srow;
                const int key = min(kt + row, k1 - 1);       // rows past the split repeat its last key
                __builtin_amdgcn_global_load_lds((glb_void*)(Kg + (size_t)key * 256 + ((slot ^ (row & 15)) << 4)),
                                                 (lds_void*)(st + i * 1024), 16, 0, 0);
            }
        };
        int issued = 0;
        for (; issued < min(ns - 1, ntile); ++issued) issue(issued);
        for (int t = 0; t < ntile; ++t) {
            ring_producer_sync((issued - t - 1) * (kMassTK / 4));
            if (issued < ntile && issued < t + ns) issue(issued++);
        }
    } else {
        // this wave's row blocks rb0 .. rb0 + nrbw - 1 (none past the pairs)
        const int rb0 = wave * per;
        const int nrbw = max(0, min(per, nrb - rb0));
        auto selrow = [&](int sr) { return nsel > 0 ? sSel[min(sr, nsel - 1)] : 0; };
        const float* qbase = a.qbuf + (size_t)bg * a.q_max * G * kDH;
        const float kLog2e = 1.4426950408889634f;
        bf16x8 qh[RBW][4], ql[RBW][4];
        float l2[RBW][4];
        int srow[RBW][4];
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int row = (rb0 + j) * 16 + lr;
            const bool ok = j < nrbw && row < R;
            const int rr = ok ? row : 0;
            const int sr = rr / G, hl = rr - sr * G;
            const float* qp = qbase + ((size_t)selrow(sr) * G + hl) * kDH;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 x0 = *(const f32x4*)(qp + 32 * c + 8 * lg);
                const f32x4 x1 = *(const f32x4*)(qp + 32 * c + 8 * lg + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = ok ? (e < 4 ? x0[e] : x1[e - 4]) * a.scale_log2 : 0.f;
                    const bf16 hi = (bf16)x;
                    qh[j][c][e] = hi;
                    ql[j][c][e] = (bf16)(x - (float)hi);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rowi = (rb0 + j) * 16 + 4 * lg + i;
                const bool oki = j < nrbw && rowi < R;
                const int ri = oki ? rowi : 0;
                const int si = ri / G, hli = ri - si * G;
                const float lse = a.LSE[((size_t)b * nq + selrow(si)) * a.H + g * G + hli];
                // an empty key set (-inf) or a padding row contributes nothing
                l2[j][i] = (oki && lse > -INFINITY) ? lse * kLog2e : INFINITY;
                srow[j][i] = oki ? si : 0;
            }
        }
        float* acc = sAcc + (size_t)wave * kps;
        for (int t = 0; t < ntile; ++t) {
            ring_consumer_sync();
            const unsigned char* st = smem + (size_t)(t % ns) * kMassStage;
            const int kt = k0 + t * kMassTK;
#pragma unroll
            for (int kb = 0; kb < kMassTK / 16; ++kb) {
                const int krow = kb * 16 + lr;
                const int key = kt + krow;
                bf16x8 kf[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kf[c] = *(const bf16x8*)(st + krow * 256 + (((c * 4 + lg) ^ (krow & 15)) << 4));
                const int ow = sOwner[min(key, k1 - 1) - k0];
                const int owner = ow == 0x7fffffff ? -1 : ow;
                const bool gated = vis_b != nullptr && owner >= 0;
                float cs = 0.f;
#pragma unroll
                for (int j = 0; j < RBW; ++j) {
                    if (j >= nrbw) break;                    // (uniform)
                    f32x4 sc = f32x4{-l2[j][0], -l2[j][1], -l2[j][2], -l2[j][3]};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[j][c], kf[c], sc, 0, 0, 0);
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[j][c], kf[c], sc, 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        bool keep = key < k1;
                        if (gated) keep = keep && ((sVis[srow[j][i] * VW + (owner >> 5)] >> (owner & 31)) & 1u);
                        const float pv = __builtin_amdgcn_exp2f(sc[i]);   // 2^-inf = 0
                        cs += keep ? pv : 0.f;
                    }
                }
                cs = sum4x(cs);
                if (lg == 0 && key < k1) acc[key - k0] = cs;
            }
        }
    }
    __syncthreads();
    // the waves' sums of each key, added in wave order
    float* part = a.part + (size_t)bg * a.N;
    for (int k = tid; k < k1 - k0; k += NT) {
        float v = sAcc[k];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += sAcc[(size_t)w * kps + k];
        part[k0 + k] = v;
    }
}

// Direct form, for more than 64 possible (row, head) pairs.  LDS layout
// (dynamic): sSel[nq] int, sOwner[kps] int, sVis[nq * VW] u32.  Up to four
// row blocks of 16 (selected row, head) pairs are held in registers at a
// time (blocks past the selection are skipped); a wave takes kMassUnroll
// consecutive 16-key blocks per round, loaded straight into MFMA fragments,
// with all their K loads in flight.
__global__ void __launch_bounds__(kMassWaves * 64) key_mass_kernel(MassArgs a)
{
    constexpr int kMassRowBlocks = 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int sNsel;
    const int nq = a.nq, G = a.G;
    const int VW = (nq + 31) >> 5;
    int* sSel = (int*)smem;
    int* sOwner = sSel + nq;
    uint32_t* sVis = (uint32_t*)(sOwner + a.keys_per_split);

    const int split = blockIdx.x % a.splits;
    const int bg = blockIdx.x / a.splits;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int k0 = split * a.keys_per_split;
    const int k1 = min(a.N, k0 + a.keys_per_split);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    const uint8_t* sel_b = a.sel + (size_t)b * nq;
    const uint8_t* vis_b = a.vis ? a.vis + (size_t)b * nq * nq : nullptr;

    // selected rows in Q order (wave 0, 64 rows per ballot)
    if (wave == 0) {
        int n = 0;
        for (int c = 0; c < nq; c += 64) {
            const int j = c + lane;
            const bool s = j < nq && sel_b[j] != 0;
            const uint64_t m = __builtin_amdgcn_ballot_w64(s);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (s) sSel[n + below] = j;
            n += __builtin_popcountll(m);
        }
        if (lane == 0) sNsel = n;
    }
    // owner row of each position of the split: the first row in Q order
    for (int k = tid; k < k1 - k0; k += kMassWaves * 64) sOwner[k] = 0x7fffffff;
    __syncthreads();
    for (int j = tid; j < nq; j += kMassWaves * 64) {
        const int p = pos_b[j];
        if (p >= k0 && p < k1) atomicMin(&sOwner[p - k0], j);
    }
    const int nsel = sNsel;
    // visibility bits of the selected rows (word w covers owner rows 32w..)
    if (vis_b) {
        for (int t = tid; t < nsel * VW; t += kMassWaves * 64) {
            const int s = t / VW, w = t - s * VW;
            const uint8_t* row = vis_b + (size_t)sSel[s] * nq;
            uint32_t bits = 0u;
            for (int e = 0; e < 32 && 32 * w + e < nq; ++e) bits |= (row[32 * w + e] != 0 ? 1u : 0u) << e;
            sVis[t] = bits;
        }
    }
    __syncthreads();

    const int R = nsel * G;                          // (selected row, head) pairs
    // row of selected slot s (clamped; with no selected row, row 0 stands in
    // and every score is dropped through L2 = +inf)
    auto selrow = [&](int s) { return nsel > 0 ? sSel[min(s, nsel - 1)] : 0; };
    const float* qbase = a.qbuf + (size_t)bg * a.q_max * G * kDH;
    float* part = a.part + (size_t)bg * a.N;
    const bf16* Kg = (const bf16*)a.Kc + (size_t)bg * a.N * kDH;
    const int nkb = (k1 - k0 + 15) >> 4;
    const float kLog2e = 1.4426950408889634f;

    for (int r0 = 0; r0 < max(R, 1); r0 += 16 * kMassRowBlocks) {
        // q fragments of up to four row blocks (rows past R: zero q, L2 = +inf)
        bf16x8 qh[kMassRowBlocks][4], ql[kMassRowBlocks][4];
        float l2[kMassRowBlocks][4];
        int srow[kMassRowBlocks][4];
#pragma unroll
        for (int rb = 0; rb < kMassRowBlocks; ++rb) {
            const int row = r0 + rb * 16 + lr;
            const bool ok = row < R;
            const int rr = ok ? row : 0;
            const int s = rr / G, hl = rr - s * G;
            const float* qp = qbase + ((size_t)selrow(s) * G + hl) * kDH;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4 x0 = *(const f32x4*)(qp + 32 * c + 8 * lg);
                const f32x4 x1 = *(const f32x4*)(qp + 32 * c + 8 * lg + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = ok ? (e < 4 ? x0[e] : x1[e - 4]) * a.scale_log2 : 0.f;
                    const bf16 hi = (bf16)x;
                    qh[rb][c][e] = hi;
                    ql[rb][c][e] = (bf16)(x - (float)hi);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rowi = r0 + rb * 16 + 4 * lg + i;
                const bool oki = rowi < R;
                const int ri = oki ? rowi : 0;
                const int si = ri / G, hli = ri - si * G;
                const int qi = selrow(si);
                const float lse = a.LSE[((size_t)b * nq + qi) * a.H + g * G + hli];
                // an empty key set (-inf) or a padding row contributes nothing
                l2[rb][i] = (oki && lse > -INFINITY) ? lse * kLog2e : INFINITY;
                srow[rb][i] = oki ? si : -1;
            }
        }
        for (int kb0 = wave * kMassUnroll; kb0 < nkb; kb0 += kMassWaves * kMassUnroll) {
            bf16x8 kf[kMassUnroll][4];
            int keyu[kMassUnroll], ownu[kMassUnroll];
#pragma unroll
            for (int u = 0; u < kMassUnroll; ++u) {
                keyu[u] = k0 + (kb0 + u) * 16 + lr;
                const int kc = min(keyu[u], k1 - 1);
#pragma unroll
                for (int c = 0; c < 4; ++c) kf[u][c] = *(const bf16x8*)(Kg + (size_t)kc * kDH + 32 * c + 8 * lg);
                ownu[u] = sOwner[kc - k0];
            }
#pragma unroll
            for (int u = 0; u < kMassUnroll; ++u) {
                const int key = keyu[u];
                const int owner = ownu[u] == 0x7fffffff ? -1 : ownu[u];
                const bool gated = vis_b != nullptr && owner >= 0;
                float colsum = 0.f;
                if (vis_b == nullptr) {
                    // no mask: every row block runs (rows past R have zero q
                    // and L2 = +inf, so they add nothing); the accumulators
                    // start at -L2, so the scores leave the MFMAs as
                    // exponents, and the hi and lo chains of the four row
                    // blocks interleave
                    f32x4 sc[kMassRowBlocks];
#pragma unroll
                    for (int rb = 0; rb < kMassRowBlocks; ++rb)
                        sc[rb] = f32x4{-l2[rb][0], -l2[rb][1], -l2[rb][2], -l2[rb][3]};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
#pragma unroll
                        for (int rb = 0; rb < kMassRowBlocks; ++rb)
                            sc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[rb][c], kf[u][c], sc[rb], 0, 0, 0);
#pragma unroll
                        for (int rb = 0; rb < kMassRowBlocks; ++rb)
                            sc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[rb][c], kf[u][c], sc[rb], 0, 0, 0);
                    }
#pragma unroll
                    for (int rb = 0; rb < kMassRowBlocks; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) colsum += __builtin_amdgcn_exp2f(sc[rb][i]);   // 2^-inf = 0
                    colsum = key < k1 ? colsum : 0.f;
                } else {
                    // under a mask, row block by row block: a key written this
                    // step is dropped for the rows that do not see its owner
#pragma unroll
                    for (int rb = 0; rb < kMassRowBlocks; ++rb) {
                        if (r0 + rb * 16 >= R) break;          // (uniform: no selected pair left)
                        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[rb][c], kf[u][c], sc, 0, 0, 0);
                            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[rb][c], kf[u][c], sc, 0, 0, 0);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            bool keep = key < k1;
                            if (gated) {
                                const int sr = max(srow[rb][i], 0);
                                keep = keep && ((sVis[sr * VW + (owner >> 5)] >> (owner & 31)) & 1u);
                            }
                            const float pv = __builtin_amdgcn_exp2f(sc[i] - l2[rb][i]);   // 2^-inf = 0
                            colsum += keep ? pv : 0.f;
                        }
                    }
                }
                colsum = sum4x(colsum);
                if (lg == 0 && key < k1) {
                    if (r0 == 0) part[key] = colsum;
                    else part[key] += colsum;
                }
            }
        }
    }
}

// Scalar form for the fp32 layers and head widths other than 128: one thread
// per (sequence, kv head, position), fp32 dot products.
template <typename T>
__global__ void __launch_bounds__(256) key_mass_generic_kernel(MassArgs a)
{
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (size_t)a.B * a.Hkv * a.N) return;
    const int p = (int)(t % a.N);
    const int bg = (int)(t / a.N);
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int nq = a.nq, G = a.G, dh = a.dh;
    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    int owner = -1;
    for (int j = 0; j < nq && owner < 0; ++j)
        if (pos_b[j] == p) owner = j;
    const T* kp = (const T*)a.Kc + ((size_t)bg * a.N + p) * dh;
    const float* qb = a.qbuf + (size_t)bg * a.q_max * G * dh;
    const float kLog2e = 1.4426950408889634f;
    float acc = 0.f;
    for (int i = 0; i < nq; ++i) {
        if (!a.sel[(size_t)b * nq + i]) continue;
        if (owner >= 0 && a.vis && !a.vis[((size_t)b * nq + i) * nq + owner]) continue;
        for (int hl = 0; hl < G; ++hl) {
            const float lse = a.LSE[((size_t)b * nq + i) * a.H + g * G + hl];
            if (!(lse > -INFINITY)) continue;
            const float* q = qb + ((size_t)i * G + hl) * dh;
            float s = 0.f;
            for (int e = 0; e < dh; ++e) s += q[e] * to_f32(kp[e]);
            acc += exp2f(s * a.scale_log2 - lse * kLog2e);
        }
    }
    a.part[t] = acc;
}

// a_p = sum over kv heads of the partial sums, in head order
__global__ void __launch_bounds__(256) key_mass_sum_kernel(const float* __restrict__ part, float* __restrict__ scores,
                                                           int B, int Hkv, int N)
{
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (size_t)B * N) return;
    const size_t b = t / N, p = t - b * N;
    const float* src = part + b * Hkv * (size_t)N + p;
    float s = 0.f;
    int g = 0;
    // up to 32 loads in flight (one memory round trip for 32 kv heads),
    // added in head order
    for (; g + 32 <= Hkv; g += 32) {
        float v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) v[u] = src[(size_t)(g + u) * N];
#pragma unroll
        for (int u = 0; u < 32; ++u) s += v[u];
    }
    for (; g + 8 <= Hkv; g += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(g + u) * N];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; g < Hkv; ++g) s += src[(size_t)g * N];
    scores[t] = s;
}

// Order-preserving unsigned image of a float (-0 folded onto +0).
__device__ __forceinline__ uint32_t ordered_bits(float x)
{
    const uint32_t u = __float_as_uint(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopThreads = 1024;
constexpr int kTopWaves = kTopThreads / 64;
constexpr int kTopPer = 16;           // consecutive positions per thread (N <= 16384)

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no trip
// through LDS as a lane shuffle would take): shifts by 1, 2, 4, 8 inside each
// row of 16 lanes (lanes shifted in from outside the row add 0), then the last
// lane of row 0 added to row 1, and of row 2 to row 3, then the last lane of
// row 1 added to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return x;
}

// Exclusive prefix sum of x over the workgroup in thread order; `total` gets
// the sum.  sTmp holds kTopWaves + 1 ints.
__device__ __forceinline__ int top_scan(int x, int* sTmp, int& total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(x);
    if (lane == 63) sTmp[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int w = lane < kTopWaves ? sTmp[lane] : 0;
        const int wi = wave_incl_scan(w);
        if (lane < kTopWaves) sTmp[lane] = wi - w;
        if (lane == kTopWaves - 1) sTmp[kTopWaves] = wi;
    }
    __syncthreads();
    const int r = sTmp[wave] + incl - x;
    total = sTmp[kTopWaves];
    __syncthreads();
    return r;
}

// One workgroup per sequence.  Candidate p has the key (ordered score bits,
// then the inverted position), so larger keys rank first and equal scores
// rank the lower position first.  The k-th largest score bits come from a
// radix select (up to four 8-bit passes over per-wave LDS histograms, three
// barriers a pass; it stops early once every key of the chosen bin is
// taken); the candidates above it, and the lowest-position ones equal to it,
// are compacted in position order and only those (a power of two >=
// min(k, N) slots) are ranked in LDS.
__global__ void __launch_bounds__(kTopThreads) select_top_kernel(const float* __restrict__ scores,
                                                                 const uint8_t* __restrict__ cand, int N, int n2,
                                                                 int k, int32_t* __restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // per-wave histograms, two sets used by alternate radix passes (one pass
    // clears the next pass's set while it reduces its own, so a pass needs
    // three barriers); after the radix select the same space holds the
    // selected keys [n2]
    int (*sHist)[kTopWaves][256] = (int (*)[kTopWaves][256])smem;
    uint64_t* key = (uint64_t*)smem;
    __shared__ int sTmp[kTopWaves + 1];
    __shared__ int sBin[2], sNeed[2], sAll[2], sCount;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* sc = scores + (size_t)b * N;
    const uint8_t* cd = cand + (size_t)b * N;

    if (tid == 0) sCount = 0;
    for (int t = tid; t < kTopWaves * 256; t += kTopThreads) (&sHist[0][0][0])[t] = 0;
    __syncthreads();
    // each thread takes kTopPer consecutive positions straight from memory
    // (all its loads in flight at once; positions past N are not valid)
    uint32_t u[kTopPer];
    uint32_t valid = 0u;
    const int p0 = tid * kTopPer;
    if (p0 + kTopPer <= N) {
#pragma unroll
        for (int i = 0; i < kTopPer; ++i) {
            u[i] = ordered_bits(sc[p0 + i]);
            valid |= (cd[p0 + i] != 0 ? 1u : 0u) << i;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kTopPer; ++i) {
            const bool in = p0 + i < N;
            u[i] = in ? ordered_bits(sc[p0 + i]) : 0u;
            valid |= ((in && cd[p0 + i] != 0) ? 1u : 0u) << i;
        }
    }
    int cnt = __builtin_popcount(valid);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) atomicAdd(&sCount, cnt);
    __syncthreads();
    const int C = sCount;

    // threshold: the k-th largest score bits among the candidates (when there
    // are more than k), and how many candidates equal to it are taken
    uint32_t thr = 0u, pmask = ~0u;
    int need = 0;
    if (C > k) {
        pmask = 0u;
        need = k;
        for (int shift = 24, par = 0; shift >= 0; shift -= 8, par ^= 1) {
            // sHist[par] was cleared before the first pass or during the pass
            // before this one.  A thread counts runs of equal digits among its
            // positions and adds each run once: the first pass (sign and
            // exponent bits) puts nearly every key in a few bins, where one
            // LDS atomic per key would serialise.
            int rb = -1, rc = 0;
#pragma unroll
            for (int i = 0; i < kTopPer; ++i) {
                if (((valid >> i) & 1u) && (u[i] & pmask) == thr) {
                    const int bin = (int)((u[i] >> shift) & 255u);
                    if (bin != rb) {
                        if (rc) atomicAdd(&sHist[par][wave][rb], rc);
                        rb = bin;
                        rc = 1;
                    } else {
                        ++rc;
                    }
                }
            }
            if (rc) atomicAdd(&sHist[par][wave][rb], rc);
            __syncthreads();
            if (tid < 256) {
                int h = 0;
#pragma unroll
                for (int w = 0; w < kTopWaves; ++w) h += sHist[par][w][tid];
                sHist[par][0][tid] = h;
            } else if (shift > 0) {
                // the next pass's set: its last reads (the bin choice of the
                // pass before this one) ended before this pass's first barrier
                for (int t = tid - 256; t < kTopWaves * 256; t += kTopThreads - 256) (&sHist[par ^ 1][0][0])[t] = 0;
            }
            __syncthreads();
            if (wave == 0) {
                // lane l holds bins 255 - 4l .. 252 - 4l; counts accumulate from the top bin down
                int c[4], s4 = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    c[j] = sHist[par][0][255 - 4 * lane - j];
                    s4 += c[j];
                }
                const int incl = wave_incl_scan(s4);
                const int excl = incl - s4;
                if (excl < need && need <= incl) {
                    int acc = excl, bin = -1, rest = 0, all = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (bin < 0 && acc + c[j] >= need) {
                            bin = 255 - 4 * lane - j;
                            rest = need - acc;
                            all = c[j] == rest;
                        }
                        acc += c[j];
                    }
                    sBin[par] = bin;
                    sNeed[par] = rest;
                    sAll[par] = all;
                }
            }
            __syncthreads();
            // sBin[par] is written again two passes on, after barriers every
            // thread reaches only once it has read it here
            thr |= (uint32_t)sBin[par] << shift;
            pmask |= 255u << shift;
            need = sNeed[par];
            // every key of the bin is taken: the digits below need not be
            // known (the selection then compares the known digits only)
            if (sAll[par]) break;
        }
    }

    // the selected candidates, compacted in position order: all of them when
    // there are at most k, else those above the threshold and the first
    // `need` equal to it.  One scan gives both counts before each thread
    // (above in the low 16 bits, equal in the high; N <= 16384): the keys
    // selected before a thread are the ones above plus min(equal, need).
    uint32_t above = valid, tie = 0u;
    if (C > k) {
        above = 0u;
#pragma unroll
        for (int i = 0; i < kTopPer; ++i) {
            const bool v = (valid >> i) & 1u;
            above |= ((v && (u[i] & pmask) > thr) ? 1u : 0u) << i;
            tie |= ((v && (u[i] & pmask) == thr) ? 1u : 0u) << i;
        }
    }
    int tot;
    const int pre = top_scan((__builtin_popcount(tie) << 16) | __builtin_popcount(above), sTmp, tot);
    const int nsel = (tot & 0xffff) + min(tot >> 16, need);
    int w = (pre & 0xffff) + min(pre >> 16, need);
    int r = pre >> 16;                                  // equal keys before this position
#pragma unroll
    for (int i = 0; i < kTopPer; ++i) {
        const bool t = (tie >> i) & 1u;
        if (((above >> i) & 1u) || (t && r < need)) {
            const uint32_t p = (uint32_t)(tid * kTopPer + i);
            key[w++] = ((uint64_t)u[i] << 32) | (uint64_t)(0xffffffffu - p);
        }
        r += t ? 1 : 0;
    }
    for (int t = nsel + tid; t < n2; t += kTopThreads) key[t] = 0;   // padding sorts last
    __syncthreads();
    if (n2 <= 256) {
        // up to 256 keys (all distinct): the rank of a key is the number of
        // larger keys, counted by 1024 / n2 threads per key (a power-of-two
        // group of lanes of one wave per key)
        const int tpk = min(min(n2, kTopThreads / n2), 64), per = n2 / tpk;
        const int i = tid / tpk, sub = tid - i * tpk;
        const bool live = i < n2;
        const uint64_t mine = live ? key[i] : 0;
        int rank = 0;
        if (live)
            for (int j = sub * per; j < (sub + 1) * per; ++j) rank += key[j] > mine ? 1 : 0;
        for (int o = 1; o < tpk; o <<= 1) rank += __shfl_xor(rank, o);
        // the keys are distinct, so their ranks are 0 .. nsel - 1: each real
        // key's position goes straight to its output slot, the slots past
        // nsel get -1
        if (live && sub == 0 && i < nsel)
            out[(size_t)b * k + rank] = (int32_t)(0xffffffffu - (uint32_t)(mine & 0xffffffffu));
        for (int t = nsel + tid; t < k; t += kTopThreads) out[(size_t)b * k + t] = -1;
        return;
    }
    // bitonic network over the n2 slots, descending overall (more than 256)
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < n2 / 2; t += kTopThreads) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t x = key[lo], y = key[hi];
                if ((x < y) == desc) { key[lo] = y; key[hi] = x; }
            }
            __syncthreads();
        }
    }
    for (int t = tid; t < k; t += kTopThreads)
        out[(size_t)b * k + t] = t < nsel ? (int32_t)(0xffffffffu - (uint32_t)(key[t] & 0xffffffffu)) : -1;
}

}  // namespace

// LDS of the bookkeeping plus the smallest ring
size_t key_mass_lds_bytes(int nq, int keys_per_split)
{
    const int VW = (nq + 31) >> 5;
    return (size_t)kMassMinStages * kMassStage + (size_t)nq * 4 + (size_t)keys_per_split * 4 +
           (size_t)nq * VW * 4;
}

hipError_t launch_key_mass(const MassArgs& a, hipStream_t s)
{
    if (a.B * a.Hkv == 0 || a.N == 0) return hipSuccess;
    const size_t book = key_mass_lds_bytes(a.nq, a.keys_per_split) - (size_t)kMassMinStages * kMassStage;
    // as many stages as fit (at most 8) beside the bookkeeping and the
    // kernel's own few bytes; two workgroups per CU when there are more
    // workgroups than CUs
    const unsigned wgs = (unsigned)(a.B * a.Hkv * a.splits);
    hipError_t e;
    const size_t rows_book = book + (size_t)kRowsWaves * a.keys_per_split * 4;
    if ((long)a.nq * a.G > 192 && (long)a.nq * a.G <= 16L * kRowsWaves * kRowsBlocks &&
        rows_book + (size_t)kMassMinStages * kMassStage + 256 <= 160 * 1024) {
        // 193 to 256 pairs, which the direct form would take in four rounds
        // (each reloading K and q): the ring with the pairs split across the
        // waves.  With fewer pairs the direct form is as fast or faster
        // (measured: 144 and 176 pairs per kv head 25 and 30 us direct against
        // 35 and 44 us here; 224 pairs 50 against about 36 us).
        const size_t budget = (wgs > 256 ? 80 : 160) * 1024 - 256 - rows_book;
        int ns = (int)std::min<size_t>(8, budget / kMassStage);
        if (ns < kMassMinStages) ns = (int)std::min<size_t>(8, (160 * 1024 - 256 - rows_book) / kMassStage);
        const size_t shm = (size_t)ns * kMassStage + rows_book;
        constexpr auto kern = key_mass_rows_kernel<kRowsWaves, kRowsBlocks>;
        (void)allow_full_lds<kern>();
        (void)hipGetLastError();
        hipLaunchKernelGGL(kern, dim3(wgs), dim3((kRowsWaves + 1) * 64), shm, s, a, ns);
    } else if ((long)a.nq * a.G <= 48) {
        // at most 48 (row, head) pairs can be selected: the K stream through
        // the LDS ring, all pairs in the registers of every wave
        const size_t budget = (wgs > 256 ? 80 : 160) * 1024 - 256 - book;
        int ns = (int)std::min<size_t>(8, budget / kMassStage);
        if (ns < kMassMinStages) ns = (int)std::min<size_t>(8, (160 * 1024 - 256 - book) / kMassStage);
        if (ns < kMassMinStages) return hipErrorInvalidValue;
        const size_t shm = (size_t)ns * kMassStage + book;
        (void)allow_full_lds<key_mass_ring_kernel>();
        (void)hipGetLastError();
        hipLaunchKernelGGL(key_mass_ring_kernel, dim3(wgs), dim3((kMassWaves + 1) * 64), shm, s, a, ns);
    } else {
        // more: the direct form keeps every pair's work in its own waves
        (void)allow_full_lds<key_mass_kernel>();
        (void)hipGetLastError();
        hipLaunchKernelGGL(key_mass_kernel, dim3(wgs), dim3(kMassWaves * 64), book, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t n = (size_t)a.B * a.N;
    hipLaunchKernelGGL(key_mass_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.part, a.scores,
                       a.B, a.Hkv, a.N);
    return hipGetLastError();
}

hipError_t launch_key_mass_generic(const MassArgs& a, int dtype, hipStream_t s)
{
    const size_t n = (size_t)a.B * a.Hkv * a.N;
    if (n == 0) return hipSuccess;
    if (dtype == 1)
        hipLaunchKernelGGL(key_mass_generic_kernel<bf16>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(key_mass_generic_kernel<float>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t m = (size_t)a.B * a.N;
    hipLaunchKernelGGL(key_mass_sum_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, a.part, a.scores,
                       a.B, a.Hkv, a.N);
    return hipGetLastError();
}

hipError_t launch_select_top(const float* scores, const uint8_t* cand, int B, int N, int k, int32_t* out,
                             hipStream_t s)
{
    if (B == 0 || k == 0) return hipSuccess;
    if (N < 1 || N > kTopThreads * kTopPer) return hipErrorInvalidValue;
    // slots for the selected keys: a power of two >= min(k, N)
    const int m = std::min(k, N);
    int n2 = 1;
    while (n2 < m) n2 <<= 1;
    const size_t shm = std::max((size_t)n2 * sizeof(uint64_t), (size_t)2 * kTopWaves * 256 * sizeof(int));
    (void)allow_full_lds<select_top_kernel>();
    (void)hipGetLastError();
    hipLaunchKernelGGL(select_top_kernel, dim3(B), dim3(kTopThreads), shm, s, scores, cand, N, n2, k, out);
    return hipGetLastError();
}

}  // namespace fdllm
