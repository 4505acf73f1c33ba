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
//  * one or two producer waves stream K/V tiles straight into a ring of LDS
//    stages with global_load_lds (16 B per lane, no registers), each keeping
//    at most 48 of its loads (48 KB) in flight; a producer waits on its own
//    vmcnt and releases each stage with a barrier.  The consumer waves never
//    issue global loads in the loop, they only read LDS and run MFMAs;
//  * LDS rows are 256 B with their 16 B chunks XOR-swizzled by the row index:
//    the K fragment reads are conflict-free; the transposed V reads are not
//    entirely (the bank-conflict counter reads about a third of the
//    LDS-active cycles on the long-context layer; a swizzle aimed at them
//    doubled it);
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 leaves each lane with one query
//    row, so the row max needs two cross-lane steps and the rescale of the
//    output accumulators is lane-local; q enters as bf16 hi + lo parts so the
//    scores keep q's fp32 accumulation precision, and the accumulators start
//    at the row's -reference max, so the exponentials need no subtraction;
//  * O^T += V^T P^T takes V^T fragments from the row-major tile with
//    ds_read_b64_tr_b16 (gfx950 transpose read) and P^T from the score
//    registers, so P never goes through LDS;
//  * consumer waves split the query rows and the keys of a tile; key-split
//    waves merge their softmax states through LDS at the end;
//  * with several cache splits, each writes its (max, sum, normalised bf16
//    output) partial state and a small second kernel merges them into O and
//    LSE (a kernel boundary is far cheaper than a device-scope fence per
//    workgroup).
//
// Key set of query row i (same definition as the CPU oracle): every cache
// position not written by this step, plus each new row j that i may see.  A
// position written by its first row j is reached through the cache (the
// projection kernel stored it there) and gated by vis[i][j]; later rows at a
// shared position live in the side buffer and are attended as extra tiles.
// Which rows own their position is read from the flags the projection
// recorded while deciding where to store each row.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kDH = 128;
constexpr int kRowB = kDH * 2;        // bytes of one K or V row
constexpr int kRing = 128 * 1024;     // LDS ring of K/V stages per workgroup (default)
constexpr int kMaxChunks = 5;         // query rows per sequence, in chunks of 64 (R <= 288)
constexpr float kNegBig = -1.0e30f;   // running max of a row that has seen no key

typedef __bf16 bf16x4g __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16x4g lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// RG row groups of 16 query rows per consumer wave, NWR x NWK consumer waves
// (rows x keys of a tile), NPROD producer waves.
template <int RG, int NWR, int NWK, int NPROD, int RING = kRing>
struct AttnCfg {
    static constexpr int NC = NWR * NWK;            // consumer waves
    static constexpr int NT = (NC + NPROD) * 64;
    static constexpr int KW = 32;                   // keys per consumer wave per tile
    static constexpr int TK = KW * NWK;             // keys per tile
    static constexpr int STAGE = TK * 2 * kRowB;    // K rows then V rows
    static constexpr int NS = RING / STAGE;
    static constexpr int DMA = STAGE / 1024;        // 1 KB DMA instructions per stage
    static constexpr int DMAP = DMA / NPROD;        // ... issued by each producer wave
    // stages in flight per producer: at most 48 of its loads, so an issue
    // never stalls on the 63-load counter (a stalled issue would hold back
    // the release of the oldest stage)
    static constexpr int AHEAD0 = 48 / DMAP > 1 ? 48 / DMAP : 1;
    static constexpr int AHEAD = AHEAD0 < NS - 1 ? AHEAD0 : NS - 1;
    static constexpr int MERGE = (NWK / 2) * NWR * RG * 64 * (32 + 2) * 4;
    static constexpr int SCRATCH = NS * STAGE > MERGE ? NS * STAGE : MERGE;
    static_assert(NS >= 2 && NS * STAGE == RING, "stage ring");
    static_assert(DMA % (2 * NPROD) == 0, "K and V halves split evenly over the producers");
};

// Producer wait: this wave's loads of stage t have landed once at most
// `younger` * DMAP of its loads are in flight (loads complete in order and
// the counter saturates at 63); then release the stage with the barrier.
template <int N>
__device__ __forceinline__ void producer_release()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int DMAP, int Y>
__device__ __forceinline__ void producer_sync(int younger)
{
    if constexpr (Y <= 0) {
        producer_release<0>();
    } else {
        if (younger >= Y) producer_release<(Y * DMAP > 63 ? 63 : Y * DMAP)>();
        else producer_sync<DMAP, Y - 1>(younger);
    }
}

// Consumer side of the same barrier: its LDS reads of the previous stage have
// returned (so the producer may overwrite that stage).
__device__ __forceinline__ void consumer_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void dma16(const unsigned char* src, unsigned char* dst)
{
    __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)dst, 16, 0, 0);
}

// max and sum over the four lanes l, l^16, l^32, l^48 (the 16-lane groups of
// a wave), with the gfx950 row-swap permutes
__device__ __forceinline__ float max4(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float sum4(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
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

// One stage of cache rows: TK rows from key `base` (rows past the split end
// repeat its last key and are masked later), K then V, as 1 KB DMA blocks of
// 4 rows; chunk c of row r lands in slot c ^ (r & 15).  Producer p issues
// blocks p, p + NPROD, ...
// Cache row of key `key` in bytes: the (sequence, kv head) slab of the flat
// layout, or through the block table staged in LDS (sTab != NULL).
__device__ __forceinline__ size_t key_offset(int key, const int* sTab, int bits, int Hkv, int g)
{
    if (!sTab) return (size_t)key * kRowB;
    return (((((size_t)sTab[key >> bits] * Hkv + g) << bits) + (key & ((1 << bits) - 1)))) * kRowB;
}

template <int TK, int DMA, int NPROD>
__device__ __forceinline__ void issue_main(unsigned char* st, int base, int klast, const unsigned char* Kg,
                                           const unsigned char* Vg, int p, int lane, const int* sTab, int bits,
                                           int Hkv, int g)
{
    const int srow = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int ii = 0; ii < DMA / 2 / NPROD; ++ii) {
        const int i = ii * NPROD + p;
        const int row = 4 * i + srow;
        const int key = min(base + row, klast);
        const size_t src = key_offset(key, sTab, bits, Hkv, g) + ((slot ^ (row & 15)) << 4);
        dma16(Kg + src, st + i * 1024);
        dma16(Vg + src, st + TK * kRowB + i * 1024);
    }
}

// A stage of side-buffer rows: duplicate number base + r is query row sDup[.]
template <int TK, int DMA, int NPROD>
__device__ __forceinline__ void issue_dup(unsigned char* st, int base, int ndup, const int* sDup,
                                          const unsigned char* SKg, const unsigned char* SVg, int p, int lane)
{
    const int srow = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int ii = 0; ii < DMA / 2 / NPROD; ++ii) {
        const int i = ii * NPROD + p;
        const int row = 4 * i + srow;
        const int j = sDup[min(base + row, ndup - 1)];
        const size_t src = (size_t)j * kRowB + ((slot ^ (row & 15)) << 4);
        dma16(SKg + src, st + i * 1024);
        dma16(SVg + src, st + TK * kRowB + i * 1024);
    }
}

template <int RG, int NWR, int NWK, int NPROD, int RING>
__global__ void __launch_bounds__((NWR * NWK + NPROD) * 64)
attn_mfma_kernel(AttnArgs a)
{
    using C = AttnCfg<RG, NWR, NWK, NPROD, RING>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int kps = a.keys_per_split;
    const int nq = a.nq;
    const int G = a.G;
    const int VW = (nq + 31) >> 5;                  // 32-bit words per visibility row
    const int tiles_max = (kps + C::TK - 1) / C::TK;
    int16_t* sSlot = (int16_t*)(smem + C::SCRATCH); // [kps] row owning a written position, or -1
    // [tiles][2] bit k of a tile: its key k is a position written this step
    uint32_t* sMask = (uint32_t*)(smem + C::SCRATCH + 2 * ((kps + 1) & ~1));
    uint32_t* sVis = sMask + 2 * tiles_max;         // [nq][VW] visibility bits
    int* sDup = (int*)(sVis + (size_t)nq * VW);     // [nq] rows that do not own their position
    int* sMisc = sDup + nq;                         // [0] number of such rows
    int* sTabLds = sMisc + 1;                       // [max_blocks] block table of the sequence (paged)
    // under a mask, when they fit: per query row and 32-key word of the split,
    // the written keys the row may not see (hidden); per owner row, its
    // key's offset in the split; per 32 rows, the rows that own a key of it
    const int TWS = kps >> 5;
    uint32_t* sHid = (uint32_t*)(sTabLds + (a.map.table != nullptr ? a.map.max_blocks : 0));   // [nq][TWS]
    int* sKt = (int*)(sHid + (size_t)nq * TWS);     // [32 VW]
    uint32_t* sOwnIn = (uint32_t*)(sKt + 32 * VW);  // [VW]
    const bool hid = a.hid_words != 0;

    const int total = a.B * a.Hkv * a.splits;
    const int logical = xcd_remap(blockIdx.x, total);
    if (logical < 0) return;
    const int bg = logical / a.splits;
    const int split = logical - bg * a.splits;
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    // valid positions and query rows of this sequence (all N and nq unless
    // the caller passes per-sequence lengths); a split past the valid
    // positions streams one masked tile of valid rows
    const int L = a.seq_len ? min(a.seq_len[b], a.N) : a.N;
    const int nqb = a.nq_seq ? a.nq_seq[b] : nq;
    const int k0 = split * kps;
    const int k1 = min(L, k0 + kps);
    const int klast = k1 > k0 ? k1 - 1 : L - 1;
    const int n_main = k1 > k0 ? (k1 - k0 + C::TK - 1) / C::TK : 1;
    const bool paged = a.map.table != nullptr;
    const int* sTab = paged ? sTabLds : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform in an SGPR, so branches on it stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const bool producer = wave >= C::NC;
    const int wk = wave % NWK, wr = wave / NWK;    // consumer coordinates
    const int nch = (nq + 63) >> 6;                 // 64-row chunks of the query set

    const size_t cache_off = paged ? 0 : (size_t)bg * a.N * kDH;
    const unsigned char* Kg = (const unsigned char*)((const bf16*)a.Kc + cache_off);
    const unsigned char* Vg = (const unsigned char*)((const bf16*)a.Vc + cache_off);
    const unsigned char* SKg = (const unsigned char*)((const bf16*)a.sideK + (size_t)bg * a.q_max * kDH);
    const unsigned char* SVg = (const unsigned char*)((const bf16*)a.sideV + (size_t)bg * a.q_max * kDH);
    const int32_t* pos_b = a.pos_ids + (size_t)b * nq;
    const uint8_t* vis_b = a.vis ? a.vis + (size_t)b * nq * nq : nullptr;
    const int nunits = vis_b ? nq * nch : 0;        // (visibility row, 64-column chunk) pairs

    // ---- every global load of the consumers is issued before the producers
    //      start streaming, so none of them waits behind the K/V tiles
    f32x4 qraw[RG][8];
    int posr[kMaxChunks], ownr[kMaxChunks];
    int vbyte[8];
    if (!producer) {
        const float* qbase = a.qbuf + (size_t)bg * a.q_max * G * kDH;
        // indices are clamped into range and the values of padding lanes
        // discarded afterwards, so the loads carry no branches
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = min((wr * RG + rg) * 16 + lr, a.R - 1);
#pragma unroll
            for (int h = 0; h < 8; ++h)
                qraw[rg][h] = *(const f32x4*)(qbase + (size_t)row * kDH + (h >> 1) * 32 + lg * 8 + (h & 1) * 4);
        }
        if (wave == 0) {
            const int8_t* own_b = a.own + (size_t)b * nq;
#pragma unroll
            for (int c = 0; c < kMaxChunks; ++c)
                if (64 * c < nq) {
                    posr[c] = pos_b[min(64 * c + lane, nq - 1)];
                    ownr[c] = own_b[min(64 * c + lane, nq - 1)];
                }
        }
        // a few mask rows: their bytes, one per lane (under a mask these are
        // read before the stream starts: issued after it they would queue
        // behind the first stages' DMA)
        if (vis_b && nunits <= 8 * C::NC) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int u = min(wave + C::NC * t, nunits - 1);
                const int i = u / nch, col = min((u - i * nch) * 64 + lane, nq - 1);
                vbyte[t] = vis_b[(size_t)i * nq + col];
            }
        }
        if (vis_b) {
            for (int k = tid; k < kps; k += C::NC * 64) sSlot[k] = -1;
            for (int t = tid; t < 2 * n_main; t += C::NC * 64) sMask[t] = 0u;
        }
        if (hid) {
            for (int t = tid; t < nq * TWS; t += C::NC * 64) sHid[t] = 0u;
            for (int t = tid; t < VW; t += C::NC * 64) sOwnIn[t] = 0u;
        }
        if (paged) {
            const int32_t* tb = a.map.table + (size_t)b * a.map.max_blocks;
            for (int t = tid; t < a.map.max_blocks; t += C::NC * 64) sTabLds[t] = tb[t];
        }
    }
    // a plain barrier: the LDS writes above must land, but the loads stay in
    // flight (a full __syncthreads would wait for them before the stream starts)
    consumer_sync();

    float m_run[RG], l_run[RG];
    // the score accumulators start at -ref, so a row's scores come out
    // relative to its reference max (ref = 0 until the row has one)
    f32x4 negref[RG];
    f32x4 o[RG][8];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        m_run[rg] = kNegBig;
        l_run[rg] = 0.f;
        negref[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (producer) {
        // ================= producer waves: K/V tiles -> LDS ring =================
        const int p = wave - C::NC;
        int issued = 0;
        for (; issued < min(C::AHEAD, n_main); ++issued)
            issue_main<C::TK, C::DMA, NPROD>(smem + (issued % C::NS) * C::STAGE, k0 + issued * C::TK, klast, Kg, Vg, p,
                                             lane, sTab, a.map.bits, a.Hkv, g);
        int ntot = n_main;
        int ndup = 0;
        // the consumers' extra barrier between their bookkeeping and the
        // hidden-key words (the stages stay in flight)
        if (hid) asm volatile("s_barrier" ::: "memory");
        for (int t = 0;; ++t) {
            producer_sync<C::DMAP, C::AHEAD - 1>(issued - t - 1);
            if (t == 0 && split == 0) {
                // the consumers published the duplicate rows before this barrier
                ndup = __builtin_amdgcn_readfirstlane(sMisc[0]);
                ntot = n_main + (ndup + C::TK - 1) / C::TK;
            }
            if (t + 1 >= ntot) break;
            for (; issued < ntot && issued < t + 1 + C::AHEAD; ++issued) {
                unsigned char* st = smem + (issued % C::NS) * C::STAGE;
                if (issued < n_main)
                    issue_main<C::TK, C::DMA, NPROD>(st, k0 + issued * C::TK, klast, Kg, Vg, p, lane, sTab,
                                                     a.map.bits, a.Hkv, g);
                else
                    issue_dup<C::TK, C::DMA, NPROD>(st, (issued - n_main) * C::TK, ndup, sDup, SKg, SVg, p, lane);
            }
        }
    } else {
        // ================= consumer waves =================
        // per-sequence bookkeeping while the first tiles stream in
        if (wave == 0) {
            // row j owns the cache write of its position unless an earlier
            // row has the same position (the projection recorded which rows
            // do); the others are listed in sDup
            int ndup = 0;
#pragma unroll
            for (int c = 0; c < kMaxChunks; ++c) {
                if (64 * c >= nq) break;
                const int j = 64 * c + lane;
                const bool own = ownr[c] > 0;
                const bool valid = j < nqb;
                const uint64_t dm = __builtin_amdgcn_ballot_w64(valid && !own);
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(dm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)dm, 0u));
                if (valid && !own) sDup[ndup + below] = j;
                ndup += __builtin_popcountll(dm);
                const bool inr = vis_b && valid && own && posr[c] >= k0 && posr[c] < k1;
                if (inr) {
                    const int kt = posr[c] - k0;
                    sSlot[kt] = (int16_t)j;
                    atomicOr(&sMask[2 * (kt / C::TK) + ((kt % C::TK) >> 5)], 1u << (kt & 31));
                    if (hid) sKt[j] = kt;
                }
                if (hid) {
                    const uint64_t om = __builtin_amdgcn_ballot_w64(inr);
                    if (lane == 0) {
                        sOwnIn[2 * c] = (uint32_t)om;
                        if (2 * c + 1 < VW) sOwnIn[2 * c + 1] = (uint32_t)(om >> 32);
                    }
                }
            }
            if (lane == 0) sMisc[0] = ndup;
        }
        // visibility rows as bit words: chunk c of row i fills words 2c, 2c+1
        // (only under a mask: without one no key is gated by visibility)
        if (vis_b && nunits <= 8 * C::NC) {
            // (the bytes were loaded before the stream started)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int u = wave + C::NC * t;
                if (u < nunits) {
                    const int i = u / nch, c = u - i * nch;
                    const uint64_t m = __builtin_amdgcn_ballot_w64(vbyte[t] != 0 && c * 64 + lane < nq);
                    if (lane == 0) {
                        sVis[i * VW + 2 * c] = (uint32_t)m;
                        if (2 * c + 1 < VW) sVis[i * VW + 2 * c + 1] = (uint32_t)(m >> 32);
                    }
                }
            }
        } else if (vis_b) {
            // a large mask: each thread packs whole 32-column words, with the
            // loads of four words in flight at once (addresses are clamped
            // into the matrix and the bytes past the row end dropped)
            const int nwords = nq * VW;
            const size_t last = (size_t)nq * nq - 1;
            for (int w0 = tid; w0 < nwords; w0 += C::NC * 64 * 4) {
                uint32_t dw[4][8];
                int cols[4];
                if ((nq & 15) == 0) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int w = min(w0 + k * C::NC * 64, nwords - 1);
                        const int i = w / VW, c32 = w - i * VW;
                        cols[k] = min(32, nq - 32 * c32);
                        const uint8_t* row = vis_b + (size_t)i * nq;
                        const u32x4 lo = *(const u32x4*)(row + 32 * c32);
                        const u32x4 hi = *(const u32x4*)(row + (cols[k] > 16 ? 32 * c32 + 16 : 32 * c32));
#pragma unroll
                        for (int e = 0; e < 4; ++e) { dw[k][e] = lo[e]; dw[k][4 + e] = hi[e]; }
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int w = min(w0 + k * C::NC * 64, nwords - 1);
                        const int i = w / VW, c32 = w - i * VW;
                        cols[k] = min(32, nq - 32 * c32);
                        const size_t b0 = (size_t)i * nq + 32 * c32;
#pragma unroll
                        for (int d = 0; d < 8; ++d) {
                            uint32_t x = 0;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                x |= (uint32_t)vis_b[min(b0 + 4 * d + e, last)] << (8 * e);
                            dw[k][d] = x;
                        }
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int w = w0 + k * C::NC * 64;
                    if (w >= nwords) continue;
                    uint32_t bits = 0u;
#pragma unroll
                    for (int d = 0; d < 8; ++d)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bits |= (((dw[k][d] >> (8 * e)) & 0xffu) != 0u ? 1u : 0u) << (4 * d + e);
                    if (cols[k] < 32) bits &= (1u << cols[k]) - 1u;
                    sVis[w] = bits;
                }
            }
        }

        // query fragments: lane holds row (wr*RG + rg)*16 + lr, dims 32c + 8lg .. +7,
        // as bf16 hi + lo parts so the scores keep q's fp32 precision; the
        // scale (log2 e / sqrt(dh)) puts the scores in log2 units
        bf16x8 qh[RG][4], ql[RG][4];
        int qrow[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = (wr * RG + rg) * 16 + lr;
            qrow[rg] = (row < a.R && row / G < nqb) ? row / G : -1;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = qraw[rg][2 * c + (e >> 2)][e & 3] * a.scale_log2;
                    const bf16 hi = (bf16)x;
                    qh[rg][c][e] = hi;
                    ql[rg][c][e] = (bf16)(x - (float)hi);
                }
        }

        // hidden-key words: pair (64-row chunk, 32-owner word) per wave
        // iteration, a lane per query row; each owner of a key in the split
        // that the row may not see sets the key's bit in the row's word.
        // Wave 0 comes to the barrier last (it did the owner bookkeeping), so
        // the pairs are dealt from the last wave down.
        if (hid) {
            consumer_sync();   // owner bookkeeping and visibility words are in LDS
            const int npairs = ((nq + 63) >> 6) * VW;
            for (int pr = C::NC - 1 - wave; pr < npairs; pr += C::NC) {
                const int rc = pr / VW, ow = pr - rc * VW;
                uint32_t om = __builtin_amdgcn_readfirstlane(sOwnIn[ow]);
                const int jrow = 64 * rc + lane;
                const int ktv = sKt[32 * ow + (lane & 31)];   // lane k < 32: owner 32 ow + k
                const uint32_t seen = jrow < nq ? sVis[jrow * VW + ow] : ~0u;
                const uint32_t hm = om & ~seen;
                if (__builtin_amdgcn_ballot_w64(hm != 0u) == 0) continue;   // every row sees these owners
                while (om != 0u) {
                    const int k = __builtin_ctz(om);
                    om &= om - 1u;
                    const int kt = __builtin_amdgcn_readlane(ktv, k);
                    if ((hm >> k) & 1u) atomicOr(&sHid[jrow * TWS + (kt >> 5)], 1u << (kt & 31));
                }
            }
        }

        // per-lane LDS offsets of the fragments within a stage
        int kofs[4], vofs[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) kofs[c] = (wk * C::KW + lr) * kRowB + (((c * 4 + lg) ^ lr) << 4);
        const int rowA = wk * C::KW + 4 * lg + (lr >> 2);   // (rowA + 16 has the same swizzle)
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int chunk = 2 * db + ((lr & 3) >> 1);
            vofs[db] = C::TK * kRowB + rowA * kRowB + ((chunk ^ (rowA & 15)) << 4) + ((lr & 1) << 3);
        }

        int ntot = n_main;
        int ndup = 0;
        for (int it0 = 0; it0 < ntot; it0 += C::NS) {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const int it = it0 + s;
                if (it >= ntot) break;
                consumer_sync();
                if (it == 0 && split == 0) {
                    ndup = __builtin_amdgcn_readfirstlane(sMisc[0]);
                    ntot = n_main + (ndup + C::TK - 1) / C::TK;
                }
                const unsigned char* st = smem + s * C::STAGE;
                // this lane's hidden-key bits of the wave's 32 keys (rows past
                // the live ones hide every written key), read ahead of the MFMAs
                uint32_t hw[RG];
                if (hid) {
                    const int itc = min(it, n_main - 1);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
                        hw[rg] = qrow[rg] >= 0 ? sHid[qrow[rg] * TWS + itc * NWK + wk] : sMask[2 * itc + wk];
                }

                // ---- S^T = K Q^T for this wave's 32 keys (rows past R run on zero q)
                constexpr int KB = C::KW / 16;                 // 16-key blocks per wave
                bf16x8 kf[KB][4];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int c = 0; c < 4; ++c) kf[kb][c] = *(const bf16x8*)(st + kofs[c] + kb * 16 * kRowB);
                // The accumulators start at the row's -ref.  With four or more
                // accumulators one chain each takes the hi then the lo products;
                // with fewer, the lo products go to a second set of chains (so
                // back-to-back MFMAs do not depend on each other) added at the end.
                f32x4 sc[RG][KB];
                if constexpr (RG * KB >= 4) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int rg = 0; rg < RG; ++rg)
                                sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    kf[kb][c], qh[rg][c], c == 0 ? negref[rg] : sc[rg][kb], 0, 0, 0);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int rg = 0; rg < RG; ++rg)
                                sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][c], ql[rg][c], sc[rg][kb], 0, 0, 0);
                } else {
                    f32x4 sl[RG][KB];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int rg = 0; rg < RG; ++rg)
                                sc[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    kf[kb][c], qh[rg][c], c == 0 ? negref[rg] : sc[rg][kb], 0, 0, 0);
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int rg = 0; rg < RG; ++rg)
                                sl[rg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    kf[kb][c], ql[rg][c], c == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sl[rg][kb], 0, 0, 0);
                    }
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) sc[rg][kb] += sl[rg][kb];
                }
                // all K fragment reads are issued before the first MFMA waits on one
                __builtin_amdgcn_sched_group_barrier(0x100, 4 * KB, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 8 * KB * RG, 0);

                // ---- masks (lane: row lr, keys kb*16 + 4lg + i of the wave's 32).
                // Under a visibility mask a tile holding positions written this
                // step gates just those keys; the split's last tile and the
                // duplicate tiles take the general path.
                const bool dup = it >= n_main;
                const int tbase = dup ? (it - n_main) * C::TK : k0 + it * C::TK;
                const int kend = dup ? ndup : k1;
                // this wave's 32 bits of the tile's written-key mask; with
                // more than a few written keys the per-lane general path is
                // cheaper than visiting them one at a time
                uint32_t wm = vis_b && !dup && !hid ? __builtin_amdgcn_readfirstlane(sMask[2 * it + wk]) : 0u;
                if (dup || tbase + C::TK > kend || __builtin_popcount(wm) > 2) {
                    // branch-free: every lane reads its keys' owners and its
                    // rows' visibility words at clamped (valid) indices
                    if (vis_b != nullptr) {
                        int jk[KB][4];
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = tbase + wk * C::KW + kb * 16 + lg * 4 + i;
                                const int kk = max(min(key, kend - 1), dup ? 0 : k0);
                                const int j = dup ? sDup[kk] : (int)sSlot[kk - k0];
                                jk[kb][i] = key < kend ? j : -2;      // -2: past the end
                            }
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int j = jk[kb][i];
                                const int jc = max(j, 0);
#pragma unroll
                                for (int rg = 0; rg < RG; ++rg) {
                                    const uint32_t w = sVis[max(qrow[rg], 0) * VW + (jc >> 5)];
                                    const bool seen = qrow[rg] >= 0 && ((w >> (jc & 31)) & 1u);
                                    const bool keep = j == -1 || (j >= 0 && seen);
                                    sc[rg][kb][i] = keep ? sc[rg][kb][i] : -INFINITY;
                                }
                            }
                    } else {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = tbase + wk * C::KW + kb * 16 + lg * 4 + i;
#pragma unroll
                                for (int rg = 0; rg < RG; ++rg)
                                    sc[rg][kb][i] = key < kend ? sc[rg][kb][i] : -INFINITY;
                            }
                    }
                } else if (hid) {
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if ((hw[rg] >> (kb * 16 + lg * 4 + i)) & 1u) sc[rg][kb][i] = -INFINITY;
                } else if (vis_b) {
                    while (wm != 0u) {
                        const int k = __builtin_ctz(wm);          // key wk*32 + k of the tile
                        wm &= wm - 1u;
                        const int j = __builtin_amdgcn_readfirstlane(sSlot[it * C::TK + wk * C::KW + k]);
                        const bool mine = lg == ((k >> 2) & 3);
#pragma unroll
                        for (int rg = 0; rg < RG; ++rg) {
                            const bool hide = mine && (qrow[rg] < 0 ||
                                                       !((sVis[max(qrow[rg], 0) * VW + (j >> 5)] >> (j & 31)) & 1u));
#pragma unroll
                            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    if (kb == (k >> 4) && i == (k & 3) && hide) sc[rg][kb][i] = -INFINITY;
                        }
                    }
                }

                // ---- online softmax.  Lazy rescale: a row's exponentials stay
                // relative to a reference max that only moves when the row's
                // max exceeds it by more than 2^8, so p <= 256 and the
                // accumulators are rescaled a few times per split.  The
                // decision is per row; the block is skipped when no row grows.
                // The scores are already relative to the reference (ref), so
                // the exponent needs no subtraction unless the reference moves.
                float pv[RG][KB][4];
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    float mx = fmaxf(fmaxf(sc[rg][0][0], sc[rg][0][1]), fmaxf(sc[rg][0][2], sc[rg][0][3]));
#pragma unroll
                    for (int kb = 1; kb < KB; ++kb)
                        mx = fmaxf(mx, fmaxf(fmaxf(sc[rg][kb][0], sc[rg][kb][1]), fmaxf(sc[rg][kb][2], sc[rg][kb][3])));
                    mx = max4(mx);
                    const float ref = -negref[rg][0];
                    const bool grow = mx + ref > m_run[rg] + 8.f;
                    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                        const float shift = grow ? mx : 0.f;
                        if (grow) {
                            const float mnew = mx + ref;
                            const float alpha = __builtin_amdgcn_exp2f(m_run[rg] - mnew);
                            l_run[rg] *= alpha;
#pragma unroll
                            for (int db = 0; db < 8; ++db) o[rg][db] *= alpha;
                            m_run[rg] = mnew;
                            negref[rg] = f32x4{-mnew, -mnew, -mnew, -mnew};
                        }
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) sc[rg][kb][i] -= shift;
                    }
                    float lsum = 0.f;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pv[rg][kb][i] = __builtin_amdgcn_exp2f(sc[rg][kb][i]);   // exp2(-inf) = 0
                            lsum = kb == 0 && i == 0 ? pv[rg][0][0] : lsum + pv[rg][kb][i];
                        }
                    l_run[rg] += lsum;
                }

                // ---- O^T += V^T P^T over the wave's 32 keys
                bf16x8 pf[RG];
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pf[rg][i] = (bf16)pv[rg][0][i];
                        pf[rg][4 + i] = (bf16)pv[rg][1][i];
                    }
                bf16x8 vf[8];
#pragma unroll
                for (int db = 0; db < 8; ++db) vf[db] = read_vt_frag(st + vofs[db], st + vofs[db] + 16 * kRowB);
#pragma unroll
                for (int db = 0; db < 8; ++db)
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
                        o[rg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf[rg], o[rg][db], 0, 0, 0);
            }
        }

        // per-lane sums -> row sums (row lr is spread over the 4 lane groups)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) l_run[rg] = sum4(l_run[rg]);
    }
    __syncthreads();   // the LDS ring is free from here on

    // ---- merge the key-split consumer waves through LDS (tree over wk)
    const bool consumer = !producer;
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
                    const float fa = __builtin_amdgcn_exp2f(m_run[rg] - mn);
                    const float fb = __builtin_amdgcn_exp2f(mb - mn);
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
                if (j >= nqb) {   // padding row of a shorter sequence: zero output
                    l_run[rg] = 0.f;
#pragma unroll
                    for (int db = 0; db < 8; ++db) o[rg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
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

    // publish this split's partial state (max in log2 units, sum, and the
    // split's normalised output O_s / l_s in bf16: half the bytes of the
    // unnormalised fp32 sum, and a weighted mean of values the output is
    // rounded to anyway); the combine kernel merges the splits after this
    // launch ends
    if (writer) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int row = (wr * RG + rg) * 16 + lr;
            if (row >= a.R) continue;
            const size_t prow = ((size_t)bg * a.splits + split) * a.Rpad + row;
            bf16* pp = a.apart + prow * kDH;
            const float inv = l_run[rg] > 0.f ? 1.f / l_run[rg] : 0.f;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                bf16x4v v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[rg][db][i] * inv);
                *(bf16x4v*)(pp + db * 16 + lg * 4) = v;
            }
            if (lg == 0) {
                a.aml[prow * 2 + 0] = m_run[rg];
                a.aml[prow * 2 + 1] = l_run[rg];
            }
        }
    }
}

// Merge of the cache splits: O = sum_s 2^(m_s - M) l_s O_s / L and
// LSE = (M + log2 L) ln 2 with M = max_s m_s, L = sum_s 2^(m_s - M) l_s, where
// O_s is split s's normalised output.
// A workgroup takes 8 query rows of one (sequence, kv head): the (m, l) of
// every split go through LDS first, then each thread sums 4 output dims of
// its row over the splits with the loads of 8 splits in flight at a time.
constexpr int kCombineRows = 8;

__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a)
{
    extern __shared__ float sW[];   // [kCombineRows][S]: split maxima, then their weights
    const int S = a.splits;
    const int wgs_per_bg = (a.R + kCombineRows - 1) / kCombineRows;
    const int bg = blockIdx.x / wgs_per_bg;
    const int r0 = (blockIdx.x - bg * wgs_per_bg) * kCombineRows;
    const int tid = threadIdx.x;
    const size_t pbase = (size_t)bg * S * a.Rpad;
    for (int t = tid; t < kCombineRows * S; t += 256) {
        const int r = t / S, sp = t - r * S;
        sW[t] = a.aml[(pbase + (size_t)sp * a.Rpad + min(r0 + r, a.R - 1)) * 2];
    }
    __syncthreads();
    // the 32 threads of a row reduce its maxima, then turn them into weights
    const int r = tid >> 5, d4 = tid & 31;
    float mx = kNegBig;
    for (int sp = d4; sp < S; sp += 32) mx = fmaxf(mx, sW[r * S + sp]);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
    __syncthreads();
    for (int sp = d4; sp < S; sp += 32) sW[r * S + sp] = __builtin_amdgcn_exp2f(sW[r * S + sp] - mx);
    __syncthreads();
    const int row = r0 + r;
    const int rowc = min(row, a.R - 1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    int sp = 0;
    auto to_f32x4 = [](bf16x4v v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; };
    for (; sp + 8 <= S; sp += 8) {
        bf16x4v v[8];
        float l[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t pr = pbase + (size_t)(sp + u) * a.Rpad + rowc;
            v[u] = *(const bf16x4v*)(a.apart + pr * kDH + d4 * 4);
            l[u] = a.aml[pr * 2 + 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float wl = sW[r * S + sp + u] * l[u];
            acc += to_f32x4(v[u]) * wl;
            L += wl;
        }
    }
    for (; sp < S; ++sp) {
        const size_t pr = pbase + (size_t)sp * a.Rpad + rowc;
        const float wl = sW[r * S + sp] * a.aml[pr * 2 + 1];
        acc += to_f32x4(*(const bf16x4v*)(a.apart + pr * kDH + d4 * 4)) * wl;
        L += wl;
    }
    if (row >= a.R) return;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const int j = row / a.G, hl = row - j * a.G;
    if (a.nq_seq && j >= a.nq_seq[b]) {     // padding row of a shorter sequence
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        L = 0.f;
    }
    const size_t orow = ((size_t)b * a.nq + j) * a.H + g * a.G + hl;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    bf16x4v v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(acc[i] * inv);
    *(bf16x4v*)((bf16*)a.O + orow * kDH + d4 * 4) = v;
    if (d4 == 0) a.LSE[orow] = L > 0.f ? (mx + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

template <int RG, int NWR, int NWK, int NPROD, int RING = kRing>
hipError_t launch_cfg(const AttnArgs& a0, hipStream_t s)
{
    using C = AttnCfg<RG, NWR, NWK, NPROD, RING>;
    AttnArgs a = a0;
    if (a.nq > 64 * kMaxChunks || a.keys_per_split % C::TK != 0) return hipErrorInvalidValue;
    const int VW = (a.nq + 31) / 32;
    const int tiles = (a.keys_per_split + C::TK - 1) / C::TK;
    const size_t book = 2 * (size_t)((a.keys_per_split + 1) & ~1) + 8 * (size_t)tiles + 4 * (size_t)a.nq * VW +
                        4 * ((size_t)a.nq + 1) + (a.map.table ? 4 * (size_t)a.map.max_blocks : 0);
    if (C::SCRATCH + book > 160 * 1024) return hipErrorInvalidValue;
    // hidden-key words under a mask, when the step writes more than two keys
    // per 32 of the split on average (fewer are gated one at a time in the
    // loop at less cost than the words' extra barrier and build) and the
    // words fit beside the rest
    const size_t hid = 4 * (size_t)a.nq * (a.keys_per_split / 32) + 4 * 32 * (size_t)VW + 4 * (size_t)VW;
    a.hid_words = a.vis != nullptr && a.nq > 2 * (a.keys_per_split / 32) && C::SCRATCH + book + hid <= 160 * 1024;
    const size_t shm = C::SCRATCH + book + (a.hid_words ? hid : 0);
    const int total = a.B * a.Hkv * a.splits;
    const int grid = ((total + 7) / 8) * 8;
    constexpr auto kern = attn_mfma_kernel<RG, NWR, NWK, NPROD, RING>;
    // the dynamic LDS limit is raised once per device; a refusal shows up as
    // a launch error below
    (void)allow_full_lds<kern>();
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), shm, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    const int cgrid = a.B * a.Hkv * ((a.R + kCombineRows - 1) / kCombineRows);
    const size_t cshm = sizeof(float) * kCombineRows * (size_t)a.splits;
    if (cshm > 64 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(cgrid), dim3(256), cshm, s, a);
    return hipGetLastError();
}

}  // namespace

// Keys per tile of the configuration chosen for R query rows per kv head.
int attn_mfma_tile_keys(int R)
{
    const int r16 = (R + 15) / 16;
    return r16 <= 6 ? 64 : 32;
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s)
{
    if (a.B * a.Hkv * a.splits == 0 || a.R == 0) return hipSuccess;
    if (!a.own) return hipErrorInvalidValue;   // the projection's ownership flags are required
    // row groups of 16 per wave x row waves x key waves x producer waves; at
    // most two waves per SIMD once a wave holds two or more row groups
    const int r16 = (a.R + 15) / 16;
    if (r16 <= 1) return launch_cfg<1, 1, 2, 1>(a, s);
    if (r16 <= 2) return launch_cfg<1, 2, 2, 2>(a, s);
    // up to three row groups: with the cache split (few kv heads, as in a
    // draft pass of one sequence) each workgroup streams only a few tiles,
    // and one wave per row group taking all keys of a tile avoids the
    // key-split waves' merge at the end (draft pass: step 35.8 -> 34.8 us);
    // over whole caches the key split's two waves per SIMD are faster
    // (verification layer: 54 against 61 us)
    if (r16 <= 3) return a.splits > 1 ? launch_cfg<1, 3, 1, 2>(a, s) : launch_cfg<1, 3, 2, 2>(a, s);
    if (r16 <= 4) {
        // more workgroups than CUs: 32-key tiles in a 64 KB ring, so two
        // workgroups share a CU and the launch runs in one round
        if ((long)a.B * a.Hkv * a.splits > 256) return launch_cfg<1, 4, 1, 2, 64 * 1024>(a, s);
        return launch_cfg<1, 4, 2, 2>(a, s);
    }
    if (r16 <= 6) return launch_cfg<2, 3, 2, 2>(a, s);
    // 9 to 11 row groups: one row group per wave, two or three waves on each
    // SIMD (with two row groups a wave, the busiest SIMD carried four: 2-7 %
    // slower on the default-window workloads)
    if (r16 <= 9) return launch_cfg<1, 9, 1, 2>(a, s);
    if (r16 <= 10) return launch_cfg<1, 10, 1, 2>(a, s);
    if (r16 <= 11) return launch_cfg<1, 11, 1, 1>(a, s);
    if (r16 <= 14) return launch_cfg<2, 7, 1, 1>(a, s);
    if (r16 <= 18) return launch_cfg<3, 6, 1, 1>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace fdllm
