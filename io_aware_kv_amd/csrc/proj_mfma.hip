// proj_mfma.hip -- gather X[Q] + QKV projection + rotary + in-place k/v write,
// as one bf16 MFMA kernel for gfx950 (head width 128).
//
// Flash-dLLM's fused kernel reads only the query rows' hidden states, builds
// q, k, v on chip and writes k, v straight into the cache (jaehun.me review,
// "How It Works: A Concrete Example", Step 1: Draft, citing the paper's
// Alg. 1; alanhou.org summary, "Core Mechanism" item 1).
//
// One workgroup owns an output tile of BM query rows x BN columns of one
// head.  The columns are a rotary-closed set: 16-column blocks {p .. p+n-1}
// and {p+4 .. p+4+n-1}, so every lane holds both halves of its rotate-half
// pairs (c, c+64).  Narrow tiles (BN = 32) give small row counts enough
// workgroups to stream the weight at full bandwidth without splitting the
// d_model loop across workgroups (which would need a device-wide reduction).
//
// A producer wave streams 128-deep d_model stages of the gathered X rows
// (addressed through Q_idx) and of the tile's W rows into an LDS ring with
// global_load_lds; the consumer waves run v_mfma_f32_16x16x32_bf16 from LDS
// (256 B rows, 16 B chunks XOR-swizzled by row: conflict-free fragment reads).
// The fp32 accumulators are rotated in registers, staged in LDS and stored as
// whole rows: q in fp32 to the attention's staging buffer, k and v rounded
// once to bf16 into Kc/Vc at the row's position (or into the side buffer when
// an earlier query row owns that position).
#include "pipeline.h"

namespace fdllm {

namespace {

constexpr int kDH = 128;          // head width

// BK: d_model depth per stage (64 or 128: a staged row is 128 or 256 B); NPROD producer waves split each stage's 1 KB DMA blocks, so up to
// NPROD x 63 blocks can be in flight per workgroup.  The ring takes as many
// stages as fit beside the row bookkeeping in the CU's 160 KB of LDS, at most
// NSMAX (which keeps two workgroups per CU for the narrow tiles): a CU's
// stream is bound by the bytes it keeps in flight, NS - 1 stages.
//
// Consumer waves form NKW x NRW x NPW groups: NRW row groups x NPW column
// groups of the tile, and NKW groups that split each stage's 32-deep MFMA
// steps between them (their partial sums are added once, in LDS, after the
// loop).  A wave reads its row and column fragments from LDS for every step
// it runs; one wave draws only about 1 KB per 40 cycles from LDS, so the
// layout keeps the MFMAs per fragment load high (a wave tile of r x c values
// costs (r + c) / 16 loads for r * c / 256 MFMAs).
template <int BM, int NCB, int NKW, int NRW, int NPW, int NSMAX, int BK, int NPROD>
struct ProjCfg {
    static constexpr int NHW = NRW * NPW;                 // waves holding the tile after the k reduction
    static constexpr int NCW = NKW * NHW;                 // consumer waves
    static constexpr int KSW = BK / 32 / NKW;             // 32-deep steps per stage per consumer wave
    static constexpr int NT = (NCW + NPROD) * 64;
    static constexpr int BN = 16 * NCB;
    static constexpr int ROWB = BK * 2;                   // bytes per staged row
    static constexpr int RPD = 1024 / ROWB;               // rows per 1 KB DMA block
    static constexpr int CPR = BK / 8;                    // 16 B chunks per staged row
    static constexpr int ROWS = BM + BN;                  // staged rows per stage
    static constexpr int STAGE = ROWS * ROWB;
    static constexpr int NS0 = (160 * 1024 - 16 * BM - 1024) / STAGE;
    static constexpr int NS = NS0 > NSMAX ? NSMAX : NS0;
    static constexpr int DMA = ROWS / RPD;                // 1 KB DMA blocks per stage
    static constexpr int DMAP = DMA / NPROD;              // per producer wave
    static constexpr int RBW = BM / 16 / NRW;             // row blocks per consumer wave
    static constexpr int PAIRS = NCB / 2;                 // rotary block pairs per tile
    static constexpr int PPW = PAIRS / NPW;               // pairs per consumer wave
    static constexpr int V4 = PAIRS * 8;                  // 16 B rotary-table loads per tile row
    // rotary-table loads per consumer lane when they are prefetched into
    // registers before the loop (0: loaded after it, where registers are short)
    static constexpr int RPF0 = (BM * V4 + NCW * 64 - 1) / (NCW * 64);
    static constexpr int RPF = (NKW == 1 && RPF0 <= 22) ? RPF0 : 0;
    static_assert(BK == 64 || BK == 128, "stage depth");
    static_assert((NS - 2) * DMAP <= 63 || NS <= 2, "in-flight DMA blocks per producer");
    static_assert(BM % (16 * NRW) == 0 && PAIRS % NPW == 0 && NS >= 2, "tile shape");
    static_assert(KSW >= 1 && KSW * NKW * 32 == BK, "k split");
    static_assert((NKW - 1) * NHW * RBW * 2 * PPW * 1024 <= NS * STAGE, "k reduction staging");
    static_assert(DMA % NPROD == 0 && BM % RPD == 0, "DMA split");
    static_assert(BM * (BN + 4) * 4 <= NS * STAGE, "epilogue staging");
    static_assert(BM * PAIRS * 16 * 8 <= NS * STAGE, "rotary table staging");
};

// Chunk swizzle of a staged row: 16 B chunk c of row r sits in slot c ^ f(r).
// With 256 B rows, f(r) = r & 15; with 128 B rows (two rows per 64-bank
// sweep), f(r) = (r >> 1) & 7.  Either way the 16 rows read by one fragment
// load hit 16 distinct 16 B bank groups.
template <int BK>
__device__ __forceinline__ int chunk_swz(int row)
{
    return BK == 128 ? (row & 15) : ((row >> 1) & 7);
}

template <int BM, int NCB, int NKW, int NRW, int NPW, int NSMAX, int BK, int NPROD>
__global__ void __launch_bounds__((NKW * NRW * NPW + NPROD) * 64)
proj_mfma_kernel(ProjArgs a, int m_tiles, int n_tiles)
{
    using C = ProjCfg<BM, NCB, NKW, NRW, NPW, NSMAX, BK, NPROD>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ size_t sXoff[BM];   // element offset of the row's X row
    __shared__ int sPos[BM];
    __shared__ int sDst[BM];       // 1: owns its position, 0: duplicate, -1: padding row

    const int total = m_tiles * n_tiles;
    const int logical = xcd_remap(blockIdx.x, total);
    if (logical < 0) return;
    const int mt = logical % m_tiles;              // row tiles of one column tile share an XCD
    const int nt = logical / m_tiles;
    constexpr int TPH = 8 / NCB;                   // column tiles per head
    const int head = (a.prefill ? a.H : 0) + nt / TPH;
    const int p0 = (nt % TPH) * C::PAIRS;          // first 16-column block of the tile
    const int M = a.B * a.rows_per_seq;
    const int m0 = mt * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;

    // row bookkeeping: one load of Q_idx and pos_ids per row.  Ownership of
    // the cache write (needed only by the epilogue) is settled by the
    // consumer waves while the first stages stream in.
    for (int r = tid; r < BM; r += C::NT) {
        int m = m0 + r;
        const bool valid = m < M;
        if (!valid) m = m0;                          // rows past M read row 0 of a sequence, then are dropped
        const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
        // rows past a shorter sequence's own count are padding: they read X
        // row 0 and write only a zero q row
        const bool pad = valid && !a.prefill && a.nq_seq && j >= a.nq_seq[b];
        const bool live = valid && !pad;
        const int xr = a.prefill ? j : (live ? a.Q_idx[m] : 0);
        sXoff[r] = ((size_t)b * a.x_rows + xr) * a.d;
        sPos[r] = live ? (a.prefill ? j : a.pos_ids[m]) : 0;
        sDst[r] = live ? 1 : (pad ? -2 : -1);
    }
    __syncthreads();

    const int nk = a.d / BK;
    // Rows of X and W sit d_model elements apart, so one stage of every row
    // falls in the same few L2 channels.  The d_model loop of a tile starts
    // at its own stage and wraps around: tiles on one XCD (which share X rows
    // and W rows through its L2) start within 8 stages of each other, so the
    // shared data is still in the L2 when the later ones read it, while the
    // XCDs start an eighth of the loop apart.
    const int krot = ((blockIdx.x & 7) * (nk / 8) + (logical & 7)) % nk;
    auto kstage = [&](int t) { const int u = t + krot; return u >= nk ? u - nk : u; };
    const bf16* X = (const bf16*)a.X;
    const bf16* W = (const bf16*)a.W;

    f32x4 acc[C::RBW][2 * C::PPW];
#pragma unroll
    for (int r = 0; r < C::RBW; ++r)
#pragma unroll
        for (int q = 0; q < 2 * C::PPW; ++q) acc[r][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wk = wave / C::NHW;                 // consumer coordinates
    const int wr = (wave % C::NHW) / NPW, wp = wave % NPW;
    const bool rotate = head < a.H + a.Hkv;
    // the tile's rotary-table rows (first-half columns of its pairs), loaded
    // by the consumer waves before the loop so the epilogue does not wait on
    // them (16 B of (cos, sin) pairs each)
    f32x4 ropepf[C::RPF > 0 ? C::RPF : 1];

    if (wave >= C::NCW) {
        // ================= producer waves =================
        const int pw = wave - C::NCW;
        const int srow = lane / C::CPR, slot = lane % C::CPR;
        // source row (with its swizzled chunk) of each of this wave's DMA
        // blocks; a stage only adds its d_model offset
        const bf16* rowp[C::DMAP];
#pragma unroll
        for (int ii = 0; ii < C::DMAP; ++ii) {
            const int i = ii * NPROD + pw;
            const int row = C::RPD * i + srow;
            const int chunk = slot ^ chunk_swz<BK>(row);
            if (C::RPD * i < BM) {
                rowp[ii] = X + sXoff[row] + chunk * 8;
            } else {
                const int wi = row - BM, blk = wi >> 4;
                const int cb = blk < C::PAIRS ? p0 + blk : p0 + 4 + (blk - C::PAIRS);
                rowp[ii] = W + ((size_t)(head * kDH + cb * 16 + (wi & 15))) * a.d + chunk * 8;
            }
        }
        auto issue = [&](int t) {
            unsigned char* st = smem + (t % C::NS) * C::STAGE + pw * 1024;
            const int k0 = kstage(t) * BK;
#pragma unroll
            for (int ii = 0; ii < C::DMAP; ++ii) dma16(rowp[ii] + k0, st + ii * NPROD * 1024);
        };
        int issued = 0;
        for (; issued < min(C::NS - 1, nk); ++issued) issue(issued);
        for (int t = 0; t < nk; ++t) {
            ring_producer_wait<C::DMAP, C::NS - 2>(issued - t - 1);
            if (issued < nk) issue(issued++);
        }
    } else {
        // ================= consumer waves =================
        if constexpr (C::RPF > 0) {
            if (rotate) {
#pragma unroll
                for (int i = 0; i < C::RPF; ++i) {
                    const int e = min(tid + i * C::NCW * 64, BM * C::V4 - 1);
                    const int row = e / C::V4, v = e - row * C::V4;
                    ropepf[i] = *(const f32x4*)&a.rope[(size_t)sPos[row] * (kDH / 2) + p0 * 16 + 2 * v];
                }
            }
        }
        if (!a.prefill && head >= a.H) {
            // first-occurrence rule: a row owns the cache write of its
            // position unless an earlier row of its sequence has the same one.
            // Each wave copies the positions of the tile's sequences (from the
            // first row of the first one) into its own slice of the last ring
            // stage, which no DMA writes before the first barrier, and
            // compares from there: one round trip to memory instead of one
            // per eight earlier rows.
            const int mlo = (m0 / a.rows_per_seq) * a.rows_per_seq;
            const int cnt = min(m0 + BM, M) - mlo;
            const int pw = (cnt + 3) & ~3;
            const bool staged = (size_t)pw * C::NCW * 4 <= (size_t)C::STAGE;
            int* sP = (int*)(smem + (size_t)(C::NS - 1) * C::STAGE) + wave * pw;
            if (staged)
                for (int e = lane; e < cnt; e += 64) sP[e] = a.pos_ids[mlo + e];
            // (the two sources in separate loops, so each compiles to its own
            // kind of load rather than a generic one)
            auto owns = [](const int* pb, int j, int p) {
                bool own = true;
                int jj = 0;
                for (; jj + 8 <= j; jj += 8) {
                    int v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) v[u] = pb[jj + u];
#pragma unroll
                    for (int u = 0; u < 8; ++u) own = own && v[u] != p;
                }
                for (; jj < j; ++jj) own = own && pb[jj] != p;
                return own;
            };
            for (int r = tid; r < BM; r += C::NCW * 64) {
                const int m = m0 + r;
                if (m >= M || sDst[r] < 0) continue;
                const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
                const bool own = staged ? owns(sP + (b * a.rows_per_seq - mlo), j, sPos[r])
                                        : owns(a.pos_ids + (size_t)b * a.rows_per_seq, j, sPos[r]);
                if (!own) sDst[r] = 0;
            }
        }
        for (int t = 0; t < nk; ++t) {
            ring_consumer_sync();
            const unsigned char* st = smem + (t % C::NS) * C::STAGE;
#pragma unroll
            for (int kk = 0; kk < C::KSW; ++kk) {
                const int ks = wk * C::KSW + kk;
                bf16x8 af[C::RBW], bfr[2 * C::PPW];
#pragma unroll
                for (int r = 0; r < C::RBW; ++r) {
                    const int row = (wr * C::RBW + r) * 16 + lr;
                    af[r] = *(const bf16x8*)(st + row * C::ROWB + (((ks * 4 + lg) ^ chunk_swz<BK>(row)) << 4));
                }
#pragma unroll
                for (int q = 0; q < 2 * C::PPW; ++q) {
                    const int blk = q < C::PPW ? wp * C::PPW + q : C::PAIRS + wp * C::PPW + (q - C::PPW);
                    const int row = BM + blk * 16 + lr;
                    bfr[q] = *(const bf16x8*)(st + row * C::ROWB + (((ks * 4 + lg) ^ chunk_swz<BK>(row)) << 4));
                }
#pragma unroll
                for (int r = 0; r < C::RBW; ++r)
#pragma unroll
                    for (int q = 0; q < 2 * C::PPW; ++q)
                        acc[r][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bfr[q], acc[r][q], 0, 0, 0);
            }
        }
    }
    __syncthreads();   // the ring is free: it stages the finished tile below

    if constexpr (NKW > 1) {
        // add the k groups' partial sums into the waves of group 0 (each
        // accumulator block is one 1 KB row of 16 B per lane: conflict-free)
        constexpr int BLK = C::RBW * 2 * C::PPW;
        f32x4* sRed = (f32x4*)smem;
        if (wk > 0 && wave < C::NCW) {
            f32x4* dst = sRed + ((size_t)((wk - 1) * C::NHW + wave % C::NHW) * BLK) * 64 + lane;
#pragma unroll
            for (int r = 0; r < C::RBW; ++r)
#pragma unroll
                for (int q = 0; q < 2 * C::PPW; ++q) dst[(r * 2 * C::PPW + q) * 64] = acc[r][q];
        }
        __syncthreads();
        if (wave < C::NHW) {
#pragma unroll
            for (int g = 1; g < NKW; ++g) {
                const f32x4* src = sRed + ((size_t)((g - 1) * C::NHW + wave) * BLK) * 64 + lane;
#pragma unroll
                for (int r = 0; r < C::RBW; ++r)
#pragma unroll
                    for (int q = 0; q < 2 * C::PPW; ++q) acc[r][q] += src[(r * 2 * C::PPW + q) * 64];
            }
        }
        __syncthreads();
    }

    // rotary on q and k heads: lane holds tile column blk*16 + lr of each block
    // (head column cb*16 + lr) and rows 4*lg + i of each row block.  The
    // table rows of the tile's positions (first-half columns of its pairs)
    // are first staged in the free ring with all loads in flight at once.
    const bool consumer = wave < C::NHW;             // the waves that hold the finished tile
    if (rotate) {
        constexpr int PC = C::PAIRS * 16;                  // table columns of the tile
        float2* sCS = (float2*)smem;                       // [BM][PC]
        constexpr int V4 = C::V4;
        if constexpr (C::RPF > 0) {
            if (consumer) {
#pragma unroll
                for (int i = 0; i < C::RPF; ++i) {
                    const int e = tid + i * C::NCW * 64;
                    if (e < BM * V4) {
                        const int row = e / V4, v = e - row * V4;
                        *(f32x4*)&sCS[row * PC + 2 * v] = ropepf[i];
                    }
                }
            }
        } else {
            // all of a thread's table loads in flight before the first store
            // (one memory round trip, not one per load), where the registers
            // allow it beside the accumulators
            constexpr int PER = (BM * V4 + C::NT - 1) / C::NT;
            constexpr bool BATCH = 4 * C::RBW * 2 * C::PPW + 4 * PER <= 160;
            if constexpr (BATCH) {
                f32x4 cs[PER];
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int e = min(tid + i * C::NT, BM * V4 - 1);
                    const int row = e / V4, v = e - row * V4;
                    cs[i] = *(const f32x4*)&a.rope[(size_t)sPos[row] * (kDH / 2) + p0 * 16 + 2 * v];
                }
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int e = tid + i * C::NT;
                    if (e < BM * V4) {
                        const int row = e / V4, v = e - row * V4;
                        *(f32x4*)&sCS[row * PC + 2 * v] = cs[i];
                    }
                }
            } else {
                for (int e = tid; e < BM * V4; e += C::NT) {
                    const int row = e / V4, v = e - row * V4;
                    *(f32x4*)&sCS[row * PC + 2 * v] =
                        *(const f32x4*)&a.rope[(size_t)sPos[row] * (kDH / 2) + p0 * 16 + 2 * v];
                }
            }
        }
        __syncthreads();
        if (consumer) {
#pragma unroll
            for (int q = 0; q < C::PPW; ++q) {
                const int c = (wp * C::PPW + q) * 16 + lr;     // table column within the tile
#pragma unroll
                for (int r = 0; r < C::RBW; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float2 cs = sCS[((wr * C::RBW + r) * 16 + lg * 4 + i) * PC + c];
                        const float y0 = acc[r][q][i], y1 = acc[r][q + C::PPW][i];
                        acc[r][q][i] = y0 * cs.x - y1 * cs.y;
                        acc[r][q + C::PPW][i] = y1 * cs.x + y0 * cs.y;
                    }
            }
        }
        __syncthreads();   // the staging below reuses the ring
    }

    // stage the tile: q rows stay fp32 (consumed on chip by the attention),
    // k/v rows are rounded once to bf16 (they are the cache contents)
    const int G = a.G;
    constexpr int BN = C::BN;
    const bool isq = head < a.H;
    if (isq) {
        constexpr int RS = BN + 4;
        float* sOut = (float*)smem;
        if (consumer) {
#pragma unroll
            for (int r = 0; r < C::RBW; ++r)
#pragma unroll
                for (int q = 0; q < 2 * C::PPW; ++q) {
                    const int blk = q < C::PPW ? wp * C::PPW + q : C::PAIRS + wp * C::PPW + (q - C::PPW);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sOut[((wr * C::RBW + r) * 16 + lg * 4 + i) * RS + blk * 16 + lr] = acc[r][q][i];
                }
        }
        __syncthreads();
        const int g = head / G, hl = head - g * G;
        constexpr int CPR = BN / 4;                  // 16 B chunks per row
        for (int c = tid; c < BM * CPR; c += C::NT) {
            const int row = c / CPR, part = c - row * CPR;
            const int kind = sDst[row];
            if (kind == -1) continue;
            const int m = m0 + row;
            const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
            const int tcol = part * 4;                                   // tile column
            const int hcol = tcol < BN / 2 ? p0 * 16 + tcol : 64 + p0 * 16 + (tcol - BN / 2);
            float* dst = a.qbuf + (((size_t)b * a.Hkv + g) * a.q_max * G + (size_t)j * G + hl) * kDH + hcol;
            *(f32x4*)dst = kind == -2 ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4*)&sOut[row * RS + tcol];
        }
        return;
    }
    constexpr int RS = BN + 8;
    bf16* sOut = (bf16*)smem;
    if (consumer) {
#pragma unroll
        for (int r = 0; r < C::RBW; ++r)
#pragma unroll
            for (int q = 0; q < 2 * C::PPW; ++q) {
                const int blk = q < C::PPW ? wp * C::PPW + q : C::PAIRS + wp * C::PPW + (q - C::PPW);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sOut[((wr * C::RBW + r) * 16 + lg * 4 + i) * RS + blk * 16 + lr] = (bf16)acc[r][q][i];
            }
    }
    __syncthreads();
    // one column tile of the first k head records the rows' ownership for
    // the attention launch (which would otherwise settle it again in every
    // (sequence, kv head) workgroup)
    if (a.own && !a.prefill && head == a.H && p0 == 0)
        for (int r = tid; r < BM; r += C::NT)
            if (m0 + r < M) a.own[m0 + r] = (int8_t)sDst[r];
    const bool isk = head < a.H + a.Hkv;
    const int g = head - a.H - (isk ? 0 : a.Hkv);
    constexpr int CPR = BN / 8;
    for (int c = tid; c < BM * CPR; c += C::NT) {
        const int row = c / CPR, part = c - row * CPR;
        const int kind = sDst[row];
        if (kind < 0) continue;
        const int m = m0 + row;
        const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
        const int tcol = part * 8;
        const int hcol = tcol < BN / 2 ? p0 * 16 + tcol : 64 + p0 * 16 + (tcol - BN / 2);
        bf16* dst;
        if (kind == 1)
            dst = (bf16*)(isk ? a.Kc : a.Vc) + cache_row(a.map, b, g, sPos[row], a.Hkv, a.N) * kDH;
        else
            dst = (bf16*)(isk ? a.sideK : a.sideV) + (((size_t)b * a.Hkv + g) * a.q_max + j) * kDH;
        *(u32x4*)(dst + hcol) = *(const u32x4*)&sOut[row * RS + tcol];
    }
}

template <int BM, int NCB, int NKW, int NRW, int NPW, int NSMAX, int BK, int NPROD>
hipError_t launch_tile(const ProjArgs& a, hipStream_t s)
{
    using C = ProjCfg<BM, NCB, NKW, NRW, NPW, NSMAX, BK, NPROD>;
    const int M = a.B * a.rows_per_seq;
    const int m_tiles = (M + BM - 1) / BM;
    const int heads = a.prefill ? 2 * a.Hkv : a.H + 2 * a.Hkv;
    const int n_tiles = heads * (8 / NCB);
    const int total = m_tiles * n_tiles;
    const int grid = ((total + 7) / 8) * 8;
    const size_t shm = (size_t)C::NS * C::STAGE;
    constexpr auto kern = proj_mfma_kernel<BM, NCB, NKW, NRW, NPW, NSMAX, BK, NPROD>;
    (void)allow_full_lds<kern>();
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), shm, s, a, m_tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace

// Tile configurations (rows BM x 16-column blocks NCB): narrow tiles with a
// 3-stage ring (two workgroups per CU), 64 x 64 tiles, and 128-column (one
// head) tiles of 96 to 256 rows; the 208-row and 176-row tiles split each
// stage's MFMA steps between two wave groups (choices 9 and 11; choices 7 and
// 6 are the same tiles without the split), the 256-row tile runs eight
// consumer waves in a 2 x 4 layout.
struct ProjChoice { int bm, ncb; };
static const ProjChoice kProjChoices[] = {
    {0, 0},
    {16, 2}, {32, 2}, {48, 2}, {64, 4},   // 1-4
    {128, 8}, {176, 8}, {208, 8}, {96, 8},  // 5-8
    {208, 8},                             // 9
    {256, 8},                             // 10
    {176, 8},                             // 11
};
constexpr int kNumChoices = (int)(sizeof(kProjChoices) / sizeof(kProjChoices[0]));

// The loop of a tile is bound by the bytes its CU takes in from the L2 (X
// and W rows), so the choice trades tile area against idle CUs and extra
// rounds.  Measured on MI355X with d_model 4096, 1..1408 rows, 48 and 96
// heads: the narrow tiles lead only for up to 32 rows of few heads (by up to
// 1.3 us), 64 x 64 tiles everywhere else up to 128 rows (up to 4 us ahead of
// the narrow ones at 96 heads).  Beyond 128 rows the order of the measured
// times follows the staged rows per CU: rounds of 256 workgroups x (BM + BN)
// (1408 rows of 96 heads: 176-row tiles in 3 rounds, 160 us, against 205 us
// for 128-row tiles in 4.1 rounds, and 172 us for 256-row tiles in 2.25;
// 1152 rows: 256-row tiles in 2 rounds, 119 us, against 154 us for 176-row
// tiles in 2.6).  The 208-row and 176-row tiles run with their k split
// (faster than without at every row count measured: 176 rows, 352 rows of 96
// heads 54.6 against 55.4 us, 1408 rows 162 against 166 us).  With the
// split a SIMD holds two consumer waves, yet the tile is no more than a few
// per cent faster: the loop is bound by the rate at which the stages land in
// LDS (the same loop without its MFMAs takes 53 of the 55 us), not by the
// fragment reads or the MFMAs.
static int default_choice(int M, int heads)
{
    if (M <= 32 && heads < 64) return M <= 16 ? 1 : 2;
    if (M <= 128) return 4;
    int best = 5;
    long best_cost = -1;
    for (int c : {4, 8, 5, 11, 9, 10}) {
        const ProjChoice& p = kProjChoices[c];
        const long tiles = (long)((M + p.bm - 1) / p.bm) * heads * (8 / p.ncb);
        const long cost = ((tiles + 255) / 256) * (p.bm + 16 * p.ncb);
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = c; }
    }
    return best;
}

ProjTile proj_mfma_tile(int M, int heads, int choice)
{
    if (choice <= 0 || choice >= kNumChoices) choice = default_choice(M, heads);
    return ProjTile{kProjChoices[choice].bm, 16 * kProjChoices[choice].ncb, choice};
}

hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t s)
{
    const int M = a.B * a.rows_per_seq;
    if (M == 0) return hipSuccess;
    if (a.d % 128 != 0) return hipErrorInvalidValue;
    const int heads = a.prefill ? 2 * a.Hkv : a.H + 2 * a.Hkv;
    switch (proj_mfma_tile(M, heads, a.tile_choice).choice) {
        case 1: return launch_tile<16, 2, 1, 1, 1, 3, 128, 2>(a, s);
        case 2: return launch_tile<32, 2, 1, 1, 1, 3, 128, 2>(a, s);
        case 3: return launch_tile<48, 2, 1, 1, 1, 3, 128, 2>(a, s);
        case 4: return launch_tile<64, 4, 1, 2, 2, 8, 128, 2>(a, s);
        case 5: return launch_tile<128, 8, 1, 2, 2, 8, 64, 2>(a, s);
        case 6: return launch_tile<176, 8, 1, 1, 4, 8, 64, 2>(a, s);
        case 7: return launch_tile<208, 8, 1, 1, 4, 8, 64, 2>(a, s);
        case 8: return launch_tile<96, 8, 1, 1, 4, 8, 64, 2>(a, s);
        case 9: return launch_tile<208, 8, 2, 1, 2, 8, 64, 2>(a, s);
        case 10: return launch_tile<256, 8, 1, 2, 4, 8, 64, 2>(a, s);
        case 11: return launch_tile<176, 8, 2, 1, 4, 8, 64, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fdllm
