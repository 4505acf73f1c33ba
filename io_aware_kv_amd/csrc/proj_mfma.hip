// proj_mfma.hip -- gather X[Q] + QKV projection + rotary + in-place k/v write,
// as one tiled bf16 MFMA kernel for gfx950 (head width 128).
//
// Flash-dLLM's fused kernel reads only the query rows' hidden states, builds
// q, k, v on chip and writes k, v straight into the cache (jaehun.me review,
// "How It Works: A Concrete Example", Step 1: Draft, citing the paper's
// Alg. 1; alanhou.org summary, "Core Mechanism" item 1).  Here one workgroup
// owns an output tile of BM query rows x one head (128 columns): the query
// rows are gathered from X by index straight into LDS, W is streamed through
// LDS once per tile, the fp32 accumulators are rotated in registers (the
// rotate-half pairs (c, c+64) sit in the same lane), and each row is stored to
// its final place: q in fp32 to the attention's staging buffer, k/v rounded
// once to bf16 into Kc/Vc at the row's position (or into the side buffer when
// an earlier query row owns that position).
//
// Small row counts leave W-bandwidth-bound work with few tiles, so the d_model
// loop can be split across workgroups; the last workgroup of a tile (atomic
// ticket) sums the fp32 partials in fixed order, so results do not depend on
// the arrival order.
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr int kBN = 128;       // one head of 128 columns
constexpr int kBK = 64;        // d_model slice per pipeline stage
constexpr int kLdsRow = kBK + 8;   // padded LDS row (bf16): 144 B, conflict-light 16 B reads
constexpr int kThreads = 256;

__device__ __forceinline__ bool owns_position(const int32_t* pos_b, int j)
{
    const int p = pos_b[j];
    for (int jj = 0; jj < j; ++jj)
        if (pos_b[jj] == p) return false;
    return true;
}

// BM rows per tile; WR waves split the rows, 4/WR waves split the 8 column
// blocks (a wave's blocks are {wc, wc + WC, ...}, closed under +4 so each lane
// holds both halves of its rotary pairs).
template <int BM, int WR>
__global__ void __launch_bounds__(kThreads) proj_mfma_kernel(ProjArgs a, int m_tiles, int n_tiles)
{
    constexpr int WC = 4 / WR;
    constexpr int RB = BM / WR / 16;       // 16-row blocks per wave
    constexpr int CB = 8 / WC;             // 16-column blocks per wave
    constexpr int XCH = BM * (kBK / 8);    // 16 B chunks of an X stage
    constexpr int XPT = (XCH + kThreads - 1) / kThreads;
    constexpr int WPT = kBN * (kBK / 8) / kThreads;  // 4
    static_assert(RB >= 1 && BM % (16 * WR) == 0, "bad tile");

    const int total = m_tiles * n_tiles * a.splitk;
    const int logical = xcd_remap(blockIdx.x, total);
    if (logical < 0) return;
    const int mt = logical % m_tiles;
    const int nz = logical / m_tiles;
    const int z = nz % a.splitk;
    const int nt = nz / a.splitk;
    const int head = a.prefill ? a.H + nt : nt;
    const int M = a.B * a.rows_per_seq;
    const int m0 = mt * BM;

    // one LDS block: the two pipeline stages of X and W, reused afterwards to
    // stage the finished tile (fp32 for q rows, bf16 for k/v rows)
    constexpr int kStageBytes = 2 * (BM + kBN) * kLdsRow * 2;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kStageBytes];
    bf16 (*sX)[BM][kLdsRow] = reinterpret_cast<bf16 (*)[BM][kLdsRow]>(smem);
    bf16 (*sW)[kBN][kLdsRow] = reinterpret_cast<bf16 (*)[kBN][kLdsRow]>(smem + 2 * BM * kLdsRow * 2);
    __shared__ int sPos[BM];
    __shared__ int sDst[BM];        // 1: owns its position, 0: duplicate, -1: padding row
    __shared__ int sLast;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC;

    if (tid < BM) {
        const int m = m0 + tid;
        if (m < M) {
            const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
            sPos[tid] = a.prefill ? j : a.pos_ids[m];
            sDst[tid] = a.prefill ? 1 : (owns_position(a.pos_ids + (size_t)b * a.rows_per_seq, j) ? 1 : 0);
        } else {
            sPos[tid] = 0;
            sDst[tid] = -1;
        }
    }

    // d_model range of this split
    const int nk_total = a.d / kBK;
    const int nk_per = (nk_total + a.splitk - 1) / a.splitk;
    const int kb0 = z * nk_per;
    const int niter = min(nk_total, kb0 + nk_per) - kb0;

    // per-thread source pointers (constant over the d_model loop)
    const bf16* xsrc[XPT];
    int xrow[XPT], xpart[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * kThreads;
        xrow[i] = c / (kBK / 8);
        xpart[i] = c % (kBK / 8);
        xsrc[i] = nullptr;
        const int m = m0 + xrow[i];
        if (c < XCH && m < M) {
            const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
            const int r = a.prefill ? j : a.Q_idx[m];
            xsrc[i] = (const bf16*)a.X + ((size_t)b * a.x_rows + r) * a.d + xpart[i] * 8;
        }
    }
    const bf16* wsrc[WPT];
    int wrow[WPT], wpart[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        const int c = tid + i * kThreads;
        wrow[i] = c / (kBK / 8);
        wpart[i] = c % (kBK / 8);
        wsrc[i] = (const bf16*)a.W + ((size_t)head * kBN + wrow[i]) * a.d + wpart[i] * 8;
    }

    uint4 xr[XPT], wreg[WPT];
    auto load_stage = [&](int kb) {
        const int koff = kb * kBK;
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            xr[i] = xsrc[i] ? *(const uint4*)(xsrc[i] + koff) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < WPT; ++i) wreg[i] = *(const uint4*)(wsrc[i] + koff);
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            if (tid + i * kThreads < XCH) *(uint4*)&sX[buf][xrow[i]][xpart[i] * 8] = xr[i];
#pragma unroll
        for (int i = 0; i < WPT; ++i) *(uint4*)&sW[buf][wrow[i]][wpart[i] * 8] = wreg[i];
    };

    f32x4 acc[RB][CB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int q = 0; q < CB; ++q) acc[r][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, lg = lane >> 4;
    if (niter > 0) load_stage(kb0);
    for (int it = 0; it < niter; ++it) {
        const int buf = it & 1;
        store_stage(buf);
        __syncthreads();
        if (it + 1 < niter) load_stage(kb0 + it + 1);
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            bf16x8 af[RB], bfr[CB];
#pragma unroll
            for (int r = 0; r < RB; ++r)
                af[r] = *(const bf16x8*)&sX[buf][(wr * RB + r) * 16 + lr][ks * 32 + lg * 8];
#pragma unroll
            for (int q = 0; q < CB; ++q)
                bfr[q] = *(const bf16x8*)&sW[buf][(wc + WC * q) * 16 + lr][ks * 32 + lg * 8];
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int q = 0; q < CB; ++q)
                    acc[r][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bfr[q], acc[r][q], 0, 0, 0);
        }
    }

    const int tile = nt * m_tiles + mt;
    if (a.splitk > 1) {
        // publish this split's partial tile in fragment order, then take a ticket
        constexpr int NACC = RB * CB;
        float4* part = (float4*)a.gpart + ((size_t)tile * a.splitk + z) * NACC * kThreads;
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int q = 0; q < CB; ++q) {
                const f32x4 v = acc[r][q];
                part[(size_t)(r * CB + q) * kThreads + tid] = make_float4(v[0], v[1], v[2], v[3]);
            }
        __threadfence();
        __syncthreads();
        if (tid == 0) sLast = (atomicAdd(&a.gticket[tile], 1u) == (unsigned)(a.splitk - 1));
        __syncthreads();
        if (!sLast) return;
        __threadfence();
        const float4* all = (const float4*)a.gpart + (size_t)tile * a.splitk * NACC * kThreads;
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int q = 0; q < CB; ++q) acc[r][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int zz = 0; zz < a.splitk; ++zz) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int q = 0; q < CB; ++q) {
                    const float4 v = all[((size_t)zz * NACC + r * CB + q) * kThreads + tid];
                    acc[r][q][0] += v.x;
                    acc[r][q][1] += v.y;
                    acc[r][q][2] += v.z;
                    acc[r][q][3] += v.w;
                }
        }
        if (tid == 0) a.gticket[tile] = 0u;
    }

    // rotary on q and k heads: lane holds column c = cb*16 + lr (< 64 for the
    // first half of the wave's blocks) and rows 4*lg + i of each row block
    const bool rotate = head < a.H + a.Hkv;
    if (rotate) {
#pragma unroll
        for (int q = 0; q < CB / 2; ++q) {
            const int c = (wc + WC * q) * 16 + lr;
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = (wr * RB + r) * 16 + lg * 4 + i;
                    const float2 cs = a.rope[(size_t)sPos[row] * (kBN / 2) + c];
                    const float y0 = acc[r][q][i], y1 = acc[r][q + CB / 2][i];
                    acc[r][q][i] = y0 * cs.x - y1 * cs.y;
                    acc[r][q + CB / 2][i] = y1 * cs.x + y0 * cs.y;
                }
        }
    }

    // stage the finished tile in LDS and store whole rows: q rows stay fp32
    // (consumed on chip by the attention, never stored as bf16), k/v rows are
    // rounded once to bf16 (they are the cache contents)
    __syncthreads();   // everyone is done reading the pipeline stages
    const int G = a.G;
    if (head < a.H) {
        constexpr int kRowF = kBN + 4;
        static_assert(kStageBytes >= BM * kRowF * 4, "fp32 staging does not fit");
        float* sOutF = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int q = 0; q < CB; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sOutF[((wr * RB + r) * 16 + lg * 4 + i) * kRowF + (wc + WC * q) * 16 + lr] = acc[r][q][i];
        __syncthreads();
        const int g = head / G, hl = head - g * G;
        constexpr int OCH = BM * (kBN / 4);
        for (int c = tid; c < OCH; c += kThreads) {
            const int row = c / (kBN / 4), part = c % (kBN / 4);
            if (sDst[row] < 0) continue;
            const int m = m0 + row;
            const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
            float* dst = a.qbuf + (((size_t)b * a.Hkv + g) * a.q_max * G + (size_t)j * G + hl) * kBN;
            *(float4*)(dst + part * 4) = *(const float4*)&sOutF[row * kRowF + part * 4];
        }
        return;
    }
    static_assert(kStageBytes >= BM * (kBN + 8) * 2, "bf16 staging does not fit");
    bf16 (*sOut)[kBN + 8] = reinterpret_cast<bf16 (*)[kBN + 8]>(smem);
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int q = 0; q < CB; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sOut[(wr * RB + r) * 16 + lg * 4 + i][(wc + WC * q) * 16 + lr] = (bf16)acc[r][q][i];
    __syncthreads();

    const bool isk = head < a.H + a.Hkv;
    const int g = head - a.H - (isk ? 0 : a.Hkv);
    constexpr int OCH = BM * (kBN / 8);
    for (int c = tid; c < OCH; c += kThreads) {
        const int row = c / (kBN / 8), part = c % (kBN / 8);
        const int kind = sDst[row];
        if (kind < 0) continue;
        const int m = m0 + row;
        const int b = m / a.rows_per_seq, j = m - b * a.rows_per_seq;
        bf16* dst;
        if (kind == 1)
            dst = (bf16*)(isk ? a.Kc : a.Vc) + (((size_t)b * a.Hkv + g) * a.N + sPos[row]) * kBN;
        else
            dst = (bf16*)(isk ? a.sideK : a.sideV) + (((size_t)b * a.Hkv + g) * a.q_max + j) * kBN;
        *(uint4*)(dst + part * 8) = *(const uint4*)&sOut[row][part * 8];
    }
}

template <int BM, int WR>
hipError_t launch_bm(const ProjArgs& a, hipStream_t s)
{
    const int M = a.B * a.rows_per_seq;
    const int m_tiles = (M + BM - 1) / BM;
    const int n_tiles = a.prefill ? 2 * a.Hkv : a.H + 2 * a.Hkv;
    const int total = m_tiles * n_tiles * a.splitk;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((proj_mfma_kernel<BM, WR>), dim3(grid), dim3(kThreads), 0, s, a, m_tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace

int proj_mfma_block_m(int M)
{
    if (M <= 16) return 16;
    if (M <= 32) return 32;
    if (M <= 48) return 48;
    if (M <= 64) return 64;
    return 128;
}

hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t s)
{
    const int M = a.B * a.rows_per_seq;
    if (M == 0) return hipSuccess;
    switch (proj_mfma_block_m(M)) {
        case 16: return launch_bm<16, 1>(a, s);
        case 32: return launch_bm<32, 2>(a, s);
        case 48: return launch_bm<48, 1>(a, s);
        case 64: return launch_bm<64, 2>(a, s);
        default: return launch_bm<128, 2>(a, s);
    }
}

}  // namespace fdllm
