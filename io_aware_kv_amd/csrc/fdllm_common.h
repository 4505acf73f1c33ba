// fdllm_common.h -- internal declarations shared by the HIP kernels and the
// C-ABI host code of libfdllm.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fdllm.h"

namespace fdllm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Where cache row (b, g, p) lives: the flat layout [B, Hkv, N, dh] when
// table is NULL, else a pool of blocks [blocks, Hkv, 2^bits, dh] with
// table[b * max_blocks + (p >> bits)] naming the block of position p.
struct CacheMap {
    const int32_t* table;
    int bits;               // log2 of the block size
    int max_blocks;         // table entries per sequence
};

__device__ __forceinline__ size_t cache_row(const CacheMap& c, int b, int g, int p, int Hkv, int N)
{
    if (!c.table) return ((size_t)b * Hkv + g) * N + p;
    const int blk = c.table[(size_t)b * c.max_blocks + (p >> c.bits)];
    return (((size_t)blk * Hkv + g) << c.bits) + (p & ((1 << c.bits) - 1));
}

// Everything a launch of the projection kernels needs.  Rows of the
// projection are m = b * rows_per_seq + j.
struct ProjArgs {
    const void* X;          // [B, x_rows, d]
    const void* W;          // [(H + 2 Hkv) dh, d]
    const int32_t* Q_idx;   // [B, nq]  (NULL in prefill mode: row j is X row j)
    const int32_t* pos_ids; // [B, nq]  (NULL in prefill mode: position j)
    const float2* rope;     // [N, dh/2] (cos, sin) of pos * base^(-2e/dh)
    void* Kc;               // [B, Hkv, N, dh]
    void* Vc;
    float* qbuf;            // [B, Hkv, q_max * G, dh] fp32, row j * G + hl  (unused in prefill)
    void* sideK;            // [B, Hkv, q_max, dh]: rows whose position an earlier row owns
    void* sideV;
    int B, N, d, H, Hkv, dh, G;
    int x_rows;
    int rows_per_seq;       // nq, or N in prefill mode
    int q_max;
    int prefill;            // 1: k/v heads only, no q, no side buffer
    int tile_choice;        // 0: default tile configuration for the row count
    CacheMap map;           // cache layout (flat when map.table is NULL)
    const int32_t* nq_seq;  // [B] query rows of each sequence (rows j >= nq_seq[b] are padding) or NULL
    int8_t* own;            // [B, rows_per_seq] per row: 1 owns the cache write of its position, 0 an
                            // earlier row does, < 0 padding (not in prefill mode); NULL: not recorded
};

struct AttnArgs {
    const float* qbuf;      // [B, Hkv, q_max * G, dh] fp32 (q is not rounded to storage)
    const void* Kc;         // [B, Hkv, N, dh]
    const void* Vc;
    const void* sideK;      // [B, Hkv, q_max, dh]
    const void* sideV;
    const int32_t* pos_ids; // [B, nq]
    const uint8_t* vis;     // [B, nq, nq] or NULL
    void* O;                // [B, nq, H, dh]
    float* LSE;             // [B, nq, H]
    bf16* apart;            // [B * Hkv, splits, Rpad, dh]  each split's normalised output (O_s / l_s)
    float* aml;             // [B * Hkv, splits, Rpad, 2]    (max in log2 units, sum)
    int B, N, H, Hkv, dh, G, nq, q_max;
    int R;                  // nq * G query rows per (sequence, kv head)
    int Rpad;               // R rounded up for the partial buffers
    int splits;
    int keys_per_split;     // multiple of the kernel's tile width
    float scale_log2;       // log2(e) / sqrt(dh)
    CacheMap map;           // cache layout (flat when map.table is NULL)
    const int32_t* seq_len; // [B] valid cache positions of each sequence (>= 1) or NULL (all N)
    const int32_t* nq_seq;  // [B] query rows of each sequence or NULL (all nq)
    const int8_t* own;      // [B, nq] the step's ownership flags, as the projection recorded them
    int hid_words;          // set by the MFMA launcher: per-row hidden-key words are built in LDS
};

// Tracked-set scores after a step: attention mass of the selected query rows
// on every cache position.
struct MassArgs {
    const float* qbuf;      // the step's q staging buffer
    const void* Kc;         // [B, Hkv, N, dh] after the step
    const int32_t* pos_ids; // [B, nq]
    const uint8_t* vis;     // [B, nq, nq] or NULL
    const uint8_t* sel;     // [B, nq] 1: the row contributes
    const float* LSE;       // [B, nq, H] of the step
    float* part;            // [B * Hkv, N] per kv head sums
    float* scores;          // [B, N]
    int B, N, H, Hkv, dh, G, nq, q_max;
    int splits, keys_per_split;
    float scale_log2;       // log2(e) / sqrt(dh)
};
hipError_t launch_key_mass(const MassArgs& a, hipStream_t s);
hipError_t launch_key_mass_generic(const MassArgs& a, int dtype, hipStream_t s);
size_t key_mass_lds_bytes(int nq, int keys_per_split);
hipError_t launch_select_top(const float* scores, const uint8_t* cand, int B, int N, int k, int32_t* out,
                             hipStream_t s);

hipError_t launch_confidence(const void* logits, int dtype, int64_t rows, int V, int mask_id, float thr,
                             int32_t* pred, float* conf, uint8_t* over, hipStream_t s);
hipError_t launch_accept(const int32_t* x_hat, const int32_t* x_tilde, const float* c_tilde, int B, int S,
                         float gamma, int32_t* n_accept, hipStream_t s);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_proj_generic(const ProjArgs& a, int dtype, hipStream_t s);
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s);
hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s);

// Tile geometry of the MFMA kernels, needed by the host planner.
struct ProjTile { int bm, bn, choice; };
ProjTile proj_mfma_tile(int M, int heads, int choice);   // choice 0: the default for M rows
int attn_mfma_tile_keys(int R);

// Launch plan of a step with nq query rows per sequence (host side).
enum { FAMILY_MFMA = 1, FAMILY_GENERIC = 2 };
struct Plan {
    int proj_family, attn_family;
    int splitk, proj_tiles, bm;
    int splits, keys_per_split, R, Rpad;
};

Plan make_plan(const fdllm_config_t& c, int G, const fdllm_tuning_t& tune, int nq);

// Raise a kernel's dynamic LDS limit to the CU's 160 KB, once per device
// (the launches then pass their exact size).
template <auto Kern>
hipError_t allow_full_lds()
{
    static std::atomic<unsigned long long> done{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_relaxed) & bit) return hipSuccess;
    e = hipFuncSetAttribute((const void*)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess) done.fetch_or(bit);
    return e;
}

// Conversions between storage types and fp32.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// XCD-aware workgroup order: consecutive workgroup ids are dispatched round
// robin over the 8 XCDs, so logical tile t runs on XCD t / per.  The grid is
// padded to a multiple of 8; ids past `total` return -1.
__device__ __forceinline__ int xcd_remap(int bid, int total)
{
    const int per = (total + 7) >> 3;
    const int logical = (bid & 7) * per + (bid >> 3);
    return logical < total ? logical : -1;
}

}  // namespace fdllm
