// fdllm_api.hip -- the C ABI of libfdllm (declared in include/fdllm.h):
// argument checks, the handle's workspace, the rotary table, launch planning
// and the launch sequence of the fused step.  No arithmetic of the step runs
// here: every step runs in the HIP kernels.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "fdllm.h"
#include "fdllm_common.h"

using namespace fdllm;

struct fdllm_ctx {
    fdllm_config_t cfg;
    int device = 0;
    int G = 1;
    size_t elt = 2;
    float2* rope = nullptr;
    float* qbuf = nullptr;
    void* sideK = nullptr;
    void* sideV = nullptr;
    int8_t* own = nullptr;        // [B, q_max] ownership flags of the step's rows
    bf16* apart = nullptr;
    float* aml = nullptr;
    size_t apart_rows = 0;        // (B*Hkv) * splits * Rpad rows available
    float* mpart = nullptr;       // [B * Hkv, N] per kv head sums of the tracked-set scores
    fdllm_tuning_t tune{0, 0, 0, 0};
    bool validate = false;        // FDLLM_VALIDATE=1 when the handle was created: range-check indices
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool env_flag(const char* name)
{
    const char* v = getenv(name);
    return v && *v && atoi(v) != 0;
}

}  // namespace

Plan fdllm::make_plan(const fdllm_config_t& c, int G, const fdllm_tuning_t& tune, int nq)
{
    Plan p{};
    int fam = tune.kernel_family;
    const bool mfma_ok = c.dtype == FDLLM_BF16 && c.dh == 128 && c.d_model % 128 == 0;
    if (fam == 0) fam = mfma_ok ? FAMILY_MFMA : FAMILY_GENERIC;
    if (fam == FAMILY_MFMA && !mfma_ok) fam = FAMILY_GENERIC;
    p.proj_family = fam;
    p.R = nq * G;
    p.Rpad = ((p.R + 15) / 16) * 16;
    p.attn_family = (fam == FAMILY_MFMA && (p.R + 15) / 16 <= 18) ? FAMILY_MFMA : FAMILY_GENERIC;

    // projection: rotary-closed column tiles give enough workgroups on their
    // own; the d_model loop is never split across workgroups
    const int M = c.B * nq;
    p.splitk = 1;
    if (p.proj_family == FAMILY_MFMA && M > 0) {
        const ProjTile pt = proj_mfma_tile(M, c.H + 2 * c.Hkv, tune.proj_tile);
        p.bm = pt.bm;
        p.proj_tiles = ((M + pt.bm - 1) / pt.bm) * (c.H + 2 * c.Hkv) * (128 / pt.bn);
    }

    // attention: (sequence, kv head) pairs x cache splits; one workgroup fills
    // a CU (its LDS ring is 128 KB), so aim at one round of 256 workgroups
    p.splits = 1;
    p.keys_per_split = c.N;
    if (p.attn_family == FAMILY_MFMA && nq > 0) {
        const int tk = attn_mfma_tile_keys(p.R);
        const int bgs = c.B * c.Hkv;
        const int max_splits = (c.N + tk - 1) / tk;
        int sp = tune.attn_splits;
        if (sp <= 0) sp = (256 + bgs - 1) / bgs;
        sp = std::max(1, std::min(sp, max_splits));
        int kps = (c.N + sp - 1) / sp;
        kps = ((kps + tk - 1) / tk) * tk;
        // the per-split slot table lives in LDS: keep a split under 8192 keys
        while (kps > 8192) kps -= tk;
        p.keys_per_split = kps;
        p.splits = (c.N + kps - 1) / kps;
    }
    return p;
}

namespace {

Plan make_plan(const fdllm_ctx* h, int nq) { return fdllm::make_plan(h->cfg, h->G, h->tune, nq); }

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return FDLLM_OK;
    if (env_flag("FDLLM_LOG")) fprintf(stderr, "fdllm: HIP error %s\n", hipGetErrorString(e));
    return FDLLM_ERR_HIP;
}

void free_ws(fdllm_ctx* h)
{
    void* ptrs[] = {h->rope, h->qbuf, h->sideK, h->sideV, h->own, h->apart, h->aml, h->mpart};
    for (void* p : ptrs)
        if (p) (void)hipFree(p);
    h->rope = nullptr; h->qbuf = nullptr; h->sideK = h->sideV = nullptr; h->own = nullptr;
    h->apart = nullptr;
    h->aml = nullptr;
    h->mpart = nullptr;
}

// Size the split buffers for every nq the handle may see.
int ensure_split_ws(fdllm_ctx* h)
{
    const fdllm_config_t& c = h->cfg;
    size_t arows = 0;
    for (int nq = 1; nq <= c.q_max; ++nq) {
        const Plan p = make_plan(h, nq);
        if (p.attn_family == FAMILY_MFMA && p.splits > 1)
            arows = std::max(arows, (size_t)c.B * c.Hkv * p.splits * p.Rpad);
    }
    if (arows > h->apart_rows) {
        if (h->apart) (void)hipFree(h->apart);
        if (h->aml) (void)hipFree(h->aml);
        h->apart = nullptr;
    h->aml = nullptr;
        if (hipMalloc(&h->apart, arows * c.dh * sizeof(bf16)) != hipSuccess ||
            hipMalloc(&h->aml, arows * 2 * sizeof(float)) != hipSuccess) {
            h->apart_rows = 0;
            return FDLLM_ERR_ALLOC;
        }
        h->apart_rows = arows;
    }
    return FDLLM_OK;
}

int set_device(const fdllm_ctx* h)
{
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FDLLM_ERR_HIP;
    if (cur != h->device && hipSetDevice(h->device) != hipSuccess) return FDLLM_ERR_HIP;
    return FDLLM_OK;
}

ProjArgs proj_args(const fdllm_ctx* h, const void* X, int x_rows, const int32_t* Q_idx, const int32_t* pos,
                   int rows_per_seq, const void* W, void* Kc, void* Vc, int prefill)
{
    const fdllm_config_t& c = h->cfg;
    ProjArgs a{};
    a.X = X; a.W = W; a.Q_idx = Q_idx; a.pos_ids = pos; a.rope = h->rope;
    a.Kc = Kc; a.Vc = Vc; a.qbuf = h->qbuf; a.sideK = h->sideK; a.sideV = h->sideV; a.own = h->own;
    a.B = c.B; a.N = c.N; a.d = c.d_model; a.H = c.H; a.Hkv = c.Hkv; a.dh = c.dh; a.G = h->G;
    a.x_rows = x_rows; a.rows_per_seq = rows_per_seq; a.q_max = c.q_max;
    a.prefill = prefill;
    a.tile_choice = prefill ? 0 : h->tune.proj_tile;
    return a;
}

}  // namespace

namespace {

// The projection launch of a step, for the flat or the paged layout, with
// optional per-sequence query counts.
int project_impl(fdllm_ctx* h, const void* X, int32_t x_rows, const int32_t* Q_idx, const int32_t* pos_ids,
                 int32_t nq, const void* W, void* Kc, void* Vc, const CacheMap& map, const int32_t* nq_seq,
                 void* stream, bool validated = false)
{
    if (!h) return FDLLM_ERR_ARG;
    const fdllm_config_t& c = h->cfg;
    if (nq < 0 || nq > c.q_max || x_rows < 1) return FDLLM_ERR_SHAPE;
    if (nq == 0) return FDLLM_OK;
    if (!X || !Q_idx || !pos_ids || !W || !Kc || !Vc) return FDLLM_ERR_ARG;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Kc) || !aligned16(Vc) ||
        (reinterpret_cast<uintptr_t>(Q_idx) & 3u) || (reinterpret_cast<uintptr_t>(pos_ids) & 3u))
        return FDLLM_ERR_ALIGN;
    int st = set_device(h);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!validated && h->validate) {
        std::vector<int32_t> qi((size_t)c.B * nq), pi((size_t)c.B * nq);
        if (hipMemcpyAsync(qi.data(), Q_idx, qi.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipMemcpyAsync(pi.data(), pos_ids, pi.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return FDLLM_ERR_HIP;
        for (size_t t = 0; t < qi.size(); ++t)
            if (qi[t] < 0 || qi[t] >= x_rows || pi[t] < 0 || pi[t] >= c.N) return FDLLM_ERR_INDEX;
    }
    const Plan p = make_plan(h, nq);
    ProjArgs pa = proj_args(h, X, x_rows, Q_idx, pos_ids, nq, W, Kc, Vc, 0);
    pa.map = map;
    pa.nq_seq = nq_seq;
    hipError_t e = p.proj_family == FAMILY_MFMA ? launch_proj_mfma(pa, s) : launch_proj_generic(pa, c.dtype, s);
    return hip_status(e);
}

// The attention launch(es) of a step, for the flat or the paged layout, with
// optional per-sequence valid lengths and query counts.
int attend_impl(fdllm_ctx* h, const int32_t* pos_ids, int32_t nq, const uint8_t* vis, const void* Kc,
                const void* Vc, void* O, float* LSE, const CacheMap& map, const int32_t* seq_len,
                const int32_t* nq_seq, void* stream)
{
    if (!h) return FDLLM_ERR_ARG;
    const fdllm_config_t& c = h->cfg;
    if (nq < 0 || nq > c.q_max) return FDLLM_ERR_SHAPE;
    if (nq == 0) return FDLLM_OK;
    if (!pos_ids || !Kc || !Vc || !O || !LSE) return FDLLM_ERR_ARG;
    if (!aligned16(Kc) || !aligned16(Vc) || !aligned16(O) || (reinterpret_cast<uintptr_t>(LSE) & 3u) ||
        (reinterpret_cast<uintptr_t>(pos_ids) & 3u))
        return FDLLM_ERR_ALIGN;
    int st = set_device(h);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const Plan p = make_plan(h, nq);
    if (p.attn_family == FAMILY_MFMA && p.splits > 1 && (size_t)c.B * c.Hkv * p.splits * p.Rpad > h->apart_rows)
        return FDLLM_ERR_ALLOC;   // not reached: the workspace is sized for every nq
    AttnArgs aa{};
    aa.qbuf = h->qbuf; aa.Kc = Kc; aa.Vc = Vc; aa.sideK = h->sideK; aa.sideV = h->sideV;
    aa.pos_ids = pos_ids; aa.vis = vis; aa.O = O; aa.LSE = LSE;
    aa.apart = h->apart; aa.aml = h->aml;
    aa.B = c.B; aa.N = c.N; aa.H = c.H; aa.Hkv = c.Hkv; aa.dh = c.dh; aa.G = h->G; aa.nq = nq; aa.q_max = c.q_max;
    aa.R = p.R; aa.Rpad = p.Rpad; aa.splits = p.splits; aa.keys_per_split = p.keys_per_split;
    aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.dh));
    aa.map = map;
    aa.seq_len = seq_len;
    aa.nq_seq = nq_seq;
    aa.own = h->own;
    hipError_t e = p.attn_family == FAMILY_MFMA ? launch_attn_mfma(aa, s) : launch_attn_generic(aa, c.dtype, s);
    return hip_status(e);
}

}  // namespace

extern "C" {

const char* fdllm_status_str(int status)
{
    switch (status) {
        case FDLLM_OK: return "FDLLM_OK";
        case FDLLM_ERR_ARG: return "FDLLM_ERR_ARG: null or invalid argument";
        case FDLLM_ERR_SHAPE: return "FDLLM_ERR_SHAPE: size out of range (nq > q_max, nq < 0, x_rows too small)";
        case FDLLM_ERR_ALIGN: return "FDLLM_ERR_ALIGN: tensor pointer not 16-byte aligned";
        case FDLLM_ERR_INDEX: return "FDLLM_ERR_INDEX: Q_idx or pos_ids out of range";
        case FDLLM_ERR_ALLOC: return "FDLLM_ERR_ALLOC: device workspace allocation failed";
        case FDLLM_ERR_HIP: return "FDLLM_ERR_HIP: HIP runtime or launch error";
        case FDLLM_ERR_UNSUPPORTED: return "FDLLM_ERR_UNSUPPORTED: shape not implemented";
        case FDLLM_ERR_SCRATCH: return "FDLLM_ERR_SCRATCH: workspace larger than the allocation-free scratch";
        default: return "FDLLM: unknown status";
    }
}

int fdllm_validate_config(const fdllm_config_t* c)
{
    if (!c) return FDLLM_ERR_ARG;
    if (c->B < 1 || c->N < 1 || c->d_model < 1 || c->H < 1 || c->Hkv < 1 || c->dh < 2 || c->q_max < 1)
        return FDLLM_ERR_ARG;
    if (c->H % c->Hkv != 0 || (c->dh & 1) || !(c->rope_base > 0.0)) return FDLLM_ERR_ARG;
    if (c->dtype != FDLLM_F32 && c->dtype != FDLLM_BF16) return FDLLM_ERR_ARG;
    const int elt = c->dtype == FDLLM_BF16 ? 2 : 4;
    // 16-byte rows everywhere: head width and model width in whole 16 B chunks
    if ((c->dh * elt) % 16 != 0 || (c->d_model * elt) % 16 != 0) return FDLLM_ERR_UNSUPPORTED;
    if (c->dh > 256) return FDLLM_ERR_UNSUPPORTED;           // scalar kernels keep dh <= 256
    if (c->q_max > 32767) return FDLLM_ERR_UNSUPPORTED;      // row slots are int16 in LDS
    if ((int64_t)c->B * c->Hkv * c->N > ((int64_t)1 << 40)) return FDLLM_ERR_UNSUPPORTED;
    return FDLLM_OK;
}

int fdllm_prefill(fdllm_handle_t h, const void* X, int32_t x_rows, const void* W, void* Kc, void* Vc,
                  void* stream)
{
    if (!h || !X || !W || !Kc || !Vc) return FDLLM_ERR_ARG;
    if (x_rows < h->cfg.N) return FDLLM_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Kc) || !aligned16(Vc)) return FDLLM_ERR_ALIGN;
    int st = set_device(h);
    if (st) return st;
    const Plan p = make_plan(h, 1);
    hipStream_t s = (hipStream_t)stream;
    ProjArgs a = proj_args(h, X, x_rows, nullptr, nullptr, h->cfg.N, W, Kc, Vc, 1);
    hipError_t e = p.proj_family == FAMILY_MFMA ? launch_proj_mfma(a, s)
                                                : launch_proj_generic(a, h->cfg.dtype, s);
    return hip_status(e);
}

int fdllm_cache_init(fdllm_handle_t* out, const fdllm_config_t* cfg, const void* X_full, const void* W,
                     void* Kc, void* Vc, void* stream)
{
    if (!out) return FDLLM_ERR_ARG;
    *out = nullptr;
    int st = fdllm_validate_config(cfg);
    if (st) return st;
    if (X_full && (!W || !Kc || !Vc)) return FDLLM_ERR_ARG;
    fdllm_ctx* h = new (std::nothrow) fdllm_ctx();
    if (!h) return FDLLM_ERR_ALLOC;
    h->cfg = *cfg;
    h->G = cfg->H / cfg->Hkv;
    h->validate = env_flag("FDLLM_VALIDATE");
    h->elt = cfg->dtype == FDLLM_BF16 ? 2 : 4;
    if (hipGetDevice(&h->device) != hipSuccess) { delete h; return FDLLM_ERR_HIP; }

    const fdllm_config_t& c = h->cfg;
    const size_t half = c.dh / 2;
    const size_t qrows = (size_t)c.B * c.Hkv * c.q_max * h->G;
    const size_t srows = (size_t)c.B * c.Hkv * c.q_max;
    bool ok = hipMalloc(&h->rope, (size_t)c.N * half * sizeof(float2)) == hipSuccess &&
              hipMalloc(&h->qbuf, qrows * c.dh * sizeof(float)) == hipSuccess &&
              hipMalloc(&h->sideK, srows * c.dh * h->elt) == hipSuccess &&
              hipMalloc(&h->sideV, srows * c.dh * h->elt) == hipSuccess &&
              hipMalloc(&h->own, (size_t)c.B * c.q_max) == hipSuccess &&
              hipMalloc(&h->mpart, (size_t)c.B * c.Hkv * c.N * sizeof(float)) == hipSuccess;
    if (!ok) { free_ws(h); delete h; return FDLLM_ERR_ALLOC; }
    st = ensure_split_ws(h);
    if (st) { free_ws(h); delete h; return st; }

    // rotary table: phase pos * base^(-2e/dh), evaluated in double, stored fp32
    std::vector<float2> tab((size_t)c.N * half);
    for (int p = 0; p < c.N; ++p)
        for (size_t e = 0; e < half; ++e) {
            const double theta = std::pow(c.rope_base, -2.0 * (double)e / (double)c.dh);
            const double phi = (double)p * theta;
            tab[(size_t)p * half + e] = make_float2((float)std::cos(phi), (float)std::sin(phi));
        }
    if (hipMemcpy(h->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
        free_ws(h); delete h; return FDLLM_ERR_HIP;
    }
    if (X_full) {
        st = fdllm_prefill(h, X_full, c.N, W, Kc, Vc, stream);
        if (st) { free_ws(h); delete h; return st; }
    }
    *out = h;
    return FDLLM_OK;
}

int fdllm_set_tuning(fdllm_handle_t h, const fdllm_tuning_t* t)
{
    if (!h) return FDLLM_ERR_ARG;
    if (t && (t->attn_splits < 0 || t->gemm_splitk < 0 || t->kernel_family < 0 || t->kernel_family > 2 ||
              t->proj_tile < 0 || t->proj_tile > 11))
        return FDLLM_ERR_ARG;
    h->tune = t ? *t : fdllm_tuning_t{0, 0, 0, 0};
    int st = set_device(h);
    if (st) return st;
    return ensure_split_ws(h);
}

int fdllm_get_plan(fdllm_handle_t h, int32_t nq, int32_t* attn_splits, int32_t* gemm_splitk, int32_t* family)
{
    if (!h) return FDLLM_ERR_ARG;
    if (nq < 0 || nq > h->cfg.q_max) return FDLLM_ERR_SHAPE;
    const Plan p = make_plan(h, nq);
    if (attn_splits) *attn_splits = p.splits;
    if (gemm_splitk) *gemm_splitk = p.splitk;
    if (family) *family = p.proj_family;
    return FDLLM_OK;
}

int fdllm_step_project(fdllm_handle_t h, const void* X, int32_t x_rows, const int32_t* Q_idx,
                       const int32_t* pos_ids, int32_t nq, const void* W, void* Kc, void* Vc, void* stream)
{
    return project_impl(h, X, x_rows, Q_idx, pos_ids, nq, W, Kc, Vc, CacheMap{nullptr, 0, 0}, nullptr, stream);
}

int fdllm_step_attend(fdllm_handle_t h, const int32_t* pos_ids, int32_t nq, const uint8_t* vis,
                      const void* Kc, const void* Vc, void* O, float* LSE, void* stream)
{
    return attend_impl(h, pos_ids, nq, vis, Kc, Vc, O, LSE, CacheMap{nullptr, 0, 0}, nullptr, nullptr, stream);
}

int fdllm_fused_step_paged(fdllm_handle_t h, const void* X, int32_t x_rows, const int32_t* Q_idx,
                           const int32_t* pos_ids, int32_t nq, const int32_t* nq_seq, const uint8_t* vis,
                           const void* W, void* Kpool, void* Vpool, const int32_t* block_table,
                           int32_t block_size, int32_t max_blocks, int32_t num_blocks, const int32_t* seq_len,
                           void* O, float* LSE, void* stream)
{
    if (!h) return FDLLM_ERR_ARG;
    const fdllm_config_t& c = h->cfg;
    if (nq < 0 || nq > c.q_max || x_rows < 1) return FDLLM_ERR_SHAPE;
    if (nq == 0) return FDLLM_OK;
    if (!X || !Q_idx || !pos_ids || !W || !Kpool || !Vpool || !O || !LSE) return FDLLM_ERR_ARG;
    if (!aligned16(O) || (reinterpret_cast<uintptr_t>(LSE) & 3u)) return FDLLM_ERR_ALIGN;
    CacheMap map{nullptr, 0, 0};
    if (block_table) {
        int bits = 0;
        while ((1 << bits) < block_size && bits < 11) ++bits;
        if (block_size < 16 || block_size > 1024 || (1 << bits) != block_size || max_blocks < 1 || num_blocks < 1)
            return FDLLM_ERR_ARG;
        if ((int64_t)max_blocks * block_size < 1) return FDLLM_ERR_ARG;
        if (reinterpret_cast<uintptr_t>(block_table) & 3u) return FDLLM_ERR_ALIGN;
        map = CacheMap{block_table, bits, max_blocks};
    }
    int st = set_device(h);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    if (h->validate) {
        // host copies of the lengths, indices and table: every row a sequence
        // uses must point inside its valid positions and allocated blocks
        std::vector<int32_t> qi((size_t)c.B * nq), pi((size_t)c.B * nq), nb(c.B, nq), L(c.B, c.N);
        std::vector<int32_t> tab(block_table ? (size_t)c.B * max_blocks : 0);
        bool ok = hipMemcpyAsync(qi.data(), Q_idx, qi.size() * 4, hipMemcpyDeviceToHost, s) == hipSuccess &&
                  hipMemcpyAsync(pi.data(), pos_ids, pi.size() * 4, hipMemcpyDeviceToHost, s) == hipSuccess;
        if (ok && nq_seq) ok = hipMemcpyAsync(nb.data(), nq_seq, nb.size() * 4, hipMemcpyDeviceToHost, s) == hipSuccess;
        if (ok && seq_len) ok = hipMemcpyAsync(L.data(), seq_len, L.size() * 4, hipMemcpyDeviceToHost, s) == hipSuccess;
        if (ok && block_table)
            ok = hipMemcpyAsync(tab.data(), block_table, tab.size() * 4, hipMemcpyDeviceToHost, s) == hipSuccess;
        if (!ok || hipStreamSynchronize(s) != hipSuccess) return FDLLM_ERR_HIP;
        for (int b = 0; b < c.B; ++b) {
            const int cap = block_table ? std::min<int64_t>(c.N, (int64_t)max_blocks * block_size) : c.N;
            if (nb[b] < 0 || nb[b] > nq || L[b] < 1 || L[b] > cap) return FDLLM_ERR_INDEX;
            for (int j = 0; j < nb[b]; ++j) {
                const size_t t = (size_t)b * nq + j;
                if (qi[t] < 0 || qi[t] >= x_rows || pi[t] < 0 || pi[t] >= L[b]) return FDLLM_ERR_INDEX;
            }
            if (block_table)
                for (int k = 0; k < (L[b] + block_size - 1) / block_size; ++k) {
                    const int32_t e = tab[(size_t)b * max_blocks + k];
                    if (e < 0 || e >= num_blocks) return FDLLM_ERR_INDEX;
                }
        }
    }
    st = project_impl(h, X, x_rows, Q_idx, pos_ids, nq, W, Kpool, Vpool, map, nq_seq, stream, true);
    if (st) return st;
    return attend_impl(h, pos_ids, nq, vis, Kpool, Vpool, O, LSE, map, seq_len, nq_seq, stream);
}

int fdllm_fused_step(fdllm_handle_t h, const void* X, int32_t x_rows, const int32_t* Q_idx,
                     const int32_t* pos_ids, int32_t nq, const uint8_t* vis, const void* W, void* Kc,
                     void* Vc, void* O, float* LSE, void* stream)
{
    if (!h) return FDLLM_ERR_ARG;
    if (nq < 0 || nq > h->cfg.q_max || x_rows < 1) return FDLLM_ERR_SHAPE;
    if (nq == 0) return FDLLM_OK;
    // check every argument of both phases before launching either
    if (!X || !Q_idx || !pos_ids || !W || !Kc || !Vc || !O || !LSE) return FDLLM_ERR_ARG;
    if (!aligned16(O) || (reinterpret_cast<uintptr_t>(LSE) & 3u)) return FDLLM_ERR_ALIGN;
    int st = fdllm_step_project(h, X, x_rows, Q_idx, pos_ids, nq, W, Kc, Vc, stream);
    if (st) return st;
    return fdllm_step_attend(h, pos_ids, nq, vis, Kc, Vc, O, LSE, stream);
}

int fdllm_tracked_scores(fdllm_handle_t h, const int32_t* pos_ids, int32_t nq, const uint8_t* vis,
                         const uint8_t* sel, const void* Kc, const float* LSE, float* scores, void* stream)
{
    if (!h) return FDLLM_ERR_ARG;
    const fdllm_config_t& c = h->cfg;
    if (nq < 0 || nq > c.q_max) return FDLLM_ERR_SHAPE;
    if (!pos_ids || !sel || !Kc || !LSE || !scores) return FDLLM_ERR_ARG;
    if (!aligned16(Kc) || (reinterpret_cast<uintptr_t>(LSE) & 3u) || (reinterpret_cast<uintptr_t>(scores) & 3u) ||
        (reinterpret_cast<uintptr_t>(pos_ids) & 3u))
        return FDLLM_ERR_ALIGN;
    int st = set_device(h);
    if (st) return st;
    MassArgs a{};
    a.qbuf = h->qbuf; a.Kc = Kc; a.pos_ids = pos_ids; a.vis = vis; a.sel = sel; a.LSE = LSE;
    a.part = h->mpart; a.scores = scores;
    a.B = c.B; a.N = c.N; a.H = c.H; a.Hkv = c.Hkv; a.dh = c.dh; a.G = h->G; a.nq = nq; a.q_max = c.q_max;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.dh));
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (nq == 0) {
        // no query row: every score is zero (the scalar form runs no row loop)
        a.splits = 1; a.keys_per_split = c.N;
        e = launch_key_mass_generic(a, c.dtype, s);
        return hip_status(e);
    }
    if (c.dtype == FDLLM_BF16 && c.dh == 128) {
        // (sequence, kv head) pairs x key splits: about one round of 256 CUs,
        // each split a multiple of 16 keys whose owner table fits in LDS
        const int bgs = c.B * c.Hkv;
        int sp = std::max(1, (256 + bgs - 1) / bgs);
        int kps = ((c.N + sp - 1) / sp + 15) / 16 * 16;
        while (key_mass_lds_bytes(nq, kps) > 150 * 1024 && kps > 16) kps = (kps / 2 + 15) / 16 * 16;
        if (key_mass_lds_bytes(nq, kps) > 150 * 1024) return FDLLM_ERR_UNSUPPORTED;
        a.keys_per_split = kps;
        a.splits = (c.N + kps - 1) / kps;
        e = launch_key_mass(a, s);
    } else {
        a.splits = 1; a.keys_per_split = c.N;
        e = launch_key_mass_generic(a, c.dtype, s);
    }
    return hip_status(e);
}

int fdllm_select_tracked(fdllm_handle_t h, const float* scores, const uint8_t* cand, int32_t k, int32_t* out,
                         void* stream)
{
    if (!h) return FDLLM_ERR_ARG;
    if (k < 0) return FDLLM_ERR_ARG;
    if (k == 0) return FDLLM_OK;
    if (!scores || !cand || !out) return FDLLM_ERR_ARG;
    if (h->cfg.N > 16384) return FDLLM_ERR_UNSUPPORTED;
    int st = set_device(h);
    if (st) return st;
    return hip_status(launch_select_top(scores, cand, h->cfg.B, h->cfg.N, k, out, (hipStream_t)stream));
}

int fdllm_confidence(const void* logits, int32_t dtype, int64_t rows, int32_t V, int32_t mask_id, float thr,
                     int32_t* pred, float* conf, uint8_t* over, void* stream)
{
    if (rows < 0 || V < 1 || (dtype != FDLLM_BF16 && dtype != FDLLM_F32)) return FDLLM_ERR_ARG;
    if (rows == 0) return FDLLM_OK;
    if (!logits || !pred || !conf) return FDLLM_ERR_ARG;
    if (rows > 0x7fffffff) return FDLLM_ERR_ARG;
    if (!aligned16(logits) || (reinterpret_cast<uintptr_t>(pred) & 3u) || (reinterpret_cast<uintptr_t>(conf) & 3u))
        return FDLLM_ERR_ALIGN;
    return hip_status(launch_confidence(logits, dtype, rows, V, mask_id, thr, pred, conf, over,
                                        (hipStream_t)stream));
}

int fdllm_accept(const int32_t* x_hat, const int32_t* x_tilde, const float* c_tilde, int32_t B, int32_t S,
                 float gamma, int32_t* n_accept, void* stream)
{
    if (B < 0 || S < 0) return FDLLM_ERR_ARG;
    if (B == 0) return FDLLM_OK;
    if (!n_accept || (S > 0 && (!x_hat || !x_tilde || !c_tilde))) return FDLLM_ERR_ARG;
    return hip_status(launch_accept(x_hat, x_tilde, c_tilde, B, S, gamma, n_accept, (hipStream_t)stream));
}

int fdllm_cache_destroy(fdllm_handle_t h)
{
    if (!h) return FDLLM_OK;
    int cur = -1;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(h->device);
    hipError_t e = hipDeviceSynchronize();
    free_ws(h);
    if (cur >= 0) (void)hipSetDevice(cur);
    delete h;
    return hip_status(e);
}

}  // extern "C"
