// noalloc.hip -- the fused step without a handle, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Its kernels' workspace (rotary rows,
// q staging, duplicate-row side buffers, split partials) lives in `scratch`,
// a file-scope device array of kScratchBytes that every device the library
// runs on holds until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device with hipGetSymbolAddress and only that address is used.
// Calls that overlap on one device share the array and race.
#include <cmath>
#include <mutex>

#include "fdllm.h"
#include "fdllm_common.h"

namespace fdllm {

namespace {

constexpr size_t kScratchBytes = FDLLM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device

int scratch_on(int dev, unsigned char** out)
{
    if (dev < 0 || dev >= kMaxDevices) return FDLLM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FDLLM_ERR_HIP;
        g_scratch[dev] = (unsigned char*)p;
    }
    *out = g_scratch[dev];
    return FDLLM_OK;
}

// The rotary rows of the step's positions, (cos, sin) of pos * base^(-2e/dh)
// evaluated in double and stored fp32 (the values the handle's table holds),
// written at row pos of an [N, dh/2] table.  Rows at a shared position get
// the same values from each writer.
__global__ void __launch_bounds__(64) rope_rows_kernel(const int32_t* pos, int N, int half, int dh, double base,
                                                       float2* tab)
{
    const int p = pos[blockIdx.x];
    if (p < 0 || p >= N) return;   // out-of-range positions are the caller's error; never written outside
    for (int e = threadIdx.x; e < half; e += 64) {
        const double theta = pow(base, -2.0 * (double)e / (double)dh);
        const double phi = (double)p * theta;
        tab[(size_t)p * half + e] = make_float2((float)cos(phi), (float)sin(phi));
    }
}

struct Layout {
    size_t rope, qbuf, sideK, sideV, own, apart, aml, total;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Offsets of the step's workspace in the scratch array (q staging and side
// buffers with nq as their row stride).
Layout layout(const fdllm_config_t& c, int nq, const Plan& p)
{
    const size_t G = c.H / c.Hkv, elt = c.dtype == FDLLM_BF16 ? 2 : 4;
    const size_t half = c.dh / 2;
    Layout l{};
    size_t at = 0;
    l.rope = at;  at += up256((size_t)c.N * half * sizeof(float2));
    l.qbuf = at;  at += up256((size_t)c.B * c.Hkv * nq * G * c.dh * sizeof(float));
    l.sideK = at; at += up256((size_t)c.B * c.Hkv * nq * c.dh * elt);
    l.sideV = at; at += up256((size_t)c.B * c.Hkv * nq * c.dh * elt);
    l.own = at;   at += up256((size_t)c.B * nq);
    const size_t arows = (p.attn_family == FAMILY_MFMA && p.splits > 1) ? (size_t)c.B * c.Hkv * p.splits * p.Rpad : 0;
    l.apart = at; at += up256(arows * c.dh * sizeof(bf16));
    l.aml = at;   at += up256(arows * 2 * sizeof(float));
    l.total = at;
    return l;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

}  // namespace fdllm

using namespace fdllm;

extern "C" int fdllm_fused_step_noalloc(const fdllm_config_t* cfg, const void* X, int32_t x_rows,
                                        const int32_t* Q_idx, const int32_t* pos_ids, int32_t nq,
                                        const uint8_t* vis_mask, const void* W_qkv, void* Kc, void* Vc, void* O,
                                        float* LSE, void* stream)
{
    int st = fdllm_validate_config(cfg);
    if (st) return st;
    const fdllm_config_t& c = *cfg;
    if (nq < 0 || nq > c.q_max || x_rows < 1) return FDLLM_ERR_SHAPE;
    if (nq == 0) return FDLLM_OK;
    if (!X || !Q_idx || !pos_ids || !W_qkv || !Kc || !Vc || !O || !LSE) return FDLLM_ERR_ARG;
    if (!aligned16(X) || !aligned16(W_qkv) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O) || !aligned4(LSE) ||
        !aligned4(Q_idx) || !aligned4(pos_ids))
        return FDLLM_ERR_ALIGN;
    const int G = c.H / c.Hkv;
    const Plan p = make_plan(c, G, fdllm_tuning_t{0, 0, 0, 0}, nq);
    const Layout lay = layout(c, nq, p);
    if (lay.total > kScratchBytes) return FDLLM_ERR_SCRATCH;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FDLLM_ERR_HIP;
    unsigned char* base = nullptr;
    st = scratch_on(dev, &base);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    float2* rope = (float2*)(base + lay.rope);

    hipLaunchKernelGGL(rope_rows_kernel, dim3(c.B * nq), dim3(64), 0, s, pos_ids, c.N, c.dh / 2, c.dh, c.rope_base,
                       rope);
    if (hipGetLastError() != hipSuccess) return FDLLM_ERR_HIP;

    ProjArgs pa{};
    pa.X = X; pa.W = W_qkv; pa.Q_idx = Q_idx; pa.pos_ids = pos_ids; pa.rope = rope;
    pa.Kc = Kc; pa.Vc = Vc;
    pa.qbuf = (float*)(base + lay.qbuf);
    pa.sideK = base + lay.sideK; pa.sideV = base + lay.sideV;
    pa.B = c.B; pa.N = c.N; pa.d = c.d_model; pa.H = c.H; pa.Hkv = c.Hkv; pa.dh = c.dh; pa.G = G;
    pa.x_rows = x_rows; pa.rows_per_seq = nq; pa.q_max = nq;
    pa.prefill = 0; pa.tile_choice = 0;
    pa.map = CacheMap{nullptr, 0, 0};
    pa.nq_seq = nullptr;
    pa.own = (int8_t*)(base + lay.own);
    hipError_t e = p.proj_family == FAMILY_MFMA ? launch_proj_mfma(pa, s) : launch_proj_generic(pa, c.dtype, s);
    if (e != hipSuccess) return FDLLM_ERR_HIP;

    AttnArgs aa{};
    aa.qbuf = pa.qbuf; aa.Kc = Kc; aa.Vc = Vc; aa.sideK = pa.sideK; aa.sideV = pa.sideV;
    aa.pos_ids = pos_ids; aa.vis = vis_mask; aa.O = O; aa.LSE = LSE;
    aa.apart = (bf16*)(base + lay.apart); aa.aml = (float*)(base + lay.aml);
    aa.B = c.B; aa.N = c.N; aa.H = c.H; aa.Hkv = c.Hkv; aa.dh = c.dh; aa.G = G; aa.nq = nq; aa.q_max = nq;
    aa.R = p.R; aa.Rpad = p.Rpad; aa.splits = p.splits; aa.keys_per_split = p.keys_per_split;
    aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.dh));
    aa.map = CacheMap{nullptr, 0, 0};
    aa.seq_len = nullptr;
    aa.nq_seq = nullptr;
    aa.own = pa.own;
    e = p.attn_family == FAMILY_MFMA ? launch_attn_mfma(aa, s) : launch_attn_generic(aa, c.dtype, s);
    return e == hipSuccess ? FDLLM_OK : FDLLM_ERR_HIP;
}
