/*
 * fdllm_oracle.c -- plain fp64 CPU reference of the IO-aware fused KV-cache
 * step of a diffusion LLM attention layer (Flash-dLLM).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests/, the smoke check and the bench's
 * CPU-baseline leg can compare the HIP kernels against an obviously correct,
 * slow implementation.  It shares no code, header, table or constant with the
 * HIP library; every input arrives as fp64 (bf16 and fp32 values upcast
 * exactly by the caller) and every step is a direct loop in fp64.
 *
 * What it computes (sources: "Flash-dLLM: IO-Aware KV Caching and Parallel
 * Decoding ...", the jaehun.me review, section "How It Works: A Concrete
 * Example" (Step 1 Draft / Step 1 Verification) and section "Flash-Verify";
 * the alanhou.org summary, "Core Mechanism" item 1):
 *   a1  gather only the query rows x[Q] of the hidden states;
 *   a2  project them to q, k, v with one fused weight W_qkv (y = W x);
 *   a3  rotate q and k by their position (rotary embedding; the two
 *       verification views share position ids);
 *   a4  write the new k, v straight into the persistent, flat, preallocated
 *       bidirectional cache at those positions;
 *   a5  attend the query rows over the whole cache (softmax(q k^T/sqrt(dh)) v,
 *       natural-log LSE);
 *   a7  under a visibility mask that stops the draft view and the [MASK] view
 *       of the verification pass from seeing each other.
 *
 * Readings where the pages are silent:
 *   - X is addressed by row (Q_idx) and the rotary phase by position
 *     (pos_ids), so the two views can share a position but not a row.
 *   - rotary variant: rotate-half pairs (i, i + dh/2), theta_i =
 *     base^(-2i/dh), phase = pos * theta_i, 0-based absolute positions.
 *   - W_qkv is [(H + 2 Hkv) dh, d_model], rows = output features ordered
 *     [q heads | k heads | v heads], each head dh contiguous; no bias.
 *   - query head h uses kv head g = floor(h * Hkv / H).
 *   - k and v are rounded once to the storage type after the rotation
 *     (round_mode): they are what the cache stores.  q never leaves the chip
 *     in the fused step (it is built on chip and consumed there), so it has
 *     no storage type and is not rounded.  O is rounded once at the end;
 *     LSE stays unrounded.
 *   - first occurrence of a position in Q order owns the cache write; later
 *     rows at the same position are attended as extra keys, never written.
 *   - key set of query row (b,i): every cache position not written by this
 *     step (old content) plus every new row j with vis[b,i,j] != 0
 *     (vis == NULL means all visible).  An empty key set gives O = 0 and
 *     LSE = -inf.
 *
 * Tracked-set scores (the same review, "How It Works", Step 1: Cache
 * selection, and the paragraph on Fig. 1b): the previously decoded tokens
 * most attended by the masked query rows are kept.  Reading: the score of
 * cache position p is the attention mass the selected query rows put on it in
 * this layer, summed over their query heads,
 *     a_p = sum_{i selected} sum_h exp(q_i,h . k_p / sqrt(dh) - LSE_i,h),
 * over the keys row i may see (the visibility rule above, the key at p being
 * the cache row after the step's write); rows that do not own their position
 * are not cache positions and get no score.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t B, N, d_model, H, Hkv, dh;
    double rope_base;
    int32_t round_mode; /* 0 exact fp64, 1 round to fp32, 2 round to bf16 */
} fdllm_oracle_cfg_t;

enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_ALLOC = -2 };

/* Round a double to the nearest bfloat16 value, ties to even.  bfloat16 has
 * 8 significant bits and the exponent range of fp32 (normal minimum 2^-126,
 * subnormal quantum 2^-133, largest finite (2 - 2^-7) * 2^127). */
static double round_to_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    (void)frexp(x, &e);           /* |x| = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                /* quantum exponent for 8 significant bits */
    if (q < -133) q = -133;       /* subnormal range has a fixed quantum */
    double r = ldexp(nearbyint(ldexp(x, -q)), q);  /* nearbyint: ties-to-even */
    const double maxbf = ldexp(255.0, 120);        /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > maxbf) r = copysign(INFINITY, x);
    return r;
}

static double round_store(double x, int mode)
{
    if (mode == 1) return (double)(float)x;  /* C conversion rounds to nearest even */
    if (mode == 2) return round_to_bf16(x);
    return x;
}

/* Threads the OpenMP loops of this library use. */
int fdllm_oracle_threads(void) { return omp_get_max_threads(); }

void fdllm_oracle_round(const double* in, double* out, int64_t n, int32_t mode)
{
    for (int64_t i = 0; i < n; ++i) out[i] = round_store(in[i], mode);
}

static int check_cfg(const fdllm_oracle_cfg_t* c)
{
    if (!c || c->B < 1 || c->N < 1 || c->d_model < 1 || c->H < 1 || c->Hkv < 1 ||
        c->dh < 2 || (c->dh & 1) || (c->H % c->Hkv) || c->rope_base <= 0.0)
        return ORC_ERR_ARG;
    return ORC_OK;
}

/* Rotary embedding of one head vector in place: rotate-half pairing. */
static void rope_rotate(double* v, int dh, int64_t pos, double base)
{
    int half = dh / 2;
    for (int i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)dh);
        double phi = (double)pos * theta;
        double c = cos(phi), s = sin(phi);
        double a = v[i], b = v[i + half];
        v[i] = a * c - b * s;
        v[i + half] = b * c + a * s;
    }
}

/* a1-a3: gather, project, rotate; k and v rounded to the storage type.
 * q_out [B,nq,H,dh], k_out/v_out [B,nq,Hkv,dh]. */
int fdllm_oracle_project(const fdllm_oracle_cfg_t* cfg, const double* X, int32_t x_rows,
                         const int32_t* Q_idx, const int32_t* pos_ids, int32_t nq,
                         const double* W, double* q_out, double* k_out, double* v_out)
{
    if (check_cfg(cfg) || !X || !Q_idx || !pos_ids || !W || !q_out || !k_out || !v_out ||
        nq < 0 || x_rows < 1)
        return ORC_ERR_ARG;
    const int B = cfg->B, d = cfg->d_model, H = cfg->H, Hkv = cfg->Hkv, dh = cfg->dh;
    const int cols = (H + 2 * Hkv) * dh;
    for (int64_t t = 0; t < (int64_t)B * nq; ++t) {
        int32_t r = Q_idx[t], p = pos_ids[t];
        if (r < 0 || r >= x_rows || p < 0 || p >= cfg->N) return ORC_ERR_ARG;
    }
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic)
    for (int64_t t = 0; t < (int64_t)B * nq; ++t) {
        int64_t b = t / nq;
        const double* x = X + ((int64_t)b * x_rows + Q_idx[t]) * d;
        double* y = (double*)malloc(sizeof(double) * cols);
        if (!y) { err = ORC_ERR_ALLOC; continue; }
        for (int o = 0; o < cols; ++o) {
            const double* w = W + (int64_t)o * d;
            double acc = 0.0;
            for (int k = 0; k < d; ++k) acc += w[k] * x[k];
            y[o] = acc;
        }
        for (int h = 0; h < H; ++h) rope_rotate(y + h * dh, dh, pos_ids[t], cfg->rope_base);
        for (int g = 0; g < Hkv; ++g) rope_rotate(y + (H + g) * dh, dh, pos_ids[t], cfg->rope_base);
        for (int o = 0; o < H * dh; ++o)
            q_out[t * H * dh + o] = y[o];  /* on-chip value: not rounded */
        for (int o = 0; o < Hkv * dh; ++o) {
            k_out[t * Hkv * dh + o] = round_store(y[H * dh + o], cfg->round_mode);
            v_out[t * Hkv * dh + o] = round_store(y[(H + Hkv) * dh + o], cfg->round_mode);
        }
        free(y);
    }
    return err;
}

/* Does row j of sequence b own the cache write of its position (first
 * occurrence of that position in Q order)? */
static int owns_write(const int32_t* pos_b, int j)
{
    for (int jj = 0; jj < j; ++jj)
        if (pos_b[jj] == pos_b[j]) return 0;
    return 1;
}

/* Full step a1-a7.  Kc/Vc [B,Hkv,N,dh] are read (old content) and updated in
 * place.  O [B,nq,H,dh], LSE [B,nq,H].  q/k/v_out are optional (may be NULL)
 * copies of the rounded projections, for tests. */
int fdllm_oracle_step(const fdllm_oracle_cfg_t* cfg, const double* X, int32_t x_rows,
                      const int32_t* Q_idx, const int32_t* pos_ids, int32_t nq,
                      const uint8_t* vis, const double* W, double* Kc, double* Vc,
                      double* O, double* LSE, double* q_keep, double* k_keep, double* v_keep)
{
    if (check_cfg(cfg) || !Kc || !Vc || !O || !LSE || nq < 0) return ORC_ERR_ARG;
    const int B = cfg->B, N = cfg->N, H = cfg->H, Hkv = cfg->Hkv, dh = cfg->dh;
    const int64_t nrow = (int64_t)B * nq;
    double* q = (double*)malloc(sizeof(double) * (nrow * H * dh + 1));
    double* k = (double*)malloc(sizeof(double) * (nrow * Hkv * dh + 1));
    double* v = (double*)malloc(sizeof(double) * (nrow * Hkv * dh + 1));
    unsigned char* written = (unsigned char*)calloc((size_t)B * N, 1);
    if (!q || !k || !v || !written) { free(q); free(k); free(v); free(written); return ORC_ERR_ALLOC; }
    int err = fdllm_oracle_project(cfg, X, x_rows, Q_idx, pos_ids, nq, W, q, k, v);
    if (err) { free(q); free(k); free(v); free(written); return err; }

    /* Positions written by this step (P_b); their old content is never attended. */
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < nq; ++j) written[(int64_t)b * N + pos_ids[(int64_t)b * nq + j]] = 1;

    /* Attention a5/a7 reads the old cache for positions outside P_b and the
     * new rows k, v directly, so it does not depend on the write-back a4.  It
     * runs first so that the in-place update below cannot be observed. */
    const double scale = 1.0 / sqrt((double)dh);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < nq; ++i) {
            for (int h = 0; h < H; ++h) {
                const int g = (int)(((int64_t)h * Hkv) / H);
                const double* qi = q + (((int64_t)b * nq + i) * H + h) * dh;
                const double* Kb = Kc + (((int64_t)b * Hkv + g) * N) * dh;
                const double* Vb = Vc + (((int64_t)b * Hkv + g) * N) * dh;
                /* pass 1: max score over the key set */
                double m = -INFINITY;
                for (int p = 0; p < N; ++p) {
                    if (written[(int64_t)b * N + p]) continue;
                    double s = 0.0;
                    for (int e = 0; e < dh; ++e) s += qi[e] * Kb[(int64_t)p * dh + e];
                    s *= scale;
                    if (s > m) m = s;
                }
                for (int j = 0; j < nq; ++j) {
                    if (vis && !vis[((int64_t)b * nq + i) * nq + j]) continue;
                    const double* kj = k + (((int64_t)b * nq + j) * Hkv + g) * dh;
                    double s = 0.0;
                    for (int e = 0; e < dh; ++e) s += qi[e] * kj[e];
                    s *= scale;
                    if (s > m) m = s;
                }
                double* o = O + (((int64_t)b * nq + i) * H + h) * dh;
                double* lse = LSE + ((int64_t)b * nq + i) * H + h;
                if (m == -INFINITY) {          /* empty key set */
                    for (int e = 0; e < dh; ++e) o[e] = 0.0;
                    *lse = -INFINITY;
                    continue;
                }
                /* pass 2: denominator and weighted values */
                double l = 0.0;
                double* acc = (double*)calloc(dh, sizeof(double));
                for (int p = 0; p < N; ++p) {
                    if (written[(int64_t)b * N + p]) continue;
                    double s = 0.0;
                    for (int e = 0; e < dh; ++e) s += qi[e] * Kb[(int64_t)p * dh + e];
                    double w = exp(s * scale - m);
                    l += w;
                    for (int e = 0; e < dh; ++e) acc[e] += w * Vb[(int64_t)p * dh + e];
                }
                for (int j = 0; j < nq; ++j) {
                    if (vis && !vis[((int64_t)b * nq + i) * nq + j]) continue;
                    const double* kj = k + (((int64_t)b * nq + j) * Hkv + g) * dh;
                    const double* vj = v + (((int64_t)b * nq + j) * Hkv + g) * dh;
                    double s = 0.0;
                    for (int e = 0; e < dh; ++e) s += qi[e] * kj[e];
                    double w = exp(s * scale - m);
                    l += w;
                    for (int e = 0; e < dh; ++e) acc[e] += w * vj[e];
                }
                for (int e = 0; e < dh; ++e) o[e] = round_store(acc[e] / l, cfg->round_mode);
                *lse = m + log(l);
                free(acc);
            }
        }

    /* a4: write-back, first occurrence of each position owns the slot. */
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < nq; ++j) {
            const int32_t* pb = pos_ids + (int64_t)b * nq;
            if (!owns_write(pb, j)) continue;
            for (int g = 0; g < Hkv; ++g) {
                int64_t dst = (((int64_t)b * Hkv + g) * N + pb[j]) * dh;
                int64_t src = (((int64_t)b * nq + j) * Hkv + g) * dh;
                memcpy(Kc + dst, k + src, sizeof(double) * dh);
                memcpy(Vc + dst, v + src, sizeof(double) * dh);
            }
        }

    if (q_keep) memcpy(q_keep, q, sizeof(double) * nrow * H * dh);
    if (k_keep) memcpy(k_keep, k, sizeof(double) * nrow * Hkv * dh);
    if (v_keep) memcpy(v_keep, v, sizeof(double) * nrow * Hkv * dh);
    free(q); free(k); free(v); free(written);
    return ORC_OK;
}

/* Cache build from a full sequence: the projection a1-a3 and write a4 with
 * the query set = every position 0..N-1 (X row p at position p).  Only the k
 * and v heads are kept. */
int fdllm_oracle_prefill(const fdllm_oracle_cfg_t* cfg, const double* X, int32_t x_rows,
                         const double* W, double* Kc, double* Vc)
{
    if (check_cfg(cfg) || !X || !W || !Kc || !Vc || x_rows < cfg->N) return ORC_ERR_ARG;
    const int B = cfg->B, N = cfg->N, H = cfg->H, Hkv = cfg->Hkv, dh = cfg->dh;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * N);
    double* q = (double*)malloc(sizeof(double) * (size_t)B * N * H * dh);
    double* k = (double*)malloc(sizeof(double) * (size_t)B * N * Hkv * dh);
    double* v = (double*)malloc(sizeof(double) * (size_t)B * N * Hkv * dh);
    if (!idx || !q || !k || !v) { free(idx); free(q); free(k); free(v); return ORC_ERR_ALLOC; }
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < N; ++p) idx[(int64_t)b * N + p] = p;
    int err = fdllm_oracle_project(cfg, X, x_rows, idx, idx, N, W, q, k, v);
    if (!err)
        for (int b = 0; b < B; ++b)
            for (int p = 0; p < N; ++p)
                for (int g = 0; g < Hkv; ++g) {
                    int64_t dst = (((int64_t)b * Hkv + g) * N + p) * dh;
                    int64_t src = (((int64_t)b * N + p) * Hkv + g) * dh;
                    memcpy(Kc + dst, k + src, sizeof(double) * dh);
                    memcpy(Vc + dst, v + src, sizeof(double) * dh);
                }
    free(idx); free(q); free(k); free(v);
    return err;
}

/* Tracked-set scores: a_p for every cache position p of every sequence.
 * q [B,nq,H,dh] (the step's unrounded q), Kc [B,Hkv,N,dh] after the step's
 * write, LSE [B,nq,H] of the step, sel [B,nq] (1: the row contributes),
 * vis [B,nq,nq] or NULL.  scores [B,N]. */
int fdllm_oracle_key_scores(const fdllm_oracle_cfg_t* cfg, const double* q, const double* Kc,
                            const double* LSE, const int32_t* pos_ids, int32_t nq, const uint8_t* vis,
                            const uint8_t* sel, double* scores)
{
    if (check_cfg(cfg) || !q || !Kc || !LSE || !pos_ids || !sel || !scores || nq < 0) return ORC_ERR_ARG;
    const int B = cfg->B, N = cfg->N, H = cfg->H, Hkv = cfg->Hkv, dh = cfg->dh;
    const double scale = 1.0 / sqrt((double)dh);
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        const int32_t* pb = pos_ids + (int64_t)b * nq;
        int* owner = (int*)malloc(sizeof(int) * (size_t)N);
        if (!owner) { err = ORC_ERR_ALLOC; continue; }
        for (int p = 0; p < N; ++p) owner[p] = -1;
        for (int j = 0; j < nq; ++j)
            if (owner[pb[j]] < 0) owner[pb[j]] = j;
        for (int p = 0; p < N; ++p) {
            double a = 0.0;
            for (int i = 0; i < nq; ++i) {
                if (!sel[(int64_t)b * nq + i]) continue;
                const int j = owner[p];
                if (j >= 0 && vis && !vis[((int64_t)b * nq + i) * nq + j]) continue;
                for (int h = 0; h < H; ++h) {
                    const double lse = LSE[((int64_t)b * nq + i) * H + h];
                    if (isinf(lse)) continue;
                    const int g = (int)(((int64_t)h * Hkv) / H);
                    const double* qi = q + (((int64_t)b * nq + i) * H + h) * dh;
                    const double* kp = Kc + (((int64_t)b * Hkv + g) * N + p) * dh;
                    double s = 0.0;
                    for (int e = 0; e < dh; ++e) s += qi[e] * kp[e];
                    a += exp(s * scale - lse);
                }
            }
            scores[(int64_t)b * N + p] = a;
        }
        free(owner);
    }
    return err;
}
