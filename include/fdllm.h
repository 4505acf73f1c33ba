/*
 * fdllm.h -- C ABI of the IO-aware fused KV-cache step of a diffusion LLM
 * attention layer (Flash-dLLM), hand-written HIP for MI355X (gfx950).
 *
 * The operation (Flash-dLLM review on jaehun.me, "How It Works: A Concrete
 * Example", Step 1: Draft and Step 1: Verification; alanhou.org summary,
 * "Core Mechanism", item 1): for every sequence b, read only the hidden
 * states of the query rows Q (tracked set plus the first beta_m masked
 * positions, or the verification layout [tracked | confident | draft view |
 * mask view]), project them to q, k, v on chip, rotate q and k by position,
 * write k and v straight into the persistent flat bidirectional cache at
 * those positions, and attend the query rows over the whole cache under a
 * visibility mask that keeps the draft view and the [MASK] view apart.
 *
 * Conventions shared by every entry point
 *   - All tensors are caller-owned, row-major, contiguous device pointers
 *     (hipMalloc / PyTorch allocations), 16-byte aligned.  Element type of
 *     X, W_qkv, Kc, Vc and O is the configuration's dtype (fp32 or bf16);
 *     LSE is fp32; index arrays are int32; the mask is uint8.
 *   - Shapes (notation of the pages): B sequences, cache length N, model
 *     width d_model, H query heads, Hkv key/value heads (H % Hkv == 0), head
 *     width dh, nq = |Q| query rows per sequence.
 *       X        [B, x_rows, d_model]   hidden states, addressed by Q_idx
 *       W_qkv    [(H + 2 Hkv) dh, d_model]  rows ordered [q heads | k heads |
 *                v heads], head-major, dh contiguous (y = W_qkv x, no bias)
 *       Kc, Vc   [B, Hkv, N, dh]        persistent cache, updated in place;
 *                the cached k is post-rotation
 *       Q_idx    [B, nq]  X row of each query row, 0 <= Q_idx < x_rows
 *       pos_ids  [B, nq]  position of each query row, 0 <= pos_ids < N; two
 *                rows may share a position (the two verification views)
 *       vis_mask [B, nq, nq] or NULL; vis_mask[b,i,j] != 0 lets query row i
 *                see the new key of row j; NULL means all visible
 *       O        [B, nq, H, dh], LSE [B, nq, H] (natural log)
 *   - Rotary embedding: rotate-half pairs (e, e + dh/2), phase
 *     pos * base^(-2e/dh).  Query head h reads kv head h * Hkv / H.
 *     Softmax scale 1/sqrt(dh).
 *   - Write rule: the first row (in Q order) at a position owns the cache
 *     write; later rows at the same position are attended as extra keys and
 *     never written.  Cache rows at positions not in pos_ids[b] are never
 *     touched.
 *   - Key set of query row (b,i): every cache position not in pos_ids[b]
 *     (old content), plus each new row j with vis_mask[b,i,j] != 0.  The old
 *     content at positions in pos_ids[b] is never attended.  An empty key set
 *     gives O = 0 and LSE = -inf.
 *   - Rounding: k and v are rounded once to the dtype after the rotation
 *     (nearest even): they are what the cache stores.  q is built and
 *     consumed on chip, so it keeps its fp32 accumulation and is never
 *     rounded to the dtype.  Accumulation is fp32; O is rounded once at the
 *     end; LSE stays fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous on that stream and never synchronise, except that a
 *     handle created while FDLLM_VALIDATE=1 is set in the environment makes
 *     its steps copy the index arrays to the host and range-check them
 *     first.
 *   - Return value: FDLLM_OK or a negative status; on any error nothing has
 *     been launched.  Indices out of range are undefined behaviour unless
 *     FDLLM_VALIDATE=1.  A handle serves one stream at a time; concurrent
 *     calls on one handle race on its workspace.
 */
#ifndef FDLLM_H
#define FDLLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FDLLM_F32 = 0, FDLLM_BF16 = 1 } fdllm_dtype_t;

enum {
    FDLLM_OK = 0,
    FDLLM_ERR_ARG = -1,      /* null pointer, null handle or invalid configuration */
    FDLLM_ERR_SHAPE = -2,    /* nq > q_max, x_rows < 1, nq < 0 */
    FDLLM_ERR_ALIGN = -3,    /* a tensor pointer not 16-byte aligned */
    FDLLM_ERR_INDEX = -4,    /* index out of range (only with FDLLM_VALIDATE=1) */
    FDLLM_ERR_ALLOC = -5,    /* device workspace allocation failed */
    FDLLM_ERR_HIP = -6,      /* a HIP runtime call or launch failed */
    FDLLM_ERR_UNSUPPORTED = -7, /* shape outside what the kernels implement */
    FDLLM_ERR_SCRATCH = -8   /* workspace larger than the allocation-free scratch */
};

typedef struct {
    int32_t B, N, d_model, H, Hkv, dh;
    int32_t q_max;          /* largest nq any fused step of this handle will use */
    double rope_base;       /* rotary base, e.g. 10000 */
    int32_t dtype;          /* fdllm_dtype_t */
} fdllm_config_t;

/* Launch-shape overrides for sweeps; 0 keeps the library's choice. */
typedef struct {
    int32_t attn_splits;    /* cache splits per (sequence, kv head) in the attention */
    int32_t gemm_splitk;    /* reserved: the projection does not split d_model (plan reports 1) */
    int32_t kernel_family;  /* 0 auto, 1 tiled MFMA (bf16 only), 2 generic scalar */
    int32_t proj_tile;      /* 0 auto, 1..11: a tile configuration of the MFMA projection */
} fdllm_tuning_t;

typedef struct fdllm_ctx* fdllm_handle_t;

/* Host-only check of a configuration (no HIP call).  Returns FDLLM_OK,
 * FDLLM_ERR_ARG or FDLLM_ERR_UNSUPPORTED. */
int fdllm_validate_config(const fdllm_config_t* cfg);

/* Create a handle for one layer's persistent cache.  The cache is the flat,
 * preallocated bidirectional KV store of the pages' system (jaehun.me review,
 * "Performance Validation: Key Results": a flat, preallocated cache without
 * padding; "How It Works: A Concrete Example", Step 1: Draft: every position
 * of it can be rewritten at any step).  The caller owns Kc/Vc [B, Hkv, N, dh];
 * this call validates cfg, allocates the handle's workspace on the current
 * device (rotary table, q staging, duplicate-row side buffer, split partials
 * and counters) and, if X_full is not NULL, builds the cache from the full
 * sequence (see fdllm_prefill with x_rows = N).  W_qkv, Kc, Vc may be NULL
 * when X_full is NULL.  *out receives the handle, or NULL on error.
 * Statuses: ARG, UNSUPPORTED, ALIGN, ALLOC, HIP. */
int fdllm_cache_init(fdllm_handle_t* out, const fdllm_config_t* cfg, const void* X_full,
                     const void* W_qkv, void* Kc, void* Vc, void* stream);

/* Cache build from a full sequence, the state the step starts from (jaehun.me
 * review, "Performance Validation: Key Results": the flat preallocated cache;
 * "How It Works: A Concrete Example", Step 1: Draft: the cache holds k and v
 * of every position, which the step then rewrites at its query positions):
 * for every b and position p < N, row p of X[b] is projected, k is rotated at
 * position p, and k, v are rounded and stored at Kc/Vc[b, :, p, :].  X is
 * [B, x_rows, d_model] with x_rows >= N, device pointers owned by the caller.
 * Asynchronous on stream.  Statuses: ARG, SHAPE, ALIGN, HIP. */
int fdllm_prefill(fdllm_handle_t h, const void* X, int32_t x_rows, const void* W_qkv,
                  void* Kc, void* Vc, void* stream);

/* One fused step (jaehun.me review, "How It Works: A Concrete Example",
 * Step 1: Draft -- only the hidden states of the query rows are read, q, k, v
 * are built on chip, k and v go straight into the cache, and the rows attend
 * over the whole cache -- and Step 1: Verification -- the draft view and the
 * [MASK] view share positions and are kept apart by the mask; alanhou.org
 * summary, "Core Mechanism" item 1: cache lookup, similarity and masked
 * attention fused so intermediates do not round-trip through HBM).
 * Computes, for every sequence b: gather X[b, Q_idx[b, j]] -> q, k, v ->
 * rotary at pos_ids[b, j] -> in-place write of k, v to Kc/Vc[b, :, pos, :]
 * (first row at a position) -> attention of every query row over the whole
 * cache under vis_mask -> O [B, nq, H, dh] (dtype) and LSE [B, nq, H] (fp32,
 * natural log).  Arguments and layouts as in the conventions above; every
 * pointer is a caller-owned device buffer; the handle's workspace holds the
 * step's q rows, duplicate-position k/v rows and ownership flags until the
 * step ends.
 * 0 <= nq <= q_max; nq == 0 launches nothing.  Asynchronous on stream.
 * Statuses: ARG, SHAPE, ALIGN, INDEX (FDLLM_VALIDATE=1 only), HIP. */
int fdllm_fused_step(fdllm_handle_t h, const void* X, int32_t x_rows, const int32_t* Q_idx,
                     const int32_t* pos_ids, int32_t nq, const uint8_t* vis_mask,
                     const void* W_qkv, void* Kc, void* Vc, void* O, float* LSE, void* stream);

/* The two launches of fdllm_fused_step, callable separately (same arguments
 * and statuses; used to time the phases or to run work between them).
 * fdllm_step_project runs gather + projection + rotary + k/v write and leaves
 * the step's fp32 q rows, duplicate-position k/v rows and the rows' ownership
 * flags (which row stored each position in the cache) in the handle's
 * workspace; fdllm_step_attend consumes them (it must follow the project call
 * of the same step on the same stream, with the same nq and pos_ids). */
int fdllm_step_project(fdllm_handle_t h, const void* X, int32_t x_rows, const int32_t* Q_idx,
                       const int32_t* pos_ids, int32_t nq, const void* W_qkv, void* Kc, void* Vc,
                       void* stream);
int fdllm_step_attend(fdllm_handle_t h, const int32_t* pos_ids, int32_t nq, const uint8_t* vis_mask,
                      const void* Kc, const void* Vc, void* O, float* LSE, void* stream);

/* The fused step over a paged cache, with per-sequence valid lengths and
 * query counts, for batched serving (jaehun.me review, "System-Level
 * Metrics": throughput grows with the batch; "What's Next?: Future
 * Directions": a block table under a paged serving stack).  Same step and conventions as
 * fdllm_fused_step, except:
 *   - block_table != NULL: Kpool/Vpool are pools of blocks
 *     [num_blocks, Hkv, block_size, dh]; position p of sequence b lives in
 *     block block_table[b * max_blocks + p / block_size], row p % block_size.
 *     block_size is a power of two in [16, 1024].  block_table == NULL: the
 *     flat layout [B, Hkv, N, dh] (block_size, max_blocks, num_blocks unused).
 *   - seq_len [B] (or NULL = N for all): sequence b has positions
 *     0 .. seq_len[b]-1 (1 <= seq_len[b] <= N and <= max_blocks * block_size);
 *     keys past it are not attended, and every position the step writes must
 *     be below it.
 *   - nq_seq [B] (or NULL = nq for all): rows j >= nq_seq[b] of sequence b
 *     are padding: their Q_idx/pos_ids are ignored, nothing is written for
 *     them, they are no keys, and their O rows are 0 and LSE rows -inf.
 * Table entries of blocks past a sequence's length are not read.
 * FDLLM_VALIDATE=1 checks lengths, indices of the live rows and the used
 * table entries (< num_blocks) on the host.
 * Statuses: ARG, SHAPE, ALIGN, INDEX (FDLLM_VALIDATE=1 only), HIP. */
int fdllm_fused_step_paged(fdllm_handle_t h, const void* X, int32_t x_rows, const int32_t* Q_idx,
                           const int32_t* pos_ids, int32_t nq, const int32_t* nq_seq, const uint8_t* vis_mask,
                           const void* W_qkv, void* Kpool, void* Vpool, const int32_t* block_table,
                           int32_t block_size, int32_t max_blocks, int32_t num_blocks, const int32_t* seq_len,
                           void* O, float* LSE, void* stream);

/* Tracked-set scores, the step after the fused step (jaehun.me review, "How
 * It Works: A Concrete Example", Step 1: Cache selection, with the paragraph
 * on Fig. 1b): the previously decoded tokens most attended by the masked
 * query rows are kept for the next step.  For every cache position p of
 * every sequence b,
 *     scores[b, p] = sum over rows i with sel_rows[b, i] != 0, over the
 *                    query heads h:  exp(q_i,h . k_p / sqrt(dh) - LSE[b, i, h])
 * with the step's q (fp32), the cache row k_p after the step's write, and the
 * step's key-set rule: a position written this step counts for row i only if
 * vis_mask[b, i, owner] != 0 (owner = the first row at that position; NULL =
 * all visible); rows that do not own their position are no cache position
 * and get no score; rows with an empty key set (LSE = -inf) add nothing.
 * It must follow the fused step (or its project call) of the same nq on the
 * same stream: it reads the step's q from the handle's workspace.
 * sel_rows [B, nq] uint8, vis_mask [B, nq, nq] or NULL, Kc [B, Hkv, N, dh] in
 * the cache dtype, LSE [B, nq, H] fp32 from the step, scores [B, N] fp32 out;
 * all device pointers owned by the caller, 16-byte aligned (sel, vis, LSE:
 * 4-byte).  Each kv head's partial sums are added in head order, so repeated
 * calls give identical bits.  Statuses: ARG, SHAPE, ALIGN, UNSUPPORTED (a
 * split of N does not fit in LDS), HIP. */
int fdllm_tracked_scores(fdllm_handle_t h, const int32_t* pos_ids, int32_t nq, const uint8_t* vis_mask,
                         const uint8_t* sel_rows, const void* Kc, const float* LSE, float* scores,
                         void* stream);

/* Top-k selection of the next tracked set: for every sequence b, out[b, :k]
 * receives the k candidate positions (cand[b, p] != 0) with the highest
 * scores[b, p], highest first; equal scores rank the lower position first;
 * -1 fills the places past the number of candidates.  scores [B, N] fp32,
 * cand [B, N] uint8, out [B, k] int32, device pointers owned by the caller.
 * 0 <= k; N <= 16384.  Statuses: ARG, UNSUPPORTED (N > 16384), HIP. */
int fdllm_select_tracked(fdllm_handle_t h, const float* scores, const uint8_t* cand, int32_t k,
                         int32_t* out, void* stream);

/* Flash-Verify decisions on the device (jaehun.me review, "Flash-Verify:
 * Cache-Based Draft-Verification Parallel Decoding" and "How It Works: A
 * Concrete Example", Step 1: Draft / Verification).  They take no handle.
 *
 * fdllm_confidence: for each of `rows` rows of logits [rows, V] (dtype
 * FDLLM_BF16 or FDLLM_F32, 16-byte aligned), pred[r] = the argmax over the ids
 * other than mask_id (equal logits: the lowest id; mask_id < 0 excludes
 * none), conf[r] = that id's probability under the softmax over all V ids
 * (fp32), and, if over != NULL, over[r] = (conf[r] >= thr): with thr = eps
 * this is the split of the draft pass into the confident set (1) and the
 * exploratory set (0); with thr = gamma it is the mask view's confidence test.
 * At least one logit of a row must be finite.  pred int32 [rows], conf fp32
 * [rows], over uint8 [rows], caller-owned device pointers.
 * With fewer rows than CUs a row is spread over several workgroups that meet
 * in a small table of the library's own device memory (8192 row slots per
 * device, each set back to zero by the row's last workgroup); each call takes
 * its rows' slots in turn, so calls in flight together on one device (other
 * streams) stay apart unless they hold more than 8192 such rows between them.
 * Results do not depend on the order the workgroups finish in.
 * Statuses: ARG (NULL pointer, V < 1, rows < 0, dtype), ALIGN, HIP. */
int fdllm_confidence(const void* logits, int32_t dtype, int64_t rows, int32_t V, int32_t mask_id, float thr,
                     int32_t* pred, float* conf, uint8_t* over, void* stream);

/* Sequential acceptance of the verification pass: for each sequence b, the
 * exploratory positions in decoding order are rows 0..S-1 of x_hat (draft
 * predictions), x_tilde and c_tilde (the [MASK] view's predictions and
 * confidences), all [B, S]; n_accept[b] = the number of leading rows with
 * x_tilde == x_hat and c_tilde >= gamma (acceptance stops at the first
 * failure).  Statuses: ARG, HIP. */
int fdllm_accept(const int32_t* x_hat, const int32_t* x_tilde, const float* c_tilde, int32_t B, int32_t S,
                 float gamma, int32_t* n_accept, void* stream);

/* Set (tuning != NULL) or reset (NULL) the launch-shape overrides of h.
 * Statuses: ARG (a negative field, kernel_family > 2, proj_tile > 11). */
int fdllm_set_tuning(fdllm_handle_t h, const fdllm_tuning_t* tuning);

/* Report the launch shapes fdllm_fused_step would use for nq: attention
 * splits, projection d_model splits and the kernel family (1 tiled MFMA,
 * 2 generic).  Any output pointer may be NULL.  Statuses: ARG, SHAPE. */
int fdllm_get_plan(fdllm_handle_t h, int32_t nq, int32_t* attn_splits, int32_t* gemm_splitk,
                   int32_t* kernel_family);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step as fdllm_fused_step with the default launch plan, without a handle.
 * cfg describes the layer (q_max bounds nq); the kernels' workspace (rotary
 * rows of the step's positions, q staging, duplicate-row side buffers, split
 * partials) lives in a static device array of FDLLM_NOALLOC_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends; the call
 * allocates nothing.  Every call on one GPU shares that array and leaves its
 * contents behind, so calls that overlap on one GPU (several streams or
 * threads) race; serialise them.  Indices are not range-checked
 * (FDLLM_VALIDATE does not apply).  Other arguments as for fdllm_fused_step.
 * Statuses: ARG, UNSUPPORTED (invalid configuration), SHAPE, ALIGN, SCRATCH
 * (the step's workspace exceeds the array: about N*dh*4 + B*Hkv*nq*dh*(4G +
 * 2*elt) bytes, plus B*Hkv*splits*R*(dh+2)*4 when the cache is split, with
 * G = H/Hkv and R = nq*G), HIP. */
#define FDLLM_NOALLOC_SCRATCH_BYTES (64ull << 20)
int fdllm_fused_step_noalloc(const fdllm_config_t* cfg, const void* X, int32_t x_rows, const int32_t* Q_idx,
                             const int32_t* pos_ids, int32_t nq, const uint8_t* vis_mask, const void* W_qkv,
                             void* Kc, void* Vc, void* O, float* LSE, void* stream);

/* Free the handle and its workspace (synchronises the device first).
 * NULL is accepted.  Statuses: HIP. */
int fdllm_cache_destroy(fdllm_handle_t h);

/* Static, human-readable name of a status code. */
const char* fdllm_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FDLLM_H */
