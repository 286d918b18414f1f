/*
 * libtwotower_attn -- the TwoTower denoiser's block-attention step and its
 * confidence-unmask SampleStep, for AMD Instinct MI355X (gfx950).
 *
 * Method: "Nemotron-TwoTower: Diffusion Language Modeling with Pretrained
 * Autoregressive Context" (arXiv 2606.26493).
 *   - tt_block_attn: section 2.1 ("Bidirectional attention"), Eq. (1). The S
 *     queries of the noisy block b at denoiser layer i attend to the
 *     concatenation of the context tower's layer-i KV cache for the clean
 *     prefix (blocks before b) and the denoiser's own layer-i KV for block b.
 *   - tt_lse_merge: the concatenation in Eq. (1) split into disjoint key
 *     sets; partial attentions over the parts combine exactly through their
 *     log-sum-exp values.
 *   - tt_conf_unmask: section 2.2 ("Sampling"), Algorithm 2, the
 *     ConfidenceSample step: commit the masked predictions whose confidence
 *     exceeds gamma, so that the block still completes within the steps left.
 *   - tt_kv_append: section 2.1, Algorithm 1, the update of the AR context
 *     after a block is committed: the context cache of each attention layer
 *     grows by the committed block's keys and values.
 *   - tt_masked_nll: section 2.2, Eq. (4), the masked-diffusion training loss
 *     L_MD: the mean negative log-likelihood of the clean tokens over the
 *     masked positions.
 *
 * Conventions shared by every call:
 *   - Pointers named as tensors are DEVICE pointers owned by the caller. The
 *     library allocates no device memory; scratch comes from a caller-owned
 *     workspace of at least tt_*_workspace_bytes(...) bytes, except in
 *     tt_block_attn_noalloc, which uses a fixed array inside the library.
 *   - Calls are asynchronous on the caller's stream and never synchronise the
 *     host. A returned TT_OK means the work was enqueued.
 *   - Arguments are validated on the host before anything is launched; a
 *     non-TT_OK status means nothing was enqueued (except TT_ERR_HIP, which
 *     reports a failed launch).
 *   - Element strides count elements, not bytes; the innermost dimension
 *     (head_dim or vocabulary) is always contiguous. For tt_block_attn and
 *     tt_lse_merge, tensor base pointers must be 16-byte aligned and strides
 *     multiples of 16 bytes; tt_conf_unmask takes any element-aligned rows.
 *   - Calls that share a workspace must not overlap in time (same stream or
 *     ordered streams). Calls with distinct workspaces are independent; the
 *     library keeps no state besides a per-device cache of the CU count and,
 *     for tt_block_attn_noalloc, each device's scratch array and its address.
 *   - No C++ exception crosses this interface.
 */
#ifndef TWOTOWER_ATTN_H
#define TWOTOWER_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TT_ABI_VERSION 3  /* 2: tt_conf_unmask_params gained uniforms; 3: tt_block_attn_params gained debug_flags */

/* Bits tt_block_attn ORs into *debug_flags in debug mode (see tt_block_attn_params). */
#define TT_DEBUG_CTX_LEN 1  /* a ctx_len[b] below 0 or above max_ctx_len was read */
#define TT_DEBUG_PAGE_ID 2  /* a page id outside [0, num_pages) was read for a prefix token */

typedef enum tt_status {
    TT_OK = 0,
    TT_ERR_NULL = 1,        /* a required pointer is NULL */
    TT_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes or strides */
    TT_ERR_DTYPE = 3,       /* unsupported element type combination */
    TT_ERR_UNSUPPORTED = 4, /* valid but not implemented (head_dim, alignment) */
    TT_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    TT_ERR_ARG = 6,         /* bad scalar argument (NaN gamma, temperature <= 0, ...) */
    TT_ERR_HIP = 7          /* the HIP runtime reported an error */
} tt_status;

typedef enum tt_dtype {
    TT_F32 = 0,  /* IEEE binary32 */
    TT_BF16 = 1  /* bfloat16 (upper half of binary32); outputs are rounded to nearest even */
} tt_dtype;

/* ABI version of the loaded library (TT_ABI_VERSION at build time). */
int tt_abi_version(void);

/* Static description of a status code; never NULL. */
const char* tt_status_string(tt_status status);

/* ------------------------------------------------------------------------ *
 * Eq. (1) block attention for one denoiser attention layer
 * ------------------------------------------------------------------------ *
 * For sequence b, query head h (KV head g = h / (Hq/Hkv)) and block position
 * s, the key set is the concatenation of
 *   - the prefix: tokens j = 0 .. ctx_len[b]-1 of the context tower's cache
 *     for this layer (pass the context cache of the same layer index: the
 *     cross-attention is layer-aligned), and
 *   - the block: tokens 0 .. S-1 of Kden/Vden (every block query sees every
 *     block key; there is no mask inside the step).
 * The call computes scaled-dot-product softmax attention over that set:
 *   sigma_j = softmax_scale * <Q[b][s][h], K_j>,
 *   O[b][s][h] = sum_j softmax(sigma)_j V_j,
 *   LSE[b][h][s] = ln sum_j exp(sigma_j)          (natural log, float32).
 * An empty key set (ctx_len[b] = 0 and Kden = NULL) yields O = 0, LSE = -inf.
 * Positional encoding, if any, is applied by the caller beforehand.
 *
 * Layouts (elements; the head_dim axis contiguous):
 *   Q          [B][S][Hq][head_dim] at Q + b*q_stride_b + s*q_stride_s + h*q_stride_h
 *   Kctx, Vctx paged cache [num_pages][Hkv][page_size][head_dim], dense.
 *              Prefix token j of sequence b is slot j % page_size of page
 *              page_table[b*max_pages + j / page_size]. A contiguous cache
 *              is the identity table (one page of page_size = max_ctx_len
 *              per sequence, or consecutive 16-token pages).
 *   page_table [B][max_pages] int32 (device). Entries past the last page a
 *              sequence uses are never read.
 *   ctx_len    [B] int32 (device): prefix length per sequence, 0 allowed, any
 *              value (the last page may be partial). Values are clamped to
 *              [0, min(max_ctx_len, max_pages*page_size)]; a page id outside
 *              [0, num_pages) is clamped into it (no fault, wrong result).
 *   Kden, Vden [B][S][Hkv][head_dim] at base + b*den_stride_b + s*den_stride_s
 *              + g*den_stride_h; both NULL for a prefix-only partial.
 *   O          [B][S][Hq][head_dim] of o_dtype at O + b*o_stride_b + ...
 *   LSE        [B][Hq][S] float32, dense; may be NULL.
 * dtype is the type of Q, Kctx, Vctx, Kden, Vden; o_dtype is dtype or TT_F32
 * (float32 partials for a later tt_lse_merge).
 *
 * Supported: dtype TT_BF16 (MFMA path, float32 accumulation) or TT_F32
 * (float32 path); head_dim 64 or 128; 1 <= S <= 64; Hq % Hkv == 0;
 * page_size a positive multiple of 16; softmax_scale finite and > 0; every
 * element stride below 2^31, B*max_pages below 2^30, and the largest element
 * offset inside one sequence of Q, O and Kden/Vden ((S-1)*stride_s +
 * (H-1)*stride_h + head_dim) below 2^30 (TT_ERR_UNSUPPORTED otherwise).
 *
 * Debug mode: when debug_flags is not NULL the kernels also check the device
 * data they read and OR TT_DEBUG_CTX_LEN (when max_ctx_len > 0: a ctx_len[b]
 * outside [0, max_ctx_len]) and TT_DEBUG_PAGE_ID (a page id outside
 * [0, num_pages) for a prefix token) into *debug_flags, a device int32 that
 * the caller zeroes beforehand and reads after the stream reaches the call.
 * The outputs are those of the clamped data either way. Debug mode also fills
 * the kernels' LDS buffers with all-ones bytes (NaN, page id -1) before the
 * call's first load into them, so a read of LDS that the call never filled
 * would show in the outputs or the flags. With debug_flags NULL nothing is
 * checked or filled.
 */
typedef struct tt_block_attn_params {
    int32_t dtype;        /* tt_dtype of Q and K/V */
    int32_t o_dtype;      /* tt_dtype of O: dtype or TT_F32 */
    int32_t B, S, Hq, Hkv, head_dim;
    float softmax_scale;  /* usually 1/sqrt(head_dim) */

    const void* Q;
    int64_t q_stride_b, q_stride_s, q_stride_h;

    const void* Kctx;
    const void* Vctx;
    int32_t page_size;
    int32_t num_pages;
    const int32_t* page_table;
    int32_t max_pages;
    const int32_t* ctx_len;
    int32_t max_ctx_len;  /* host-side upper bound of ctx_len[] */

    const void* Kden;
    const void* Vden;
    int64_t den_stride_b, den_stride_s, den_stride_h;

    void* O;
    int64_t o_stride_b, o_stride_s, o_stride_h;
    float* LSE;
    int32_t* debug_flags; /* NULL, or a device int32 that enables the debug-mode checks */
} tt_block_attn_params;

/* Workspace bytes tt_block_attn needs for these parameters (0 if none). The
 * size depends on B, S, Hq, Hkv, head_dim, dtype and the number of compute
 * units of the current device. Returns 0 for NULL. */
size_t tt_block_attn_workspace_bytes(const tt_block_attn_params* p);

/* Enqueue Eq. (1) on `stream`. workspace: device memory of ws_bytes bytes
 * (may be NULL when the required size is 0). */
tt_status tt_block_attn(const tt_block_attn_params* p, void* workspace, size_t ws_bytes,
                        hipStream_t stream);

/* Allocation-free variant of tt_block_attn, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses that
 * forbid allocation). Same parameters, kernels and results as tt_block_attn;
 * instead of a caller workspace it uses a fixed scratch array of
 * TT_NOALLOC_SCRATCH_BYTES inside the library, which each GPU the library
 * runs on holds until the process ends (its address is looked up on the first
 * call on each device). It calls no allocator. Returns TT_ERR_WORKSPACE,
 * before launching anything, when tt_block_attn_workspace_bytes(p) exceeds
 * TT_NOALLOC_SCRATCH_BYTES (at head_dim 128 that allows about 750 (sequence,
 * kv head, 256-row block) pairs with bf16 output, 250 with float32 output).
 * Nothing in the array needs clearing between calls. All calls on one GPU
 * share that GPU's array:
 * calls that overlap in time on one GPU (different streams, or different
 * host threads) race and must be ordered by the caller. */
#define TT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tt_status tt_block_attn_noalloc(const tt_block_attn_params* p, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Log-sum-exp merge of P partial attentions over disjoint key sets
 * ------------------------------------------------------------------------ *
 * Per row (b, s, h): M = max_p lse_p, w_p = exp(lse_p - M),
 *   O = sum_p w_p O_p / sum_p w_p,  lse = M + ln(sum_p w_p).
 * A part with lse = -inf holds no keys and has weight 0; if every part is
 * empty the row gets O = 0 and lse = -inf. Merging tt_block_attn over the
 * prefix only (Kden = NULL, o_dtype TT_F32) with tt_block_attn over the block
 * only (ctx_len = 0) reproduces tt_block_attn over both.
 *   O_parts   [P][B][S][Hq][d] float32, dense (device)
 *   lse_parts [P][B][Hq][S] float32, dense (device)
 *   O_out     [B][S][Hq][d] of o_dtype (TT_F32 or TT_BF16), dense
 *   lse_out   [B][Hq][S] float32, dense; may be NULL
 * Requires P >= 1, B >= 0, S >= 1, Hq >= 1, d >= 4 with d % 4 == 0.
 */
tt_status tt_lse_merge(int P, const float* O_parts, const float* lse_parts, int B, int S, int Hq,
                       int d, void* O_out, tt_dtype o_dtype, float* lse_out, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * ConfidenceSample: one step of confidence unmasking (Algorithm 2)
 * ------------------------------------------------------------------------ *
 * For each sequence b and each MASKED position l (mask_in[b][l] != 0), over
 * the V logits x of row (b, l):
 *   a_l    = the smallest v with x_v = max_u x_u        (greedy prediction)
 *   conf_l = max_v softmax(x / temperature)_v = 1 / sum_v exp((x_v - max x)/temperature)
 * Let M be the number of masked positions and k = ceil(M / steps_left)
 * (steps_left = T - r + 1 at step r of T). If at least k masked positions
 * have conf_l > gamma (strictly), exactly those are committed; otherwise the
 * k masked positions with the highest confidence are committed (equal
 * confidences: the lower position first). A committed position gets
 * tokens[b][l] = a_l and mask_out[b][l] = 0. Every other position keeps its
 * token and mask; rows of unmasked positions are not read. At steps_left = 1
 * every masked position is committed, so T steps always complete the block.
 *
 *   logits   [B][S][V] (dtype), row (b,l) at logits + (b*S + l)*logits_stride_row
 *   mask_in  [B][S] uint8, 1 = masked
 *   mask_out [B][S] uint8 (may alias mask_in)
 *   tokens   [B][S] int32, in/out (the caller fills masked positions with its
 *            mask token id)
 *   conf     [B][S] float32, optional: written for masked positions only
 *   num_masked [B] int32, optional: masked positions left after the step
 * Requires 1 <= S <= 64, V >= 1, logits_stride_row >= V, gamma not NaN,
 * temperature finite and > 0, steps_left >= 1. Rows must hold at least one
 * finite logit; -inf logits have probability 0.
 *
 * Stochastic draw (the sampler's temperature argument, section 2.2
 * "Sampling"): when uniforms is not NULL, a_l is drawn from
 * p = softmax(x / temperature) instead of taken greedily, by inverse transform
 * sampling with u = uniforms[b][l]: a_l is the smallest v whose cumulative
 * probability p_0 + ... + p_v exceeds u (the largest v with p_v > 0 when none
 * does), and conf_l = p_{a_l}. The commit rule is unchanged.
 *   uniforms [B][S] float32 device array, optional; values outside [0, 1] are
 *            clamped to it and NaN counts as 0. The caller owns the generator:
 *            the library draws no random numbers. The cumulative sums are
 *            float32, so a u within about 1e-5 of a cumulative value may select
 *            the neighbouring token. With uniforms the vocabulary is cut
 *            into at most 64 splits of at most 2^21 logits each, so
 *            V <= 2^27 is accepted and a larger V returns TT_ERR_SHAPE
 *            before anything is launched.
 */
typedef struct tt_conf_unmask_params {
    int32_t dtype;  /* tt_dtype of logits */
    int32_t B, S, V;
    const void* logits;
    int64_t logits_stride_row;
    const uint8_t* mask_in;
    uint8_t* mask_out;
    int32_t* tokens;
    float gamma;
    float temperature;
    int32_t steps_left;
    float* conf;
    int32_t* num_masked;
    const float* uniforms;
} tt_conf_unmask_params;

size_t tt_conf_unmask_workspace_bytes(const tt_conf_unmask_params* p);

tt_status tt_conf_unmask(const tt_conf_unmask_params* p, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Commit-time KV append: the context cache grows by the committed block
 * ------------------------------------------------------------------------ *
 * Algorithm 1 (section 2.1): once block b is committed, the context tower
 * runs causally over its S tokens and extends its per-layer KV cache, so the
 * next block's Eq. (1) sees a prefix longer by S. This call is the cache side
 * of that update for one layer: the S new rows of every sequence b are written
 * at prefix positions ctx_len[b] .. ctx_len[b]+S-1 and ctx_len[b] grows by S.
 *
 * Position j of sequence b is slot j % page_size of page
 * page_table[b*max_pages + j / page_size] (the layout tt_block_attn reads).
 * A table entry < 0 that a new position needs is filled from the caller's
 * pool of free page ids, pool[0 .. *pool_count-1], taken from the top: the
 * first page needed (lowest sequence, then lowest position) gets
 * pool[*pool_count-1], the next pool[*pool_count-2], and so on; *pool_count
 * decreases by the number taken. The assignment is therefore deterministic.
 *
 * All or nothing: the call changes no cache row, table entry, ctx_len or
 * *pool_count, and writes *status != 0, if any sequence would pass
 * max_pages*page_size positions (status 1), more pages are needed than the
 * pool holds (status 2; pool may be NULL when no page is needed), or a page id
 * it would write to (from the table or the pool) is outside [0, num_pages)
 * (status 3). Otherwise it performs the append and writes *status = 0.
 * status is device memory; read it after the stream reaches the call.
 *
 *   Kctx, Vctx [num_pages][Hkv][page_size][head_dim] of dtype, in/out
 *   page_table [B][max_pages] int32, in/out
 *   ctx_len    [B] int32, in/out (a negative length counts as 0)
 *   Knew, Vnew [B][S][Hkv][head_dim] of dtype at base + b*new_stride_b +
 *              s*new_stride_s + g*new_stride_h
 *   pool       int32 page ids (device, may be NULL); pool_count, status: one
 *              device int32 each
 * Requires dtype TT_BF16 or TT_F32, B >= 0, 1 <= S <= 64, Hkv >= 1,
 * head_dim >= 1 with head_dim * element size a multiple of 16 bytes,
 * page_size >= 1, num_pages >= 1, max_pages >= 1, B*max_pages below 2^30;
 * Kctx, Vctx, Knew, Vnew 16-byte aligned with strides that keep 16-byte
 * alignment (TT_ERR_UNSUPPORTED otherwise). The new rows must not overlap the
 * cache. Needs no workspace.
 */
typedef struct tt_kv_append_params {
    int32_t dtype;  /* tt_dtype of the caches and the new rows */
    int32_t B, S, Hkv, head_dim;
    void* Kctx;
    void* Vctx;
    int32_t page_size, num_pages, max_pages;
    int32_t* page_table;
    int32_t* ctx_len;
    const void* Knew;
    const void* Vnew;
    int64_t new_stride_b, new_stride_s, new_stride_h;
    const int32_t* pool;
    int32_t* pool_count;
    int32_t* status;
} tt_kv_append_params;

tt_status tt_kv_append(const tt_kv_append_params* p, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Masked negative log-likelihood L_MD (Eq. 4)
 * ------------------------------------------------------------------------ *
 * Section 2.2, Eq. (4): the denoiser is trained on the average negative
 * log-likelihood of the clean token over the masked positions (the 1/t
 * importance weight omitted). For each masked position (mask[b][l] != 0) with
 * clean token y = targets[b][l] and logits x of row (b, l):
 *   nll[b][l] = ln sum_v exp(x_v) - x_y            (softmax at temperature 1)
 *   *loss     = sum of nll over masked positions / their number (0 if none)
 *   *count    = the number of masked positions
 * Rows of unmasked positions are not read and their nll is not written. A
 * target outside [0, V) makes that row's nll (and the loss) NaN.
 *
 *   logits  [B][S][V] (dtype), row (b,l) at logits + (b*S + l)*logits_stride_row
 *   targets [B][S] int32;  mask [B][S] uint8, 1 = masked
 *   nll     [B][S] float32, optional;  loss: one device float32;  count: one
 *           device int32, optional
 * Requires B >= 0, S >= 1, V >= 1, logits_stride_row >= V, B*S below 2^31,
 * logits aligned to its element size. Rows need at least one finite logit.
 */
typedef struct tt_masked_nll_params {
    int32_t dtype; /* tt_dtype of logits */
    int32_t B, S, V;
    const void* logits;
    int64_t logits_stride_row;
    const int32_t* targets;
    const uint8_t* mask;
    float* nll;
    float* loss;
    int32_t* count;
} tt_masked_nll_params;

size_t tt_masked_nll_workspace_bytes(const tt_masked_nll_params* p);

tt_status tt_masked_nll(const tt_masked_nll_params* p, void* workspace, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TWOTOWER_ATTN_H */
