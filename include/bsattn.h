/*
 * libbsattn — content-aware block-sparse, head-masked self-attention for
 * AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Device buffers are allocated by the
 * caller; the library allocates no device memory and keeps no pointer to a
 * caller's buffer after a call returns.  The device state it holds is fixed
 * at load: the kernels' code objects and, per GPU, the static scratch array
 * of bsattn_select_no_alloc.  Every GPU call only enqueues work on
 * the caller's HIP stream (passed as `void*`, a hipStream_t; NULL = the null
 * stream) and never synchronises, except bsattn_mask_density, which is meant
 * to be called off the hot path.
 *
 * Errors: every function returns a bsattn_status.  Validation failures return
 * before anything is enqueued and leave every output untouched.  A failed
 * launch returns BSATTN_ERR_HIP.  Device faults surface at the caller's next
 * synchronisation.  Nothing is printed and nothing exits.
 *
 * Host state: a per-device table of the scratch array's address (filled on
 * first use, under a lock) and a per-device occupancy figure of the fp8
 * kernel; the stage objects are the caller's.  Calls are thread-safe except
 * that bsattn_select_no_alloc calls overlapping on one GPU share its
 * scratch.  Calls that share output buffers on one stream are ordered by the
 * stream; across streams the caller orders them.
 *
 * Sources, pages in the reference bundle:
 *  - SD.Next commit view, modules/attention/sparse: the selector paragraph,
 *    the layout paragraph, the radial-control paragraph, the synchronisation
 *    paragraph (three host syncs per call removed: ranking instead of a
 *    host-sized top-k, per-layout geometry, lazy density), the live-runs
 *    paragraph (text padded to 512, sequence to a multiple of 256, padding
 *    dropped) and the flex-consumer paragraph (only selected tiles computed).
 *  - haagenti_sparse crate docs and lib.rs: per-layer head masks (AttentionMask,
 *    MaskBuilder), DEFAULT_SPARSITY = 0.5 (fraction of heads skipped),
 *    MIN_ACTIVE_HEADS = 4, SparseError/Result as status codes.
 *  - inferensys glossary "Sparse Attention": sliding-window and block-sparse
 *    entries; the CSR-like per-row list of kept blocks.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (the crate's SparseError/Result convention as plain ints). */
typedef enum {
    BSATTN_OK = 0,
    BSATTN_ERR_NULL = 1,        /* a required pointer is NULL                          */
    BSATTN_ERR_DTYPE = 2,       /* unknown dtype, or q/k/v/out dtypes differ           */
    BSATTN_ERR_SHAPE = 3,       /* sizes inconsistent or outside the supported set     */
    BSATTN_ERR_STRIDE = 4,      /* negative/overlapping strides or misaligned pointers */
    BSATTN_ERR_LAYOUT = 5,      /* bad segment kind, lengths not summing to N, too many */
    BSATTN_ERR_BUDGET = 6,      /* budget/density NaN or <= 0; bad head-mask args      */
    BSATTN_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required             */
    BSATTN_ERR_HIP = 8,         /* a HIP runtime call or kernel launch failed          */
    BSATTN_ERR_UNSUPPORTED = 9  /* valid request the library has no kernel for         */
} bsattn_status;

/* Element types of q, k, v and out.  FP8_E4M3 (OCP e4m3: 1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, max 448, no infinities) is accepted only
 * by bsattn_quantize_fp8 (output) and bsattn_forward_fp8[_masked] (inputs). */
typedef enum { BSATTN_BF16 = 0, BSATTN_F32 = 1, BSATTN_FP8_E4M3 = 2 } bsattn_dtype;

/*
 * A device tensor viewed as [B][H][N][D].  Strides are in elements; the D
 * axis must be contiguous (stride 1).  `data` must be 16-byte aligned and
 * stride_n * element size must be a multiple of 16 bytes and below 32 MiB
 * (BSATTN_ERR_STRIDE otherwise).
 */
typedef struct {
    void* data;
    int32_t dtype;              /* bsattn_dtype */
    int64_t B, H, N, D;
    int64_t stride_b, stride_h, stride_n;
} bsattn_tensor;

/*
 * Token kinds of a packed sequence (SD.Next layout paragraph): image and
 * video tokens are sparsifiable; text, conditioning, audio and anything else
 * pin their block's rows and columns dense; padding blocks are dropped.
 */
typedef enum {
    BSATTN_SEG_TEXT = 0,
    BSATTN_SEG_CONDITIONING = 1,
    BSATTN_SEG_AUDIO = 2,
    BSATTN_SEG_OTHER = 3,
    BSATTN_SEG_IMAGE = 4,
    BSATTN_SEG_VIDEO = 5,
    BSATTN_SEG_PADDING = 6
} bsattn_seg_kind;

typedef struct {
    int32_t kind;               /* bsattn_seg_kind */
    int64_t length;             /* tokens, > 0 */
} bsattn_segment;

#define BSATTN_MAX_SEGMENTS 32

/*
 * Token layout, read during the call only (host memory).
 *  block         : tokens per block, 32 or 64.
 *  n_segments    : 0..BSATTN_MAX_SEGMENTS.  0 = no layout: every block is
 *                  sparsifiable (the whole sequence is sparsified).
 *  segments      : ordered segments whose lengths sum to N.
 *  window_tokens : 0 = none; otherwise a sliding window of total span W
 *                  tokens: a pair of sparsifiable blocks is always kept when
 *                  some query token and key token are at most W/2 apart.
 * A block is DROPPED when all its tokens are padding, SPARSE when all its
 * tokens lie in one image or video segment, PINNED otherwise (a block that
 * straddles a segment boundary pins).
 */
typedef struct {
    int32_t block;
    int32_t n_segments;
    const bsattn_segment* segments;
    int32_t window_tokens;
} bsattn_layout;

/*
 * Block mask in CSR-like form (glossary: CSR, row-wise).  Device buffers
 * owned by the caller:
 *   mask  uint8 [B][H][nqb][nkb]  1 = the (query block, key block) tile is kept
 *   count int32 [B][H][nqb]       kept tiles per query block
 *   index int32 [B][H][nqb][nkb]  kept key blocks in ascending order; only
 *                                 the first count entries are written/valid
 * B and H may be 1 to share one mask across batch entries or heads
 * (bsattn_radial writes a single layout-only mask that way).
 * is_dense and k are host out-fields, written synchronously by the call:
 *   k        candidates kept per sparsifiable row
 *   is_dense 1 when the budget covers every candidate (the layout-only mask
 *            is written instead of a scored one).
 */
typedef struct {
    int32_t B, H, nqb, nkb;
    uint8_t* mask;
    int32_t* count;
    int32_t* index;
    int32_t is_dense;
    int32_t k;
} bsattn_block_mask;

/* Human-readable name of a status code (static storage). */
const char* bsattn_status_string(bsattn_status st);

/*
 * Host-side geometry (SD.Next synchronisation paragraph: the parts that
 * depend only on the layout are computed on the host, so no device value is
 * ever read back).  classes[NB] receives 0 = SPARSE, 1 = PINNED,
 * 2 = DROPPED for NB = N / layout->block blocks; *n_cand the number of
 * SPARSE blocks.  No GPU needed.
 */
bsattn_status bsattn_layout_classes(const bsattn_layout* layout, int64_t N,
                                    uint8_t* classes, int32_t* n_cand);

/*
 * Budget rule (SD.Next selector paragraph: a fraction of the sparsifiable
 * candidates; a budget covering every candidate reports dense):
 *   k = max(1, min(n_cand, floor(budget * n_cand + 1e-9))),
 *   is_dense = (k >= n_cand); n_cand == 0 gives k = 0, is_dense = 1.
 * budget must be finite and > 0.  No GPU needed.
 */
bsattn_status bsattn_budget_k(int32_t n_cand, double budget, int32_t* k, int32_t* is_dense);

/*
 * Workspace bytes bsattn_select needs (device memory, 256-byte aligned): the
 * block sums of Q and K for the sparsifiable blocks, taken in float64 and
 * kept as float32 high and low parts, plus a norm bound per block.  An upper
 * bound that holds for every layout with these sizes.
 */
size_t bsattn_select_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                     int32_t block, int64_t D);

/*
 * Content-aware selection (SD.Next selector + layout paragraphs).
 *  q [B][H][N][D], k [B][Hkv][N][D] (Hkv divides H; query head h scores
 *  against kv head h / (H / Hkv), no key expansion), same dtype, D in
 *  {32, 64, 128}, N a multiple of layout->block.
 *  For every (b, h) and every SPARSE query block i: block sums of Q and K,
 *  unscaled scores S_ij = <sum Q_i, sum K_j> over SPARSE j (ranking equals
 *  that of mean-pooled scores), keep the diagonal plus the k-1 best other
 *  candidates (higher score first, ties to the lower block index), OR the
 *  sliding window, then apply pins and drops.  PINNED rows keep every
 *  non-dropped column; DROPPED rows and columns are empty.
 *  The kept set follows the exact scores: block sums are taken in float64;
 *  each row is ranked on float32 scores and kept as ranked only when the gap
 *  at the budget boundary exceeds a bound on their rounding error, otherwise
 *  the candidates near the boundary are ranked again by float64 scores.
 *  Only scores within about 2^-40 of each other (relative to the summed term
 *  magnitudes) can order differently from exact arithmetic.
 *  out: B == q->B, H == q->H, nqb == nkb == N / block; mask, count and index
 *  fully written.  out->k and out->is_dense are set before returning.
 *  When is_dense, no scoring runs and the layout-only mask is written.
 *  workspace: device, >= bsattn_select_workspace_bytes(...), 256-aligned.
 *  Limits: number of sparsifiable blocks <= 2048.
 *  Enqueues two kernels on `stream`; never synchronises.
 */
bsattn_status bsattn_select(const bsattn_tensor* q, const bsattn_tensor* k,
                            const bsattn_layout* layout, double budget,
                            bsattn_block_mask* out, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * bsattn_select under a per-layer head mask (haagenti_sparse crate docs: the
 * heads a layer's mask turns off are skipped, their output is zero).
 *  head_mask: device uint8 [H] (one byte per query head), or NULL for every
 *  head (then exactly bsattn_select).  The rows of every head with
 *  head_mask[h] != 0 are bit-identical to bsattn_select's; every row of a
 *  head with head_mask[h] == 0 is written empty (mask row all 0, count 0,
 *  index untouched), and that head's Q is not pooled, nor the K of a K/V
 *  head whose query heads are all masked.  bsattn_forward with the same
 *  head_mask gives the same output as after bsattn_select.
 *  Everything else (arguments, workspace, validation, errors, stream) as
 *  bsattn_select.  The head mask is read on the device, so a mask that
 *  changes between calls needs no host synchronisation.
 */
bsattn_status bsattn_select_heads(const bsattn_tensor* q, const bsattn_tensor* k,
                                  const bsattn_layout* layout, double budget,
                                  const uint8_t* head_mask, bsattn_block_mask* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsattn_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results, validation and errors as bsattn_select, without
 * the workspace: the pooled sums go to a static device array of
 * BSATTN_NO_ALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends.  The call allocates nothing (no hipMalloc, no hipFree);
 * its first use on a device looks up that device's address of the array.
 *  BSATTN_ERR_WORKSPACE when bsattn_select_workspace_bytes(...) for these
 *  sizes exceeds BSATTN_NO_ALLOC_SCRATCH_BYTES.
 * All calls on one GPU share the array and it keeps the last call's
 * contents: calls that overlap on one GPU (several streams, several host
 * threads) race and must be ordered by the caller.
 */
#define BSATTN_NO_ALLOC_SCRATCH_BYTES (32u << 20)
bsattn_status bsattn_select_no_alloc(const bsattn_tensor* q, const bsattn_tensor* k,
                                     const bsattn_layout* layout, double budget,
                                     bsattn_block_mask* out, void* stream);

/*
 * Radial control (SD.Next radial-control paragraph): every SPARSE row keeps
 * the k SPARSE candidates nearest the diagonal, ordered by (|i - j|, j), with
 * k from the same budget rule applied to `density`; same window, pins and
 * drops as bsattn_select.  N = out->nqb * layout->block.  The layout-only
 * result is written to every (b, h) slice of out (out->B, out->H >= 1; use 1
 * and 1 for one shared mask).  Enqueues one kernel; never synchronises.
 */
bsattn_status bsattn_radial(const bsattn_layout* layout, double density,
                            bsattn_block_mask* out, void* stream);

/*
 * Block-sparse attention forward (SD.Next flex-consumer paragraph; glossary
 * block-sparse entry; head masks from the haagenti_sparse crate).
 *  q, out [B][H][N][D]; k, v [B][Hkv][N][D]; same dtype.
 *  For each (b, h) with head_mask[h] != 0 and each query block i, the output
 *  rows equal softmax(scale * Q_i K^T + M) V where M is 0 on the key blocks
 *  listed in mask->index[b][h][i][0..count) and -inf elsewhere.  Rows with no
 *  kept block, and all rows of heads with head_mask[h] == 0, are written as 0.
 *  mask: nqb == nkb == N / block; mask->B in {1, B}, mask->H in {1, H};
 *        only count and index are read.  NULL = every block kept (dense).
 *  block: 64 when mask is NULL; otherwise N / mask->nqb, which must be 32
 *        or 64.
 *  head_mask: device uint8 [H], or NULL = every head active.
 *  scale: <= 0 means 1/sqrt(D).
 *  bf16 inputs use the bf16 MFMA path (block 64, D 64 or 128; K/V stride_n
 *  <= 2^24) with fp32 softmax and one final rounding to bf16; fp32 inputs,
 *  and bf16 of block 32 or D 32, use the fp32 MFMA path (scores, softmax, P
 *  and accumulation in fp32).  Enqueues one kernel; never synchronises.
 */
bsattn_status bsattn_forward(const bsattn_tensor* q, const bsattn_tensor* k,
                             const bsattn_tensor* v, const bsattn_block_mask* mask,
                             const uint8_t* head_mask, float scale,
                             bsattn_tensor* out, void* stream);

/* Selection and attention in one call: the result of bsattn_select(q, k,
 *  layout, budget, mask, ...) followed by bsattn_forward(q, k, v, mask,
 *  head_mask, scale, out, ...).  The selection is the one the SD.Next commit
 *  view of modules/attention/sparse computes (its selector paragraph:
 *  mean-pooled block scores, diagonal first, top budget share of the
 *  sparsifiable blocks) and the attention the block-sparse entry of the
 *  inferensys glossary describes (softmax over the kept blocks only).
 *  Arguments, layouts, ownership and errors are those of the two calls; mask
 *  is an output here (mask, count and index written, k and is_dense set) and
 *  is required.  workspace: bsattn_select_workspace_bytes(...) bytes,
 *  256-byte aligned.
 *  Where every block of the sequence is a candidate and a row fits one
 *  wavefront -- bf16, D 64, block 64, no layout segments, no window, at most
 *  64 blocks, a budget that keeps fewer than all of them, no head mask --
 *  two kernels run: the block pooling of K, then one attention kernel whose
 *  workgroups sum their own query block and rank their own rows from float64
 *  scores (resolved to 2^-17 relative: the same masks as bsattn_select
 *  except where two scores lie that close) and attend over the kept blocks;
 *  otherwise the two calls run as written.  Enqueues only; never
 *  synchronises.
 */
bsattn_status bsattn_select_forward(const bsattn_tensor* q, const bsattn_tensor* k,
                                    const bsattn_tensor* v, const bsattn_layout* layout,
                                    double budget, const uint8_t* head_mask, float scale,
                                    bsattn_tensor* out, bsattn_block_mask* mask,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * bsattn_forward with a per-token key mask composed with the block mask
 * (SD.Next sparse-stage paragraph: a backend declaring masked_block takes the
 * token attention mask and the block mask together).
 *  key_mask: device uint8, key_mask[b * key_mask_stride_b + j] for key token
 *        j of batch b; 0 masks the key (its logit is -inf in every row), any
 *        other value keeps it.  key_mask_stride_b >= N, or 0 for one mask
 *        shared by the batch.  NULL behaves exactly as bsattn_forward.
 *  A row whose kept keys are all masked is written as 0.  Everything else,
 *  including errors, as bsattn_forward; BSATTN_ERR_STRIDE when
 *  0 < key_mask_stride_b < N.  Caller owns the mask; it is read by the
 *  enqueued kernel only.
 */
bsattn_status bsattn_forward_masked(const bsattn_tensor* q, const bsattn_tensor* k,
                                    const bsattn_tensor* v, const bsattn_block_mask* mask,
                                    const uint8_t* head_mask, const uint8_t* key_mask,
                                    int64_t key_mask_stride_b, float scale,
                                    bsattn_tensor* out, void* stream);

/*
 * fp8 quantisation for the quantized consumer (SD.Next stage paragraph: a
 * quantized kernel joins as a block-mask consumer).  x: bf16 [B][H][N][D];
 * out: FP8_E4M3 with the same B, H, N, D (its own strides, in bytes).  Per
 * (b, h): scale[b * H + h] = max|x| / 448 (1 when the head is all zero), and
 * out = e4m3(clamp(x / scale, -448, 448)), rounded to nearest even, with the
 * division in fp32.  scale: device float[B * H]; ws: device scratch of at
 * least B * H * 4 bytes, 4-byte aligned.  Enqueues three kernels; never
 * synchronises.
 */
bsattn_status bsattn_quantize_fp8(const bsattn_tensor* x, bsattn_tensor* out, float* scale, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * Block-sparse attention on fp8 inputs (the quantized consumer).
 *  q [B][H][N][D], k, v [B][Hkv][N][D] of dtype FP8_E4M3 with real values
 *  code * q_scale[b * H + h] (k_scale, v_scale: [b * Hkv + kv head]; device
 *  float arrays); out bf16 [B][H][N][D].  Same block mask, head mask and
 *  scale rules as bsattn_forward (block 64, D 64 or 128).  P is rounded to
 *  e4m3 for the P V product, and the softmax denominators sum the same
 *  rounded values.  Enqueues one kernel; never synchronises.
 */
bsattn_status bsattn_forward_fp8(const bsattn_tensor* q, const bsattn_tensor* k, const bsattn_tensor* v,
                                 const float* q_scale, const float* k_scale, const float* v_scale,
                                 const bsattn_block_mask* mask, const uint8_t* head_mask, float scale,
                                 bsattn_tensor* out, void* stream);

/*
 * bsattn_forward_fp8 with a per-token key mask composed with the block mask
 * (SD.Next sparse-stage paragraph: the token attention mask and the block
 * mask go to the consumer together; here the quantized one).  key_mask and
 * key_mask_stride_b as in bsattn_forward_masked: device uint8,
 * key_mask[b * key_mask_stride_b + j], 0 masks key j; stride >= N or 0 for a
 * mask shared by the batch; NULL behaves exactly as bsattn_forward_fp8.  A
 * row whose kept keys are all masked is written as 0.  Errors as
 * bsattn_forward_fp8, plus BSATTN_ERR_STRIDE when 0 < key_mask_stride_b < N.
 */
bsattn_status bsattn_forward_fp8_masked(const bsattn_tensor* q, const bsattn_tensor* k, const bsattn_tensor* v,
                                        const float* q_scale, const float* k_scale, const float* v_scale,
                                        const bsattn_block_mask* mask, const uint8_t* head_mask,
                                        const uint8_t* key_mask, int64_t key_mask_stride_b, float scale,
                                        bsattn_tensor* out, void* stream);

/*
 * Per-layer head mask (haagenti_sparse AttentionMask / MaskBuilder with
 * DEFAULT_SPARSITY and MIN_ACTIVE_HEADS): skip floor(sparsity * H) heads but
 * keep at least min(H, min_active); the kept heads are those with the highest
 * importance, ties to the lower head index.  Host memory in and out
 * (importance double[H], out uint8[H]).  sparsity in [0, 1], min_active >= 0.
 * No GPU needed.
 */
bsattn_status bsattn_head_mask(const double* importance, int32_t H, double sparsity,
                               int32_t min_active, uint8_t* out);

/*
 * Lazy density (SD.Next synchronisation paragraph: density is read back only
 * when asked): kept tiles / (B * H * nqb * nkb).  Copies `count` to the host
 * and SYNCHRONISES `stream`; not for the hot path.
 */
bsattn_status bsattn_mask_density(const bsattn_block_mask* m, void* stream, double* density);

/* ------------------------------------------------------------------------
 * Host stage policy (SD.Next commit view, modules/attention/sparse: the
 * stage-gating, budget-schedule, minimum-length, exclusion-list, decline-log
 * and no-layout paragraphs).  Decides per attention call whether the sparse
 * stage serves it and at which budget; pure host code, no GPU.
 * ------------------------------------------------------------------------ */
typedef enum {
    BSATTN_STAGE_SPARSE = 0,          /* serve the call with select + forward      */
    BSATTN_DECLINE_DISABLED = 1,      /* the feature is switched off               */
    BSATTN_DECLINE_NO_BACKEND = 2,    /* no backend in the chain consumes a block
                                         mask: attention stays dense (warned)      */
    BSATTN_DECLINE_EXCLUDED = 3,      /* the model matched the exclusion list      */
    BSATTN_DECLINE_NOT_SELF = 4,      /* not self attention (role, or query and
                                         key lengths differ)                       */
    BSATTN_DECLINE_SHORT = 5,         /* sequence shorter than the minimum length  */
    BSATTN_DECLINE_CAUSAL = 6,        /* the call carries a causal flag            */
    BSATTN_DECLINE_TOKEN_MASK = 7     /* a token mask and no backend that composes
                                         it with a block mask (masked_block)       */
} bsattn_stage_outcome;

typedef enum {
    BSATTN_NOTE_NONE = 0,
    BSATTN_NOTE_NO_LAYOUT = 1         /* served, but no token layout was published:
                                         the whole sequence is sparsified          */
} bsattn_stage_note;

#define BSATTN_DEFAULT_MIN_LENGTH 8192   /* the measured dense/sparse crossover    */

typedef struct {
    int32_t enabled;
    int64_t min_length;       /* tokens; 0 = no floor; negative values are reserved
                                 (a derived floor) and rejected                    */
    int32_t n_steps;          /* length of the per-step budget schedule, >= 1       */
    double budget_first;      /* budget of steps [0, switch_step)                  */
    double budget_later;      /* budget of steps >= switch_step (the schedule has at
                                 most these two distinct values)                   */
    int32_t switch_step;      /* 0..n_steps; n_steps = one value throughout         */
    const char* exclude;      /* comma-separated names, matched case-insensitively
                                 against the architecture, the pipeline class and
                                 the denoiser class; NULL or "" = none.  Copied.    */
    int32_t backend_block_mask;   /* an active backend consumes block masks        */
    int32_t backend_masked_block; /* ... and takes a token mask with the block mask */
} bsattn_stage_config;

typedef struct {
    const char* architecture; /* model names (any may be NULL); the exclusion      */
    const char* pipeline;     /* result is resolved once per distinct triple        */
    const char* denoiser;
    int32_t self_attention;   /* the component role is self attention               */
    int64_t q_len, kv_len;    /* tokens                                             */
    int32_t has_token_mask;
    int32_t causal;
    int32_t step;             /* denoising step, >= 0; steps past n_steps use the
                                 last value of the schedule                         */
    int32_t has_layout;       /* the pipeline published a token layout              */
} bsattn_stage_call;

typedef struct {
    int32_t outcome;          /* bsattn_stage_outcome                               */
    int32_t note;             /* bsattn_stage_note                                  */
    double budget;            /* this step's budget (outcome SPARSE), else 0        */
    int32_t use_key_mask;     /* pass the call's token mask to bsattn_forward_masked */
    int32_t first_report;     /* 1 when this (outcome, note, length) is reported for
                                 the first time by this stage object: the caller
                                 logs it once, then stays quiet                     */
} bsattn_stage_decision;

typedef struct bsattn_stage bsattn_stage;   /* opaque host object */

/* Validates the configuration and creates a stage object (host memory, owned
 * by the caller until bsattn_stage_destroy).  BSATTN_ERR_BUDGET for a budget
 * outside (0, inf) or NaN, a negative minimum length or a schedule whose
 * switch step is outside [0, n_steps]; BSATTN_ERR_NULL for NULL pointers. */
bsattn_status bsattn_stage_create(const bsattn_stage_config* cfg, bsattn_stage** out);

/* Decides one call.  Thread-safe (an internal lock guards the report memory
 * and the exclusion cache).  BSATTN_ERR_SHAPE for negative lengths or step. */
bsattn_status bsattn_stage_decide(bsattn_stage* stage, const bsattn_stage_call* call,
                                  bsattn_stage_decision* out);

void bsattn_stage_destroy(bsattn_stage* stage);

/* Short human-readable reason for an outcome (static storage). */
const char* bsattn_stage_outcome_string(int32_t outcome);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
