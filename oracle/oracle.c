/*
 * CPU oracle for content-aware block-sparse, head-masked self-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the bench's CPU-baseline leg may load it.  It shares no code,
 * header, constant or helper with the GPU library and the GPU library never
 * calls it.
 *
 * Everything is computed in double precision from the exact values the GPU
 * sees (bf16 or fp32 inputs upcast without rounding).  Loops follow the
 * definitions one step at a time; there is no tiling, no online softmax, no
 * pooling shortcut and no compaction.
 *
 * Sources (pages in the reference bundle):
 *  [SDN]  SD.Next commit view, modules/attention/sparse: the selector paragraph
 *         (tile mean-pooling, unscaled tile-pair scores, per-row budget over the
 *         sparsifiable candidates, diagonal kept, full budget reports dense), the
 *         layout paragraph (sparsifiable vs pinned vs dropped token kinds,
 *         straddling tile pins), the radial-control paragraph (band around the
 *         diagonal at the selector's density, honouring the layout pins), and
 *         the flex-consumer paragraph (only selected tiles are computed; output
 *         must equal sdpa fed the same tiles).
 *  [HAA]  haagenti_sparse crate docs and lib.rs source: per-layer head masks
 *         skip whole heads; the constants DEFAULT_SPARSITY (fraction of heads
 *         skipped) and MIN_ACTIVE_HEADS (floor on active heads per layer).
 *  [GLO]  inferensys glossary "Sparse Attention": the sliding-window entry
 *         (window around the query position) and the block-sparse entry
 *         (grid of blocks, only connected blocks computed).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes with its reason):
 *  - k = max(1, min(n_cand, floor(budget * n_cand + 1e-9))), is_dense when
 *    k >= n_cand; the forced diagonal counts inside k.
 *  - Ties between equal scores go to the lower key-block index.
 *  - A row is a near tie when the last kept and first dropped non-diagonal
 *    scores differ by at most 1e-4 of the larger magnitude.
 *  - Window W (tokens): blocks i, j are connected when some query token of i
 *    and key token of j are at most W/2 apart.
 *  - Radial: the k candidates nearest the diagonal, ordered by (|i-j|, j).
 *  - Padding query rows are dropped too; empty rows and masked heads give 0.
 *  - Head mask: skip floor(sparsity*H) heads but keep at least min_active,
 *    keeping the most important heads, ties to the lower head index.
 *
 * Parity pins: every function here is checked by the CPU tests against
 * brute force, closed forms, library routines (float64 sdpa) or values
 * printed in the pages.  One reading stays partly unpinned: how a fractional
 * budget rounds to k (floor here).  The pages print no k for any layout, so
 * beyond the cases where every rounding agrees (8 candidates at 0.5, budget
 * 1.0) the floor is "parity unpinned"; the GPU library follows the same
 * reading, and the tests pin its properties (never above the budget, at
 * least 1, full budget reports dense).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Token kinds, the oracle's own numbering (the Python wrapper maps names). */
enum { ORC_TEXT = 0, ORC_CONDITIONING = 1, ORC_AUDIO = 2, ORC_OTHER = 3,
       ORC_IMAGE = 4, ORC_VIDEO = 5, ORC_PADDING = 6 };
/* Block classes. */
enum { ORC_SPARSE = 0, ORC_PINNED = 1, ORC_DROPPED = 2 };

/* ------------------------------------------------------------------------ */
/* Layout classes [SDN layout paragraph].                                     */
/* A block is DROPPED when all its tokens are padding, SPARSE when all its    */
/* tokens lie inside one image or video segment, PINNED otherwise (text,      */
/* conditioning, audio, unrecognised kinds, and any block that straddles a    */
/* segment boundary).  Without a layout every block is SPARSE.                */
/* Returns 0 on success, -1 if the segment lengths do not sum to N.           */
/* ------------------------------------------------------------------------ */
int orc_block_classes(int n_seg, const int32_t* kind, const int64_t* length,
                      int64_t N, int32_t block, uint8_t* cls)
{
    int64_t NB = N / block;
    if (n_seg == 0) {
        for (int64_t b = 0; b < NB; ++b) cls[b] = ORC_SPARSE;
        return 0;
    }
    int64_t total = 0;
    for (int s = 0; s < n_seg; ++s) total += length[s];
    if (total != N) return -1;

    for (int64_t b = 0; b < NB; ++b) {
        int all_padding = 1;
        int first_seg = -1, one_segment = 1, all_sparsifiable = 1;
        for (int64_t t = b * block; t < (b + 1) * block; ++t) {
            /* find the segment holding token t by walking the segments */
            int s = 0;
            int64_t start = 0;
            while (t >= start + length[s]) { start += length[s]; ++s; }
            int kd = kind[s];
            if (kd != ORC_PADDING) all_padding = 0;
            if (kd != ORC_IMAGE && kd != ORC_VIDEO) all_sparsifiable = 0;
            if (first_seg < 0) first_seg = s;
            else if (s != first_seg) one_segment = 0;
        }
        if (all_padding) cls[b] = ORC_DROPPED;
        else if (one_segment && all_sparsifiable) cls[b] = ORC_SPARSE;
        else cls[b] = ORC_PINNED;
    }
    return 0;
}

/* Budget -> number of kept candidates per row [SDN selector paragraph]. */
void orc_budget(int64_t n_cand, double budget, int64_t* k_out, int32_t* is_dense_out)
{
    if (n_cand <= 0) { *k_out = 0; *is_dense_out = 1; return; }
    double x = floor(budget * (double)n_cand + 1e-9);
    int64_t k = (x >= (double)n_cand) ? n_cand : (int64_t)x;
    if (k < 1) k = 1;
    *k_out = k;
    *is_dense_out = (k >= n_cand) ? 1 : 0;
}

/* Sliding window [GLO sliding-window entry]: some token of block i and some */
/* token of block j are at most W/2 apart, i.e. 2*min|t-s| <= W.             */
static int window_connects(int64_t i, int64_t j, int32_t block, int32_t window_tokens)
{
    if (window_tokens <= 0) return 0;
    int64_t d = i > j ? i - j : j - i;
    int64_t min_token_gap = (d == 0) ? 0 : (d - 1) * block + 1;
    return 2 * min_token_gap <= (int64_t)window_tokens;
}

/* Final mask entry from classes and the per-pair choice [SDN layout]. */
static uint8_t pin_or_drop(uint8_t ci, uint8_t cj, uint8_t chosen)
{
    if (ci == ORC_DROPPED || cj == ORC_DROPPED) return 0;
    if (ci == ORC_PINNED || cj == ORC_PINNED) return 1;
    return chosen;
}

typedef struct { double score; int64_t j; } cand_t;

/* Order: higher score first, then lower block index. */
static int cand_cmp(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Content-aware selection [SDN selector + layout paragraphs].               */
/* q: [B][H][N][D], k: [B][Hkv][N][D], doubles.  cls: [NB] from               */
/* orc_block_classes.  Writes mask [B][H][NB][NB] (0/1) and near_tie          */
/* [B][H][NB] (1 where the kept set rests on a near tie, SPARSE rows only).  */
/* ------------------------------------------------------------------------ */
int orc_select(const double* q, const double* k, int64_t B, int64_t H, int64_t Hkv,
               int64_t N, int64_t D, int32_t block, const uint8_t* cls,
               double budget, int32_t window_tokens, uint8_t* mask, uint8_t* near_tie)
{
    if (Hkv <= 0 || H % Hkv != 0 || N % block != 0) return -1;
    const int64_t NB = N / block;
    int64_t n_cand = 0;
    for (int64_t b = 0; b < NB; ++b) n_cand += (cls[b] == ORC_SPARSE);
    int64_t kkeep; int32_t is_dense;
    orc_budget(n_cand, budget, &kkeep, &is_dense);

    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t bb = 0; bb < B; ++bb)
    for (int64_t h = 0; h < H; ++h) {
        const int64_t g = h / (H / Hkv);   /* query heads score against their kv head */
        const double* qh = q + (bb * H + h) * N * D;
        const double* kh = k + (bb * Hkv + g) * N * D;
        uint8_t* mh = mask + (bb * H + h) * NB * NB;
        uint8_t* th = near_tie + (bb * H + h) * NB;

        /* step 1: mean-pool every block of Q and K */
        double* qp = (double*)calloc((size_t)(NB * D), sizeof(double));
        double* kp = (double*)calloc((size_t)(NB * D), sizeof(double));
        cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(NB > 0 ? NB : 1));
        uint8_t* chosen = (uint8_t*)malloc((size_t)(NB > 0 ? NB : 1));
        for (int64_t i = 0; i < NB; ++i)
            for (int64_t d = 0; d < D; ++d) {
                double sq = 0.0, sk = 0.0;
                for (int64_t t = i * block; t < (i + 1) * block; ++t) {
                    sq += qh[t * D + d];
                    sk += kh[t * D + d];
                }
                qp[i * D + d] = sq / block;
                kp[i * D + d] = sk / block;
            }

        for (int64_t i = 0; i < NB; ++i) {
            th[i] = 0;
            for (int64_t j = 0; j < NB; ++j) chosen[j] = 0;
            if (cls[i] == ORC_SPARSE) {
                /* step 2: unscaled scores of the other sparse candidates */
                int64_t nc = 0;
                for (int64_t j = 0; j < NB; ++j) {
                    if (cls[j] != ORC_SPARSE || j == i) continue;
                    double s = 0.0;
                    for (int64_t d = 0; d < D; ++d) s += qp[i * D + d] * kp[j * D + d];
                    cand[nc].score = s;
                    cand[nc].j = j;
                    ++nc;
                }
                /* step 3: the diagonal first, then by score; keep k in total */
                qsort(cand, (size_t)nc, sizeof(cand_t), cand_cmp);
                chosen[i] = 1;
                for (int64_t r = 0; r < kkeep - 1 && r < nc; ++r) chosen[cand[r].j] = 1;
                /* near tie between the last kept and the first dropped */
                if (kkeep >= 2 && kkeep < n_cand) {
                    double a = cand[kkeep - 2].score, bsc = cand[kkeep - 1].score;
                    double mag = fabs(a) > fabs(bsc) ? fabs(a) : fabs(bsc);
                    if (fabs(a - bsc) <= 1e-4 * mag) th[i] = 1;
                }
                /* step 4: the sliding window is kept on top of the selection */
                for (int64_t j = 0; j < NB; ++j)
                    if (cls[j] == ORC_SPARSE && window_connects(i, j, block, window_tokens))
                        chosen[j] = 1;
            }
            /* step 5: pins and drops */
            for (int64_t j = 0; j < NB; ++j)
                mh[i * NB + j] = pin_or_drop(cls[i], cls[j], chosen[j]);
        }
        free(qp); free(kp); free(cand); free(chosen);
    }
    return 0;
}

typedef struct { int64_t dist; int64_t j; } near_t;

static int near_cmp(const void* a, const void* b)
{
    const near_t* x = (const near_t*)a;
    const near_t* y = (const near_t*)b;
    if (x->dist != y->dist) return x->dist < y->dist ? -1 : 1;
    return (x->j < y->j) ? -1 : (x->j > y->j) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Radial control [SDN radial-control paragraph]: every sparse row keeps the */
/* k sparse candidates nearest the diagonal by (|i-j|, j), k from the same   */
/* budget rule as the selector; same window and pins.  mask: [NB][NB].       */
/* ------------------------------------------------------------------------ */
int orc_radial(int64_t NB, int32_t block, const uint8_t* cls, double density,
               int32_t window_tokens, uint8_t* mask)
{
    int64_t n_cand = 0;
    for (int64_t b = 0; b < NB; ++b) n_cand += (cls[b] == ORC_SPARSE);
    int64_t kkeep; int32_t is_dense;
    orc_budget(n_cand, density, &kkeep, &is_dense);
    near_t* cand = (near_t*)malloc(sizeof(near_t) * (size_t)(NB > 0 ? NB : 1));
    uint8_t* chosen = (uint8_t*)malloc((size_t)(NB > 0 ? NB : 1));
    for (int64_t i = 0; i < NB; ++i) {
        for (int64_t j = 0; j < NB; ++j) chosen[j] = 0;
        if (cls[i] == ORC_SPARSE) {
            int64_t nc = 0;
            for (int64_t j = 0; j < NB; ++j) {
                if (cls[j] != ORC_SPARSE) continue;
                cand[nc].dist = i > j ? i - j : j - i;
                cand[nc].j = j;
                ++nc;
            }
            qsort(cand, (size_t)nc, sizeof(near_t), near_cmp);
            for (int64_t r = 0; r < kkeep && r < nc; ++r) chosen[cand[r].j] = 1;
            for (int64_t j = 0; j < NB; ++j)
                if (cls[j] == ORC_SPARSE && window_connects(i, j, block, window_tokens))
                    chosen[j] = 1;
        }
        for (int64_t j = 0; j < NB; ++j)
            mask[i * NB + j] = pin_or_drop(cls[i], cls[j], chosen[j]);
    }
    free(cand); free(chosen);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention under an explicit -inf block mask [SDN flex-consumer paragraph, */
/* GLO block-sparse entry; head mask from HAA].                              */
/* q: [B][H][N][D], k, v: [B][Hkv][N][D].  mask: [mB][mH][NB][NB] with       */
/* mB in {1,B} and mH in {1,H} (1 = shared by all).  head_mask: [H] or NULL  */
/* (all active).  Computes the R query rows named by (rb, rh, rt) into       */
/* out [R][D].  Each row: logits scale*q.k_j over all N keys, -inf where the */
/* key's block is not kept, softmax with max subtraction, then the weighted  */
/* sum of V.  A row whose logits are all -inf, and every row of a masked     */
/* head, is exactly 0.                                                       */
/* key_mask: [B][N] per-token key mask or NULL [SDN sparse-stage paragraph:  */
/* a backend declaring masked_block takes the token attention mask and the   */
/* block mask together]; key j of batch b is -inf as well where it is 0.     */
/* ------------------------------------------------------------------------ */
int orc_attention_rows(const double* q, const double* k, const double* v,
                       int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D,
                       int32_t block, const uint8_t* mask, int64_t mB, int64_t mH,
                       const uint8_t* head_mask, double scale,
                       int64_t R, const int64_t* rb, const int64_t* rh, const int64_t* rt,
                       double* out, const uint8_t* key_mask)
{
    if (Hkv <= 0 || H % Hkv != 0 || N % block != 0) return -1;
    if (!(mB == 1 || mB == B) || !(mH == 1 || mH == H)) return -1;
    const int64_t NB = N / block;

    #pragma omp parallel
    {
        double* logit = (double*)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < R; ++r) {
            const int64_t bb = rb[r], h = rh[r], t = rt[r];
            double* o = out + r * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            if (head_mask && head_mask[h] == 0) continue;
            const int64_t g = h / (H / Hkv);
            const double* qt = q + ((bb * H + h) * N + t) * D;
            const double* kh = k + (bb * Hkv + g) * N * D;
            const double* vh = v + (bb * Hkv + g) * N * D;
            const uint8_t* mrow = mask + (((mB == 1 ? 0 : bb) * mH + (mH == 1 ? 0 : h)) * NB + t / block) * NB;

            double m = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                if (!mrow[j / block]) { logit[j] = -INFINITY; continue; }
                if (key_mask && !key_mask[bb * N + j]) { logit[j] = -INFINITY; continue; }
                double s = 0.0;
                for (int64_t d = 0; d < D; ++d) s += qt[d] * kh[j * D + d];
                logit[j] = scale * s;
                if (logit[j] > m) m = logit[j];
            }
            if (m == -INFINITY) continue;           /* empty row: output 0 */
            double denom = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                double p = (logit[j] == -INFINITY) ? 0.0 : exp(logit[j] - m);
                logit[j] = p;
                denom += p;
            }
            for (int64_t j = 0; j < N; ++j) {
                if (logit[j] == 0.0) continue;
                double w = logit[j] / denom;
                for (int64_t d = 0; d < D; ++d) o[d] += w * vh[j * D + d];
            }
        }
        free(logit);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-layer head mask [HAA: AttentionMask / MaskBuilder, DEFAULT_SPARSITY,  */
/* MIN_ACTIVE_HEADS]: skip floor(sparsity*H) heads, keep at least            */
/* min_active (capped at H), keeping the most important heads with ties to   */
/* the lower head index.  out: [H] 0/1.                                      */
/* ------------------------------------------------------------------------ */
typedef struct { double imp; int64_t h; } head_t;

static int head_cmp(const void* a, const void* b)
{
    const head_t* x = (const head_t*)a;
    const head_t* y = (const head_t*)b;
    if (x->imp > y->imp) return -1;
    if (x->imp < y->imp) return 1;
    return (x->h < y->h) ? -1 : (x->h > y->h) ? 1 : 0;
}

int orc_head_mask(const double* importance, int64_t H, double sparsity,
                  int64_t min_active, uint8_t* out)
{
    if (H <= 0) return -1;
    int64_t skip = (int64_t)floor(sparsity * (double)H);
    int64_t n_act = H - skip;
    if (n_act < min_active) n_act = min_active;
    if (n_act > H) n_act = H;
    head_t* hs = (head_t*)malloc(sizeof(head_t) * (size_t)H);
    for (int64_t h = 0; h < H; ++h) { hs[h].imp = importance[h]; hs[h].h = h; out[h] = 0; }
    qsort(hs, (size_t)H, sizeof(head_t), head_cmp);
    for (int64_t r = 0; r < n_act; ++r) out[hs[r].h] = 1;
    free(hs);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 8-bit float E4M3 for the quantized consumer [SDN stage paragraph: a      */
/* quantized kernel joins as a block-mask consumer].  The pages name no     */
/* format; the reading taken is the OCP E4M3 encoding: sign bit, 4 exponent */
/* bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals     */
/* m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; there is no infinity,    */
/* the largest finite value is 448.                                         */
/* ------------------------------------------------------------------------ */
double orc_e4m3_decode(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest finite E4M3 value to x (a float, compared exactly in double);    */
/* halfway cases go to the even code (mantissa bit 0 clear).  |x| > 448     */
/* saturates to 448.  The sign of x is kept (so -0 and tiny negatives give   */
/* the negative zero code 0x80).                                            */
uint8_t orc_e4m3_encode(float x)
{
    const double ax = fabs((double)x);
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7e; ++c) {           /* every non-negative finite code */
        const double d = fabs(orc_e4m3_decode((uint8_t)c) - ax);
        if (d < bestd || (d == bestd && (c & 1) == 0)) { best = c; bestd = d; }
    }
    return (uint8_t)(sign | best);
}

void orc_e4m3_decode_array(const uint8_t* c, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

/* Per-(b, head) quantisation of x [B][H][N][D] (exact bf16 values given in */
/* double): scale = max|x| / 448 in float (1 when the head is all zero),    */
/* code = encode(clamp(x / scale, -448, 448)) with the division in float.   */
int orc_quantize_e4m3(const double* x, int64_t B, int64_t H, int64_t N, int64_t D,
                      uint8_t* out, float* scale)
{
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double* xh = x + bh * N * D;
        float amax = 0.0f;
        for (int64_t i = 0; i < N * D; ++i) {
            const float a = fabsf((float)xh[i]);
            if (a > amax) amax = a;
        }
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        scale[bh] = sc;
        for (int64_t i = 0; i < N * D; ++i) {
            float v = (float)xh[i] / sc;
            if (v > 448.0f) v = 448.0f;
            if (v < -448.0f) v = -448.0f;
            out[bh * N * D + i] = orc_e4m3_encode(v);
        }
    }
    return 0;
}

/* Threads the OpenMP loops above use (reported with CPU timings). */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
