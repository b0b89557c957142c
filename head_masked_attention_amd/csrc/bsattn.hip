// C-ABI layer of libbsattn: validation, host geometry and launches.
//
// Everything that depends only on the layout (block classes, candidate
// count, k, is_dense, window width) is host arithmetic, so no call ever reads
// a device value back (SD.Next commit view, modules/attention/sparse,
// synchronisation paragraph).  Validation returns before any HIP call.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/bsattn.h"
#include "common.h"
#include "internal.h"

using namespace bsattn;

namespace {

size_t elem_size(int32_t dtype) { return dtype == BSATTN_F32 ? 4 : dtype == BSATTN_FP8_E4M3 ? 1 : 2; }

bool dtype_ok(int32_t dtype) { return dtype == BSATTN_BF16 || dtype == BSATTN_F32; }

// A [B][H][N][D] view: D contiguous, supported D, 16-byte aligned rows.
// fp8: accept only FP8_E4M3 (the fp8 entry points), else bf16 / fp32.
bsattn_status check_tensor(const bsattn_tensor* t, bool fp8 = false) {
    if (t == nullptr || t->data == nullptr) return BSATTN_ERR_NULL;
    if (fp8 ? t->dtype != BSATTN_FP8_E4M3 : !dtype_ok(t->dtype)) return BSATTN_ERR_DTYPE;
    if (t->B <= 0 || t->H <= 0 || t->N <= 0 || t->D <= 0) return BSATTN_ERR_SHAPE;
    if (t->D != 32 && t->D != 64 && t->D != 128) return BSATTN_ERR_SHAPE;
    if (t->B > INT32_MAX || t->H > INT32_MAX || t->N > INT32_MAX) return BSATTN_ERR_SHAPE;
    if (t->stride_b <= 0 || t->stride_h <= 0 || t->stride_n < t->D) return BSATTN_ERR_STRIDE;
    const size_t es = elem_size(t->dtype);
    if (((uintptr_t)t->data) % 16 != 0) return BSATTN_ERR_STRIDE;
    if ((t->stride_b * es) % 16 || (t->stride_h * es) % 16 || (t->stride_n * es) % 16)
        return BSATTN_ERR_STRIDE;
    // stage tiles are addressed as a base plus 32-bit lane offsets spanning up
    // to 64 rows: row pitch below 32 MiB
    if (t->stride_n * (int64_t)es >= (int64_t(1) << 25)) return BSATTN_ERR_STRIDE;
    return BSATTN_OK;
}

TView view_of(const bsattn_tensor* t) {
    return TView{t->data, t->stride_b, t->stride_h, t->stride_n};
}

bool budget_ok(double x) { return std::isfinite(x) && x > 0.0; }

// Block classes from ordered segments: a block is DROPPED when every segment
// it overlaps is padding, SPARSE when it lies inside one image/video segment,
// PINNED otherwise.  Calls f(block, class) for every block in order (no heap
// allocation).  Returns false on a malformed layout, before any call of f.
template <typename F>
bool for_each_block_class(const bsattn_layout* lay, int64_t N, F f) {
    const int64_t block = lay->block;
    const int64_t nb = N / block;
    if (lay->n_segments == 0) {
        for (int64_t b = 0; b < nb; ++b) f(b, (int32_t)CLS_SPARSE);
        return true;
    }
    int64_t total = 0;
    for (int s = 0; s < lay->n_segments; ++s) {
        const bsattn_segment& sg = lay->segments[s];
        if (sg.length <= 0 || sg.kind < BSATTN_SEG_TEXT || sg.kind > BSATTN_SEG_PADDING) return false;
        total += sg.length;
    }
    if (total != N) return false;
    int s = 0;
    int64_t seg_start = 0;
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * block, hi = lo + block;   // [lo, hi)
        while (seg_start + lay->segments[s].length <= lo) { seg_start += lay->segments[s].length; ++s; }
        bool all_pad = true, single = true, sparsifiable = true;
        int64_t st = seg_start;
        for (int u = s; u < lay->n_segments && st < hi; st += lay->segments[u].length, ++u) {
            const int32_t kd = lay->segments[u].kind;
            if (kd != BSATTN_SEG_PADDING) all_pad = false;
            if (kd != BSATTN_SEG_IMAGE && kd != BSATTN_SEG_VIDEO) sparsifiable = false;
            if (u != s) single = false;
        }
        f(b, (int32_t)(all_pad ? CLS_DROPPED : (single && sparsifiable) ? CLS_SPARSE : CLS_PINNED));
    }
    return true;
}

void budget_rule(int32_t n_cand, double budget, int32_t* k, int32_t* is_dense) {
    if (n_cand <= 0) { *k = 0; *is_dense = 1; return; }
    const double x = std::floor(budget * (double)n_cand + 1e-9);
    int32_t kk = x >= (double)n_cand ? n_cand : (int32_t)x;
    if (kk < 1) kk = 1;
    *k = kk;
    *is_dense = kk >= n_cand ? 1 : 0;
}

// Window half-width in blocks: the largest d with a token pair of blocks d
// apart within W/2, i.e. 2 * ((d - 1) * block + 1) <= W.
int32_t window_blocks(int32_t W, int32_t block) {
    if (W <= 0) return -1;
    if (W < 2) return 0;
    return (W - 2) / (2 * block) + 1;
}

bsattn_status check_layout(const bsattn_layout* lay) {
    if (lay == nullptr) return BSATTN_ERR_NULL;
    if (lay->block != 32 && lay->block != 64) return BSATTN_ERR_SHAPE;
    if (lay->n_segments < 0 || lay->n_segments > BSATTN_MAX_SEGMENTS) return BSATTN_ERR_LAYOUT;
    if (lay->n_segments > 0 && lay->segments == nullptr) return BSATTN_ERR_NULL;
    if (lay->window_tokens < 0) return BSATTN_ERR_LAYOUT;
    return BSATTN_OK;
}

bsattn_status make_geometry(const bsattn_layout* lay, int64_t N, double budget, Geometry& g) {
    std::memset(&g, 0, sizeof g);
    g.nb = (int32_t)(N / lay->block);
    g.block = lay->block;
    // run-length classes, built while the classes are computed
    int32_t n_sparse = 0, n_other = 0, runs = 0;
    bool too_many = false;
    const bool ok = for_each_block_class(lay, N, [&](int64_t b, int32_t cls) {
        if (runs > 0 && g.run_cls[runs - 1] == cls) { ++g.run_len[runs - 1]; }
        else if (runs == kMaxRuns) { too_many = true; return; }
        else {
            g.run_first[runs] = (int32_t)b;
            g.run_len[runs] = 1;
            g.run_cls[runs] = cls;
            g.run_off[runs] = cls == CLS_SPARSE ? n_sparse : n_other;
            ++runs;
        }
        if (cls == CLS_SPARSE) ++n_sparse; else ++n_other;
    });
    if (!ok || too_many) return BSATTN_ERR_LAYOUT;
    g.n_runs = runs;
    g.n_cand = n_sparse;
    g.n_other = n_other;
    budget_rule(n_sparse, budget, &g.k, &g.is_dense);
    g.w = window_blocks(lay->window_tokens, lay->block);
    return BSATTN_OK;
}

bsattn_status check_mask_out(const bsattn_block_mask* m) {
    if (m == nullptr || m->mask == nullptr || m->count == nullptr || m->index == nullptr)
        return BSATTN_ERR_NULL;
    if (m->B <= 0 || m->H <= 0 || m->nqb <= 0 || m->nqb != m->nkb) return BSATTN_ERR_SHAPE;
    return BSATTN_OK;
}

}  // namespace

extern "C" {

const char* bsattn_status_string(bsattn_status st) {
    switch (st) {
        case BSATTN_OK: return "ok";
        case BSATTN_ERR_NULL: return "required pointer is NULL";
        case BSATTN_ERR_DTYPE: return "unsupported or mismatched dtype";
        case BSATTN_ERR_SHAPE: return "inconsistent or unsupported shape";
        case BSATTN_ERR_STRIDE: return "bad stride or misaligned pointer";
        case BSATTN_ERR_LAYOUT: return "malformed token layout";
        case BSATTN_ERR_BUDGET: return "budget/density or head-mask arguments out of range";
        case BSATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case BSATTN_ERR_HIP: return "HIP runtime error";
        case BSATTN_ERR_UNSUPPORTED: return "no kernel for this configuration";
    }
    return "unknown status";
}

bsattn_status bsattn_layout_classes(const bsattn_layout* layout, int64_t N, uint8_t* classes,
                                    int32_t* n_cand) {
    bsattn_status st = check_layout(layout);
    if (st != BSATTN_OK) return st;
    if (classes == nullptr || n_cand == nullptr) return BSATTN_ERR_NULL;
    if (N <= 0 || N % layout->block != 0 || N / layout->block > INT32_MAX) return BSATTN_ERR_SHAPE;
    int32_t nc = 0;
    if (!for_each_block_class(layout, N, [&](int64_t b, int32_t cls) {
            classes[b] = (uint8_t)cls;
            nc += cls == CLS_SPARSE;
        }))
        return BSATTN_ERR_LAYOUT;
    *n_cand = nc;
    return BSATTN_OK;
}

bsattn_status bsattn_budget_k(int32_t n_cand, double budget, int32_t* k, int32_t* is_dense) {
    if (k == nullptr || is_dense == nullptr) return BSATTN_ERR_NULL;
    if (n_cand < 0) return BSATTN_ERR_SHAPE;
    if (!budget_ok(budget)) return BSATTN_ERR_BUDGET;
    budget_rule(n_cand, budget, k, is_dense);
    return BSATTN_OK;
}

size_t bsattn_select_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int32_t block,
                                     int64_t D) {
    if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || D <= 0 || (block != 32 && block != 64)) return 0;
    // >= the pooled rows of any layout of this length
    return pool_space(B, H, Hkv, pooled_rows(N / block), D).bytes;
}

}  // extern "C"

namespace {
// Validation and geometry of a selection call (no HIP call).
bsattn_status select_validate(const bsattn_tensor* q, const bsattn_tensor* k, const bsattn_layout* layout,
                              double budget, const bsattn_block_mask* out, Geometry& g) {
    bsattn_status st;
    if ((st = check_tensor(q)) != BSATTN_OK) return st;
    if ((st = check_tensor(k)) != BSATTN_OK) return st;
    if ((st = check_layout(layout)) != BSATTN_OK) return st;
    if (out == nullptr) return BSATTN_ERR_NULL;
    if ((st = check_mask_out(out)) != BSATTN_OK) return st;
    if (q->dtype != k->dtype) return BSATTN_ERR_DTYPE;
    if (q->B != k->B || q->N != k->N || q->D != k->D) return BSATTN_ERR_SHAPE;
    if (q->H % k->H != 0) return BSATTN_ERR_SHAPE;
    if (q->N % layout->block != 0) return BSATTN_ERR_SHAPE;
    const int64_t nb = q->N / layout->block;
    if (out->B != q->B || out->H != q->H || out->nqb != nb) return BSATTN_ERR_SHAPE;
    if (!budget_ok(budget)) return BSATTN_ERR_BUDGET;
    if ((st = make_geometry(layout, q->N, budget, g)) != BSATTN_OK) return st;
    if (!g.is_dense && g.n_cand > kMaxCand) return BSATTN_ERR_UNSUPPORTED;
    // the pool kernel indexes its (tensor, b, head, candidate) items in 32 bits
    if (!g.is_dense && q->B * (q->H + k->H) * g.n_cand > INT32_MAX) return BSATTN_ERR_SHAPE;
    return BSATTN_OK;
}

// The launches of a validated selection; `workspace` holds the pooled sums.
bsattn_status select_launch(const bsattn_tensor* q, const bsattn_tensor* k, const bsattn_layout* layout,
                            const Geometry& g, bsattn_block_mask* out, void* workspace, const uint8_t* head_mask,
                            hipStream_t s) {
    const MaskOut mo{out->mask, out->count, out->index};
    out->k = g.k;
    out->is_dense = g.is_dense;
    hipError_t e;
    if (g.is_dense) {
        e = launch_layout_fill(g, (int)(q->B * q->H), (int)q->H, head_mask, mo, s);
    } else {
        const PoolSpace ps = pool_space(q->B, q->H, k->H, pooled_rows(g.n_cand), q->D);
        const PooledSums qp = pooled_part(workspace, ps.q_hi, ps.q_lo, ps.q_nrm);
        const PooledSums kp = pooled_part(workspace, ps.k_hi, ps.k_lo, ps.k_nrm);
        // the XCD-grouped order when an XCD's share of the pooled Q and K fits
        // in its L2, where the attention launch that follows finds it
        const int64_t pooled_bytes = q->B * (q->H + k->H) * g.n_cand * layout->block * q->D *
                                     (q->dtype == BSATTN_F32 ? 4 : 2);
        const int xcd_groups = pooled_bytes / kNumXcd <= kL2BytesPerXcd ? 1 : 0;
        e = launch_pool(q->dtype == BSATTN_F32, (int)q->D, layout->block, view_of(q), view_of(k),
                        (int)q->B, (int)q->H, (int)k->H, g, qp, kp, xcd_groups, head_mask, s);
        if (e == hipSuccess)
            e = launch_score_rank((int)q->D, qp, kp, (int)q->B, (int)q->H, (int)k->H, g, mo, xcd_groups,
                                  head_mask, s);
    }
    return e == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}
}  // namespace

extern "C" {

bsattn_status bsattn_select_heads(const bsattn_tensor* q, const bsattn_tensor* k,
                                  const bsattn_layout* layout, double budget, const uint8_t* head_mask,
                                  bsattn_block_mask* out, void* workspace, size_t workspace_bytes, void* stream) {
    Geometry g;
    const bsattn_status st = select_validate(q, k, layout, budget, out, g);
    if (st != BSATTN_OK) return st;
    if (!g.is_dense) {
        const size_t need = bsattn_select_workspace_bytes(q->B, q->H, k->H, q->N, layout->block, q->D);
        if (workspace == nullptr) return BSATTN_ERR_WORKSPACE;
        if (workspace_bytes < need || ((uintptr_t)workspace) % 256 != 0) return BSATTN_ERR_WORKSPACE;
    }
    return select_launch(q, k, layout, g, out, workspace, head_mask, (hipStream_t)stream);
}

bsattn_status bsattn_select(const bsattn_tensor* q, const bsattn_tensor* k,
                            const bsattn_layout* layout, double budget, bsattn_block_mask* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return bsattn_select_heads(q, k, layout, budget, nullptr, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Selection without a caller workspace, for callers that cannot allocate
// device memory.  The pooled sums live in `scratch`, a file-scope device
// array that the code object carries: each GPU the library runs on holds its
// own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); the device address comes from hipGetSymbolAddress, taken once
// per device with that device current.  Every call on one GPU shares the
// array, so calls that overlap on one GPU race.  Nothing in it has to start
// at zero: the pool kernel writes every sum and norm the score kernel reads
// for the candidates (rows past them, the padding of a 16-row tile, only feed
// score columns that are never ranked).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[BSATTN_NO_ALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on its first use).
bsattn_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return BSATTN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return BSATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BSATTN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BSATTN_OK;
}
}  // namespace

extern "C" {

bsattn_status bsattn_select_no_alloc(const bsattn_tensor* q, const bsattn_tensor* k,
                                     const bsattn_layout* layout, double budget,
                                     bsattn_block_mask* out, void* stream) {
    Geometry g;
    bsattn_status st = select_validate(q, k, layout, budget, out, g);
    if (st != BSATTN_OK) return st;
    void* ws = nullptr;
    if (!g.is_dense) {
        const size_t need = bsattn_select_workspace_bytes(q->B, q->H, k->H, q->N, layout->block, q->D);
        if (need > (size_t)BSATTN_NO_ALLOC_SCRATCH_BYTES) return BSATTN_ERR_WORKSPACE;
        if ((st = scratch_address(&ws)) != BSATTN_OK) return st;
    }
    return select_launch(q, k, layout, g, out, ws, nullptr, (hipStream_t)stream);
}

bsattn_status bsattn_quantize_fp8(const bsattn_tensor* x, bsattn_tensor* out, float* scale, void* ws,
                                  size_t ws_bytes, void* stream) {
    bsattn_status st;
    if ((st = check_tensor(x)) != BSATTN_OK) return st;
    if ((st = check_tensor(out, true)) != BSATTN_OK) return st;
    if (x->dtype != BSATTN_BF16) return BSATTN_ERR_DTYPE;
    if (out->B != x->B || out->H != x->H || out->N != x->N || out->D != x->D) return BSATTN_ERR_SHAPE;
    if (scale == nullptr || ws == nullptr) return BSATTN_ERR_NULL;
    if (ws_bytes < (size_t)(x->B * x->H) * 4 || ((uintptr_t)ws) % 4 != 0 || ((uintptr_t)scale) % 4 != 0)
        return BSATTN_ERR_WORKSPACE;
    if (x->B * x->H > INT32_MAX / 2) return BSATTN_ERR_SHAPE;
    const hipError_t e = launch_quant_fp8(view_of(x), view_of(out), (int)x->B, (int)x->H, x->N, (int)x->D,
                                          (uint32_t*)ws, scale, (hipStream_t)stream);
    return e == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

bsattn_status bsattn_forward_fp8(const bsattn_tensor* q, const bsattn_tensor* k, const bsattn_tensor* v,
                                 const float* q_scale, const float* k_scale, const float* v_scale,
                                 const bsattn_block_mask* mask, const uint8_t* head_mask, float scale,
                                 bsattn_tensor* out, void* stream) {
    return bsattn_forward_fp8_masked(q, k, v, q_scale, k_scale, v_scale, mask, head_mask, nullptr, 0, scale, out,
                                     stream);
}

bsattn_status bsattn_forward_fp8_masked(const bsattn_tensor* q, const bsattn_tensor* k, const bsattn_tensor* v,
                                        const float* q_scale, const float* k_scale, const float* v_scale,
                                        const bsattn_block_mask* mask, const uint8_t* head_mask,
                                        const uint8_t* key_mask, int64_t key_mask_stride_b, float scale,
                                        bsattn_tensor* out, void* stream) {
    bsattn_status st;
    if ((st = check_tensor(q, true)) != BSATTN_OK) return st;
    if ((st = check_tensor(k, true)) != BSATTN_OK) return st;
    if ((st = check_tensor(v, true)) != BSATTN_OK) return st;
    if ((st = check_tensor(out)) != BSATTN_OK) return st;
    if (out->dtype != BSATTN_BF16) return BSATTN_ERR_DTYPE;
    if (q_scale == nullptr || k_scale == nullptr || v_scale == nullptr) return BSATTN_ERR_NULL;
    if (k->B != q->B || v->B != q->B || out->B != q->B) return BSATTN_ERR_SHAPE;
    if (k->N != q->N || v->N != q->N || out->N != q->N) return BSATTN_ERR_SHAPE;
    if (k->D != q->D || v->D != q->D || out->D != q->D) return BSATTN_ERR_SHAPE;
    if (v->H != k->H || out->H != q->H || q->H % k->H != 0) return BSATTN_ERR_SHAPE;
    if (q->D != 64 && q->D != 128) return BSATTN_ERR_UNSUPPORTED;
    const int64_t block = 64;
    if (q->N % block != 0) return BSATTN_ERR_SHAPE;
    if (mask != nullptr) {
        if (mask->count == nullptr || mask->index == nullptr) return BSATTN_ERR_NULL;
        if (mask->nqb != q->N / block || mask->nkb != mask->nqb) return BSATTN_ERR_SHAPE;
        if (!(mask->B == 1 || mask->B == q->B) || !(mask->H == 1 || mask->H == q->H)) return BSATTN_ERR_SHAPE;
    }
    if (!std::isfinite(scale)) return BSATTN_ERR_BUDGET;
    if (k->stride_n > (1 << 24) || v->stride_n > (1 << 24)) return BSATTN_ERR_UNSUPPORTED;
    if (key_mask != nullptr && (key_mask_stride_b < 0 || (key_mask_stride_b > 0 && key_mask_stride_b < q->N)))
        return BSATTN_ERR_STRIDE;
    AttnArgs a{};
    a.q = view_of(q);
    a.k = view_of(k);
    a.v = view_of(v);
    a.o = out->data;
    a.o_sb = out->stride_b;
    a.o_sh = out->stride_h;
    a.o_sn = out->stride_n;
    a.B = (int32_t)q->B;
    a.H = (int32_t)q->H;
    a.Hkv = (int32_t)k->H;
    a.nqb = (int32_t)(q->N / block);
    a.nkb = a.nqb;
    a.mB = mask ? mask->B : 1;
    a.mH = mask ? mask->H : 1;
    a.count = mask ? mask->count : nullptr;
    a.index = mask ? mask->index : nullptr;
    a.head_mask = head_mask;
    a.key_mask = key_mask;
    a.km_sb = key_mask_stride_b;
    a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)q->D);
    a.n_work = (int64_t)a.B * a.H * a.nqb;
    const hipError_t e = launch_attn_fp8(a, (int)q->D, q_scale, k_scale, v_scale, (hipStream_t)stream);
    return e == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

bsattn_status bsattn_radial(const bsattn_layout* layout, double density, bsattn_block_mask* out,
                            void* stream) {
    bsattn_status st;
    if ((st = check_layout(layout)) != BSATTN_OK) return st;
    if (out == nullptr) return BSATTN_ERR_NULL;
    if ((st = check_mask_out(out)) != BSATTN_OK) return st;
    if (!budget_ok(density)) return BSATTN_ERR_BUDGET;
    const int64_t N = (int64_t)out->nqb * layout->block;
    Geometry g;
    if ((st = make_geometry(layout, N, density, g)) != BSATTN_OK) return st;
    out->k = g.k;
    out->is_dense = g.is_dense;
    const MaskOut mo{out->mask, out->count, out->index};
    const hipError_t e = launch_layout_fill(g, out->B * out->H, 0, nullptr, mo, (hipStream_t)stream);
    return e == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

bsattn_status bsattn_forward(const bsattn_tensor* q, const bsattn_tensor* k,
                             const bsattn_tensor* v, const bsattn_block_mask* mask,
                             const uint8_t* head_mask, float scale, bsattn_tensor* out,
                             void* stream) {
    return bsattn_forward_masked(q, k, v, mask, head_mask, nullptr, 0, scale, out, stream);
}

bsattn_status bsattn_forward_masked(const bsattn_tensor* q, const bsattn_tensor* k,
                                    const bsattn_tensor* v, const bsattn_block_mask* mask,
                                    const uint8_t* head_mask, const uint8_t* key_mask,
                                    int64_t key_mask_stride_b, float scale, bsattn_tensor* out,
                                    void* stream) {
    bsattn_status st;
    if ((st = check_tensor(q)) != BSATTN_OK) return st;
    if ((st = check_tensor(k)) != BSATTN_OK) return st;
    if ((st = check_tensor(v)) != BSATTN_OK) return st;
    if ((st = check_tensor(out)) != BSATTN_OK) return st;
    if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype) return BSATTN_ERR_DTYPE;
    if (k->B != q->B || v->B != q->B || out->B != q->B) return BSATTN_ERR_SHAPE;
    if (k->N != q->N || v->N != q->N || out->N != q->N) return BSATTN_ERR_SHAPE;
    if (k->D != q->D || v->D != q->D || out->D != q->D) return BSATTN_ERR_SHAPE;
    if (v->H != k->H || out->H != q->H || q->H % k->H != 0) return BSATTN_ERR_SHAPE;
    int64_t block;
    if (mask == nullptr) {
        block = 64;
        if (q->N % block != 0) return BSATTN_ERR_SHAPE;
    } else {
        if (mask->count == nullptr || mask->index == nullptr) return BSATTN_ERR_NULL;
        if (mask->nqb <= 0 || mask->nqb != mask->nkb || q->N % mask->nqb != 0) return BSATTN_ERR_SHAPE;
        block = q->N / mask->nqb;
        if (block != 32 && block != 64) return BSATTN_ERR_SHAPE;
        if (!(mask->B == 1 || mask->B == q->B) || !(mask->H == 1 || mask->H == q->H))
            return BSATTN_ERR_SHAPE;
    }
    if (!(std::isfinite(scale))) return BSATTN_ERR_BUDGET;
    if (key_mask != nullptr && (key_mask_stride_b < 0 || (key_mask_stride_b > 0 && key_mask_stride_b < q->N)))
        return BSATTN_ERR_STRIDE;

    AttnArgs a{};
    a.q = view_of(q);
    a.k = view_of(k);
    a.v = view_of(v);
    a.o = out->data;
    a.o_sb = out->stride_b;
    a.o_sh = out->stride_h;
    a.o_sn = out->stride_n;
    a.B = (int32_t)q->B;
    a.H = (int32_t)q->H;
    a.Hkv = (int32_t)k->H;
    a.nqb = (int32_t)(q->N / block);
    a.nkb = a.nqb;
    a.mB = mask ? mask->B : 1;
    a.mH = mask ? mask->H : 1;
    a.count = mask ? mask->count : nullptr;
    a.index = mask ? mask->index : nullptr;
    a.head_mask = head_mask;
    a.key_mask = key_mask;
    a.km_sb = key_mask ? key_mask_stride_b : 0;
    a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)q->D);
    a.n_work = (int64_t)a.B * a.H * a.nqb;

    const hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (q->dtype == BSATTN_BF16 && block == 64 && (q->D == 64 || q->D == 128)) {
        // the MFMA kernel keeps per-thread K/V row offsets of one block in 32 bits
        if (k->stride_n > (1 << 24) || v->stride_n > (1 << 24)) return BSATTN_ERR_UNSUPPORTED;
        e = launch_attn_mfma(a, (int)q->D, s);
    }
    else
        e = launch_attn_f32(a, q->dtype == BSATTN_F32, (int)q->D, (int)block, s);
    return e == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

bsattn_status bsattn_select_forward(const bsattn_tensor* q, const bsattn_tensor* k,
                                    const bsattn_tensor* v, const bsattn_layout* layout, double budget,
                                    const uint8_t* head_mask, float scale, bsattn_tensor* out,
                                    bsattn_block_mask* mask, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (q == nullptr || k == nullptr || v == nullptr || layout == nullptr || out == nullptr || mask == nullptr)
        return BSATTN_ERR_NULL;
    // The fused kernel covers the shape where every block of the sequence is
    // a candidate and a row fits one wavefront: bf16, D 64, block 64, no
    // layout segments and no window, at most 64 blocks, a selective budget,
    // no head mask.  Everything else is bsattn_select followed by
    // bsattn_forward, with identical results.
    bool fused = q->dtype == BSATTN_BF16 && q->D == 64 && layout->block == 64 && layout->n_segments == 0 &&
                 layout->window_tokens == 0 && head_mask == nullptr && q->N > 0 && q->N % 64 == 0 &&
                 q->N / 64 <= 64 && k->stride_n <= (1 << 24) && v->stride_n <= (1 << 24);
    Geometry g;
    if (fused) fused = make_geometry(layout, q->N, budget, g) == BSATTN_OK && !g.is_dense && g.n_runs == 1 &&
                       g.run_cls[0] == CLS_SPARSE && g.n_cand == q->N / 64;
    if (!fused) {
        bsattn_status st = bsattn_select(q, k, layout, budget, mask, workspace, workspace_bytes, stream);
        if (st != BSATTN_OK) return st;
        return bsattn_forward(q, k, v, mask, head_mask, scale, out, stream);
    }
    // the checks of bsattn_select and bsattn_forward
    bsattn_status st;
    if ((st = check_tensor(q)) != BSATTN_OK) return st;
    if ((st = check_tensor(k)) != BSATTN_OK) return st;
    if ((st = check_tensor(v)) != BSATTN_OK) return st;
    if ((st = check_tensor(out)) != BSATTN_OK) return st;
    if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype) return BSATTN_ERR_DTYPE;
    if (k->B != q->B || v->B != q->B || out->B != q->B) return BSATTN_ERR_SHAPE;
    if (k->N != q->N || v->N != q->N || out->N != q->N) return BSATTN_ERR_SHAPE;
    if (k->D != q->D || v->D != q->D || out->D != q->D) return BSATTN_ERR_SHAPE;
    if (v->H != k->H || out->H != q->H || q->H % k->H != 0) return BSATTN_ERR_SHAPE;
    const int64_t nb = q->N / 64;
    if (mask->B != q->B || mask->H != q->H || mask->nqb != nb || mask->nkb != nb) return BSATTN_ERR_SHAPE;
    if (mask->mask == nullptr || mask->count == nullptr || mask->index == nullptr) return BSATTN_ERR_NULL;
    if (!budget_ok(budget)) return BSATTN_ERR_BUDGET;
    if (!(std::isfinite(scale))) return BSATTN_ERR_BUDGET;
    if (q->B * (q->H + k->H) * g.n_cand > INT32_MAX) return BSATTN_ERR_SHAPE;
    const size_t need = bsattn_select_workspace_bytes(q->B, q->H, k->H, q->N, 64, q->D);
    if (workspace == nullptr) return BSATTN_ERR_WORKSPACE;
    if (workspace_bytes < need || ((uintptr_t)workspace) % 256 != 0) return BSATTN_ERR_WORKSPACE;

    const hipStream_t s = (hipStream_t)stream;
    mask->k = g.k;
    mask->is_dense = 0;
    // K's block sums only: each attention workgroup sums its own query block
    const PoolSpace ps = pool_space(q->B, q->H, k->H, pooled_rows(g.n_cand), q->D);
    const PooledSums kp = pooled_part(workspace, ps.k_hi, ps.k_lo, ps.k_nrm);
    const int64_t pooled_bytes = q->B * k->H * g.n_cand * 64 * q->D * 2;
    const int xcd_groups = pooled_bytes / kNumXcd <= kL2BytesPerXcd ? 1 : 0;
    hipError_t e = launch_pool(0, 64, 64, view_of(q), view_of(k), (int)q->B, (int)q->H, (int)k->H, g,
                               PooledSums{nullptr, nullptr, nullptr}, kp, xcd_groups, nullptr, s);
    if (e != hipSuccess) return BSATTN_ERR_HIP;
    AttnArgs a{};
    a.q = view_of(q);
    a.k = view_of(k);
    a.v = view_of(v);
    a.o = out->data;
    a.o_sb = out->stride_b;
    a.o_sh = out->stride_h;
    a.o_sn = out->stride_n;
    a.B = (int32_t)q->B;
    a.H = (int32_t)q->H;
    a.Hkv = (int32_t)k->H;
    a.nqb = (int32_t)nb;
    a.nkb = (int32_t)nb;
    a.mB = 1;
    a.mH = 1;
    a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)q->D);
    a.n_work = (int64_t)a.B * a.H * a.nqb;
    a.kp = kp.hi;
    a.kp_lo = kp.lo;
    a.prow = (int32_t)pooled_rows(g.n_cand);
    a.keep = g.k;
    a.m_out = mask->mask;
    a.c_out = mask->count;
    a.i_out = mask->index;
    e = launch_attn_fused(a, s);
    return e == hipSuccess ? BSATTN_OK : BSATTN_ERR_HIP;
}

bsattn_status bsattn_head_mask(const double* importance, int32_t H, double sparsity,
                               int32_t min_active, uint8_t* out) {
    if (importance == nullptr || out == nullptr) return BSATTN_ERR_NULL;
    if (H <= 0) return BSATTN_ERR_SHAPE;
    if (!(sparsity >= 0.0 && sparsity <= 1.0) || min_active < 0) return BSATTN_ERR_BUDGET;
    for (int32_t h = 0; h < H; ++h)
        if (!std::isfinite(importance[h])) return BSATTN_ERR_BUDGET;
    int32_t n_act = H - (int32_t)std::floor(sparsity * (double)H);
    if (n_act < min_active) n_act = min_active;
    if (n_act > H) n_act = H;
    // a head is kept when fewer than n_act heads rank above it
    for (int32_t h = 0; h < H; ++h) {
        int32_t above = 0;
        for (int32_t o = 0; o < H; ++o)
            above += importance[o] > importance[h] || (importance[o] == importance[h] && o < h);
        out[h] = above < n_act ? 1 : 0;
    }
    return BSATTN_OK;
}

bsattn_status bsattn_mask_density(const bsattn_block_mask* m, void* stream, double* density) {
    if (m == nullptr || m->count == nullptr || density == nullptr) return BSATTN_ERR_NULL;
    if (m->B <= 0 || m->H <= 0 || m->nqb <= 0 || m->nkb <= 0) return BSATTN_ERR_SHAPE;
    const size_t rows = (size_t)m->B * m->H * m->nqb;
    std::vector<int32_t> host(rows);
    const hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(host.data(), m->count, rows * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return BSATTN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return BSATTN_ERR_HIP;
    double kept = 0.0;
    for (size_t r = 0; r < rows; ++r) kept += host[r];
    *density = kept / ((double)rows * m->nkb);
    return BSATTN_OK;
}

}  // extern "C"
