// Selector kernels of libbsattn (gfx950).
//
//  pool_kernel        block sums of Q and K over the SPARSE blocks (HBM bound;
//                     16-byte coalesced loads, fp32 accumulation).
//  score_rank_kernel  per (b, h, tile of candidate rows): fp32 MFMA scores of
//                     every candidate pair, a wavefront bitonic sort of each
//                     row with ties to the lower block index, then pins,
//                     drops, the sliding window and CSR compaction.  PINNED and
//                     DROPPED rows are written by the same launch.
//  layout_kernel      the radial band and the layout-only (dense) mask.
//
// SD.Next commit view, modules/attention/sparse: the selector paragraph
// (tile mean-pooling, unscaled pair scores, a per-row budget over the
// sparsifiable candidates, diagonal kept, full budget reports dense), the
// layout paragraph (pins and drops), the radial-control paragraph (band at the
// selector's density honouring the pins) and the synchronisation paragraph
// (ranking replaces a host-sized top-k; no host sync anywhere here).
#include "common.h"
#include "internal.h"
#include "rank.h"

namespace bsattn {

typedef float f4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Pooled sums in the workspace, per (b, head): row tiles of 16 candidates,
// each laid out in the order the score MFMA (16x16x4 fp32) reads them.  With
// KQ = D / 4, lane l = li + 16 gq of the MFMA takes row li of the tile and d
// = gq KQ + 4 c + e for k-step (c, e); element (row p, d) sits at
//   tile(p) * 16 D + ((c * 4 + gq) * 16 + li) * 4 + e
// so each lane's four k-steps of one c are one 16-byte read, and the 64
// lanes of a wavefront read 1 KB of consecutive bytes per c.  Rows are padded
// to a multiple of 16 per head.
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// K1: block sums.  One wavefront per (tensor, b, head, candidate block).
// Ranking by <sum Q_i, sum K_j> equals ranking by the mean-pooled score: the
// factor 1/block^2 is a positive constant.
// ---------------------------------------------------------------------------
// xcd_groups: items in (b, K/V head) groups -- the query heads of the group,
// then the K/V head -- in the XCD-grouped workgroup order of the attention
// kernel, so that the XCD that pools a group's Q and K is the one whose
// attention workgroups read them next, from its L2 when an XCD's share fits
// there (the host decides).  Otherwise the plain order (tensor, b, head,
// block).  qp.hi NULL: K only (the fused attention sums its own query block).
// The sums are taken in float64 (exact for bf16 inputs short of extreme
// exponent spreads) and stored as PooledSums: float32 hi and lo parts and a
// norm bound of the hi row, which the score kernel's error bound uses.
template <typename T, int D, int BLOCK>
__global__ __launch_bounds__(256) void pool_kernel(TView q, TView k, int B, int H, int Hkv,
                                                   Geometry g, PooledSums qp, PooledSums kp, int xcd_groups,
                                                   const uint8_t* head_mask) {
    constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
    constexpr int CPR = D / EPC;               // chunks per token row
    constexpr int RPI = 64 / CPR;              // token rows per wave instruction
    constexpr int NL = BLOCK / RPI;            // loads per lane
    static_assert(CPR <= 64 && 64 % CPR == 0 && BLOCK % RPI == 0, "pool geometry");

    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform: scalar lookups
    // 32-bit index arithmetic (the host checks that the items fit): the
    // division sequences sit in front of every wavefront's loads
    const uint32_t nc = (uint32_t)g.n_cand;
    const bool with_q = qp.hi != nullptr;
    const uint32_t nq = with_q ? (uint32_t)B * (uint32_t)H * nc : 0u, nk = (uint32_t)B * (uint32_t)Hkv * nc;
    // which tensor, (b, head) and candidate this wavefront pools; the
    // tensor's fields are selected by value (a pointer to a kernel argument
    // would put both views in scratch memory)
    bool is_q;
    uint32_t hh, b, p;
    if (xcd_groups) {
        const uint32_t item = (uint32_t)xcd_logical_id(blockIdx.x, gridDim.x) * 4u + wave;   // grid: a multiple of 8
        if (item >= nq + nk) return;
        const uint32_t rep = with_q ? (uint32_t)(H / Hkv) : 0u;
        const uint32_t per_group = (rep + 1) * nc;
        const uint32_t grp = item / per_group, r = item - grp * per_group;
        b = grp / (uint32_t)Hkv;
        const uint32_t kvh = grp - b * (uint32_t)Hkv;
        is_q = r < rep * nc;
        if (is_q) {
            const uint32_t j = r / nc;
            hh = kvh * rep + j;
            p = r - j * nc;
        } else {
            hh = kvh;
            p = r - rep * nc;
        }
    } else {
        const uint32_t item = blockIdx.x * 4u + wave;
        if (item >= nq + nk) return;
        is_q = item < nq;
        const uint32_t rem = is_q ? item : item - nq;
        const uint32_t heads = is_q ? (uint32_t)H : (uint32_t)Hkv;
        const uint32_t bh = rem / nc;
        p = rem - bh * nc;
        b = bh / heads;
        hh = bh - b * heads;
    }
    // under a head mask: a masked query head's Q, and the K of a K/V head
    // whose query heads are all masked, are never scored
    if (head_mask != nullptr) {
        bool live = false;
        if (is_q) {
            live = head_mask[hh] != 0;
        } else {
            const uint32_t rep = (uint32_t)(H / Hkv);
            for (uint32_t j = 0; j < rep; ++j) live = live || head_mask[hh * rep + j] != 0;
        }
        if (!live) return;
    }
    const T* src_p = (const T*)(is_q ? q.p : k.p);
    const int64_t sb = is_q ? q.sb : k.sb, sh = is_q ? q.sh : k.sh, sn = is_q ? q.sn : k.sn;
    const int64_t heads = is_q ? H : Hkv;
    const PooledSums out = is_q ? qp : kp;

    const int64_t blk = cand_block(g, (int32_t)p);
    const int64_t head_row0 = ((int64_t)b * heads + hh) * pooled_rows(g.n_cand);

    const T* base = src_p + b * sb + hh * sh + (blk * BLOCK + lane / CPR) * sn + (lane % CPR) * EPC;
    uint4 raw[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l)
        raw[l] = *(const uint4*)(base + (int64_t)l * RPI * sn);

    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const uint32_t w[4] = {raw[l].x, raw[l].y, raw[l].z, raw[l].w};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += (double)__uint_as_float(w[e] << 16);
                acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(w[e]);
        }
    }
    // lanes holding the same chunk of different rows: lane % CPR equal
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += lane_xor_f64(acc[e], off);

    // every lane now holds its chunk's sums; split them, and sum the squares
    // of the hi parts over the row's CPR chunks (lanes 0 .. CPR - 1)
    float hi[EPC], lo[EPC];
    double n2 = 0.0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        hi[e] = (float)acc[e];
        lo[e] = (float)(acc[e] - (double)hi[e]);
        n2 += (double)hi[e] * (double)hi[e];
    }
#pragma unroll
    for (int off = 1; off < CPR; off <<= 1) n2 += lane_xor_f64(n2, off);
    if (lane < CPR) {
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            const int64_t o = head_row0 * D + pooled_offset<D>((int32_t)p, lane * EPC + e);
            *(f4v*)(out.hi + o) = f4v{hi[e], hi[e + 1], hi[e + 2], hi[e + 3]};
            *(f4v*)(out.lo + o) = f4v{lo[e], lo[e + 1], lo[e + 2], lo[e + 3]};
        }
    }
    // rounded up: an upper bound of the norm
    if (lane == 0) out.nrm[head_row0 + p] = (float)(sqrt(n2) * (1.0 + 0x1p-20));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// Descending bitonic sort of 64*E keys spread over one wavefront; element
// e = lane * E + r lives in key[r].
template <int E>
__device__ __forceinline__ void wave_bitonic_desc(uint64_t (&key)[E], int lane) {
    constexpr int NTOT = 64 * E;
#pragma unroll
    for (int size = 2; size <= NTOT; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride < E) {
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    if (r & stride) continue;
                    const int e = lane * E + r;
                    const bool desc = (e & size) == 0;
                    const uint64_t a = key[r], b = key[r | stride];
                    const bool swap = desc ? (a < b) : (a > b);
                    key[r] = swap ? b : a;
                    key[r | stride] = swap ? a : b;
                }
            } else {
                const int lm = stride / E;
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const int e = lane * E + r;
                    const uint64_t other = shfl_xor_u64(key[r], lm);
                    const bool lower = (e & stride) == 0;
                    const bool desc = (e & size) == 0;
                    const uint64_t mx = key[r] > other ? key[r] : other;
                    const uint64_t mn = key[r] > other ? other : key[r];
                    key[r] = (lower == desc) ? mx : mn;
                }
            }
        }
    }
}

// Column codes of a whole row, cached in LDS by the kernels below when the
// sequence has at most kCodeTable blocks (else column_code scans the runs).
constexpr int kCodeTable = 1024;

// Writes one mask row (all nb columns), its ascending index list and count,
// with one wavefront.  keep(j, code) decides SPARSE columns; PINNED columns
// are kept and DROPPED ones are not, unless `row_dropped` (then nothing).
// Each lane takes four consecutive columns per pass: the mask goes out as one
// 32-bit store per lane (vec4: nb % 4 == 0 and a 4-byte aligned mask), and a
// lane's slot in the index list is the wavefront prefix sum of the per-lane
// counts (0..4), taken bit-plane by bit-plane with ballots.
// The pass is branch-free so that its LDS reads overlap: the four codes come
// in one 8-byte read of the code table, and keep() is evaluated for every
// column at a clamped code (>= 0; an LDS read in keep() stays in its row)
// and its result used only for live SPARSE columns.
template <typename KeepFn>
__device__ __forceinline__ void compact_row(const Geometry& g, const int16_t* codes, bool vec4, int lane,
                                            bool row_dropped, bool row_pinned, uint8_t* mrow,
                                            int32_t* irow, int32_t* cnt_out, KeepFn keep) {
    const uint64_t below = (1ull << lane) - 1ull;
    int32_t cnt = 0;
    for (int32_t j0 = 0; j0 < g.nb; j0 += 256) {
        const int32_t jl = j0 + 4 * lane;
        int32_t code[4];
        if (codes != nullptr) {
            // jl + 3 < kCodeTable: j0 < nb <= kCodeTable and j0 % 256 == 0
            const uint2 c4 = *(const uint2*)(codes + jl);
            code[0] = (int32_t)(int16_t)(c4.x & 0xffffu);
            code[1] = (int32_t)(int16_t)(c4.x >> 16);
            code[2] = (int32_t)(int16_t)(c4.y & 0xffffu);
            code[3] = (int32_t)(int16_t)(c4.y >> 16);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) code[u] = jl + u < g.nb ? column_code(g, jl + u) : -2;
        }
        // table entries past nb are never used
#pragma unroll
        for (int u = 0; u < 4; ++u) code[u] = jl + u < g.nb && !row_dropped ? code[u] : -2;
        uint32_t kbits = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) kbits |= (uint32_t)keep(jl + u, code[u] > 0 ? code[u] : 0) << u;
        // the empty asm keeps the four keep() evaluations (LDS reads) ahead
        // of the branches below, so that they are waited for once
        asm volatile("" : "+v"(kbits));
        // bitwise rather than short-circuit logic: selects, not branches
        uint32_t bits = 0, c = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t live = code[u] != -2 ? 1u : 0u;
            const uint32_t pin = (code[u] == -1 ? 1u : 0u) | (row_pinned ? 1u : 0u);
            const uint32_t v = live & (pin | ((kbits >> u) & 1u));
            bits |= v << (8 * u);
            c += v;
        }
        const uint64_t b0 = __ballot(c & 1), b1 = __ballot(c & 2), b2 = __ballot(c & 4);
        // unsigned slot: the store takes the list base from scalar registers
        uint32_t n = (uint32_t)cnt + __popcll(b0 & below) + 2 * __popcll(b1 & below) + 4 * __popcll(b2 & below);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if ((bits >> (8 * u)) & 1u) irow[n++] = jl + u;
        if (vec4) {
            if (jl < g.nb) *(uint32_t*)(mrow + jl) = bits;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (jl + u < g.nb) mrow[jl + u] = (uint8_t)((bits >> (8 * u)) & 1u);
        }
        cnt += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    }
    if (lane == 0) *cnt_out = cnt;
}

// Fills the LDS column-code table (all threads of the workgroup take part;
// the caller synchronises before use).  Returns the table, or nullptr when
// the sequence is too long for it.
__device__ __forceinline__ const int16_t* fill_codes(const Geometry& g, int16_t* table) {
    if (g.nb > kCodeTable) return nullptr;
    for (int32_t j = threadIdx.x; j < g.nb; j += blockDim.x) table[j] = (int16_t)column_code(g, j);
    return table;
}

// Float64 dot product of two candidate rows' (hi + lo) block sums (row p of
// the query head's sums, row pos of the key head's), four partial sums so
// the loads of an unrolled group issue together and the FMA chains overlap.
template <int D>
__device__ __forceinline__ double pooled_dot64(const float* qhi, const float* qlo, const float* khi,
                                               const float* klo, int p, int pos) {
    double t[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
    for (int c = 0; c < D / 4; ++c) {
        const int64_t oq = pooled_offset<D>(p, 4 * c), ok = pooled_offset<D>(pos, 4 * c);
        const f4v qh = *(const f4v*)(qhi + oq), ql = *(const f4v*)(qlo + oq);
        const f4v kh = *(const f4v*)(khi + ok), kl = *(const f4v*)(klo + ok);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            t[e] = fma((double)qh[e] + (double)ql[e], (double)kh[e] + (double)kl[e], t[e]);
    }
    return (t[0] + t[1]) + (t[2] + t[3]);
}

// A row ranked from float64 scores: for every candidate but the diagonal,
// the dot product of the (hi + lo) block sums in float64; keys are the
// order-preserving image of that score with its low index bits replaced by
// the reversed candidate position (relative resolution 2^-41), the diagonal
// first; one wavefront sorts them (64-bit bitonic) and marks the first
// `keep` in keep_row (cleared by the caller).  The slow, exact path taken by
// the rows whose float32 ranking could not be certified.
template <int D, int E>
__device__ __noinline__ void exact_rank(const float* qhi, const float* qlo, const float* khi, const float* klo,
                                        int p, int n_cand, int keep, int lane, uint8_t* keep_row) {
    constexpr int NPAD = 64 * E;
    constexpr uint64_t IM = (uint64_t)NPAD - 1;
    uint64_t key[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int pos = lane * E + r;
        const uint64_t low = IM - (uint64_t)pos;
        const double acc = pos < n_cand && pos != p ? pooled_dot64<D>(qhi, qlo, khi, klo, p, pos) : 0.0;
        if (pos >= n_cand) key[r] = 0ull;
        else if (pos == p) key[r] = ~IM | low;
        else key[r] = (orderable64(acc) & ~IM) | low;
    }
    wave_bitonic_desc<E>(key, lane);
#pragma unroll
    for (int r = 0; r < E; ++r)
        if (lane * E + r < keep) keep_row[IM - (key[r] & IM)] = 1;
}

// Rows per workgroup and wavefronts per workgroup of the score/rank kernel:
// one 16-row MFMA tile per workgroup (more workgroups beat longer ones:
// 32-row tiles took 32 -> 26 us on the joint text+image shape and 100 -> 70 us
// on the video shape).  Up to 128 candidates each wavefront ranks one row:
// the compaction of a row is a few hundred scalar and vector instructions,
// so rows compact side by side rather than one after another.  At D <= 64
// four workgroups share a tile -- each computes the (small) tile and ranks
// four of its rows -- spreading the rows over more CUs with fewer
// wavefronts per SIMD (SDXL shape 9.4 -> 8.8 us); at D = 128 one workgroup
// of 16 wavefronts takes the tile (a split would reload 32 KB of key sums per
// workgroup: 64-layer stack 18.6 -> 20.6 us).  Longer rows are ranked two at a
// time by one wavefront, whose interleaved sorting networks hide each other's
// exchange latency.
#ifndef BSATTN_RANK_ONE_ROW_EMAX
#define BSATTN_RANK_ONE_ROW_EMAX 2
#endif
template <int D, int E>
struct RankShape {
    static constexpr bool SHORT = E <= BSATTN_RANK_ONE_ROW_EMAX;
    static constexpr bool SPLIT = SHORT && D <= 64;   // at D = 128 each split reloads 32 KB of key sums
    static constexpr int RT = 16;                       // rows of the score MFMA tile
    static constexpr int RQ = SPLIT ? 4 : 16;           // rows ranked per workgroup
    static constexpr int WAVES = SPLIT ? 4 : (SHORT ? 16 : 8);
    // 512 candidates: the LDS holds three workgroups per CU, and the
    // registers are held to that (six wavefronts per SIMD) with the key-sum
    // operands loaded per tile instead of one tile ahead -- on the video
    // shape the 768 workgroups then run in one round (62 -> 55-58 us)
    static constexpr int MIN_WAVES_PER_SIMD = E == 8 ? 6 : 1;
    static constexpr bool PREFETCH = MIN_WAVES_PER_SIMD < 6;
};

// ---------------------------------------------------------------------------
// K2: scores, rank and compaction for one (b, h) and RT candidate rows.
// The workgroup also writes its share of the PINNED/DROPPED rows.
//
// Rank keys.  Up to 512 candidates (E <= 8) a key is 32 bits: the
// order-preserving image of the fp32 score with its low log2(64*E) bits
// replaced by the reversed candidate position.  The kept bits resolve scores
// to better than 2^-14 relative (6.1e-5): two scores that differ by more than
// that always keep their order, so every row whose last kept and first
// dropped scores differ by more than the 1e-4 near-tie window ranks exactly
// as the exact ordering would, and closer scores fall to the lower block
// index.  Larger candidate sets use 64-bit keys (full score, then position).
// ---------------------------------------------------------------------------
template <int D, int E>
__global__ __launch_bounds__((RankShape<D, E>::WAVES * 64))
__attribute__((amdgpu_waves_per_eu(RankShape<D, E>::MIN_WAVES_PER_SIMD))) void score_rank_kernel(
    PooledSums qp, PooledSums kp, int B, int H, int Hkv, Geometry g,
    MaskOut out, int n_tiles, int xcd_groups, const uint8_t* head_mask) {
    constexpr int NPAD = 64 * E;
    constexpr int RT = RankShape<D, E>::RT;
    constexpr int RQ = RankShape<D, E>::RQ;
    constexpr int SPLITS = RT / RQ;            // workgroups per tile
    constexpr int WAVES = RankShape<D, E>::WAVES;
    constexpr bool K32 = E <= 8;
    constexpr int RPW = RQ / WAVES;            // rows per wavefront
    constexpr int RR = RPW >= 2 ? 2 : 1;       // rows ranked together (32-bit keys)
    constexpr int SSTR = NPAD + 4;             // LDS row stride (floats)
    // rows of more than 128 candidates (padded to 256 or 512) are ranked by
    // radix selection of the k-th key, shorter ones by a full sort; the counters (2^RADIX_DB of 32
    // bits) fit in the wavefront's keep rows
    constexpr bool RADIX = K32 && E >= 4;
    constexpr int RADIX_DB = RR * NPAD >= 1024 ? 8 : 7;
    constexpr int KQ = D / 4;                  // MFMA k-steps; lane group gq owns d in [gq*KQ, gq*KQ+KQ)
    static_assert(RPW >= 1 && RPW % RR == 0, "rows per wavefront");
    static_assert(!RADIX || RR * NPAD >= (4 << RADIX_DB), "radix counters fit in the keep rows");
    __shared__ float s_score[RT * SSTR];
    __shared__ __attribute__((aligned(16))) uint8_t s_keep[WAVES][K32 ? RR : 1][NPAD];
    __shared__ __attribute__((aligned(8))) int16_t s_code[kCodeTable];
    __shared__ int32_t s_rowblk[RT];             // block index of each row of the tile
    const int16_t* codes = fill_codes(g, s_code);
    const bool vec4 = (g.nb & 3) == 0 && ((uintptr_t)out.mask & 3u) == 0;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // xcd_groups: the (b, head, tile) order of the XCD-grouped workgroup ids
    // (the grid is then padded to a multiple of 8)
    const int64_t wg = xcd_groups ? xcd_logical_id(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    if (wg >= (int64_t)B * H * n_tiles * SPLITS) return;
    const int sub = (int)(wg % SPLITS);        // which RQ rows of the tile this workgroup ranks
    const int tile = (int)((wg / SPLITS) % n_tiles);
    const int64_t bh = wg / SPLITS / n_tiles;
    const int64_t b = bh / H, h = bh % H;
    const int64_t g_kv = h / (H / Hkv);
    const int p0 = tile * RT;
    const int rows = min(RT, g.n_cand - p0);
    // looked up here, next to the operand loads, rather than at each row's
    // compaction, where every argument read would wait a memory round trip
    if (threadIdx.x < RT) s_rowblk[threadIdx.x] = cand_block(g, p0 + (int)threadIdx.x);

    // a masked head (its sums were never pooled): every row this workgroup
    // writes is left empty -- mask row 0, count 0
    if (head_mask != nullptr && head_mask[h] == 0) {
        const int64_t sl = b * H + h;
        auto clear_row = [&](int32_t i) {
            uint8_t* mrow = out.mask + (sl * g.nb + i) * g.nb;
            for (int32_t j = 4 * lane; j < g.nb; j += 256) {
                if (vec4) {
                    *(uint32_t*)(mrow + j) = 0u;
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (j + u < g.nb) mrow[j + u] = 0;
                }
            }
            if (lane == 0) out.count[sl * g.nb + i] = 0;
        };
        for (int rl = sub * RQ + wave; rl < sub * RQ + RQ && rl < rows; rl += WAVES) clear_row(cand_block(g, p0 + rl));
        for (int t = (tile * SPLITS + sub) * WAVES + wave; t < g.n_other; t += n_tiles * SPLITS * WAVES)
            clear_row(other_block(g, t));
        return;
    }

    const int64_t prow = pooled_rows(g.n_cand);
    const float* qbase = qp.hi + bh * prow * D;
    const float* kbase = kp.hi + (b * Hkv + g_kv) * prow * D;
    const float* qlo = qp.lo + bh * prow * D;
    const float* klo = kp.lo + (b * Hkv + g_kv) * prow * D;
    // the largest key-row norm of this (b, K/V head), for the error bound of
    // the float32 scores (each wavefront reduces it on its own)
    float kmax = 0.f;
    {
        const float* kn = kp.nrm + (b * Hkv + g_kv) * prow;
        for (int j = lane; j < g.n_cand; j += 64) kmax = fmaxf(kmax, kn[j]);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) kmax = fmaxf(kmax, __uint_as_float(lane_xor(__float_as_uint(kmax), off)));
    }
    const float* qnrm = qp.nrm + bh * prow;

    // ---- scores S[p0 + r][c] = <Qsum_(p0+r), Ksum_c> with fp32 MFMA 16x16x4;
    // operands come straight from the tiled sums (1 KB per wave read)
    const int li = lane & 15, gq = lane >> 4;
    const int n_ct = (int)(prow / 16);
    f4v a[RT / 16][KQ / 4];
#pragma unroll
    for (int rt = 0; rt < RT / 16; ++rt) {
        const int tq = min(p0 / 16 + rt, n_ct - 1);
        const f4v* src = (const f4v*)(qbase + (int64_t)tq * 16 * D) + lane;
#pragma unroll
        for (int c = 0; c < KQ / 4; ++c) a[rt][c] = src[c * 64];
    }
    auto load_b = [&](int ct, f4v (&bv)[KQ / 4]) {
        const f4v* src = (const f4v*)(kbase + (int64_t)ct * 16 * D) + lane;
#pragma unroll
        for (int c = 0; c < KQ / 4; ++c) bv[c] = src[c * 64];
    };
    constexpr bool PREFETCH = RankShape<D, E>::PREFETCH;
    f4v bnext[KQ / 4];
    if (PREFETCH && wave < n_ct) load_b(wave, bnext);
    for (int ct = wave; ct < n_ct; ct += WAVES) {
        f4v bv[KQ / 4];
        if constexpr (PREFETCH) {
#pragma unroll
            for (int c = 0; c < KQ / 4; ++c) bv[c] = bnext[c];
            if (ct + WAVES < n_ct) load_b(ct + WAVES, bnext);
        } else {
            load_b(ct, bv);
        }
#pragma unroll
        for (int rt = 0; rt < RT / 16; ++rt) {
            f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KQ / 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt][c][e], bv[c][e], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s_score[(rt * 16 + 4 * gq + r) * SSTR + ct * 16 + li] = acc[r];
        }
    }
    __syncthreads();

    const int64_t slice = b * H + h;
    const int64_t nb = g.nb;
    const int32_t w = g.w;
    auto compact_sparse = [&](int p, const uint8_t* keep_row) {
        const int32_t i = __builtin_amdgcn_readfirstlane(s_rowblk[p - p0]);
        compact_row(g, codes, vec4, lane, false, false, out.mask + (slice * nb + i) * nb,
                    out.index + (slice * nb + i) * nb, out.count + slice * nb + i,
                    [&](int32_t j, int32_t code) {
                        return (keep_row[code] != 0) | ((w >= 0) & (abs(j - i) <= w));
                    });
    };

    // Marks the kept candidates of one row in keep_row (cleared by the
    // caller) from this wavefront's ranked keys.  pos_of(r): candidate
    // position of the lane's r-th key; in_top(r): that key is among the k
    // largest (the diagonal's included); score_last() and score_next(): the
    // float32 scores of the k-th and (k + 1)-th largest keys; tb: the keys
    // resolve scores to 2^-tb relative (0: exact float32 scores).  Slot
    // lane * E + r holds a candidate exactly when it is below n_cand, both for
    // keys sorted in descending order (the padding sorts last) and for keys
    // left in candidate order.
    //
    // Every float32 score is within err = (2 D + 16) 2^-24 |Q_i| max_j |K_j|
    // of the exact block-sum score (the float32 MFMA's accumulation and the
    // hi/lo split, bounded through the norms), and the sort sees it to within
    // T = 2^(1 - tb) max(|a|, |b|), where a and b are the scores at ranks k - 1
    // (last kept) and k (first dropped).  If a - b > M = 2 err + 2 T, every
    // kept candidate's exact score exceeds every dropped one's: the sort's
    // top k is the exact top k.  Otherwise a candidate scoring above a + M is
    // certainly kept, one below b - M certainly dropped, and the remaining
    // slots go to the best of the band between, ranked by float64 scores of
    // the (hi + lo) sums with ties to the lower block (a band of more than 64
    // ranks the whole row in float64).  Nothing to rank when k < 2 (the
    // diagonal alone) or every candidate is kept.
    __shared__ int16_t s_band[WAVES][64];
    __shared__ double s_bandt[WAVES][64];
    auto select_row = [&](auto score_last, auto score_next, auto in_top, auto pos_of, int p, int rl, int tb,
                          float qn, uint8_t* keep_row) {
        auto mark_sorted = [&]() {
#pragma unroll
            for (int r = 0; r < E; ++r)
                if (in_top(r)) keep_row[pos_of(r)] = 1;
        };
        if (g.k < 2 || g.k >= g.n_cand) { mark_sorted(); return; }
        const float a = score_last(), b = score_next();
        const float err = (float)(2 * D + 16) * 0x1p-24f * qn * kmax + 0x1p-100f;
        const float T = tb ? ldexpf(fmaxf(fabsf(a), fabsf(b)), 1 - tb) : 0.f;
        const float M = 2.f * err + 2.f * T;
        if (a - b > M) { mark_sorted(); return; }
        const float hi_edge = a + M, lo_edge = b - M;
        const float* srow = s_score + rl * SSTR;
        const uint64_t below = (1ull << lane) - 1ull;
        int n_in = 0, m = 0;
        bool band[E];
        int pos[E];
#pragma unroll
        for (int r = 0; r < E; ++r) {
            pos[r] = pos_of(r);
            // ranks past the candidates hold the padding keys
            const bool real = lane * E + r < g.n_cand && pos[r] != p;
            const float sc = srow[real ? pos[r] : 0];
            const bool in = real && sc > hi_edge;
            band[r] = real && !in && sc >= lo_edge;
            n_in += __popcll(__ballot(in));
            m += __popcll(__ballot(band[r]));
            if (in) keep_row[pos[r]] = 1;
        }
        if (lane == 0) keep_row[p] = 1;                     // the diagonal
        if (m > 64) {
            // a wide band: the whole row from float64 scores
#pragma unroll
            for (int r = 0; r < E; ++r) keep_row[lane * E + r] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            exact_rank<D, E>(qbase, qlo, kbase, klo, p, g.n_cand, g.k, lane, keep_row);
            return;
        }
        // the band's positions, one per lane
        int base = 0;
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const uint64_t bal = __ballot(band[r]);
            if (band[r]) s_band[wave][base + __popcll(bal & below)] = (int16_t)pos[r];
            base += __popcll(bal);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // float64 scores of the band, four candidates at a time, sixteen lanes
        // each (a lane takes a quarter-row slice of 4-dimension groups, so
        // all its loads issue together), summed across the sixteen lanes
        constexpr int G4 = D / 4, PER = (G4 + 15) / 16;
        for (int c0 = 0; c0 < m; c0 += 4) {
            const int cb = c0 + (lane >> 4), sl = lane & 15;
            double t = 0.0;
            if (cb < m) {
                const int pos = s_band[wave][cb];
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int gi = sl + 16 * u;
                    if (gi < G4) {
                        const int64_t oq = pooled_offset<D>(p, 4 * gi), ok = pooled_offset<D>(pos, 4 * gi);
                        const f4v qh = *(const f4v*)(qbase + oq), ql = *(const f4v*)(qlo + oq);
                        const f4v kh = *(const f4v*)(kbase + ok), kl = *(const f4v*)(klo + ok);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            t = fma((double)qh[e] + (double)ql[e], (double)kh[e] + (double)kl[e], t);
                    }
                }
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) t += lane_xor_f64(t, off);
            if (sl == 0 && cb < m) s_bandt[wave][cb] = t;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int my_pos = lane < m ? (int)s_band[wave][lane] : 0;
        const double t = lane < m ? s_bandt[wave][lane] : 0.0;
        // rank within the band: better = higher score, then lower block
        const uint64_t tu = (uint64_t)__double_as_longlong(t);
        int ahead = 0;
        for (int i = 0; i < m; ++i) {
            const uint32_t lo32 = __builtin_amdgcn_readlane((uint32_t)tu, i);
            const uint32_t hi32 = __builtin_amdgcn_readlane((uint32_t)(tu >> 32), i);
            const int pi = __builtin_amdgcn_readlane(my_pos, i);
            const double ti = __longlong_as_double((long long)(((uint64_t)hi32 << 32) | lo32));
            ahead += (ti > t || (ti == t && pi < my_pos)) ? 1 : 0;
        }
        if (lane < m && ahead < (g.k - 1) - n_in) keep_row[my_pos] = 1;
    };

    if constexpr (K32) {
        // ---- RR rows at a time per wavefront
        constexpr int IB = __builtin_ctz(NPAD);            // index bits
        constexpr uint32_t IMASK = (1u << IB) - 1u;
        for (int r0 = sub * RQ + wave * RPW; r0 < sub * RQ + wave * RPW + RPW; r0 += RR) {
            uint32_t key[RR][E];
#pragma unroll
            for (int q = 0; q < RR; ++q) {
                const int rl = r0 + q;
                const int p = p0 + rl;
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const int pos = lane * E + r;
                    const uint32_t low = IMASK - (uint32_t)pos;
                    uint32_t kv;
                    if (rl >= rows || pos >= g.n_cand) kv = 0u;
                    else if (pos == p) kv = (0xffffffffu << IB) | low;
                    else kv = (orderable(s_score[rl * SSTR + pos]) & ~IMASK) | low;
                    key[q][r] = kv;
                }
            }
            // the rows' query norms, loaded while the keys are ranked
            float qn[RR];
#pragma unroll
            for (int q = 0; q < RR; ++q) qn[q] = qnrm[min(p0 + r0 + q, g.n_cand - 1)];
            // the k-th and (k + 1)-th largest key of each row (radix ranking)
            uint32_t kth[RR], next[RR];
            if constexpr (RADIX) {
                // the wavefront's keep rows serve as its radix counters until
                // they are cleared below
                uint32_t* hist = (uint32_t*)&s_keep[wave][0][0];
#pragma unroll
                for (int q = 0; q < RR; ++q) {
                    const int p = p0 + r0 + q;
                    const uint32_t diag = (0xffffffffu << IB) | (IMASK - (uint32_t)p);
                    kth[q] = 1u;                        // k >= n_cand: every candidate (keys > 0)
                    next[q] = 0u;
                    if (r0 + q >= rows || g.k >= g.n_cand) continue;
                    if (g.k == 1) { kth[q] = diag; continue; }
                    // the other candidates: neither padding (0) nor the diagonal
                    bool part[E];
#pragma unroll
                    for (int r = 0; r < E; ++r) part[r] = key[q][r] != 0u && key[q][r] < (0xffffffffu << IB);
                    kth[q] = wave_kth_key<E, RADIX_DB>(key[q], part, g.k - 1, lane, hist);
                    uint32_t below = 0u;
#pragma unroll
                    for (int r = 0; r < E; ++r) below = key[q][r] < kth[q] ? max(below, key[q][r]) : below;
                    next[q] = __builtin_amdgcn_readfirstlane(wave_max_u32(below));
                }
            } else {
                wave_bitonic_desc32<RR, E>(key, lane);
            }
#pragma unroll
            for (int q = 0; q < RR; ++q)
#pragma unroll
                for (int r = 0; r < E; ++r) s_keep[wave][q][lane * E + r] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < RR; ++q) {
                if (r0 + q >= rows) continue;
                // the float32 score of a key (its candidate position in the low bits)
                auto score_of = [&](uint32_t kv) -> float {
                    return s_score[(r0 + q) * SSTR + (int)(IMASK - (kv & IMASK))];
                };
                // the key at a rank of the sorted keys
                auto key_at = [&](int rank) -> uint32_t {
                    uint32_t kv = 0u;
#pragma unroll
                    for (int r = 0; r < E; ++r)
                        if (r == rank % E) kv = key[q][r];
                    return __builtin_amdgcn_readlane(kv, rank / E);
                };
                // the kept bits of a 32-bit key resolve scores to 2^-(23 - IB)
                if constexpr (RADIX)
                    select_row([&]() { return score_of(kth[q]); }, [&]() { return score_of(next[q]); },
                               [&](int r) { return key[q][r] >= kth[q]; },
                               [&](int r) { return lane * E + r; },
                               p0 + r0 + q, r0 + q, 23 - IB, qn[q], s_keep[wave][q]);
                else
                    select_row([&]() { return score_of(key_at(g.k - 1)); }, [&]() { return score_of(key_at(g.k)); },
                               [&](int r) { return lane * E + r < g.k; },
                               [&](int r) { return (int)(IMASK - (key[q][r] & IMASK)); },
                               p0 + r0 + q, r0 + q, 23 - IB, qn[q], s_keep[wave][q]);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < RR; ++q)
                if (r0 + q < rows) compact_sparse(p0 + r0 + q, s_keep[wave][q]);
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        // ---- 64-bit keys, one row at a time
        for (int rl = sub * RQ + wave * RPW; rl < sub * RQ + wave * RPW + RPW; ++rl) {
            if (rl >= rows) break;
            const int p = p0 + rl;
            uint64_t key[E];
#pragma unroll
            for (int r = 0; r < E; ++r) {
                const int pos = lane * E + r;
                const uint32_t low = 0xffffffffu - (uint32_t)pos;
                if (pos >= g.n_cand) key[r] = 0ull;
                else if (pos == p) key[r] = (0xffffffffull << 32) | low;
                else key[r] = ((uint64_t)orderable(s_score[rl * SSTR + pos]) << 32) | low;
            }
            const float qn = qnrm[p];
            wave_bitonic_desc<E>(key, lane);
#pragma unroll
            for (int r = 0; r < E; ++r) s_keep[wave][0][lane * E + r] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            auto score_at = [&](int rank) -> float {
                uint64_t kv = 0ull;
#pragma unroll
                for (int r = 0; r < E; ++r)
                    if (r == rank % E) kv = key[r];
                const uint32_t lo32 = __builtin_amdgcn_readlane((uint32_t)kv, rank / E);
                return s_score[rl * SSTR + (int)(0xffffffffu - lo32)];
            };
            select_row([&]() { return score_at(g.k - 1); }, [&]() { return score_at(g.k); },
                       [&](int r) { return lane * E + r < g.k; },
                       [&](int r) { return (int)(0xffffffffu - (uint32_t)key[r]); },
                       p, rl, 0, qn, s_keep[wave][0]);
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            compact_sparse(p, s_keep[wave][0]);
            __builtin_amdgcn_wave_barrier();
        }
    }

    // ---- this workgroup's share of the PINNED and DROPPED rows
    for (int t = (tile * SPLITS + sub) * WAVES + wave; t < g.n_other; t += n_tiles * SPLITS * WAVES) {
        const int32_t i = other_block(g, t);
        const int32_t cls = block_class(g, i);
        compact_row(g, codes, vec4, lane, cls == CLS_DROPPED, cls == CLS_PINNED,
                    out.mask + (slice * nb + i) * nb, out.index + (slice * nb + i) * nb,
                    out.count + slice * nb + i, [](int32_t, int32_t) { return false; });
    }
}

// ---------------------------------------------------------------------------
// K3: layout-only masks.  Each SPARSE row keeps the k candidates nearest the
// diagonal by (|i - j|, j) — a contiguous run of candidate positions — plus
// the window; k = n_cand gives the dense (layout-only) mask.  grid.y = slice.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void layout_kernel(Geometry g, MaskOut out, int H, const uint8_t* head_mask) {
    __shared__ __attribute__((aligned(8))) int16_t s_code[kCodeTable];
    const int16_t* codes = fill_codes(g, s_code);
    __syncthreads();
    const bool vec4 = (g.nb & 3) == 0 && ((uintptr_t)out.mask & 3u) == 0;
    const int lane = threadIdx.x & 63;
    const int32_t i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= g.nb) return;
    const int64_t slice = blockIdx.y;
    const int64_t nb = g.nb;
    const int32_t code_i = column_code(g, i);

    // The k nearest candidates by (|i - j|, j) are the run of candidate
    // positions [lo, lo + k) that holds the diagonal p.  Against the run one
    // step to the right it trades candidate lo for lo + k, and the right one
    // is better exactly when lo + k is strictly nearer; along lo that test
    // flips once from true to false, so lo is the first position where it is
    // false (binary search, wave-uniform).
    int32_t lo = 0, kk = g.n_cand;
    if (code_i >= 0 && !g.is_dense) {
        kk = g.k;
        const int32_t p = code_i;
        int32_t a = max(0, p - kk + 1), b = min(p, g.n_cand - kk);   // lo in [a, b]
        while (a < b) {
            const int32_t m = (a + b) >> 1;
            const bool right = (cand_block(g, m + kk) - i) < (i - cand_block(g, m));
            if (right) a = m + 1; else b = m;
        }
        lo = a;
    }
    const int32_t w = g.w;
    // every row of a masked head is empty
    const bool head_off = head_mask != nullptr && head_mask[slice % H] == 0;
    compact_row(g, codes, vec4, lane, code_i == -2 || head_off, code_i == -1, out.mask + (slice * nb + i) * nb,
                out.index + (slice * nb + i) * nb, out.count + slice * nb + i,
                [&](int32_t j, int32_t code) {
                    return (code >= lo && code < lo + kk) || (w >= 0 && abs(j - i) <= w);
                });
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_pool_t(int block, TView q, TView k, int B, int H, int Hkv,
                                const Geometry& g, PooledSums qp, PooledSums kp, int xcd_groups,
                                const uint8_t* hmask, hipStream_t s) {
    const int64_t items = (int64_t)B * ((qp.hi == nullptr ? 0 : H) + Hkv) * g.n_cand;
    const int64_t wgs = (items + 3) / 4;
    const dim3 grid((unsigned)(xcd_groups ? (wgs + kNumXcd - 1) / kNumXcd * kNumXcd : wgs));
    if (block == 64)
        return launch(pool_kernel<T, D, 64>, grid, dim3(256), s, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask);
    return launch(pool_kernel<T, D, 32>, grid, dim3(256), s, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask);
}

hipError_t launch_pool(int dtype_is_f32, int D, int block, TView q, TView k, int B, int H,
                       int Hkv, const Geometry& g, PooledSums qp, PooledSums kp, int xcd_groups,
                       const uint8_t* hmask, hipStream_t s) {
    if (dtype_is_f32) {
        if (D == 32) return launch_pool_t<float, 32>(block, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask, s);
        if (D == 64) return launch_pool_t<float, 64>(block, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask, s);
        return launch_pool_t<float, 128>(block, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask, s);
    }
    if (D == 32) return launch_pool_t<uint16_t, 32>(block, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask, s);
    if (D == 64) return launch_pool_t<uint16_t, 64>(block, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask, s);
    return launch_pool_t<uint16_t, 128>(block, q, k, B, H, Hkv, g, qp, kp, xcd_groups, hmask, s);
}

template <int D, int E>
static hipError_t launch_score_t(PooledSums qp, PooledSums kp, int B, int H, int Hkv,
                                 const Geometry& g, MaskOut out, int xcd_groups, const uint8_t* hmask,
                                 hipStream_t s) {
    constexpr int RT = RankShape<D, E>::RT;
    const int n_tiles = (g.n_cand + RT - 1) / RT;
    const int64_t wgs = (int64_t)B * H * n_tiles * (RT / RankShape<D, E>::RQ);
    const dim3 grid((unsigned)(xcd_groups ? (wgs + kNumXcd - 1) / kNumXcd * kNumXcd : wgs));
    return launch(score_rank_kernel<D, E>, grid, dim3(RankShape<D, E>::WAVES * 64), s, qp, kp, B, H, Hkv, g,
                  out, n_tiles, xcd_groups, hmask);
}

template <int D>
static hipError_t launch_score_d(PooledSums qp, PooledSums kp, int B, int H, int Hkv,
                                 const Geometry& g, MaskOut out, int xg, const uint8_t* hm, hipStream_t s) {
    const int n = g.n_cand;
    if (n <= 64) return launch_score_t<D, 1>(qp, kp, B, H, Hkv, g, out, xg, hm, s);
    if (n <= 128) return launch_score_t<D, 2>(qp, kp, B, H, Hkv, g, out, xg, hm, s);
    if (n <= 256) return launch_score_t<D, 4>(qp, kp, B, H, Hkv, g, out, xg, hm, s);
    if (n <= 512) return launch_score_t<D, 8>(qp, kp, B, H, Hkv, g, out, xg, hm, s);
    if (n <= 1024) return launch_score_t<D, 16>(qp, kp, B, H, Hkv, g, out, xg, hm, s);
    return launch_score_t<D, 32>(qp, kp, B, H, Hkv, g, out, xg, hm, s);
}

hipError_t launch_score_rank(int D, PooledSums qp, PooledSums kp, int B, int H, int Hkv,
                             const Geometry& g, MaskOut out, int xcd_groups, const uint8_t* hmask,
                             hipStream_t s) {
    if (D == 32) return launch_score_d<32>(qp, kp, B, H, Hkv, g, out, xcd_groups, hmask, s);
    if (D == 64) return launch_score_d<64>(qp, kp, B, H, Hkv, g, out, xcd_groups, hmask, s);
    return launch_score_d<128>(qp, kp, B, H, Hkv, g, out, xcd_groups, hmask, s);
}

hipError_t launch_layout_fill(const Geometry& g, int slices, int H, const uint8_t* hmask, MaskOut out,
                              hipStream_t s) {
    const dim3 grid((unsigned)((g.nb + 3) / 4), (unsigned)slices);
    return launch(layout_kernel, grid, dim3(256), s, g, out, H, hmask);
}

}  // namespace bsattn
