// Block-sparse attention forward, bf16 MFMA path (gfx950).
//
// One workgroup per (b, h, 64-token query block).  A pair of wavefronts
// covers the 64 query rows (32 each); with SPLIT = 2 a second pair covers
// the same rows over the other half of the keys -- at D = 64 the second 32
// keys of every kept key block, at D = 128 every other kept block -- and the
// two partial softmax states are merged at the end.
// Each pair walks the compacted list of kept key blocks (CSR-like, ascending)
// in stages of KT keys:
//   - K and V stage tiles go from HBM/L2 straight into LDS with
//     buffer_load_dwordx4 ... lds (no register staging): V two stages deep, K
//     one, and the next K tile loads as soon as every wavefront has read
//     this stage's K fragments (two barriers per stage, neither of which
//     waits for tiles still in flight);
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with the Q^T fragments held in
//     VGPRs for the whole loop;
//   - online softmax in fp32: exp2 with the scale folded into log2 units,
//     exponentials taken against the running row maximum, which is raised
//     (and the running output rescaled) only on a row's first live stage or
//     when a stage's exponentials sum past 2^16; exact after the final
//     division, so the row maximum is not computed on most stages;
//   - O^T += V^T P^T with the V^T fragments read by ds_read_b64_tr_b16 from
//     the row-major V tile, so V is never transposed in memory.
// Every lane holds one query's scores and one query's output column; the
// softmax statistics of a row live in the lane pair (lane, lane ^ 32).  K rows
// feed the MFMA row slots in a fixed permutation so that each lane's eight P
// values of a 16-key step are consecutive keys — the B-operand layout of the
// P V product — so P never moves between lanes.
// LDS tiles use an XOR swizzle of 16-byte chunks, chosen so that both the
// 16-byte K fragment reads and the transposing V reads are free of bank
// conflicts.  The kept-block indices are read with scalar loads.  Masked
// heads and rows without kept blocks write zeros and exit.
//
// Sources: SD.Next commit view, modules/attention/sparse, flex-consumer
// paragraph (only the selected tiles are computed); inferensys glossary,
// block-sparse entry; haagenti_sparse crate docs (heads skipped under a
// per-layer mask).
#include "common.h"
#include "internal.h"
#include "rank.h"

// 1: workgroups of the query heads sharing a K/V head are neighbours
#ifndef BSATTN_GQA_ORDER
#define BSATTN_GQA_ORDER 1
#endif
// 1: two query heads of a K/V group share stage tiles when their lists agree
// (video length, 24 query heads on 6 K/V heads, radial mask: 4.17 -> 3.91 ms)
#ifndef BSATTN_GQA_SHARE
#define BSATTN_GQA_SHARE 1
#endif
// 1: with two key-block groups of 32-key stages, group g takes the 32-key
// half g of every kept block (rather than every other kept block), so both
// groups run exactly one stage per kept block whatever its count
#ifndef BSATTN_HALVES
#define BSATTN_HALVES 1
#endif
// 1: a wavefront's issue priority falls as its workgroup progresses
#ifndef BSATTN_PRIO
#define BSATTN_PRIO 1
#endif

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef short s4v __attribute__((ext_vector_type(4)));
typedef short s8v __attribute__((ext_vector_type(8)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));


// MFMA row slot -> key within a 32-key tile.
__device__ __forceinline__ int slot_key(int s) {
    const int q = s >> 3, hh = (s >> 2) & 1, r = s & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + r;
}

// XOR swizzle of the 16-byte chunks of LDS row r (see the header comment).
template <int D>
__device__ __forceinline__ int chunk_swizzle(int r) {
    if constexpr (D == 64) {
        const int m = (r >> 1) & 7;
        return ((m & 1) << 2) | (m >> 1);
    } else {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    }
}

// Two floats to packed bf16 (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf2v to_bf16x2(float lo, float hi) {
    return __builtin_convertvector((f2v){lo, hi}, bf2v);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, to_bf16x2(lo, hi));
}

__device__ __forceinline__ int g16_of(int lane) { return lane >> 4; }

// max / sum of x over the lane pair (l, l ^ 32).  v_permlane32_swap (gfx950)
// exchanges the two 32-lane halves in the VALU, without the LDS crossbar
// round trip of ds_bpermute: of the pair it returns, one element is x and the
// other the partner's x, in either order.
__device__ __forceinline__ float pair_max32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS stages.  __syncthreads() also waits for
// every vector-memory operation of the wave (vmcnt 0), and the LDS-DMA stage
// loads count there, so a barrier in mid-stage would wait for the next
// stage's tiles too.  Here the wave's own LDS reads complete first (the
// buffer a stage frees may be overwritten once every wave is past the
// barrier), the compiler may not move memory accesses across it, and the
// tile loads are waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS stage buffering of the attention kernel: both K and V double-buffered,
// V single (loaded after a stage's first barrier, waited for before P V), or
// K single (the next stage's K is loaded once every wavefront holds this
// stage's K fragments in registers).
enum StageBuf { BUF_KV2 = 0, BUF_V1 = 1, BUF_K1 = 2 };

// SPLIT key-block groups per workgroup: group g (wavefronts 2g, 2g + 1)
// takes keys 32 g .. 32 g + 31 of every kept block at D = 64 (HALVES: both
// groups run one 32-key stage per kept block), else the kept blocks at list
// positions g, g + SPLIT, g + 2 SPLIT, ...;
// each group has its own LDS stages, and the groups' partial softmax states
// are merged through LDS at the end.  More wavefronts per query block hide
// more latency when the grid alone cannot fill the chip.
//
// SHARE (query heads of a K/V group with one shared block mask): the two
// wavefront pairs are two query heads of the same K/V head and query block
// instead of two key-block groups.  They walk the same kept list, so each
// K/V stage tile is loaded into LDS once (by all four wavefronts) and read
// by both heads; there is no merge, each pair writes its own head.
// FUSED (bsattn_select_forward; D 64, every block of the sequence a candidate,
// at most 64 of them): the workgroup ranks its own row from its query block's
// sum and the selector's pooled key sums, both in float64 -- the selector's
// 32-bit keys and wavefront bitonic sort: the diagonal first, then by score
// with ties to the lower block, resolved to 2^-17 relative -- keeps the top
// `keep`, writes the row's mask, count and ascending index list, and leaves
// the list in LDS for the stage loop.  The NW wavefronts share the float64
// work: wavefront w sums query rows [DW w, DW w + DW) (DW = 64 / NW) and
// scores every candidate over dimensions [DW w, DW w + DW), its query and
// key-sum loads issued together; the partial sums meet in LDS (`part`: 2 NW
// x 64 doubles, free until the first stage tiles are requested) in a fixed
// wavefront order, and wavefront 0 ranks and compacts.  Sums of 64 bf16
// values are exact in float64 short of extreme exponent spreads, so the
// query sum is then the pooled one whatever the order.
template <int NW>
__device__ __forceinline__ void fused_rank_row(const AttnArgs& a, int b, int h, int kvh, int qb, int wave, int lane,
                                               int32_t* s_list, uint8_t* s_flag, double* part) {
    constexpr uint32_t IMASK = 63u;           // 64 candidate positions
    constexpr int DW = 64 / NW;               // query rows and dimensions per wavefront
    static_assert(64 % NW == 0 && DW % 8 == 0, "row and dimension shares");
    const int n = a.nkb;
    const int64_t krow0 = ((int64_t)b * a.Hkv + kvh) * a.prow * 64;
    double* qpart = part;                     // [NW][64] partial query sums
    double* spart = part + NW * 64;           // [NW][64] partial scores
    // this wavefront's query rows: lane reads chunk lane % 8 (dimensions
    // 8 (lane % 8) ..) of rows DW wave + lane / 8 + 8 l
    uint4 raw[DW / 8];
    {
        const uint16_t* qsrc = (const uint16_t*)a.q.p + b * a.q.sb + h * a.q.sh +
                               ((int64_t)qb * 64 + DW * wave + lane / 8) * a.q.sn + (lane % 8) * 8;
#pragma unroll
        for (int l = 0; l < DW / 8; ++l) raw[l] = *(const uint4*)(qsrc + (int64_t)l * 8 * a.q.sn);
    }
    // key sums (hi, lo) of candidate `lane` over this wavefront's dimensions;
    // lanes past the candidates read row 0 (in bounds, unused)
    float4 kh[DW / 4], kl[DW / 4];
    {
        const int cand = lane < n ? lane : 0;
#pragma unroll
        for (int m = 0; m < DW / 4; ++m) {
            const int64_t o = krow0 + pooled_offset<64>(cand, DW * wave + 4 * m);
            kh[m] = *(const float4*)(a.kp + o);
            kl[m] = *(const float4*)(a.kp_lo + o);
        }
    }
    {
        double qs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[e] = 0.0;
#pragma unroll
        for (int l = 0; l < DW / 8; ++l) {
            const uint32_t w[4] = {raw[l].x, raw[l].y, raw[l].z, raw[l].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qs[2 * e] += (double)__uint_as_float(w[e] << 16);
                qs[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int off = 8; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) qs[e] += lane_xor_f64(qs[e], off);
        if (lane < 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qpart[wave * 64 + 8 * lane + e] = qs[e];
        }
    }
    lds_barrier();                            // every partial query sum in LDS
    {
        double sc = 0.0;
#pragma unroll
        for (int m = 0; m < DW / 4; ++m) {
            double qd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = DW * wave + 4 * m + e;
                qd[e] = qpart[d];
#pragma unroll
                for (int w = 1; w < NW; ++w) qd[e] += qpart[w * 64 + d];
            }
            sc = fma(qd[0], (double)kh[m].x + (double)kl[m].x, sc);
            sc = fma(qd[1], (double)kh[m].y + (double)kl[m].y, sc);
            sc = fma(qd[2], (double)kh[m].z + (double)kl[m].z, sc);
            sc = fma(qd[3], (double)kh[m].w + (double)kl[m].w, sc);
        }
        spart[wave * 64 + lane] = sc;
    }
    lds_barrier();                            // every partial score in LDS
    if (wave != 0) return;
    // float64 score of the lane's candidate, rounded to float32 for the
    // 32-bit key: the ranking follows the exact block-mean scores up to 2^-17
    // relative
    uint32_t key[1][1] = {{0u}};
    if (lane < n) {
        if (lane == qb) {
            key[0][0] = (0xffffffffu & ~IMASK) | (IMASK - (uint32_t)lane);
        } else {
            double sc = spart[lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) sc += spart[w * 64 + lane];
            key[0][0] = (orderable((float)sc) & ~IMASK) | (IMASK - (uint32_t)lane);
        }
    }
    wave_bitonic_desc32<1, 1>(key, lane);          // lane r: the key of rank r
    s_flag[lane] = 0;
    s_list[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < a.keep) s_flag[IMASK - (key[0][0] & IMASK)] = 1;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const bool kept = lane < n && s_flag[lane] != 0;
    const uint64_t bal = __ballot(kept);
    const int slot = __popcll(bal & ((1ull << lane) - 1ull));
    if (kept) s_list[slot] = lane;
    if (a.m_out != nullptr) {
        const int64_t row = ((int64_t)b * a.H + h) * a.nqb + qb;
        if (lane < n) a.m_out[row * n + lane] = kept ? 1 : 0;
        if (kept) a.i_out[row * n + slot] = lane;
        if (lane == 0) a.c_out[row] = __popcll(bal);
    }
}

template <int D, int KT, int SPLIT, int WPE, int BUF, bool KMASK, bool SHARE, bool FUSED = false>
__global__ __launch_bounds__(128 * SPLIT) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void attn_mfma_kernel(AttnArgs a) {
    constexpr int BLK = 64;
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int NT = 128 * SPLIT;          // threads per workgroup
    constexpr int LT = SHARE ? NT : 128;     // threads loading one stage tile
    constexpr int NI = KT * CPR / LT;        // loads per thread per tensor per stage
    constexpr int GT = SHARE ? 1 : SPLIT;    // stage tiles per LDS object
    constexpr int TILE = KT * D;             // bf16 elements per K (or V) stage tile
    constexpr int NKT = KT / 32;             // 32-key S^T tiles per stage
    constexpr int NKS = D / 16;              // k-steps of S^T
    constexpr int NDT = D / 32;              // 32-row d tiles of O^T
    constexpr int NPS = KT / 16;             // 16-key steps of O^T per stage
    constexpr int SUB = BLK / KT;            // stages per key block
    constexpr float kSumCap = 65536.0f;      // largest stage sum of exponentials kept per lane
    constexpr float kTau = 8.0f;             // key-mask variant: lazy-rescale threshold (log2 units)
    static_assert(NI >= 1 && KT * CPR % LT == 0, "stage tiling");
    static_assert(!SHARE || SPLIT == 2, "two query heads per workgroup");
    static_assert(SPLIT == 1 || SPLIT == 2, "one or two key-block groups");
    static_assert(SPLIT == 1 || SPLIT * TILE * 2 >= D * 128, "merge buffer fits in one stage object");
    static_assert(!KMASK || KT == 32, "key-mask words cover one 32-key stage");
    static_assert(!FUSED || (D == 64 && !SHARE && !KMASK), "fused selection: D 64, per-head path");

    // one LDS object per stage (holding every group's tile): distinct objects
    // let the compiler see that the reads of one stage never alias the loads
    // in flight into the other
    __shared__ __attribute__((aligned(16))) uint16_t K0[GT * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t V0[GT * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t K1[BUF == BUF_K1 ? 8 : GT * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t V1[BUF == BUF_V1 ? 8 : GT * TILE];
    static_assert((TILE * 2) % (D * 2) == 0, "tiles hold whole rows");

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    // the grid is padded to a multiple of the XCD count: padding workgroups
    // exit here (SHARE: one workgroup per pair of query heads, so half the
    // (b, head, query block) items)
    if (a.head_mask == nullptr && L >= (SHARE ? a.n_work / 2 : a.n_work)) return;
    // work order (b, kv head, query block, query head within the group): the
    // query heads that share one K/V head run the same query block on
    // neighbouring workgroups of one XCD, so their K/V tiles meet in its L2
    // (the XCD-grouped ids keep neighbours together).  With one query head
    // per K/V head this is the plain (b, h, query block) order.
    // Under a head mask the active heads' query blocks come first instead,
    // so that the work the mask keeps spreads evenly over the XCDs.
    int32_t qb, h, b;
    bool active = true;
    if constexpr (SHARE) {
        // (b, kv head, query block, pair of query heads); the pair's second
        // head is taken by wavefronts 2 and 3
        const int32_t rep = a.H / a.Hkv;
        const int32_t hp = (int32_t)(L % (rep / 2));
        const int64_t rest = L / (rep / 2);
        qb = (int32_t)(rest % a.nqb);
        const int64_t bg = rest / a.nqb;
        b = (int32_t)(bg / a.Hkv);
        h = (int32_t)(bg % a.Hkv) * rep + 2 * hp + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 7));
    } else if (a.head_mask != nullptr) {
        const HeadWork hw = head_masked_order(blockIdx.x, gridDim.x, a.head_mask, a.B, a.H, a.nqb);
        if (!hw.valid) return;
        qb = hw.qb, h = hw.h, b = hw.b, active = hw.active;
    } else {
#if BSATTN_GQA_ORDER
        const int32_t rep = a.H / a.Hkv;
        const int32_t hr = (int32_t)(L % rep);
        const int64_t rest = L / rep;
        qb = (int32_t)(rest % a.nqb);
        const int64_t bg = rest / a.nqb;
        b = (int32_t)(bg / a.Hkv);
        h = (int32_t)(bg % a.Hkv) * rep + hr;
#else
        qb = (int32_t)(L % a.nqb);
        const int64_t bh = L / a.nqb;
        h = (int32_t)(bh % a.H);
        b = (int32_t)(bh / a.H);
#endif
    }
    const int32_t kvh = h / (a.H / a.Hkv);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 1;               // key-block group (SHARE: query head of the pair)
    const int wq = wave & 1;                 // query rows 32*wq .. 32*wq + 31
    const int gtid = tid & 127;              // thread within the group
    const int ltid = SHARE ? tid : gtid;     // thread within the tile's loaders
    const int gofs = SHARE ? 0 : grp * TILE; // the group's tile within a stage object
    const int hl = lane >> 5, ql = lane & 31;

    // Q^T fragments: lane holds Q[32*wq + ql][16*ks + 8*hl + 0..7].  Without
    // the fused ranking they are requested before the kept-block count and
    // list are waited for, so the two memory round trips of a workgroup's
    // start overlap instead of following each other.
    const uint16_t* qbase = (const uint16_t*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qb * BLK * a.q.sn;
    bf16x8 qf[NKS];
    auto load_q = [&]() {
        const uint16_t* qr = qbase + (int64_t)(32 * wq + ql) * a.q.sn + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qr + 16 * ks);
    };
    if constexpr (!FUSED) {
        if (active) load_q();
    }

    int32_t cnt = a.nkb;
    const int32_t* list = nullptr;
    // HALVES: the two groups split every kept block (the first half to group
    // 0, the second to group 1) instead of taking alternate blocks.  At D = 64
    // (SDXL: 19 kept blocks, 20 stages per group with alternate blocks, 19
    // with halves) 37.5 against 38.6 us; at D = 128 the halves measured
    // 0.5-0.8 % slower (joint, video, stack), so there the groups alternate.
    constexpr bool HALVES = BSATTN_HALVES && !SHARE && SPLIT == 2 && SUB == 2 && D == 64;
    int32_t blk0 = SHARE || HALVES ? 0 : grp;   // the group's first key block
    if (a.count != nullptr) {
        const int64_t ms = (int64_t)(a.mB == 1 ? 0 : b) * a.mH + (a.mH == 1 ? 0 : h);
        cnt = a.count[ms * a.nqb + qb];
        list = a.index + (ms * a.nqb + qb) * (int64_t)a.nkb;
        // read together with the count rather than after it (an entry of the
        // row either way; unused when the group has no block)
        blk0 = ((const __attribute__((address_space(4))) int32_t*)list)[!SHARE && !HALVES && grp < a.nkb ? grp : 0];
    }
    __shared__ int32_t s_list[FUSED ? 64 : 1];
    __shared__ uint8_t s_flag[FUSED ? 64 : 1];
    if constexpr (FUSED) {
        // the ranking's partial sums use the second V stage buffer, whose
        // first tile is requested only at stage 0's first barrier
        static_assert(BUF == BUF_K1 && 2 * (2 * SPLIT) * 64 * 8 <= GT * TILE * 2, "ranking partials fit in V1");
        fused_rank_row<2 * SPLIT>(a, b, h, kvh, qb, wave, lane, s_list, s_flag, (double*)V1);
        lds_barrier();                       // the list in LDS; the mask row's stores drain meanwhile
        cnt = a.keep;
        blk0 = s_list[HALVES ? 0 : grp];     // unused when the group has no block
    }
    uint16_t* obase = (uint16_t*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qb * BLK * a.o_sn;

    if (!active || cnt <= 0) {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int c = SHARE ? gtid : tid; c < BLK * CPR; c += SHARE ? 128 : NT)
            *(uint4*)(obase + (int64_t)(c / CPR) * a.o_sn + (c % CPR) * 8) = z;
        return;
    }

    const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.sb + kvh * a.k.sh;
    const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.sb + kvh * a.v.sh;
    if constexpr (FUSED) load_q();
    // every group runs the same number of stages (the barriers are
    // workgroup-wide); stages past the group's own blocks only synchronise
    const int T = SHARE ? cnt * SUB : HALVES ? cnt : ((cnt + SPLIT - 1) / SPLIT) * SUB;
    const int Tg = SHARE || HALVES ? T : ((cnt - grp + SPLIT - 1) / SPLIT) * SUB;
    // kept key block of stage t: a scalar (constant address space) load, so
    // waiting for it never waits for the stage loads in flight
    const __attribute__((address_space(4))) int32_t* klist =
        (const __attribute__((address_space(4))) int32_t*)list;
    auto block_of = [&](int t) -> int32_t {
        if constexpr (HALVES) {
            if constexpr (FUSED) return t == 0 ? blk0 : __builtin_amdgcn_readfirstlane(s_list[t]);
            return t == 0 ? blk0 : (list == nullptr ? t : klist[t]);
        }
        const int i = SHARE ? t / SUB : (t / SUB) * SPLIT + grp;
        if constexpr (FUSED) return t < SUB ? blk0 : __builtin_amdgcn_readfirstlane(s_list[i]);
        return t < SUB ? blk0 : (list == nullptr ? i : klist[i]);
    };
    // first key of stage t within its block
    auto half_of = [&](int t) -> int { return HALVES ? grp : t % SUB; };
    // per-thread source offsets of the NI chunks it loads per stage: chunk
    // slot s = i*LT + ltid of the tile holds row s / CPR, global chunk
    // (s % CPR) ^ swizzle
    // Per-lane byte offsets within a stage tile (the tile's first row is the
    // buffer base of its loads).
    uint32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int s = i * LT + ltid;
        const int r = s / CPR;
        const int c = (s % CPR) ^ chunk_swizzle<D>(r);
        koff[i] = (uint32_t)(r * (int32_t)a.k.sn + c * 8) * 2u;
        voff[i] = (uint32_t)(r * (int32_t)a.v.sn + c * 8) * 2u;
    }
    auto issue_tile = [&](const uint16_t* base, int64_t sn, const uint32_t (&off)[NI], int t, uint16_t* dst) {
        const int64_t row0 = (int64_t)block_of(t) * BLK + half_of(t) * KT;
#pragma unroll
        for (int i = 0; i < NI; ++i) chunk_to_lds(base + row0 * sn, off[i], dst + (i * LT + (SHARE ? wave : wq) * 64) * 8);
    };
    // issue the K (or V) loads of stage t into the group's tile at Kd (Vd)
    auto issue_k = [&](int t, uint16_t* Kd) { issue_tile(kbase, a.k.sn, koff, t, Kd); };
    auto issue_v = [&](int t, uint16_t* Vd) { issue_tile(vbase, a.v.sn, voff, t, Vd); };
    // KMASK: lanes 0..31 fetch the mask bytes of the 32 keys of a stage with
    // its K tile (after its V); at the stage a ballot turns them into one
    // wave-uniform 32-bit word.
    const uint8_t* kmbase = KMASK ? a.key_mask + (int64_t)b * a.km_sb : nullptr;
    uint32_t km_next = 1u;
    auto issue_m = [&](int t) {
        if constexpr (KMASK) {
            const int64_t row0 = (int64_t)block_of(t) * BLK + half_of(t) * KT;
            km_next = lane < 32 ? (uint32_t)kmbase[row0 + lane] : 1u;
        }
    };
    // One of K and V may have a single tile per group, which keeps the
    // workgroup's LDS small enough for five (D = 64) or six (D = 128)
    // workgroups per CU.
    //  BUF_V1: V of stage t is loaded after the stage's first barrier (every
    //    wave is past the previous P V) and waited for at a second barrier
    //    before this stage's P V; K is double-buffered.
    //  BUF_K1: the K fragments of stage t are read right after the first
    //    barrier; a second barrier then frees the K tile and K of stage t + 1
    //    is loaded while stage t computes.  V is double-buffered and loaded a
    //    stage ahead, so both tiles have about a whole stage to arrive.
    if (Tg > 0) {
        if constexpr (BUF == BUF_K1) issue_v(0, V0 + gofs);
        issue_m(0);
        issue_k(0, K0 + gofs);
        if constexpr (BUF == BUF_KV2) issue_v(0, V0 + gofs);
    }

    // Per-lane byte offsets of this lane's LDS fragments within a stage
    // object (the group's tile included).  Row bases are multiples of the row
    // size and the swizzle acts on the 16-byte chunk field only, so a
    // fragment further along the contraction (ks) or along d (dt) is the
    // base XOR a constant, and a later 16-key step is the base plus a
    // constant: three registers instead of one address per fragment.
    //   K fragment ks:  kb ^ (32 ks)          (chunk (2ks + hl) ^ swz(r))
    //   V operand (dt, ks): (vb0 ^ (64 dt)) + 32 D ks, and vb1 for rows + 4
    uint32_t kb, vb0, vb1;
    {
        const int r = slot_key(ql);
        kb = (uint32_t)(gofs * 2 + r * D * 2 + 16 * (hl ^ chunk_swizzle<D>(r)));
        const int c0 = 2 * (g16_of(lane) & 1) + ((lane & 3) >> 1);
        const int half = lane & 1;
        const int r0 = 8 * hl + ((lane & 15) >> 2), r1 = r0 + 4;
        vb0 = (uint32_t)(gofs * 2 + r0 * D * 2 + 16 * (c0 ^ chunk_swizzle<D>(r0)) + 8 * half);
        vb1 = (uint32_t)(gofs * 2 + r1 * D * 2 + 16 * (c0 ^ chunk_swizzle<D>(r1)) + 8 * half);
    }

    const float sl2 = a.scale * 1.4426950408889634f;   // scale * log2(e)
    float m_run = -INFINITY, l_run = 0.f;
    f16v oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;

    // one stage: wait for its tiles, make them visible, start the loads of
    // stage t + 1 into the buffers freed by stage t - 1, then compute
    auto stage = [&](int t, const uint16_t* Kt, const uint16_t* Vt, uint16_t* Kn, uint16_t* Vn) {
#if BSATTN_PRIO
        // Issue priority 3, 2, 1, 0 over the four quarters of the workgroup's
        // stages.  The SIMD arbiter otherwise prefers the oldest wavefront:
        // the workgroups of one CU, started together with equal work, then
        // finish one after another and the last ones run at low occupancy.
        // Favouring the least advanced keeps them abreast.
        {
            const int pr = 3 - min(3, (4 * t) / T);
            if (pr == 3) __builtin_amdgcn_s_setprio(3);
            else if (pr == 2) __builtin_amdgcn_s_setprio(2);
            else if (pr == 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
#endif
        wait_vmcnt<0>();
        lds_barrier();
        // this stage's key-mask word (wave-uniform); all ones without KMASK
        uint32_t kw = 0xffffffffu;
        if constexpr (KMASK) kw = (uint32_t)__ballot(km_next != 0u);
        if constexpr (BUF == BUF_V1) {
            if (t < Tg) issue_v(t, V0 + gofs);
            if (t + 1 < Tg) { issue_m(t + 1); issue_k(t + 1, Kn); }
        } else if constexpr (BUF == BUF_K1) {
            if (t + 1 < Tg) issue_v(t + 1, Vn);
        } else if (t + 1 < Tg) {
            issue_m(t + 1);
            issue_k(t + 1, Kn);
            issue_v(t + 1, Vn);
        }
        // no work: past the group's blocks, or every key of the stage masked
        const bool work = t < Tg && !(KMASK && kw == 0u);

        const uint8_t* Kb = (const uint8_t*)Kt;
        const uint8_t* Vb = (const uint8_t*)Vt;
        // S^T = K Q^T for NKT 32-key tiles
        f16v sacc[NKT];
        if (work) {
            bf16x8 kf[NKT][NKS];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    kf[kt][ks] = *(const bf16x8*)(Kb + (kb ^ (uint32_t)(32 * ks)) + 64 * D * kt);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt][ks], qf[ks], sacc[kt], 0, 0, 0);
            }
        }
        if constexpr (BUF == BUF_K1) {
            lds_barrier();   // every wave has read its K fragments: the K tile is free
            if (t + 1 < Tg) { issue_m(t + 1); issue_k(t + 1, Kn); }
        }
        if (!work) {
            if constexpr (BUF == BUF_V1) lds_barrier();   // the stage's second barrier
            return;
        }

        // V^T operands of O^T += V^T P^T.  Within each 16-lane group, lane j
        // supplies V[kb + j/4][d0 + 4*(j%4) .. +3]; lane i then receives
        // V[kb + 0..3][d0 + i].
        auto v_operand = [&](int dt, int ks) -> bf16x8 {
            const uint32_t o0 = (vb0 ^ (uint32_t)(64 * dt)) + 32 * D * ks;
            const uint32_t o1 = (vb1 ^ (uint32_t)(64 * dt)) + 32 * D * ks;
            const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(Vb + o0));
            const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(Vb + o1));
            const s8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, both);
        };

        if constexpr (KMASK) {
            // masked keys of a partly masked stage: -inf scores.  Element r of
            // lane half hl holds key (r & 7) | (hl << 3) | ((r >> 3) << 4).
            if (kw != 0xffffffffu) {
                const uint32_t wl = kw >> (8 * hl);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!((wl >> ((r & 7) | ((r >> 3) << 4))) & 1u)) sacc[0][r] = -INFINITY;
            }
        }

        // Online softmax.  P = exp2(S * scale * log2(e) - m_run) in bf16, packed
        // as the B operand of P V (one per 16-key step); the stage's row sums
        // come from bf16 dot products of the same packed values.
        bf16x8 pf[NPS];
        const bf2v one2 = {(__bf16)1.f, (__bf16)1.f};
        auto make_p = [&]() -> float {
            float psum2[2] = {0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf2v w[4];
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * u + e], sl2, -m_run));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * u + e + 1], sl2, -m_run));
                        w[e >> 1] = to_bf16x2(p0, p1);
                        psum2[(e >> 1) & 1] =
                            __builtin_amdgcn_fdot2_f32_bf16(w[e >> 1], one2, psum2[(e >> 1) & 1], false);
                    }
                    pf[2 * kt + u] = __builtin_bit_cast(
                        bf16x8, (uint4){__builtin_bit_cast(uint32_t, w[0]), __builtin_bit_cast(uint32_t, w[1]),
                                        __builtin_bit_cast(uint32_t, w[2]), __builtin_bit_cast(uint32_t, w[3])});
                }
            return psum2[0] + psum2[1];
        };
        // Exact step: the row maximum of the stage (a tree of three-input
        // maxima, then the lane pair), the running maximum raised to it, and
        // the running sum and output rescaled by exp2(old - new).
        auto stage_max = [&]() -> float {
            float mk[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                const f16v& x = sacc[kt];
                const float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
                const float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
                const float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
                mk[kt] = fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15]));
            }
#pragma unroll
            for (int kt = 1; kt < NKT; ++kt) mk[0] = fmaxf(mk[0], mk[kt]);
            return pair_max32(mk[0]) * sl2;
        };
        auto rescale = [&](float m_new) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -inf
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        };
        auto raise_max = [&]() { rescale(fmaxf(m_run, stage_max())); };
        // The running maximum is only raised when it must be.  A row's first
        // live stage takes the exact step.  Later stages exponentiate against
        // the current maximum and check the lane's stage sum: at most kSumCap
        // (every exponential <= kSumCap, so the fp32 sums and outputs stay far
        // from overflow; their relative precision does not depend on the
        // scale) keeps the values, otherwise (a score far above the running
        // maximum, an overflow to inf included) the stage takes the exact step
        // and exponentiates again.  Each branch is wave-uniform.
        // The key-mask variant takes the exact step on every stage (raising
        // the maximum only when it grows by more than 2^kTau): holding S for a
        // second pass would cost it a workgroup per CU at D = 64.
        float ps;
        if constexpr (KMASK) {
            const float mx = stage_max();
            const bool grow = mx > m_run + kTau;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) rescale(grow ? mx : m_run);   // wave-uniform
            ps = make_p();
        } else if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0) {
            raise_max();
            ps = make_p();
        } else {
            ps = make_p();
            if (__builtin_amdgcn_ballot_w64(ps > kSumCap) != 0) {
                raise_max();
                ps = make_p();
            }
        }
        l_run += ps;

        if constexpr (BUF == BUF_V1) {
            // this stage's V has landed; the next stage's K may still fly
            if (t + 1 < Tg) wait_vmcnt<NI>();
            else wait_vmcnt<0>();
            lds_barrier();
        }

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int ks = 0; ks < NPS; ++ks) {
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(dt, ks), pf[ks], oacc[dt], 0, 0, 0);
            }
    };
    for (int t = 0; t < T; t += 2) {
        if constexpr (BUF == BUF_K1) {
            stage(t, K0, V0, K0 + gofs, V1 + gofs);
            if (t + 1 < T) stage(t + 1, K0, V1, K0 + gofs, V0 + gofs);
        } else {
            stage(t, K0, V0, K1 + gofs, (BUF == BUF_V1 ? V0 : V1) + gofs);
            if (t + 1 < T) stage(t + 1, K1, BUF == BUF_V1 ? V0 : V1, K0 + gofs, V0 + gofs);
        }
    }

    if constexpr (SPLIT == 2 && !SHARE) {
        // merge: group 1 leaves its (O, m, l) in LDS, group 0 rescales both
        // partial states to the larger running maximum and adds them.  No
        // stage load is in flight here (the last stage waited for all).
        __syncthreads();
        float* po = (float*)(wq == 0 ? K0 : V0);        // [NDT * 16][64 lanes]
        float* pml = (float*)(BUF == BUF_K1 ? V1 : K1) + wq * 128;   // m [64 lanes], l [64 lanes]
        if (grp == 1) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) po[(dt * 16 + r) * 64 + lane] = oacc[dt][r];
            pml[lane] = m_run;
            pml[64 + lane] = l_run;
        }
        __syncthreads();
        if (grp == 1) return;
        // group 0 always has at least one block, so m_run is finite; a group 1
        // without blocks has m = -inf and contributes exp2(-inf) = 0
        const float m1 = pml[lane], l1 = pml[64 + lane];
        const float m = fmaxf(m_run, m1);
        // with a key mask a group (or both) may have seen no live key: m = -inf
        const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] = oacc[dt][r] * a0 + po[(dt * 16 + r) * 64 + lane] * a1;
        l_run = l_run * a0 + l1 * a1;
    }

    // normalise and store: oacc[dt][r] = O[query][32*dt + 8*(r/4) + 4*hl + r%4]
    const float l_tot = pair_sum32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // 0: every kept key masked
    uint16_t* orow = obase + (int64_t)(32 * wq + ql) * a.o_sn;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            uint2 w;
            w.x = pack_bf16x2(oacc[dt][4 * j4] * inv, oacc[dt][4 * j4 + 1] * inv);
            w.y = pack_bf16x2(oacc[dt][4 * j4 + 2] * inv, oacc[dt][4 * j4 + 3] * inv);
            *(uint2*)(orow + 32 * dt + 8 * j4 + 4 * hl) = w;
        }
}

// Launch shapes per head dim: keys per LDS stage, key-block groups per
// workgroup, waves per EU, stage buffering.  Chosen by measured sweeps.
#ifndef BSATTN_D64_KT
#define BSATTN_D64_KT 32
#endif
#ifndef BSATTN_D64_SPLIT
#define BSATTN_D64_SPLIT 2
#endif
#ifndef BSATTN_D64_WPE
#define BSATTN_D64_WPE 5
#endif
#ifndef BSATTN_D64_KM_WPE
#define BSATTN_D64_KM_WPE 4
#endif
#ifndef BSATTN_D64_BUF
#define BSATTN_D64_BUF BUF_K1
#endif
#ifndef BSATTN_D128_BUF
#define BSATTN_D128_BUF BUF_K1
#endif
#ifndef BSATTN_D128_KT
#define BSATTN_D128_KT 32
#endif
#ifndef BSATTN_D128_SPLIT
#define BSATTN_D128_SPLIT 2
#endif
#ifndef BSATTN_D128_KM_WPE
#define BSATTN_D128_KM_WPE 2
#endif
#ifndef BSATTN_D128_WPE
#define BSATTN_D128_WPE 3
#endif

template <bool KMASK, bool SHARE>
static hipError_t launch_attn_mfma_t(const AttnArgs& a, int D, hipStream_t s) {
    const dim3 grid((unsigned)attn_grid(SHARE ? a.n_work / 2 : a.n_work, a.head_mask != nullptr));
    if (D == 128)
        // the masked variant needs a few more registers
        return launch(attn_mfma_kernel<128, BSATTN_D128_KT, SHARE ? 2 : BSATTN_D128_SPLIT,
                                       KMASK ? BSATTN_D128_KM_WPE : BSATTN_D128_WPE, BSATTN_D128_BUF, KMASK, SHARE>,
                      grid, dim3(128 * (SHARE ? 2 : BSATTN_D128_SPLIT)), s, a);
    // the masked variant needs a few more registers
    return launch(attn_mfma_kernel<64, KMASK ? 32 : BSATTN_D64_KT, SHARE ? 2 : BSATTN_D64_SPLIT,
                                   KMASK ? BSATTN_D64_KM_WPE : BSATTN_D64_WPE, BSATTN_D64_BUF, KMASK, SHARE>,
                  grid, dim3(128 * (SHARE ? 2 : BSATTN_D64_SPLIT)), s, a);
}

hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)attn_grid(a.n_work, false));
    return launch(attn_mfma_kernel<64, BSATTN_D64_KT, BSATTN_D64_SPLIT, BSATTN_D64_WPE, BSATTN_D64_BUF, false, false, true>,
                  grid, dim3(128 * BSATTN_D64_SPLIT), s, a);
}

hipError_t launch_attn_mfma(const AttnArgs& a, int D, hipStream_t s) {
    // Query heads of a K/V group share the stage tiles when they walk the same
    // kept lists: one mask for all heads (or none), no head mask, and an even
    // number of query heads per K/V head.
    const int32_t rep = a.H / a.Hkv;
    const bool share = BSATTN_GQA_SHARE && rep >= 2 && rep % 2 == 0 && a.head_mask == nullptr &&
                       (a.count == nullptr || a.mH == 1);
    if (a.key_mask != nullptr)
        return share ? launch_attn_mfma_t<true, true>(a, D, s) : launch_attn_mfma_t<true, false>(a, D, s);
    return share ? launch_attn_mfma_t<false, true>(a, D, s) : launch_attn_mfma_t<false, false>(a, D, s);
}

}  // namespace bsattn
