// Block-sparse attention forward, bf16 MFMA path (gfx950).
//
// One workgroup of two wavefronts per (b, h, 64-token query block); each
// wavefront owns 32 query rows.  The workgroup walks the compacted list of
// kept key blocks (CSR-like, ascending) in stages of KT keys:
//   - K and V stage tiles go from HBM/L2 straight into LDS with
//     global_load_lds_dwordx4 (no register staging), NST stages deep, one
//     barrier per stage;
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with the Q^T fragments held in
//     VGPRs for the whole loop;
//   - online softmax in fp32: exp2 with the scale folded into log2 units, and
//     the running output rescaled only when a row maximum grows by more than
//     2^8 (exponentials stay <= 256, exact after the final division);
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

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ROWSUM_MFMA: the softmax denominators come from one extra O^T tile whose
// A operand is all ones (the MFMA pipe sums the bf16 P it multiplies);
// otherwise the VALU sums packed P with bf16 dot products.
template <int D, int KT, int NST, bool ROWSUM_MFMA, int WPE>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void attn_mfma_kernel(AttnArgs a) {
    constexpr int BLK = 64;
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int NI = KT * CPR / 128;       // loads per thread per tensor per stage
    constexpr int TILE_ELEMS = KT * D;       // bf16 elements per K (or V) stage tile
    constexpr int NKT = KT / 32;             // 32-key S^T tiles per stage
    constexpr int NKS = D / 16;              // k-steps of S^T
    constexpr int NDT = D / 32;              // 32-row d tiles of O^T
    constexpr int NPS = KT / 16;             // 16-key steps of O^T per stage
    constexpr int SUB = BLK / KT;            // stages per key block
    constexpr float kTau = 8.0f;             // lazy-rescale threshold (log2 units)
    static_assert(NI >= 1 && KT * CPR % 128 == 0, "stage tiling");

    // one LDS object per stage: distinct objects let the compiler see that the
    // reads of one stage never alias the loads in flight into the others
    __shared__ __attribute__((aligned(16))) uint16_t K0[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t V0[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t K1[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t V1[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t K2[NST > 2 ? TILE_ELEMS : 8];
    __shared__ __attribute__((aligned(16))) uint16_t V2[NST > 2 ? TILE_ELEMS : 8];
    static_assert(NST == 2 || NST == 3, "two or three LDS stages");

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    if (L >= a.n_work) return;
    const int32_t qb = (int32_t)(L % a.nqb);
    const int64_t bh = L / a.nqb;
    const int32_t h = (int32_t)(bh % a.H);
    const int32_t b = (int32_t)(bh / a.H);
    const int32_t kvh = h / (a.H / a.Hkv);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ql = lane & 31;

    const bool active = (a.head_mask == nullptr) || (a.head_mask[h] != 0);
    int32_t cnt = a.nkb;
    const int32_t* list = nullptr;
    if (a.count != nullptr) {
        const int64_t ms = (int64_t)(a.mB == 1 ? 0 : b) * a.mH + (a.mH == 1 ? 0 : h);
        cnt = a.count[ms * a.nqb + qb];
        list = a.index + (ms * a.nqb + qb) * (int64_t)a.nkb;
    }
    uint16_t* obase = (uint16_t*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qb * BLK * a.o_sn;

    if (!active || cnt <= 0) {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int c = tid; c < BLK * CPR; c += 128)
            *(uint4*)(obase + (int64_t)(c / CPR) * a.o_sn + (c % CPR) * 8) = z;
        return;
    }

    const uint16_t* qbase = (const uint16_t*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qb * BLK * a.q.sn;
    const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.sb + kvh * a.k.sh;
    const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.sb + kvh * a.v.sh;

    // Q^T fragments: lane holds Q[32*wave + ql][16*ks + 8*hl + 0..7]
    bf16x8 qf[NKS];
    {
        const uint16_t* qr = qbase + (int64_t)(32 * wave + ql) * a.q.sn + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qr + 16 * ks);
    }
    const int T = cnt * SUB;   // stages
    // kept key block of stage t: a scalar (constant address space) load, so
    // waiting for it never waits for the stage loads in flight
    const __attribute__((address_space(4))) int32_t* klist =
        (const __attribute__((address_space(4))) int32_t*)list;
    auto block_of = [&](int t) -> int32_t {
        const int i = t / SUB;
        return list == nullptr ? i : klist[i];
    };
    // per-thread source offsets of the NI chunks it loads per stage: LDS chunk
    // slot s = i*128 + tid holds row s / CPR, global chunk (s % CPR) ^ swizzle
    int32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int s = i * 128 + tid;
        const int r = s / CPR;
        const int c = (s % CPR) ^ chunk_swizzle<D>(r);
        koff[i] = r * (int32_t)a.k.sn + c * 8;
        voff[i] = r * (int32_t)a.v.sn + c * 8;
    }
    // issue the K and V loads of stage t into LDS buffer (Kd, Vd)
    auto issue = [&](int t, uint16_t* Kd, uint16_t* Vd) {
        const int64_t row0 = (int64_t)block_of(t) * BLK + (t % SUB) * KT;
        const uint16_t* kt = kbase + row0 * a.k.sn;
        const uint16_t* vt = vbase + row0 * a.v.sn;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int dst = (i * 128 + wave * 64) * 8;   // wave-uniform element offset
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(kt + koff[i]),
                (__attribute__((address_space(3))) void*)(Kd + dst), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(vt + voff[i]),
                (__attribute__((address_space(3))) void*)(Vd + dst), 16, 0, 0);
        }
    };
    issue(0, K0, V0);
    if (NST > 2 && T > 1) issue(1, K1, V1);

    const float sl2 = a.scale * 1.4426950408889634f;   // scale * log2(e)
    float m_run = -INFINITY, l_run = 0.f;
    f16v oacc[NDT];
    f16v lacc;                                          // row sums (ROWSUM_MFMA)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

    const int g16 = lane >> 4, j16 = lane & 15;

    // one stage: wait for its tiles (the next stage's loads may stay in
    // flight), make them visible, start the loads of stage t + NST - 1 into
    // the buffers freed by stage t - 1, then compute from this stage
    auto stage = [&](int t, const uint16_t* Kt, const uint16_t* Vt, uint16_t* Kn, uint16_t* Vn) {
        if (NST > 2 && t + 1 < T) wait_vmcnt<(NST > 2 ? 2 * NI : 0)>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (t + NST - 1 < T) issue(t + NST - 1, Kn, Vn);

        // S^T for NKT 32-key tiles
        f16v sacc[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
            const int r = 32 * kt + slot_key(ql);
            const int sw = chunk_swizzle<D>(r);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 kf = *(const bf16x8*)(Kt + (r * CPR + ((2 * ks + hl) ^ sw)) * 8);
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
            }
        }

        // online softmax with lazy rescaling; the row maximum as a tree
        float mq[NKT * 4];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mq[4 * kt + q] = fmaxf(fmaxf(sacc[kt][4 * q], sacc[kt][4 * q + 1]),
                                       fmaxf(sacc[kt][4 * q + 2], sacc[kt][4 * q + 3]));
#pragma unroll
        for (int n = NKT * 4; n > 1; n >>= 1)
#pragma unroll
            for (int q = 0; q < n / 2; ++q) mq[q] = fmaxf(mq[q], mq[q + n / 2]);
        float mx = fmaxf(mq[0], __shfl_xor(mq[0], 32)) * sl2;
        const bool grow = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform
            const float m_new = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            if constexpr (ROWSUM_MFMA)
#pragma unroll
                for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
        }

        bf16x8 pf[NPS];   // B operand of P V, one per 16-key step
        float psum2[2] = {0.f, 0.f};
        const bf2v one2 = {(__bf16)1.f, (__bf16)1.f};
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
                    if constexpr (!ROWSUM_MFMA)
                        psum2[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(w[e >> 1], one2, psum2[(e >> 1) & 1], false);
                }
                pf[2 * kt + u] = __builtin_bit_cast(
                    bf16x8, (uint4){__builtin_bit_cast(uint32_t, w[0]), __builtin_bit_cast(uint32_t, w[1]),
                                    __builtin_bit_cast(uint32_t, w[2]), __builtin_bit_cast(uint32_t, w[3])});
                if constexpr (ROWSUM_MFMA)
                    lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf[2 * kt + u], lacc, 0, 0, 0);
            }
        l_run += psum2[0] + psum2[1];

        // O^T += V^T P^T.  Within each 16-lane group, lane j supplies
        // V[kb + j/4][d0 + 4*(j%4) .. +3]; lane i then receives V[kb + 0..3][d0 + i].
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int d = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3);
            const int c = d >> 3, half = (d >> 2) & 1;
#pragma unroll
            for (int ks = 0; ks < NPS; ++ks) {
                const int r0 = 16 * ks + 8 * hl + (j16 >> 2);
                const int r1 = r0 + 4;
                const uint16_t* p0 = Vt + (r0 * CPR + (c ^ chunk_swizzle<D>(r0))) * 8 + half * 4;
                const uint16_t* p1 = Vt + (r1 * CPR + (c ^ chunk_swizzle<D>(r1))) * 8 + half * 4;
                const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(p0));
                const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(p1));
                const s8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[ks],
                                                                  oacc[dt], 0, 0, 0);
            }
        }
    };
    if constexpr (NST == 2) {
        for (int t = 0; t < T; t += 2) {
            stage(t, K0, V0, K1, V1);
            if (t + 1 < T) stage(t + 1, K1, V1, K0, V0);
        }
    } else {
        // stage t reads buffer t % 3 and loads stage t + 2 into buffer (t + 2) % 3
        for (int t = 0; t < T; t += 3) {
            stage(t, K0, V0, K2, V2);
            if (t + 1 < T) stage(t + 1, K1, V1, K0, V0);
            if (t + 2 < T) stage(t + 2, K2, V2, K1, V1);
        }
    }

    // normalise and store: oacc[dt][r] = O[query][32*dt + 8*(r/4) + 4*hl + r%4]
    // every row of the ones tile holds the full sum of the bf16 P of this query
    const float l_tot = ROWSUM_MFMA ? lacc[0] : l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    uint16_t* orow = obase + (int64_t)(32 * wave + ql) * a.o_sn;
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

// ---------------------------------------------------------------------------
// Sixteen-row variant: four wavefronts per query block, each owning 16 query
// rows, on v_mfma_f32_16x16x32_bf16.  Twice the wavefronts of the 32-row
// kernel and a third of its registers, for shapes whose grids are too small to
// hide latency with 32-row wavefronts.  Layouts (lane l, g = l / 16):
//   S^T tile (16 keys x 16 queries): lane holds keys 4g..4g+3 of query l % 16;
//   the PV step of 32 keys takes k-slots 8g + 4*kt + r = key 16*kt + 4g + r,
//   so P never moves between lanes and each V^T operand is two transposing
//   reads of four consecutive keys.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int chunk_swizzle16(int r) {
    if constexpr (D == 64) return (r & 7) ^ ((r >> 1) & 7);
    else return (r & 15) ^ ((r & 1) << 3);
}

typedef float f4v_ __attribute__((ext_vector_type(4)));

template <int D, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void attn_m16_kernel(AttnArgs a) {
    constexpr int BLK = 64, KT = 32;
    constexpr int CPR = D / 8;
    constexpr int NI = KT * CPR / 256;        // loads per thread per tensor per stage
    constexpr int TILE_ELEMS = KT * D;
    constexpr int NKS = D / 32;               // k-steps of S^T
    constexpr int NDT = D / 16;               // 16-row d tiles of O^T
    constexpr int SUB = BLK / KT;
    constexpr float kTau = 8.0f;
    static_assert(NI >= 1 && KT * CPR % 256 == 0, "stage tiling");

    __shared__ __attribute__((aligned(16))) uint16_t K0[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t V0[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t K1[TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t V1[TILE_ELEMS];

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    if (L >= a.n_work) return;
    const int32_t qb = (int32_t)(L % a.nqb);
    const int64_t bh = L / a.nqb;
    const int32_t h = (int32_t)(bh % a.H);
    const int32_t b = (int32_t)(bh / a.H);
    const int32_t kvh = h / (a.H / a.Hkv);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;

    const bool active = (a.head_mask == nullptr) || (a.head_mask[h] != 0);
    int32_t cnt = a.nkb;
    const int32_t* list = nullptr;
    if (a.count != nullptr) {
        const int64_t ms = (int64_t)(a.mB == 1 ? 0 : b) * a.mH + (a.mH == 1 ? 0 : h);
        cnt = a.count[ms * a.nqb + qb];
        list = a.index + (ms * a.nqb + qb) * (int64_t)a.nkb;
    }
    uint16_t* obase = (uint16_t*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qb * BLK * a.o_sn;
    if (!active || cnt <= 0) {
        const uint4 z = {0u, 0u, 0u, 0u};
        for (int c = tid; c < BLK * CPR; c += 256)
            *(uint4*)(obase + (int64_t)(c / CPR) * a.o_sn + (c % CPR) * 8) = z;
        return;
    }
    const uint16_t* qbase = (const uint16_t*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qb * BLK * a.q.sn;
    const uint16_t* kbase = (const uint16_t*)a.k.p + b * a.k.sb + kvh * a.k.sh;
    const uint16_t* vbase = (const uint16_t*)a.v.p + b * a.v.sb + kvh * a.v.sh;

    // Q^T fragments: lane holds Q[16*wave + li][32*ks + 8*g + 0..7]
    bf16x8 qf[NKS];
    {
        const uint16_t* qr = qbase + (int64_t)(16 * wave + li) * a.q.sn + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qr + 32 * ks);
    }
    int32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int s = i * 256 + tid;
        const int r = s / CPR;
        const int c = (s % CPR) ^ chunk_swizzle16<D>(r);
        koff[i] = r * (int32_t)a.k.sn + c * 8;
        voff[i] = r * (int32_t)a.v.sn + c * 8;
    }
    const int T = cnt * SUB;
    const __attribute__((address_space(4))) int32_t* klist =
        (const __attribute__((address_space(4))) int32_t*)list;
    auto issue = [&](int t, uint16_t* Kd, uint16_t* Vd) {
        const int i0 = t / SUB;
        const int32_t blk = list == nullptr ? i0 : klist[i0];
        const int64_t row0 = (int64_t)blk * BLK + (t % SUB) * KT;
        const uint16_t* kt = kbase + row0 * a.k.sn;
        const uint16_t* vt = vbase + row0 * a.v.sn;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int dst = (i * 256 + wave * 64) * 8;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + koff[i]),
                                             (__attribute__((address_space(3))) void*)(Kd + dst), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vt + voff[i]),
                                             (__attribute__((address_space(3))) void*)(Vd + dst), 16, 0, 0);
        }
    };
    issue(0, K0, V0);

    const float sl2 = a.scale * 1.4426950408889634f;
    float m_run = -INFINITY, l_run = 0.f;
    f4v_ oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = (f4v_){0.f, 0.f, 0.f, 0.f};
    const bf2v one2 = {(__bf16)1.f, (__bf16)1.f};

    auto stage = [&](int t, const uint16_t* Kt, const uint16_t* Vt, uint16_t* Kn, uint16_t* Vn) {
        wait_vmcnt<0>();
        __syncthreads();
        if (t + 1 < T) issue(t + 1, Kn, Vn);

        // S^T: two 16-key tiles
        f4v_ sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sacc[kt] = (f4v_){0.f, 0.f, 0.f, 0.f};
            const int r = 16 * kt + li;
            const int sw = chunk_swizzle16<D>(r);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 kf = *(const bf16x8*)(Kt + (r * CPR + ((4 * ks + g) ^ sw)) * 8);
                sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
            }
        }
        // row max over the 32 keys: 8 in lane, then the four lane groups
        float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
        const bool grow = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        }
        // P: k-slot 8g + 4kt + r <-> key 16kt + 4g + r
        bf2v w[4];
        float psum2[2] = {0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sl2, -m_run));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r + 1], sl2, -m_run));
                w[2 * kt + r / 2] = to_bf16x2(p0, p1);
                psum2[kt] = __builtin_amdgcn_fdot2_f32_bf16(w[2 * kt + r / 2], one2, psum2[kt], false);
            }
        l_run += psum2[0] + psum2[1];
        const bf16x8 pf = __builtin_bit_cast(
            bf16x8, (uint4){__builtin_bit_cast(uint32_t, w[0]), __builtin_bit_cast(uint32_t, w[1]),
                            __builtin_bit_cast(uint32_t, w[2]), __builtin_bit_cast(uint32_t, w[3])});
        // O^T += V^T P^T: per 16-lane group, lane j supplies V[kb + j/4][16*dt + 4*(j%4)]
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int d = 16 * dt + 4 * (li & 3);
            const int c = d >> 3, half = (d >> 2) & 1;
            const int r0 = 4 * g + (li >> 2);
            const int r1 = r0 + 16;
            const uint16_t* p0 = Vt + (r0 * CPR + (c ^ chunk_swizzle16<D>(r0))) * 8 + half * 4;
            const uint16_t* p1 = Vt + (r1 * CPR + (c ^ chunk_swizzle16<D>(r1))) * 8 + half * 4;
            const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(p0));
            const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(p1));
            const s8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, both), pf, oacc[dt], 0, 0, 0);
        }
    };
    for (int t = 0; t < T; t += 2) {
        stage(t, K0, V0, K1, V1);
        if (t + 1 < T) stage(t + 1, K1, V1, K0, V0);
    }

    // l over the row: the four lane groups hold disjoint keys
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = 1.f / l_tot;
    // oacc[dt][r] = O[query 16*wave + li][16*dt + 4g + r]
    uint16_t* orow = obase + (int64_t)(16 * wave + li) * a.o_sn;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        uint2 w2;
        w2.x = pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv);
        w2.y = pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv);
        *(uint2*)(orow + 16 * dt + 4 * g) = w2;
    }
}

// Launch shapes (keys per LDS stage, row-sum mode, waves per EU) per head dim.
#ifndef BSATTN_D64_KT
#define BSATTN_D64_KT 32
#endif
#ifndef BSATTN_D64_ROWSUM_MFMA
#define BSATTN_D64_ROWSUM_MFMA false
#endif
#ifndef BSATTN_D64_WPE
#define BSATTN_D64_WPE 3
#endif
#ifndef BSATTN_D128_KT
#define BSATTN_D128_KT 32
#endif
#ifndef BSATTN_D128_ROWSUM_MFMA
#define BSATTN_D128_ROWSUM_MFMA false
#endif
#ifndef BSATTN_D128_WPE
#define BSATTN_D128_WPE 2
#endif
#ifndef BSATTN_D64_NST
#define BSATTN_D64_NST 2
#endif
#ifndef BSATTN_D128_NST
#define BSATTN_D128_NST 2
#endif
// 16-row kernel per head dim (0 = the 32-row kernel) and its waves per EU
#ifndef BSATTN_D64_ROWS16
#define BSATTN_D64_ROWS16 0
#endif
#ifndef BSATTN_D128_ROWS16
#define BSATTN_D128_ROWS16 0
#endif
#ifndef BSATTN_M16_WPE
#define BSATTN_M16_WPE 4
#endif

hipError_t launch_attn_mfma(const AttnArgs& a, int D, hipStream_t s) {
    const int64_t padded = ((a.n_work + kNumXcd - 1) / kNumXcd) * kNumXcd;
    const dim3 grid((unsigned)padded);
    if (D == 128 && BSATTN_D128_ROWS16)
        return launch(attn_m16_kernel<128, BSATTN_M16_WPE>, grid, dim3(256), s, a);
    if (D == 64 && BSATTN_D64_ROWS16)
        return launch(attn_m16_kernel<64, BSATTN_M16_WPE>, grid, dim3(256), s, a);
    if (D == 128)
        return launch(attn_mfma_kernel<128, BSATTN_D128_KT, BSATTN_D128_NST, BSATTN_D128_ROWSUM_MFMA, BSATTN_D128_WPE>, grid,
                      dim3(128), s, a);
    return launch(attn_mfma_kernel<64, BSATTN_D64_KT, BSATTN_D64_NST, BSATTN_D64_ROWSUM_MFMA, BSATTN_D64_WPE>, grid, dim3(128),
                  s, a);
}

}  // namespace bsattn
