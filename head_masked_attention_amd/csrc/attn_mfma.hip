// Block-sparse attention forward, bf16 MFMA path (gfx950).
//
// One workgroup of two wavefronts per (b, h, 64-token query block); each
// wavefront owns 32 query rows.  The workgroup walks the compacted list of
// kept key blocks (CSR-like, ascending), stages each 64-key K and V tile in
// LDS, and runs
//     S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, Q^T fragments held in VGPRs)
//     online softmax in fp32 (exp2 with the scale folded into log2 units)
//     O^T += V^T P^T (V^T fragments read with ds_read_b64_tr_b16)
// so that every lane holds one query's scores and one query's output column
// and the softmax statistics never leave the lane pair (lane, lane ^ 32).
// The K rows are loaded into MFMA row slots in a fixed permutation chosen so
// that each lane's eight P values of a 16-key step are consecutive keys, which
// is exactly the B-operand layout of the P V product: no shuffle of P.
// Masked heads and rows without kept blocks write zeros and exit.
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

// MFMA row slot -> key within a 32-key tile.
__device__ __forceinline__ int slot_key(int s) {
    const int q = s >> 3, hh = (s >> 2) & 1, r = s & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;   // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int D>
__global__ __launch_bounds__(128) void attn_mfma_kernel(AttnArgs a) {
    constexpr int BLK = 64;
    constexpr int KS = D + 8;      // K tile row stride (bf16): conflict-free 16-byte row reads
    constexpr int VS = D + 32;     // V tile row stride (bf16): conflict-free transpose reads
    constexpr int CPR = D / 8;     // 16-byte chunks per row
    constexpr int NCH = BLK * CPR / 128;   // chunks per thread per tile
    constexpr int NKS = D / 16;    // k-steps of S^T
    constexpr int NDT = D / 32;    // d tiles of O^T
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[BLK * VS];

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    if (L >= a.n_work) return;
    const int32_t qb = (int32_t)(L % a.nqb);
    const int64_t bh = L / a.nqb;
    const int32_t h = (int32_t)(bh % a.H);
    const int32_t b = (int32_t)(bh / a.H);
    const int32_t kvh = h / (a.H / a.Hkv);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c = tid + 128 * t;
            *(uint4*)(obase + (int64_t)(c / CPR) * a.o_sn + (c % CPR) * 8) = z;
        }
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

    uint4 kreg[NCH], vreg[NCH];
    auto prefetch = [&](int32_t kb) {
        const uint16_t* kt = kbase + (int64_t)kb * BLK * a.k.sn;
        const uint16_t* vt = vbase + (int64_t)kb * BLK * a.v.sn;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c = tid + 128 * t;
            kreg[t] = *(const uint4*)(kt + (int64_t)(c / CPR) * a.k.sn + (c % CPR) * 8);
            vreg[t] = *(const uint4*)(vt + (int64_t)(c / CPR) * a.v.sn + (c % CPR) * 8);
        }
    };
    prefetch(list ? list[0] : 0);

    const float sl2 = a.scale * 1.4426950408889634f;   // scale * log2(e)
    float m_run = -INFINITY, l_run = 0.f;
    f16v oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;

    const int krow = slot_key(ql);   // K row this lane feeds into MFMA row slot ql
    const int g16 = lane >> 4, j16 = lane & 15;

    for (int32_t it = 0; it < cnt; ++it) {
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c = tid + 128 * t;
            *(uint4*)(Ks + (c / CPR) * KS + (c % CPR) * 8) = kreg[t];
            *(uint4*)(Vs + (c / CPR) * VS + (c % CPR) * 8) = vreg[t];
        }
        __syncthreads();
        if (it + 1 < cnt) prefetch(list ? list[it + 1] : it + 1);

        // S^T for two 32-key tiles
        f16v sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
            const uint16_t* kr = Ks + (32 * kt + krow) * KS + 8 * hl;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 kf = *(const bf16x8*)(kr + 16 * ks);
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
            }
        }

        // online softmax (lane: query 32*wave + ql; keys split with lane ^ 32)
        float mx = sacc[0][0];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * sl2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;

        bf16x8 pf[4];   // B operand of P V for the four 16-key steps
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * u + e], sl2, -m_new));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * u + e + 1], sl2, -m_new));
                    psum += p0 + p1;
                    w[e >> 1] = pack_bf16x2(p0, p1);
                }
                pf[2 * kt + u] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

        // O^T += V^T P^T: V^T fragments via transpose reads of the row-major tile.
        // Within each 16-lane group, lane j supplies V[kb + j/4][d0 + 4*(j%4)];
        // lane i then receives V[kb + 0..3][d0 + i].
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int d0 = 32 * dt + 16 * (g16 & 1);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kb0 = 16 * ks + 8 * hl;
                const uint16_t* p0 = Vs + (kb0 + (j16 >> 2)) * VS + d0 + 4 * (j16 & 3);
                const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4v*)(p0));
                const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s4v*)(p0 + 4 * VS));
                const s8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf[ks],
                                                                  oacc[dt], 0, 0, 0);
            }
        }
    }

    // normalise and store: oacc[dt][r] = O[query][32*dt + 8*(r/4) + 4*hl + r%4]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
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

hipError_t launch_attn_mfma(const AttnArgs& a, int D, hipStream_t s) {
    const int64_t padded = ((a.n_work + kNumXcd - 1) / kNumXcd) * kNumXcd;
    const dim3 grid((unsigned)padded);
    if (D == 128) hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace bsattn
