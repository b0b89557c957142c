// Block-sparse attention forward on fp8 (OCP e4m3) inputs (gfx950).
//
// The quantized consumer of the block mask: Q, K and V are fp8 with one fp32
// scale per (b, head) (x = code * scale), the products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales), and the output is
// bf16.  One workgroup of two wavefronts per (b, query block, query head),
// each wavefront owning 32 query rows; one stage per kept 64-key block, K and
// V double-buffered in LDS (buffer_load_dwordx4 ... lds, 16-byte chunks XOR-
// swizzled by row).
//   - S^T = K Q^T: two 32-key tiles per stage and D / 64 k-steps; the K rows
//     enter the MFMA row slots in an order that leaves lane half h holding the
//     scores of keys 32 h + 0..31 of its query, in byte order of the P
//     operand below;
//   - online softmax in fp32 (exp2, scale folded in log2 units, lazy rescale
//     by 2^8 as in the bf16 kernel), so P <= 256 fits e4m3 (max 448);
//   - P is rounded to e4m3 once; the row sums come from one more MFMA of the
//     same fp8 P against a ones operand, so numerator and denominator use the
//     same rounded weights;
//   - O^T += V^T P^T with the V^T operand read by ds_read_b64_tr_b8 (lane J
//     of a 16-lane group supplies 8 bytes of row 2e + J/2 ... so lane i
//     receives byte column i of 8 consecutive rows).
// Rows without kept blocks and heads with head_mask 0 are written as 0.
// With a key mask (KMASK), a block whose 64 keys are all masked is skipped and
// the masked keys of a partly masked block get -inf scores.
//
// Sources: SD.Next commit view, modules/attention/sparse, the stage paragraph
// (a quantized kernel joins as a block-mask consumer) and the flex-consumer
// paragraph (only selected tiles are computed); haagenti_sparse crate docs
// (heads skipped under a per-layer mask).
#include "common.h"
#include "internal.h"

#include <map>
#include <mutex>
#include <utility>


namespace bsattn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float f16v8 __attribute__((ext_vector_type(16)));

// 16-byte chunk swizzle of an fp8 tile row: eight consecutive rows (one
// transposing V read) and the rows of one K-fragment read land on distinct
// chunks.
template <int D>
__device__ __forceinline__ int f8_swizzle(int r) {
    if constexpr (D == 128) return (r & 7) ^ (((r >> 5) & 1) << 2);
    else return (r & 3) ^ (((r >> 5) & 1) << 1) ^ ((r >> 2) & 2);
}

// S^T tile kt, MFMA row slot m -> key of the 64-key stage.  Lane half h of
// row slots 8(r/4) + 4h + r%4 then holds keys 32 h + 16 kt + r.
__device__ __forceinline__ int f8_slot_key(int kt, int m) {
    return 32 * ((m >> 2) & 1) + 16 * kt + (((m >> 3) << 2) | (m & 3));
}

// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding)
__device__ __forceinline__ void wait_vmcnt_f8() {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

__device__ __forceinline__ float f8_pair_max32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ uint32_t f8_pack_bf16x2(float lo, float hi) {
    typedef float f2v_ __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2v_ __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v_){lo, hi}, bf2v_));
}

template <int D, int WPE, bool KMASK>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void attn_fp8_kernel(AttnArgs a, const float* __restrict__ q_scale, const float* __restrict__ k_scale,
                     const float* __restrict__ v_scale, int one_round) {
    constexpr int BLK = 64;                  // keys per stage = one key block
    constexpr int CPR = D / 16;              // 16-byte chunks per fp8 row
    constexpr int NI = BLK * CPR / 128;      // DMA loads per thread per tensor per stage
    constexpr int TILE = BLK * D;            // bytes per K (or V) stage tile
    constexpr int NKS = D / 64;              // k-steps of S^T
    constexpr int NDT = D / 32;              // 32-row d tiles of O^T
    constexpr float kTau = 8.0f;
    static_assert(NI >= 1 && BLK * CPR % 128 == 0, "stage tiling");

    __shared__ __attribute__((aligned(16))) uint8_t K0[TILE];
    __shared__ __attribute__((aligned(16))) uint8_t V0[TILE];
    __shared__ __attribute__((aligned(16))) uint8_t K1[TILE];
    __shared__ __attribute__((aligned(16))) uint8_t V1[TILE];

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    if (a.head_mask == nullptr && L >= a.n_work) return;
    // (b, K/V head, query block, query head within the group) order, or
    // under a head mask the active heads' query blocks first
    int32_t qb, h, b;
    bool active = true;
    if (a.head_mask != nullptr) {
        const HeadWork hw = head_masked_order(blockIdx.x, gridDim.x, a.head_mask, a.B, a.H, a.nqb);
        if (!hw.valid) return;
        qb = hw.qb, h = hw.h, b = hw.b, active = hw.active;
    } else {
        const int32_t rep = a.H / a.Hkv;
        const int32_t hr = (int32_t)(L % rep);
        const int64_t rest = L / rep;
        qb = (int32_t)(rest % a.nqb);
        const int64_t bg = rest / a.nqb;
        b = (int32_t)(bg / a.Hkv);
        h = (int32_t)(bg % a.Hkv) * rep + hr;
    }
    const int32_t kvh = h / (a.H / a.Hkv);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane >> 5, ql = lane & 31;

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
        for (int c = tid; c < BLK * D / 8; c += 128)
            *(uint4*)(obase + (int64_t)(c / (D / 8)) * a.o_sn + (c % (D / 8)) * 8) = z;
        return;
    }

    const uint8_t* qbase = (const uint8_t*)a.q.p + b * a.q.sb + h * a.q.sh + (int64_t)qb * BLK * a.q.sn;
    const uint8_t* kbase = (const uint8_t*)a.k.p + b * a.k.sb + kvh * a.k.sh;
    const uint8_t* vbase = (const uint8_t*)a.v.p + b * a.v.sb + kvh * a.v.sh;
    const float sq = q_scale[(int64_t)b * a.H + h];
    const float sk = k_scale[(int64_t)b * a.Hkv + kvh];
    const float sv = v_scale[(int64_t)b * a.Hkv + kvh];

    // Q^T operand: lane (query 32 wave + ql, half hl) holds Q[query][64 ks + 32 hl + 0..31]
    v8i qf[NKS];
    {
        const uint8_t* qr = qbase + (int64_t)(32 * wave + ql) * a.q.sn + 32 * hl;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint4 lo = *(const uint4*)(qr + 64 * ks), hi = *(const uint4*)(qr + 64 * ks + 16);
            qf[ks] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    }

    const __attribute__((address_space(4))) int32_t* klist =
        (const __attribute__((address_space(4))) int32_t*)list;
    auto block_of = [&](int t) -> int32_t { return list == nullptr ? t : klist[t]; };
    // per-thread source offsets: chunk slot s = i*128 + tid holds row s / CPR,
    // global chunk (s % CPR) ^ swizzle
    uint32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int s = i * 128 + tid;
        const int r = s / CPR;
        const int c = (s % CPR) ^ f8_swizzle<D>(r);
        koff[i] = (uint32_t)(r * (int32_t)a.k.sn + c * 16);
        voff[i] = (uint32_t)(r * (int32_t)a.v.sn + c * 16);
    }
    // KMASK: each lane fetches the mask byte of one key of the stage's block
    // with its tiles; at the stage a ballot makes it one wave-uniform 64-bit
    // word (bit j = key j of the block live).
    const uint8_t* kmbase = KMASK ? a.key_mask + (int64_t)b * a.km_sb : nullptr;
    uint32_t km_next = 1u;
    auto issue = [&](int t, uint8_t* Kd, uint8_t* Vd) {
        const int64_t row0 = (int64_t)block_of(t) * BLK;
        if constexpr (KMASK) km_next = (uint32_t)kmbase[row0 + lane];
        const uint8_t* kt = kbase + row0 * a.k.sn;
        const uint8_t* vt = vbase + row0 * a.v.sn;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int dst = (i * 128 + wave * 64) * 16;   // wave-uniform byte offset
            chunk_to_lds(kt, koff[i], Kd + dst);
            chunk_to_lds(vt, voff[i], Vd + dst);
        }
    };
    issue(0, K0, V0);

    const float sl2 = a.scale * sq * sk * 1.4426950408889634f;
    float m_run = -INFINITY;
    f16v8 oacc[NDT], lacc;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
    const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0

    const int g16 = lane >> 4, j16 = lane & 15;

    auto stage = [&](int t, const uint8_t* Kt, const uint8_t* Vt, uint8_t* Kn, uint8_t* Vn) {
        if (one_round) {
            // issue priority 3..0 over the quarters of the row's blocks, so
            // that the workgroups of a CU, which start together, stay abreast
            // (with several rounds it only delays the ones about to finish)
            const int pr = 3 - min(3, (4 * t) / cnt);
            if (pr == 3) __builtin_amdgcn_s_setprio(3);
            else if (pr == 2) __builtin_amdgcn_s_setprio(2);
            else if (pr == 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        wait_vmcnt_f8();
        __syncthreads();
        uint64_t kw = ~0ull;
        if constexpr (KMASK) kw = __ballot(km_next != 0u);
        if (t + 1 < cnt) issue(t + 1, Kn, Vn);
        if (KMASK && kw == 0ull) return;   // every key of the block masked

        // S^T: two 32-key tiles
        f16v8 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
            const int key = f8_slot_key(kt, ql);
            const uint8_t* krow = Kt + key * D;
            const int sw = f8_swizzle<D>(key);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = 4 * ks + 2 * hl;
                const uint4 lo = *(const uint4*)(krow + ((c0 ^ sw) << 4));
                const uint4 hi = *(const uint4*)(krow + (((c0 + 1) ^ sw) << 4));
                const v8i kf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[ks], sacc[kt], 0, 0, 0, 127, 0, 127);
            }
        }

        if constexpr (KMASK) {
            // masked keys of a partly masked block: -inf scores (element r of
            // tile kt is key 32 hl + 16 kt + r)
            if (kw != ~0ull) {
                const uint32_t wl = (uint32_t)(kw >> (32 * hl));
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (!((wl >> (16 * kt + r)) & 1u)) sacc[kt][r] = -INFINITY;
            }
        }

        // online softmax, lazy rescale
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const f16v8& x = sacc[kt];
            const float a0 = fmaxf(fmaxf(x[0], x[1]), x[2]), a1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
            const float a2 = fmaxf(fmaxf(x[6], x[7]), x[8]), a3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
            const float a4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
            mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), x[15])));
        }
        mx = f8_pair_max32(mx) * sl2;
        const bool grow = mx > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? mx : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
        }

        // P in e4m3: byte 16 kt + r of this lane's operand = key 32 hl + 16 kt + r
        v8i pf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][4 * q], sl2, -m_run));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][4 * q + 1], sl2, -m_run));
                const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][4 * q + 2], sl2, -m_run));
                const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][4 * q + 3], sl2, -m_run));
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
                pf[4 * kt + q] = w;
            }
        // row sums of the rounded P (every row of the ones product holds it)
        lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, 127, 0, 127);

        // O^T += V^T P^T.  Read q of d tile dt: lane j16 of 16-lane group g16
        // supplies 8 bytes of row 32 (g16 >> 1) + 8 q + j16 / 2 at byte column
        // 32 dt + 16 (g16 & 1) + 8 (j16 & 1); lane i then holds byte column
        // 32 dt + 16 (g16 & 1) + i of those 8 rows.
        const int hv = g16 >> 1;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int c = 2 * dt + (g16 & 1);
            v8i vf;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int R = 32 * hv + 8 * q + (j16 >> 1);
                const uint8_t* p = Vt + R * D + ((c ^ f8_swizzle<D>(R)) << 4) + 8 * (j16 & 1);
                const v2i tr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
                vf[2 * q] = tr[0];
                vf[2 * q + 1] = tr[1];
            }
            oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, oacc[dt], 0, 0, 0, 127, 0, 127);
        }
    };
    for (int t = 0; t < cnt; t += 2) {
        stage(t, K0, V0, K1, V1);
        if (t + 1 < cnt) stage(t + 1, K1, V1, K0, V0);
    }

    // normalise (V's scale folded in) and store bf16:
    // oacc[dt][r] = O[query][32 dt + 8 (r / 4) + 4 hl + r % 4]
    const float l_tot = lacc[0];
    const float f = l_tot > 0.f ? sv / l_tot : 0.f;
    uint16_t* orow = obase + (int64_t)(32 * wave + ql) * a.o_sn;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            uint2 w;
            w.x = f8_pack_bf16x2(oacc[dt][4 * j4] * f, oacc[dt][4 * j4 + 1] * f);
            w.y = f8_pack_bf16x2(oacc[dt][4 * j4 + 2] * f, oacc[dt][4 * j4 + 3] * f);
            *(uint2*)(orow + 32 * dt + 8 * j4 + 4 * hl) = w;
        }
}

// ---------------------------------------------------------------------------
// Per-(b, head) fp8 quantisation of a bf16 tensor: scale = max|x| / 448 (1 for
// an all-zero head), code = e4m3(clamp(x / scale, -448, 448)) rounded to
// nearest even by v_cvt_pk_fp8_f32.  Three launches: clear the maxima, take
// them (atomic max on the bit patterns of non-negative floats), convert.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_clear_kernel(uint32_t* amax, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) amax[i] = 0u;
}

constexpr int kQuantRows = 256;  // token rows per workgroup of the quantiser

template <int D>
__global__ __launch_bounds__(256) void fp8_amax_kernel(TView x, int H, int64_t N, uint32_t* amax) {
    constexpr int CPR = D / 8;                     // 16-byte chunks of a bf16 row
    const int64_t bh = blockIdx.y;
    const int64_t b = bh / H, h = bh % H;
    const int64_t r0 = (int64_t)blockIdx.x * kQuantRows;
    float m = 0.f;
    for (int c = threadIdx.x; c < kQuantRows * CPR; c += 256) {
        const int64_t r = r0 + c / CPR;
        if (r >= N) break;
        const uint4 w = *(const uint4*)((const uint16_t*)x.p + b * x.sb + h * x.sh + r * x.sn + (c % CPR) * 8);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m = fmaxf(m, fmaxf(fabsf(__uint_as_float(u[e] << 16)), fabsf(__uint_as_float(u[e] & 0xffff0000u))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    // one atomic per workgroup: many workgroups share one (b, head) word
    __shared__ float wmax[4];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicMax(amax + bh, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

template <int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(TView x, TView y, int H, int64_t N, const uint32_t* amax,
                                                        float* scale) {
    constexpr int CPR = D / 8;
    const int64_t bh = blockIdx.y;
    const int64_t b = bh / H, h = bh % H;
    const float am = __uint_as_float(amax[bh]);
    const float sc = am > 0.f ? am / 448.f : 1.f;
    if (blockIdx.x == 0 && threadIdx.x == 0) scale[bh] = sc;
    const int64_t r0 = (int64_t)blockIdx.x * kQuantRows;
    for (int c = threadIdx.x; c < kQuantRows * CPR; c += 256) {
        const int64_t r = r0 + c / CPR;
        if (r >= N) break;
        const uint4 w = *(const uint4*)((const uint16_t*)x.p + b * x.sb + h * x.sh + r * x.sn + (c % CPR) * 8);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
        uint32_t packed[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float v[4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                v[2 * k] = fminf(fmaxf(__uint_as_float(u[2 * e + k] << 16) / sc, -448.f), 448.f);
                v[2 * k + 1] = fminf(fmaxf(__uint_as_float(u[2 * e + k] & 0xffff0000u) / sc, -448.f), 448.f);
            }
            int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
            packed[e] = (uint32_t)p;
        }
        *(uint2*)((uint8_t*)y.p + b * y.sb + h * y.sh + r * y.sn + (c % CPR) * 8) = make_uint2(packed[0], packed[1]);
    }
}

hipError_t launch_quant_fp8(TView x, TView y, int B, int H, int64_t N, int D, uint32_t* amax, float* scale,
                            hipStream_t s) {
    const int n = B * H;
    hipError_t e = launch(fp8_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, amax, n);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((N + kQuantRows - 1) / kQuantRows), (unsigned)n);
    if (D == 128) {
        e = launch(fp8_amax_kernel<128>, grid, dim3(256), s, x, H, N, amax);
        if (e == hipSuccess) e = launch(fp8_quant_kernel<128>, grid, dim3(256), s, x, y, H, N, (const uint32_t*)amax, scale);
    } else if (D == 64) {
        e = launch(fp8_amax_kernel<64>, grid, dim3(256), s, x, H, N, amax);
        if (e == hipSuccess) e = launch(fp8_quant_kernel<64>, grid, dim3(256), s, x, y, H, N, (const uint32_t*)amax, scale);
    } else {
        e = launch(fp8_amax_kernel<32>, grid, dim3(256), s, x, H, N, amax);
        if (e == hipSuccess) e = launch(fp8_quant_kernel<32>, grid, dim3(256), s, x, y, H, N, (const uint32_t*)amax, scale);
    }
    return e;
}

// Workgroups of `kernel` resident on the device at once (CUs x occupancy),
// queried once per device and kernel.
template <typename K>
static int64_t resident_workgroups(K kernel, int threads) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const std::pair<int, const void*> key{dev, (const void*)kernel};
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
        return 0;
    return cache[key] = (int64_t)cus * per_cu;
}

template <int D, int WPE, bool KMASK>
static hipError_t launch_attn_fp8_t(const AttnArgs& a, const float* qs, const float* ks, const float* vs,
                                    hipStream_t s) {
    const int64_t n = attn_grid(a.n_work, a.head_mask != nullptr);
    const int one_round = n <= resident_workgroups(attn_fp8_kernel<D, WPE, KMASK>, 128) ? 1 : 0;
    return launch(attn_fp8_kernel<D, WPE, KMASK>, dim3((unsigned)n), dim3(128), s, a, qs, ks, vs, one_round);
}

hipError_t launch_attn_fp8(const AttnArgs& a, int D, const float* qs, const float* ks, const float* vs,
                           hipStream_t s) {
    if (a.key_mask != nullptr)
        return D == 128 ? launch_attn_fp8_t<128, 2, true>(a, qs, ks, vs, s) : launch_attn_fp8_t<64, 3, true>(a, qs, ks, vs, s);
    return D == 128 ? launch_attn_fp8_t<128, 2, false>(a, qs, ks, vs, s) : launch_attn_fp8_t<64, 3, false>(a, qs, ks, vs, s);
}

}  // namespace bsattn
