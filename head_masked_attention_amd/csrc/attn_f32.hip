// Block-sparse attention forward on the fp32 matrix cores (gfx950): fp32
// inputs, and the bf16 shapes the bf16 MFMA kernel does not cover (32-token
// blocks, D 32), with scores, softmax, P and the output accumulation in fp32.
//
// One wavefront per (b, h, 32 query rows).  Each kept key block is taken in
// 32-key tiles: S^T = K Q^T on v_mfma_f32_32x32x2f32 (D / 2 steps, the Q^T
// operand held in registers), an online softmax in fp32, then O^T += V^T P^T
// on the same instruction (16 steps per tile and 32-dimension slice).  The K
// rows enter the MFMA row slots in a fixed permutation (slot i holds key
// 2 r + h for output register r and lane half h), so the scores a lane holds
// after the first product are exactly the P^T operand it feeds to the second:
// P stays in fp32 in the lane that computed it.  K and V are read straight
// from global memory (L1/L2) in operand order; no LDS and no barriers.
// Key masks (per key, the masked_block consumer) set masked scores to -inf
// and skip wholly masked tiles; masked heads and rows with no kept key block
// write zeros.
//
// Sources: SD.Next commit view, modules/attention/sparse, flex-consumer
// paragraph (only the kept tiles are computed) and sparse-stage paragraph
// (token mask with the block mask); inferensys glossary, block-sparse entry
// (block structure on matrix hardware); haagenti_sparse crate docs (per-layer
// head masks).
#include "common.h"
#include "internal.h"

namespace bsattn {

namespace {

typedef float f16v32 __attribute__((ext_vector_type(16)));

// Elements 2 j + h (j = 0 .. 2 EPL - 1 ... of one 16-byte load): the values a
// lane of half h feeds to consecutive k-steps of the fp32 MFMA.
template <typename T>
struct Pairs;
template <>
struct Pairs<float> {
    static constexpr int PER = 2;     // k-steps per 16-byte load (4 fp32)
    __device__ static void get(const uint4 w, int h, float (&out)[2]) {
        out[0] = __uint_as_float(h ? w.y : w.x);
        out[1] = __uint_as_float(h ? w.w : w.z);
    }
};
template <>
struct Pairs<uint16_t> {
    static constexpr int PER = 4;     // k-steps per 16-byte load (8 bf16)
    __device__ static void get(const uint4 w, int h, float (&out)[4]) {
        const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(h ? (v[e] & 0xffff0000u) : (v[e] << 16));
    }
};

template <typename T>
__device__ __forceinline__ float load1(const T* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
    *(float4*)p = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
    uint2 w;
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)c) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)d) << 16);
    *(uint2*)p = w;   // round to nearest even, once
}

__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

template <typename T, int D, int BLOCK, bool KMASK>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
    constexpr int EPL = 16 / (int)sizeof(T);     // elements per 16-byte load
    constexpr int NL = D / EPL;                  // 16-byte loads per row
    constexpr int PER = Pairs<T>::PER;           // k-steps per load
    constexpr int NDT = D / 32;                  // 32-dimension slices of O^T
    constexpr int HALVES = BLOCK / 32;           // 32-row parts of a block
    static_assert(NL * PER == D / 2, "k-steps");

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    if (L >= a.n_work * HALVES) return;
    const int32_t hq = (int32_t)(L % HALVES);
    const int64_t item = L / HALVES;
    const int32_t qb = (int32_t)(item % a.nqb);
    const int64_t bh = item / a.nqb;
    const int32_t h = (int32_t)(bh % a.H);
    const int32_t b = (int32_t)(bh / a.H);
    const int32_t kvh = h / (a.H / a.Hkv);
    const int lane = threadIdx.x, hl = lane >> 5, ql = lane & 31;

    const bool active = a.head_mask == nullptr || a.head_mask[h] != 0;
    int32_t cnt = a.nkb;
    const int32_t* list = nullptr;
    if (a.count != nullptr) {
        const int64_t ms = (int64_t)(a.mB == 1 ? 0 : b) * a.mH + (a.mH == 1 ? 0 : h);
        cnt = a.count[ms * a.nqb + qb];
        list = a.index + (ms * a.nqb + qb) * (int64_t)a.nkb;
    }
    const int64_t q0 = (int64_t)qb * BLOCK + 32 * hq;            // first query row of the wavefront
    T* orow = (T*)a.o + b * a.o_sb + h * a.o_sh + (q0 + ql) * a.o_sn;   // this lane's query row
    if (!active || cnt <= 0) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) store4<T>(orow + 32 * dt + 8 * g + 4 * hl, 0.f, 0.f, 0.f, 0.f);
        return;
    }

    // Q^T operand: lane (hl, ql) holds Q[q0 + ql][2 j + hl] for k-step j
    float qf[D / 2];
    {
        const T* qr = (const T*)a.q.p + b * a.q.sb + h * a.q.sh + (q0 + ql) * a.q.sn;
#pragma unroll
        for (int c = 0; c < NL; ++c) {
            float v[PER];
            Pairs<T>::get(*(const uint4*)(qr + c * EPL), hl, v);
#pragma unroll
            for (int e = 0; e < PER; ++e) qf[c * PER + e] = v[e];
        }
    }
    const T* kbase = (const T*)a.k.p + b * a.k.sb + kvh * a.k.sh;
    const T* vbase = (const T*)a.v.p + b * a.v.sb + kvh * a.v.sh;
    // MFMA row slot ql of the S^T product holds key 2 r + h of the tile, with
    // r = 4 (ql / 8) + ql % 4 and h = (ql / 4) % 2: output register r of lane
    // half h then holds key 2 r + h
    const int slot_key = 2 * (4 * (ql >> 3) + (ql & 3)) + ((ql >> 2) & 1);
    const float sl2 = a.scale * 1.4426950408889634f;   // scale * log2(e)

    f16v32 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int32_t it = 0; it < cnt; ++it) {
        const int32_t kb = list != nullptr ? list[it] : it;
#pragma unroll
        for (int kt = 0; kt < BLOCK / 32; ++kt) {
            const int64_t k0 = (int64_t)kb * BLOCK + 32 * kt;      // first key of the tile
            uint32_t kw = 0xffffffffu;                             // bit k: key k of the tile live
            if constexpr (KMASK) {
                const uint8_t km = lane < 32 ? a.key_mask[(int64_t)b * a.km_sb + k0 + lane] : 1;
                kw = (uint32_t)__ballot(km != 0);
                if (kw == 0u) continue;                            // every key of the tile masked
            }
            // S^T = K Q^T
            f16v32 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
            const T* kr = kbase + (k0 + slot_key) * a.k.sn;
#pragma unroll
            for (int c = 0; c < NL; ++c) {
                float kv[PER];
                Pairs<T>::get(*(const uint4*)(kr + c * EPL), hl, kv);
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[c * PER + e], s, 0, 0, 0);
            }
            // online softmax in log2 units; register r of half hl is key 2 r + hl
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (KMASK && !((kw >> (2 * r + hl)) & 1u)) s[r] = -INFINITY;
                mx = fmaxf(mx, s[r]);
            }
            const float m_new = fmaxf(m_run, pair_max(mx) * sl2);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -inf
            m_run = m_new;
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -m_new));
                ps += s[r];
            }
            l_run = l_run * alpha + ps;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            // O^T += V^T P^T: k-step r takes keys 2 r (half 0) and 2 r + 1 (half 1)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const T* vr = vbase + (k0 + 2 * r + hl) * a.v.sn + ql;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(load1<T>(vr + 32 * dt), s[r], oacc[dt], 0, 0, 0);
            }
        }
    }
    // normalise and store: oacc[dt][r] = O[q0 + ql][32 dt + 8 (r / 4) + 4 hl + r % 4]
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;   // 0: every kept key masked
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            store4<T>(orow + 32 * dt + 8 * g + 4 * hl, oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                      oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
}

template <typename T, int D, bool KMASK>
static hipError_t launch_f32_t(const AttnArgs& a, int block, hipStream_t s) {
    const int64_t items = a.n_work * (block / 32);
    const dim3 grid((unsigned)(((items + kNumXcd - 1) / kNumXcd) * kNumXcd));
    if (block == 64) return launch(attn_f32_kernel<T, D, 64, KMASK>, grid, dim3(64), s, a);
    return launch(attn_f32_kernel<T, D, 32, KMASK>, grid, dim3(64), s, a);
}

template <typename T, bool KMASK>
static hipError_t launch_f32_d(const AttnArgs& a, int D, int block, hipStream_t s) {
    if (D == 32) return launch_f32_t<T, 32, KMASK>(a, block, s);
    if (D == 64) return launch_f32_t<T, 64, KMASK>(a, block, s);
    return launch_f32_t<T, 128, KMASK>(a, block, s);
}

hipError_t launch_attn_f32(const AttnArgs& a, int dtype_is_f32, int D, int block, hipStream_t s) {
    const bool km = a.key_mask != nullptr;
    if (dtype_is_f32)
        return km ? launch_f32_d<float, true>(a, D, block, s) : launch_f32_d<float, false>(a, D, block, s);
    return km ? launch_f32_d<uint16_t, true>(a, D, block, s) : launch_f32_d<uint16_t, false>(a, D, block, s);
}

}  // namespace bsattn
