// Block-sparse attention forward, fp32 vector path (gfx950).
//
// Used for fp32 inputs, whose products and softmax must stay in fp32 end to
// end, and for bf16 shapes the MFMA kernel does not cover (block 32, D 32).
// One workgroup per (b, h, query block), one thread per query row.  Each kept
// key block is staged in LDS as fp32; every thread reads the same K/V row at
// the same time (LDS broadcast).  The online softmax keeps a running max and
// denominator per row, as in the MFMA path; products and sums are fp32.
//
// Sources: SD.Next commit view, modules/attention/sparse, flex-consumer
// paragraph; inferensys glossary, block-sparse entry; haagenti_sparse crate
// docs (per-layer head masks).
#include "common.h"
#include "internal.h"

namespace bsattn {

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) {
    return __uint_as_float((uint32_t)(*p) << 16);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, float v) {
    const __bf16 b = (__bf16)v;    // round to nearest even
    *p = __builtin_bit_cast(uint16_t, b);
}

template <typename T, int D, int BLOCK>
__global__ __launch_bounds__(BLOCK) void attn_vec_kernel(AttnArgs a) {
    __shared__ float Ks[BLOCK][D];
    __shared__ float Vs[BLOCK][D];
    __shared__ float Bs[BLOCK];        // 0 for a live key, -inf for a masked one

    const int64_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    if (L >= a.n_work) return;
    const int32_t qb = (int32_t)(L % a.nqb);
    const int64_t bh = L / a.nqb;
    const int32_t h = (int32_t)(bh % a.H);
    const int32_t b = (int32_t)(bh / a.H);
    const int32_t kvh = h / (a.H / a.Hkv);
    const int t = threadIdx.x;

    const bool active = (a.head_mask == nullptr) || (a.head_mask[h] != 0);
    int32_t cnt = a.nkb;
    const int32_t* list = nullptr;
    if (a.count != nullptr) {
        const int64_t ms = (int64_t)(a.mB == 1 ? 0 : b) * a.mH + (a.mH == 1 ? 0 : h);
        cnt = a.count[ms * a.nqb + qb];
        list = a.index + (ms * a.nqb + qb) * (int64_t)a.nkb;
    }
    T* orow = (T*)a.o + b * a.o_sb + h * a.o_sh + ((int64_t)qb * BLOCK + t) * a.o_sn;
    if (!active || cnt <= 0) {
        for (int d = 0; d < D; ++d) store_elem<T>(orow + d, 0.f);
        return;
    }

    const T* qrow = (const T*)a.q.p + b * a.q.sb + h * a.q.sh + ((int64_t)qb * BLOCK + t) * a.q.sn;
    const T* kbase = (const T*)a.k.p + b * a.k.sb + kvh * a.k.sh;
    const T* vbase = (const T*)a.v.p + b * a.v.sb + kvh * a.v.sh;

    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) { q[d] = load_elem<T>(qrow + d); o[d] = 0.f; }
    float m_run = -INFINITY, l_run = 0.f;

    for (int32_t it = 0; it < cnt; ++it) {
        const int32_t kb = list ? list[it] : it;
        __syncthreads();
        const T* kr = kbase + ((int64_t)kb * BLOCK + t) * a.k.sn;
        const T* vr = vbase + ((int64_t)kb * BLOCK + t) * a.v.sn;
        for (int d = 0; d < D; ++d) { Ks[t][d] = load_elem<T>(kr + d); Vs[t][d] = load_elem<T>(vr + d); }
        Bs[t] = (a.key_mask == nullptr || a.key_mask[b * a.km_sb + (int64_t)kb * BLOCK + t] != 0) ? 0.f : -INFINITY;
        __syncthreads();

        // pass 1: block max of the scaled scores; pass 2 recomputes each score
        // with identical arithmetic and accumulates (no per-thread score array)
        float mx = -INFINITY;
        for (int j = 0; j < BLOCK; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[j][d], acc);
            mx = fmaxf(mx, acc * a.scale + Bs[j]);
        }
        if (mx == -INFINITY) continue;   // every key of this block masked
        const float m_new = fmaxf(m_run, mx);
        const float alpha = expf(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        for (int j = 0; j < BLOCK; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[j][d], acc);
            const float p = expf(acc * a.scale + Bs[j] - m_new);
            psum += p;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[j][d], o[d]);
        }
        l_run = l_run * alpha + psum;
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;   // 0: every kept key masked
    for (int d = 0; d < D; ++d) store_elem<T>(orow + d, o[d] * inv);
}

template <typename T, int D>
static hipError_t launch_vec_t(const AttnArgs& a, int block, hipStream_t s) {
    const int64_t padded = ((a.n_work + kNumXcd - 1) / kNumXcd) * kNumXcd;
    const dim3 grid((unsigned)padded);
    if (block == 64) return launch(attn_vec_kernel<T, D, 64>, grid, dim3(64), s, a);
    return launch(attn_vec_kernel<T, D, 32>, grid, dim3(32), s, a);
}

hipError_t launch_attn_vec(const AttnArgs& a, int dtype_is_f32, int D, int block, hipStream_t s) {
    if (dtype_is_f32) {
        if (D == 32) return launch_vec_t<float, 32>(a, block, s);
        if (D == 64) return launch_vec_t<float, 64>(a, block, s);
        return launch_vec_t<float, 128>(a, block, s);
    }
    if (D == 32) return launch_vec_t<uint16_t, 32>(a, block, s);
    if (D == 64) return launch_vec_t<uint16_t, 64>(a, block, s);
    return launch_vec_t<uint16_t, 128>(a, block, s);
}

}  // namespace bsattn
