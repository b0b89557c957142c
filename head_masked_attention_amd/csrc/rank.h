// Wavefront ranking helpers shared by the selector and the fused
// select-and-attend kernel (gfx950): lane exchanges, the order-preserving
// key of a score, and the descending bitonic sort of 32-bit keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

// The value of lane (lane ^ m), m a power of two below 64 known at compile
// time after unrolling, without the LDS crossbar where the VALU can do it:
// DPP quad permutes for 1 and 2, mirror compositions for 4 (i ^ 7 ^ 3) and 8
// (i ^ 15 ^ 7), a swizzle for 16 and the half swap for 32 (which returns the
// lower half's value first and the upper half's second, on every lane).
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int m) {
    switch (m) {
    case 1: return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);          // quad_perm [1,0,3,2]
    case 2: return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);          // quad_perm [2,3,0,1]
    case 4: return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false),
                                            0x1B, 0xF, 0xF, false);            // row_half_mirror, quad_perm [3,2,1,0]
    case 8: return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false),
                                            0x141, 0xF, 0xF, false);           // row_mirror, row_half_mirror
    case 16: return __builtin_amdgcn_ds_swizzle(x, 0x1F | (0x10 << 10));        // bit mode, xor 16
    case 32: {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (__lane_id() & 32) ? r[0] : r[1];
    }
    default: return __shfl_xor(x, m);
    }
}

// lane_xor of a float64 (its two 32-bit halves exchanged the same way).
__device__ __forceinline__ double lane_xor_f64(double x, int m) {
    const uint64_t u = __double_as_longlong(x);
    const uint32_t lo = lane_xor((uint32_t)u, m), hi = lane_xor((uint32_t)(u >> 32), m);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Order-preserving map of a float64 to uint64 (-0 taken as +0).
__device__ __forceinline__ uint64_t orderable64(double f) {
    uint64_t u = (uint64_t)__double_as_longlong(f);
    if ((u << 1) == 0) u = 0;                       // -0 -> +0
    return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Order-preserving map of a float to uint32 (-0 taken as +0).
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;                       // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Descending bitonic sort of R independent rows of 64*E 32-bit keys, one
// wavefront per row set; element e = lane * E + r of row q lives in key[q][r].
// The R networks are interleaved so their shuffles overlap.
template <int R, int E>
__device__ __forceinline__ void wave_bitonic_desc32(uint32_t (&key)[R][E], int lane) {
    constexpr int NTOT = 64 * E;
#pragma unroll
    for (int size = 2; size <= NTOT; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride < E) {
#pragma unroll
                for (int q = 0; q < R; ++q)
#pragma unroll
                    for (int r = 0; r < E; ++r) {
                        if (r & stride) continue;
                        const bool desc = ((lane * E + r) & size) == 0;
                        const uint32_t a = key[q][r], b = key[q][r | stride];
                        const uint32_t hi = max(a, b), lo = min(a, b);
                        key[q][r] = desc ? hi : lo;
                        key[q][r | stride] = desc ? lo : hi;
                    }
            } else {
                const int lm = stride / E;
#pragma unroll
                for (int q = 0; q < R; ++q)
#pragma unroll
                    for (int r = 0; r < E; ++r) {
                        const int e = lane * E + r;
                        const uint32_t other = lane_xor(key[q][r], lm);
                        const bool take_max = ((e & stride) == 0) == ((e & size) == 0);
                        key[q][r] = take_max ? max(key[q][r], other) : min(key[q][r], other);
                    }
            }
        }
    }
}

// Wavefront-wide maximum and minimum (every lane gets the result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = max(v, lane_xor(v, off));
    return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = min(v, lane_xor(v, off));
    return v;
}

// Inclusive prefix sum over the lanes of a wavefront: Hillis-Steele steps by
// DPP row shifts inside each row of 16 lanes, then the row totals added on.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v, int lane) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                   r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// The n-th largest (n >= 1) of the keys of one row that take part (part[r]),
// the row's 64 * E keys spread over a wavefront (element lane * E + r in
// key[r]); at least n keys take part.  Most-significant-digit radix
// selection: the leading bits that every taking part key shares (from the
// wavefront's minimum and maximum) are fixed at once; then each pass counts
// the keys that agree with the bits fixed so far by the value of their next
// DB bits, in 2^DB 32-bit counters of LDS (`hist`, 16-byte aligned, this
// wavefront's own), and fixes the digit whose bucket holds rank n.  When rank
// n becomes the bucket's largest or smallest key the pass ends the search
// with a wavefront maximum or minimum.  Returns the key itself.
template <int E, int DB>
__device__ __forceinline__ uint32_t wave_kth_key(const uint32_t (&key)[E], const bool (&part)[E], int n,
                                                 int lane, uint32_t* hist) {
    constexpr int BPL = (1 << DB) / 64;                  // counters per lane
    static_assert(BPL == 2 || BPL == 4, "2^DB counters: 128 or 256");
    // keys that take no part become 0: below every key that does, so that
    // counting them changes no rank up to the number taking part
    uint32_t sk[E];
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        sk[r] = part[r] ? key[r] : 0u;
        lo = min(lo, part[r] ? key[r] : 0xffffffffu);
        hi = max(hi, sk[r]);
    }
    // wave-uniform from here on: the search runs on scalar registers
    lo = __builtin_amdgcn_readfirstlane(wave_min_u32(lo));
    hi = __builtin_amdgcn_readfirstlane(wave_max_u32(hi));
    if (n == 1 || lo == hi) return hi;
    int s = 32 - __clz((int)(lo ^ hi));                  // bits s.. 31 are shared
    uint32_t fmask = s == 32 ? 0u : ~0u << s;
    uint32_t prefix = hi & fmask;
    uint32_t need = (uint32_t)n;
    while (s > 0) {
        const int b = s < DB ? s : DB, shift = s - b;
        if constexpr (BPL == 4) *(uint4*)(hist + 4 * lane) = uint4{0u, 0u, 0u, 0u};
        else *(uint2*)(hist + 2 * lane) = uint2{0u, 0u};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < E; ++r)
            // DB bits from `shift` (in the last, narrower pass the top ones are
            // fixed bits, equal for every counted key: the digit only moves)
            if ((sk[r] & fmask) == prefix) atomicAdd(hist + __builtin_amdgcn_ubfe(sk[r], shift, DB), 1u);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t c[BPL];
        if constexpr (BPL == 4) {
            const uint4 w = *(const uint4*)(hist + 4 * lane);
            c[0] = w.x; c[1] = w.y; c[2] = w.z; c[3] = w.w;
        } else {
            const uint2 w = *(const uint2*)(hist + 2 * lane);
            c[0] = w.x; c[1] = w.y;
        }
        uint32_t tot = 0;
#pragma unroll
        for (int i = 0; i < BPL; ++i) tot += c[i];
        const uint32_t incl = wave_prefix_sum(tot, lane);
        const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
        // ge[i]: keys in digits >= lane * BPL + i (non-increasing over the digits)
        uint32_t ge[BPL];
        ge[0] = total - (incl - tot);
#pragma unroll
        for (int i = 1; i < BPL; ++i) ge[i] = ge[i - 1] - c[i - 1];
        const uint64_t bal = __ballot(ge[0] >= need);    // lane 0 always: ge[0] = total >= need
        const int L = 63 - __clzll((long long)(bal | 1ull));
        int j = 0;
        uint32_t above = ge[0] - c[0], cnt = c[0];
#pragma unroll
        for (int i = 1; i < BPL; ++i)
            if (ge[i] >= need) { j = i; above = ge[i] - c[i]; cnt = c[i]; }
        const uint32_t d = (uint32_t)(L * BPL) + (uint32_t)__builtin_amdgcn_readlane(j, L);
        need -= __builtin_amdgcn_readlane(above, L);
        const uint32_t in_bucket = __builtin_amdgcn_readlane(cnt, L);
        prefix |= d << shift;
        fmask = ~0u << shift;
        s = shift;
        __builtin_amdgcn_wave_barrier();
        if (s > 0 && (need == 1 || need == in_bucket)) {
            // rank n is the bucket's largest (need 1) or smallest key
            uint32_t v = need == 1 ? 0u : 0xffffffffu;
#pragma unroll
            for (int r = 0; r < E; ++r)
                if ((sk[r] & fmask) == prefix) v = need == 1 ? max(v, sk[r]) : min(v, sk[r]);
            return __builtin_amdgcn_readfirstlane(need == 1 ? wave_max_u32(v) : wave_min_u32(v));
        }
    }
    return prefix;
}

}  // namespace bsattn
