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

}  // namespace bsattn
