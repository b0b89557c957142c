// Shared device/host definitions of libbsattn (gfx950).
//
// The layout of a packed sequence reaches the kernels as a run-length
// encoding of the per-block classes, passed by value as a kernel argument
// (no host-to-device copy and no device state): the SD.Next synchronisation
// paragraph moves everything that depends only on geometry and layout to the
// host, so a call never reads a device value back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace bsattn {

enum BlockClass : int32_t { CLS_SPARSE = 0, CLS_PINNED = 1, CLS_DROPPED = 2 };

constexpr int kMaxRuns = 72;      // class runs; <= 2 * BSATTN_MAX_SEGMENTS + 1 in practice
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int64_t kL2BytesPerXcd = 4 << 20;   // MI355X: 4 MB of L2 per XCD
constexpr int kMaxCand = 2048;    // sparsifiable blocks handled by the selector

// Rows per (b, head) of the pooled sums in the selector workspace: the
// candidates, padded to whole 16-row tiles.
__host__ __device__ __forceinline__ int64_t pooled_rows(int64_t n_cand) { return (n_cand + 15) / 16 * 16; }

// Element (p, d) of a head's pooled sums in the selector workspace: 16-row
// tiles stored in the order the score MFMA reads its operands (see the
// selector source for the derivation).
template <int D>
__device__ __forceinline__ int64_t pooled_offset(int32_t p, int32_t d) {
    constexpr int KQ = D / 4;
    const int li = p & 15, gq = d / KQ, c = (d % KQ) >> 2, e = d & 3;
    return (int64_t)(p >> 4) * 16 * D + ((c * 4 + gq) * 16 + li) * 4 + e;
}

// Block sums of one tensor (Q or K) in the selector workspace, per (b, head)
// and candidate row: the float64 sum split into a float32 high part `hi` (in
// the score MFMA's operand order, pooled_offset) and the float32 residual `lo`
// (same order), so hi + lo carries the sum to about 2^-48 relative; and `nrm`,
// an upper bound on the Euclidean norm of the row's hi part.  hi == NULL: the
// tensor is not pooled.
struct PooledSums {
    float* hi;
    float* lo;
    float* nrm;
};

// Per-layout geometry, host-computed once per call and passed by value.
struct Geometry {
    int32_t nb;          // blocks in the sequence (N / block)
    int32_t block;       // tokens per block
    int32_t n_cand;      // SPARSE blocks (selector candidates)
    int32_t n_other;     // PINNED + DROPPED blocks
    int32_t k;           // candidates kept per SPARSE row
    int32_t is_dense;    // k >= n_cand
    int32_t w;           // window half-width in blocks, -1 = no window
    int32_t n_runs;
    int32_t run_first[kMaxRuns];   // first block of the run
    int32_t run_len[kMaxRuns];     // blocks in the run
    int32_t run_cls[kMaxRuns];     // BlockClass of every block in the run
    int32_t run_off[kMaxRuns];     // position of run_first among blocks of the
                                   // same group (SPARSE, or PINNED+DROPPED)
};

// Strided view of a [B][H][N][D] tensor; D contiguous.  Strides in elements.
struct TView {
    const void* p;
    int64_t sb, sh, sn;
};

struct MaskOut {
    uint8_t* mask;       // [B][H][nqb][nkb]
    int32_t* count;      // [B][H][nqb]
    int32_t* index;      // [B][H][nqb][nkb]
};

// ---- run lookups (runs are few; a linear scan is cheapest) ----------------
// The fields of the first kFastRuns runs are read at constant indices into
// SGPRs: wave-uniform scalar loads that the compiler issues with the other
// kernel arguments.  Indexed reads would be per-lane vector loads of the
// uncached argument block, one dependent round trip each, whenever lanes look
// up different blocks.  (The empty asm keeps the optimizer from folding the
// reads of different runs back into one indexed load.)  Runs past kFastRuns,
// layouts of many segments, take the indexed loop.
constexpr int kFastRuns = 4;

struct Run {
    int32_t first, len, cls, off;
};
__device__ __forceinline__ int32_t pin_sgpr(int32_t v) {
    asm volatile("" : "+s"(v));
    return v;
}
template <int R>
__device__ __forceinline__ Run fast_run(const Geometry& g) {
    return {pin_sgpr(g.run_first[R]), pin_sgpr(g.run_len[R]), pin_sgpr(g.run_cls[R]), pin_sgpr(g.run_off[R])};
}
__device__ __forceinline__ Run slow_run(const Geometry& g, int r) {
    return {g.run_first[r], g.run_len[r], g.run_cls[r], g.run_off[r]};
}

// f(run) returns true when the run answers the lookup (it stores the answer);
// runs are visited in order and the first answer wins.
template <typename F>
__device__ __forceinline__ bool visit_runs(const Geometry& g, F f) {
    if (g.n_runs > 0 && f(fast_run<0>(g))) return true;
    if (g.n_runs > 1 && f(fast_run<1>(g))) return true;
    if (g.n_runs > 2 && f(fast_run<2>(g))) return true;
    if (g.n_runs > 3 && f(fast_run<3>(g))) return true;
    static_assert(kFastRuns == 4, "fast runs visited above");
    for (int r = kFastRuns; r < g.n_runs; ++r)
        if (f(slow_run(g, r))) return true;
    return false;
}

__device__ __forceinline__ int32_t block_class(const Geometry& g, int32_t j) {
    int32_t cls = CLS_DROPPED;
    visit_runs(g, [&](const Run& u) {
        if (j >= u.first + u.len) return false;
        cls = u.cls;
        return true;
    });
    return cls;
}

// Block index of the pos-th SPARSE block.
__device__ __forceinline__ int32_t cand_block(const Geometry& g, int32_t pos) {
    int32_t blk = -1;
    visit_runs(g, [&](const Run& u) {
        if (u.cls != CLS_SPARSE || pos >= u.off + u.len) return false;
        blk = u.first + (pos - u.off);
        return true;
    });
    return blk;
}

// Block index of the pos-th non-SPARSE block.
__device__ __forceinline__ int32_t other_block(const Geometry& g, int32_t pos) {
    int32_t blk = -1;
    visit_runs(g, [&](const Run& u) {
        if (u.cls == CLS_SPARSE || pos >= u.off + u.len) return false;
        blk = u.first + (pos - u.off);
        return true;
    });
    return blk;
}

// Column code used by the compaction passes: candidate position (>= 0) for a
// SPARSE block, -1 for PINNED, -2 for DROPPED.
__device__ __forceinline__ int32_t column_code(const Geometry& g, int32_t j) {
    int32_t code = -2;
    visit_runs(g, [&](const Run& u) {
        if (j >= u.first + u.len) return false;
        code = u.cls == CLS_SPARSE ? u.off + (j - u.first) : (u.cls == CLS_PINNED ? -1 : -2);
        return true;
    });
    return code;
}

// XCD-aware workgroup order: hardware workgroup w runs on XCD w % 8, so the
// logical id groups consecutive logical work (the query blocks of one head)
// on one XCD and its L2.  `padded` is the launched grid, a multiple of 8;
// logical ids >= the real count exit.
__device__ __forceinline__ int64_t xcd_logical_id(int64_t w, int64_t padded) {
    const int64_t per = padded / kNumXcd;
    return (w % kNumXcd) * per + (w / kNumXcd);
}

// Work order under a per-layer head mask (one wavefront's view; every
// wavefront of a workgroup computes the same).  Hardware workgroup w runs on
// XCD w % 8 as that XCD's (w / 8)-th workgroup.  The active heads' query
// blocks (A items, in (b, active head, query block) order) and the masked
// heads' (I items) are each split into eight equal contiguous shares, and XCD
// x takes its share of active items first, then its share of masked ones:
// the kept work spreads evenly over the XCDs whatever heads the mask keeps,
// and one head's query blocks stay neighbours on one XCD.  The grid holds
// 8 * (ceil(n_work / 8) + 1) workgroups, enough for both shares of every XCD;
// workgroups past them get valid = false.
struct HeadWork {
    int32_t b, h, qb;
    bool active, valid;
};

__device__ __forceinline__ HeadWork head_masked_order(int64_t w, int64_t padded, const uint8_t* head_mask,
                                                      int32_t B, int32_t H, int32_t nqb) {
    const int lane = threadIdx.x & 63;
    int32_t n_act = 0;
    for (int32_t h0 = 0; h0 < H; h0 += 64)
        n_act += __popcll(__ballot(h0 + lane < H && head_mask[h0 + lane] != 0));
    const int64_t A = (int64_t)B * n_act * nqb;
    const int64_t I = (int64_t)B * (H - n_act) * nqb;
    const int64_t x = w % kNumXcd, s = w / kNumXcd;
    const int64_t a0 = x * A / kNumXcd, a1 = (x + 1) * A / kNumXcd;
    const int64_t i0 = x * I / kNumXcd, i1 = (x + 1) * I / kNumXcd;
    (void)padded;
    HeadWork hw;
    hw.valid = true;
    int64_t item;
    if (s < a1 - a0) { hw.active = true; item = a0 + s; }
    else if (s - (a1 - a0) < i1 - i0) { hw.active = false; item = i0 + (s - (a1 - a0)); }
    else { hw.valid = false; hw.active = false; hw.b = hw.h = hw.qb = 0; return hw; }
    const int32_t nh = hw.active ? n_act : H - n_act;
    hw.qb = (int32_t)(item % nqb);
    const int64_t r = item / nqb;
    int32_t j = (int32_t)(r % nh);
    hw.b = (int32_t)(r / nh);
    hw.h = 0;
    for (int32_t h0 = 0; h0 < H; h0 += 64) {
        uint64_t m = __ballot(h0 + lane < H && (head_mask[h0 + lane] != 0) == hw.active);
        const int32_t c = __popcll(m);
        if (j < c) {
            for (int32_t k = 0; k < j; ++k) m &= m - 1;   // drop the j lowest set bits
            hw.h = h0 + __builtin_ctzll(m);
            break;
        }
        j -= c;
    }
    return hw;
}

// Grid of the attention kernels: n_work workgroups padded to a multiple of
// the XCD count, plus one more round of eight under a head mask.
__host__ __forceinline__ int64_t attn_grid(int64_t n_work, bool head_masked) {
    return ((n_work + kNumXcd - 1) / kNumXcd + (head_masked ? 1 : 0)) * kNumXcd;
}

// LDS-DMA of one 16-byte chunk per lane through a buffer resource based at
// `base` (raw buffer, 32-bit data format; the range only has to cover the
// stage tile): lane l's chunk at base + off lands at dst + 16 l.  The loads
// of a tile share the scalar resource, so each is base plus the lane's
// 32-bit offset with no per-load address arithmetic.
// (Kernels build their resources only through helpers like this one: a
// kernel body that itself named the buffer-resource type compiled without
// error, but hipcc's host pass then left that file's kernel launch stubs
// undefined and the library would not load.)
__device__ __forceinline__ void chunk_to_lds(const void* base, uint32_t off, void* dst) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Launches `kernel` and returns the status of this launch itself (not an
// error left pending by earlier, unrelated runtime calls).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args&&... args) {
    std::tuple<std::decay_t<KArgs>...> vals(std::forward<Args>(args)...);
    void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto&... v) {
        size_t i = 0;
        ((ptrs[i++] = (void*)&v), ...);
    }, vals);
    return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, s);
}

}  // namespace bsattn
