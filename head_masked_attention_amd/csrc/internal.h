// Kernel launchers shared between the C-ABI layer and the kernel sources.
#pragma once

#include "common.h"

namespace bsattn {

// Arguments of the attention kernels (by value).
struct AttnArgs {
    TView q, k, v;
    void* o;
    int64_t o_sb, o_sh, o_sn;
    int32_t B, H, Hkv, nqb, nkb;
    int32_t mB, mH;              // mask batch/head extents (1 = shared)
    const int32_t* count;        // NULL = dense (every block kept)
    const int32_t* index;
    const uint8_t* head_mask;    // NULL = every head active
    const uint8_t* key_mask;     // NULL = every key live; else key_mask[b * km_sb + j]
    int64_t km_sb;               // batch stride of key_mask (0 = shared)
    float scale;                 // softmax scale (> 0)
    int64_t n_work;              // B * H * nqb workgroups of real work
    // fused selection (bsattn_select_forward): the selector's pooled key
    // sums (each workgroup sums its own query block), the candidates kept
    // per row, and the block mask written out
    const float* kp;             // [B][Hkv][prow][D] hi parts, NULL in the plain forward
    const float* kp_lo;          // ... and their float32 residuals (same layout)
    int32_t prow;                // pooled rows per head
    int32_t keep;                // k
    uint8_t* m_out;
    int32_t* c_out;
    int32_t* i_out;
};

// Selector workspace: PooledSums of Q ([B][H] heads) then of K ([B][Hkv]
// heads), `rows` candidate rows per head, D dimensions; every part 256-byte
// aligned.  Offsets in bytes from the workspace base.
struct PoolSpace {
    size_t q_hi, k_hi, q_lo, k_lo, q_nrm, k_nrm, bytes;
};
__host__ inline size_t align_up256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ inline PoolSpace pool_space(int64_t B, int64_t H, int64_t Hkv, int64_t rows, int64_t D) {
    PoolSpace ps;
    const size_t qs = align_up256((size_t)B * H * rows * D * 4), ks = align_up256((size_t)B * Hkv * rows * D * 4);
    const size_t qn = align_up256((size_t)B * H * rows * 4), kn = align_up256((size_t)B * Hkv * rows * 4);
    ps.q_hi = 0;
    ps.k_hi = qs;
    ps.q_lo = qs + ks;
    ps.k_lo = 2 * qs + ks;
    ps.q_nrm = 2 * (qs + ks);
    ps.k_nrm = 2 * (qs + ks) + qn;
    ps.bytes = 2 * (qs + ks) + qn + kn;
    return ps;
}
__host__ inline PooledSums pooled_part(void* ws, size_t hi, size_t lo, size_t nrm) {
    char* b = (char*)ws;
    return PooledSums{(float*)(b + hi), (float*)(b + lo), (float*)(b + nrm)};
}

// xcd_groups: the selector's two launches take their work in the attention
// kernel's XCD-grouped (b, K/V head) order, so that pooled sums, masks and
// lists are written by the XCD whose attention workgroups read them next
// (chosen by the host when an XCD's share of Q and K fits in its L2).
// qp.hi NULL: pool K only.
// head_mask (device uint8 [H] or NULL): the heads whose byte is 0 are not
// pooled or ranked; their rows are written empty.
hipError_t launch_pool(int dtype_is_f32, int D, int block, TView q, TView k, int B, int H,
                       int Hkv, const Geometry& g, PooledSums qp, PooledSums kp, int xcd_groups,
                       const uint8_t* head_mask, hipStream_t s);
hipError_t launch_score_rank(int D, PooledSums qp, PooledSums kp, int B, int H, int Hkv,
                             const Geometry& g, MaskOut out, int xcd_groups, const uint8_t* head_mask,
                             hipStream_t s);
// slices: B * H (slice b * H + h); the head mask applies when H > 0
hipError_t launch_layout_fill(const Geometry& g, int slices, int H, const uint8_t* head_mask, MaskOut out,
                              hipStream_t s);
// bf16, D 64, block 64, every block a candidate (nkb <= 64), no head or key
// mask: each workgroup sums its query block, ranks its row against the
// pooled key sums, writes the row of the block mask and attends over the
// kept blocks.
hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t s);

// bf16, block 64, D in {64, 128}: MFMA path.
hipError_t launch_attn_mfma(const AttnArgs& a, int D, hipStream_t s);
// fp8 (e4m3) q/k/v with per-(b, head) scales, block 64, D in {64, 128}; bf16 out.
hipError_t launch_attn_fp8(const AttnArgs& a, int D, const float* q_scale, const float* k_scale,
                           const float* v_scale, hipStream_t s);
// bf16 [B][H][N][D] -> e4m3 codes + per-(b, head) scale; amax: B*H words of scratch.
hipError_t launch_quant_fp8(TView x, TView y, int B, int H, int64_t N, int D, uint32_t* amax, float* scale,
                            hipStream_t s);
// fp32 inputs, and bf16 of block 32 or D 32: fp32 MFMA path (block 32/64, D 32/64/128).
hipError_t launch_attn_f32(const AttnArgs& a, int dtype_is_f32, int D, int block, hipStream_t s);

}  // namespace bsattn
