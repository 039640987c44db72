// Fragment helpers shared by the matrix-core attention kernels (bf16, head dim 512).
#pragma once

#include "attn_rows.hpp"
#include "common.hpp"

namespace csa {
namespace amfma {

constexpr int WD = 512;         // head dim
constexpr int WR = 32;          // rows per tile
constexpr int KKN = WD / 32;    // k-chunks of S^T (q^T fragments)
constexpr int NDN = WD / 16;    // 16-dim output tiles
constexpr float kLazy = 16.f;   // log2 headroom of the reference maximum
constexpr int kIdxCache = 3072; // top-k indices of one split kept in LDS (more are read from memory)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef unsigned int u32x4w __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
// word 3 of a raw buffer resource on gfx9-class parts (32-bit data format, no swizzle)
constexpr int kBufDword3 = 0x00020000;
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2w __attribute__((ext_vector_type(2)));  // converts with v_cvt_pk_bf16_f32 (RNE)
// two fp32 values rounded to nearest-even bf16 and packed (low = a) by v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2w));
}

// B operand of ones (bf16 1.0 = 0x3f80): P x ones gives every head's row sum of P
__device__ __forceinline__ bf16x8 ones_bf16x8() {
    return __builtin_bit_cast(bf16x8, u32x4w{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
}

// Row scaling of a 16x16 fp32 accumulator tile on the matrix cores: row i (head 4g + r of
// the C layout) times alpha_i. With A_r[i][k] = alpha_i if i == 4k + r (else 0) and
// B_r[k][n] = C[4k + r][n] (component r of every lane), sum_r A_r B_r = diag(alpha) C,
// four 16x16x4 fp32 products, each exact to one fp32 rounding. ar[r] is alpha_i on the lane
// with l % 16 == 4 (l / 16) + r and 0 elsewhere.
__device__ __forceinline__ f32x4 scale_rows(const f32x4 c, const float ar[4]) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) z = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[r], c[r], z, 0, 0, 0);
    return z;
}

// LDS pitch of a tile row: 512 bf16 + 16 bf16 of padding. With the 32-byte pad both the
// 16-byte row-fragment reads of 16 rows and the transposing reads of 16 rows x 32 bytes
// are spread over all banks (measured ~190-205 B/clk/CU, against ~117 for an unpadded
// XOR-swizzled row).
constexpr int WP = WD + 16;

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4w *>(p));
}

__device__ __forceinline__ v4i16 ld_tr(const bf16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)((__attribute__((address_space(3))) bf16_t *)p));
}

// Row of slot j of a query (a top-k row, a summary or an SWA row), or `standin` when the
// slot holds no row. Slots [j0, j0 + kIdxCache) of the top-k list are read from `sidx`.
// kv_row: bf16 elements between consecutive compressed rows (WD, or half the byte size of
// an FP8-format row).
__device__ __forceinline__ const bf16_t *slot_row(const RowCtx &c, int64_t j, int64_t j0, int64_t j1, int ratio,
                                                  const int32_t *sidx, const int32_t *idx_t, int64_t N,
                                                  const bf16_t *kv, const bf16_t *swa, int swa_rows,
                                                  const bf16_t *standin, int64_t kv_row = WD) {
    const bf16_t *p = standin;
    if (j < j1) {
        if (j < c.nmain) {
            const int64_t id = (ratio > 0) ? j : (j - j0 < kIdxCache ? (int64_t)sidx[j - j0] : (int64_t)idx_t[j]);
            if (id >= 0 && id < N) p = kv + ((int64_t)c.s * N + id) * kv_row;
        } else {
            const int64_t r = c.lo + (j - c.nmain) - c.swa0;
            if (r >= 0 && r < swa_rows) p = swa + ((int64_t)c.s * swa_rows + r) * WD;
        }
    }
    return p;
}

// Rotation of the last R dims of a q^T fragment (dims 32kk + 8g .. +7), in fp32, rounded
// once to bf16; fragments below the rotated dims pass through.
__device__ __forceinline__ bf16x8 rope_fragment(bf16x8 v, int kk, int g, const float *rope_t, int R) {
    const int d0 = 32 * kk + 8 * g;
    if (rope_t == nullptr || d0 + 8 <= WD - R) return v;
    const u32x4w raw = __builtin_bit_cast(u32x4w, v);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x0 = lo_bf16(raw[e]), x1 = hi_bf16(raw[e]);
        const int d = d0 + 2 * e;
        if (d >= WD - R) {
            const int p = (d - (WD - R)) >> 1;
            const float cs = rope_t[2 * p], sn = rope_t[2 * p + 1];
            const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
            x0 = y0;
            x1 = y1;
        }
        o[e] = pack_bf16x2(x0, x1);
    }
    return __builtin_bit_cast(bf16x8, u32x4w{o[0], o[1], o[2], o[3]});
}

// The same rotation with the fragment's four (cos, sin) pairs already in registers.
__device__ __forceinline__ bf16x8 rope_fragment_cs(bf16x8 v, int kk, int g, const float cs[4], const float sn[4],
                                                   int R) {
    const int d0 = 32 * kk + 8 * g;
    if (d0 + 8 <= WD - R) return v;
    const u32x4w raw = __builtin_bit_cast(u32x4w, v);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x0 = lo_bf16(raw[e]), x1 = hi_bf16(raw[e]);
        if (d0 + 2 * e >= WD - R) {
            const float y0 = x0 * cs[e] - x1 * sn[e], y1 = x0 * sn[e] + x1 * cs[e];
            x0 = y0;
            x1 = y1;
        }
        o[e] = pack_bf16x2(x0, x1);
    }
    return __builtin_bit_cast(bf16x8, u32x4w{o[0], o[1], o[2], o[3]});
}

// (cos, sin) of the pair holding dim d, or of pair 0 when d is not rotated (the caller
// ignores it then); always a valid table entry, so a batch of these loads needs no branch
__device__ __forceinline__ float2 rope_pair(const float *rope_t, int d, int R) {
    const int p = d >= WD - R ? (d - (WD - R)) >> 1 : 0;
    return *reinterpret_cast<const float2 *>(rope_t + 2 * p);
}

// raw buffer resource over `bytes` bytes from p, with the address read out of lane 0 (the
// caller passes a wave-uniform pointer) so the resource sits in scalar registers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, (int)bytes, kBufDword3);
}

// q^T fragment (B operand of S^T = K Q^T) of one head: dims 32kk + 8g .. +7 of row `qrow`,
// with the rotation of the last R dims applied.
__device__ __forceinline__ bf16x8 q_fragment(const bf16_t *qrow, int kk, int g, const float *rope_t, int R) {
    return rope_fragment(ld_bf16x8(qrow + 32 * kk + 8 * g), kk, g, rope_t, R);
}

}  // namespace amfma
}  // namespace csa
