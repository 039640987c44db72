// Shared-KV MQA with an attention sink, 64 heads per workgroup, on gfx950 matrix cores.
//
// "DeepSeek-V4 混合注意力" §4.2 (one compressed vector is both K and V for every query head),
// §5 (HCA: every visible summary), §6 (SWA rows, sink softmax, partial RoPE / inverse RoPE).
//
// One workgroup = one query x 64 heads (x a range of row slots when split). Per 32-row tile:
//   - the rows (bf16, 1 KiB each) are staged in LDS, rows padded to 1056 bytes so both
//     read patterns below spread over the banks. The next tile's rows load into registers
//     while this one is computed (one 1 KiB row per wavefront instruction, its address
//     resolved in scalar registers) and are stored to the other LDS buffer during the
//     output matrix ops;
//   - S^T = K Q^T (rows x heads, MFMA 16x16x32 bf16): A = 16-byte row fragments from LDS,
//     read a few chunks ahead into a register ring; B = the wavefront's q^T fragments,
//     held in registers for the whole query;
//   - in the C layout of S^T every lane holds 8 rows of one head, which is exactly the
//     A-operand layout of P for O = P V, so P never leaves registers;
//   - V fragments (8 rows of one dim per lane) come from ds_read_b64_tr_b16 transposing
//     reads of the row-major tile; O accumulates in fp32 registers, and one more matrix op
//     per tile against a ones operand accumulates the softmax denominators;
//   - online softmax with a lazy reference maximum: O and the denominators are rescaled
//     only when a head's running maximum grows by more than 2^16 (exponentials stay below
//     2^16), and the rescale itself runs on the matrix cores.
#include "attn_rows.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

constexpr int WD = 512;     // head dim
constexpr int WR = 32;      // rows per tile
constexpr int WH = 64;      // heads per workgroup (16 per wavefront)
constexpr float kLazy = 16.f; // log2 headroom of the reference maximum
#ifndef SD_AHEAD
#define SD_AHEAD 3  // K-fragment chunks read ahead of the score matrix ops
#endif
#ifndef PV_AHEAD
#define PV_AHEAD 4  // V-fragment chunks read ahead of the output matrix ops
#endif
#ifndef SD2_AHEAD
#define SD2_AHEAD 3  // the same two depths for the dim-split layout
#endif
#ifndef PV2_AHEAD
#define PV2_AHEAD 4
#endif
constexpr int kIdxCache = 4096; // top-k indices of one split kept in LDS (k <= 4096)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef unsigned int u32x4w __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4w gu32x4;
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2w __attribute__((ext_vector_type(2)));  // converts with v_cvt_pk_bf16_f32 (RNE)
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

// Layouts (DS = slices of the head dim, HT = 16-head tiles per wavefront):
//   <1,1>: 4 wavefronts, each 16 heads x 512 dims;
//   <2,1>: 8 wavefronts, the pair (w, w ^ 4) owns 16 heads and splits the dims in halves;
//   <2,2>: 4 wavefronts, the pair (w, w ^ 2) owns 32 heads and splits the dims in halves,
//          so every K / V fragment read from LDS feeds two matrix ops.
// With DS == 2 the two partial score tiles of a pair are summed through LDS.
template <int DS, int HT>
__global__ void __launch_bounds__(256 * DS / HT, 1)
attn_wide_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ kv, const float *__restrict__ sink,
                 const int32_t *__restrict__ idx, int k, int ratio, float scale_log2,
                 const bf16_t *__restrict__ swa, const int64_t *__restrict__ swa_pos0, int swa_rows,
                 int window, const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos,
                 const float *__restrict__ rope_cs, int R, int T, int B, int64_t N, int H,
                 bf16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part,
                 int nsplit, int64_t split_slots)
{
    constexpr int NW = 4 * DS / HT;  // wavefronts
    constexpr int NT = 64 * NW;      // threads
    constexpr int HGW = 4 / HT;      // head groups of 16 * HT heads per workgroup
    constexpr int DW = WD / DS;      // dims per wavefront
    constexpr int KKN = DW / 32;     // k-chunks of S^T (q^T fragments)
    constexpr int NDN = DW / 16;     // 16-dim output tiles
    constexpr int RPW = WR / NW;     // tile rows staged per wavefront
    constexpr int SDA0 = HT == 2 ? SD2_AHEAD : SD_AHEAD;
    constexpr int PVA0 = HT == 2 ? PV2_AHEAD : PV_AHEAD;
    constexpr int SDA = SDA0 < KKN ? SDA0 : KKN - 1;
    constexpr int PVA = PVA0 < NDN ? PVA0 : NDN - 1;
    __shared__ __attribute__((aligned(16))) bf16_t KV[2][WR * WP];
    __shared__ int32_t sidx[kIdxCache];
    __shared__ f32x4 SX[DS == 2 ? NW * HT * 2 * 64 : 1];  // partial S^T tiles, one set per wavefront

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int hw = w % HGW, dh = w / HGW;  // head group within the 64, dim slice
    const int dbase = dh * DW;

    // XCD-aware placement: units (query, split, head group) are dealt to the 8 XCDs in
    // contiguous runs, so neighbouring queries (which share SWA rows and summaries) meet
    // in one L2
    const int HGN = H / WH;
    const int64_t U = (int64_t)T * nsplit * HGN;
    const int64_t per_xcd = (U + 7) / 8;
    const int64_t bid = blockIdx.x;
    const int64_t u = (bid & 7) * per_xcd + (bid >> 3);
    if ((bid >> 3) >= per_xcd || u >= U) return;
    const int hg = (int)(u % HGN);
    const int64_t tu = u / HGN;
    const int t = (int)(tu / nsplit), sp = (int)(tu % nsplit);
    const int head0 = hg * WH + 16 * HT * hw;  // head tile ht covers head0 + 16ht .. +15

    const RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    const int64_t j0 = (int64_t)sp * split_slots;
    int64_t j1 = j0 + split_slots;
    if (j1 > c.nslots) j1 = c.nslots;

    // ---- q^T fragments (B operand of S^T): head head0 + 16ht + l16, dims dbase + 32kk + 8g4 ..
    bf16x8 qf[HT][KKN];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const bf16_t *qrow = q + ((int64_t)t * H + head0 + 16 * ht + l16) * WD;
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk) {
            const int d0 = dbase + 32 * kk + 8 * g4;
            uint4 raw = *reinterpret_cast<const uint4 *>(qrow + d0);
            if (rope_cs != nullptr && d0 + 8 > WD - R) {
                const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x0 = lo_bf16(wd[e]), x1 = hi_bf16(wd[e]);
                    const int d = d0 + 2 * e;
                    if (d >= WD - R) {
                        const int p = (d - (WD - R)) >> 1;
                        const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2];
                        const float sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
                        const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
                        x0 = y0;
                        x1 = y1;
                    }
                    o[e] = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
                }
                raw = make_uint4(o[0], o[1], o[2], o[3]);
            }
            qf[ht][kk] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    // softmax state: m_ref[ht] of head head0 + 16ht + l16 (replicated over the 4 lane
    // groups); the denominators live in the output layout (head head0 + 16ht + 4g4 + r in
    // component r of lacc[ht]) and are accumulated by one extra matrix op per tile
    // against a ones operand, so they sum the same bf16 weights that enter O; the sink
    // contributes 2^(m_ref - m_ref) = 1.
    const bool single = (nsplit == 1);
    float m_ref[HT];
    f32x4 lacc[HT];
    f32x4 acc[HT][NDN];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        m_ref[ht] = single ? sink[head0 + 16 * ht + l16] * kLog2e : -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            lacc[ht][r] = (single && sink[head0 + 16 * ht + 4 * g4 + r] != -INFINITY) ? 1.f : 0.f;
#pragma unroll
        for (int nd = 0; nd < NDN; ++nd) acc[ht][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The split's top-k indices are read once into LDS, so a tile's row addresses cost no
    // global round trip (k <= kIdxCache is a precondition of the sparse call).
    const int64_t jm = (j1 < c.nmain) ? j1 : c.nmain;  // main slots of this split: [j0, jm)
    if (ratio <= 0)
        for (int64_t x = threadIdx.x; x < jm - j0; x += NT) sidx[x] = idx[(int64_t)t * k + j0 + x];
    __syncthreads();
    // Rows without data read a valid stand-in address (this wave's own q rows) and are
    // masked out of the softmax, so every load is issued unconditionally and the wait
    // counts stay static.
    const bf16_t *standin = q + ((int64_t)t * H + head0) * WD;
    // Row addresses of the tile at slot jt: lane r < 32 resolves slot jt + r to a byte
    // address (the stand-in when the slot has no row) and the tile's 32-bit validity mask
    // comes from a ballot.
    auto tile_rows = [&](int64_t jt, uint64_t &addr) -> uint32_t {
        const int64_t j = jt + (lane & 31);
        const bf16_t *p = standin;
        if (j < j1) {
            if (j < c.nmain) {
                const int64_t id = (ratio <= 0) ? (int64_t)sidx[j - j0] : j;
                if (id >= 0 && id < N) p = kv + ((int64_t)c.s * N + id) * WD;
            } else {
                const int64_t r = c.lo + (j - c.nmain) - c.swa0;
                if (r >= 0 && r < swa_rows) p = swa + ((int64_t)c.s * swa_rows + r) * WD;
            }
        }
        addr = (uint64_t)(uintptr_t)p;
        return (uint32_t)(__ballot(p != standin) & 0xffffffffull);
    };
    // Wave w stages rows RPW*w .. RPW*w + RPW-1 of a tile, 16 bytes of each per lane, in
    // named registers (macros, so nothing is an array the compiler could keep in memory).
    // A load's row is the same for the whole wave: its address is read out of the
    // resolving lane into scalar registers.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint4 st0, st1, st2, st3, st4, st5, st6, st7;
#define CSA_LD1(I, ADDR)                                                              \
    {                                                                                 \
        const uint32_t lo_ = __builtin_amdgcn_readlane((uint32_t)(ADDR), RPW * wu + (I)); \
        const uint32_t hi_ = __builtin_amdgcn_readlane((uint32_t)((ADDR) >> 32), RPW * wu + (I)); \
        const gu32x4 *rp_ = (const gu32x4 *)(((uint64_t)hi_ << 32) | lo_);           \
        st##I = __builtin_bit_cast(uint4, rp_[lane]);                                 \
    }
#define CSA_TILE_LOAD(A)                                                              \
    CSA_LD1(0, A) CSA_LD1(1, A) CSA_LD1(2, A) CSA_LD1(3, A)                           \
    if constexpr (RPW > 4) { CSA_LD1(4, A) CSA_LD1(5, A) CSA_LD1(6, A) CSA_LD1(7, A) }
    // the next tile's loads are spread over the score matrix ops, one per LDSTEP chunks
    constexpr int LDSTEP = KKN / RPW;
#define CSA_LD_SLOT(KK, A)                                                            \
    if ((KK) == 0 * LDSTEP) CSA_LD1(0, A)                                             \
    if ((KK) == 1 * LDSTEP) CSA_LD1(1, A)                                             \
    if ((KK) == 2 * LDSTEP) CSA_LD1(2, A)                                             \
    if ((KK) == 3 * LDSTEP) CSA_LD1(3, A)                                             \
    if constexpr (RPW > 4) {                                                          \
        if ((KK) == 4 * LDSTEP) CSA_LD1(4, A)                                         \
        if ((KK) == 5 * LDSTEP) CSA_LD1(5, A)                                         \
        if ((KK) == 6 * LDSTEP) CSA_LD1(6, A)                                         \
        if ((KK) == 7 * LDSTEP) CSA_LD1(7, A)                                         \
    }
#define CSA_ST1(I, BUF) *reinterpret_cast<uint4 *>(&KV[(BUF)][(RPW * wu + (I)) * WP + lane * 8]) = st##I;
    // the staged rows go to the other buffer during the output matrix ops, one store per
    // STSTEP output tiles (that buffer was last read before the previous barrier)
    constexpr int STSTEP = NDN / RPW;
#define CSA_ST_SLOT(ND, BUF)                                                          \
    if ((ND) == 0 * STSTEP) CSA_ST1(0, BUF)                                           \
    if ((ND) == 1 * STSTEP) CSA_ST1(1, BUF)                                           \
    if ((ND) == 2 * STSTEP) CSA_ST1(2, BUF)                                           \
    if ((ND) == 3 * STSTEP) CSA_ST1(3, BUF)                                           \
    if constexpr (RPW > 4) {                                                          \
        if ((ND) == 4 * STSTEP) CSA_ST1(4, BUF)                                       \
        if ((ND) == 5 * STSTEP) CSA_ST1(5, BUF)                                       \
        if ((ND) == 6 * STSTEP) CSA_ST1(6, BUF)                                       \
        if ((ND) == 7 * STSTEP) CSA_ST1(7, BUF)                                       \
    }
#define CSA_TILE_STORE(BUF)                                                           \
    CSA_ST1(0, BUF) CSA_ST1(1, BUF) CSA_ST1(2, BUF) CSA_ST1(3, BUF)                   \
    if constexpr (RPW > 4) { CSA_ST1(4, BUF) CSA_ST1(5, BUF) CSA_ST1(6, BUF) CSA_ST1(7, BUF) }

    uint32_t valid = 0u, valid_next = 0u;
    uint64_t ra;  // row addresses of the next tile, resolved one iteration ahead
    if (j0 < j1) {
        valid = tile_rows(j0, ra);
        CSA_TILE_LOAD(ra)
        CSA_TILE_STORE(0)
    }
    valid_next = tile_rows(j0 + WR, ra);
    __syncthreads();
    // Every prologue load (Q fragments, first tile) has landed: without this the
    // loop's wait counters start pessimistic and stall the first matrix ops.
    __builtin_amdgcn_s_waitcnt(0);

    int it = 0;
    for (int64_t jt = j0; jt < j1; jt += WR, ++it) {
        const int buf = it & 1;
        const bf16_t *tile = KV[buf];
        uint64_t ra2;
        uint32_t valid_next2;

        // ---- S^T = K Q^T: a register ring keeps SDA chunks of K fragments in flight; past
        // the last tile every slot of the next tile resolves to the stand-in, so the
        // loads (and the stores below) need no branch
        f32x4 sacc[HT][2];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) sacc[ht][0] = sacc[ht][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            bf16x8 ring[SDA + 1][2];
            const bf16_t *kb = tile + l16 * WP + dbase + g4 * 8;
#pragma unroll
            for (int cc = 0; cc < SDA; ++cc) {
                ring[cc][0] = ld_bf16x8(kb + 32 * cc);
                ring[cc][1] = ld_bf16x8(kb + 16 * WP + 32 * cc);
            }
#pragma unroll
            for (int kk = 0; kk < KKN; ++kk) {
                if (kk + SDA < KKN) {
                    ring[(kk + SDA) % (SDA + 1)][0] = ld_bf16x8(kb + 32 * (kk + SDA));
                    ring[(kk + SDA) % (SDA + 1)][1] = ld_bf16x8(kb + 16 * WP + 32 * (kk + SDA));
                }
                CSA_LD_SLOT(kk, ra)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                    for (int m = 0; m < 2; ++m)
                        sacc[ht][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[kk % (SDA + 1)][m], qf[ht][kk],
                                                                              sacc[ht][m], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // rows of the tile after next: the index read and the address arithmetic overlap
        // the matrix ops still in flight
        valid_next2 = tile_rows(jt + 2 * WR, ra2);
        if constexpr (DS == 2) {
            // full scores = the two dim halves' partial sums, added in the same order by
            // both wavefronts of the pair so their softmax states stay identical
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int m = 0; m < 2; ++m) SX[((w * HT + ht) * 2 + m) * 64 + lane] = sacc[ht][m];
            __syncthreads();
            const int pw = w ^ HGW;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const f32x4 o = SX[((pw * HT + ht) * 2 + m) * 64 + lane];
                    sacc[ht][m] = dh == 0 ? sacc[ht][m] + o : o + sacc[ht][m];
                }
        }

        // ---- online softmax with the lazy reference maximum
        // rows without data (only in a split's last tile or for padded / missing slots) are
        // masked to -inf; full tiles skip the mask
        if (valid != 0xffffffffu) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (!((valid >> (16 * m + 4 * g4 + r)) & 1u)) sacc[ht][m][r] = -INFINITY;
        }
        float tmax[HT];
        bool grow = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            // the scale is positive, so the max of the raw scores gives the max logit
            float smax = fmaxf(fmaxf(fmaxf(sacc[ht][0][0], sacc[ht][0][1]), fmaxf(sacc[ht][0][2], sacc[ht][0][3])),
                               fmaxf(fmaxf(sacc[ht][1][0], sacc[ht][1][1]), fmaxf(sacc[ht][1][2], sacc[ht][1][3])));
            const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
            smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
            const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
            smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
            tmax[ht] = smax * scale_log2;
            grow = grow || (tmax[ht] > m_ref[ht] + kLazy);
        }
        if (__ballot(grow) != 0ull) {
            // rare: the accumulators are rescaled on the matrix cores, so they are only ever
            // touched by matrix ops (and stay in accumulation registers); before the first
            // P V product O is still zero
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const float mn = fmaxf(m_ref[ht], tmax[ht]);
                const float alpha = (m_ref[ht] == -INFINITY || mn == -INFINITY)
                                        ? (mn == -INFINITY ? 1.f : 0.f)
                                        : exp2f(m_ref[ht] - mn);
                m_ref[ht] = mn;
                float ar[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) ar[r] = (l16 == 4 * g4 + r) ? alpha : 0.f;
                lacc[ht] = scale_rows(lacc[ht], ar);
                if (it != 0) {
#pragma unroll
                    for (int nd = 0; nd < NDN; ++nd) acc[ht][nd] = scale_rows(acc[ht][nd], ar);
                }
            }
        }
        // p = 2^(s * scale - m_ref) <= 2^kLazy, packed to bf16: the C layout of S^T gives
        // every lane 8 rows of one head, the A-operand layout of P for O = P V.
        // v_exp_f32 flushes results below 2^-126 to zero, which only drops weights that
        // no bf16 sum could hold.
        bf16x8 pf[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const float nmu = (m_ref[ht] == -INFINITY) ? 0.f : -m_ref[ht];
            uint32_t pk[4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[ht][m][r], scale_log2, nmu));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[ht][m][r + 1], scale_log2, nmu));
                    pk[2 * m + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{p0, p1}, bf16x2w));
                }
            pf[ht] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            lacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ht], ones_bf16x8(), lacc[ht], 0, 0, 0);
        }

        // ---- O += P V: V fragments (8 rows of one dim per lane, in the row order of the
        // C layout above) from transposing LDS reads, riding a register ring PVA ops ahead
        {
            const int s4 = l16 >> 2, sc = l16 & 3;
            const bf16_t *v0 = tile + (4 * g4 + s4) * WP + dbase + 4 * sc;
            const bf16_t *v1 = v0 + 16 * WP;
            bf16x4v vr[PVA + 1][2];
#pragma unroll
            for (int cc = 0; cc < PVA; ++cc) {
                vr[cc][0] = __builtin_bit_cast(bf16x4v, ld_tr(v0 + 16 * cc));
                vr[cc][1] = __builtin_bit_cast(bf16x4v, ld_tr(v1 + 16 * cc));
            }
#pragma unroll
            for (int nd = 0; nd < NDN; ++nd) {
                if (nd + PVA < NDN) {
                    vr[(nd + PVA) % (PVA + 1)][0] = __builtin_bit_cast(bf16x4v, ld_tr(v0 + 16 * (nd + PVA)));
                    vr[(nd + PVA) % (PVA + 1)][1] = __builtin_bit_cast(bf16x4v, ld_tr(v1 + 16 * (nd + PVA)));
                }
                CSA_ST_SLOT(nd, buf ^ 1)
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 vf = __builtin_shufflevector(vr[nd % (PVA + 1)][0], vr[nd % (PVA + 1)][1], 0, 1, 2, 3,
                                                          4, 5, 6, 7);
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    acc[ht][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[ht], vf, acc[ht][nd], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        valid = valid_next;
        valid_next = valid_next2;
        ra = ra2;
        __syncthreads();
    }
#undef CSA_TILE_STORE
#undef CSA_ST_SLOT
#undef CSA_ST1
#undef CSA_LD_SLOT
#undef CSA_TILE_LOAD
#undef CSA_LD1

    // ---- epilogue: O rows are heads head0 + 16ht + 4g4 + r, columns dim dbase + 16nd + l16
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        if (single) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = head0 + 16 * ht + 4 * g4 + r;
                const float lv = lacc[ht][r];
                const float mr = __shfl(m_ref[ht], 4 * g4 + r);
                if (lse != nullptr && l16 == 0 && dh == 0) {
                    const float mu = (mr == -INFINITY) ? 0.f : mr;
                    lse[(int64_t)t * H + h] = (lv > 0.f) ? (mu + log2f(lv)) * kLn2 : -INFINITY;
                }
                const float inv = lv > 0.f ? 1.f / lv : 0.f;
                bf16_t *orow = out + ((int64_t)t * H + h) * WD;
#pragma unroll
                for (int nd = 0; nd < NDN; ++nd) {
                    const int d = dbase + 16 * nd + l16;
                    float x = acc[ht][nd][r] * inv;
                    const float y = __shfl_xor(x, 1);
                    if (rope_cs != nullptr && d >= WD - R) {
                        const int p = (d - (WD - R)) >> 1;
                        const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2];
                        const float sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
                        x = (d & 1) ? (x * cs - y * sn) : (x * cs + y * sn);
                    }
                    orow[d] = f32_to_bf16(x);
                }
            }
        } else {
            const int64_t pu = ((int64_t)t * nsplit + sp) * H + head0 + 16 * ht;
            float *pml = part;                                  // [T][nsplit][H][2]
            float *pacc = part + (int64_t)T * nsplit * H * 2;   // [T][nsplit][H][D]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mr = __shfl(m_ref[ht], 4 * g4 + r);
                if (l16 == 0 && dh == 0) {
                    pml[(pu + 4 * g4 + r) * 2] = mr;
                    pml[(pu + 4 * g4 + r) * 2 + 1] = lacc[ht][r];
                }
                float *prow = pacc + (pu + 4 * g4 + r) * WD;
#pragma unroll
                for (int nd = 0; nd < NDN; ++nd) prow[dbase + 16 * nd + l16] = acc[ht][nd][r];
            }
        }
    }
}

}  // namespace

bool wide_attn_ok(csa_dtype dt, int H, int D) { return dt == CSA_BF16 && D == WD && H % WH == 0; }

int launch_attn_wide(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st) {
    const int64_t U = (int64_t)a.T * nsplit * (a.H / WH);
    const int64_t blocks = ((U + 7) / 8) * 8;
#define CSA_WIDE_LAUNCH(DS_, HT_)                                                                              \
    hipLaunchKernelGGL((attn_wide_kernel<DS_, HT_>), dim3((unsigned)blocks), dim3(256 * DS_ / HT_), 0, st,     \
                       (const bf16_t *)a.q, (const bf16_t *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2,            \
                       (const bf16_t *)a.swa, a.swa_pos0, a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs,   \
                       a.rope_dim, a.T, a.B, a.N, a.H, (bf16_t *)a.out, a.lse, (float *)a.ws, nsplit, split_slots);
    // measured: the gathered (sparse) rows run best with two wavefronts per SIMD, whose
    // extra memory-level parallelism hides the gather latency; the dense summaries, read
    // from L2, with one wavefront of 16 heads x 512 dims
    if (a.ratio <= 0) {
        CSA_WIDE_LAUNCH(2, 1)
    } else {
        CSA_WIDE_LAUNCH(1, 1)
    }
#undef CSA_WIDE_LAUNCH
    return check_launch("attn_wide_kernel");
}

}  // namespace csa
