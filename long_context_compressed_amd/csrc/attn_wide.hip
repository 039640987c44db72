// Shared-KV MQA with an attention sink, 64 heads per workgroup, on gfx950 matrix cores.
//
// "DeepSeek-V4 混合注意力" §4.2 (one compressed vector is both K and V for every query head),
// §5 (HCA: every visible summary), §6 (SWA rows, sink softmax, partial RoPE / inverse RoPE).
//
// One workgroup = one query x 64 heads (x a range of row slots when split); wavefront w
// owns heads 16w..16w+15 over the full head dim D = 512, so softmax needs no cross-wave
// exchange. Per 32-row tile:
//   - the rows (bf16, 1 KiB each) are staged in LDS (rows padded to 1056 bytes so both
//     read patterns below spread over the banks); two tiles are in flight in registers
//     while one is computed;
//   - S^T = K Q^T (rows x heads, 32 MFMA 16x16x32): A = 16-byte row fragments from LDS,
//     B = the wave's q^T fragments, held in VGPRs for the whole query;
//   - in the C layout of S^T every lane holds 8 rows of one head, which is exactly the
//     A-operand layout of P for O = P V, so P never leaves registers;
//   - V fragments (8 rows of one dim per lane) come from ds_read_b64_tr_b16 transposing
//     reads of the row-major tile; O (16 heads x 512 dims fp32) accumulates in registers;
//   - online softmax with a lazy reference maximum: O and the denominator are rescaled
//     only when a head's running maximum grows by more than 2^8, so the exponentials
//     stay below 256 and the 128 accumulator registers are rarely touched.
#include "attn_rows.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

constexpr int WD = 512;     // head dim
constexpr int WR = 32;      // rows per tile
constexpr int WH = 64;      // heads per workgroup (16 per wavefront)
constexpr float kLazy = 8.f; // log2 headroom of the reference maximum
#ifndef SD_AHEAD
#define SD_AHEAD 3  // K-fragment chunks read ahead of the score matrix ops
#endif
#ifndef PV_AHEAD
#define PV_AHEAD 4  // V-fragment chunks read ahead of the output matrix ops
#endif
constexpr int kIdxCache = 4096; // top-k indices of one split kept in LDS (k <= 4096)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef unsigned int u32x4w __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4w gu32x4;
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2w __attribute__((ext_vector_type(2)));  // converts with v_cvt_pk_bf16_f32 (RNE)

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

__global__ void __launch_bounds__(256, 1)
attn_wide_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ kv, const float *__restrict__ sink,
                 const int32_t *__restrict__ idx, int k, int ratio, float scale_log2,
                 const bf16_t *__restrict__ swa, const int64_t *__restrict__ swa_pos0, int swa_rows,
                 int window, const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos,
                 const float *__restrict__ rope_cs, int R, int T, int B, int64_t N, int H,
                 bf16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part,
                 int nsplit, int64_t split_slots)
{
    __shared__ __attribute__((aligned(16))) bf16_t KV[2][WR * WP];
    __shared__ int32_t sidx[kIdxCache];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

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
    const int head0 = hg * WH + 16 * w;  // first head of this wave

    const RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    const int64_t j0 = (int64_t)sp * split_slots;
    int64_t j1 = j0 + split_slots;
    if (j1 > c.nslots) j1 = c.nslots;

    // ---- q^T fragments (B operand of S^T): head head0 + l16, dims 32kk + 8g4 .. +7 ---------
    bf16x8 qf[16];
    {
        const bf16_t *qrow = q + ((int64_t)t * H + head0 + l16) * WD;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int d0 = 32 * kk + 8 * g4;
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
            qf[kk] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    // softmax state of head head0 + l16 (replicated over the 4 lane groups)
    const bool single = (nsplit == 1);
    float m_ref = single ? sink[head0 + l16] * kLog2e : -INFINITY;
    float l_sum = (single && m_ref != -INFINITY) ? 1.f : 0.f;
    f32x4 acc[32];
#pragma unroll
    for (int nd = 0; nd < 32; ++nd) acc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The split's top-k indices are read once into LDS, so a tile's row addresses cost no
    // global round trip.
    // (k <= kIdxCache is a precondition of the sparse call)
    const int64_t jm = (j1 < c.nmain) ? j1 : c.nmain;  // main slots of this split: [j0, jm)
    if (ratio <= 0)
        for (int64_t x = threadIdx.x; x < jm - j0; x += 256) sidx[x] = idx[(int64_t)t * k + j0 + x];
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
    // Wave w stages rows 8w..8w+7 of a tile, 16 bytes of each per lane, in eight named
    // registers (macros, so nothing is an array the compiler could keep in memory). A
    // load's row is the same for the whole wave: its address is read out of the
    // resolving lane into scalar registers.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint4 st0, st1, st2, st3, st4, st5, st6, st7;
#define CSA_LD1(I, ADDR)                                                              \
    {                                                                                 \
        const uint32_t lo_ = __builtin_amdgcn_readlane((uint32_t)(ADDR), 8 * wu + (I)); \
        const uint32_t hi_ = __builtin_amdgcn_readlane((uint32_t)((ADDR) >> 32), 8 * wu + (I)); \
        const gu32x4 *rp_ = (const gu32x4 *)(((uint64_t)hi_ << 32) | lo_);           \
        st##I = __builtin_bit_cast(uint4, rp_[lane]);                                 \
    }
#define CSA_TILE_LOAD(A)                                                              \
    CSA_LD1(0, A) CSA_LD1(1, A) CSA_LD1(2, A) CSA_LD1(3, A)                           \
    CSA_LD1(4, A) CSA_LD1(5, A) CSA_LD1(6, A) CSA_LD1(7, A)
#define CSA_ST1(I, BUF) *reinterpret_cast<uint4 *>(&KV[(BUF)][(8 * wu + (I)) * WP + lane * 8]) = st##I;
#define CSA_TILE_STORE(BUF)                                                           \
    CSA_ST1(0, BUF) CSA_ST1(1, BUF) CSA_ST1(2, BUF) CSA_ST1(3, BUF)                   \
    CSA_ST1(4, BUF) CSA_ST1(5, BUF) CSA_ST1(6, BUF) CSA_ST1(7, BUF)

    uint32_t valid = 0u, valid_next = 0u;
    if (j0 < j1) {
        uint64_t ra;
        valid = tile_rows(j0, ra);
        CSA_TILE_LOAD(ra)
        CSA_TILE_STORE(0)
    }
    __syncthreads();
    // Every prologue load (Q fragments, first tile) has landed: without this the
    // loop's wait counters start pessimistic and stall the first matrix ops.
    __builtin_amdgcn_s_waitcnt(0);

    int it = 0;
    for (int64_t jt = j0; jt < j1; jt += WR, ++it) {
        const int buf = it & 1;
        const bool has_next = jt + WR < j1;
        if (has_next) {  // the next tile's rows load while this one is computed
            uint64_t ra;
            valid_next = tile_rows(jt + WR, ra);
            CSA_TILE_LOAD(ra)
        }
        const bf16_t *tile = KV[buf];
    {
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        {
            // Register ring of K fragments: chunk kk (rows of both 16-row halves) is
            // read SD_AHEAD chunks before its two matrix ops issue.
            bf16x8 ring[SD_AHEAD + 1][2];
            const bf16_t *kb = tile + l16 * WP + g4 * 8;
#pragma unroll
            for (int c = 0; c < SD_AHEAD; ++c) {
                ring[c][0] = ld_bf16x8(kb + 32 * c);
                ring[c][1] = ld_bf16x8(kb + 16 * WP + 32 * c);
            }
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                if (kk + SD_AHEAD < 16) {
                    ring[(kk + SD_AHEAD) % (SD_AHEAD + 1)][0] = ld_bf16x8(kb + 32 * (kk + SD_AHEAD));
                    ring[(kk + SD_AHEAD) % (SD_AHEAD + 1)][1] = ld_bf16x8(kb + 16 * WP + 32 * (kk + SD_AHEAD));
                }
                __builtin_amdgcn_sched_barrier(0);
                sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[kk % (SD_AHEAD + 1)][0], qf[kk], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[kk % (SD_AHEAD + 1)][1], qf[kk], sacc[1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        float z[2][4], tmax = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * m + 4 * g4 + r;
                z[m][r] = ((valid >> row) & 1u) ? sacc[m][r] * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, z[m][r]);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (__ballot(tmax > m_ref + kLazy) != 0ull) {
            const float mn = fmaxf(m_ref, tmax);
            const float alpha = (m_ref == -INFINITY || mn == -INFINITY) ? (mn == -INFINITY ? 1.f : 0.f)
                                                                        : exp2f(m_ref - mn);
            l_sum *= alpha;
            m_ref = mn;
            f32x4 ao;
#pragma unroll
            for (int r = 0; r < 4; ++r) ao[r] = __shfl(alpha, 4 * g4 + r);
#pragma unroll
            for (int nd = 0; nd < 32; ++nd) acc[nd] *= ao;
        }
        bf16x8 pf;
        {
            const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
            float rs = 0.f;
            uint32_t pk[4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float p0 = exp2f(z[m][r] - mu), p1 = exp2f(z[m][r + 1] - mu);
                    rs += p0 + p1;
                    pk[2 * m + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{p0, p1}, bf16x2w));
                }
            rs += __shfl_xor(rs, 16);
            rs += __shfl_xor(rs, 32);
            l_sum += rs;
            pf = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }

        {
            const int s4 = l16 >> 2, sc = l16 & 3;
        const bf16_t *v0 = tile + (4 * g4 + s4) * WP + 4 * sc;
        const bf16_t *v1 = v0 + 16 * WP;
        // V fragments ride a register ring PV_AHEAD matrix ops ahead.
        bf16x4v vr[PV_AHEAD + 1][2];
#pragma unroll
        for (int c = 0; c < PV_AHEAD; ++c) {
            vr[c][0] = __builtin_bit_cast(bf16x4v, ld_tr(v0 + 16 * c));
            vr[c][1] = __builtin_bit_cast(bf16x4v, ld_tr(v1 + 16 * c));
        }
#pragma unroll
        for (int nd = 0; nd < 32; ++nd) {
            if (nd + PV_AHEAD < 32) {
                vr[(nd + PV_AHEAD) % (PV_AHEAD + 1)][0] = __builtin_bit_cast(bf16x4v, ld_tr(v0 + 16 * (nd + PV_AHEAD)));
                vr[(nd + PV_AHEAD) % (PV_AHEAD + 1)][1] = __builtin_bit_cast(bf16x4v, ld_tr(v1 + 16 * (nd + PV_AHEAD)));
            }
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8 vf = __builtin_shufflevector(vr[nd % (PV_AHEAD + 1)][0], vr[nd % (PV_AHEAD + 1)][1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf, acc[nd], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        }
    }

        if (has_next) {
            CSA_TILE_STORE(buf ^ 1)
            valid = valid_next;
        }
        __syncthreads();
    }
#undef CSA_TILE_STORE
#undef CSA_TILE_LOAD
#undef CSA_ST1
#undef CSA_LD1

    // ---- epilogue: O rows are heads head0 + 4g4 + r, columns dim 16nd + l16 ----------------
    if (single) {
        if (lse != nullptr && g4 == 0) {
            const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
            lse[(int64_t)t * H + head0 + l16] = (l_sum > 0.f) ? (mu + log2f(l_sum)) * kLn2 : -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float lv = __shfl(l_sum, 4 * g4 + r);
            const float inv = lv > 0.f ? 1.f / lv : 0.f;
            bf16_t *orow = out + ((int64_t)t * H + head0 + 4 * g4 + r) * WD;
#pragma unroll
            for (int nd = 0; nd < 32; ++nd) {
                const int d = 16 * nd + l16;
                float x = acc[nd][r] * inv;
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
        const int64_t pu = ((int64_t)t * nsplit + sp) * H + head0;
        float *pml = part;                                  // [T][nsplit][H][2]
        float *pacc = part + (int64_t)T * nsplit * H * 2;   // [T][nsplit][H][D]
        if (g4 == 0) {
            pml[(pu + l16) * 2] = m_ref;
            pml[(pu + l16) * 2 + 1] = l_sum;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *prow = pacc + (pu + 4 * g4 + r) * WD;
#pragma unroll
            for (int nd = 0; nd < 32; ++nd) prow[16 * nd + l16] = acc[nd][r];
        }
    }
}

}  // namespace

bool wide_attn_ok(csa_dtype dt, int H, int D) { return dt == CSA_BF16 && D == WD && H % WH == 0; }

int launch_attn_wide(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st) {
    const int64_t U = (int64_t)a.T * nsplit * (a.H / WH);
    const int64_t blocks = ((U + 7) / 8) * 8;
    hipLaunchKernelGGL(attn_wide_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16_t *)a.q,
                       (const bf16_t *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2, (const bf16_t *)a.swa, a.swa_pos0,
                       a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs, a.rope_dim, a.T, a.B, a.N, a.H,
                       (bf16_t *)a.out, a.lse, (float *)a.ws, nsplit, split_slots);
    return check_launch("attn_wide_kernel");
}

}  // namespace csa
