// Shared-KV MQA with an attention sink, 128 heads per workgroup, 32 heads per wavefront,
// on gfx950 matrix cores.
//
// "DeepSeek-V4 混合注意力" §4.2 (one compressed vector is both K and V for every query head),
// §5 (HCA: every visible summary), §6 (SWA rows, sink softmax, partial RoPE / inverse RoPE).
//
// The tile loop of shared-KV attention streams every row of a tile out of LDS twice per
// wavefront (as K fragments for S^T and as transposed V fragments for P V), 1 KiB of LDS
// per 16x16x32 matrix op. With 16 heads per wavefront that is twice what LDS delivers
// while the matrix cores run. Here a wavefront owns 32 heads, so every fragment read feeds
// two matrix ops: one workgroup of 4 wavefronts (one per SIMD) covers 128 heads of one
// query, and each wavefront holds its 32 x 512 fp32 output in the 256 accumulation
// registers (AGPRs) while q^T (32 heads x 512 dims, bf16) and the tile work sit in the
// 256 ordinary ones. Per 32-row tile:
//   - the rows go from memory straight into LDS by buffer loads with the LDS destination,
//     into the other of two tile buffers while this tile is computed (8 rows per wave);
//   - S^T = K Q^T (rows x heads, MFMA 16x16x32 bf16) for the two 16-head blocks;
//   - the C layout of S^T is the A-operand layout of P, so P never leaves registers;
//   - V fragments from ds_read_b64_tr_b16 transposing reads, each used for both head
//     blocks; the softmax denominators ride one more matrix op per head block against a
//     ones operand;
//   - online softmax against a reference maximum fixed by the first tile; O is never
//     rescaled. If a later tile's maximum exceeds it by more than 2^24 (rare), the pass is
//     abandoned, a pass of S^T alone finds every head's exact maximum, and O is
//     accumulated once more against that.
#include <type_traits>

#include "attn_mfma.hpp"
#include "internal.hpp"

namespace csa {

namespace {

using namespace amfma;

constexpr int NWV = 4;            // wavefronts per workgroup
constexpr int HB = 2;             // 16-head blocks per wavefront
constexpr int WH = 16 * HB * NWV; // heads per workgroup
constexpr int RPW = WR / NWV;     // tile rows loaded per wavefront
static_assert(kIdxCache % (64 * NWV) == 0, "the index cache splits evenly over the threads");
constexpr int SDA = 1;            // K fragment chunks read ahead
constexpr int PVA = 2;            // V fragment chunks read ahead
constexpr float kHeadroom = 24.f; // log2 growth of a head's maximum the tile loop absorbs

// The output accumulators and denominators live in AGPRs: the matrix ops that update them
// are written out with an "a" constraint (the compiler's own MFMA selection would keep
// every result in one register class and shuffle the 256 accumulators between the two).
// The compiler does not see these as matrix ops, so the hazards it would otherwise cover
// are covered here: a VALU result read by a matrix op gets >= 5 wait states (the s_nop at
// the head of the first product that reads it), and the results are read back only after
// two s_nop 15 (pv_fence).
__device__ __forceinline__ void pv_mfma(f32x4 &acc, const bf16x8 a, const bf16x8 b) {
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// the first products of a tile, both head blocks in one statement behind the wait states
// for P's VALU writes
__device__ __forceinline__ void pv_mfma2_after_valu(f32x4 &acc0, f32x4 &acc1, const bf16x8 a, const bf16x8 b0,
                                                    const bf16x8 b1) {
    asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\tv_mfma_f32_16x16x32_bf16 %1, %2, %4, %1"
                 : "+a"(acc0), "+a"(acc1)
                 : "v"(a), "v"(b0), "v"(b1));
}
// one accumulator read out of its AGPR where it is used (left to itself the compiler copies
// every accumulator to VGPRs at the loop exit, more than there are)
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
__device__ __forceinline__ void pv_fence() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }


// The 32 heads of one wavefront for one query (or one split of its rows), computed from
// scratch with plain VALU arithmetic and two passes over the rows (exact maximum, then the
// weighted sums in fp32). It backs the tile loop when a head's maximum grows past the
// loop's headroom; lane l holds dims 8l .. 8l+7.
__device__ __forceinline__ void unit_fallback(
    const bf16_t *q, const float *sink, const RowCtx c, int64_t j0, int64_t j1, int ratio, const int32_t *sidx,
    const int32_t *idx_t, int64_t N, const bf16_t *kv, const bf16_t *swa, int swa_rows, const float *rope_t, int R,
    float scale_log2, int t, int T, int H, int head0, int nsplit, int sp, bf16_t *out, float *lse, float *part)
{
    const int lane = threadIdx.x & 63;
    const int d0 = 8 * lane;
    const bool single = (nsplit == 1);
    for (int hh = 0; hh < 16 * HB; ++hh) {
        const int h = head0 + hh;
        // q with the rotation of the last R dims, rounded once to bf16 (as the tile loop)
        float qv[8];
        {
            const uint4 raw = *reinterpret_cast<const uint4 *>(q + ((int64_t)t * H + h) * WD + d0);
            const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0 = lo_bf16(wd[e]), x1 = hi_bf16(wd[e]);
                const int d = d0 + 2 * e;
                if (rope_t != nullptr && d >= WD - R) {
                    const int p = (d - (WD - R)) >> 1;
                    const float cs = rope_t[2 * p], sn = rope_t[2 * p + 1];
                    const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
                    x0 = y0;
                    x1 = y1;
                }
                qv[2 * e] = bf16_to_f32(f32_to_bf16(x0));
                qv[2 * e + 1] = bf16_to_f32(f32_to_bf16(x1));
            }
        }
        auto score = [&](const bf16_t *row, float rv[8]) -> float {
            const uint4 raw = *reinterpret_cast<const uint4 *>(row + d0);
            const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
            float sdot = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rv[2 * e] = lo_bf16(wd[e]);
                rv[2 * e + 1] = hi_bf16(wd[e]);
                sdot = fmaf(qv[2 * e], rv[2 * e], sdot);
                sdot = fmaf(qv[2 * e + 1], rv[2 * e + 1], sdot);
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) sdot += __shfl_xor(sdot, m);
            return sdot * scale_log2;
        };
        float mx = -INFINITY;
        for (int64_t j = j0; j < j1; ++j) {
            const bf16_t *row = slot_row(c, j, j0, j1, ratio, sidx, idx_t, N, kv, swa, swa_rows, nullptr);
            if (row == nullptr) continue;
            float rv[8];
            mx = fmaxf(mx, score(row, rv));
        }
        const float sk = single ? sink[h] * kLog2e : -INFINITY;
        const float m = fmaxf(mx, sk);
        float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (mx != -INFINITY) {
            for (int64_t j = j0; j < j1; ++j) {
                const bf16_t *row = slot_row(c, j, j0, j1, ratio, sidx, idx_t, N, kv, swa, swa_rows, nullptr);
                if (row == nullptr) continue;
                float rv[8];
                const float p = exp2f(score(row, rv) - m);
                l += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(p, rv[e], o[e]);
            }
        }
        if (single) {
            const float lv = l + ((sk == -INFINITY) ? 0.f : exp2f(sk - m));
            if (lse != nullptr && lane == 0)
                lse[(int64_t)t * H + h] = (lv > 0.f) ? (((m == -INFINITY) ? 0.f : m) + log2f(lv)) * kLn2 : -INFINITY;
            const float inv = lv > 0.f ? 1.f / lv : 0.f;
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0 = o[2 * e] * inv, x1 = o[2 * e + 1] * inv;
                const int d = d0 + 2 * e;
                if (rope_t != nullptr && d >= WD - R) {
                    const int p = (d - (WD - R)) >> 1;
                    const float cs = rope_t[2 * p], sn = rope_t[2 * p + 1];
                    const float y0 = x0 * cs + x1 * sn, y1 = x1 * cs - x0 * sn;
                    x0 = y0;
                    x1 = y1;
                }
                pk[e] = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
            }
            *reinterpret_cast<uint4 *>(out + ((int64_t)t * H + h) * WD + d0) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        } else {
            const int64_t pu = ((int64_t)t * nsplit + sp) * H + h;
            if (lane == 0) {
                part[pu * 2] = mx;
                part[pu * 2 + 1] = l;
            }
            bf16_t *prow = reinterpret_cast<bf16_t *>(part + (int64_t)T * nsplit * H * 2) + pu * WD + d0;
            *reinterpret_cast<uint4 *>(prow) = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                          pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
        }
    }
}

__global__ void __launch_bounds__(64 * NWV, 1)
attn_w32_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ kv, const float *__restrict__ sink,
                const int32_t *__restrict__ idx, int k, int ratio, float scale_log2,
                const bf16_t *__restrict__ swa, const int64_t *__restrict__ swa_pos0, int swa_rows, int window,
                const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos,
                const float *__restrict__ rope_cs, int R, int T, int B, int64_t N, int H,
                bf16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part, int nsplit,
                int64_t split_slots)
{
    __shared__ __attribute__((aligned(16))) bf16_t KV0[WR * WP];  // tile buffers (separate arrays,
    __shared__ __attribute__((aligned(16))) bf16_t KV1[WR * WP];  // see the row loads below)
    __shared__ int32_t sidx[kIdxCache];
    __shared__ int redo;

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
    const int head0 = hg * WH + 16 * HB * w;  // first head of this wave; block b = head0 + 16b ..

    // The loads that depend only on the unit (q, its RoPE pairs, the sinks, the split's
    // top-k indices) are all issued before anything waits on the row context.
    const int64_t j0 = (int64_t)sp * split_slots;
    constexpr int IPT = kIdxCache / (64 * NWV);  // top-k indices per thread
    int32_t ir[IPT];
    {
        const int64_t nc0 = (ratio <= 0) ? (k - j0 < kIdxCache ? k - j0 : kIdxCache) : 0;
#pragma unroll
        for (int m = 0; m < IPT; ++m) {
            const int x = threadIdx.x + 64 * NWV * m;
            ir[m] = (x < nc0) ? idx[(int64_t)t * k + j0 + x] : 0;
        }
    }
    float sk[HB];
#pragma unroll
    for (int b = 0; b < HB; ++b) sk[b] = sink[head0 + 16 * b + l16];

    // q^T fragments of both head blocks, for the whole query. Every load is issued first
    // (they overlap; the (cos, sin) pairs of the last 64 dims included), then the fragments
    // that hold rotated dims are rotated.
    const float *rope_t = rope_cs ? rope_cs + (int64_t)t * R : nullptr;
    bf16x8 qf[HB][KKN];
    {
        float2 qr[2][4];
        if (rope_t != nullptr) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) qr[j][e] = rope_pair(rope_t, 32 * (KKN - 2 + j) + 8 * g4 + 2 * e, R);
        }
#pragma unroll
        for (int b = 0; b < HB; ++b) {
            const bf16_t *qrow = q + ((int64_t)t * H + head0 + 16 * b + l16) * WD;
#pragma unroll
            for (int kk = 0; kk < KKN; ++kk) qf[b][kk] = ld_bf16x8(qrow + 32 * kk + 8 * g4);
        }
        if (rope_t != nullptr) {
#pragma unroll
            for (int b = 0; b < HB; ++b) {
#pragma unroll
                for (int kk = 0; kk < KKN - 2; ++kk) qf[b][kk] = rope_fragment(qf[b][kk], kk, g4, rope_t, R);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float cs[4] = {qr[j][0].x, qr[j][1].x, qr[j][2].x, qr[j][3].x};
                    const float sn[4] = {qr[j][0].y, qr[j][1].y, qr[j][2].y, qr[j][3].y};
                    qf[b][KKN - 2 + j] = rope_fragment_cs(qf[b][KKN - 2 + j], KKN - 2 + j, g4, cs, sn, R);
                }
            }
        }
    }

    const RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    int64_t j1 = j0 + split_slots;
    if (j1 > c.nslots) j1 = c.nslots;

    // softmax state per head block: m_ref of head 16b + l16 (replicated over the 4 lane
    // groups); the denominators live in the output layout (head 16b + 4g4 + r in component
    // r of lacc[b]) and are accumulated by a matrix op against a ones operand, so they sum
    // the same bf16 weights that enter O. The sink's 2^(sink - m_ref) is added at the end.
    const bool single = (nsplit == 1);
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4w{0u, 0u, 0u, 0u});
    float m_ref[HB];
    f32x4 lacc[HB];
    f32x4 acc[HB][NDN];
    auto reset_sums = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < HB; ++b) {
            lacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            // zeroed by a matrix op into AGPRs, so the accumulators never pass through VGPRs
#pragma unroll
            for (int nd = 0; nd < NDN; ++nd)
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(acc[b][nd]) : "v"(zero8));
        }
    };
#pragma unroll
    for (int b = 0; b < HB; ++b) {
        m_ref[b] = single ? sk[b] * kLog2e : -INFINITY;
    }
    reset_sums();

    // The split's top-k indices (up to kIdxCache of them) are read once into LDS.
    const int64_t jm = (j1 < c.nmain) ? j1 : c.nmain;  // main slots of this split: [j0, jm)
    const int64_t ncache = (jm - j0 < kIdxCache) ? jm - j0 : kIdxCache;
    if (ratio <= 0) {
#pragma unroll
        for (int m = 0; m < IPT; ++m) {
            const int x = threadIdx.x + 64 * NWV * m;
            if (x < ncache) sidx[x] = ir[m];
        }
    }
    if (threadIdx.x == 0) redo = 0;
    __syncthreads();
    // Every row of the query lives in one of two regions: its sequence's compressed rows
    // (kv) or its SWA rows. Each gets one buffer resource for the whole unit, and a row is
    // named by a 32-bit code (region bit | row), so a row load only needs that code in a
    // scalar register (the row's byte offset goes in the load's scalar offset). Rows
    // without data are masked out of the softmax and load row 0 (a buffer load past the
    // region's end returns zeros, so nothing outside it is ever touched).
    const int32_t *idx_t = (ratio > 0) ? nullptr : idx + (int64_t)t * k;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int s_u = __builtin_amdgcn_readfirstlane(c.s);
    const __amdgpu_buffer_rsrc_t kv_rs = uniform_rsrc(kv + (int64_t)s_u * N * WD, (uint32_t)(N * WD * 2));
    const __amdgpu_buffer_rsrc_t swa_rs =
        uniform_rsrc(swa != nullptr ? swa + (int64_t)s_u * swa_rows * WD : kv, swa != nullptr ? (uint32_t)swa_rows * WD * 2 : 0u);
    constexpr int32_t kSwaBit = 0x40000000;
    // Row codes of the tile at slot jt: lane r < 32 codes slot jt + r (-1: no row); the
    // tile's 32-bit validity mask comes from a ballot.
    auto tile_rows = [&](int64_t jt, int32_t &code) __attribute__((always_inline)) -> uint32_t {
        const int64_t j = jt + (lane & 31);
        int32_t cd = -1;
        if (j < j1) {
            if (j < c.nmain) {
                const int64_t id = (ratio > 0) ? j : (j - j0 < kIdxCache ? (int64_t)sidx[j - j0] : (int64_t)idx_t[j]);
                if (id >= 0 && id < N) cd = (int32_t)id;
            } else {
                const int64_t r = c.lo + (j - c.nmain) - c.swa0;
                if (r >= 0 && r < swa_rows) cd = kSwaBit | (int32_t)r;
            }
        }
        code = cd;
        return (uint32_t)(__ballot(cd >= 0) & 0xffffffffull);
    };
    // Wavefront w loads rows RPW*w .. RPW*w + RPW-1 of a tile, one 1 KiB row per
    // buffer-load instruction (16 bytes per lane, LDS destination).
    auto dma_row = [&](bf16_t *buf, int i, int32_t cd) __attribute__((always_inline)) {
        const int row = RPW * wu + i;
        const uint32_t off = cd < 0 ? 0u : (uint32_t)(cd & (kSwaBit - 1)) * (WD * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds((cd >= 0 && (cd & kSwaBit)) ? swa_rs : kv_rs,
                                                 (__attribute__((address_space(3))) void *)(buf + row * WP), 16,
                                                 lane * 16, off, 0, 0);
    };
    // Dense attention walks the summaries in order, so a tile whose 32 slots are all
    // summaries is 32 consecutive rows: one buffer resource covers it and no address leaves
    // a lane (the per-row read-out above costs the wave more than the load itself).
    const int64_t jc = (j1 < c.nmain) ? j1 : c.nmain;  // slots before jc are summaries
    auto contig = [&](int64_t jn) __attribute__((always_inline)) { return ratio > 0 && jn + WR <= jc; };
    // buffer resource over the 32 rows from slot jn (the address is read out of lane 0 so
    // the compiler knows it is uniform)
    auto contig_rsrc = [&](int64_t jn) __attribute__((always_inline)) {
        const uint64_t a = (uint64_t)(uintptr_t)(kv + ((int64_t)c.s * N + jn) * WD);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
        return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, WR * WD * 2, kBufDword3);
    };
    auto dma_row_contig = [&](bf16_t *buf, int i, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
        const int row = RPW * wu + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(buf + row * WP), 16,
                                                 lane * 16, row * WD * 2, 0, 0);
    };

    uint32_t valid = 0u, valid_next = 0u;
    int32_t ra;  // row codes of the next tile, resolved one tile ahead

    // One 32-row tile: compute from `tile`, load the next tile's rows into `nxt`. Past the
    // last tile every slot of the next tile resolves to the stand-in, so the loads need no
    // branch. O accumulates against the reference maximum set by the first tile and is
    // never rescaled (so it is only ever touched by the products into it); a later tile
    // whose maximum exceeds the reference by more than 2^kHeadroom raises `redo`.
    auto tile_step = [&](const bf16_t *tile, bf16_t *nxt, int64_t jt, bool first) __attribute__((always_inline)) {
        int32_t ra2 = -1;
        uint32_t valid_next2;
        int32_t dma_rows_code[RPW];
        const bool cn = contig(jt + WR);  // the tile loaded during this one
        const __amdgpu_buffer_rsrc_t crs = contig_rsrc(cn ? jt + WR : j0);
        if (cn) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) dma_row_contig(nxt, i, crs);
        } else {
#pragma unroll
            for (int i = 0; i < RPW; ++i) dma_rows_code[i] = __builtin_amdgcn_readlane(ra, RPW * wu + i);
            // all codes are in scalar registers before the first load goes out
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < RPW; ++i) dma_row(nxt, i, dma_rows_code[i]);
        }

        // ---- S^T = K Q^T: each K fragment feeds both head blocks
        f32x4 sacc[2][HB];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int b = 0; b < HB; ++b) sacc[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            bf16x8 ring[SDA + 1][2];
            const bf16_t *kb = tile + l16 * WP + g4 * 8;
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
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int b = 0; b < HB; ++b)
                        sacc[m][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[kk % (SDA + 1)][m], qf[b][kk],
                                                                             sacc[m][b], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // rows of the tile after next: the index read and the address arithmetic overlap
        // the matrix ops still in flight
        valid_next2 = contig(jt + 2 * WR) ? 0xffffffffu : tile_rows(jt + 2 * WR, ra2);

        // rows without data are masked to -inf; full tiles skip the mask
        if (valid != 0xffffffffu) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!((valid >> (16 * m + 4 * g4 + r)) & 1u)) {
#pragma unroll
                        for (int b = 0; b < HB; ++b) sacc[m][b][r] = -INFINITY;
                    }
        }
        bf16x8 pf[HB];
#pragma unroll
        for (int b = 0; b < HB; ++b) {
            // the next tile's row loads ride the softmax (VALU work, LDS idle): issued among
            // it they queue in the address unit while the wave computes, where one burst at
            // the start of the tile stalls every wavefront behind the others' loads

            // the scale is positive, so the max of the raw scores gives the max logit
            float smax = fmaxf(fmaxf(fmaxf(sacc[0][b][0], sacc[0][b][1]), fmaxf(sacc[0][b][2], sacc[0][b][3])),
                               fmaxf(fmaxf(sacc[1][b][0], sacc[1][b][1]), fmaxf(sacc[1][b][2], sacc[1][b][3])));
            {
                const auto x32 =
                    __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
                smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
                const auto x16 =
                    __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
                smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
            }
            const float tmax = smax * scale_log2;
            if (first) {
                m_ref[b] = fmaxf(m_ref[b], tmax);  // O and the sums are still zero
            } else if (__ballot(tmax > m_ref[b] + kHeadroom) != 0ull) {
                if (lane == 0) redo = 1;  // the loop is abandoned after this tile
            }
            // p = 2^(s * scale - m_ref), packed to bf16 in the A-operand layout of P.
            // v_exp_f32 flushes results below 2^-126 to zero, which only drops weights that
            // no bf16 sum could hold.

            const float nmu = (m_ref[b] == -INFINITY) ? 0.f : -m_ref[b];
            uint32_t pk[4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[m][b][r], scale_log2, nmu));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[m][b][r + 1], scale_log2, nmu));
                    pk[2 * m + r / 2] = pack_bf16x2(p0, p1);
                }
            pf[b] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_bf16x8(), pf[b], lacc[b], 0, 0, 0);
        }

        {
            // ---- O += P V: V fragments (8 rows of one dim per lane, in the row order of the
            // C layout above) from transposing LDS reads, each feeding both head blocks. The
            // first product after P's VALU writes carries the wait states they need.
            const int s4 = l16 >> 2, sc = l16 & 3;
            const bf16_t *v0 = tile + (4 * g4 + s4) * WP + 4 * sc;
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
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 vf = __builtin_shufflevector(vr[nd % (PVA + 1)][0], vr[nd % (PVA + 1)][1], 0, 1, 2, 3,
                                                          4, 5, 6, 7);
                if (nd == 0) {
                    pv_mfma2_after_valu(acc[0][0], acc[1][0], vf, pf[0], pf[1]);
                } else {
#pragma unroll
                    for (int b = 0; b < HB; ++b) pv_mfma(acc[b][nd], vf, pf[b]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        valid = valid_next;
        valid_next = valid_next2;
        ra = ra2;
        // the next tile's rows have landed in `nxt` (this wave's own loads), and after the
        // barrier everyone's have and nobody reads `tile` any more
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (j0 < j1) {
        if (contig(j0)) {
            valid = 0xffffffffu;
#pragma unroll
            for (int i = 0; i < RPW; ++i) dma_row_contig(KV0, i, contig_rsrc(j0));
        } else {
            valid = tile_rows(j0, ra);
#pragma unroll
            for (int i = 0; i < RPW; ++i) dma_row(KV0, i, __builtin_amdgcn_readlane(ra, RPW * wu + i));
        }
    }
    valid_next = contig(j0 + WR) ? 0xffffffffu : tile_rows(j0 + WR, ra);
    // every prologue load has landed before the loop (the loop's wait counters then start
    // from a clean state)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Tiles go in pairs (one per buffer) and the loop has a single exit: an odd count ends
    // with a tile past j1, whose slots are all masked (no weight). An abandoned loop still
    // runs to the end; its results are replaced below.
    for (int64_t jt = j0; jt < j1; jt += 2 * WR) {
        tile_step(KV0, KV1, jt, jt == j0);
        tile_step(KV1, KV0, jt + WR, false);
    }
    const bool abandoned = redo != 0;

    // (cos, sin) pairs of the lane's last 64 output dims, loaded in one batch
    float2 orp[4][2];
    if (rope_t != nullptr) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 2; ++e) orp[j][e] = rope_pair(rope_t, 16 * (NDN - 4 + j) + 4 * g4 + 2 * e, R);
    }
    pv_fence();
    // ---- epilogue. Each wavefront stages one 16-head block of bf16 output rows in its own
    // part of the (now idle) tile buffers, so no other wavefront's data is touched.
    constexpr int OSP = WD + 16;  // staged row pitch (bf16): 1056 bytes spread the banks
    static_assert(2 * 16 * OSP <= WR * WP, "two wavefronts' staging fits one tile buffer");
    bf16_t *const ostage = (wu < 2 ? KV0 : KV1) + (wu & 1) * 16 * OSP;
    // The products computed O^T: lane (l16, g4) holds dims 16nd + 4g4 + r
    // (r = 0..3, four consecutive dims) of head 16b + l16, and the denominator of that head
    // in every component of lacc[b], so each lane normalises, rotates back the last R dims
    // (pairs sit in one lane) and stores 8 bytes per dim block.
#pragma unroll
    for (int b = 0; b < HB; ++b) {
        const int h = head0 + 16 * b + l16;
        if (single) {
            const float sk = sink[h] * kLog2e;
            const float mr = m_ref[b];
            const float lv = lacc[b][0] + ((sk == -INFINITY) ? 0.f : exp2f(sk - mr));
            if (lse != nullptr && g4 == 0) {
                const float mu = (mr == -INFINITY) ? 0.f : mr;
                lse[(int64_t)t * H + h] = (lv > 0.f) ? (mu + log2f(lv)) * kLn2 : -INFINITY;
            }
            const float inv = lv > 0.f ? 1.f / lv : 0.f;
            const int nd_r = (WD - R) >> 4;
            // groups of 8 blocks: all 8 are packed before the 8 stores go out, so a store's
            // data registers are not rewritten while it is still in flight (one block at a
            // time, every store waited for the one before)
            constexpr int EG = 8;
#pragma unroll
            for (int ng = 0; ng < NDN; ng += EG) {
                uint2 pk[EG];
#pragma unroll
                for (int q8 = 0; q8 < EG; ++q8) {
                    const int nd = ng + q8;
                    const int d0 = 16 * nd + 4 * g4;
                    float x[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = agpr_read(acc[b][nd][r]) * inv;
                    // blocks before nd_r hold no rotated dim (a uniform test); within a
                    // block each pair is checked
                    if (rope_t != nullptr && nd >= nd_r) {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const float2 cp = (nd >= NDN - 4) ? orp[nd >= NDN - 4 ? nd - (NDN - 4) : 0][e]
                                                              : rope_pair(rope_t, d0 + 2 * e, R);
                            if (d0 + 2 * e >= WD - R) {
                                const float x0 = x[2 * e], x1 = x[2 * e + 1];
                                x[2 * e] = x0 * cp.x + x1 * cp.y;
                                x[2 * e + 1] = x1 * cp.x - x0 * cp.y;
                            }
                        }
                    }
                    pk[q8] = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                }
#pragma unroll
                for (int q8 = 0; q8 < EG; ++q8)
                    *reinterpret_cast<uint2 *>(ostage + l16 * OSP + 16 * (ng + q8) + 4 * g4) = pk[q8];
                // one group at a time: hoisted reads of later groups would need registers
                // the accumulators still hold
                __builtin_amdgcn_sched_barrier(0);
            }
            // the block's 16 head rows go out whole: one 1 KiB row per store instruction (a
            // lane's 8-byte pieces of 16 rows would be 16 partial-line writes per store)
#pragma unroll
            for (int hr = 0; hr < 16; ++hr)
                *reinterpret_cast<uint4 *>(out + ((int64_t)t * H + head0 + 16 * b + hr) * WD + 8 * lane) =
                    *reinterpret_cast<const uint4 *>(ostage + hr * OSP + 8 * lane);
        } else {
            const int64_t pu = ((int64_t)t * nsplit + sp) * H + h;
            float *pml = part;                                                               // [T][nsplit][H][2]
            bf16_t *pacc = reinterpret_cast<bf16_t *>(part + (int64_t)T * nsplit * H * 2);  // [T][nsplit][H][D] bf16
            if (g4 == 0) {
                pml[pu * 2] = m_ref[b];
                pml[pu * 2 + 1] = lacc[b][0];
            }
#pragma unroll
            for (int ng = 0; ng < NDN; ng += 4) {
                uint2 v[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    v[q4] = make_uint2(pack_bf16x2(agpr_read(acc[b][ng + q4][0]), agpr_read(acc[b][ng + q4][1])),
                                       pack_bf16x2(agpr_read(acc[b][ng + q4][2]), agpr_read(acc[b][ng + q4][3])));
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<uint2 *>(pacc + pu * WD + 16 * (ng + q4) + 4 * g4) = v[q4];
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (abandoned) {
        // rare: a head's maximum grew past the headroom after the first tile; this wave's
        // 32 heads are computed again by a plain two-pass routine, which overwrites what the
        // epilogue above stored (the same wave wrote it, so the stores land in order)
        unit_fallback(q, sink, c, j0, j1, ratio, sidx, idx_t, N, kv, swa, swa_rows,
                      rope_cs ? rope_cs + (int64_t)t * R : nullptr, R, scale_log2, t, T, H, head0, nsplit, sp,
                      out, lse, part);
    }
}

}  // namespace

// bf16, D = 512, whole 128-head groups, and rows addressable by a 32-bit byte offset within
// a sequence's region (2^21 rows of 1 KiB)
bool w32_attn_ok(csa_dtype dt, int H, int D, int64_t N, int swa_rows) {
    return dt == CSA_BF16 && D == WD && H % WH == 0 && N <= (int64_t{1} << 21) && swa_rows <= (1 << 21);
}

int launch_attn_w32(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st) {
    const int64_t U = (int64_t)a.T * nsplit * (a.H / WH);
    const int64_t blocks = ((U + 7) / 8) * 8;
    hipLaunchKernelGGL(attn_w32_kernel, dim3((unsigned)blocks), dim3(64 * NWV), 0, st, (const bf16_t *)a.q,
                       (const bf16_t *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2, (const bf16_t *)a.swa, a.swa_pos0,
                       a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs, a.rope_dim, a.T, a.B, a.N, a.H,
                       (bf16_t *)a.out, a.lse, (float *)a.ws, nsplit, split_slots);
    return check_launch("attn_w32_kernel");
}

}  // namespace csa
