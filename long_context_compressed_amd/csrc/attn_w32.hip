// Shared-KV MQA with an attention sink, 128 heads per workgroup, on gfx950 matrix cores.
//
// "DeepSeek-V4 混合注意力" §4.2 (one compressed vector is both K and V for every query head),
// §5 (HCA: every visible summary), §6 (SWA rows, sink softmax, partial RoPE / inverse RoPE).
//
// One workgroup of 4 wavefronts (one per SIMD) covers 128 heads of one query. The two
// products of a 32-row tile are split differently over the wavefronts:
//   - S^T = K Q^T (rows x heads, MFMA 32x32x16 bf16): wavefront w owns heads 32w .. 32w+31
//     and all 512 dims, so q^T (32 heads x 512 dims, bf16) stays in 128 registers; each
//     lane's 16 scores belong to one head, so a head's maximum needs one lane swap. The C
//     layout of S^T gives P in the B-operand layout of the next product; each wavefront
//     turns its S^T into P (online softmax against a reference maximum fixed by the first
//     tile, so O is never rescaled) and puts it into LDS (two 16-row k-steps, 1 KiB each,
//     lane-linear).
//   - O^T += V^T P^T (MFMA 32x32x16 bf16): wavefront w owns dims 128w .. 128w+127 of all
//     128 heads (its 128 x 128 fp32 output block fills the 256 accumulation registers),
//     reads P of every head from LDS and only its quarter of the V fragments (transposing
//     reads); each V fragment and each P fragment feeds four matrix ops.
// The 32x32x16 ops (rather than 16x16x32) halve the matrix instructions a wavefront issues.
// Tiles are pipelined over four LDS tile buffers. While tile i's S^T runs, the rows of tile
// i+2 go from memory straight into LDS (buffer loads with the LDS destination), one row per
// two of its matrix-op steps; then the products of tile i-1 run with the softmax of tile i
// (VALU work) issued a micro-step at a time between them. A single wavefront per SIMD issues
// one instruction at a time, so the loop is written to keep the non-matrix instructions
// few: the main slots and the SWA slots start on tile boundaries (every tile's rows come
// from one region, one buffer resource per tile), and each row's offset is formed in a lane
// beforehand. The softmax denominators ride one more matrix op per head block against a
// ones operand. If a later tile's maximum exceeds the reference by more than 2^24 (rare),
// the results are abandoned and a plain two-pass routine computes the wavefront's 32 heads
// again.
#include <type_traits>

#include "attn_mfma.hpp"
#include "internal.hpp"

namespace csa {

namespace {

using namespace amfma;

constexpr int NWV = 4;            // wavefronts per workgroup
constexpr int HB = 2;             // 16-head blocks of a wavefront's S^T
constexpr int WH = 16 * HB * NWV; // heads per workgroup
constexpr int OB = WH / 16;       // 16-head blocks of the workgroup (every one in P V)
constexpr int DPW = NDN / NWV;    // 16-dim output blocks of a wavefront
constexpr int RPW = WR / NWV;     // tile rows loaded per wavefront
constexpr int TB = WR * WP;       // bf16 elements of one tile buffer
constexpr int NTB = 4;            // tile buffers
constexpr int kW32Idx = 1024;     // top-k entries of a query kept in LDS (the whole list)
static_assert(kW32Idx % (64 * NWV) == 0, "the index copy splits evenly over the threads");
static_assert(kW32Idx <= kIdxCache, "the two-pass routine reads the LDS copy below kIdxCache");
// s_waitcnt: every LDS access done, all but the last RPW vector-memory operations (the row
// loads of the tile two ahead) done
constexpr int kWaitTileAhead = RPW | (7 << 4) | (0 << 8);
static_assert(NDN % NWV == 0, "the output dims split evenly over the wavefronts");
constexpr int SDA = 3;            // K fragment chunks (16 dims) read ahead
constexpr int PVA = 2;            // P fragments read ahead
constexpr float kHeadroom = 24.f; // log2 growth of a head's maximum the tile loop absorbs

typedef int i32x4s __attribute__((ext_vector_type(4)));

// max of two scores (finite or -inf) without the operand canonicalisation fmaxf brings:
// the median of a, b and +inf
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// The output accumulators live in AGPRs: the matrix ops that update them are written out
// with an "a" constraint (the compiler's own MFMA selection would keep every result in one
// register class and shuffle the 256 accumulators between the two). The compiler does not
// see these as matrix ops, so the hazards it would otherwise cover are covered here: a
// source register possibly written by a VALU move gets >= 5 wait states (the s_nop at the
// head of the first product of each V fragment), and the results are read back only after
// two s_nop 15 (pv_fence).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void pv_mfma32(f32x16 &acc, const bf16x8 a, const bf16x8 b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void pv_mfma32_after_valu(f32x16 &acc, const bf16x8 a, const bf16x8 b) {
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// one accumulator read out of its AGPR where it is used (left to itself the compiler copies
// every accumulator to VGPRs at once, more than there are)
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}
__device__ __forceinline__ void pv_fence() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// raw buffer resource words over [p, p + bytes) (wave-uniform; loads past the end return
// zeros)
__device__ __forceinline__ i32x4s rows_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const int lo = (int)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const int hi = (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    return i32x4s{lo, hi, (int)__builtin_amdgcn_readfirstlane(bytes), kBufDword3};
}

// LDS position of 16-byte chunk g (dims 8g .. 8g+7) of a tile row. Within each 256-byte
// group (128 dims) the bits (s1, bb, h, j) of g = 8 s1 + 4 bb + 2 h + j move to
// 8 h + 4 s1 + 2 bb + j: the two 16-dim halves (h) of a 32-dim block then sit 128 bytes
// apart, so the transposing V reads of the two 16-lane groups of a half fall in disjoint
// banks. Rows with bit 3 set also flip bit 0 of the position: a 16-byte read is served 16
// lanes at a time, and rows r and r + 8 (1,056 bytes x 8 apart) would otherwise share banks.
__host__ __device__ constexpr int chunk_pos(int g) {
    return (g & ~15) | (((g >> 1) & 1) << 3) | (((g >> 3) & 1) << 2) | (((g >> 2) & 1) << 1) | (g & 1);
}
// the chunk whose position is p (the inverse permutation)
__host__ __device__ constexpr int chunk_at(int p) {
    return (p & ~15) | (((p >> 2) & 1) << 3) | (((p >> 1) & 1) << 2) | (((p >> 3) & 1) << 1) | (p & 1);
}
static_assert(chunk_at(chunk_pos(13)) == 13 && chunk_pos(chunk_at(6)) == 6 && chunk_pos(2) == 8, "inverse pair");

// One 1 KiB row from memory straight into LDS: lane i moves bytes 16i .. 16i+15 of the row
// at `soff` within the resource to LDS byte address dst + 16i. Written as assembly so that
// the compiler does not track it (it would otherwise wait for these loads before every LDS
// read it cannot prove disjoint from them, which drains the prefetch); completion is waited
// for explicitly before the barrier that ends a tile. It sets M0 (the LDS address of the
// direct-to-LDS load; one wait state before the load reads it); nothing else in this
// file's kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void row_dma(i32x4s rs, uint32_t voff, uint32_t soff, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "s"(dst)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// workgroup barrier without a memory fence (the fence would wait for every load in flight,
// the row loads of the tile two ahead included); the wait before it says what has
// completed, and the empty asm keeps the compiler from moving memory accesses across it
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

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
                bf16_t *__restrict__ out, float *__restrict__ lse, int64_t max_slots)
{
    __shared__ __attribute__((aligned(16))) bf16_t KVB[NTB * TB];  // tile buffers
    __shared__ __attribute__((aligned(16))) u32x4w PB[2][OB * 64];  // P of two tiles, fragment order
    __shared__ int32_t sidx[kW32Idx];
    __shared__ float invs[WH];
    __shared__ int redo;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n32 = lane & 31, kg = lane >> 5;  // lane of a 32-wide matrix-op row, and its half
    // XCD-aware placement: units (query, head group) are dealt to the 8 XCDs in contiguous
    // runs, so neighbouring queries (which share SWA rows and summaries) meet in one L2
    const int HGN = H / WH;
    const int64_t U = (int64_t)T * HGN;
    const int64_t per_xcd = (U + 7) / 8;
    const int64_t bid = blockIdx.x;
    const int64_t u = (bid & 7) * per_xcd + (bid >> 3);
    if ((bid >> 3) >= per_xcd || u >= U) return;
    const int hg = (int)(u % HGN);
    const int t = (int)(u / HGN);
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int hw0 = hg * WH;                 // first head of the workgroup
    const int head0 = hw0 + 16 * HB * wu;    // first S^T head of this wave; block b = head0 + 16b ..

    // The loads that depend only on the query (q, its RoPE pairs, the sinks, the top-k
    // indices) are all issued before anything waits on the row context.
    constexpr int IPT = kW32Idx / (64 * NWV);  // top-k indices per thread
    int32_t ir[IPT];
    {
        const int64_t nc0 = (ratio <= 0) ? (k < kW32Idx ? k : kW32Idx) : 0;
#pragma unroll
        for (int m = 0; m < IPT; ++m) {
            const int x = threadIdx.x + 64 * NWV * m;
            ir[m] = (x < nc0) ? idx[(int64_t)t * k + x] : 0;
        }
    }
    const float sk = sink[head0 + n32];  // the sink of this lane's S^T head

    // q^T fragments of the wave's 32 heads for the whole query, the B operands of the
    // 32x32x16 S^T products: chunk kc holds dims 16kc + 8(l / 32) .. +7 of head l % 32.
    // Every load is issued first (they overlap; the (cos, sin) pairs of the last 64 dims
    // included), then the chunks that reach the rotated dims are rotated.
    constexpr int QC = 2 * KKN;  // 16-dim chunks of a head
    const float *rope_t = rope_cs ? rope_cs + (int64_t)t * R : nullptr;
    bf16x8 qf[QC];
    {
        float2 qr[4][4];
        if (rope_t != nullptr) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) qr[j][e] = rope_pair(rope_t, 16 * (QC - 4 + j) + 8 * kg + 2 * e, R);
        }
        const bf16_t *qrow = q + ((int64_t)t * H + head0 + n32) * WD;
#pragma unroll
        for (int kc = 0; kc < QC; ++kc) qf[kc] = ld_bf16x8(qrow + 16 * kc + 8 * kg);
        if (rope_t != nullptr) {
            // (chunk kc = dims 32(kc / 2) + 8g with g = 2(kc % 2) + kg, the form the rotation helpers take)
#pragma unroll
            for (int kc = 0; kc < QC - 4; ++kc)
                if (16 * (kc + 1) > WD - R)  // (wave-uniform: only chunks that reach the rotated dims)
                    qf[kc] = rope_fragment(qf[kc], kc >> 1, 2 * (kc & 1) + kg, rope_t, R);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kc = QC - 4 + j;
                const float cs[4] = {qr[j][0].x, qr[j][1].x, qr[j][2].x, qr[j][3].x};
                const float sn[4] = {qr[j][0].y, qr[j][1].y, qr[j][2].y, qr[j][3].y};
                qf[kc] = rope_fragment_cs(qf[kc], kc >> 1, 2 * (kc & 1) + kg, cs, sn, R);
            }
        }
    }

    const RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    const int64_t j1 = (max_slots < c.nslots) ? max_slots : c.nslots;  // slots [0, j1)

    // softmax state of this lane's S^T head (head0 + l % 32): the reference maximum m_ref,
    // and the denominator, accumulated by matrix ops against a ones operand (every component
    // of lacc holds it) so it sums the same bf16 weights that enter O. The sink's
    // 2^(sink - m_ref) is added at the end.
    const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4w{0u, 0u, 0u, 0u});
    float m_ref = sk * kLog2e;
    f32x16 lacc = {};
    // O^T in 32 x 32 blocks: head block hb (heads 32hb .. 32hb+31 of the workgroup) x dim block db
    // (dims 128w + 32db ..); lane l holds head 32hb + l % 32, dims 32db + 8(j / 4) + 4(l / 32) + j % 4
    f32x16 acc[OB / 2][DPW / 2];
    // zeroed by matrix ops into AGPRs, so the accumulators never pass through VGPRs; the
    // zero operand may have just been written by a VALU move, hence the wait states
#pragma unroll
    for (int hb = 0; hb < OB / 2; ++hb)
#pragma unroll
        for (int db = 0; db < DPW / 2; ++db)
            asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc[hb][db]) : "v"(zero8));

    // The top-k indices are read once into LDS.
    const int64_t jm = (j1 < c.nmain) ? j1 : c.nmain;  // main slots: [0, jm)
    const int64_t ncache = (jm < kW32Idx) ? jm : kW32Idx;
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
    const int s_u = __builtin_amdgcn_readfirstlane(c.s);
    const i32x4s kv_rs = rows_rsrc(kv + (int64_t)s_u * N * WD, (uint32_t)(N * WD * 2));
    const i32x4s swa_rs = rows_rsrc(swa != nullptr ? swa + (int64_t)s_u * swa_rows * WD : kv,
                                    swa != nullptr ? (uint32_t)swa_rows * WD * 2 : 0u);
    const uint32_t kvb = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(const char *)KVB);
    // lane i fills LDS chunk i of a row; rows with bit 3 set (the rows of odd waves) hold
    // their chunks with bit 0 of the position flipped
    const uint32_t voff = (uint32_t)chunk_at(lane ^ (wu & 1)) * 16u;
    // Tiles 0 .. ntm-1 hold the main slots (top-k entries or summaries, 32 per tile, the
    // last one padded), tiles ntm .. nt-1 the SWA slots, so the rows of a tile all come from
    // one region. Lane r < 32 describes row r of a tile: its byte offset in the region (row
    // 0 when the row has no data), and a ballot gives the tile's validity mask. A sparse
    // slot's top-k entry is read from the LDS copy of the list (this kernel runs only when
    // it holds the whole list) well before the offset is formed. 32-bit arithmetic: slots
    // and rows stay below 2^31.
    const int nmain32 = (int)jm, nwin32 = (int)(j1 - jm);
    const int ntm = __builtin_amdgcn_readfirstlane((nmain32 + WR - 1) / WR);  // (wave-uniform)
    const int lo_rel = (int)(c.lo - c.swa0), nkv32 = (int)N;
    auto code_read = [&](int i) __attribute__((always_inline)) -> int {
        const int j = i * WR + (lane & 31);
        if (ratio > 0) return j;
        return sidx[j < kW32Idx ? j : kW32Idx - 1];
    };
    auto code_finish = [&](int i, int id, uint32_t &off) __attribute__((always_inline)) -> uint32_t {
        const int r = lane & 31;
        bool ok;
        int row;
        if (i < ntm) {
            row = id;
            ok = i * WR + r < nmain32 && id >= 0 && id < nkv32;
        } else {
            const int w = (i - ntm) * WR + r;
            row = lo_rel + w;
            ok = w < nwin32 && row >= 0 && row < swa_rows;
        }
        off = ok ? (uint32_t)row * (WD * 2) : 0u;
        return (uint32_t)(__ballot(ok) & 0xffffffffull);
    };
    // byte offsets of this wave's RPW rows of a tile, in scalar registers
    auto row_offs = [&](uint32_t offs, uint32_t (&so)[RPW]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) so[r] = __builtin_amdgcn_readlane(offs, RPW * wu + r);
    };
    // row r of this wave's share of a tile into the tile buffer at bf16 offset nb
    auto issue_row = [&](const i32x4s rs, int nb, int r, uint32_t soff) __attribute__((always_inline)) {
        row_dma(rs, voff, soff, kvb + (uint32_t)(nb + (RPW * wu + r) * WP) * 2u);
    };

    // O^T += V^T P^T for the tile in the buffer at bf16 offset vb, with P from PB[pr], in
    // 32 x 32 x 16 matrix ops: the tile's 32 rows are two k-steps of 16, each row set taken
    // in the order the S^T C layout hands P over (k-step s: rows 16s + 4kg + 0..3 and
    // 16s + 8 + 4kg + 0..3 for the lanes of half kg). Per k-step the V fragments of the
    // wave's four 32-dim blocks (two transposing reads each) stay in registers while the P
    // fragments of the four 32-head blocks stream past, each feeding four products. P of
    // 32 heads for one k-step is one 16-byte LDS read per lane, in the order S^T wrote it.
    // The first k-step's V fragments and the first P fragments are read ahead (pv_pre).
    // `step(p)` is called after product p (0 .. 31) and, with p = 100 + s, before the first
    // product of k-step s: the softmax of the next tile goes there, an instruction at a time.
    auto vfrag = [&](int vb, int db, int s) __attribute__((always_inline)) -> bf16x8 {
        const bf16_t *base = KVB + vb + 16 * DPW * wu + 32 * (db >> 1) + 16 * (db & 1) + 64 * ((lane >> 4) & 1) +
                             4 * (lane & 3) +
                             ((lane & 15) >> 2) * WP;
        const bf16x4v lo = __builtin_bit_cast(bf16x4v, ld_tr(base + (16 * s + 4 * kg) * WP));
        // (rows 8..15 of a 16: chunk position bit 0 flipped, i.e. 8 elements over)
        const bf16x4v hi = __builtin_bit_cast(bf16x4v, ld_tr(base + (16 * s + 8 + 4 * kg) * WP + 8 - 16 * ((lane >> 1) & 1)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto pfrag = [&](int pr, int hb, int s) __attribute__((always_inline)) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, PB[pr][(2 * hb + s) * 64 + lane]);
    };
    struct PvPre {
        bf16x8 a[DPW / 2];
        bf16x8 b[PVA];
    };
    auto pv_pre = [&](int vb, int pr, PvPre &P) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < DPW / 2; ++db) P.a[db] = vfrag(vb, db, 0);
#pragma unroll
        for (int cc = 0; cc < PVA; ++cc) P.b[cc] = pfrag(pr, cc, 0);
    };
    auto pv_phase = [&](int vb, int pr, const PvPre &P, auto &&step) __attribute__((always_inline)) {
        static_for<0, 2>([&](auto SK) __attribute__((always_inline)) {
            constexpr int sk2 = decltype(SK)::value;
            bf16x8 va[DPW / 2];
            bf16x8 pr_[PVA + 1];
            if constexpr (sk2 == 0) {
#pragma unroll
                for (int db = 0; db < DPW / 2; ++db) va[db] = P.a[db];
#pragma unroll
                for (int cc = 0; cc < PVA; ++cc) pr_[cc] = P.b[cc];
            } else {
#pragma unroll
                for (int db = 0; db < DPW / 2; ++db) va[db] = vfrag(vb, db, 1);
#pragma unroll
                for (int cc = 0; cc < PVA; ++cc) pr_[cc] = pfrag(pr, cc, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            step(std::integral_constant<int, 100 + sk2>{});
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, OB / 2>([&](auto HBI) __attribute__((always_inline)) {
                constexpr int hb = decltype(HBI)::value;
                if constexpr (hb + PVA < OB / 2) pr_[(hb + PVA) % (PVA + 1)] = pfrag(pr, hb + PVA, sk2);
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, DPW / 2>([&](auto DBI) __attribute__((always_inline)) {
                    constexpr int db = decltype(DBI)::value;
                    if constexpr (hb == 0)
                        pv_mfma32_after_valu(acc[hb][db], va[db], pr_[hb % (PVA + 1)]);
                    else
                        pv_mfma32(acc[hb][db], va[db], pr_[hb % (PVA + 1)]);
                    step(std::integral_constant<int, 16 * sk2 + 4 * hb + db>{});
                    __builtin_amdgcn_sched_barrier(0);
                });
            });
        });
    };

    const int nt = ntm + (nwin32 + WR - 1) / WR;  // tiles

    // Tile i (in buffer i % 4): S^T, with the rows of tile i+2 requested a row at a time
    // between its matrix ops, then its softmax interleaved with the products of tile i-1
    // (none for the first tile), and P of tile i into PB[i & 1].
    uint32_t v0 = 0u, v1 = 0u, v2 = 0u;  // validity of tiles i, i+1, i+2
    uint32_t oa = 0u;                     // row offsets of tile i+2
    float growth = -INFINITY;  // largest tile maximum above the reference, log2 units
    float nmu = 0.f;             // -m_ref (0 for an empty reference), fixed after the first tile
    auto tile_iter = [&](int i, auto FIRST) __attribute__((always_inline)) {
        constexpr bool kFirst = decltype(FIRST)::value;
        const int cb = (i & 3) * TB, pb = ((i + 3) & 3) * TB, db = ((i + 2) & 3) * TB;
        uint32_t so[RPW];
        row_offs(oa, so);
        const i32x4s drs = (i + 2 >= ntm) ? swa_rs : kv_rs;
        const int id3 = code_read(i + 3);
        PvPre pre;

        // ---- S^T = K Q^T (rows x the wave's 32 heads) in 32 matrix ops of 16 dims; lane l
        // reads row l % 32, dims 16kc + 8(l / 32) .. +7 (rows 1,056 bytes apart: the 8 lanes a
        // 16-byte read serves hit distinct banks)
        f32x16 sacc = {};
        {
            bf16x8 ring[SDA + 1];
            const bf16_t *kb = KVB + cb + n32 * WP + 8 * (kg ^ ((n32 >> 3) & 1));  // + 8 chunk_pos(2kc)
#pragma unroll
            for (int cc = 0; cc < SDA; ++cc) ring[cc] = ld_bf16x8(kb + 8 * chunk_pos(2 * cc));
#pragma unroll
            for (int kc = 0; kc < QC; ++kc) {
                if (kc + SDA < QC) ring[(kc + SDA) % (SDA + 1)] = ld_bf16x8(kb + 8 * chunk_pos(2 * (kc + SDA)));
                if (!kFirst && kc == QC - 5) pv_pre(pb, (i - 1) & 1, pre);
                if ((kc & 3) == 3) issue_row(drs, db, kc >> 2, so[kc >> 2]);
                __builtin_amdgcn_sched_barrier(0);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[kc % (SDA + 1)], qf[kc], sacc, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        static_assert(QC == 4 * RPW, "one row load per four k-chunks");
        // row offsets of tile i+3
        uint32_t oa3;
        const uint32_t v3 = code_finish(i + 3, id3, oa3);
        // rows without data are masked to -inf; full tiles skip the mask
        if (v0 != 0xffffffffu) {
            const uint32_t vb = v0 >> (4 * kg);  // bit 8q + r: row 8q + 4kg + r (component 4q + r)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!((vb >> (8 * q4 + r)) & 1u)) sacc[4 * q4 + r] = -INFINITY;
        }
        // ---- softmax of this tile in 26 micro-steps of one to four independent instructions
        // (each depending on an earlier step), spread between the matrix ops of the previous
        // tile so that every dependency has a matrix op to hide behind:
        // p = 2^(s * scale - m_ref) packed to bf16, components 8s .. 8s+7 being the B
        // operand of k-step s of P V. v_exp_f32 flushes results below 2^-126 to zero, which
        // only drops weights that no bf16 sum could hold.
        float tq[8];
        float ev[16];
        uint32_t pk[8];
        auto sm_micro = [&](auto UI) __attribute__((always_inline)) {
            constexpr int u = decltype(UI)::value;
            if constexpr (u < 4) {
                tq[2 * u] = fmax2(sacc[4 * u], sacc[4 * u + 1]);
                tq[2 * u + 1] = fmax2(sacc[4 * u + 2], sacc[4 * u + 3]);
            } else if constexpr (u == 4) {
                tq[0] = fmax2(tq[0], tq[1]);
                tq[2] = fmax2(tq[2], tq[3]);
            } else if constexpr (u == 5) {
                tq[4] = fmax2(tq[4], tq[5]);
                tq[6] = fmax2(tq[6], tq[7]);
            } else if constexpr (u == 6) {
                tq[0] = fmax2(tq[0], tq[2]);
                tq[4] = fmax2(tq[4], tq[6]);
            } else if constexpr (u == 7) {
                tq[0] = fmax2(tq[0], tq[4]);
            } else if constexpr (u == 8) {
                const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(tq[0]), __float_as_uint(tq[0]), false,
                                                                false);
                tq[1] = __uint_as_float(x[0]);
                tq[2] = __uint_as_float(x[1]);
            } else if constexpr (u == 9) {
                tq[0] = fmax2(tq[1], tq[2]);
            } else if constexpr (u == 10) {
                // the scale is positive, so the max of the raw scores gives the max logit
                const float tmax = tq[0] * scale_log2;
                if constexpr (kFirst) {
                    m_ref = fmaxf(m_ref, tmax);  // O and the sums are still zero
                    nmu = (m_ref == -INFINITY) ? 0.f : -m_ref;
                } else {
                    growth = fmaxf(growth, tmax - m_ref);
                }
            } else if constexpr (u >= 11 && u <= 19) {
                constexpr int q2 = u - 11;  // exponents of values 2q2-2, 2q2-1; arguments of 2q2, 2q2+1
                if constexpr (q2 >= 1) {
                    ev[2 * q2 - 2] = __builtin_amdgcn_exp2f(ev[2 * q2 - 2]);
                    ev[2 * q2 - 1] = __builtin_amdgcn_exp2f(ev[2 * q2 - 1]);
                }
                if constexpr (q2 < 8) {
                    ev[2 * q2] = fmaf(sacc[2 * q2], scale_log2, nmu);
                    ev[2 * q2 + 1] = fmaf(sacc[2 * q2 + 1], scale_log2, nmu);
                }
            } else if constexpr (u >= 20 && u <= 23) {
                constexpr int j = u - 20;
                pk[2 * j] = pack_bf16x2(ev[4 * j], ev[4 * j + 1]);
                pk[2 * j + 1] = pack_bf16x2(ev[4 * j + 2], ev[4 * j + 3]);
            } else if constexpr (u == 24) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16x8 pf = __builtin_bit_cast(
                        bf16x8, make_uint4(pk[4 * s2], pk[4 * s2 + 1], pk[4 * s2 + 2], pk[4 * s2 + 3]));
                    lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones_bf16x8(), pf, lacc, 0, 0, 0);
                }
            } else if constexpr (u == 25) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    PB[i & 1][(2 * wu + s2) * 64 + lane] =
                        u32x4w{pk[4 * s2], pk[4 * s2 + 1], pk[4 * s2 + 2], pk[4 * s2 + 3]};
            }
        };
        constexpr int kMicro = 26;
        if constexpr (kFirst) {
            static_for<0, kMicro>([&](auto UI) __attribute__((always_inline)) { sm_micro(UI); });
        } else {
            // micro-steps 0-1 before the first product, 16-17 while the second k-step's
            // fragments are read, the others one after each product
            pv_phase(pb, (i - 1) & 1, pre, [&](auto PI) __attribute__((always_inline)) {
                constexpr int p = decltype(PI)::value;
                if constexpr (p == 100) {
                    sm_micro(std::integral_constant<int, 0>{});
                    sm_micro(std::integral_constant<int, 1>{});
                } else if constexpr (p == 101) {
                    sm_micro(std::integral_constant<int, 16>{});
                    sm_micro(std::integral_constant<int, 17>{});
                } else if constexpr (p < 14 || (p >= 16 && p < 24)) {
                    sm_micro(std::integral_constant<int, p + 2>{});
                }
            });
        }

        v0 = v1;
        v1 = v2;
        v2 = v3;
        oa = oa3;
        // tile i+1's rows have landed (this wave's loads of it are older than the 8 of tile
        // i+2), P of this tile is in LDS; after the barrier everyone's have, and nobody
        // reads tile i-1 or P of tile i-1 any more
        __builtin_amdgcn_s_waitcnt(kWaitTileAhead);
        stage_barrier();
    };

    if (nt > 0) {
        uint32_t o0, o1, so[RPW];
        v0 = code_finish(0, code_read(0), o0);
        v1 = code_finish(1, code_read(1), o1);
        v2 = code_finish(2, code_read(2), oa);
        row_offs(o0, so);
#pragma unroll
        for (int r = 0; r < RPW; ++r) issue_row(ntm > 0 ? kv_rs : swa_rs, 0, r, so[r]);
        row_offs(o1, so);
#pragma unroll
        for (int r = 0; r < RPW; ++r) issue_row(ntm > 1 ? kv_rs : swa_rs, TB, r, so[r]);
        __builtin_amdgcn_s_waitcnt(kWaitTileAhead);
        stage_barrier();
        tile_iter(0, std::true_type{});
        for (int i = 1; i < nt; ++i) tile_iter(i, std::false_type{});
    }
    // (cos, sin) pairs of the lane's output dims when this wave's dims reach the rotated
    // ones, loaded before the last products. (The row loads of the two tiles past the end,
    // stand-ins, may still be landing in their tile buffers, which nothing below touches;
    // the kernel waits for them before it ends.)
    const bool rot = rope_t != nullptr && 16 * DPW * (wu + 1) > WD - R;
    float2 orp[DPW / 2][4][2];
    if (rot) {
#pragma unroll
        for (int db = 0; db < DPW / 2; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    orp[db][q4][e] = rope_pair(rope_t, 16 * DPW * wu + 32 * db + 8 * q4 + 4 * kg + 2 * e, R);
    }
    // denominator of this lane's S^T head, shared with the waves that hold its outputs
    float lse_v;
    {
        const float skl = sk * kLog2e;
        const float lv = lacc[0] + ((skl == -INFINITY) ? 0.f : exp2f(skl - m_ref));
        const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
        lse_v = (lv > 0.f) ? (mu + log2f(lv)) * kLn2 : -INFINITY;
        if (kg == 0) invs[32 * wu + n32] = lv > 0.f ? 1.f / lv : 0.f;
    }
    if (__ballot(growth > kHeadroom) != 0ull && lane == 0) redo = 1;
    __syncthreads();
    const bool abandoned = redo != 0;
    if (!abandoned) {
        if (nt > 0) {
            PvPre pre;
            pv_pre(((nt - 1) & 3) * TB, (nt - 1) & 1, pre);
            pv_phase(((nt - 1) & 3) * TB, (nt - 1) & 1, pre, [](auto) __attribute__((always_inline)) {});
        }
        pv_fence();
        if (lse != nullptr && kg == 0) lse[(int64_t)t * H + head0 + n32] = lse_v;
        // ---- epilogue. Lane l holds, per 32 x 32 block (hb, db), dims 32db + 8q + 4kg + r
        // (q, r = 0..3: four runs of four consecutive dims) of head 32hb + l % 32: it
        // normalises them, rotates back the rotated dims (pairs sit in one lane) and stages 8
        // bytes per run; each head block's 32 x 256-byte row pieces then go out as eight
        // 1 KiB stores (four whole rows each). Staged rows are 256 bytes, 16-byte chunk c of
        // row h at chunk c ^ (h % 16), so the 32 rows' writes of one chunk spread over the
        // banks and the reads stay 16-byte aligned. The staging alternates between two tile
        // buffers that no wave reads any more (and no row load writes), so a head block's
        // normalisation overlaps the previous block's LDS round trip and stores.
        constexpr int OSP = 16 * DPW;  // staged row pitch (bf16): 256 bytes
        static_assert(NWV * 32 * OSP <= TB, "the staging of every wave fits one tile buffer");
        bf16_t *const ostage0 = KVB + ((nt + 2) & 3) * TB + wu * 32 * OSP;
        bf16_t *const ostage1 = KVB + (nt & 3) * TB + wu * 32 * OSP;
#pragma unroll
        for (int hb = 0; hb < OB / 2; ++hb) {
            const float inv = invs[32 * hb + n32];
            uint2 pko[DPW / 2][4];
#pragma unroll
            for (int db = 0; db < DPW / 2; ++db) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d0 = 16 * DPW * wu + 32 * db + 8 * q4 + 4 * kg;
                    float x[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = agpr_read(acc[hb][db][4 * q4 + r]) * inv;
                    // blocks below the rotated dims skip the test (a uniform one); within a
                    // block each pair is checked
                    if (rot && 16 * DPW * wu + 32 * db + 32 > WD - R) {
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            if (d0 + 2 * e >= WD - R) {
                                const float2 cp = orp[db][q4][e];
                                const float x0 = x[2 * e], x1 = x[2 * e + 1];
                                x[2 * e] = x0 * cp.x + x1 * cp.y;
                                x[2 * e + 1] = x1 * cp.x - x0 * cp.y;
                            }
                        }
                    }
                    pko[db][q4] = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                }
            }
            bf16_t *const ostage = (hb & 1) ? ostage1 : ostage0;
#pragma unroll
            for (int db = 0; db < DPW / 2; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<uint2 *>(ostage + n32 * OSP + 8 * ((4 * db + q4) ^ (n32 & 15)) + 4 * kg) =
                        pko[db][q4];
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const int hr = 4 * s2 + (lane >> 4), cw = lane & 15;
                *reinterpret_cast<uint4 *>(out + ((int64_t)t * H + hw0 + 32 * hb + hr) * WD + 16 * DPW * wu + 8 * cw) =
                    *reinterpret_cast<const uint4 *>(ostage + hr * OSP + 8 * (cw ^ (hr & 15)));
            }
        }
    } else {
        // rare: a head's maximum grew past the headroom after the first tile; this wave's
        // 32 S^T heads are computed again by a plain two-pass routine (nothing was stored)
        unit_fallback(q, sink, c, 0, j1, ratio, sidx, idx_t, N, kv, swa, swa_rows, rope_t, R, scale_log2, t, T, H,
                      head0, 1, 0, out, lse, nullptr);
    }
    // no load into this workgroup's LDS may still be in flight when it ends
    __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

// bf16, D = 512, whole 128-head groups, rows addressable by a 32-bit byte offset within a
// sequence's region (2^21 rows of 1 KiB), and a top-k list that fits the LDS copy
bool w32_attn_ok(csa_dtype dt, int H, int D, int64_t N, int swa_rows, int ratio, int k) {
    return dt == CSA_BF16 && D == WD && H % WH == 0 && N <= (int64_t{1} << 21) && swa_rows <= (1 << 21) &&
           (ratio > 0 || k <= kW32Idx);
}

int launch_attn_w32(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st) {
    if (nsplit != 1) return fail(CSA_EUNSUPPORTED, "attn_w32_kernel: one split per query only");
    const int64_t U = (int64_t)a.T * (a.H / WH);
    const int64_t blocks = ((U + 7) / 8) * 8;
    hipLaunchKernelGGL(attn_w32_kernel, dim3((unsigned)blocks), dim3(64 * NWV), 0, st, (const bf16_t *)a.q,
                       (const bf16_t *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2, (const bf16_t *)a.swa, a.swa_pos0,
                       a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs, a.rope_dim, a.T, a.B, a.N, a.H,
                       (bf16_t *)a.out, a.lse, split_slots);
    return check_launch("attn_w32_kernel");
}

}  // namespace csa
