// Lightning Indexer scores with MXFP4 operands on gfx950 ("DeepSeek-V4 混合注意力" §2 and
// §4.2: the indexer QK runs in FP4; the MXFP4 checkpoint page: E2M1 values with one E8M0
// scale per 32 elements):
//   s[t][i] = sum_h w[t][h] * ReLU(<q_I[t][h], k_I[i][h]>)
//
// Prefill: many queries share one key store, so per head the products form a dense
// (queries x entries) contraction over 128 dims, done by v_mfma_scale_f32_16x16x128_f8f6f4
// (one instruction = one head's full dot for a 16 x 16 tile; E2M1 products are exact and
// the E8M0 block scales are applied inside the instruction).
//
// Workgroup: 4 wavefronts, a 128-query x 128-entry tile; wave (qg, eg) owns 64 queries x
// 64 entries (4 x 4 matrix-op tiles with the entries as the A operand and the queries as
// B, so a lane's 4 results of a tile belong to one query and need one head weight). The
// loop runs over the 64 heads: per head the tile's q and k codes (8 + 8 KiB) go from
// global memory straight into one of two LDS stages (direct-to-LDS buffer loads issued
// one head ahead), and per group of 4 heads the tile's E8M0 scale words and head weights
// (16-byte row slices) into one of two word buffers. The ReLU.w epilogue of each matrix
// op is VALU work (an integer max and an fma per product), which with the matrix ops and
// the LDS operand reads sets the kernel's time. Three workgroups share a compute unit
// (45 KB of LDS, under 128 registers each), so the SIMDs interleave their wavefronts.
//
// Decode (a few queries per key store): there is no reuse of keys across queries, so each
// query streams its keys from HBM (index_mxfp4_scan_kernel below) and the same matrix op
// computes 16 heads' dots of one entry on its diagonal.
#include "common.hpp"
#include "internal.hpp"
#include "topk_select.hpp"

namespace csa {

namespace {

constexpr int TQ = 128;  // queries per workgroup
constexpr int TE = 128;  // entries per workgroup
constexpr int NBUF = 2;  // LDS stages of one head's codes

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef int i32x4s __attribute__((ext_vector_type(4)));

// XOR swizzle of a code row's four 16-byte chunks in LDS: chunk c of row r sits in slot
// c ^ swz(r), so the 16-byte operand reads of 8 consecutive rows (the lanes a 16-byte read
// serves together) fall in distinct banks.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// raw buffer resource words over [p, p + bytes) (wave-uniform): loads past the end return
// zeros
__device__ __forceinline__ i32x4s tile_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const int lo = (int)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const int hi = (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    const int n = (int)__builtin_amdgcn_readfirstlane(bytes);
    return i32x4s{lo, hi, n, 0x00020000};
}

// LDS byte address of a pointer into __shared__ memory (wave-uniform)
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)(const char *)p);
}

// Direct-to-LDS load: lane i writes 16 bytes at LDS address dst + 16 i. Written as
// assembly so that the compiler does not track it: it would otherwise wait for every such
// load in flight before each LDS read it cannot prove disjoint from them, which drains the
// prefetch. Completion is waited for explicitly (vmcnt) before the barrier that publishes
// a stage. The instruction has no register result. It sets M0 (the LDS address register
// of the direct-to-LDS load; one wait state before the load reads it); nothing else in
// this file's kernels uses M0 (the compiler reserves it and warns about the clobber).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4s rs, uint32_t off, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(off), "s"(rs), "s"(dst)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// wait until every vector-memory operation and LDS access of this wavefront has completed
__device__ __forceinline__ void wait_vm_lds() { __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 0); }

// workgroup barrier without a memory fence (the fence would wait for every load in flight,
// the direct-to-LDS ones included); the wait before it says what has completed, and the
// empty asm keeps the compiler from moving memory accesses across it
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS: two stages of one head's codes; two buffers of a head group's scale words and
// weights (row-major, the 4 heads of a row in 16 bytes)
constexpr int ST_Q = 0, ST_K = TQ * 64, STAGE = ST_K + TE * 64;
constexpr int MT_QS = 0, MT_KS = TQ * 16, MT_W = MT_KS + TE * 16, META = MT_W + TQ * 16;

// The direct-to-LDS loads of one wavefront. Codes (per head; add h * 64): wave wv moves q
// rows and k rows wv*32 .. wv*32+31 of the tile, two 16-row groups each (1 KiB per
// instruction); lane i of a group fills LDS slot (row i/4, 16-byte slot i%4), which holds
// the row's chunk (i%4) ^ swz(row). Scale words and weights (per group of 4 heads; add
// g * 16): 16 bytes of a row per lane, one 64-row block per instruction: waves 0-1 move
// the q scale words and the weights of query rows 64wv.., waves 2-3 the k scale words of
// entry rows 64(wv-2)...
struct Fp4Loads {
    i32x4s qrs, krs, srs, wrs;
    uint32_t coff, moff, sdst, wdst;
    bool two;  // waves 0-1: scale words and weights
};

__device__ __forceinline__ void fp4_load_codes(const Fp4Loads &L, int h, int wv, uint32_t d) {
    const uint32_t o = L.coff + (uint32_t)(wv * 32) * 4096u + (uint32_t)h * 64u;
    dma16(L.qrs, o, d + ST_Q + wv * 32 * 64);
    dma16(L.qrs, o + 16u * 4096u, d + ST_Q + (wv * 32 + 16) * 64);
    dma16(L.krs, o, d + ST_K + wv * 32 * 64);
    dma16(L.krs, o + 16u * 4096u, d + ST_K + (wv * 32 + 16) * 64);
}

__device__ __forceinline__ void fp4_load_words(const Fp4Loads &L, int g, uint32_t d) {
    dma16(L.srs, L.moff + (uint32_t)g * 16u, d + L.sdst);
    if (L.two) dma16(L.wrs, L.moff + (uint32_t)g * 16u, d + L.wdst);
}

// Per-lane LDS byte offsets of one wavefront's reads. The swizzle of a row depends only
// on its row within a 16-row block (l16), so the 4 row blocks of a lane are 1 KiB apart
// in a code stage and 256 bytes apart in the word buffers (immediate offsets).
struct Fp4Lane {
    uint32_t kc, qc;  // codes: entry row eg*64 + l16 / query row qg*64 + l16, the lane's 16-byte chunk
    uint32_t ks, qs;  // scale byte g4 (block) of entry / query row, head 0
    uint32_t wq;      // weight of query row qg*64 + l16, head 0
};

// One head (hs of its group) for one wavefront: 16 matrix ops, each 16-query row block's
// 4 results followed by their ReLU.w epilogue into the lane's accumulators (entries
// 16n + 4g4 + r of query 16m + l16). `rs` / `ms`: LDS byte offsets of the head's code
// stage and of its group's word buffer.
__device__ __forceinline__ void fp4_head(const char *lds, uint32_t rs, uint32_t ms, int hs, const Fp4Lane &O,
                                         f32x4 (&acc)[4][4]) {
    const char *kc = lds + rs + O.kc, *qc = lds + rs + O.qc;
    const uint8_t *ks = reinterpret_cast<const uint8_t *>(lds + ms + MT_KS + O.ks + 4 * hs);
    const uint8_t *qs = reinterpret_cast<const uint8_t *>(lds + ms + MT_QS + O.qs + 4 * hs);
    const float *wq = reinterpret_cast<const float *>(lds + ms + MT_W + O.wq + 4 * hs);
    i32x8 Ae[4];
    int sa[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const i32x4v v = *reinterpret_cast<const i32x4v *>(kc + ST_K + 1024 * n);
        Ae[n] = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        sa[n] = ks[256 * n];  // the E8M0 byte of block g4 of the lane's row
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const i32x4v v = *reinterpret_cast<const i32x4v *>(qc + ST_Q + 1024 * m);
        const i32x8 Bq = i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        const int sb = qs[256 * m];
        const float w = wq[64 * m];
        f32x4 c[4];
#pragma unroll
        for (int n = 0; n < 4; ++n)
            c[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Ae[n], Bq, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                   sa[n], 0, sb);
        // ReLU is an integer max on the bits (negative floats are negative integers)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[m][n][r] = fmaf(w, __int_as_float(max(__float_as_int(c[n][r]), 0)), acc[m][n][r]);
    }
}

// Reads the keys of sequence 0 only: launch_index_mxfp4 dispatches here just when B == 1.
// second argument: wavefronts per SIMD the register allocation must allow
__global__ void __launch_bounds__(256, 3)
index_mxfp4_mfma_kernel(const uint8_t *__restrict__ qI, const uint8_t *__restrict__ qS,
                        const float *__restrict__ w, const uint8_t *__restrict__ kI,
                        const uint8_t *__restrict__ kS, const int32_t *__restrict__ q_seq,
                        const int64_t *__restrict__ q_pos, int T, int64_t N, int ratio, int nqb, int neb,
                        float *__restrict__ scores)
{
    __shared__ __attribute__((aligned(16))) char lds[NBUF * STAGE + 2 * META];
    __shared__ int32_t nvis_s[TQ];
    __shared__ int red[1];

    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    // XCD-aware order: the workgroups of one XCD (b, b+8, ...) run the query blocks
    // xcd, xcd+8, ... against a group of entry blocks at a time, so at any moment an XCD's
    // L2 holds a few query and entry tiles, each read by several of its workgroups
    const int b = blockIdx.x;
    const int xcd = b & 7, r8 = b >> 3;
    const int QX = (nqb + 7) >> 3;                 // query blocks per XCD
    const int EGN = QX >= 64 ? 1 : 64 / QX;        // entry blocks per group
    const int grp = r8 / (QX * EGN), within = r8 - grp * (QX * EGN);
    const int qb = (within % QX) * 8 + xcd, eb = grp * EGN + within / QX;
    if (qb >= nqb) return;
    const int t0 = qb * TQ;
    const int64_t i0 = (int64_t)eb * TE;

    // visibility of each query of the tile (a query of another sequence sees nothing);
    // N < 2^31 entries (checked by the caller), so counts fit 32 bits
    if (tid < TQ) {
        const int t = t0 + tid;
        int64_t nv = 0;
        if (t < T && q_seq[t] == 0) {
            nv = q_pos[t] / ratio;
            nv = nv < 0 ? 0 : (nv > N ? N : nv);
        }
        nvis_s[tid] = (int32_t)nv;
    }
    if (tid == 0) red[0] = 0;
    __syncthreads();
    if (tid < TQ && nvis_s[tid] > i0) atomicOr(&red[0], 1);
    __syncthreads();
    const bool any_visible = red[0] != 0;

    // wave (qg, eg) owns queries qg*64.. and entries eg*64.. of the tile
    const int qg = wv & 1, eg = wv >> 1;
    f32x4 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (any_visible) {
        // rows past T or N read zeros (their scores are not stored)
        const int rq = T - t0 < TQ ? T - t0 : TQ;
        const int re = N - i0 < TE ? (int)(N - i0) : TE;
        Fp4Loads L;
        L.qrs = tile_rsrc(qI + (int64_t)t0 * 4096, (uint32_t)rq * 4096u);
        L.krs = tile_rsrc(kI + i0 * 4096, (uint32_t)re * 4096u);
        L.two = wv < 2;
        L.srs = L.two ? tile_rsrc(qS + (int64_t)t0 * 256, (uint32_t)rq * 256u)
                      : tile_rsrc(kS + i0 * 256, (uint32_t)re * 256u);
        L.wrs = tile_rsrc(w + (int64_t)t0 * 64, (uint32_t)rq * 256u);
        const int crow = lane >> 2;  // row within a 16-row group (the swizzle depends only on it)
        L.coff = (uint32_t)crow * 4096u + (uint32_t)(((lane & 3) ^ swz(crow)) * 16);
        L.moff = (uint32_t)(64 * (wv & 1) + lane) * 256u;
        L.sdst = (L.two ? MT_QS : MT_KS) + (uint32_t)(wv & 1) * 1024u;
        L.wdst = MT_W + (uint32_t)(wv & 1) * 1024u;
        const uint32_t lbase = lds_addr(lds);
        Fp4Lane O;
        O.kc = (uint32_t)((eg * 64 + l16) * 64 + ((g4 ^ swz(l16)) * 16));
        O.qc = (uint32_t)((qg * 64 + l16) * 64 + ((g4 ^ swz(l16)) * 16));
        O.ks = (uint32_t)((eg * 64 + l16) * 16 + g4);
        O.qs = (uint32_t)((qg * 64 + l16) * 16 + g4);
        O.wq = (uint32_t)((qg * 64 + l16) * 16);

        // head group 0's words, then head 0's codes (a group's words always go out before
        // the codes of its first head, so waiting for those codes covers the words: loads
        // complete in issue order)
        fp4_load_words(L, 0, lbase + NBUF * STAGE);
        fp4_load_codes(L, 0, wv, lbase);
#pragma unroll 1
        for (int h = 0; h < 64; ++h) {
            // head h's loads have landed and every wavefront has finished head h-1, whose
            // stage (and at a group's start, the word buffer of the group before) the next
            // loads reuse
            wait_vm_lds();
            stage_barrier();
            const int g = h >> 2, hs = h & 3;
            if (hs == 0 && g + 1 < 16) fp4_load_words(L, g + 1, lbase + NBUF * STAGE + ((g + 1) & 1) * META);
            if (h + 1 < 64) fp4_load_codes(L, h + 1, wv, lbase + ((h + 1) & 1) * STAGE);
            __builtin_amdgcn_sched_barrier(0);
            fp4_head(lds, (uint32_t)(h & 1) * STAGE, NBUF * STAGE + (uint32_t)(g & 1) * META, hs, O, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // scores: lane holds entries 16n + 4g4 + r (r = 0..3, 16 contiguous bytes) of query
    // 16m + l16 of the wave tile (plain stores: non-temporal ones wrote each 128-byte line
    // as separate 64-byte pieces, 43 % more HBM writes)
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qq = qg * 64 + 16 * m + l16;
        const int t = t0 + qq;
        if (t >= T) continue;
        const int64_t nv = nvis_s[qq];
        float *srow = scores + (int64_t)t * N;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int64_t i = i0 + eg * 64 + 16 * n + 4 * g4;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (i + r < nv) ? acc[m][n][r] : -INFINITY;
            if (vec && i + 3 < N) {
                *reinterpret_cast<f32x4 *>(srow + i) = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (i + r < N) srow[i + r] = v[r];
            }
        }
    }
}

// ---- few queries per key store (decode): an HBM stream of each query's keys --------
// One wavefront per run of SE entries of one query. Per entry, the 64 heads' codes
// (4 KiB) arrive as four coalesced 1 KiB loads already in the A-operand layout of the FP4
// matrix op (row = head 16hb + l16, 16-byte k-chunk g4 of its 64 bytes); the query's codes
// for the same 16 heads are the B operand (column = head). The product's diagonal
// C[h][h] is then the 16 heads' dot products (exact E2M1 products, E8M0 block scales
// applied inside the instruction); lane (l16, g4) holds C[4g4 + r][l16], so the diagonal
// sits in the lanes with l16 / 4 == g4, component l16 % 4. The entry's 256 bytes of key
// scales come in as one 4-byte load per lane (head `lane`'s four blocks) and reach the
// lanes that need them by a permute. SP entries are in flight per wavefront; the code
// loads are non-temporal (each byte is read once).
constexpr int SE = 64;  // entries per wavefront
constexpr int SP = 4;   // entries loaded ahead

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)); // row_ror:4
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)); // row_ror:8
    // every lane now holds its row's sum; the four row sums come out of lanes 0, 16, 32, 48
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}

// The query side of one decode query (codes, scales and head weights of the 16 heads a
// lane's matrix-op column serves) and the score of one entry from its codes and scales.
struct Fp4Query {
    i32x8 qb[4];
    int sb[4];
    float wd[4];
};

__device__ __forceinline__ Fp4Query load_fp4_query(const uint8_t *qI, const uint8_t *qS, const float *w, int t) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    Fp4Query f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        const int64_t qh = (int64_t)t * 64 + 16 * hb + l16;
        const uint4 v = *reinterpret_cast<const uint4 *>(qI + qh * 64 + 16 * g4);
        f.qb[hb] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        f.sb[hb] = (int)qS[qh * 4 + g4];
        f.wd[hb] = w[qh];
    }
    return f;
}

// s = sum_h w_h ReLU(<q_h, k_h>) of one entry (kc: its codes in the A-operand layout, kw:
// head `lane`'s four block scales); the total is uniform over the wavefront
__device__ __forceinline__ float fp4_entry_score(const Fp4Query &f, const i32x4v (&kc)[4], uint32_t kw) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const bool diag = (l16 >> 2) == g4;
    const int r = lane & 3;
    float acc = 0.f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
        const int sa = (__builtin_amdgcn_ds_bpermute(4 * (16 * hb + l16), (int)kw) >> (8 * g4)) & 0xFF;
        const i32x8 A = i32x8{kc[hb].x, kc[hb].y, kc[hb].z, kc[hb].w, 0, 0, 0, 0};
        const f32x4 c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, f.qb[hb], f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4,
                                                                         0, sa, 0, f.sb[hb]);
        const float x = r == 0 ? c[0] : (r == 1 ? c[1] : (r == 2 ? c[2] : c[3]));
        acc = fmaf(f.wd[hb], __int_as_float(max(__float_as_int(x), 0)), acc);
    }
    return wave_sum_dpp(diag ? acc : 0.f);
}

// visible entries of query t: the first q_pos / ratio of its sequence (none for a query of
// no sequence)
__device__ __forceinline__ int64_t fp4_visible(int t, const int32_t *q_seq, const int64_t *q_pos, int B, int64_t N,
                                               int ratio, int &s) {
    s = q_seq[t];
    int64_t nv = (s >= 0 && s < B) ? q_pos[t] / ratio : 0;
    return nv < 0 ? 0 : (nv > N ? N : nv);
}

__global__ void __launch_bounds__(256)
index_mxfp4_scan_kernel(const uint8_t *__restrict__ qI, const uint8_t *__restrict__ qS,
                        const float *__restrict__ w, const uint8_t *__restrict__ kI,
                        const uint8_t *__restrict__ kS, const int32_t *__restrict__ q_seq,
                        const int64_t *__restrict__ q_pos, int T, int B, int64_t N, int ratio,
                        float *__restrict__ scores)
{
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const int64_t e0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * SE;
    if (e0 >= N) return;
    const int64_t e1 = e0 + SE < N ? e0 + SE : N;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        int s;
        const int64_t nv = fp4_visible(t, q_seq, q_pos, B, N, ratio, s);
        const int64_t ev = e1 < nv ? e1 : nv;  // visible entries of the run: [e0, ev)
        float out = -INFINITY;                 // lane j: the score of entry e0 + j
        if (ev > e0) {
            const Fp4Query f = load_fp4_query(qI, qS, w, t);
            const uint8_t *kb = kI + (int64_t)s * N * 4096 + l16 * 64 + 16 * g4;
            const uint32_t *ksb = reinterpret_cast<const uint32_t *>(kS + (int64_t)s * N * 256) + lane;
            i32x4v kc[SP][4];
            uint32_t kw[SP];
            // entries past the run re-read its last visible entry (cache hits), so every load
            // is unconditional and the waits stay exact
            auto load = [&](int u, int64_t e) __attribute__((always_inline)) {
                e = e < ev ? e : ev - 1;
#pragma unroll
                for (int hb = 0; hb < 4; ++hb)
                    kc[u][hb] = __builtin_nontemporal_load(reinterpret_cast<const i32x4v *>(kb + e * 4096 + hb * 1024));
                kw[u] = ksb[e * 64];
            };
#pragma unroll
            for (int u = 0; u < SP; ++u) load(u, e0 + u);
            for (int64_t eb = e0; eb < ev; eb += SP) {
#pragma unroll
                for (int u = 0; u < SP; ++u) {
                    const int64_t e = eb + u;
                    if (e < ev) {
                        const float tot = fp4_entry_score(f, kc[u], kw[u]);
                        out = (lane == (int)(e - e0)) ? tot : out;
                    }
                    load(u, eb + SP + u);
                }
            }
        }
        if (e0 + lane < e1) scores[(int64_t)t * N + e0 + lane] = out;
    }
}

// ---- the decode scan fused with the top-k ("DeepSeek-V4 混合注意力" §4.2: the FP4 index
// scores of every compressed entry, then the k best) -------------------------------------
// Workgroup (chunk, query): 8 wavefronts stream the 4,096 entries of the chunk (wavefront
// w, run j: entries c0 + 512 j + 64 w .. +63, the loads of the next run already in flight
// at the end of a run); each lane keeps its scores in registers as selection keys, so the
// chunk's exact top-k (select_chunk: ties to the lower position, ascending position
// order) comes straight out of the registers and only the k (value, index) winners reach
// memory. The exact top-k of a row is a subset of the union of its chunks' top-k sets, so
// the csa_topk selection over the winners (kept in position order, with their indices)
// finishes the job. At the Pro 1M decode shape (64 chunks x 1,024 winners per query) that
// selection runs in two short launches (8,192-winner chunks, then 8,192 survivors), which
// measured faster than one 1,024-lane workgroup over each query's 65,536 winners.
constexpr int FT_RT = 512;            // lanes per workgroup
constexpr int FT_J0 = 8;              // keys per lane
constexpr int FT_CH = FT_RT * FT_J0;  // entries per chunk
static_assert(64 % SP == 0, "a run of 64 entries is a whole number of load groups");

__global__ void __launch_bounds__(FT_RT)
index_mxfp4_topk_kernel(const uint8_t *__restrict__ qI, const uint8_t *__restrict__ qS,
                        const float *__restrict__ w, const uint8_t *__restrict__ kI,
                        const uint8_t *__restrict__ kS, const int32_t *__restrict__ q_seq,
                        const int64_t *__restrict__ q_pos, int T, int B, int64_t N, int ratio, int k,
                        float *__restrict__ win_v, int32_t *__restrict__ win_i, int64_t win_ld)
{
    __shared__ tksel::SelectLds<FT_RT, FT_J0> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int t = blockIdx.y;
    const int64_t chunk = blockIdx.x;
    const int64_t c0 = chunk * FT_CH;
    tksel::select_begin(sm);

    int s;
    const int64_t nv = fp4_visible(t, q_seq, q_pos, B, N, ratio, s);
    uint32_t key[FT_J0];
#pragma unroll
    for (int j = 0; j < FT_J0; ++j) key[j] = 0u;
    const int64_t wb = c0 + 64 * wv;  // first entry of the wavefront's run 0
    if (wb < nv) {
        const Fp4Query f = load_fp4_query(qI, qS, w, t);
        const uint8_t *kb = kI + (int64_t)s * N * 4096 + l16 * 64 + 16 * g4;
        const uint32_t *ksb = reinterpret_cast<const uint32_t *>(kS + (int64_t)s * N * 256) + lane;
        i32x4v kc[SP][4];
        uint32_t kw[SP];
        // step i of the wavefront (0 .. 64 FT_J0 - 1) is entry wb + 512 (i / 64) + i % 64;
        // steps past the visible entries re-read the last visible one (cache hits), so every
        // load is unconditional and the waits stay exact
        auto load = [&](int u, int i) __attribute__((always_inline)) {
            int64_t e = wb + (int64_t)FT_RT * (i >> 6) + (i & 63);
            e = e < nv ? e : nv - 1;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
                kc[u][hb] = __builtin_nontemporal_load(reinterpret_cast<const i32x4v *>(kb + e * 4096 + hb * 1024));
            kw[u] = ksb[e * 64];
        };
#pragma unroll
        for (int u = 0; u < SP; ++u) load(u, u);
#pragma unroll
        for (int j = 0; j < FT_J0; ++j) {
            const int64_t rb = wb + (int64_t)FT_RT * j;
            float out = -INFINITY;  // lane x: the score of entry rb + x
            for (int i0 = 0; i0 < 64; i0 += SP) {
#pragma unroll
                for (int u = 0; u < SP; ++u) {
                    if (rb + i0 + u < nv) {
                        const float tot = fp4_entry_score(f, kc[u], kw[u]);
                        out = (lane == i0 + u) ? tot : out;
                    }
                    load(u, 64 * j + i0 + u + SP);
                }
            }
            key[j] = tksel::order_key(out);
        }
    }
    const int n = (int)((N - c0 < FT_CH) ? (N > c0 ? N - c0 : 0) : FT_CH);
    const int64_t o = (int64_t)t * win_ld + chunk * k;
    tksel::select_chunk<FT_RT, FT_J0>(key, n, k, nullptr, c0, win_v ? win_v + o : nullptr, win_i + o, k, sm);
}

// chunks per query row of N entries (one empty chunk when N == 0, so the output is padded)
int64_t fused_chunks(int64_t N) { return N > 0 ? (N + FT_CH - 1) / FT_CH : 1; }

}  // namespace

// MXFP4 scores: the matrix-core tile kernel when many queries read the one key store
// (B == 1, prefill); otherwise (decode, several key stores) each query streams its keys.
int launch_index_mxfp4(const uint8_t *qI, const uint8_t *qs, const float *w, const uint8_t *kI,
                       const uint8_t *ks, const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                       int ratio, float *scores, hipStream_t st)
{
    if (B == 1 && T > 16) {
        const int nqb = (T + TQ - 1) / TQ;
        const int neb = (int)((N + TE - 1) / TE);
        const int64_t blocks = (int64_t)((nqb + 7) / 8) * 8 * neb;
        hipLaunchKernelGGL(index_mxfp4_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, st, qI, qs, w, kI, ks,
                           q_seq, q_pos, T, N, ratio, nqb, neb, scores);
        return check_launch("index_mxfp4_mfma_kernel");
    }
    const dim3 grid((unsigned)((N + 4 * SE - 1) / (4 * SE)), (unsigned)(T < 65535 ? T : 65535));
    hipLaunchKernelGGL(index_mxfp4_scan_kernel, grid, dim3(256), 0, st, qI, qs, w, kI, ks, q_seq, q_pos, T, B, N,
                       ratio, scores);
    return check_launch("index_mxfp4_scan_kernel");
}

size_t index_topk_workspace_bytes(int T, int64_t N, int k) {
    if (T <= 0 || k < 1) return 0;
    const int64_t nch = fused_chunks(N);
    if (nch == 1) return 0;  // the chunk's winners are the output
    const int64_t L = nch * k;
    const size_t pairs = (size_t)T * (size_t)L * 8u;
    return ((pairs + 255) / 256) * 256 + topk_workspace_bytes(T, L, k);
}

int launch_index_topk_mxfp4(const uint8_t *qI, const uint8_t *qs, const float *w, const uint8_t *kI,
                            const uint8_t *ks, const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                            int ratio, int k, int32_t *idx, float *vals, void *ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t nch = fused_chunks(N);
    const size_t need = index_topk_workspace_bytes(T, N, k);
    if (need > ws_bytes || (need > 0 && ws == nullptr))
        return fail(CSA_EWORKSPACE, "csa_index_topk: workspace smaller than csa_index_topk_workspace_bytes()");
    const dim3 grid((unsigned)nch, (unsigned)T);
    if (nch == 1) {
        // a single chunk: its winners are the answer (a NULL value output goes to a dropped,
        // zero-length buffer inside the selection)
        hipLaunchKernelGGL(index_mxfp4_topk_kernel, grid, dim3(FT_RT), 0, st, qI, qs, w, kI, ks, q_seq, q_pos, T, B, N,
                           ratio, k, vals, idx, (int64_t)k);
        return check_launch("index_mxfp4_topk_kernel");
    }
    const int64_t L = nch * k;
    float *wv = static_cast<float *>(ws);
    int32_t *wi = reinterpret_cast<int32_t *>(wv + (size_t)T * L);
    const size_t pair_bytes = (((size_t)T * (size_t)L * 8u + 255) / 256) * 256;
    hipLaunchKernelGGL(index_mxfp4_topk_kernel, grid, dim3(FT_RT), 0, st, qI, qs, w, kI, ks, q_seq, q_pos, T, B, N,
                       ratio, k, wv, wi, L);
    const int rc = check_launch("index_mxfp4_topk_kernel");
    if (rc != CSA_OK) return rc;
    return launch_topk(wv, wi, T, L, k, idx, vals, static_cast<char *>(ws) + pair_bytes, ws_bytes - pair_bytes, st);
}

}  // namespace csa
