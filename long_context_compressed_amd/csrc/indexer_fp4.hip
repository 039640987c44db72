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
// Workgroup: 8 wavefronts, a 256-query x 128-entry tile, wave (qg, eg) owns 64 queries x
// 64 entries (4 x 4 MFMA tiles, 64 fp32 score accumulators per lane). The loop runs over
// the 64 heads; per head the tile's q and k codes (16 + 8 KiB) are staged in LDS, double
// buffered: head h+2 is loaded into registers while head h is computed, and head h+1 is
// written to the other buffer. The E8M0 scales are staged 8 heads at a time (32 bytes of
// each row per load, not 4), since the scattered 4-byte loads of one head's scales cost
// more address-unit cycles than its codes. The epilogue of every MFMA (ReLU, times
// w[t][h], accumulate) is VALU work and bounds the kernel. The 16-byte chunks of each
// 64-byte code row are XOR-swizzled in LDS so the per-lane 16-byte operand reads of 8
// consecutive rows hit distinct banks. The head weights of the tile's queries sit in LDS
// head-major, so the 4 weights a lane needs per MFMA tile (4 consecutive queries) are one
// 16-byte read.
//
// Decode (a few queries per key store): there is no reuse of keys across queries, so each
// query streams its keys from HBM (index_mxfp4_scan_kernel below) and the same matrix op
// computes 16 heads' dots of one entry on its diagonal.
#include "common.hpp"
#include "internal.hpp"
#include "topk_select.hpp"

namespace csa {

namespace {

constexpr int TQ = 128;       // queries per workgroup
constexpr int TE = 128;       // entries per workgroup

typedef int i32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// Two workgroups of 4 wavefronts share a compute unit (77 KB of LDS each): each keeps its
// own barriers, so while one runs a head's matrix ops the other can run its ReLU.w
// epilogue on the same SIMDs (within one wavefront the two do not overlap).
__global__ void __launch_bounds__(256, 2)
index_mxfp4_mfma_kernel(const uint8_t *__restrict__ qI, const uint8_t *__restrict__ qS,
                        const float *__restrict__ w, const uint8_t *__restrict__ kI,
                        const uint8_t *__restrict__ kS, const int32_t *__restrict__ q_seq,
                        const int64_t *__restrict__ q_pos, int T, int64_t N, int ratio, int nqb, int neb,
                        float *__restrict__ scores)
{
    __shared__ __attribute__((aligned(16))) uint8_t Qs[2][TQ * 64];
    __shared__ __attribute__((aligned(16))) uint8_t Ks[2][TE * 64];
    // scale words of 4 heads at a time, head-major ([head % 4][row]), double buffered
    __shared__ __attribute__((aligned(16))) uint32_t QSs[2][4][TQ];
    __shared__ __attribute__((aligned(16))) uint32_t KSs[2][4][TE];
    __shared__ __attribute__((aligned(16))) float Ws[64 * TQ];  // head-major: [head][query]
    __shared__ int32_t nvis_s[TQ];
    __shared__ int red[2];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    // XCD-aware order: workgroups b, b+8, ... share an XCD; one query block per XCD at a
    // time (its q tile stays in that XCD's L2) while the entry blocks stream
    const int b = blockIdx.x;
    const int xcd = b & 7, r8 = b >> 3;
    const int qb = (r8 / neb) * 8 + xcd, eb = r8 % neb;
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
        // head weights of the tile's queries
#pragma unroll 4
        for (int x = tid; x < TQ * 64; x += 256) {
            const int qq = x % TQ, h = x / TQ;
            const int t = t0 + qq;
            Ws[h * TQ + qq] = (t < T) ? w[(int64_t)t * 64 + h] : 0.f;
        }
        // per-wave share of one head's codes: 32 q rows and 32 k rows (16 bytes per lane per
        // 16-row group), loaded into registers while the previous head is computed, then
        // written to LDS
        const int qrow0 = wv * 32 + (lane >> 2), qrow1 = qrow0 + 16;
        const int krow0 = qrow0, krow1 = qrow1;
        const int qpos0 = ((lane & 3) ^ swz(qrow0)) * 16, qpos1 = ((lane & 3) ^ swz(qrow1)) * 16;
        const int kpos0 = qpos0, kpos1 = qpos1;
        int tq0 = t0 + qrow0, tq1 = t0 + qrow1;
        tq0 = tq0 < T ? tq0 : T - 1;
        tq1 = tq1 < T ? tq1 : T - 1;
        int64_t ek0 = i0 + krow0, ek1 = i0 + krow1;
        ek0 = ek0 < N ? ek0 : N - 1;
        ek1 = ek1 < N ? ek1 : N - 1;
        const uint8_t *qsrc0 = qI + (int64_t)tq0 * 4096 + (lane & 3) * 16;
        const uint8_t *qsrc1 = qI + (int64_t)tq1 * 4096 + (lane & 3) * 16;
        const uint8_t *ksrc0 = kI + ek0 * 4096 + (lane & 3) * 16;
        const uint8_t *ksrc1 = kI + ek1 * 4096 + (lane & 3) * 16;
        // scales, 4 heads (16 bytes of a row) at a time: threads 0..127 load q row tid,
        // threads 128..255 k row tid - 128; a block's scales are loaded at its predecessor's
        // first head and stored at its last
        const bool sq = tid < TQ;
        const int srow = sq ? tid : tid - TQ;
        int tsq = t0 + srow;
        tsq = tsq < T ? tsq : T - 1;
        int64_t esk = i0 + srow;
        esk = esk < N ? esk : N - 1;
        const uint8_t *ssrc = sq ? qS + (int64_t)tsq * 256 : kS + esk * 256;
        uint4 rs;
#define FP4_SLOAD(BLK)                                                                   \
    {                                                                                   \
        rs = *reinterpret_cast<const uint4 *>(ssrc + (BLK) * 16);                        \
    }
#define FP4_SSTORE(SB)                                                                   \
    {                                                                                   \
        uint32_t(*dst)[TQ] = sq ? QSs[SB] : KSs[SB];                                    \
        dst[0][srow] = rs.x;                                                            \
        dst[1][srow] = rs.y;                                                            \
        dst[2][srow] = rs.z;                                                            \
        dst[3][srow] = rs.w;                                                            \
    }
        // two register sets (A: even heads, B: odd heads): head h+2 is loaded while head h
        // is computed, and head h+1 (loaded one head earlier) is written to LDS after it
        uint4 rq0A, rq1A, rk0A, rk1A, rq0B, rq1B, rk0B, rk1B;
#define FP4_LOAD(S, HH)                                                                  \
    {                                                                                   \
        rq0##S = *reinterpret_cast<const uint4 *>(qsrc0 + (HH) * 64);                   \
        rq1##S = *reinterpret_cast<const uint4 *>(qsrc1 + (HH) * 64);                   \
        rk0##S = *reinterpret_cast<const uint4 *>(ksrc0 + (HH) * 64);                   \
        rk1##S = *reinterpret_cast<const uint4 *>(ksrc1 + (HH) * 64);                   \
    }
#define FP4_STORE(S, BUF)                                                                \
    {                                                                                   \
        *reinterpret_cast<uint4 *>(&Qs[BUF][qrow0 * 64 + qpos0]) = rq0##S;              \
        *reinterpret_cast<uint4 *>(&Qs[BUF][qrow1 * 64 + qpos1]) = rq1##S;              \
        *reinterpret_cast<uint4 *>(&Ks[BUF][krow0 * 64 + kpos0]) = rk0##S;              \
        *reinterpret_cast<uint4 *>(&Ks[BUF][krow1 * 64 + kpos1]) = rk1##S;              \
    }

        // one head's contraction over LDS buffer BUF: the k codes of the wave's 4 entry tiles
        // stay in registers, the q codes are read per query tile
#define FP4_COMPUTE(HH, BUF, HS)                                                         \
    {                                                                                   \
        i32x4v Bv[4];                                                                   \
        int sb[4];                                                                      \
        _Pragma("unroll") for (int n = 0; n < 4; ++n) {                                 \
            const int row = eg * 64 + 16 * n + l16;                                     \
            Bv[n] = *reinterpret_cast<const i32x4v *>(&Ks[BUF][row * 64 + ((g4 ^ swz(row)) * 16)]); \
            sb[n] = (int)((KSs[sbuf][HS][row] >> (8 * g4)) & 0xFFu);                    \
        }                                                                               \
        _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                 \
            const int row = qg * 64 + 16 * m + l16;                                     \
            const i32x4v av = *reinterpret_cast<const i32x4v *>(&Qs[BUF][row * 64 + ((g4 ^ swz(row)) * 16)]); \
            const i32x8 A = i32x8{av[0], av[1], av[2], av[3], 0, 0, 0, 0};              \
            const int sa = (int)((QSs[sbuf][HS][row] >> (8 * g4)) & 0xFFu);             \
            const float4 w4 = *reinterpret_cast<const float4 *>(&Ws[(HH) * TQ + qg * 64 + 16 * m + 4 * g4]); \
            const float wr[4] = {w4.x, w4.y, w4.z, w4.w};                               \
            _Pragma("unroll") for (int n = 0; n < 4; ++n) {                             \
                const i32x8 Bn = i32x8{Bv[n][0], Bv[n][1], Bv[n][2], Bv[n][3], 0, 0, 0, 0}; \
                const f32x4 c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(       \
                    A, Bn, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, sa, 0, sb[n]);           \
                _Pragma("unroll") for (int r = 0; r < 4; ++r)                           \
                    acc[m][n][r] = fmaf(wr[r], __int_as_float(max(__float_as_int(c[r]), 0)), acc[m][n][r]); \
            }                                                                           \
        }                                                                               \
    }

        // ReLU is an integer max on the bits (negative floats are negative integers): one
        // instruction, where fmaxf also quiets NaNs. Loads past the last head or block re-read
        // the last one and their stores go to a buffer nobody reads again, so every load and
        // store is unconditional and the waits stay exact.
        FP4_SLOAD(0)
        FP4_LOAD(A, 0)
        FP4_LOAD(B, 1)
        FP4_SSTORE(0)
        FP4_STORE(A, 0)
        __syncthreads();
#pragma unroll 1
        for (int hb = 0; hb < 64; hb += 4) {
            const int sbuf = (hb >> 2) & 1;
            FP4_SLOAD(hb + 4 < 64 ? (hb >> 2) + 1 : 15)
#pragma unroll 1
            for (int hs = 0; hs < 4; hs += 2) {
                const int h = hb + hs;
                FP4_LOAD(A, h + 2 < 64 ? h + 2 : 63)
                FP4_COMPUTE(h, 0, hs)
                FP4_STORE(B, 1)
                __syncthreads();
                FP4_LOAD(B, h + 3 < 64 ? h + 3 : 63)
                FP4_COMPUTE(h + 1, 1, hs + 1)
                if (hs == 2) FP4_SSTORE(sbuf ^ 1)
                FP4_STORE(A, 0)
                __syncthreads();
            }
        }
#undef FP4_LOAD
#undef FP4_STORE
#undef FP4_SLOAD
#undef FP4_SSTORE
#undef FP4_COMPUTE
    }

    // scores: lane holds (query 16m + 4g4 + r, entry 16n + l16) of the wave tile
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int qq = qg * 64 + 16 * m + 4 * g4 + r;
            const int t = t0 + qq;
            if (t >= T) continue;
            const int64_t nv = nvis_s[qq];
            float *srow = scores + (int64_t)t * N;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int64_t i = i0 + eg * 64 + 16 * n + l16;
                if (i < N) srow[i] = (i < nv) ? acc[m][n][r] : -INFINITY;
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
