// Lightning Indexer scores on gfx950 ("DeepSeek-V4 混合注意力" §4.2):
//   s[t][i] = sum_h w[t][h] * ReLU(<q_I[t][h], k_I[i][h]>),  64 heads x 128 dims.
//
// Decode scan (bf16 / fp32 keys). Every visible entry's 64x128 key block is read
// once; with one query per sequence there is no reuse to feed a matrix core, so this
// is an HBM stream:
//  - one wavefront owns a run of consecutive entries of one query; per entry each lane
//    issues 16-byte non-temporal loads that together cover the block contiguously
//    (1 KiB per wave instruction), and the next entry's loads are in flight while the
//    current one is reduced;
//  - the query's 64x128 operand sits in VGPRs, in the same lane layout as the keys;
//  - per-lane partial dots of the lanes sharing a head are combined by a transposed
//    butterfly (each xor step halves the values a lane carries), after which every lane
//    holds one head's full dot: ReLU, times w, and one 64-lane sum give the score.
//  - entries that the query cannot see are written as -inf without being read.
// Shared keys (one key per entry for all heads) run on the matrix cores instead (below).
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

template <typename KT> struct ScanTraits {
    static constexpr int VEC = 16 / (int)sizeof(KT);  // elements per 16-byte load
    static constexpr int G = 128 / VEC;               // lanes that share one head
    static constexpr int J = 8192 / (64 * VEC);       // 16-byte loads per lane per entry
    static constexpr int HPL = 64 / G;                // heads covered by one wave load
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot16B(const u32x4 &a, const u32x4 &b, float acc, bf16_t) {
    // components are copied to scalars first: a bit_cast of a vector-element lvalue
    // reads element 0 whatever the component
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t x = a[c], y = b[c];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, x), __builtin_bit_cast(bf16x2v, y),
                                              acc, false);
    }
    return acc;
}

__device__ __forceinline__ float dot16B(const u32x4 &a, const u32x4 &b, float acc, float) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
    return acc;
}

template <typename KT>
__device__ __forceinline__ void load_entry(u32x4 (&buf)[ScanTraits<KT>::J], const u32x4 *p, int lane) {
#pragma unroll
    for (int j = 0; j < ScanTraits<KT>::J; ++j) buf[j] = __builtin_nontemporal_load(p + j * 64 + lane);
}

// ---- cross-lane exchange ------------------------------------------------------------
// DPP lane permutations inside a row of 16 lanes (no LDS traffic). Each is an
// involution; row_mirror pairs lanes differing in bit 3, half_mirror in bit 2 (with
// bit 3 equal), quad reverse in bit 1 (bits 3..2 equal), quad swap in bit 0.
enum : int { kRowMirror = 0x140, kRowHalfMirror = 0x141, kQuadRev = 0x1B, kQuadSwap = 0xB1 };

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// partner of a lane for the butterfly step whose role bit is ROLE (8, 4, 2, 1: DPP
// inside a row; 16, 32: across rows)
template <int ROLE>
__device__ __forceinline__ float partner(float x) {
    if constexpr (ROLE == 8) return dpp<kRowMirror>(x);
    else if constexpr (ROLE == 4) return dpp<kRowHalfMirror>(x);
    else if constexpr (ROLE == 2) return dpp<kQuadRev>(x);
    else if constexpr (ROLE == 1) return dpp<kQuadSwap>(x);
    else return __shfl_xor(x, ROLE);
}

// Transposed butterfly: v[0..2*LEN) of every lane in a group of lanes that differ in the
// role bits ROLE, ROLE/2, ..., 1. Each step keeps the half selected by the lane's role
// bit and adds the partner's copy of the same half, so after log2(2*LEN) steps lane L
// holds the group-sum of element j = (L's role bits read as a binary number).
template <int ROLE, int LEN, int J>
__device__ __forceinline__ void tbutterfly(float (&v)[J], int lane) {
    const bool up = (lane & ROLE) != 0;
#pragma unroll
    for (int x = 0; x < LEN; ++x) {
        const float keep = up ? v[x + LEN] : v[x];
        const float send = up ? v[x] : v[x + LEN];
        v[x] = keep + partner<ROLE>(send);
    }
    if constexpr (ROLE > 1) tbutterfly<ROLE / 2, LEN / 2, J>(v, lane);
}

// sum over all 64 lanes (every lane gets the total)
__device__ __forceinline__ float wave_sum(float r) {
    r += dpp<kRowMirror>(r);
    r += dpp<kRowHalfMirror>(r);
    r += dpp<kQuadRev>(r);
    r += dpp<kQuadSwap>(r);
    r += __shfl_xor(r, 16);
    r += __shfl_xor(r, 32);
    return r;
}

// full score of the entry held in `buf` (wave-uniform result)
template <typename KT>
__device__ __forceinline__ float entry_score(const u32x4 (&buf)[ScanTraits<KT>::J],
                                             const u32x4 (&qf)[ScanTraits<KT>::J], float wl, int lane) {
    using TR = ScanTraits<KT>;
    float v[TR::J];
#pragma unroll
    for (int j = 0; j < TR::J; ++j) v[j] = dot16B(qf[j], buf[j], 0.f, KT());
    // after it, lane L holds the complete dot of load slot j = L % G
    tbutterfly<TR::G / 2, TR::J / 2, TR::J>(v, lane);
    return wave_sum(fmaxf(v[0], 0.f) * wl);
}

// kCand: the wave's slots are positions of a per-query candidate list (cand [T][L], entry
// index or -1) instead of consecutive entries, and scores are written per slot
// ([T][L]); a slot whose entry is negative, past N or not visible scores -inf (its loads
// read entry 0, so every load stays unconditional).
template <typename KT, int EPW, bool kCand>
__global__ void __launch_bounds__(256)
index_scan_kernel(const KT *__restrict__ qI, const float *__restrict__ w, const KT *__restrict__ kI,
                  const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos, int B,
                  int64_t N, int ratio, const int32_t *__restrict__ cand, int64_t L, float *__restrict__ scores)
{
    using TR = ScanTraits<KT>;
    constexpr int EU = 8192 / TR::VEC;  // 16-byte units per entry
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.y;
    const int64_t e0 = ((int64_t)blockIdx.x * 4 + wv) * EPW;
    if (e0 >= L) return;
    const int64_t e1 = (e0 + EPW < L) ? e0 + EPW : L;

    const int s = q_seq[t];
    int64_t nvis = q_pos[t] / ratio;
    if (nvis > N) nvis = N;
    if (nvis < 0 || s < 0 || s >= B) nvis = 0;
    // consecutive entries: [e0, ev) are read, [ev, e1) masked; candidate slots: all read
    const int64_t ev = kCand ? (nvis > 0 ? e1 : e0) : ((e1 < nvis) ? e1 : nvis);
    int32_t my_id = -1;  // candidate slots: lane j holds the entry of slot e0 + j
    if (kCand && lane < (int)(e1 - e0)) my_id = cand[(int64_t)t * L + e0 + lane];
    const bool my_ok = !kCand || (my_id >= 0 && (int64_t)my_id < nvis);

    float my_score = -INFINITY;
    if (e0 < ev) {
        u32x4 qf[TR::J];
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(qI + (int64_t)t * 8192);
#pragma unroll
        for (int j = 0; j < TR::J; ++j) qf[j] = qp[j * 64 + lane];
        const float wl = w[(int64_t)t * 64 + (lane % TR::G) * TR::HPL + lane / TR::G];

        const u32x4 *kb = reinterpret_cast<const u32x4 *>(kI + ((int64_t)s * N) * 8192);
        // entry of slot e (wave-uniform)
        auto ent = [&](int64_t e) __attribute__((always_inline)) -> int64_t {
            if (!kCand) return e;
            const int id = __builtin_amdgcn_readlane(my_ok ? my_id : 0, (int)(e - e0));
            return (int64_t)id;
        };
        u32x4 bufA[TR::J], bufB[TR::J];
        load_entry<KT>(bufA, kb + ent(e0) * EU, lane);
        int64_t e = e0;
        // steady state: both loads of an iteration are unconditional, so the wait before
        // scoring A leaves B's loads in flight
        for (; e + 2 < ev; e += 2) {
            load_entry<KT>(bufB, kb + ent(e + 1) * EU, lane);
            float sc = entry_score<KT>(bufA, qf, wl, lane);
            if (lane == (int)(e - e0)) my_score = sc;
            load_entry<KT>(bufA, kb + ent(e + 2) * EU, lane);
            sc = entry_score<KT>(bufB, qf, wl, lane);
            if (lane == (int)(e + 1 - e0)) my_score = sc;
        }
        if (e + 1 < ev) {
            load_entry<KT>(bufB, kb + ent(e + 1) * EU, lane);
            float sc = entry_score<KT>(bufA, qf, wl, lane);
            if (lane == (int)(e - e0)) my_score = sc;
            sc = entry_score<KT>(bufB, qf, wl, lane);
            if (lane == (int)(e + 1 - e0)) my_score = sc;
        } else {
            const float sc = entry_score<KT>(bufA, qf, wl, lane);
            if (lane == (int)(e - e0)) my_score = sc;
        }
        if (!my_ok) my_score = -INFINITY;
    }
    if (lane < (int)(e1 - e0)) scores[(int64_t)t * L + e0 + lane] = my_score;
}

// ---- shared keys: one 128-dim key per entry for all 64 heads ----------------------------
// Per query the scores are a 64 x 128 by 128 x N contraction, so they run on the matrix
// cores: per 16-entry tile S^T = K Q^T (4 k-chunks x 4 head tiles of MFMA 16x16x32 bf16;
// A = 16-byte fragments of the 16 keys straight from memory, B = the query's q^T fragments
// in registers), then ReLU, times w, summed over the 4 head tiles in registers and over
// the 16 lanes of a row (the 16 heads of a tile) by DPP. A 16-entry tile is 4 KiB of
// contiguous keys, read by the wavefront's four 16-byte loads per lane.
constexpr int SH_TPW = 8;  // 16-entry tiles per wavefront

__device__ __forceinline__ float row_sum16(float r) {
    r += dpp<kRowMirror>(r);
    r += dpp<kRowHalfMirror>(r);
    r += dpp<kQuadRev>(r);
    r += dpp<kQuadSwap>(r);
    return r;
}

__global__ void __launch_bounds__(256)
index_shared_kernel(const bf16_t *__restrict__ qI, const float *__restrict__ w, const bf16_t *__restrict__ kI,
                    const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos, int B, int64_t N,
                    int ratio, float *__restrict__ scores)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int t = blockIdx.y;
    const int64_t e0 = ((int64_t)blockIdx.x * 4 + wv) * (16 * SH_TPW);
    if (e0 >= N) return;
    const int64_t e1 = (e0 + 16 * SH_TPW < N) ? e0 + 16 * SH_TPW : N;
    const int s = q_seq[t];
    int64_t nvis = q_pos[t] / ratio;
    if (nvis > N) nvis = N;
    if (nvis < 0 || s < 0 || s >= B) nvis = 0;
    const int64_t ev = (e1 < nvis) ? e1 : nvis;  // [e0, ev) are read, [ev, e1) masked

    if (e0 < ev) {
        // q^T fragments: head 16ht + l16, dims 32kk + 8g .. +7; w of the same heads
        bf16x8 qf[4][4];
        float wl[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            const bf16_t *qrow = qI + ((int64_t)t * 64 + 16 * ht + l16) * 128 + 8 * g;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qf[ht][kk] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * kk);
            wl[ht] = w[(int64_t)t * 64 + 16 * ht + l16];
        }
        const bf16_t *kb = kI + (int64_t)s * N * 128 + 8 * g;
        // lane l16 reads entry tb + l16 (the ragged tail re-reads the last visible entry;
        // those results are not written)
        auto load_tile = [&](int64_t tb, bf16x8 (&a)[4]) {
            const int64_t er = (tb + l16 < ev) ? tb + l16 : ev - 1;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) a[kk] = *reinterpret_cast<const bf16x8 *>(kb + er * 128 + 32 * kk);
        };
        bf16x8 cur[4], nxt[4];
        load_tile(e0, cur);
        for (int64_t tb = e0; tb < ev; tb += 16) {
            if (tb + 16 < ev) load_tile(tb + 16, nxt);
            f32x4 acc[4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int ht = 0; ht < 4; ++ht)
                    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur[kk], qf[ht][kk], acc[ht], 0, 0, 0);
            // acc[ht][r] = dot of head 16ht + l16 with entry tb + 4g + r
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = 0.f;
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) x = fmaf(wl[ht], fmaxf(acc[ht][r], 0.f), x);
                v[r] = row_sum16(x);
            }
            const int64_t e = tb + 4 * g + l16;
            if (l16 < 4 && e < ev) {
                const float o = l16 == 0 ? v[0] : (l16 == 1 ? v[1] : (l16 == 2 ? v[2] : v[3]));
                scores[(int64_t)t * N + e] = o;
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) cur[kk] = nxt[kk];
        }
    }
    for (int64_t e = (e0 > ev ? e0 : ev) + lane; e < e1; e += 64) scores[(int64_t)t * N + e] = -INFINITY;
}

}  // namespace

// Launches put queries on grid.y, which holds at most 65,535 rows: larger T goes out in
// slices of queries (pointer offsets into the per-query tensors).
constexpr int kMaxGridY = 65535;

int launch_index_scores(const void *qI, const uint8_t *qs, const float *w, const void *kI,
                        const uint8_t *ks, const int32_t *q_seq, const int64_t *q_pos, int T,
                        int B, int64_t N, int k_heads, int ratio, csa_dtype dt, float *scores, hipStream_t st)
{
    if (T == 0 || N == 0) return CSA_OK;
    if (dt == CSA_MXFP4)
        return launch_index_mxfp4((const uint8_t *)qI, qs, w, (const uint8_t *)kI, ks, q_seq, q_pos, T, B, N,
                                  ratio, scores, st);
    const size_t qbytes = (dt == CSA_F32 ? 4 : 2) * (size_t)64 * 128;  // one query's q_I
    for (int t0 = 0; t0 < T; t0 += kMaxGridY) {
        const int tn = (T - t0 < kMaxGridY) ? T - t0 : kMaxGridY;
        const void *q_t = (const char *)qI + (size_t)t0 * qbytes;
        const float *w_t = w + (int64_t)t0 * 64;
        float *s_t = scores + (int64_t)t0 * N;
        if (k_heads == 1) {  // shared keys (bf16; checked by the caller)
            dim3 grid((unsigned)((N + 4 * 16 * SH_TPW - 1) / (4 * 16 * SH_TPW)), (unsigned)tn);
            hipLaunchKernelGGL(index_shared_kernel, grid, dim3(256), 0, st, (const bf16_t *)q_t, w_t,
                               (const bf16_t *)kI, q_seq + t0, q_pos + t0, B, N, ratio, s_t);
            continue;
        }
        constexpr int EPW = 64;
        dim3 grid((unsigned)((N + 4 * EPW - 1) / (4 * EPW)), (unsigned)tn);
        if (dt == CSA_BF16) {
            hipLaunchKernelGGL((index_scan_kernel<bf16_t, EPW, false>), grid, dim3(256), 0, st, (const bf16_t *)q_t,
                               w_t, (const bf16_t *)kI, q_seq + t0, q_pos + t0, B, N, ratio, nullptr, N, s_t);
        } else {
            hipLaunchKernelGGL((index_scan_kernel<float, EPW, false>), grid, dim3(256), 0, st, (const float *)q_t,
                               w_t, (const float *)kI, q_seq + t0, q_pos + t0, B, N, ratio, nullptr, N, s_t);
        }
    }
    return check_launch(k_heads == 1 ? "index_shared_kernel" : "index_scan_kernel");
}

int launch_index_rescore(const void *qI, const float *w, const void *kI, const int32_t *cand, int M,
                         const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N, int ratio,
                         csa_dtype dt, float *scores, hipStream_t st)
{
    if (T == 0 || M == 0) return CSA_OK;
    constexpr int EPW = 64;
    const size_t qbytes = (dt == CSA_F32 ? 4 : 2) * (size_t)64 * 128;
    for (int t0 = 0; t0 < T; t0 += kMaxGridY) {
        const int tn = (T - t0 < kMaxGridY) ? T - t0 : kMaxGridY;
        const void *q_t = (const char *)qI + (size_t)t0 * qbytes;
        const float *w_t = w + (int64_t)t0 * 64;
        const int32_t *c_t = cand + (int64_t)t0 * M;
        float *s_t = scores + (int64_t)t0 * M;
        dim3 grid((unsigned)((M + 4 * EPW - 1) / (4 * EPW)), (unsigned)tn);
        if (dt == CSA_BF16) {
            hipLaunchKernelGGL((index_scan_kernel<bf16_t, EPW, true>), grid, dim3(256), 0, st, (const bf16_t *)q_t,
                               w_t, (const bf16_t *)kI, q_seq + t0, q_pos + t0, B, N, ratio, c_t, (int64_t)M, s_t);
        } else {
            hipLaunchKernelGGL((index_scan_kernel<float, EPW, true>), grid, dim3(256), 0, st, (const float *)q_t,
                               w_t, (const float *)kI, q_seq + t0, q_pos + t0, B, N, ratio, c_t, (int64_t)M, s_t);
        }
    }
    return check_launch("index_scan_kernel");
}

}  // namespace csa
