// bf16 matrix-core GEMMs on gfx950 for the projections around the attention path:
//   - the compressor fed from hidden states: C^a, Z^a, C^b, Z^b = H W^T ("DeepSeek-V4
//     混合注意力" §4.1: the compressor produces two sets of contents and weight logits
//     from H; §7: Compressor.forward starts with project_a / project_b of the hidden
//     state), with the per-channel softmax pooling of §4.1 / §5 fused into the epilogue,
//     so the n x 4c projected rows never reach memory;
//   - the grouped output projection after the attention (§4.2: the outputs are
//     aggregated per group and projected back to the model width; §7:
//     grouped_output_projection(inverse_rope(output))).
//
// One GEMM core serves both: C[m][n] = sum_k A[m][k] B[n][k] (both operands K-contiguous,
// as activations [rows][K] and weights [out][in] are stored), fp32 accumulation on
// v_mfma_f32_32x32x16_bf16.
//   - workgroup tile 64 MI (M) x 64 WN (N), 2 x WN wavefronts of 32 MI x 64 (MI x 2 blocks
//     of 32 x 32): MI = 4, WN = 4 (256 x 256, 8 wavefronts) for the plain GEMM, MI = 2,
//     WN = 2 (128 x 128) for the compressor (its epilogue tile has to fit LDS);
//   - the K loop runs over 64-wide slices in 2 LDS stages (32-wide slices in 4 stages when
//     K is an odd multiple of 32); slices go from memory straight into LDS by buffer loads
//     with the LDS destination (16 bytes per lane), all but one stage ahead of the slice
//     being multiplied, one barrier per slice;
//   - a slice row is 128 (64) bytes = eight (four) 16-byte chunks; chunk c of tile row r sits
//     in LDS slot c ^ ((r / 2) % 8) (c ^ ((r / 4) % 4)) (the lanes of a load fetch the
//     permuted chunks, so the LDS side stays one contiguous 1 KiB write per instruction),
//     which spreads the 16 rows that a 16-byte fragment read serves together over all banks;
//   - rows past the operand's end, and the 4 rows before a sequence's first token when no
//     carry is given, read as zeros (buffer loads past the resource end return 0).
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4g __attribute__((ext_vector_type(4)));

constexpr int kBufWord3 = 0x00020000;                // raw buffer, 32-bit data format
constexpr uint32_t kOob = 0xFFFFFFF0u;               // an offset past any resource: no access

// Tile shapes: MI 32-row blocks per wavefront in M, WN wavefronts in N (the workgroup's
// 2 x WN wavefronts cover 64 MI rows x 64 WN columns), NST LDS stages in the K ring, K
// slices of BK (32 or 64).
template <int MI, int NST_, int WN = 2, int BK_ = 32>
struct Tile {
    static constexpr int BK = BK_;
    static constexpr int NST = NST_;
    static constexpr int ROW = BK * 2;     // bytes of one slice row
    static constexpr int CPR = BK / 8;     // 16-byte chunks per slice row
    static constexpr int RPL = 64 / CPR;   // rows per load instruction (1 KiB)
    static constexpr int BM = 64 * MI;
    static constexpr int BN = 64 * WN;
    static constexpr int NW = 2 * WN;   // wavefronts
    static constexpr int A_BYTES = BM * ROW;
    static constexpr int B_BYTES = BN * ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = NST_ * STAGE;
    static constexpr int AQ = BM / (RPL * NW);  // A load instructions per wavefront and slice
    static constexpr int BQ = BN / (RPL * NW);  // B load instructions per wavefront and slice
    static_assert(BK == 32 || BK == 64, "slices of 32 or 64");
    static_assert(AQ * RPL * NW == BM && BQ * RPL * NW == BN, "the rows split evenly over the wavefronts");
    // LDS byte offset of (tile row r, 16-byte chunk c) within one operand tile: chunk c sits
    // in slot c ^ swz(r), so the 16 rows that one 16-byte read serves together fall in
    // distinct banks (64-byte rows: (r / 4) % 4; 128-byte rows: (r / 2) % 8)
    __device__ static __forceinline__ int swz(int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
    __device__ static __forceinline__ int slot_off(int r, int c) { return r * ROW + ((c ^ swz(r)) << 4); }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint64_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, (int)n, kBufWord3);
}

__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off, void *lds_row) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds_row, 16, off, 0, 0,
                                             0);
}

// vmcnt wait (loads complete in issue order: every load issued before the last n landed)
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}


// Row sources of one operand tile. A lane's load covers tile row r; `off(r, c)` gives the
// byte offset of 16-byte chunk c of that row's current K slice in `main` (kOob when the row
// is not there), and for operands with a second source (the compressor's carry rows)
// `off2` the same in `second`.
struct Operand {
    __amdgpu_buffer_rsrc_t main;
    __amdgpu_buffer_rsrc_t second;
    bool has_second;
};

// The GEMM core: accumulates the BM x BN tile for K slices [0, K) into acc (per wave a
// 32 MI x 64 block as MI x 2 32x32 MFMA accumulators). rowA(r) / rowB(r) return the byte
// offset of K element 0 of tile row r in the main resource (or kOob), rowA2(r) in the
// second A resource (or kOob). K % 32 == 0.
template <int MI, int NST, int WN, int BK, bool kSecondA, class RA, class RA2, class RB>
__device__ __forceinline__ void gemm_core(char *lds, const Operand &opA, const Operand &opB, int64_t K, RA rowA,
                                          RA2 rowA2, RB rowB, f32x16 (&acc)[MI][2]) {
    using TL = Tile<MI, NST, WN, BK>;
    constexpr int AQ = TL::AQ, BQ = TL::BQ, CPR = TL::CPR, RPL = TL::RPL, ROW = TL::ROW;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WN, wn = w % WN;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // per load instruction: RPL rows x CPR chunks; lane l: row RPL q' + l / CPR, LDS slot
    // l % CPR, which holds chunk (l % CPR) ^ swz(row) of the row. Each wavefront loads AQ
    // instructions' worth of A rows and BQ of B rows per slice.
    uint32_t offA[AQ], offA2[AQ], offB[BQ];
    bool useA2[AQ];
    const int slot = lane % CPR;
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int r = RPL * (AQ * w + q) + lane / CPR;
        const int chunk = slot ^ TL::swz(r);
        const uint32_t a = rowA(r);
        offA[q] = a == kOob ? kOob : a + 16u * chunk;
        useA2[q] = false;
        if constexpr (kSecondA) {
            const uint32_t a2 = rowA2(r);
            offA2[q] = a2 == kOob ? kOob : a2 + 16u * chunk;
            useA2[q] = a2 != kOob;
        }
    }
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
        const int r = RPL * (BQ * w + q) + lane / CPR;
        const uint32_t b = rowB(r);
        offB[q] = b == kOob ? kOob : b + 16u * (slot ^ TL::swz(r));
    }
    const int64_t nk = K / BK;
    auto issue = [&](int64_t ks) __attribute__((always_inline)) {
        char *st = lds + (int)(ks % NST) * TL::STAGE;
        const uint32_t kb = ks < nk ? (uint32_t)(ks * ROW) : kOob;  // past the end: no access
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            char *dst = st + RPL * (AQ * w + q) * ROW;  // the instruction's 1 KiB destination
            // every lane writes its LDS slot exactly once (a load past a resource's end
            // writes zeros), so a lane whose row comes from the second source takes only
            // that load: the two loads run under complementary lane masks
            if (kSecondA && useA2[q])
                lds_load16(opA.second, kb == kOob ? kOob : offA2[q] + kb, dst);
            else
                lds_load16(opA.main, (offA[q] == kOob || kb == kOob) ? kOob : offA[q] + kb, dst);
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q)
            lds_load16(opB.main, (offB[q] == kOob || kb == kOob) ? kOob : offB[q] + kb,
                       st + TL::A_BYTES + RPL * (BQ * w + q) * ROW);
    };
    // loads per slice and wave that always issue (with two A sources one lane mask may be
    // empty and its load skipped: counting the minimum keeps the waits exact-or-stricter)
    constexpr int kLoadsPerSlice = AQ + BQ;
#pragma unroll
    for (int s = 0; s < NST - 1; ++s) issue(s);

    // fragment reads: lane l reads tile row (l % 32) of its 32-row block, chunk
    // 2 * ksub + l / 32 (8 K values)
    const int fr = lane & 31, fc = lane >> 5;
    for (int64_t ks = 0; ks < nk; ++ks) {
        wait_vm<kLoadsPerSlice * (NST - 2)>();
        lds_barrier();
        issue(ks + NST - 1);
        const char *st = lds + (int)(ks % NST) * TL::STAGE;
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            bf16x8 af[MI], bfr[2];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int ra = 32 * MI * wm + 32 * i + fr;
                af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4g *>(st + TL::slot_off(ra, 2 * sub + fc)));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int rb = 64 * wn + 32 * j + fr;
                bfr[j] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4g *>(st + TL::A_BYTES + TL::slot_off(rb, 2 * sub + fc)));
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    wait_vm<0>();
    lds_barrier();  // every wave is done with the ring; the epilogue may reuse it
}

// accumulator element v of a 32 x 32 block: row 8 (v / 4) + 4 (lane / 32) + v % 4,
// column lane % 32
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ---------------------------------------------------------------------------------------
// plain batched GEMM: C[z][m][n] = sum_k A[z][m][k] B[z][n][k]; C bf16 or fp32
// ---------------------------------------------------------------------------------------
template <typename OT, int MI, int NST, int WN, int BK>
__global__ void __launch_bounds__(128 * WN)
gemm_bf16_kernel(const bf16_t *__restrict__ A, int64_t lda, int64_t sA, const bf16_t *__restrict__ Bw,
                 int64_t ldb, int64_t sB, OT *__restrict__ C, int64_t ldc, int64_t sC, int64_t M, int64_t N,
                 int64_t K, int mtiles)
{
    using TL = Tile<MI, NST, WN, BK>;
    __shared__ __attribute__((aligned(16))) char lds[TL::LDS];
    const int z = blockIdx.z;
    constexpr int BM = TL::BM, BN = TL::BN;
    const int64_t m0 = (int64_t)(blockIdx.x % mtiles) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x / mtiles) * BN;
    const bf16_t *Ab = A + (int64_t)z * sA + m0 * lda;
    const bf16_t *Bb = Bw + (int64_t)z * sB + n0 * ldb;
    const int64_t mr = M - m0 < BM ? M - m0 : BM, nr = N - n0 < BN ? N - n0 : BN;
    Operand oa, ob;
    oa.main = oa.second = make_rsrc(Ab, (uint64_t)((mr - 1) * lda + K) * 2);
    ob.main = ob.second = make_rsrc(Bb, (uint64_t)((nr - 1) * ldb + K) * 2);
    oa.has_second = ob.has_second = false;
    f32x16 acc[MI][2];
    gemm_core<MI, NST, WN, BK, false>(
        lds, oa, ob, K, [&](int r) { return r < mr ? (uint32_t)(r * lda * 2) : kOob; },
        [&](int) { return kOob; }, [&](int r) { return r < nr ? (uint32_t)(r * ldb * 2) : kOob; }, acc);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WN, wn = w % WN;
    OT *Cb = C + (int64_t)z * sC;
    const int64_t r0 = m0 + 32 * MI * wm + 4 * (lane >> 5), c0 = n0 + 64 * wn + (lane & 31);
    if (m0 + BM <= M && n0 + BN <= N) {
        // whole tile: no bounds tests
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                OT *cp = Cb + (r0 + 32 * i) * ldc + c0 + 32 * j;
#pragma unroll
                for (int v = 0; v < 16; ++v) elem<OT>::store(cp, (8 * (v >> 2) + (v & 3)) * ldc, acc[i][j][v]);
            }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t col = c0 + 32 * j;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = r0 + 32 * i + 8 * (v >> 2) + (v & 3);
                    if (row < M && col < N) elem<OT>::store(Cb, row * ldc + col, acc[i][j][v]);
                }
                // one accumulator block at a time (the scheduler would otherwise convert
                // every block ahead of its stores and run out of registers)
                __builtin_amdgcn_sched_barrier(0);
            }
    }
}

// ---------------------------------------------------------------------------------------
// compressor from hidden states: projection + per-channel softmax pooling
// ---------------------------------------------------------------------------------------
// ratio 4 (overlapped): tile rows 0..127 are tokens t0 - 4 .. t0 + 123 with t0 = 124 * mt,
// so the tile holds 31 whole entries (entry e: b-rows 4e..4e+3, a-rows 4e+4..4e+7); the
// tile's columns are CW = 64 channels x the 4 projections (C^a, Z^a, C^b, Z^b), column
// CW p + x = channel CW nt + x of projection p. Tokens before 0 come from the carry rows
// (the last 4 hidden rows of the previous chunk) or are absent (weight 0).
// ratio 128: tile rows are the 128 tokens of entry mt; columns 128 channels x (C, Z).
// K slices of 64 in 2 stages when d % 64 == 0, else of 32 in 4 stages (a 96 KiB ring); the
// fp32 epilogue tile takes 128 KiB: one workgroup of 8 wavefronts per CU
constexpr int kCompressWN = 4;  // wavefronts in N: 128 x 256 tiles of 8 wavefronts
template <int BK>
using CompressTile = Tile<2, BK == 64 ? 2 : 4, kCompressWN, BK>;
// the ring, and after the products the fp32 epilogue tile
template <int BK>
constexpr int compress_lds() {
    using TL = CompressTile<BK>;
    return TL::LDS > TL::BM * TL::BN * 4 ? TL::LDS : TL::BM * TL::BN * 4;
}

template <int RATIO, typename OT, int BK>
__global__ void __launch_bounds__(128 * kCompressWN)
compress_hidden_kernel(const bf16_t *__restrict__ Hs, const bf16_t *__restrict__ carry, const bf16_t *__restrict__ W,
                       const float *__restrict__ bias, int64_t n, int64_t d, int c, OT *__restrict__ out,
                       int64_t out_bstride, int mtiles, int ntiles)
{
    using TL = CompressTile<BK>;
    __shared__ __attribute__((aligned(16))) char lds[compress_lds<BK>()];
    constexpr bool kOv = RATIO == 4;
    constexpr int NP = kOv ? 4 : 2;          // projections
    constexpr int BN = TL::BN;
    constexpr int CW = BN / NP;              // channels per tile
    constexpr int TS = kOv ? 124 : 128;      // tokens per tile step
    constexpr int LEAD = kOv ? 4 : 0;        // rows before the tile's first whole entry
    constexpr int NE = kOv ? 31 : 1;         // entries per tile
    const int b = blockIdx.z;
    const int mt = blockIdx.x % mtiles, nt = blockIdx.x / mtiles;
    (void)ntiles;
    const int64_t t0 = (int64_t)mt * TS;
    const bf16_t *Hb = Hs + (int64_t)b * n * d;
    Operand oa, ob;
    oa.main = oa.second = make_rsrc(Hb, (uint64_t)n * d * 2);
    oa.has_second = kOv && carry != nullptr;
    if (oa.has_second) oa.second = make_rsrc(carry + (int64_t)b * 4 * d, (uint64_t)4 * d * 2);
    ob.main = ob.second = make_rsrc(W, (uint64_t)NP * c * d * 2);
    ob.has_second = false;
    auto rowA = [&](int r) -> uint32_t {
        const int64_t tok = t0 - LEAD + r;
        return (tok >= 0 && tok < n) ? (uint32_t)(tok * d * 2) : kOob;
    };
    auto rowA2 = [&](int r) -> uint32_t {
        const int64_t tok = t0 - LEAD + r;
        return (tok < 0 && carry != nullptr) ? (uint32_t)((tok + 4) * d * 2) : kOob;
    };
    auto rowB = [&](int r) -> uint32_t {
        const int p = r / CW, ch = nt * CW + r % CW;
        return ch < c ? (uint32_t)(((int64_t)p * c + ch) * d * 2) : kOob;
    };
    f32x16 acc[2][2];
    if (kOv && carry != nullptr)
        gemm_core<2, TL::NST, kCompressWN, BK, true>(lds, oa, ob, d, rowA, rowA2, rowB, acc);
    else
        gemm_core<2, TL::NST, kCompressWN, BK, false>(lds, oa, ob, d, rowA, rowA2, rowB, acc);

    // the fp32 tile into LDS: [128 rows][256 columns]
    constexpr int TP = BN;
    float *tile = reinterpret_cast<float *>(lds);
    {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const int wm = w / kCompressWN, wn = w % kCompressWN;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = 64 * wn + 32 * j + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) tile[(64 * wm + 32 * i + acc_row(v, lane)) * TP + col] = acc[i][j][v];
            }
    }
    __syncthreads();

    const int tid = threadIdx.x;
    const int64_t E = n / RATIO;  // whole entries of the chunk
    if constexpr (kOv) {
        // 31 entries x 32 channels, four pairs per thread
        const int x = tid % CW;
        const int ch = nt * CW + x;
        for (int e = tid / CW; e < NE; e += 128 * kCompressWN / CW) {
            const int64_t ei = (int64_t)mt * NE + e;
            if (ei >= E || ch >= c) continue;
            float z[8], v[8];
            bool has[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int r = 4 * e + s;  // b-rows 4e..4e+3, a-rows 4e+4..4e+7
                const bool isb = s < 4;
                const int64_t tok = t0 - LEAD + r;
                has[s] = !(isb && tok < 0 && carry == nullptr);
                z[s] = tile[r * TP + (isb ? 3 : 1) * CW + x];
                v[s] = tile[r * TP + (isb ? 2 : 0) * CW + x];
                if (bias != nullptr) z[s] += bias[(int64_t)s * c + ch];
            }
            float m = -INFINITY;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (has[s]) m = fmaxf(m, z[s]);
            float den = 0.f, num = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                if (has[s]) {
                    const float p = __expf(z[s] - m);
                    den += p;
                    num = fmaf(p, v[s], num);
                }
            elem<OT>::store(out, (int64_t)b * out_bstride + ei * c + ch, num / den);
        }
    } else {
        // one entry x 64 channels: four row quarters per channel, merged in LDS (the
        // quarters' states go where the tile was, once every thread has read its rows)
        const int x = tid & (CW - 1), qtr = tid / CW;
        const int ch = nt * CW + x;
        float m = -INFINITY, den = 0.f, num = 0.f;
        for (int r = 32 * qtr; r < 32 * qtr + 32; ++r) {
            float z = tile[r * TP + CW + x];
            if (bias != nullptr) z += bias[(int64_t)r * c + (ch < c ? ch : 0)];
            const float v = tile[r * TP + x];
            const float mn = fmaxf(m, z);
            const float a = __expf(m - mn), p = __expf(z - mn);
            den = den * a + p;
            num = num * a + p * v;
            m = mn;
        }
        __syncthreads();
        float(*red)[4][CW] = reinterpret_cast<float(*)[4][CW]>(lds);
        red[0][qtr][x] = m;
        red[1][qtr][x] = den;
        red[2][qtr][x] = num;
        __syncthreads();
        if (qtr == 0 && ch < c && (int64_t)mt < E) {
            float M = red[0][0][x];
#pragma unroll
            for (int u = 1; u < 4; ++u) M = fmaxf(M, red[0][u][x]);
            float D = 0.f, U = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float f = __expf(red[0][u][x] - M);
                D += red[1][u][x] * f;
                U += red[2][u][x] * f;
            }
            elem<OT>::store(out, (int64_t)b * out_bstride + (int64_t)mt * c + ch, U / D);
        }
    }
}

// the compressor's ring also holds its fp32 epilogue tile
static_assert(compress_lds<32>() <= 160 * 1024 && compress_lds<64>() <= 160 * 1024, "one workgroup fits a CU's LDS");
// the plain GEMM: 256 x 256 tiles of 8 wavefronts, one workgroup per CU (128 KiB of LDS):
// K slices of 64 in 2 stages (one barrier per 32 matrix ops of a wavefront) when K % 64 == 0,
// else slices of 32 in 4 stages
constexpr int kGemmMI = 4, kGemmWN = 4;

template <int NST, int BK, int WN = kGemmWN, int MI = kGemmMI>
void launch_gemm_cfg(const bf16_t *A, int64_t lda, int64_t sA, const bf16_t *B, int64_t ldb, int64_t sB, void *C,
                     int64_t ldc, int64_t sC, bool c_f32, int64_t M, int64_t N, int64_t K, int batch,
                     hipStream_t st) {
    using TL = Tile<MI, NST, WN, BK>;
    const int mtiles = (int)((M + TL::BM - 1) / TL::BM), ntiles = (int)((N + TL::BN - 1) / TL::BN);
    const dim3 grid((unsigned)((int64_t)mtiles * ntiles), 1, (unsigned)batch);
    if (c_f32)
        hipLaunchKernelGGL((gemm_bf16_kernel<float, MI, NST, WN, BK>), grid, dim3(128 * WN), 0, st, A, lda, sA,
                           B, ldb, sB, (float *)C, ldc, sC, M, N, K, mtiles);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<bf16_t, MI, NST, WN, BK>), grid, dim3(128 * WN), 0, st, A, lda,
                           sA, B, ldb, sB, (bf16_t *)C, ldc, sC, M, N, K, mtiles);
}

// Columns of C that 256 x 256 tiles cover in whole rounds of one workgroup per compute
// unit; the rest go to a second launch of 256 x 128 tiles, so the last round is not a
// partial one of full-size tiles (Pro width: 896 tiles = 3.5 rounds become 768 + 256
// half-size tiles). 0 when the tiles already fill whole rounds or fill less than one.
inline int64_t gemm_round_columns(int64_t M, int64_t N, int batch) {
    const int cu = device_cu_count();
    const int64_t mt = (M + 255) / 256, nt = (N + 255) / 256, per_nt = mt * batch;
    const int64_t tiles = per_nt * nt;
    if (cu <= 0 || tiles <= cu || tiles % cu == 0) return 0;
    const int64_t main_nt = (tiles / cu) * cu / per_nt;
    return (main_nt >= 1 && main_nt < nt) ? main_nt * 256 : 0;
}

}  // namespace

int launch_gemm_bf16(const bf16_t *A, int64_t lda, int64_t sA, const bf16_t *B, int64_t ldb, int64_t sB, void *C,
                     int64_t ldc, int64_t sC, bool c_f32, int64_t M, int64_t N, int64_t K, int batch,
                     hipStream_t st) {
    if (M == 0 || N == 0 || batch == 0) return CSA_OK;
    if (K % 64 == 0) {
        const int64_t n1 = gemm_round_columns(M, N, batch);
        if (n1 == 0) {
            launch_gemm_cfg<2, 64>(A, lda, sA, B, ldb, sB, C, ldc, sC, c_f32, M, N, K, batch, st);
        } else {
            launch_gemm_cfg<2, 64>(A, lda, sA, B, ldb, sB, C, ldc, sC, c_f32, M, n1, K, batch, st);
            void *C2 = c_f32 ? (void *)((float *)C + n1) : (void *)((bf16_t *)C + n1);
            launch_gemm_cfg<2, 64, 2>(A, lda, sA, B + n1 * ldb, ldb, sB, C2, ldc, sC, c_f32, M, N - n1, K, batch, st);
        }
    } else
        launch_gemm_cfg<4, 32>(A, lda, sA, B, ldb, sB, C, ldc, sC, c_f32, M, N, K, batch, st);
    return check_launch("gemm_bf16_kernel");
}

template <int BK>
void launch_compress_cfg(const bf16_t *Hs, const bf16_t *carry, const bf16_t *W, const float *bias, int B, int64_t n,
                         int64_t d, int c, int ratio, void *out, bool out_f32, int64_t bs, hipStream_t st) {
    if (ratio == 4) {
        const int mtiles = (int)((n + 123) / 124), ntiles = (c + 16 * kCompressWN - 1) / (16 * kCompressWN);
        const dim3 grid((unsigned)((int64_t)mtiles * ntiles), 1, (unsigned)B);
        if (out_f32)
            hipLaunchKernelGGL((compress_hidden_kernel<4, float, BK>), grid, dim3(128 * kCompressWN), 0, st, Hs, carry, W, bias,
                               n, d, c, (float *)out, bs, mtiles, ntiles);
        else
            hipLaunchKernelGGL((compress_hidden_kernel<4, bf16_t, BK>), grid, dim3(128 * kCompressWN), 0, st, Hs, carry, W,
                               bias, n, d, c, (bf16_t *)out, bs, mtiles, ntiles);
    } else {
        const int mtiles = (int)(n / ratio), ntiles = (c + 32 * kCompressWN - 1) / (32 * kCompressWN);
        const dim3 grid((unsigned)((int64_t)mtiles * ntiles), 1, (unsigned)B);
        if (out_f32)
            hipLaunchKernelGGL((compress_hidden_kernel<128, float, BK>), grid, dim3(128 * kCompressWN), 0, st, Hs, carry, W,
                               bias, n, d, c, (float *)out, bs, mtiles, ntiles);
        else
            hipLaunchKernelGGL((compress_hidden_kernel<128, bf16_t, BK>), grid, dim3(128 * kCompressWN), 0, st, Hs, carry, W,
                               bias, n, d, c, (bf16_t *)out, bs, mtiles, ntiles);
    }
}

int launch_compress_hidden(const bf16_t *Hs, const bf16_t *carry, const bf16_t *W, const float *bias, int B,
                           int64_t n, int64_t d, int c, int ratio, void *out, bool out_f32, int64_t out_bstride,
                           hipStream_t st) {
    const int64_t E = n / ratio;
    if (B == 0 || E == 0) return CSA_OK;
    const int64_t bs = out_bstride ? out_bstride : E * c;
    if (d % 64 == 0)
        launch_compress_cfg<64>(Hs, carry, W, bias, B, n, d, c, ratio, out, out_f32, bs, st);
    else
        launch_compress_cfg<32>(Hs, carry, W, bias, B, n, d, c, ratio, out, out_f32, bs, st);
    return check_launch("compress_hidden_kernel");
}

}  // namespace csa
