// Shared-KV multi-query attention with an attention sink on gfx950.
//
// "DeepSeek-V4 混合注意力" §4.2 (one compressed vector serves as K and V for every query
// head; CSA reads the top-k selected entries), §5 (HCA reads every visible summary), §6
// (128-token SWA rows, attention sink p_i = e^{z_i} / (e^{z_s} + sum_j e^{z_j}), RoPE on
// the last 64 dims of q and inverse RoPE on the output).
//
// Row slots of query t: first the main rows (top-k indices, or summaries 0..nvis-1),
// then the SWA positions max(0, t-window+1)..t that the caller's SWA buffer holds.
//
// bf16, D = 512, H % 64 == 0: the matrix-core kernel. A workgroup (4 wavefronts) owns
// one query, 64 heads and a range of row slots; wavefront w owns dims [128w, 128w+128).
// Per 32-row tile:
//   - each wave loads its 128-dim slice of the 32 gathered rows straight from global
//     memory into MFMA B fragments (16 contiguous bytes per lane per fragment) and forms
//     the partial logits S_w = Q[:, slice] K[:, slice]^T (64 x 32, 32 MFMA 16x16x32);
//   - it stages the same slice transposed in LDS (rows contiguous per dim) for P V;
//   - the four partial S planes meet in LDS; wave w reduces heads 16w..16w+15, runs the
//     online softmax (fp32 state in registers: running max, denominator) and writes
//     P (bf16) and the rescale factors;
//   - every wave accumulates O[:, slice] += P V[:, slice] (32 MFMA) in registers.
// The sink seeds the running state (max = sink, denominator = 1). For few queries the
// row slots are split over workgroups that write (max, denominator, O) partials, merged
// by attn_merge_kernel (log-sum-exp merge + sink + inverse RoPE).
//
// Any other shape/dtype: attn_valu_kernel, one wavefront per (query, head), rows one by
// one with a wave-wide dot product and the same online softmax.
#include "attn_rows.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

// ======================================================================================
// generic kernel: one wavefront per (query, head); lane l holds dims [l*VPL, (l+1)*VPL)
// ======================================================================================
template <typename ET, int VPL>
__global__ void __launch_bounds__(256)
attn_valu_kernel(const ET *__restrict__ q, const ET *__restrict__ kv, const float *__restrict__ sink,
                 const int32_t *__restrict__ idx, int k, int ratio, float scale_log2,
                 const ET *__restrict__ swa, const int64_t *__restrict__ swa_pos0, int swa_rows,
                 int window, const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos,
                 const float *__restrict__ rope_cs, int R, int T, int B, int64_t N, int H,
                 ET *__restrict__ out, float *__restrict__ lse)
{
    constexpr int D = 64 * VPL;
    __shared__ float obuf[4][D];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t unit0 = (int64_t)blockIdx.x * 4 + wv;
    const bool active = unit0 < (int64_t)T * H;  // inactive waves still reach the barrier
    const int64_t unit = active ? unit0 : 0;
    const int t = (int)(unit / H), g = (int)(unit % H);
    RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    if (!active) c.nslots = 0;

    float qv[VPL], acc[VPL];
    const ET *qrow = q + ((int64_t)t * H + g) * D;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int d = lane * VPL + v;
        float x = elem<ET>::load(qrow, d);
        if (rope_cs != nullptr && d >= D - R) {
            const int p = (d - (D - R)) >> 1;
            const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2], sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
            const float y = elem<ET>::load(qrow, d ^ 1);
            x = (d & 1) ? (y * sn + x * cs) : (x * cs - y * sn);
        }
        qv[v] = x;
        acc[v] = 0.f;
    }
    float m = sink[g] * kLog2e, l = (m == -INFINITY) ? 0.f : 1.f;  // e^{sink - m}
    for (int64_t j = 0; j < c.nslots; ++j) {
        const ET *rp = row_ptr<ET>(c, j, t, kv, idx, k, ratio, N, swa, swa_pos0, swa_rows, D);
        if (rp == nullptr) continue;
        float x[VPL], dot = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            x[v] = elem<ET>::load(rp, lane * VPL + v);
            dot = fmaf(qv[v], x[v], dot);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
        const float z = dot * scale_log2;
        const float mn = fmaxf(m, z);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float a = exp2f(m - mu), e = exp2f(z - mu);
        l = l * a + e;
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[v] = acc[v] * a + e * x[v];
        m = mn;
    }
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) obuf[wv][lane * VPL + v] = acc[v] * inv;
    __syncthreads();
    if (!active) return;
    ET *orow = out + ((int64_t)t * H + g) * D;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int d = lane * VPL + v;
        float x = obuf[wv][d];
        if (rope_cs != nullptr && d >= D - R) {
            const int p = (d - (D - R)) >> 1;
            const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2], sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
            const float y = obuf[wv][d ^ 1];
            x = (d & 1) ? (x * cs - y * sn) : (x * cs + y * sn);
        }
        elem<ET>::store(orow, d, x);
    }
    if (lse != nullptr && lane == 0) {
        const float mu = (m == -INFINITY) ? 0.f : m;
        lse[(int64_t)t * H + g] = (l > 0.f) ? (mu + log2f(l)) * kLn2 : -INFINITY;
    }
}

// ======================================================================================
// matrix-core kernel: bf16, D = 512, 64 heads per workgroup
// ======================================================================================
constexpr int MD = 512;      // head dim
constexpr int MHG = 64;      // heads per workgroup
constexpr int MTR = 32;      // rows per tile
constexpr int SPAD = 36;     // fp32 pitch of a head row of partial logits
constexpr int VPAD = 40;     // bf16 pitch of a transposed dim row (32 rows + pad)

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__global__ void __launch_bounds__(256, 1)
attn_mfma_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ kv, const float *__restrict__ sink,
                 const int32_t *__restrict__ idx, int k, int ratio, float scale_log2,
                 const bf16_t *__restrict__ swa, const int64_t *__restrict__ swa_pos0, int swa_rows,
                 int window, const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos,
                 const float *__restrict__ rope_cs, int R, int T, int B, int64_t N, int H,
                 bf16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part,
                 int nsplit, int64_t split_slots)
{
    __shared__ float Sp[4][MHG][SPAD];
    __shared__ __attribute__((aligned(16))) bf16_t Ps[MHG][MTR];
    __shared__ __attribute__((aligned(16))) bf16_t KVT[4][128][VPAD];
    __shared__ float alpha_s[MHG];
    __shared__ float m_s[MHG];
    __shared__ float l_s[MHG];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    // XCD-aware placement: workgroups b and b+8 run on the same XCD; the head groups of
    // one (query, split) unit are adjacent in that order so they share the L2
    const int HGN = H / MHG;
    const int64_t U = (int64_t)T * nsplit;
    const int64_t per_xcd = (U + 7) / 8;
    const int64_t bid = blockIdx.x;
    const int xcd = (int)(bid & 7);
    const int64_t r8 = bid >> 3;
    const int hg = (int)(r8 % HGN);
    const int64_t uu = r8 / HGN;
    const int64_t u = xcd * per_xcd + uu;
    if (uu >= per_xcd || u >= U) return;
    const int t = (int)(u / nsplit), sp = (int)(u % nsplit);

    const RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    const int64_t j0 = (int64_t)sp * split_slots;
    int64_t j1 = j0 + split_slots;
    if (j1 > c.nslots) j1 = c.nslots;

    // ---- Q fragments (A operand): head 16m + l16, dims 128w + 32kk + 8g4 .. +7 ----------
    bf16x8 qa[4][4];
    {
        const int head0 = hg * MHG;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16_t *qrow = q + ((int64_t)t * H + head0 + 16 * m + l16) * MD;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int d0 = 128 * w + 32 * kk + 8 * g4;
                uint4 raw = *reinterpret_cast<const uint4 *>(qrow + d0);
                if (rope_cs != nullptr && d0 + 8 > MD - R) {
                    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
                    uint32_t o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x0 = lo_bf16(wd[e]), x1 = hi_bf16(wd[e]);
                        const int d = d0 + 2 * e;
                        if (d >= MD - R) {
                            const int p = (d - (MD - R)) >> 1;
                            const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2];
                            const float sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
                            const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
                            x0 = y0;
                            x1 = y1;
                        }
                        o[e] = pack2(x0, x1);
                    }
                    raw = make_uint4(o[0], o[1], o[2], o[3]);
                }
                qa[m][kk] = as_bf16x8(raw);
            }
        }
    }

    // softmax state of head 16w + lane/4 (replicated over the 4 lanes of a head)
    const bool single = (nsplit == 1);
    float m_run = single ? sink[hg * MHG + 16 * w + (lane >> 2)] * kLog2e : -INFINITY;
    float l_run = (single && m_run != -INFINITY) ? 1.f : 0.f;  // e^{sink - m_run}

    f32x4 acc[4][8];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) acc[m][nd] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment loads of one tile: rows 16n + l16, dims 128w + 32kk + 8g4 .. +7
    auto load_tile = [&](int64_t jt, uint4 (&kf)[2][4], uint32_t &valid) {
        valid = 0u;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int64_t j = jt + 16 * n + l16;
            const bf16_t *rp = (j < j1) ? row_ptr<bf16_t>(c, j, t, kv, idx, k, ratio, N, swa, swa_pos0,
                                                          swa_rows, MD)
                                        : nullptr;
            const uint64_t bal = __ballot(rp != nullptr);
            valid |= (uint32_t)((bal >> 0) & 0xffffu) << (16 * n);  // lanes 0..15 carry rows 0..15
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (rp != nullptr)
                    kf[n][kk] = *reinterpret_cast<const uint4 *>(rp + 128 * w + 32 * kk + 8 * g4);
                else
                    kf[n][kk] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    uint4 kf[2][4], kfn[2][4];
    uint32_t valid = 0u, validn = 0u;
    if (j0 < j1) load_tile(j0, kf, valid);

    for (int64_t jt = j0; jt < j1; jt += MTR) {
        // ---- partial logits over this wave's dims --------------------------------------
        f32x4 sacc[4][2];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n) sacc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    sacc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[m][kk], as_bf16x8(kf[n][kk]),
                                                                         sacc[m][n], 0, 0, 0);
        // ---- stage V^T: KVT[w][dim][row] ---------------------------------------------
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint32_t wd[4] = {kf[n][kk].x, kf[n][kk].y, kf[n][kk].z, kf[n][kk].w};
                const int row = 16 * n + l16;
                const int dim0 = 32 * kk + 8 * g4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    KVT[w][dim0 + 2 * e][row] = (bf16_t)(wd[e] & 0xffffu);
                    KVT[w][dim0 + 2 * e + 1][row] = (bf16_t)(wd[e] >> 16);
                }
            }
        // ---- prefetch the next tile ---------------------------------------------------
        const bool has_next = jt + MTR < j1;
        if (has_next) load_tile(jt + MTR, kfn, validn);
        // ---- partial logits to LDS: lane holds S[16m + 4g4 + r][16n + l16] -------------
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sp[w][16 * m + 4 * g4 + r][16 * n + l16] = sacc[m][n][r];
        __syncthreads();
        // ---- online softmax of heads 16w..16w+15: lane -> head lane/4, rows 8(lane%4).. --
        {
            const int hh = 16 * w + (lane >> 2);
            const int r0 = 8 * (lane & 3);
            float z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
                for (int e = 0; e < 8; ++e) z[e] += Sp[w2][hh][r0 + e];
            float tmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                z[e] = ((valid >> (r0 + e)) & 1u) ? z[e] * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, z[e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 1));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 2));
            const float mn = fmaxf(m_run, tmax);
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            const float a = exp2f(m_run - mu);
            float p[8], rs = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = exp2f(z[e] - mu);
                rs += p[e];
            }
            rs += __shfl_xor(rs, 1);
            rs += __shfl_xor(rs, 2);
            l_run = l_run * a + rs;
            m_run = mn;
            uint4 pk = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
            *reinterpret_cast<uint4 *>(&Ps[hh][r0]) = pk;
            if ((lane & 3) == 0) alpha_s[hh] = a;
        }
        __syncthreads();
        // ---- O[:, slice] = O * alpha + P V[:, slice] -----------------------------------
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 al;
#pragma unroll
            for (int r = 0; r < 4; ++r) al[r] = alpha_s[16 * m + 4 * g4 + r];
#pragma unroll
            for (int nd = 0; nd < 8; ++nd) acc[m][nd] *= al;
        }
        bf16x8 pa[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) pa[m] = as_bf16x8(*reinterpret_cast<const uint4 *>(&Ps[16 * m + l16][8 * g4]));
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) {
            const bf16x8 vb = as_bf16x8(*reinterpret_cast<const uint4 *>(&KVT[w][16 * nd + l16][8 * g4]));
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[m], vb, acc[m][nd], 0, 0, 0);
        }
        if (has_next) {
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kf[n][kk] = kfn[n][kk];
            valid = validn;
        }
    }

    // ---- epilogue --------------------------------------------------------------------
    if ((lane & 3) == 0) {
        m_s[16 * w + (lane >> 2)] = m_run;
        l_s[16 * w + (lane >> 2)] = l_run;
    }
    __syncthreads();
    const int head0 = hg * MHG;
    if (single) {
        if (lse != nullptr && (lane & 3) == 0) {
            const float mu = (m_run == -INFINITY) ? 0.f : m_run;
            lse[(int64_t)t * H + head0 + 16 * w + (lane >> 2)] = (l_run > 0.f) ? (mu + log2f(l_run)) * kLn2 : -INFINITY;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = 16 * m + 4 * g4 + r;
                const float lv = l_s[hh];
                const float inv = lv > 0.f ? 1.f / lv : 0.f;
                bf16_t *orow = out + ((int64_t)t * H + head0 + hh) * MD;
#pragma unroll
                for (int nd = 0; nd < 8; ++nd) {
                    const int d = 128 * w + 16 * nd + l16;
                    float x = acc[m][nd][r] * inv;
                    const float y = __shfl_xor(x, 1);
                    if (rope_cs != nullptr && d >= MD - R) {
                        const int p = (d - (MD - R)) >> 1;
                        const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2];
                        const float sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
                        x = (d & 1) ? (x * cs - y * sn) : (x * cs + y * sn);
                    }
                    orow[d] = f32_to_bf16(x);
                }
            }
        }
    } else {
        const int64_t pu = ((int64_t)t * nsplit + sp) * H + head0;
        float *pml = part;                                       // [T][nsplit][H][2]
        float *pacc = part + (int64_t)T * nsplit * H * 2;        // [T][nsplit][H][D]
        if ((lane & 3) == 0) {
            pml[(pu + 16 * w + (lane >> 2)) * 2] = m_run;
            pml[(pu + 16 * w + (lane >> 2)) * 2 + 1] = l_run;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *prow = pacc + (pu + 16 * m + 4 * g4 + r) * MD;
#pragma unroll
                for (int nd = 0; nd < 8; ++nd) prow[128 * w + 16 * nd + l16] = acc[m][nd][r];
            }
    }
}

// log-sum-exp merge of split partials + sink + inverse RoPE; one block per (query, head).
// The per-split weights 2^(m_s - M) are formed once in LDS; every thread then streams
// its two output dims over all splits with independent loads.
template <typename ET>
__global__ void __launch_bounds__(256)
attn_merge_kernel(const float *__restrict__ part, const float *__restrict__ sink, int nsplit,
                  const float *__restrict__ rope_cs, int R, int T, int H, int D,
                  ET *__restrict__ out, float *__restrict__ lse)
{
    __shared__ float fs[256];
    __shared__ float red[2];
    const int64_t unit = blockIdx.x;
    const int t = (int)(unit / H), g = (int)(unit % H);
    const float *pml = part;
    const float *pacc = part + (int64_t)T * nsplit * H * 2;
    const float sk = sink[g] * kLog2e;
    if (threadIdx.x < 64) {
        // one wavefront forms the global max, the denominator and the split weights
        const int lane = threadIdx.x;
        float M = sk;
        for (int s2 = lane; s2 < nsplit; s2 += 64) M = fmaxf(M, pml[(((int64_t)t * nsplit + s2) * H + g) * 2]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float mu = (M == -INFINITY) ? 0.f : M;
        float L = 0.f;
        for (int s2 = lane; s2 < nsplit; s2 += 64) {
            const int64_t o = (((int64_t)t * nsplit + s2) * H + g) * 2;
            const float f = exp2f(pml[o] - mu);
            fs[s2] = f;
            L += pml[o + 1] * f;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
        L += exp2f(sk - mu);
        if (lane == 0) {
            red[0] = mu;
            red[1] = L;
        }
    }
    __syncthreads();
    const float mu = red[0], L = red[1];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int d0 = 2 * threadIdx.x; d0 < D; d0 += 2 * blockDim.x) {
        float x0 = 0.f, x1 = 0.f;
        const float *pp = pacc + (((int64_t)t * nsplit) * H + g) * D + d0;
#pragma unroll 8
        for (int s2 = 0; s2 < nsplit; ++s2) {
            const float2 v = *reinterpret_cast<const float2 *>(pp + (int64_t)s2 * H * D);
            x0 = fmaf(v.x, fs[s2], x0);
            x1 = fmaf(v.y, fs[s2], x1);
        }
        x0 *= inv;
        x1 *= inv;
        if (rope_cs != nullptr && d0 >= D - R) {
            const int p = (d0 - (D - R)) >> 1;
            const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2], sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
            const float y0 = x0 * cs + x1 * sn, y1 = -x0 * sn + x1 * cs;
            x0 = y0;
            x1 = y1;
        }
        ET *orow = out + ((int64_t)t * H + g) * D;
        elem<ET>::store(orow, d0, x0);
        elem<ET>::store(orow, d0 + 1, x1);
    }
    if (lse != nullptr && threadIdx.x == 0) lse[(int64_t)t * H + g] = L > 0.f ? (mu + log2f(L)) * kLn2 : -INFINITY;
}

// Row splits per (query, head group): enough workgroups to cover the CUs once, at least
// four 32-row tiles per split, at most 256 splits (the merge keeps one weight per split).
int mfma_splits(int T, int H, int64_t max_rows) {
    const int64_t base = (int64_t)T * (H / MHG);
    const int64_t tiles = (max_rows + MTR - 1) / MTR;
    if (base >= 256 || tiles < 8) return 1;
    int64_t ns = (256 + base - 1) / base;
    const int64_t cap = tiles / 4;
    if (ns > cap) ns = cap;
    if (ns > 256) ns = 256;
    return ns < 1 ? 1 : (int)ns;
}

bool use_mfma(csa_dtype dt, int H, int D) { return dt == CSA_BF16 && D == MD && H % MHG == 0; }

template <typename ET, int VPL>
void launch_valu_t(const AttnArgs &a, float sl2, hipStream_t st) {
    const int64_t units = (int64_t)a.T * a.H;
    hipLaunchKernelGGL((attn_valu_kernel<ET, VPL>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st,
                       (const ET *)a.q, (const ET *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2, (const ET *)a.swa,
                       a.swa_pos0, a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs, a.rope_dim, a.T, a.B,
                       a.N, a.H, (ET *)a.out, a.lse);
}

template <typename ET>
int launch_valu(const AttnArgs &a, float sl2, hipStream_t st) {
    switch (a.D / 64) {
#define CSA_VPL(V) \
    case V: launch_valu_t<ET, V>(a, sl2, st); break;
        CSA_VPL(1) CSA_VPL(2) CSA_VPL(3) CSA_VPL(4) CSA_VPL(5) CSA_VPL(6) CSA_VPL(7) CSA_VPL(8)
        CSA_VPL(9) CSA_VPL(10) CSA_VPL(11) CSA_VPL(12) CSA_VPL(13) CSA_VPL(14) CSA_VPL(15) CSA_VPL(16)
#undef CSA_VPL
        default: return fail(CSA_EUNSUPPORTED, "attention: D must be a multiple of 64 and <= 1024");
    }
    return check_launch("attn_valu_kernel");
}

}  // namespace

size_t attn_workspace_bytes(int T, int H, int D, int64_t max_rows) {
    if (D != MD || H % MHG != 0) return 0;
    const int ns = mfma_splits(T, H, max_rows);
    if (ns <= 1) return 0;
    return (size_t)T * ns * H * (size_t)(D + 2) * sizeof(float);
}

int launch_attn(const AttnArgs &a, hipStream_t st) {
    if (a.T == 0) return CSA_OK;
    const float sl2 = a.scale * kLog2e;
    if (!use_mfma(a.dt, a.H, a.D)) {
        return a.dt == CSA_F32 ? launch_valu<float>(a, sl2, st) : launch_valu<bf16_t>(a, sl2, st);
    }
    const int64_t max_rows = (a.ratio > 0 ? a.N : (int64_t)a.k) + ((a.swa && a.window > 0) ? a.window : 0);
    const int ns = mfma_splits(a.T, a.H, max_rows);
    const size_t need = attn_workspace_bytes(a.T, a.H, a.D, max_rows);
    if (need > a.ws_bytes || (need > 0 && a.ws == nullptr))
        return fail(CSA_EWORKSPACE, "attention: workspace smaller than csa_attn_workspace_bytes()");
    const int64_t tiles = (max_rows + MTR - 1) / MTR;
    const int64_t split_slots = ((tiles + ns - 1) / ns) * MTR;
    int rc;
    if (wide_attn_ok(a.dt, a.H, a.D)) {
        rc = launch_attn_wide(a, sl2, ns, split_slots, st);
        if (rc != CSA_OK || ns == 1) return rc;
        hipLaunchKernelGGL(attn_merge_kernel<bf16_t>, dim3((unsigned)((int64_t)a.T * a.H)), dim3(256), 0, st,
                           (const float *)a.ws, a.sink, ns, a.rope_cs, a.rope_dim, a.T, a.H, a.D,
                           (bf16_t *)a.out, a.lse);
        return check_launch("attn_merge_kernel");
    }
    const int64_t U = (int64_t)a.T * ns;
    const int64_t blocks = ((U + 7) / 8) * 8 * (a.H / MHG);
    hipLaunchKernelGGL(attn_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16_t *)a.q,
                       (const bf16_t *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2, (const bf16_t *)a.swa,
                       a.swa_pos0, a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs, a.rope_dim, a.T, a.B,
                       a.N, a.H, (bf16_t *)a.out, a.lse, (float *)a.ws, ns, split_slots);
    rc = check_launch("attn_mfma_kernel");
    if (rc != CSA_OK || ns == 1) return rc;
    hipLaunchKernelGGL(attn_merge_kernel<bf16_t>, dim3((unsigned)((int64_t)a.T * a.H)), dim3(256), 0, st,
                       (const float *)a.ws, a.sink, ns, a.rope_cs, a.rope_dim, a.T, a.H, a.D, (bf16_t *)a.out,
                       a.lse);
    return check_launch("attn_merge_kernel");
}

}  // namespace csa
