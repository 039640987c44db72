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
// bf16, D = 512, H % 64 == 0: the matrix-core kernel of attn_wide.hip (one workgroup per
// query and 64 heads, 32-row tiles through LDS, S^T and O = P V on MFMA 16x16x32). For few
// queries the row slots are split over workgroups that write (max, denominator, O)
// partials, merged here by attn_merge_kernel (log-sum-exp merge + sink + inverse RoPE).
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
// bf16, D = 512, H % 64 == 0: the matrix-core kernel lives in attn_wide.hip; it shares
// the row-split heuristic, the workspace layout and the merge kernel below
// ======================================================================================
constexpr int MD = 512;      // head dim
constexpr int MHG = 64;      // heads per workgroup
constexpr int MTR = 32;      // rows per tile

// log-sum-exp merge of split partials + sink + inverse RoPE; one wavefront per (query, head),
// eight dims per lane. Workspace layout: [T][nsplit][H][2] fp32 (m_s, l_s), then
// [T][nsplit][H][D] bf16 partial sums (each split's unnormalised O, rounded once to bf16:
// half the bytes of fp32, and the merged output is bf16 anyway). Lane s holds the weights
// of splits s, s + 64, s + 128, s + 192; the partial rows are fetched 16 bytes per lane in
// batches of 32 splits whose loads are all issued before the first is used (the merge is a
// latency problem: a few MB spread over 256 compute units), and the wave-uniform weight of
// each split is read out of its lane with readlane into a scalar register.
__global__ void __launch_bounds__(64)
attn_merge_kernel(const float *__restrict__ part, const float *__restrict__ sink, int nsplit,
                  const float *__restrict__ rope_cs, int R, int T, int H,
                  bf16_t *__restrict__ out, float *__restrict__ lse)
{
    constexpr int D = MD;
    constexpr int MB = 32;  // partial rows in flight per lane
    const int64_t unit = blockIdx.x;
    const int t = (int)(unit / H), g = (int)(unit % H);
    const int lane = threadIdx.x;
    const int64_t hs = (int64_t)H * 2;  // stride of one split in the (m, l) array
    const float *pml = part + ((int64_t)t * nsplit * H + g) * 2;
    const int64_t vs = (int64_t)H * D / 8;  // stride of one split in 16-byte units
    const uint4 *pacc = reinterpret_cast<const uint4 *>(part + (int64_t)T * nsplit * H * 2) +
                        ((int64_t)t * nsplit * H + g) * (D / 8) + lane;
    float mv[4], lv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int s = lane + 64 * c;
        mv[c] = s < nsplit ? pml[s * hs] : -INFINITY;
        lv[c] = s < nsplit ? pml[s * hs + 1] : 0.f;
    }
    uint4 v[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) v[i] = i < nsplit ? pacc[i * vs] : make_uint4(0u, 0u, 0u, 0u);
    const float sk = sink[g] * kLog2e;
    float M = fmaxf(sk, fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float mu = (M == -INFINITY) ? 0.f : M;
    float f[4], L = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        f[c] = exp2f(mv[c] - mu);
        L += lv[c] * f[c];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    L += exp2f(sk - mu);
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto fold = [&](const uint4 &w, float fw) {
        x[0] = fmaf(lo_bf16(w.x), fw, x[0]);
        x[1] = fmaf(hi_bf16(w.x), fw, x[1]);
        x[2] = fmaf(lo_bf16(w.y), fw, x[2]);
        x[3] = fmaf(hi_bf16(w.y), fw, x[3]);
        x[4] = fmaf(lo_bf16(w.z), fw, x[4]);
        x[5] = fmaf(hi_bf16(w.z), fw, x[5]);
        x[6] = fmaf(lo_bf16(w.w), fw, x[6]);
        x[7] = fmaf(hi_bf16(w.w), fw, x[7]);
    };
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int b = 0; b < 64; b += MB) {
            const int s0 = 64 * c + b;
            if (s0 >= nsplit) break;
            if (s0 > 0) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    v[i] = s0 + i < nsplit ? pacc[(s0 + i) * vs] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
                fold(v[i], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f[c]), b + i)));
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int d0 = 8 * lane;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        float x0 = x[e] * inv, x1 = x[e + 1] * inv;
        const int d = d0 + e;
        if (rope_cs != nullptr && d >= D - R) {
            const int p = (d - (D - R)) >> 1;
            const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2], sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
            const float y0 = x0 * cs + x1 * sn, y1 = -x0 * sn + x1 * cs;
            x0 = y0;
            x1 = y1;
        }
        x[e] = x0;
        x[e + 1] = x1;
    }
    bf16_t *orow = out + ((int64_t)t * H + g) * D + d0;
    if ((reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)f32_to_bf16(x[2 * e]) |
                   ((uint32_t)f32_to_bf16(x[2 * e + 1]) << 16);
        *reinterpret_cast<uint4 *>(orow) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) orow[e] = f32_to_bf16(x[e]);
    }
    if (lse != nullptr && lane == 0) lse[(int64_t)t * H + g] = L > 0.f ? (mu + log2f(L)) * kLn2 : -INFINITY;
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
    return (size_t)T * ns * H * (2 * sizeof(float) + (size_t)D * sizeof(bf16_t));
}

int launch_attn(const AttnArgs &a, hipStream_t st) {
    if (a.T == 0) return CSA_OK;
    const float sl2 = a.scale * kLog2e;
    if (!wide_attn_ok(a.dt, a.H, a.D)) {
        return a.dt == CSA_F32 ? launch_valu<float>(a, sl2, st) : launch_valu<bf16_t>(a, sl2, st);
    }
    const int64_t max_rows = (a.ratio > 0 ? a.N : (int64_t)a.k) + ((a.swa && a.window > 0) ? a.window : 0);
    const int ns = mfma_splits(a.T, a.H, max_rows);
    const size_t need = attn_workspace_bytes(a.T, a.H, a.D, max_rows);
    if (need > a.ws_bytes || (need > 0 && a.ws == nullptr))
        return fail(CSA_EWORKSPACE, "attention: workspace smaller than csa_attn_workspace_bytes()");
    if (need > 0 && (reinterpret_cast<uintptr_t>(a.ws) & 15) != 0)
        return fail(CSA_EINVAL, "attention: workspace must be 16-byte aligned");
    const int64_t tiles = (max_rows + MTR - 1) / MTR;
    const int64_t split_slots = ((tiles + ns - 1) / ns) * MTR;
    const int rc = launch_attn_wide(a, sl2, ns, split_slots, st);
    if (rc != CSA_OK || ns == 1) return rc;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((int64_t)a.T * a.H)), dim3(64), 0, st,
                       (const float *)a.ws, a.sink, ns, a.rope_cs, a.rope_dim, a.T, a.H, (bf16_t *)a.out, a.lse);
    return check_launch("attn_merge_kernel");
}

}  // namespace csa
