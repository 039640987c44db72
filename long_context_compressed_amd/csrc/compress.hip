// Token-level KV compressor on gfx950.
//
// "DeepSeek-V4 混合注意力" §4.1 (ratio 4: one per-channel softmax over the b-branch rows
// of block i-1 and the a-branch rows of block i) and §5 (ratio 128: one per-channel
// softmax over the rows of block i).
//
// HBM-bound: every input row is read once. The main kernel (compress_vec_kernel) gives each
// lane 16 bytes of a row (8 bf16 or 4 fp32 channels), so one wave instruction moves 1 KiB:
//   - ratio 4: a thread owns (entry, 16-byte channel group) and loads all 8 slots of both
//     tensors in one batch (16 independent 16-byte loads), then the softmax per channel;
//   - ratio 128: a workgroup owns (entry, 8 channel groups); its 32 row groups of 4 rows
//     each load in one batch, and their (max, denominator, numerator) states merge by a
//     tree in LDS.
// Rows whose channel count or addresses do not allow 16-byte accesses take the scalar
// kernel (compress_kernel): a block per entry and channel tile, lanes along the channels.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

template <typename T>
__global__ void __launch_bounds__(256)
compress_kernel(const T *__restrict__ Ca, const T *__restrict__ Cb, const T *__restrict__ Za,
                const T *__restrict__ Zb, const T *__restrict__ cCb, const T *__restrict__ cZb,
                const float *__restrict__ bias, int64_t n, int c, int ratio, int overlap,
                T *__restrict__ out, int64_t out_bstride, int64_t E, int ctiles)
{
    const int CX = blockDim.x, SG = blockDim.y;
    const int tx = threadIdx.x, ty = threadIdx.y;
    int64_t blk = blockIdx.x;
    const int ct = (int)(blk % ctiles);
    blk /= ctiles;
    const int64_t i = blk % E;
    const int64_t b = blk / E;
    const int j = ct * CX + tx;
    const int S = (1 + overlap) * ratio;

    // the slots of this thread are read in batches of 8 independent loads before any
    // arithmetic, so a thread waits for one memory round trip per batch
    float m = -INFINITY, den = 0.f, num = 0.f;
    if (j < c) {
        for (int s0 = ty; s0 < S; s0 += 8 * SG) {
            float z[8], v[8];
            bool has[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = s0 + u * SG;
                has[u] = s < S;
                z[u] = -INFINITY;
                v[u] = 0.f;
                if (!has[u]) continue;
                if (overlap && s < ratio) {
                    if (i >= 1) {
                        const int64_t o = (b * n + (i - 1) * ratio + s) * c + j;
                        z[u] = elem<T>::load(Zb, o);
                        v[u] = elem<T>::load(Cb, o);
                    } else if (cCb != nullptr) {
                        const int64_t o = (b * ratio + s) * c + j;
                        z[u] = elem<T>::load(cZb, o);
                        v[u] = elem<T>::load(cCb, o);
                    } else {
                        has[u] = false;  // absent slot: weight 0
                    }
                } else {
                    const int64_t o = (b * n + i * ratio + (s - overlap * ratio)) * c + j;
                    z[u] = elem<T>::load(Za, o);
                    v[u] = elem<T>::load(Ca, o);
                }
                if (has[u] && bias != nullptr) z[u] += bias[(int64_t)s * c + j];
            }
            float bm = -INFINITY;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (has[u]) bm = fmaxf(bm, z[u]);
            if (bm == -INFINITY) continue;
            const float M = fmaxf(m, bm);
            const float a = expf(m - M);
            num *= a;
            den *= a;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (has[u]) {
                    const float e = expf(z[u] - M);
                    num += e * v[u];
                    den += e;
                }
            m = M;
        }
    }
    if (SG > 1) {
        __shared__ float sm[3][256];
        const int id = ty * CX + tx;
        sm[0][id] = m;
        sm[1][id] = den;
        sm[2][id] = num;
        __syncthreads();
        if (ty != 0) return;
        for (int g = 1; g < SG; ++g) {
            const float m2 = sm[0][g * CX + tx], d2 = sm[1][g * CX + tx], n2 = sm[2][g * CX + tx];
            const float M = fmaxf(m, m2);
            if (M == -INFINITY) continue;
            const float a = expf(m - M), a2 = expf(m2 - M);
            den = den * a + d2 * a2;
            num = num * a + n2 * a2;
            m = M;
        }
    }
    if (j < c) elem<T>::store(out, b * out_bstride + i * c + j, num / den);
}

// 16 bytes of a row: V channels, widened to fp32 / rounded back (RNE for bf16)
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
    static constexpr int V = 8;
    __device__ __forceinline__ static void unpack(uint4 r, float (&x)[8]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = lo_bf16(w[i]);
            x[2 * i + 1] = hi_bf16(w[i]);
        }
    }
    __device__ __forceinline__ static uint4 pack(const float (&x)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(x[2 * i]) | ((uint32_t)f32_to_bf16(x[2 * i + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <> struct Vec16<float> {
    static constexpr int V = 4;
    __device__ __forceinline__ static void unpack(uint4 r, float (&x)[4]) {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
    __device__ __forceinline__ static uint4 pack(const float (&x)[4]) {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
};

typedef unsigned int u32x4n __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load16(const void *p) {
    const u32x4n v = __builtin_nontemporal_load(reinterpret_cast<const u32x4n *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// RATIO 4 (overlapped: 8 slots = the b-branch rows of block e-1, then the a-branch rows of
// block e) or 128 (one branch, 128 slots). cg: the thread's 16-byte channel group; E
// entries per sequence, B sequences.
template <typename T, int RATIO>
__device__ __forceinline__ void
compress_vec_body(const T *__restrict__ Ca, const T *__restrict__ Cb, const T *__restrict__ Za,
                  const T *__restrict__ Zb, const T *__restrict__ cCb, const T *__restrict__ cZb,
                  const float *__restrict__ bias, int64_t n, int c, T *__restrict__ out, int64_t out_bstride,
                  int64_t E, int B, int64_t bid)
{
    constexpr int V = Vec16<T>::V;
    constexpr bool OV = RATIO == 4;
    constexpr int S = OV ? 2 * RATIO : RATIO;  // slots per entry
    constexpr int RG = OV ? 1 : 32;            // row groups per entry
    constexpr int RPT = S / RG;                // slots per thread
    constexpr int CPB = 256 / RG;              // channel groups per workgroup (row groups > 1)
    static_assert(RG == 1 || RG * CPB == 256, "row groups tile the workgroup");
    const int CG = c / V;
    int64_t e, b;
    int cg, rg;
    if constexpr (RG == 1) {
        const int64_t g = bid * 256 + threadIdx.x;
        cg = (int)(g % CG);
        const int64_t be = g / CG;
        e = be % E;
        b = be / E;
        if (b >= B) return;  // the grid's tail (no barrier below in this form)
        rg = 0;
    } else {
        const int64_t ctiles = (CG + CPB - 1) / CPB;
        int64_t blk = bid;
        const int ct = (int)(blk % ctiles);
        blk /= ctiles;
        e = blk % E;
        b = blk / E;
        cg = ct * CPB + (int)(threadIdx.x % CPB);
        rg = (int)(threadIdx.x / CPB);
    }
    const bool act = cg < CG;
    const int64_t col = (int64_t)cg * V;

    // all the thread's slots, both tensors, in one batch of independent 16-byte loads
    uint4 zr[RPT], vr[RPT];
    bool has[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int s = rg * RPT + u;
        const T *zp = nullptr, *vp = nullptr;
        if (OV && s < RATIO) {
            if (e >= 1) {
                const int64_t o = (b * n + (e - 1) * RATIO + s) * c + col;
                zp = Zb + o;
                vp = Cb + o;
            } else if (cCb != nullptr) {
                const int64_t o = (b * RATIO + s) * c + col;
                zp = cZb + o;
                vp = cCb + o;
            }
        } else {
            const int64_t o = (b * n + e * RATIO + (s - (OV ? RATIO : 0))) * c + col;
            zp = Za + o;
            vp = Ca + o;
        }
        has[u] = act && zp != nullptr;
        // every input byte is read once: non-temporal (streaming) loads
        zr[u] = has[u] ? nt_load16(zp) : make_uint4(0u, 0u, 0u, 0u);
        vr[u] = has[u] ? nt_load16(vp) : make_uint4(0u, 0u, 0u, 0u);
    }
    // per channel: the slots' maximum, then the weights' sum and the weighted sum, with the
    // logits in base 2 (z log2 e), so every weight is one v_exp_f32
    float m[V], den[V], num[V];
#pragma unroll
    for (int x = 0; x < V; ++x) {
        m[x] = -INFINITY;
        den[x] = 0.f;
        num[x] = 0.f;
    }
    float z[RPT][V];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        Vec16<T>::unpack(zr[u], z[u]);
        if (bias != nullptr && has[u]) {
            const float *bp = bias + (int64_t)(rg * RPT + u) * c + col;
#pragma unroll
            for (int x = 0; x < V; ++x) z[u][x] += bp[x];
        }
#pragma unroll
        for (int x = 0; x < V; ++x) {
            z[u][x] *= kLog2e;
            if (has[u]) m[x] = fmaxf(m[x], z[u][x]);
        }
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        float v[V];
        Vec16<T>::unpack(vr[u], v);
#pragma unroll
        for (int x = 0; x < V; ++x)
            if (has[u]) {
                const float w = __builtin_amdgcn_exp2f(z[u][x] - m[x]);
                den[x] += w;
                num[x] = fmaf(w, v[x], num[x]);
            }
    }
    if constexpr (RG > 1) {
        // tree merge of the row groups' states: (m, den, num) of group g at sm[.][g][channel group]
        __shared__ float sm[3][RG][CPB * V];
        const int ci = (int)(threadIdx.x % CPB) * V;
#pragma unroll
        for (int x = 0; x < V; ++x) {
            sm[0][rg][ci + x] = m[x];
            sm[1][rg][ci + x] = den[x];
            sm[2][rg][ci + x] = num[x];
        }
        __syncthreads();
#pragma unroll
        for (int h = RG / 2; h >= 1; h >>= 1) {
            if (rg < h) {
#pragma unroll
                for (int x = 0; x < V; ++x) {
                    const float m2 = sm[0][rg + h][ci + x], d2 = sm[1][rg + h][ci + x], n2 = sm[2][rg + h][ci + x];
                    const float M = fmaxf(m[x], m2);
                    if (M != -INFINITY) {
                        const float a = __builtin_amdgcn_exp2f(m[x] - M), a2 = __builtin_amdgcn_exp2f(m2 - M);
                        den[x] = den[x] * a + d2 * a2;
                        num[x] = num[x] * a + n2 * a2;
                        m[x] = M;
                    }
                    sm[0][rg][ci + x] = m[x];
                    sm[1][rg][ci + x] = den[x];
                    sm[2][rg][ci + x] = num[x];
                }
            }
            __syncthreads();
        }
        if (rg != 0) return;
    }
    if (!act) return;
    float o[V];
#pragma unroll
    for (int x = 0; x < V; ++x) o[x] = num[x] / den[x];
    *reinterpret_cast<uint4 *>(out + b * out_bstride + e * c + col) = Vec16<T>::pack(o);
}

// workgroups of one pooling (either ratio)
inline int64_t vec_blocks(int B, int64_t E, int c, int V, int ratio) {
    const int64_t CG = c / V;
    return ratio == 4 ? ((int64_t)B * E * CG + 255) / 256 : (int64_t)B * E * ((CG + 7) / 8);
}

template <typename T, int RATIO>
__global__ void __launch_bounds__(256)
compress_vec_kernel(const T *__restrict__ Ca, const T *__restrict__ Cb, const T *__restrict__ Za,
                    const T *__restrict__ Zb, const T *__restrict__ cCb, const T *__restrict__ cZb,
                    const float *__restrict__ bias, int64_t n, int c, T *__restrict__ out, int64_t out_bstride,
                    int64_t E, int B)
{
    compress_vec_body<T, RATIO>(Ca, Cb, Za, Zb, cCb, cZb, bias, n, c, out, out_bstride, E, B, blockIdx.x);
}

// Several poolings in one launch (the decode step's KV entry, index key and summary): job j
// owns workgroups [first[j], first[j + 1]); the job index is uniform per workgroup.
constexpr int kMaxCompressJobs = 8;
struct CompressJobs {
    const void *Ca[kMaxCompressJobs], *Cb[kMaxCompressJobs], *Za[kMaxCompressJobs], *Zb[kMaxCompressJobs];
    const void *cCb[kMaxCompressJobs], *cZb[kMaxCompressJobs];
    const float *bias[kMaxCompressJobs];
    void *out[kMaxCompressJobs];
    int64_t n[kMaxCompressJobs], E[kMaxCompressJobs], out_bstride[kMaxCompressJobs];
    int c[kMaxCompressJobs], ratio[kMaxCompressJobs], B[kMaxCompressJobs];
    int64_t first[kMaxCompressJobs + 1];
    int njobs;
};

template <typename T>
__global__ void __launch_bounds__(256) compress_batch_kernel(CompressJobs J)
{
    int jb = 0;
    while (jb + 1 < J.njobs && (int64_t)blockIdx.x >= J.first[jb + 1]) ++jb;
    const int64_t bid = (int64_t)blockIdx.x - J.first[jb];
    if (J.ratio[jb] == 4)
        compress_vec_body<T, 4>((const T *)J.Ca[jb], (const T *)J.Cb[jb], (const T *)J.Za[jb], (const T *)J.Zb[jb],
                                (const T *)J.cCb[jb], (const T *)J.cZb[jb], J.bias[jb], J.n[jb], J.c[jb],
                                (T *)J.out[jb], J.out_bstride[jb], J.E[jb], J.B[jb], bid);
    else
        compress_vec_body<T, 128>((const T *)J.Ca[jb], nullptr, (const T *)J.Za[jb], nullptr, nullptr, nullptr,
                                  J.bias[jb], J.n[jb], J.c[jb], (T *)J.out[jb], J.out_bstride[jb], J.E[jb], J.B[jb],
                                  bid);
}

// 16-byte row accesses need whole 16-byte channel groups and 16-byte aligned rows
bool vec_ok(const void *Ca, const void *Cb, const void *Za, const void *Zb, const void *cCb, const void *cZb, int c,
            int ratio, int overlap, csa_dtype dt, const void *out, int64_t out_bstride) {
    const int V = dt == CSA_F32 ? 4 : 8;
    auto al16 = [](const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return c % V == 0 && out_bstride % V == 0 && al16(Ca) && al16(Cb) && al16(Za) && al16(Zb) && al16(cCb) &&
           al16(cZb) && al16(out) && ((ratio == 4 && overlap == 1) || (ratio == 128 && overlap == 0));
}

int launch_compress(const void *Ca, const void *Cb, const void *Za, const void *Zb,
                    const void *cCb, const void *cZb, const float *bias, int B, int64_t n, int c,
                    int ratio, int overlap, csa_dtype dt, void *out, int64_t out_bstride,
                    hipStream_t st)
{
    const int64_t E = n / ratio;
    if (B == 0 || E == 0) return CSA_OK;
    if (out_bstride == 0) out_bstride = E * c;
    const int V = dt == CSA_F32 ? 4 : 8;
    if (vec_ok(Ca, Cb, Za, Zb, cCb, cZb, c, ratio, overlap, dt, out, out_bstride)) {
        const int64_t blocks = vec_blocks(B, E, c, V, ratio);
#define CSA_CVEC(T_, R_)                                                                                       \
    hipLaunchKernelGGL((compress_vec_kernel<T_, R_>), dim3((unsigned)blocks), dim3(256), 0, st, (const T_ *)Ca,  \
                       (const T_ *)Cb, (const T_ *)Za, (const T_ *)Zb, (const T_ *)cCb, (const T_ *)cZb, bias, n, c, \
                       (T_ *)out, out_bstride, E, B)
        if (dt == CSA_F32) {
            if (ratio == 4) CSA_CVEC(float, 4);
            else CSA_CVEC(float, 128);
        } else {
            if (ratio == 4) CSA_CVEC(bf16_t, 4);
            else CSA_CVEC(bf16_t, 128);
        }
#undef CSA_CVEC
        return check_launch("compress_vec_kernel");
    }
    // long pools: 16 slot groups of 8 slots (one batch of loads each) over 16 channels
    const int SG = ratio * (1 + overlap) >= 64 ? 16 : 1;
    const int CX = 256 / SG;
    const int ctiles = (c + CX - 1) / CX;
    const int64_t blocks = (int64_t)ctiles * E * B;
    dim3 grid((unsigned)blocks), block(CX, SG);
    if (dt == CSA_F32) {
        hipLaunchKernelGGL(compress_kernel<float>, grid, block, 0, st, (const float *)Ca,
                           (const float *)Cb, (const float *)Za, (const float *)Zb,
                           (const float *)cCb, (const float *)cZb, bias, n, c, ratio, overlap,
                           (float *)out, out_bstride, E, ctiles);
    } else {
        hipLaunchKernelGGL(compress_kernel<bf16_t>, grid, block, 0, st, (const bf16_t *)Ca,
                           (const bf16_t *)Cb, (const bf16_t *)Za, (const bf16_t *)Zb,
                           (const bf16_t *)cCb, (const bf16_t *)cZb, bias, n, c, ratio, overlap,
                           (bf16_t *)out, out_bstride, E, ctiles);
    }
    return check_launch("compress_kernel");
}

int launch_compress_batch(const CompressJobArgs *jobs, int njobs, csa_dtype dt, hipStream_t st) {
    if (njobs > kMaxCompressJobs) return fail(CSA_EUNSUPPORTED, "csa_compress_batch: at most 8 jobs");
    CompressJobs J{};
    int64_t blocks = 0;
    int nj = 0;
    bool all_vec = true;
    for (int i = 0; i < njobs; ++i) {
        const CompressJobArgs &a = jobs[i];
        const int64_t E = a.n / a.ratio;
        const int64_t ob = a.out_bstride == 0 ? E * a.c : a.out_bstride;
        if (a.B == 0 || E == 0) continue;
        all_vec = all_vec && vec_ok(a.Ca, a.Cb, a.Za, a.Zb, a.cCb, a.cZb, a.c, a.ratio, a.overlap, dt, a.out, ob);
        J.Ca[nj] = a.Ca; J.Cb[nj] = a.Cb; J.Za[nj] = a.Za; J.Zb[nj] = a.Zb; J.cCb[nj] = a.cCb; J.cZb[nj] = a.cZb;
        J.bias[nj] = a.bias; J.out[nj] = a.out; J.n[nj] = a.n; J.E[nj] = E; J.out_bstride[nj] = ob;
        J.c[nj] = a.c; J.ratio[nj] = a.ratio; J.B[nj] = a.B;
        J.first[nj] = blocks;
        blocks += vec_blocks(a.B, E, a.c, dt == CSA_F32 ? 4 : 8, a.ratio);
        ++nj;
    }
    if (nj == 0) return CSA_OK;
    if (!all_vec) {  // a job without 16-byte rows: one launch per job
        for (int i = 0; i < njobs; ++i) {
            const CompressJobArgs &a = jobs[i];
            const int rc = launch_compress(a.Ca, a.Cb, a.Za, a.Zb, a.cCb, a.cZb, a.bias, a.B, a.n, a.c, a.ratio,
                                           a.overlap, dt, a.out, a.out_bstride, st);
            if (rc != CSA_OK) return rc;
        }
        return CSA_OK;
    }
    J.first[nj] = blocks;
    J.njobs = nj;
    if (dt == CSA_F32)
        hipLaunchKernelGGL(compress_batch_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, J);
    else
        hipLaunchKernelGGL(compress_batch_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, J);
    return check_launch("compress_batch_kernel");
}

}  // namespace csa
