// Token-level KV compressor on gfx950.
//
// "DeepSeek-V4 混合注意力" §4.1 (ratio 4: one per-channel softmax over the b-branch rows
// of block i-1 and the a-branch rows of block i) and §5 (ratio 128: one per-channel
// softmax over the rows of block i).
//
// HBM-bound: every input row is read once. A block owns one compressed entry and a
// tile of channels; lanes run along the channels (coalesced row reads) and, for the
// 128-row pool, the rows are split over `SG` slot groups whose running
// (max, denominator, numerator) states merge in LDS.
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

int launch_compress(const void *Ca, const void *Cb, const void *Za, const void *Zb,
                    const void *cCb, const void *cZb, const float *bias, int B, int64_t n, int c,
                    int ratio, int overlap, csa_dtype dt, void *out, int64_t out_bstride,
                    hipStream_t st)
{
    const int64_t E = n / ratio;
    if (B == 0 || E == 0) return CSA_OK;
    // long pools: 16 slot groups of 8 slots (one batch of loads each) over 16 channels
    const int SG = ratio * (1 + overlap) >= 64 ? 16 : 1;
    const int CX = 256 / SG;
    const int ctiles = (c + CX - 1) / CX;
    const int64_t blocks = (int64_t)ctiles * E * B;
    if (out_bstride == 0) out_bstride = E * c;
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

}  // namespace csa
