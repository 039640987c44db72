// MXFP4 encoding of indexer operands on gfx950, with the optional Hadamard rotation in
// front of it (the DeepSeek-V4-Pro-MXFP4 page, Indexer section: the query passes through
// RoPE and a Hadamard rotation before the FP4 index dot products; the same orthonormal
// rotation on the keys leaves every exact score unchanged).
//
// One wavefront per row of D = 64 * E elements; lane l holds the E consecutive elements
// [E*l, E*l + E). The Walsh-Hadamard butterflies (a + b, a - b) on pairs (i, i + h) run
// in registers for h < E and across lanes (partner lane l ^ (h / E)) above, in fp32, in
// the order h = 1, 2, .., D/2, then one multiply by the fp32 value of 1/sqrt(D). Each
// block of 32 elements (32 / E lanes) takes its E8M0 exponent from the bits of its largest
// magnitude (OCP Microscaling v1.0: floor(log2(amax)) - 2) and each element the nearest
// E2M1 code by exact comparisons against the midpoints of the grid.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

template <int E>
__global__ void __launch_bounds__(256)
quantize_mxfp4_kernel(const void *__restrict__ x, int64_t rows, csa_dtype dt, int hadamard, float inv_sqrt_d,
                      uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, int64_t group_rows,
                      int64_t group_stride)
{
    constexpr int D = 64 * E;
    constexpr int LPB = 32 / E;  // lanes per 32-element block
    const int lane = threadIdx.x & 63;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4) {
        float v[E];
        if (dt == CSA_F32) {
            const float *src = static_cast<const float *>(x) + row * D + E * lane;
#pragma unroll
            for (int j = 0; j < E; ++j) v[j] = src[j];
        } else {
            const bf16_t *src = static_cast<const bf16_t *>(x) + row * D + E * lane;
#pragma unroll
            for (int j = 0; j < E; ++j) v[j] = bf16_to_f32(src[j]);
        }
        if (hadamard) {
#pragma unroll
            for (int h = 1; h < E; h <<= 1)
#pragma unroll
                for (int j = 0; j < E; ++j)
                    if (!(j & h)) {
                        const float a = v[j], b = v[j + h];
                        v[j] = a + b;
                        v[j + h] = a - b;
                    }
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const bool upper = (lane & m) != 0;
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const float p = __shfl_xor(v[j], m);
                    v[j] = upper ? p - v[j] : v[j] + p;  // (lower + upper, lower - upper)
                }
            }
#pragma unroll
            for (int j = 0; j < E; ++j) v[j] *= inv_sqrt_d;
        }
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
        for (int m = 1; m < LPB; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
        const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
        const int es = ex == 0 ? -127 : (ex - 129 < -127 ? -127 : ex - 129);
        uint32_t nib[E];
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float m = ldexpf(fabsf(v[j]), -es);
            uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                         (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.f);
            if (v[j] < 0.f && c != 0u) c |= 8u;
            nib[j] = c;
        }
        uint32_t packed = 0u;
#pragma unroll
        for (int j = 0; j < E; ++j) packed |= nib[j] << (4 * j);
        const int64_t orow = group_rows > 0 ? (row / group_rows) * group_stride + row % group_rows : row;
        uint8_t *dst = codes + orow * (D / 2) + (E / 2) * lane;
        if (E == 2) *dst = (uint8_t)packed;
        else if (E == 4) *reinterpret_cast<uint16_t *>(dst) = (uint16_t)packed;
        else *reinterpret_cast<uint32_t *>(dst) = packed;
        if (lane % LPB == 0) scales[orow * (D / 32) + lane / LPB] = (uint8_t)(es + 127);
    }
}

}  // namespace

int launch_quantize_mxfp4(const void *x, int64_t rows, int D, csa_dtype dt, bool hadamard, uint8_t *codes,
                          uint8_t *scales, int64_t group_rows, int64_t group_stride, hipStream_t st) {
    const float inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
    int64_t blocks = (rows + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid((unsigned)blocks);
    switch (D) {
        case 128:
            hipLaunchKernelGGL(quantize_mxfp4_kernel<2>, grid, dim3(256), 0, st, x, rows, dt, (int)hadamard,
                               inv_sqrt_d, codes, scales, group_rows, group_stride);
            break;
        case 256:
            hipLaunchKernelGGL(quantize_mxfp4_kernel<4>, grid, dim3(256), 0, st, x, rows, dt, (int)hadamard,
                               inv_sqrt_d, codes, scales, group_rows, group_stride);
            break;
        default:
            hipLaunchKernelGGL(quantize_mxfp4_kernel<8>, grid, dim3(256), 0, st, x, rows, dt, (int)hadamard,
                               inv_sqrt_d, codes, scales, group_rows, group_stride);
            break;
    }
    return check_launch("quantize_mxfp4_kernel");
}

}  // namespace csa
