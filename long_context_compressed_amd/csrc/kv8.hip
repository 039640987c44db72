// FP8 storage of compressed KV rows on gfx950 ("DeepSeek-V4 混合注意力" §4.2, last
// paragraph: the RoPE-related dims of the compressed representation stay in BF16, the rest
// is stored in FP8), in the OCP Microscaling v1.0 MXFP8 form for the non-RoPE dims.
//
// A 512-dim row becomes 592 bytes: 448 E4M3 codes (dims 0..447), the 64 RoPE dims as bf16
// (bytes 448..575), 14 E8M0 scales, one per 32 codes (bytes 576..589), 2 zero bytes.
// Block scale exponent e = floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), clamped to
// [-127, 127] (-127 for an all-zero block); element code = the finite E4M3 value nearest to
// |x| / 2^e, ties to the even code, saturating at 448, with the sign of x unless 0.
//
// One wavefront per row: lanes 0..55 encode 8 consecutive dims each (four lanes per block
// of 32 share its maximum through lane swaps), lanes 56..63 round the 8 RoPE dims each to
// bf16; every lane writes its bytes with one store.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

constexpr int kD = 512, kR = 64, kQ = kD - kR;

// E4M3 code of |x| / 2^e (RNE, saturating at 448), with x's sign unless the code is 0
__device__ __forceinline__ uint32_t e4m3_code(float x, int e) {
    const float v = __builtin_ldexpf(__builtin_fabsf(x), -e);
    uint32_t code;
    if (!(v < 464.f)) {
        code = 0x7Eu;  // 448: everything from the midpoint to the next (absent) value up
    } else if (v < 0.015625f) {
        code = (uint32_t)__builtin_rintf(v * 512.f);  // subnormal steps of 2^-9; 8 is 2^-6 = code 8
    } else {
        int E = __builtin_amdgcn_frexp_expf(v) - 1;  // floor(log2 v): v = m 2^(E+1), m in [0.5, 1)
        const float mant = __builtin_ldexpf(v, -E);
        int mm = (int)__builtin_rintf((mant - 1.f) * 8.f);
        if (mm == 8) {
            ++E;
            mm = 0;
        }
        code = (uint32_t)(((E + 7) << 3) | mm);
    }
    if (code != 0u && __builtin_signbit(x)) code |= 0x80u;
    return code;
}

template <typename ET>
__global__ void __launch_bounds__(256)
quantize_kv8_kernel(const ET *__restrict__ x, int64_t rows, uint8_t *__restrict__ out, int64_t group_rows,
                    int64_t group_stride)
{
    const int lane = threadIdx.x & 63;
    for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += (int64_t)gridDim.x * 4) {
        const ET *xr = x + r * kD;
        const int64_t orow = group_rows > 0 ? (r / group_rows) * group_stride + r % group_rows : r;
        uint8_t *o = out + orow * kKv8RowBytes;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = elem<ET>::load(xr, 8 * lane + i);
        if (lane < kQ / 8) {
            float am = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(v[i]));
            am = fmaxf(am, __shfl_xor(am, 1));
            am = fmaxf(am, __shfl_xor(am, 2));  // the block of 32: lanes 4b .. 4b+3
            int e = (am > 0.f) ? (__builtin_amdgcn_frexp_expf(am) - 1) - 8 : -127;
            e = e < -127 ? -127 : (e > 127 ? 127 : e);
            uint32_t lo = 0u, hi = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo |= e4m3_code(v[i], e) << (8 * i);
                hi |= e4m3_code(v[4 + i], e) << (8 * i);
            }
            *reinterpret_cast<uint2 *>(o + 8 * lane) = make_uint2(lo, hi);
            if ((lane & 3) == 0) o[kQ + 2 * kR + lane / 4] = (uint8_t)(e + 127);
            if (lane == 0) *reinterpret_cast<uint16_t *>(o + kQ + 2 * kR + kQ / 32) = 0;
        } else {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
            *reinterpret_cast<uint4 *>(o + kQ + 16 * (lane - kQ / 8)) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

}  // namespace

int launch_quantize_kv8(const void *x, int64_t rows, csa_dtype dt, uint8_t *out, int64_t group_rows,
                        int64_t group_stride, hipStream_t st) {
    if (rows == 0) return CSA_OK;
    const int64_t blocks64 = (rows + 3) / 4;
    const unsigned blocks = (unsigned)(blocks64 < 65536 ? blocks64 : 65536);
    if (dt == CSA_F32)
        hipLaunchKernelGGL(quantize_kv8_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float *)x, rows, out,
                           group_rows, group_stride);
    else
        hipLaunchKernelGGL(quantize_kv8_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t *)x, rows, out,
                           group_rows, group_stride);
    return check_launch("quantize_kv8_kernel");
}

}  // namespace csa
