// RMSNorm of a row followed by RoPE on its last R dims, the step that the DeepSeek-V4 notes
// ("DeepSeek-V4 混合注意力" §6) put on the queries and on each compressed entry before it
// is cached: y = x / sqrt(mean(x^2) + eps) * g, then the interleaved pairs
// (D-R+2p, D-R+2p+1) of y turn by the caller's (cos, sin) of pair p.
//
// One wavefront per row of D = 64 * E elements; lane l holds the E consecutive elements
// [E*l, E*l + E), so every RoPE pair sits in one lane and a row moves as one coalesced
// 16-byte (bf16, D = 512) or wider access per lane; a wavefront takes 4 rows per pass and
// loads the next 4 into a second register set before it normalises these, so loads stay in
// flight behind the stores. The sum of squares is an fp32 lane sum and a DPP reduction across the
// wavefront. The pass is a pure HBM stream: D * (in + out) bytes per row plus the angle
// table row, which rows of one position share.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

constexpr int RW = 4;  // rows per wavefront per pass: their loads are all in flight together

// E consecutive elements of a row to fp32 (16-byte aligned rows: one vector access per lane)
template <int E, bool BF>
__device__ __forceinline__ void load_row(const void *base, int64_t off, float *v) {
    if constexpr (!BF) {
        const float *p = static_cast<const float *>(base) + off;
        if constexpr (E == 2) {
            const float2 a = *reinterpret_cast<const float2 *>(p);
            v[0] = a.x; v[1] = a.y;
        } else {
#pragma unroll
            for (int i = 0; i < E / 4; ++i) {
                const float4 a = reinterpret_cast<const float4 *>(p)[i];
                v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
            }
        }
    } else {
        const bf16_t *b = static_cast<const bf16_t *>(base) + off;
        uint32_t w[E / 2];
        if constexpr (E == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(b);
        } else if constexpr (E == 4) {
            const uint2 a = *reinterpret_cast<const uint2 *>(b);
            w[0] = a.x; w[1] = a.y;
        } else {
            const uint4 a = *reinterpret_cast<const uint4 *>(b);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        }
#pragma unroll
        for (int i = 0; i < E / 2; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}

template <int E, bool BF>
__device__ __forceinline__ void store_row(void *base, int64_t off, const float *v) {
    if constexpr (!BF) {
        float *p = static_cast<float *>(base) + off;
        if constexpr (E == 2) {
            *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
        } else {
#pragma unroll
            for (int i = 0; i < E / 4; ++i)
                reinterpret_cast<float4 *>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
    } else {
        bf16_t *b = static_cast<bf16_t *>(base) + off;
        uint32_t w[E / 2];
#pragma unroll
        for (int i = 0; i < E / 2; ++i)
            w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        if constexpr (E == 2) *reinterpret_cast<uint32_t *>(b) = w[0];
        else if constexpr (E == 4) *reinterpret_cast<uint2 *>(b) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<uint4 *>(b) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// sum over the wavefront, the same value in every lane: quad and row rotations by DPP, then
// the four row sums out of lanes 0, 16, 32, 48
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)); // row_ror:4
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)); // row_ror:8
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}

// The loads of a group: rows past the end re-read the last row (never stored), and every
// lane reads the (cos, sin) of its pairs' slots (a lane without rotated dims reads slot 0),
// so no load sits behind a branch and the waits stay exact.
template <int E, bool BF>
__device__ __forceinline__ void load_group(const void *x, const float *cs_base, int R, int64_t group, int p0,
                                           int64_t row0, int64_t rows, int d0, float (&v)[RW][E],
                                           float (&cs)[RW][E]) {
    constexpr int D = 64 * E;
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const int64_t r = row0 + k < rows ? row0 + k : rows - 1;
        load_row<E, BF>(x, r * D + d0, v[k]);
        // E floats at a multiple of E (16-byte aligned table): vector loads
        const float *c = cs_base + (r / group) * R + 2 * p0;
        if constexpr (E == 2) {
            const float2 a = *reinterpret_cast<const float2 *>(c);
            cs[k][0] = a.x; cs[k][1] = a.y;
        } else {
#pragma unroll
            for (int i = 0; i < E / 4; ++i) {
                const float4 a = reinterpret_cast<const float4 *>(c)[i];
                cs[k][4 * i] = a.x; cs[k][4 * i + 1] = a.y; cs[k][4 * i + 2] = a.z; cs[k][4 * i + 3] = a.w;
            }
        }
    }
}

// normalise, rotate and store one group of RW rows held in registers
template <int E, bool BO>
__device__ __forceinline__ void finish_group(float (&v)[RW][E], const float (&cs)[RW][E], int64_t row0,
                                             int64_t rows, int d0, int R, const float (&gv)[E], float eps,
                                             void *out) {
    constexpr int D = 64 * E;
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < E; ++j) ss = fmaf(v[k][j], v[k][j], ss);
        ss = wave_sum(ss);
        const float den2 = ss * (1.f / (float)D) + eps;  // D is a power of two: exact scaling
        const float inv = den2 > 0.f ? 1.f / sqrtf(den2) : 0.f;
#pragma unroll
        for (int j = 0; j < E; j += 2) {
            const float y0 = v[k][j] * inv * gv[j], y1 = v[k][j + 1] * inv * gv[j + 1];
            const bool r = d0 + j >= D - R;
            const float c = cs[k][j], s = cs[k][j + 1];
            v[k][j] = r ? y0 * c - y1 * s : y0;
            v[k][j + 1] = r ? y0 * s + y1 * c : y1;
        }
        if (row0 + k < rows) store_row<E, BO>(out, (row0 + k) * D + d0, v[k]);
    }
}

// Each wavefront walks row groups gridDim.x * 4 groups apart with two register sets: the
// next group's loads go out before the current group is finished, and the two sets take
// turns, so a wavefront always has a group of loads in flight behind its stores.
template <int E, bool BI, bool BO>
__global__ void __launch_bounds__(256)
rmsnorm_rope_kernel(const void *__restrict__ x, int64_t rows, const float *__restrict__ g, float eps,
                    const float *__restrict__ rope_cs, int R, int64_t group, void *__restrict__ out)
{
    constexpr int D = 64 * E;
    const int lane = threadIdx.x & 63;
    const int d0 = E * lane;
    float gv[E];
#pragma unroll
    for (int j = 0; j < E; ++j) gv[j] = g[d0 + j];
    // first (cos, sin) slot of this lane's elements: pair (d0 - (D - R)) / 2, or slot 0
    const int p0 = d0 >= D - R ? (d0 - (D - R)) >> 1 : 0;
    const int64_t stride = (int64_t)gridDim.x * 4 * RW;
    int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RW;
    float va[RW][E], vb[RW][E], ca[RW][E], cb[RW][E];
    load_group<E, BI>(x, rope_cs, R, group, p0, row0, rows, d0, va, ca);
    while (row0 < rows) {
        load_group<E, BI>(x, rope_cs, R, group, p0, row0 + stride, rows, d0, vb, cb);
        finish_group<E, BO>(va, ca, row0, rows, d0, R, gv, eps, out);
        row0 += stride;
        if (row0 >= rows) break;
        load_group<E, BI>(x, rope_cs, R, group, p0, row0 + stride, rows, d0, va, ca);
        finish_group<E, BO>(vb, cb, row0, rows, d0, R, gv, eps, out);
        row0 += stride;
    }
}

// workgroups of one instantiation that fit a compute unit at once (queried once)
template <int E, bool BI, bool BO>
int resident_per_cu() {
    static const int n = [] {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, reinterpret_cast<const void *>(rmsnorm_rope_kernel<E, BI, BO>),
                                                         256, 0) != hipSuccess || b <= 0)
            b = 2;
        return b;
    }();
    return n;
}

template <int E, bool BI, bool BO>
void launch_one(const void *x, int64_t rows, const float *g, float eps, const float *cs, int R, int64_t group,
                void *out, hipStream_t st) {
    // no more workgroups than the chip holds at once: each streams many row groups, and a
    // second wave of workgroups would run on a fraction of the chip
    int64_t blocks = (rows + 4 * RW - 1) / (4 * RW);
    const int cu = device_cu_count();
    const int64_t resident = (int64_t)(cu > 0 ? cu : 256) * resident_per_cu<E, BI, BO>();
    if (blocks > resident) blocks = resident;
    hipLaunchKernelGGL((rmsnorm_rope_kernel<E, BI, BO>), dim3((unsigned)blocks), dim3(256), 0, st, x, rows, g, eps,
                       cs, R, group, out);
}

template <int E>
void launch_e(const void *x, bool bi, int64_t rows, const float *g, float eps, const float *cs, int R,
              int64_t group, void *out, bool bo, hipStream_t st) {
    if (bi && bo) launch_one<E, true, true>(x, rows, g, eps, cs, R, group, out, st);
    else if (bi) launch_one<E, true, false>(x, rows, g, eps, cs, R, group, out, st);
    else if (bo) launch_one<E, false, true>(x, rows, g, eps, cs, R, group, out, st);
    else launch_one<E, false, false>(x, rows, g, eps, cs, R, group, out, st);
}

}  // namespace

int launch_rmsnorm_rope(const void *x, csa_dtype dt_in, int64_t rows, int D, const float *g, float eps,
                        const float *rope_cs, int R, int64_t group, void *out, csa_dtype dt_out, hipStream_t st) {
    // without rotation the (cos, sin) reads go to the gains (any readable pair; never used)
    const float *cs = R > 0 ? rope_cs : g;
    const bool bi = dt_in == CSA_BF16, bo = dt_out == CSA_BF16;
    switch (D) {
        case 128: launch_e<2>(x, bi, rows, g, eps, cs, R, group, out, bo, st); break;
        case 256: launch_e<4>(x, bi, rows, g, eps, cs, R, group, out, bo, st); break;
        default: launch_e<8>(x, bi, rows, g, eps, cs, R, group, out, bo, st); break;
    }
    return check_launch("rmsnorm_rope_kernel");
}

}  // namespace csa
