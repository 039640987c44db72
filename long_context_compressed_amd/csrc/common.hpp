// Shared device/host helpers of the gfx950 CSA / HCA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/csa.h"

namespace csa {

// ---- error state (thread-local detail string behind csa_last_error) ----------------
void set_error(const std::string &msg);
void clear_error();
int fail(int status, const std::string &msg);
int check_launch(const char *what);

// ---- scalar types ------------------------------------------------------------------
typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

// round-to-nearest-even fp32 -> bf16 (inputs here are finite or +-inf)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (bf16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// low / high bf16 of a packed 32-bit word, widened to fp32
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> struct elem;
template <> struct elem<float> {
    __device__ __forceinline__ static float load(const float *p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(bf16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// bytes of one compressed KV row in the FP8 storage format (512 dims: 448 E4M3 codes, 64
// bf16 RoPE dims, 14 E8M0 scales, 2 zero bytes)
constexpr int kKv8RowBytes = 592;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace csa
