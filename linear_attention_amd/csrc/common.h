// Device helpers shared by the seg_la kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {


typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// bfloat16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element loads/stores for the two I/O element types.
template <typename T> struct io;

template <> struct io<uint16_t> {  // bf16 stored as raw bits
    __device__ static float ld(const uint16_t *p) { return bf16_to_f32(*p); }
    __device__ static void st(uint16_t *p, float x) { *p = f32_to_bf16(x); }
};

template <> struct io<float> {
    __device__ static float ld(const float *p) { return *p; }
    __device__ static void st(float *p, float x) { *p = x; }
};

}  // namespace la
