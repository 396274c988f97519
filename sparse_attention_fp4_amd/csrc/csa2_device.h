// Device-side helpers shared by the CSA2 HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 lds_f16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));

#define CSA2_WAVE 64

// Value of a non-negative OCP E4M3 magnitude code (0..126), exact in fp32.
__device__ __forceinline__ float e4m3_mag_value(int b)
{
    int e = b >> 3, m = b & 7;
    return e == 0 ? (float)m * 0x1p-9f : __uint_as_float((uint32_t)((e + 120) << 23) | (uint32_t)(m << 20));
}

// Full OCP E4M3 byte -> fp32 (exact; the NaN codes are never produced here).
__device__ __forceinline__ float e4m3_to_f32(uint32_t bits)
{
    float v = e4m3_mag_value((int)(bits & 0x7F));
    return (bits & 0x80) ? -v : v;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, CSA2_WAVE); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (CSA2_WAVE - 1)); }
