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

#include "csa2_host.h"

// Debug builds (-DCSA2_DEBUG): each translation unit counts, in a device word
// of its own, the out-of-range values that its kernels skip (CSA2_DCHECK), and
// an entry point ends with CSA2_FINISH, which then waits for the stream, reads
// and clears the count, and returns CSA2_ERR_DEVICE_CHECK when it is not zero.
// Release builds compile the checks away and CSA2_FINISH only checks the
// launch status.
#ifdef CSA2_DEBUG
static __device__ unsigned int csa2_dbg_skipped;
#define CSA2_DCHECK(bad) do { if (bad) atomicAdd(&csa2_dbg_skipped, 1u); } while (0)
static inline csa2_status_t csa2_debug_finish(hipStream_t st, const char* who)
{
    const csa2_status_t ls = ::csa2::check_launch(who);
    if (ls != CSA2_OK) return ls;
    if (hipStreamSynchronize(st) != hipSuccess)
        return ::csa2::fail(CSA2_ERR_LAUNCH, "%s: stream synchronisation failed (debug build)", who);
    unsigned int c = 0, z = 0;
    if (hipMemcpyFromSymbol(&c, HIP_SYMBOL(csa2_dbg_skipped), sizeof c, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return ::csa2::fail(CSA2_ERR_LAUNCH, "%s: reading the device check count failed", who);
    if (c == 0) return CSA2_OK;
    if (hipMemcpyToSymbol(HIP_SYMBOL(csa2_dbg_skipped), &z, sizeof z, 0, hipMemcpyHostToDevice) != hipSuccess)
        return ::csa2::fail(CSA2_ERR_LAUNCH, "%s: clearing the device check count failed", who);
    return ::csa2::fail(CSA2_ERR_DEVICE_CHECK, "%s: kernels skipped %u out-of-range values in device memory", who,
                        c);
}
#define CSA2_FINISH(st, who) csa2_debug_finish((st), (who))
#else
#define CSA2_DCHECK(bad) ((void)0)
#define CSA2_FINISH(st, who) ::csa2::check_launch(who)
#endif

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

// Reductions between lanes 16 (32) apart without an LDS round trip:
// v_permlane16_swap(x, x) hands each lane of an even 16-lane row, in its
// second result, the value of the lane 16 above (and each lane of an odd row,
// in its first result, the value 16 below), while the other result keeps the
// lane's own value; v_permlane32_swap does the same for the two halves of the
// wave.  So op(first, second) is op(own, partner) in every lane.
__device__ __forceinline__ float max_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t umax_xor16(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return r[0] > r[1] ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t umax_xor32(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] > r[1] ? r[0] : r[1];
}
// Max over aligned groups of 8 lanes with DPP: quad permutations [1,0,3,2] and
// [2,3,0,1], then the mirror within each half row (lane i <-> 7 - i, which
// lies in the other quad of the same 8 lanes).
__device__ __forceinline__ float max_over8(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
}
__device__ __forceinline__ float sum_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (CSA2_WAVE - 1)); }
