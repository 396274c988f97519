// Quantize + append into the FP4 main-KV cache.
//
// Format (FP4 KV cache paragraph of section 一 of the teardown "DeepSeek V4.1
// Flash 拆解", austincafe.tech): E2M1 codes with one E4M3 scale per 16
// channels.  Scale rule: E4M3(amax / 6), nearest-even, saturating; codes are
// the nearest E2M1 value to x / scale (ties to even, clipped at 6).
//
// One thread quantizes one 16-channel group: it reads the group's 32 (bf16)
// or 64 (fp32) contiguous bytes, so consecutive threads read consecutive
// bytes; it writes 8 code bytes and 1 scale byte.  No division is used:
// every decision is an exact fp32 comparison against a threshold with at most
// 7 significant bits.
#include "csa2_device.h"
#include "csa2_host.h"

namespace {

// Index of the E4M3 magnitude nearest to amax / 6, ties to the even code,
// saturating at code 126 (448): the number of grid midpoints that amax / 6
// passes, found by binary search.  6 * midpoint = 3 * (v_k + v_{k+1}) is
// exact in fp32.
__device__ __forceinline__ int scale_code(float amax)
{
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        float t = 3.0f * (e4m3_mag_value(mid) + e4m3_mag_value(mid + 1));
        bool up = amax > t || (amax == t && (mid & 1));
        if (up) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// E2M1 magnitude code (0..7) nearest to a / s, ties to even: count the
// midpoints {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} * s passed, where landing
// exactly on a midpoint moves up only when the upper neighbour is even.
__device__ __forceinline__ uint32_t e2m1_mag(float a, float s)
{
    uint32_t c = (a > 0.25f * s);
    c += (a >= 0.75f * s);
    c += (a > 1.25f * s);
    c += (a >= 1.75f * s);
    c += (a > 2.5f * s);
    c += (a >= 3.5f * s);
    c += (a > 5.0f * s);
    return c;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_quantize_append(const void* __restrict__ x, int32_t T,
                                                         int32_t D,
                                                         const int64_t* __restrict__ dst_row,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         int64_t cache_rows)
{
    const int G = D >> 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)T * G) return;
    const int64_t t = gid / G;
    const int g = (int)(gid - t * G);
    const int64_t r = dst_row[t];
    CSA2_DCHECK(g == 0 && (r < 0 || r >= cache_rows));
    if (r < 0 || r >= cache_rows) return;

    float v[16];
    if (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + t * D + g * 16);
        uint4 a = p[0], b = p[1];
        uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + t * D + g * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 f = p[i];
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int S = scale_code(amax);
    const float s = e4m3_mag_value(S);

    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t mag = (s == 0.0f) ? 0u : e2m1_mag(fabsf(v[i]), s);
        uint32_t c = mag | ((__float_as_uint(v[i]) >> 28) & 8u);
        if (i < 8) lo |= c << (4 * i);
        else hi |= c << (4 * (i - 8));
    }
    *reinterpret_cast<uint2*>(codes + r * (D >> 1) + g * 8) = make_uint2(lo, hi);
    scales[r * G + g] = (uint8_t)S;
}

}  // namespace

extern "C" csa2_status_t csa2_quantize_append(const void* x, int32_t x_dtype, int32_t T, int32_t D,
                                              const int64_t* dst_row, uint8_t* codes,
                                              uint8_t* scales, int64_t cache_rows, void* stream)
{
    CSA2_REQUIRE(T >= 0, CSA2_ERR_SHAPE, "quantize_append: T=%d < 0", T);
    CSA2_REQUIRE(D >= 16 && D % 16 == 0, CSA2_ERR_SHAPE, "quantize_append: D=%d must be a positive multiple of 16", D);
    CSA2_REQUIRE(D <= 8192, CSA2_ERR_UNSUPPORTED, "quantize_append: D=%d > 8192", D);
    CSA2_REQUIRE(cache_rows >= 0, CSA2_ERR_SHAPE, "quantize_append: cache_rows < 0");
    CSA2_REQUIRE(x_dtype == CSA2_F32 || x_dtype == CSA2_BF16, CSA2_ERR_UNSUPPORTED,
                 "quantize_append: x_dtype=%d is neither CSA2_F32 nor CSA2_BF16", x_dtype);
    if (T == 0) return CSA2_OK;
    CSA2_REQUIRE(x && dst_row && codes && scales, CSA2_ERR_NULL, "quantize_append: NULL pointer argument");
    const int64_t threads = (int64_t)T * (D / 16);
    const int64_t blocks = (threads + 255) / 256;
    CSA2_REQUIRE(blocks <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED, "quantize_append: too many rows");
    hipStream_t st = csa2::as_stream(stream);
    if (x_dtype == CSA2_BF16)
        hipLaunchKernelGGL(k_quantize_append<true>, dim3((unsigned)blocks), dim3(256), 0, st, x, T, D,
                           dst_row, codes, scales, cache_rows);
    else
        hipLaunchKernelGGL(k_quantize_append<false>, dim3((unsigned)blocks), dim3(256), 0, st, x, T, D,
                           dst_row, codes, scales, cache_rows);
    return CSA2_FINISH(st, "quantize_append");
}
