// Drives the host side of the CSA2 library (argument validation, workspace
// queries, status strings, the thread-local error message) with arguments
// that fail every check, at the extremes of every size, so that a build with
// AddressSanitizer and UndefinedBehaviorSanitizer checks that code.  No call
// here reaches a kernel launch: each one fails validation, or has nothing to
// do (R = 0), before any HIP call.  Exit status 0 and "abi ok" on success.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <climits>

#include "../../include/csa2.h"

static int failures = 0;
#define EXPECT(call, want)                                                                                \
    do {                                                                                                  \
        const int got_ = (int)(call);                                                                     \
        if (got_ != (want)) {                                                                             \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, (want), \
                    csa2_last_error());                                                                   \
            ++failures;                                                                                   \
        }                                                                                                 \
    } while (0)

int main()
{
    void* F = reinterpret_cast<void*>(0x1000);   // never dereferenced
    const uint8_t* u8 = static_cast<const uint8_t*>(F);
    const float* f32 = static_cast<const float*>(F);
    const int64_t* i64 = static_cast<const int64_t*>(F);
    const int32_t* i32 = static_cast<const int32_t*>(F);
    int32_t* o32 = static_cast<int32_t*>(F);
    float* of = static_cast<float*>(F);
    const uint16_t* u16 = static_cast<const uint16_t*>(F);
    uint8_t* o8 = static_cast<uint8_t*>(F);

    for (int s = -3; s < 10; ++s) {
        const char* name = csa2_status_string(static_cast<csa2_status_t>(s));
        if (!name || !*name) ++failures;
    }
    EXPECT(csa2_abi_version(), CSA2_ABI_VERSION);
    EXPECT(strlen(csa2_last_error()) < 512, 1);

    // quantize-append
    EXPECT(csa2_quantize_append(F, CSA2_BF16, INT_MIN, 512, i64, o8, o8, 10, nullptr), CSA2_ERR_SHAPE);
    EXPECT(csa2_quantize_append(F, CSA2_BF16, 4, INT_MAX, i64, o8, o8, 10, nullptr), CSA2_ERR_SHAPE);
    EXPECT(csa2_quantize_append(F, CSA2_BF16, 4, INT_MIN, i64, o8, o8, 10, nullptr), CSA2_ERR_SHAPE);
    EXPECT(csa2_quantize_append(F, 99, 4, 512, i64, o8, o8, 10, nullptr), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_quantize_append(F, CSA2_F32, 4, 512, i64, o8, o8, -1, nullptr), CSA2_ERR_SHAPE);
    EXPECT(csa2_quantize_append(nullptr, CSA2_F32, 4, 512, i64, o8, o8, 10, nullptr), CSA2_ERR_NULL);
    EXPECT(csa2_quantize_append(F, CSA2_F32, INT_MAX, 8192, i64, o8, o8, 10, nullptr), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_quantize_append(nullptr, CSA2_F32, 0, 512, nullptr, nullptr, nullptr, 0, nullptr), CSA2_OK);

    // workspace queries at the extremes of their arguments
    const int32_t ext[] = {INT_MIN, -1, 0, 1, 7, 65535, 65536, INT_MAX};
    size_t sink = 0;
    for (int32_t a : ext)
        for (int32_t b : ext) {
            sink += csa2_index_full_workspace_bytes(a, b, 64, 512, 2048, 8);
            sink += csa2_index_full_workspace_bytes(a, b, b, a, b, a);
            sink += csa2_index_reindex_workspace_bytes(a, 64, b, b, 8);
            sink += csa2_sparse_attn_workspace_bytes(a, b, 512, 512, 128);
            sink += csa2_sparse_attn_workspace_bytes(a, 64, b, a, b);
        }
    EXPECT(csa2_index_full_workspace_bytes(-1, 100, 64, 512, 2048, 8), 0);
    (void)sink;

    // Full index: every size check
    auto full = [&](int32_t R, int32_t Hi, int32_t Di, int32_t max_len, int32_t K, int32_t P, int32_t block,
                    int32_t* pool, size_t wsb, void* ws) {
        return csa2_index_full(u8, f32, u8, i64, i32, i32, R, Hi, Di, max_len, K, P, block, o32, pool, ws, wsb,
                               nullptr);
    };
    const size_t big = (size_t)1 << 40;
    EXPECT(full(2, 64, 128, 100, 0, 2048, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(2, 64, 128, 100, INT_MAX, 2048, 8, o32, big, F), CSA2_ERR_UNSUPPORTED);
    EXPECT(full(2, 64, 128, 100, 512, INT_MIN, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(2, INT_MAX, 128, 100, 512, 2048, 8, o32, big, F), CSA2_ERR_UNSUPPORTED);
    EXPECT(full(2, INT_MIN, 128, 100, 512, 2048, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(2, 64, INT_MIN, 100, 512, 2048, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(2, 64, INT_MAX, 100, 512, 2048, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(2, 64, 128, INT_MAX, 512, 2048, 8, o32, big, F), CSA2_ERR_UNSUPPORTED);
    EXPECT(full(2, 64, 128, INT_MIN, 512, 2048, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(INT_MAX, 64, 128, 100, 512, 2048, 8, o32, big, F), CSA2_ERR_UNSUPPORTED);
    EXPECT(full(INT_MIN, 64, 128, 100, 512, 2048, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(2, 64, 128, 100, 512, 2048, INT_MAX, o32, big, F), CSA2_ERR_UNSUPPORTED);
    EXPECT(full(2, 64, 128, 100, 512, 2048, 8, o32, 0, F), CSA2_ERR_WORKSPACE);
    EXPECT(full(2, 64, 128, 100, 512, 2048, 8, o32, big, reinterpret_cast<void*>(0x1004)), CSA2_ERR_WORKSPACE);
    EXPECT(full(2, 64, 128, 100, 512, 0, 8, o32, big, F), CSA2_ERR_SHAPE);
    EXPECT(full(0, 64, 128, 100, 512, 2048, 8, o32, 0, nullptr), CSA2_OK);
    EXPECT(csa2_index_full(nullptr, f32, u8, i64, i32, i32, 2, 64, 128, 100, 512, 2048, 8, o32, o32, F, big,
                           nullptr),
           CSA2_ERR_NULL);
    EXPECT(csa2_index_full(u8, f32, u8, nullptr, i32, i32, 2, 64, 128, 100, 512, 2048, 8, o32, o32, F, big,
                           nullptr),
           CSA2_ERR_NULL);

    // Reindex
    auto reidx = [&](int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t P, size_t wsb) {
        return csa2_index_reindex(u8, f32, u8, i64, i32, i32, i32, R, Hi, Di, K, P, 8, o32, F, wsb, nullptr);
    };
    EXPECT(reidx(2, 64, 128, 512, INT_MAX, big), CSA2_ERR_UNSUPPORTED);
    EXPECT(reidx(2, 64, 128, 512, INT_MIN, big), CSA2_ERR_SHAPE);
    EXPECT(reidx(2, 64, 128, INT_MIN, 2048, big), CSA2_ERR_SHAPE);
    EXPECT(reidx(INT_MAX, 64, 128, 512, 2048, big), CSA2_ERR_UNSUPPORTED);
    EXPECT(reidx(2, 64, 128, 512, 2048, 3), CSA2_ERR_WORKSPACE);
    EXPECT(reidx(0, 64, 128, 512, 2048, 0), CSA2_OK);

    // attention
    auto attn = [&](int32_t R, int32_t H, int32_t D, int32_t K, int32_t W, size_t wsb) {
        return csa2_sparse_attn(u16, u8, u8, i64, i32, i32, i32, K, u8, i64, i32, R, H, D, W, 0.04f, of, nullptr,
                                F, wsb, nullptr);
    };
    EXPECT(attn(32, INT_MAX, 512, 512, 128, big), CSA2_ERR_UNSUPPORTED);
    EXPECT(attn(32, INT_MIN, 512, 512, 128, big), CSA2_ERR_SHAPE);
    EXPECT(attn(32, 64, INT_MAX, 512, 128, big), CSA2_ERR_SHAPE);
    EXPECT(attn(32, 64, 1024, 512, 128, big), CSA2_ERR_UNSUPPORTED);
    EXPECT(attn(32, 64, 512, INT_MAX, 128, big), CSA2_ERR_UNSUPPORTED);
    EXPECT(attn(32, 64, 512, 512, INT_MIN, big), CSA2_ERR_SHAPE);
    EXPECT(attn(INT_MAX, 64, 512, 512, 128, big), CSA2_ERR_UNSUPPORTED);
    EXPECT(attn(INT_MIN, 64, 512, 512, 128, big), CSA2_ERR_SHAPE);
    EXPECT(attn(0, 64, 512, 512, 128, 0), CSA2_OK);
    EXPECT(csa2_sparse_attn_phys(u16, u8, u8, 0, i32, 512, u8, i64, i32, nullptr, 2, 64, 512, 128, 0.04f, of,
                                 nullptr, F, big, nullptr),
           CSA2_ERR_SHAPE);
    EXPECT(csa2_sparse_attn_phys(u16, u8, u8, INT64_MAX, i32, 512, u8, i64, i32, nullptr, INT_MAX, 64, 512, 128,
                                 0.04f, of, nullptr, F, big, nullptr),
           CSA2_ERR_UNSUPPORTED);

    // paged calls and row translation
    EXPECT(csa2_paged_rows(i32, 64, 3, 100, i32, i32, i32, 4, 512, o32, nullptr), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_paged_rows(i32, 64, 1 << 30, 100, i32, i32, i32, 4, 512, o32, nullptr), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_paged_rows(i32, INT_MIN, 64, 100, i32, i32, i32, 4, 512, o32, nullptr), CSA2_ERR_SHAPE);
    EXPECT(csa2_paged_rows(i32, 64, 64, INT64_MIN, i32, i32, i32, 4, 512, o32, nullptr), CSA2_ERR_SHAPE);
    EXPECT(csa2_paged_rows(i32, 64, 64, 100, i32, i32, i32, INT_MAX, INT_MAX, o32, nullptr), CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_paged_rows(i32, 64, 64, 100, i32, i32, i32, 0, 512, nullptr, nullptr), CSA2_OK);
    EXPECT(csa2_index_full_paged(u8, f32, u8, 100, i32, 64, 48, i32, i32, 2, 64, 128, 100, 512, 2048, 8, o32,
                                 nullptr, o32, F, big, nullptr),
           CSA2_ERR_UNSUPPORTED);
    EXPECT(csa2_index_reindex_paged(u8, f32, u8, 100, nullptr, 64, 64, i32, i32, i32, 2, 64, 128, 512, 2048, 8,
                                    o32, nullptr, F, big, nullptr),
           CSA2_ERR_NULL);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("abi ok\n");
    return 0;
}
