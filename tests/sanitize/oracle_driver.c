/*
 * Drives every entry point of the CPU oracle (oracle/csa2_oracle.c) on small
 * inputs that reach its edge paths — saturating, zero and negative-zero
 * groups, out-of-range destinations, empty and ragged rows, short rows with K
 * above n, pools holding -1 and out-of-range ids, index lists with -1 and
 * out-of-range ids, empty and partial windows — so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer checks its memory accesses
 * and arithmetic.  Each result is also checked against a property that holds
 * by definition (ascending, -1 padded lists; Top-K inside the pool when
 * P >= K; a single key attends to itself).  Exit status 0 and "oracle ok" on
 * success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double csa2_ref_e2m1_value(int code);
double csa2_ref_e4m3_value(int bits);
int csa2_ref_e4m3_encode(double v);
int csa2_ref_quantize_append(const void* x, int dtype, int32_t T, int32_t D, const int64_t* dst_row,
                             uint8_t* codes, uint8_t* scales, int64_t cache_rows);
int csa2_ref_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t D, double* out);
int csa2_ref_index_scores(const uint8_t* qI, const float* w, const uint8_t* ikeys, const int64_t* seq_start,
                          const int32_t* row_seq, const int32_t* row_len, int32_t R, int32_t Hi, int32_t Di,
                          int32_t max_len, float* scores);
int csa2_ref_index_full(const uint8_t* qI, const float* w, const uint8_t* ikeys, const int64_t* seq_start,
                        const int32_t* row_seq, const int32_t* row_len, int32_t R, int32_t Hi, int32_t Di,
                        int32_t max_len, int32_t K, int32_t P, int32_t block, int32_t* topk_idx,
                        int32_t* pool_blocks);
int csa2_ref_index_reindex(const uint8_t* qI, const float* w, const uint8_t* ikeys, const int64_t* seq_start,
                           const int32_t* row_seq, const int32_t* row_len, const int32_t* pool_blocks, int32_t R,
                           int32_t Hi, int32_t Di, int32_t K, int32_t P, int32_t block, int32_t* topk_idx);
int csa2_ref_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* seq_start,
                         const int32_t* row_seq, const int32_t* row_len, const int32_t* topk_idx, int32_t K,
                         const uint8_t* swa, const int64_t* swa_row_start, const int32_t* swa_len, int32_t R,
                         int32_t H, int32_t D, int32_t W, float softmax_scale, float* out, float* lse,
                         const uint8_t* rows_mask);
int csa2_ref_dense_attn(const uint16_t* q, const double* kv, const int64_t* seq_start, const int32_t* row_seq,
                        const int32_t* row_len, const double* swa_vals, const int64_t* swa_row_start,
                        const int32_t* swa_len, int32_t R, int32_t H, int32_t D, double scale, double* out);

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++failures; } \
    } while (0)

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 33);
}
static double unif(void) { return (rnd() + 0.5) / 2147483648.0; }
static double gauss(void) { return sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif()); }
static uint8_t int3_e4m3(void)
{
    static const uint8_t v[7] = {0xC4, 0xC0, 0xB8, 0x00, 0x38, 0x40, 0x44};   /* -3 .. 3 in E4M3 */
    return v[rnd() % 7];
}

/* ascending valid ids, then only -1 */
static int list_ok(const int32_t* a, int K, int limit)
{
    int k = 0;
    while (k < K && a[k] >= 0) {
        if (a[k] >= limit || (k > 0 && a[k] <= a[k - 1])) return 0;
        ++k;
    }
    for (; k < K; ++k)
        if (a[k] != -1) return 0;
    return 1;
}

static void formats(void)
{
    for (int c = 0; c < 16; ++c) CHECK(isfinite(csa2_ref_e2m1_value(c)));
    for (int b = 0; b < 256; ++b) {
        double v = csa2_ref_e4m3_value(b);
        if ((b & 0x7F) == 0x7F) continue;
        CHECK(isfinite(v));
        if (!(b & 0x80)) CHECK(csa2_ref_e4m3_encode(v) == b);
    }
    CHECK(csa2_ref_e4m3_encode(1e9) == 0x7E);
    CHECK(csa2_ref_e4m3_encode(0.0) == 0);
}

static void quantize(void)
{
    enum { T = 7, D = 64, ROWS = 6 };
    float x[T * D];
    for (int i = 0; i < T * D; ++i) x[i] = (float)gauss();
    for (int c = 0; c < D; ++c) {
        x[1 * D + c] = 0.0f;                  /* an all-zero row */
        x[2 * D + c] = -0.0f;                 /* negative zeros */
        x[3 * D + c] = (c & 1) ? 1e6f : -3e5f;   /* saturating scale */
        x[4 * D + c] = (float)(c % 16) * 1e-7f;  /* scales in the subnormal range */
    }
    int64_t dst[T] = {0, 1, 2, 3, 4, -1, 99};   /* the last two are skipped */
    uint8_t codes[ROWS * D / 2], scales[ROWS * D / 16];
    memset(codes, 0xAB, sizeof codes);
    memset(scales, 0xAB, sizeof scales);
    CHECK(csa2_ref_quantize_append(x, 0, T, D, dst, codes, scales, ROWS) == 0);
    CHECK(codes[5 * D / 2] == 0xAB && scales[5 * D / 16] == 0xAB);   /* row 5 untouched */
    for (int g = 0; g < D / 16; ++g) CHECK(scales[1 * D / 16 + g] == 0 && scales[3 * D / 16 + g] == 0x7E);
    double deq[ROWS * D];
    CHECK(csa2_ref_dequant_rows(codes, scales, ROWS, D, deq) == 0);
    for (int c = 0; c < D; ++c) CHECK(deq[1 * D + c] == 0.0 && fabs(deq[3 * D + c]) == 2688.0);
    /* bf16 input of the same values */
    uint16_t xb[T * D];
    for (int i = 0; i < T * D; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        xb[i] = (uint16_t)(u >> 16);
    }
    CHECK(csa2_ref_quantize_append(xb, 1, T, D, dst, codes, scales, ROWS) == 0);
    CHECK(csa2_ref_quantize_append(x, 0, T, 24, dst, codes, scales, ROWS) < 0);   /* D not a multiple of 16 */
    x[3] = NAN;
    CHECK(csa2_ref_quantize_append(x, 0, T, D, dst, codes, scales, ROWS) < 0);   /* non-finite input */
}

static void indexing(void)
{
    enum { S = 2, Hi = 3, Di = 32, R = 4, MAXLEN = 150, K = 12, P = 16, B = 8 };
    const int lens[S] = {150, 37};
    int64_t seq_start[S] = {0, 150};
    uint8_t keys[(150 + 37) * Di];
    for (int i = 0; i < (int)sizeof keys; ++i) keys[i] = int3_e4m3();
    uint8_t qI[R * Hi * Di];
    for (int i = 0; i < (int)sizeof qI; ++i) qI[i] = int3_e4m3();
    float w[R * Hi];
    for (int i = 0; i < R * Hi; ++i) w[i] = (float)(rnd() % 17) / 16.0f;
    int32_t row_seq[R] = {0, 1, 0, 1};
    int32_t row_len[R] = {150, 37, 5, 0};    /* ragged, K > n, empty */
    float sc[R * MAXLEN];
    CHECK(csa2_ref_index_scores(qI, w, keys, seq_start, row_seq, row_len, R, Hi, Di, MAXLEN, sc) == 0);
    for (int r = 0; r < R; ++r)
        for (int j = 0; j < MAXLEN; ++j) CHECK((j < row_len[r]) == !isnan(sc[r * MAXLEN + j]));
    int32_t topk[R * K], pool[R * P];
    CHECK(csa2_ref_index_full(qI, w, keys, seq_start, row_seq, row_len, R, Hi, Di, MAXLEN, K, P, B, topk, pool)
          == 0);
    for (int r = 0; r < R; ++r) {
        int n = row_len[r], nb = (n + B - 1) / B;
        CHECK(list_ok(topk + r * K, K, n));
        CHECK(list_ok(pool + r * P, P, nb));
        for (int k = 0; k < K && topk[r * K + k] >= 0; ++k) {   /* Top-K inside the pool (P >= K) */
            int in = 0;
            for (int p = 0; p < P; ++p) in |= pool[r * P + p] == topk[r * K + k] / B;
            CHECK(in);
        }
        int cnt = 0;
        while (cnt < K && topk[r * K + cnt] >= 0) ++cnt;
        CHECK(cnt == (n < K ? n : K));
    }
    CHECK(csa2_ref_index_full(qI, w, keys, seq_start, row_seq, row_len, R, Hi, Di, MAXLEN, K, 0, B, topk, NULL)
          == 0);
    int32_t bad_len[R] = {151, 37, 5, 0};   /* past max_len: rejected */
    CHECK(csa2_ref_index_full(qI, w, keys, seq_start, row_seq, bad_len, R, Hi, Di, MAXLEN, K, P, B, topk, pool)
          < 0);
    /* Reindex over pools with -1, out-of-range and unsorted ids */
    int32_t rpool[R * P];
    for (int r = 0; r < R; ++r)
        for (int p = 0; p < P; ++p) rpool[r * P + p] = (p % 5 == 0) ? -1 : (p % 7 == 0 ? 1000 + p : P - 1 - p);
    int32_t rt[R * K];
    CHECK(csa2_ref_index_reindex(qI, w, keys, seq_start, row_seq, row_len, rpool, R, Hi, Di, K, P, B, rt) == 0);
    for (int r = 0; r < R; ++r) CHECK(list_ok(rt + r * K, K, row_len[r]));
    rpool[3] = rpool[4];   /* duplicate ids: rejected */
    CHECK(csa2_ref_index_reindex(qI, w, keys, seq_start, row_seq, row_len, rpool, R, Hi, Di, K, P, B, rt) < 0);
}

static uint16_t bf16(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void attention(void)
{
    enum { R = 3, H = 2, D = 32, K = 6, W = 4, ROWS = 20, SWAROWS = 12 };
    uint16_t q[R * H * D];
    for (int i = 0; i < R * H * D; ++i) q[i] = bf16(gauss());
    float x[ROWS * D];
    for (int i = 0; i < ROWS * D; ++i) x[i] = (float)gauss();
    int64_t dst[ROWS];
    for (int i = 0; i < ROWS; ++i) dst[i] = i;
    uint8_t codes[ROWS * D / 2], scales[ROWS * D / 16];
    CHECK(csa2_ref_quantize_append(x, 0, ROWS, D, dst, codes, scales, ROWS) == 0);
    uint8_t swa[SWAROWS * D];
    for (int i = 0; i < SWAROWS * D; ++i) swa[i] = int3_e4m3();
    int64_t seq_start[1] = {0}, swa_row_start[R] = {0, 4, 8};
    int32_t row_seq[R] = {0, 0, 0}, row_len[R] = {20, 10, 0};
    int32_t swa_len[R] = {4, 9, 0};    /* full, longer than W (clamped), empty */
    int32_t topk[R * K] = {0, 3, 19, -1, 25, 7,     /* out of range 25 */
                           2, -1, -1, 9, 10, 1,     /* 10 is past row_len = 10 */
                           -1, -1, -1, -1, -1, -1}; /* nothing: row 2 has an empty key set */
    float out[R * H * D], lse[R * H];
    CHECK(csa2_ref_sparse_attn(q, codes, scales, seq_start, row_seq, row_len, topk, K, swa, swa_row_start, swa_len,
                               R, H, D, W, 0.17f, out, lse, NULL) == 0);
    for (int i = 0; i < 2 * H * D; ++i) CHECK(isfinite(out[i]));
    for (int h = 0; h < H; ++h) CHECK(isinf(lse[2 * H + h]) && lse[2 * H + h] < 0);
    uint8_t mask[R] = {0, 1, 0};
    CHECK(csa2_ref_sparse_attn(q, codes, scales, seq_start, row_seq, row_len, topk, K, swa, swa_row_start, swa_len,
                               R, H, D, W, 0.17f, out, lse, mask) == 0);
    /* a single key attends to itself */
    int32_t one[K] = {5, -1, -1, -1, -1, -1};
    int32_t zero_len[1] = {0};
    float o1[H * D];
    CHECK(csa2_ref_sparse_attn(q, codes, scales, seq_start, row_seq, row_len, one, K, swa, swa_row_start, zero_len,
                               1, H, D, W, 0.17f, o1, NULL, NULL) == 0);
    double deq[ROWS * D];
    CHECK(csa2_ref_dequant_rows(codes, scales, ROWS, D, deq) == 0);
    for (int h = 0; h < H; ++h)
        for (int c = 0; c < D; ++c) CHECK(o1[h * D + c] == (float)deq[5 * D + c]);
    /* dense attention over every entry of row 0 */
    double swa_vals[SWAROWS * D], dout[R * H * D];
    for (int i = 0; i < SWAROWS * D; ++i) swa_vals[i] = csa2_ref_e4m3_value(swa[i]);
    int32_t dl[R] = {4, 4, 0};
    CHECK(csa2_ref_dense_attn(q, deq, seq_start, row_seq, row_len, swa_vals, swa_row_start, dl, R, H, D, 0.17,
                              dout) == 0);
    for (int i = 0; i < R * H * D; ++i) CHECK(isfinite(dout[i]));
}

int main(void)
{
    formats();
    quantize();
    indexing();
    attention();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle ok\n");
    return 0;
}
