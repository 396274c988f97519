/*
 * csa2_oracle.c — plain CPU oracle for the CSA2 decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library, and the HIP library
 * never loads it.
 *
 * What it computes comes from the blog teardown "DeepSeek V4.1 Flash 拆解：
 * KV Cache 压掉 3/4 的工程胜利，与它没解决的三个问题" (austincafe.tech),
 * section 一 ("它到底新在哪"):
 *   - the three CSA2 layer modes (Full / Reindex / Reuse),
 *   - the Hierarchical Sparse Indexer (Top-512 first, then a pool of
 *     2048 blocks x 8 positions that later layers rescore),
 *   - the FP4 KV cache (E2M1 codes with one E4M3 scale per 16 channels; the
 *     sliding-window KV stays in FP8),
 * and from the arXiv abstract of "DeepSeek-V4.1-Flash: Pushing the Limits of
 * KV Cache Compression" (cross-layer KV reuse in CSA2 with FP4 KV caching).
 * Where those pages are silent the readings used are stated next to the
 * function that relies on them.
 *
 * Arithmetic: doubles throughout, one final rounding to float where an output
 * is float.  Loops are plain; OpenMP only splits independent rows.
 * Every entry point returns 0 on success and a negative value on a violated
 * precondition (the oracle checks its inputs; it never guesses).
 * The entry points are the twins of the library's calls: csa2_ref_<name> takes
 * the arguments of csa2_<name> in the same order, as host arrays, without the
 * stream and workspace (csa2_ref_sparse_attn adds an optional row mask).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

/* E2M1 (FP4) value of a 4-bit code: bit 3 sign, bits 2..1 exponent with bias
 * 1, bit 0 mantissa.  Exponent field 0 is subnormal: m * 2^-1.
 * (FP4 KV cache paragraph: main KV codes are E2M1.) */
double csa2_ref_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* OCP FP8 E4M3 ("fn", no infinities) value of a byte: bit 7 sign, bits 6..3
 * exponent with bias 7, bits 2..0 mantissa.  Exponent field 0 is subnormal:
 * m/8 * 2^-6.  0x7F and 0xFF are NaN.  (FP4 KV cache paragraph: one E4M3
 * scale per 16 channels; the SWA KV is FP8.) */
double csa2_ref_e4m3_value(int bits)
{
    int s = (bits >> 7) & 1, e = (bits >> 3) & 15, m = bits & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp(m / 8.0, -6);
    else        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Round a real number to E4M3, nearest representable finite value, ties to
 * the even code, saturating at +-448.  Written as the definition of rounding
 * to nearest on a sorted grid: the magnitude code is the number of grid
 * midpoints that |v| lies above, where lying exactly on a midpoint moves up
 * only if that lands on the even neighbour.  The grid is codes 0..126 (0 to
 * 448); midpoints are exact in double.  Any |v| above the last midpoint maps
 * to 448 (satfinite).  The sign bit is copied from v. */
int csa2_ref_e4m3_encode(double v)
{
    double a = fabs(v);
    int code = 0;
    for (int k = 0; k < 126; ++k) {
        double mid = 0.5 * (csa2_ref_e4m3_value(k) + csa2_ref_e4m3_value(k + 1));
        if (a > mid || (a == mid && (k & 1))) code = k + 1;
        else break;
    }
    return (signbit(v) ? 0x80 : 0) | code;
}

/* Nearest E2M1 magnitude code (0..7) to a/s for a >= 0, s > 0, ties to the
 * even code, saturating at 6.  Same grid-midpoint definition as above, with
 * the midpoints scaled by s (exact in double). */
static int e2m1_mag_code(double a, double s)
{
    int code = 0;
    for (int k = 0; k < 7; ++k) {
        double mid = 0.5 * (csa2_ref_e2m1_value(k) + csa2_ref_e2m1_value(k + 1)) * s;
        if (a > mid || (a == mid && (k & 1))) code = k + 1;
        else break;
    }
    return code;
}

/* Decoded values of every E4M3 byte and E2M1 code, filled from the two
 * definitions above before any parallel region (a cache of those functions,
 * nothing more). */
static double g_e4m3[256], g_e2m1[16];
static int g_tables_ready = 0;

static void build_tables(void)
{
    if (g_tables_ready) return;
    for (int b = 0; b < 256; ++b) g_e4m3[b] = csa2_ref_e4m3_value(b);
    for (int c = 0; c < 16; ++c) g_e2m1[c] = csa2_ref_e2m1_value(c);
    g_tables_ready = 1;
}

static inline double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* dtype 0 = float32, 1 = bfloat16 (raw 16-bit patterns). */
static inline double load_x(const void* x, int dtype, int64_t i)
{
    if (dtype == 0) return (double)((const float*)x)[i];
    return bf16_bits_to_double(((const uint16_t*)x)[i]);
}

/* ------------------------------------------------------------------------ */
/* Quantize + append (FP4 KV cache paragraph)                                */
/* ------------------------------------------------------------------------ */

/* Quantize one group of 16 channels.  Reading of the scale rule (the pages
 * give only "one E4M3 scale per 16 channels", NVFP4-style): the scale is
 * E4M3(amax / 6), rounded to nearest even and saturated, so the largest
 * magnitude maps to the top E2M1 value 6; every element is then the nearest
 * E2M1 value to x / scale (ties to even, clipped at +-6).  A scale that
 * decodes to 0 gives all-zero magnitudes.  The sign bit of each code copies
 * the sign of x (so -0.0 keeps its sign bit). */
static void quantize_group(const double* x, uint8_t* mag_sign /*16*/, uint8_t* scale_bits)
{
    double amax = 0.0;
    for (int c = 0; c < 16; ++c) if (fabs(x[c]) > amax) amax = fabs(x[c]);
    int S = csa2_ref_e4m3_encode(amax / 6.0);
    double s = csa2_ref_e4m3_value(S);
    *scale_bits = (uint8_t)S;
    for (int c = 0; c < 16; ++c) {
        int mag = (s == 0.0) ? 0 : e2m1_mag_code(fabs(x[c]), s);
        mag_sign[c] = (uint8_t)((signbit(x[c]) ? 8 : 0) | mag);
    }
}

/* Quantize T rows of D channels (float32 or bf16) and store row t at cache
 * row dst_row[t].  Codes are packed two per byte, channel 2i in the low
 * nibble and 2i+1 in the high nibble; scales are one E4M3 byte per group.
 * Rows whose destination lies outside [0, cache_rows) are skipped. */
int csa2_ref_quantize_append(const void* x, int dtype, int32_t T, int32_t D,
                        const int64_t* dst_row, uint8_t* codes, uint8_t* scales,
                        int64_t cache_rows)
{
    build_tables();
    if (D <= 0 || D % 16 || T < 0 || (dtype != 0 && dtype != 1)) return -1;
    for (int32_t t = 0; t < T; ++t) {
        for (int c = 0; c < D; ++c)
            if (!isfinite(load_x(x, dtype, (int64_t)t * D + c))) return -2;
    }
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
        int64_t r = dst_row[t];
        if (r < 0 || r >= cache_rows) continue;
        for (int g = 0; g < D / 16; ++g) {
            double xv[16];
            uint8_t q[16], S;
            for (int c = 0; c < 16; ++c) xv[c] = load_x(x, dtype, (int64_t)t * D + g * 16 + c);
            quantize_group(xv, q, &S);
            scales[r * (D / 16) + g] = S;
            for (int c = 0; c < 16; c += 2)
                codes[r * (D / 2) + g * 8 + c / 2] = (uint8_t)(q[c] | (q[c + 1] << 4));
        }
    }
    return 0;
}

/* Value of channel c of cache row r: E2M1 code times its group's E4M3 scale. */
static inline double deq(const uint8_t* codes, const uint8_t* scales, int32_t D, int64_t r, int c)
{
    uint8_t b = codes[r * (D / 2) + c / 2];
    int code = (c & 1) ? (b >> 4) : (b & 15);
    return g_e2m1[code] * g_e4m3[scales[r * (D / 16) + c / 16]];
}

int csa2_ref_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t D, double* out)
{
    if (D <= 0 || D % 16) return -1;
    build_tables();
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < D; ++c) out[r * D + c] = deq(codes, scales, D, r, c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Indexer scores (Full mode runs its own indexer; Reindex rescores with its */
/* own indexer Q)                                                            */
/* ------------------------------------------------------------------------ */

/* Reading of the score (the pages name an indexer with a query, keys and
 * per-head weights but give no formula): score_j = sum_h w_h * ReLU(q_h . k_j)
 * over the indexer heads h, with q and k decoded from E4M3. */
static double index_score(const uint8_t* qI /*[Hi,Di]*/, const float* w /*[Hi]*/,
                          const uint8_t* key /*[Di]*/, int32_t Hi, int32_t Di)
{
    double s = 0.0;
    for (int h = 0; h < Hi; ++h) {
        double dot = 0.0;
        for (int d = 0; d < Di; ++d)
            dot += g_e4m3[qI[h * Di + d]] * g_e4m3[key[d]];
        s += (double)w[h] * (dot > 0.0 ? dot : 0.0);
    }
    return s;
}

/* Scores of every visible entry of every row, rounded once to float.
 * scores is [R, max_len]; positions at or beyond row_len[r] are set to NaN. */
int csa2_ref_index_scores(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                     const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                     int32_t R, int32_t Hi, int32_t Di, int32_t max_len, float* scores)
{
    build_tables();
    if (R < 0 || Hi <= 0 || Di <= 0) return -1;
    for (int32_t r = 0; r < R; ++r) if (row_len[r] < 0 || row_len[r] > max_len) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; ++r) {
        const uint8_t* kb = ikeys + seq_start[row_seq[r]] * Di;
        for (int32_t j = 0; j < max_len; ++j) {
            scores[(int64_t)r * max_len + j] = (j < row_len[r])
                ? (float)index_score(qI + (int64_t)r * Hi * Di, w + (int64_t)r * Hi,
                                     kb + (int64_t)j * Di, Hi, Di)
                : NAN;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Selection: Top-K entries and the block pool                               */
/* ------------------------------------------------------------------------ */

typedef struct { double v; int64_t id; } item_t;

/* Strict total order: larger value first, then lower id first (reading: ties
 * go to the lowest index).  Values compare as reals, so -0 equals +0. */
static int by_value_desc_id_asc(const void* a, const void* b)
{
    const item_t* x = (const item_t*)a;
    const item_t* y = (const item_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int by_id_asc(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x < y) ? -1 : (x > y);
}

/* Keep the first min(K, n) items of the order above, write their ids in
 * ascending order and pad to K with -1. */
static void take_first_k(item_t* it, int64_t n, int32_t K, int32_t* out)
{
    qsort(it, (size_t)n, sizeof(item_t), by_value_desc_id_asc);
    int32_t k = (int32_t)(n < K ? n : K);
    for (int32_t i = 0; i < k; ++i) out[i] = (int32_t)it[i].id;
    qsort(out, (size_t)k, sizeof(int32_t), by_id_asc);
    for (int32_t i = k; i < K; ++i) out[i] = -1;
}

/* Full mode (Hierarchical Sparse Indexer paragraph): the first decoder layer
 * selects a Top-K over all of a row's visible entries, then builds the pool:
 * blocks of `block` consecutive positions aligned at multiples of `block`,
 * ranked by the largest score among the block's visible positions (reading:
 * block-max), top P kept.  Both outputs are ascending and -1 padded.
 * pool_blocks may be NULL (no pool requested). */
int csa2_ref_index_full(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                   const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                   int32_t R, int32_t Hi, int32_t Di, int32_t max_len,
                   int32_t K, int32_t P, int32_t block,
                   int32_t* topk_idx, int32_t* pool_blocks)
{
    build_tables();
    if (R < 0 || K <= 0 || P < 0 || block <= 0 || Hi <= 0 || Di <= 0) return -1;
    for (int32_t r = 0; r < R; ++r) if (row_len[r] < 0 || row_len[r] > max_len) return -2;
    /* rows one after another; the independent entry scores of a row in parallel */
    for (int32_t r = 0; r < R; ++r) {
        int32_t n = row_len[r];
        int64_t nb = ((int64_t)n + block - 1) / block;
        const uint8_t* kb = ikeys + seq_start[row_seq[r]] * Di;
        item_t* it = (item_t*)malloc(sizeof(item_t) * (size_t)(n > 0 ? n : 1));
        item_t* bl = (item_t*)malloc(sizeof(item_t) * (size_t)(nb > 0 ? nb : 1));
        if (!it || !bl) { free(it); free(bl); return -3; }
#pragma omp parallel for schedule(static)
        for (int32_t j = 0; j < n; ++j) {
            /* scores are the float results, as the library returns them */
            it[j].v = (double)(float)index_score(qI + (int64_t)r * Hi * Di, w + (int64_t)r * Hi,
                                                 kb + (int64_t)j * Di, Hi, Di);
            it[j].id = j;
        }
        for (int64_t b = 0; b < nb; ++b) {
            double m = -INFINITY;
            for (int64_t j = b * block; j < (b + 1) * block && j < n; ++j) if (it[j].v > m) m = it[j].v;
            bl[b].v = m;
            bl[b].id = b;
        }
        take_first_k(it, n, K, topk_idx + (int64_t)r * K);
        if (pool_blocks) take_first_k(bl, nb, P, pool_blocks + (int64_t)r * P);
        free(it); free(bl);
    }
    return 0;
}

/* Reindex mode (CSA2 modes and Hierarchical Sparse Indexer paragraphs): reuse
 * the earlier layer's indexer keys, rescore only the pool's positions with this
 * layer's own indexer query and weights, and keep this layer's own Top-K.
 * Candidates are positions block*b + t (t < block) of every pool block b that
 * is not -1, restricted to visible positions.  Pool ids outside
 * [0, ceil(n/block)) are ignored; duplicate pool ids are a precondition
 * violation. */
int csa2_ref_index_reindex(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                      const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                      const int32_t* pool_blocks, int32_t R, int32_t Hi, int32_t Di,
                      int32_t K, int32_t P, int32_t block, int32_t* topk_idx)
{
    build_tables();
    if (R < 0 || K <= 0 || P <= 0 || block <= 0 || Hi <= 0 || Di <= 0) return -1;
    for (int32_t r = 0; r < R; ++r) {
        const int32_t* pool = pool_blocks + (int64_t)r * P;
        for (int32_t p = 0; p < P; ++p)
            for (int32_t q = 0; q < p; ++q)
                if (pool[p] >= 0 && pool[q] == pool[p]) return -2;
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:err)
    for (int32_t r = 0; r < R; ++r) {
        int32_t n = row_len[r];
        int64_t nb = ((int64_t)n + block - 1) / block;
        const int32_t* pool = pool_blocks + (int64_t)r * P;
        const uint8_t* kb = ikeys + seq_start[row_seq[r]] * Di;
        item_t* it = (item_t*)malloc(sizeof(item_t) * (size_t)P * block);
        if (!it) { err = 1; continue; }
        int64_t c = 0;
        for (int32_t p = 0; p < P; ++p) {
            int32_t b = pool[p];
            if (b < 0 || b >= nb) continue;
            for (int64_t j = (int64_t)b * block; j < (int64_t)(b + 1) * block && j < n; ++j) {
                it[c].v = (double)(float)index_score(qI + (int64_t)r * Hi * Di, w + (int64_t)r * Hi,
                                                     kb + j * Di, Hi, Di);
                it[c].id = j;
                ++c;
            }
        }
        take_first_k(it, c, K, topk_idx + (int64_t)r * K);
        free(it);
    }
    return err ? -3 : 0;
}

/* ------------------------------------------------------------------------ */
/* Sparse attention (Reuse mode attends sparsely with inherited indices; the  */
/* SWA window is FP8)                                                         */
/* ------------------------------------------------------------------------ */

/* Readings used here: one cached latent per entry serves as both key and
 * value (many query heads share it); the selected main entries and the row's
 * SWA window rows form one key set under one softmax (entries in list order,
 * SWA rows after them; an index that is -1 or outside [0, row_len) contributes
 * nothing); logits are scale * q.k; an empty key set gives o = 0 and
 * lse = -inf.  The SWA window of row r is rows [swa_row_start[r],
 * + min(swa_len[r], W)) of a [*, D] E4M3 buffer.
 *
 * Gather the key set of row r into kbuf [nk, D]; returns nk. */
static int32_t gather_keys(const uint8_t* codes, const uint8_t* scales, int64_t base,
                           const int32_t* idx, int32_t K, int32_t n,
                           const uint8_t* swa, int64_t swa0, int32_t nswa, int32_t D, double* kbuf)
{
    int32_t nk = 0;
    for (int32_t i = 0; i < K; ++i) {
        int32_t j = idx[i];
        if (j < 0 || j >= n) continue;
        for (int c = 0; c < D; ++c) kbuf[(int64_t)nk * D + c] = deq(codes, scales, D, base + j, c);
        ++nk;
    }
    for (int32_t i = 0; i < nswa; ++i) {
        for (int c = 0; c < D; ++c) kbuf[(int64_t)nk * D + c] = g_e4m3[swa[(swa0 + i) * D + c]];
        ++nk;
    }
    return nk;
}

/* Softmax attention of one query head over nk keys (values = keys). */
static void attend_one(const uint16_t* q /*[D]*/, const double* kbuf, int32_t nk, int32_t D,
                       double scale, double* lg /*[nk]*/, float* out, float* lse)
{
    if (nk == 0) {
        for (int c = 0; c < D; ++c) out[c] = 0.0f;
        if (lse) *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int32_t i = 0; i < nk; ++i) {
        double dot = 0.0;
        for (int c = 0; c < D; ++c) dot += bf16_bits_to_double(q[c]) * kbuf[(int64_t)i * D + c];
        lg[i] = scale * dot;
        if (lg[i] > m) m = lg[i];
    }
    double l = 0.0;
    for (int32_t i = 0; i < nk; ++i) { lg[i] = exp(lg[i] - m); l += lg[i]; }
    for (int c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int32_t i = 0; i < nk; ++i) acc += lg[i] * kbuf[(int64_t)i * D + c];
        out[c] = (float)(acc / l);
    }
    if (lse) *lse = (float)(m + log(l));
}

/* q [R,H,D] bf16 bits; topk_idx [R,K]; out [R,H,D]; lse [R,H] or NULL.
 * `rows_mask` (may be NULL) selects which rows to compute; skipped rows are
 * left untouched. */
int csa2_ref_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                    const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                    const int32_t* topk_idx, int32_t K,
                    const uint8_t* swa, const int64_t* swa_row_start, const int32_t* swa_len,
                    int32_t R, int32_t H, int32_t D, int32_t W, float softmax_scale,
                    float* out, float* lse, const uint8_t* rows_mask)
{
    build_tables();
    if (R < 0 || H <= 0 || D <= 0 || D % 16 || K < 0 || W < 0) return -1;
    double* kbuf = (double*)malloc(sizeof(double) * (size_t)(K + W + 1) * D);
    if (!kbuf) return -3;
    int err = 0;
    for (int32_t r = 0; r < R; ++r) {
        if (rows_mask && !rows_mask[r]) continue;
        int32_t nswa = swa_len ? swa_len[r] : 0;
        if (nswa > W) nswa = W;
        if (nswa < 0) nswa = 0;
        int32_t nk = gather_keys(codes, scales, seq_start[row_seq[r]], topk_idx + (int64_t)r * K, K,
                                 row_len[r], swa, swa_row_start ? swa_row_start[r] : 0, nswa, D, kbuf);
#pragma omp parallel for schedule(dynamic, 1) reduction(|:err)
        for (int32_t h = 0; h < H; ++h) {
            double* lg = (double*)malloc(sizeof(double) * (size_t)(nk + 1));
            if (!lg) { err = 1; continue; }
            attend_one(q + ((int64_t)r * H + h) * D, kbuf, nk, D, (double)softmax_scale, lg,
                       out + ((int64_t)r * H + h) * D, lse ? lse + (int64_t)r * H + h : NULL);
            free(lg);
        }
    }
    free(kbuf);
    return err ? -3 : 0;
}

/* Dense attention over ALL of a row's visible entries plus its SWA rows, with
 * no selection at all.  Kept separate from csa2_ref_sparse_attn so that the
 * "sparse equals dense when K >= n" check compares two independent loops. */
int csa2_ref_dense_attn(const uint16_t* q, const double* kv /*[rows, D] dequantized*/,
                   const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                   const double* swa_vals /*[*, D]*/, const int64_t* swa_row_start,
                   const int32_t* swa_len, int32_t R, int32_t H, int32_t D, double scale,
                   double* out /*[R,H,D]*/)
{
    build_tables();
    for (int32_t r = 0; r < R; ++r) {
        int64_t base = seq_start[row_seq[r]];
        int32_t n = row_len[r], ns = swa_len[r];
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t* qh = q + ((int64_t)r * H + h) * D;
            double* o = out + ((int64_t)r * H + h) * D;
            double m = -INFINITY, l = 0.0;
            double* lg = (double*)malloc(sizeof(double) * (size_t)(n + ns + 1));
            if (!lg) return -3;
            for (int32_t i = 0; i < n + ns; ++i) {
                const double* k = (i < n) ? kv + (base + i) * D : swa_vals + (swa_row_start[r] + i - n) * D;
                double d = 0.0;
                for (int c = 0; c < D; ++c) d += bf16_bits_to_double(qh[c]) * k[c];
                lg[i] = scale * d;
                if (lg[i] > m) m = lg[i];
            }
            for (int c = 0; c < D; ++c) o[c] = 0.0;
            for (int32_t i = 0; i < n + ns; ++i) {
                const double* k = (i < n) ? kv + (base + i) * D : swa_vals + (swa_row_start[r] + i - n) * D;
                double p = exp(lg[i] - m);
                l += p;
                for (int c = 0; c < D; ++c) o[c] += p * k[c];
            }
            for (int c = 0; c < D; ++c) o[c] = (n + ns) ? o[c] / l : 0.0;
            free(lg);
        }
    }
    return 0;
}
