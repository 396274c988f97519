/*
 * csa2.h — C ABI of the CSA2 (Compressed Sparse Attention 2) decode hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the CSA2 attention step as described in section
 * 一 of the teardown "DeepSeek V4.1 Flash 拆解：KV Cache 压掉 3/4 的工程胜利，
 * 与它没解决的三个问题" (austincafe.tech) and in the arXiv abstract of
 * "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression":
 *   - the main KV cache is stored as FP4 (E2M1 codes plus one E4M3 scale per
 *     16 channels, "MXFP4" in the page's words); the sliding-window (SWA) KV
 *     stays in FP8;
 *   - a Full-mode layer runs its own indexer over every cached entry, keeps a
 *     Top-K and builds a candidate pool of whole 8-position blocks;
 *   - a Reindex-mode layer rescores only the pool with its own indexer query
 *     and keeps its own Top-K;
 *   - a Reuse-mode layer attends sparsely with an earlier layer's indices.
 *
 * Conventions shared by every call
 *   - Every pointer argument except `stream` is a DEVICE pointer owned by the
 *     caller.  The library never allocates, frees or synchronises, keeps no
 *     pointer after returning, and holds no global state other than a
 *     thread-local copy of the last error message.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued asynchronously on it.
 *   - The main cache is packed: sequence b occupies cache rows
 *     [seq_start[b], seq_start[b] + n) and entry ids inside a sequence are
 *     sequence-local (0 .. n-1).  A query row r belongs to sequence
 *     row_seq[r] and sees its first row_len[r] entries.
 *   - Index lists are int32, ascending, padded at the end with -1.
 *   - Arguments are validated on the host before any HIP call; on failure
 *     the call returns a non-zero status, enqueues nothing and leaves every
 *     output untouched.  Values stored in device memory (row lengths, index
 *     lists) cannot be validated on the host: kernels skip any index outside
 *     its valid range instead of reading or writing out of bounds.
 *   - Calls that share a workspace must not overlap on different streams.
 *   - Debug builds (compiled with -DCSA2_DEBUG, shipped as libcsa2_debug.so)
 *     also count, on the device, every out-of-range value that a kernel
 *     skips (an index outside its list's range, a row length outside
 *     [0, max_len], a destination row outside the cache, a window length
 *     outside [0, W]); such a call synchronises its stream before returning
 *     and returns CSA2_ERR_DEVICE_CHECK if the count is not zero.  Outputs are
 *     still those of the release build.  Release builds never synchronise.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Under C++ the enums take int as their fixed underlying type, so any int
 * (e.g. a status code a C caller stored) is a valid value of the type. */
#ifdef __cplusplus
#define CSA2_ENUM_BASE : int
#else
#define CSA2_ENUM_BASE
#endif

typedef enum csa2_status_e CSA2_ENUM_BASE {
    CSA2_OK = 0,
    CSA2_ERR_NULL = 1,         /* a required pointer is NULL */
    CSA2_ERR_SHAPE = 2,        /* a size argument is negative or inconsistent */
    CSA2_ERR_UNSUPPORTED = 3,  /* well-defined, but outside this library's limits */
    CSA2_ERR_WORKSPACE = 4,    /* workspace missing, too small or not 256-byte aligned */
    CSA2_ERR_LAUNCH = 5,       /* a HIP launch failed (detail in csa2_last_error) */
    CSA2_ERR_DEVICE_CHECK = 6  /* debug builds only: a kernel met an out-of-range
                                  value in device memory and skipped it */
} csa2_status_t;

typedef enum csa2_dtype_e CSA2_ENUM_BASE {
    CSA2_F32 = 0,   /* IEEE binary32 */
    CSA2_BF16 = 1   /* bfloat16 */
} csa2_dtype_t;

/* Name of a status code (static storage); "CSA2_ERR_UNKNOWN" for any other value. */
const char* csa2_status_string(csa2_status_t status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* csa2_last_error(void);

/* ABI version of this header; bumped on any incompatible change. */
#define CSA2_ABI_VERSION 2
int csa2_abi_version(void);

/* ---------------------------------------------------------------------- */
/* Quantize + append.  FP4 KV cache paragraph: E2M1 codes with one E4M3      */
/* scale per 16 channels.                                                    */
/* ---------------------------------------------------------------------- */
/*
 * Quantize T rows of D channels and store row t at cache row dst_row[t].
 *   x        [T, D] in `x_dtype` (CSA2_F32 or CSA2_BF16), row-major.
 *   dst_row  [T] int64 destination cache rows; rows outside [0, cache_rows)
 *            are skipped.
 *   codes    [cache_rows, D/2] uint8: channel 2i in the low nibble, 2i+1 in
 *            the high nibble; bit 3 of a code is the sign, bits 0..2 the
 *            E2M1 magnitude.
 *   scales   [cache_rows, D/16] uint8: OCP E4M3 bits, one per 16 channels.
 * Rule per group of 16 channels: scale = E4M3(amax/6) rounded to nearest
 * even, saturating at 448; each code is the E2M1 value nearest to x/scale
 * (ties to even, clipped at +-6); a scale of zero gives zero magnitudes;
 * the code's sign bit copies the sign of x.  Inputs must be finite.
 * Limits: T >= 0, 16 <= D <= 8192, D % 16 == 0.
 */
csa2_status_t csa2_quantize_append(const void* x, int32_t x_dtype, int32_t T, int32_t D,
                                   const int64_t* dst_row, uint8_t* codes, uint8_t* scales,
                                   int64_t cache_rows, void* stream);

/* ---------------------------------------------------------------------- */
/* Full mode: own indexer over every entry, Top-K, block pool.               */
/* CSA2 modes and Hierarchical Sparse Indexer paragraphs.                    */
/* ---------------------------------------------------------------------- */
/*
 * Score of entry j for query row r (the pages give none; the reading used):
 *   s_j = sum_h w[r,h] * max(0, sum_d qI[r,h,d] * ikeys[seq_start + j, d])
 * with qI and ikeys decoded from OCP E4M3, computed in fp32 (exact whenever
 * the inputs are small integers, as in every shipped workload).
 *   qI        [R, Hi, Di] uint8 E4M3     w  [R, Hi] float32
 *   ikeys     [rows, Di] uint8 E4M3 (one key per cache row)
 *   seq_start [S] int64   row_seq [R] int32   row_len [R] int32 in
 *             [0, max_len] (values outside are clamped to that range)
 *   topk_idx  [R, K] int32 out: the min(K, n) entries first in the order
 *             (score descending, entry id ascending), written ascending and
 *             padded with -1.  Scores compare as reals (-0 == +0).
 *   pool_blocks [R, P] int32 out (may be NULL): the min(P, ceil(n/8)) blocks
 *             [8b, 8b+8) first in the order (block max descending, block id
 *             ascending), where a block's max is over its visible entries;
 *             ascending, -1 padded.
 *   workspace: csa2_index_full_workspace_bytes(R, max_len, Hi, K, P, block)
 *             bytes of device memory, 256-byte aligned, contents ignored.
 * Limits: block == 8; 1 <= K <= 2048; 0 <= P <= 2048 (P == 0 iff
 * pool_blocks == NULL); 1 <= Hi <= 64; 32 <= Di <= 256, Di % 32 == 0;
 * 0 <= max_len < 2^31 - 64.
 */
size_t csa2_index_full_workspace_bytes(int32_t R, int32_t max_len, int32_t Hi, int32_t K, int32_t P,
                                       int32_t block);
csa2_status_t csa2_index_full(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                              const int64_t* seq_start, const int32_t* row_seq,
                              const int32_t* row_len, int32_t R, int32_t Hi, int32_t Di,
                              int32_t max_len, int32_t K, int32_t P, int32_t block,
                              int32_t* topk_idx, int32_t* pool_blocks,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Reindex mode: rescore only the pool with this layer's own indexer query.  */
/* CSA2 modes and Hierarchical Sparse Indexer paragraphs.                    */
/* ---------------------------------------------------------------------- */
/*
 * Candidates of row r are positions 8b + t (t < 8, 8b + t < row_len[r]) of
 * every pool block b = pool_blocks[r, p] that is in [0, ceil(n/8)); -1 and
 * out-of-range ids are skipped, and an id listed more than once counts once
 * (debug builds report duplicates as out-of-range values).  Scores use this call's
 * qI / w with the shared ikeys (same formula as csa2_index_full); the output
 * is the Top-K of the candidates in the same order, ascending, -1 padded.
 * Workspace: csa2_index_reindex_workspace_bytes(R, Hi, K, P, block) bytes,
 * 256-byte aligned, contents ignored.
 * Limits: block == 8; 1 <= K <= 2048; 1 <= P <= 2048; Hi, Di as above.
 */
size_t csa2_index_reindex_workspace_bytes(int32_t R, int32_t Hi, int32_t K, int32_t P, int32_t block);
csa2_status_t csa2_index_reindex(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                 const int64_t* seq_start, const int32_t* row_seq,
                                 const int32_t* row_len, const int32_t* pool_blocks,
                                 int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t P,
                                 int32_t block, int32_t* topk_idx,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * csa2_index_reindex with the score buffer in a fixed device array of
 * CSA2_NOALLOC_SCRATCH_BYTES inside the library instead of a workspace.
 * Arguments, outputs and limits are those of csa2_index_reindex (without
 * workspace / workspace_bytes); the outputs are identical.  The call also
 * needs csa2_index_reindex_workspace_bytes(R, Hi, K, P, block) to be at most
 * CSA2_NOALLOC_SCRATCH_BYTES (at P = 2048: up to 256 rows) and returns
 * CSA2_ERR_UNSUPPORTED otherwise, before any HIP call.  It allocates nothing:
 * each GPU holds one copy of the array from its first use until the process
 * ends, found on the first call on that device.  Every call on a GPU shares
 * that GPU's copy, so calls that overlap on one GPU (different streams or
 * threads) race; calls in one stream are ordered as usual.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (16u << 20)
csa2_status_t csa2_index_reindex_noalloc(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                         const int64_t* seq_start, const int32_t* row_seq,
                                         const int32_t* row_len, const int32_t* pool_blocks,
                                         int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t P,
                                         int32_t block, int32_t* topk_idx, void* stream);

/* ---------------------------------------------------------------------- */
/* Sparse attention (Reuse mode = this call with inherited indices).        */
/* CSA2 modes paragraph; FP4 main KV and FP8 SWA KV.                         */
/* ---------------------------------------------------------------------- */
/*
 * For query row r and head h, one softmax over the key set
 *   { deq(main entry j) : j in topk_idx[r, :], 0 <= j < row_len[r] }
 *   followed by { SWA rows swa_row_start[r] .. + min(swa_len[r], W) - 1 },
 * where one cached latent per entry is both key and value (all H heads share
 * it): out[r,h] = sum_k softmax(scale * q[r,h] . key_k) * key_k, and
 * lse[r,h] = log-sum-exp of the logits.  An empty key set gives out = 0 and
 * lse = -inf.
 *   q        [R, H, D] bfloat16 bits.  Used in the matrix cores as fp16, which
 *            holds every bf16 value of magnitude in [2^-14, 65504] exactly;
 *            |q| must stay below 65504.
 *   codes / scales: the main cache as written by csa2_quantize_append.
 *   topk_idx [R, K] int32, -1 = no entry.
 *   swa      [swa_rows, D] uint8 E4M3 (unscaled FP8 SWA rows).
 *   out      [R, H, D] float32;  lse [R, H] float32 (may be NULL).
 *   workspace: csa2_sparse_attn_workspace_bytes(R, H, D, K, W) bytes,
 *            256-byte aligned (may be 0 bytes and NULL when that is 0).
 *            Its first 1 KiB holds arrival words of the merge of a row's key
 *            splits: they must be zero before the first call, and every
 *            call leaves them zero again, so a workspace is zero-filled once
 *            and then reused by attention calls (the index calls' workspaces
 *            carry no such state; one they used must be zeroed again).  Other
 *            contents give wrong outputs (debug builds report
 *            CSA2_ERR_DEVICE_CHECK).
 * Arithmetic: dequantised keys are exact in fp16; logits accumulate in fp32,
 * and are exact (then rounded once) for key tiles whose scales or FP8 bytes
 * allow |value| > 8; softmax in fp32; probabilities enter the PV product
 * rounded to fp16 (split into two fp16 parts in those tiles) and the output is
 * normalised by the sum of the weights PV used; outputs accumulate in fp32;
 * lse uses the unrounded fp32 probabilities.
 * Limits: H >= 1; D in {128, 256, 512}; 0 <= K <= 4096; 0 <= W <= 4096.
 */
size_t csa2_sparse_attn_workspace_bytes(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W);
csa2_status_t csa2_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                               const int64_t* seq_start, const int32_t* row_seq,
                               const int32_t* row_len, const int32_t* topk_idx, int32_t K,
                               const uint8_t* swa, const int64_t* swa_row_start,
                               const int32_t* swa_len, int32_t R, int32_t H, int32_t D,
                               int32_t W, float softmax_scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * csa2_sparse_attn_fp4mma: csa2_sparse_attn whose query-key products for the
 * selected main entries run on the scaled FP4 matrix-core product (the E2M1
 * codes straight from the cache, no dequantisation) wherever that product is
 * exact, and on the dequantising path elsewhere.  The E2M1 codes and E4M3
 * scales are those of the FP4 KV cache paragraph of section 一 of the
 * teardown; the hardware product takes one power-of-two scale per 32
 * channels on each operand, so a 16-key fragment takes the native product
 * only if, for every one of its entries, both E4M3 scales of each 32-channel
 * block are the same power of two, and only if the row's query (per head
 * group) is exact as E4M3 under one power-of-two scale per 32 channels.
 * Where it is taken, each product is exact and the logits are those of the
 * dequantising path whenever the fp32 sums are exact (e.g. values on a common
 * grid of bounded range); otherwise they may differ in the last bits of the
 * fp32 accumulation.  The value operand of the PV product is dequantised as in
 * csa2_sparse_attn, SWA rows always take the dequantising path.
 *   native_fragments: int32 device counter (may be NULL); the call adds the
 *            number of 16-key fragments whose logits came from the native
 *            product.
 * Every other argument, the workspace (size and zero-between-calls rule),
 * limits and errors are those of csa2_sparse_attn.  A research form: it
 * moves the same bytes and is not faster.
 */
csa2_status_t csa2_sparse_attn_fp4mma(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                      const int64_t* seq_start, const int32_t* row_seq,
                                      const int32_t* row_len, const int32_t* topk_idx, int32_t K,
                                      const uint8_t* swa, const int64_t* swa_row_start,
                                      const int32_t* swa_len, int32_t R, int32_t H, int32_t D,
                                      int32_t W, float softmax_scale, float* out, float* lse,
                                      int32_t* native_fragments, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ---------------------------------------------------------------------- */
/* Paged main cache and SWA ring.  The pages fix only what is cached (FP4    */
/* main KV, FP8 SWA window, FP8 indexer keys; section 一 of the teardown);   */
/* how a server lays those rows out is left open.  These calls compute       */
/* exactly what the packed calls above compute, with different addressing.  */
/* ---------------------------------------------------------------------- */
/*
 * Paged addressing, shared by the calls below:
 *   block_table [S, max_pages] int32; page_rows a power of two in [8, 2^20].
 *   Entry j of sequence s lives in cache row
 *       block_table[s, j / page_rows] * page_rows + j % page_rows.
 *   An entry whose page index is >= max_pages, whose table value is negative,
 *   or whose row is >= cache_rows is not visible: it scores -inf, is never
 *   selected, and counts as absent in its block (as an entry past row_len).
 *   Visible entries need not be contiguous in the cache; pages may be shared.
 *   row_seq[r] must be in [0, S) (not checkable on the host).
 *
 * csa2_index_full_paged / csa2_index_reindex_paged: csa2_index_full /
 * csa2_index_reindex with `ikeys` [cache_rows, Di] addressed through the block
 * table instead of seq_start.  Outputs are identical to those of the packed
 * calls on a packed copy of the visible entries.  topk_rows [R, K] int32 (may
 * be NULL) also receives the cache row of each Top-K entry, -1 padded (what
 * csa2_paged_rows gives for topk_idx), ready for csa2_sparse_attn_phys.
 * Workspace sizes are those of the packed calls; every other argument and
 * limit is unchanged.
 */
csa2_status_t csa2_index_full_paged(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                    int64_t cache_rows, const int32_t* block_table,
                                    int32_t max_pages, int32_t page_rows,
                                    const int32_t* row_seq, const int32_t* row_len,
                                    int32_t R, int32_t Hi, int32_t Di, int32_t max_len,
                                    int32_t K, int32_t P, int32_t block,
                                    int32_t* topk_idx, int32_t* topk_rows, int32_t* pool_blocks,
                                    void* workspace, size_t workspace_bytes, void* stream);
csa2_status_t csa2_index_reindex_paged(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                       int64_t cache_rows, const int32_t* block_table,
                                       int32_t max_pages, int32_t page_rows,
                                       const int32_t* row_seq, const int32_t* row_len,
                                       const int32_t* pool_blocks, int32_t R, int32_t Hi,
                                       int32_t Di, int32_t K, int32_t P, int32_t block,
                                       int32_t* topk_idx, int32_t* topk_rows,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Translate index lists into cache rows (for lists the paged index calls did
 * not produce):
 *   phys[r, k] = cache row of entry idx[r, k] of sequence row_seq[r], or -1
 *   when idx[r, k] is -1, outside [0, row_len[r]), or not visible.
 *   idx, phys [R, K] int32 (phys may not alias idx).  The order of idx is kept.
 * Limits: R, K >= 0; cache rows above 2^31 - 1 map to -1.
 */
csa2_status_t csa2_paged_rows(const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                              int64_t cache_rows, const int32_t* row_seq, const int32_t* row_len,
                              const int32_t* idx, int32_t R, int32_t K, int32_t* phys,
                              void* stream);

/*
 * csa2_sparse_attn over cache rows: the main key set of row r is
 *   { deq(cache row c) : c in phys_idx[r, :], 0 <= c < cache_rows },
 * with codes [cache_rows, D/2] and scales [cache_rows, D/16].  Use
 * csa2_paged_rows to build phys_idx from a Top-K list.  With swa_head == NULL
 * the window is as in csa2_sparse_attn.  With swa_head [R] int32 the window of
 * row r is a ring of W rows starting at swa_row_start[r]: its i-th oldest row
 * (i < min(swa_len[r], W)) sits in slot (swa_head[r] + i) mod W, so the caller
 * overwrites slot (head + len) mod W on append instead of moving rows.
 * All W slots of a ring must lie inside `swa`.
 * The keys are the packed call's (window unrolled), taken in the same order
 * through the same arithmetic, so results are bit-identical to csa2_sparse_attn
 * on a packed copy.  Workspace and limits as csa2_sparse_attn; cache rows are
 * int32 (below 2^31), with no limit on the cache's size in bytes.
 */
csa2_status_t csa2_sparse_attn_phys(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                    int64_t cache_rows, const int32_t* phys_idx, int32_t K,
                                    const uint8_t* swa, const int64_t* swa_row_start,
                                    const int32_t* swa_len, const int32_t* swa_head, int32_t R,
                                    int32_t H, int32_t D, int32_t W, float softmax_scale,
                                    float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
