// Full-mode and Reindex-mode indexer: scoring, Top-K and block pool.
//
// CSA2 modes and Hierarchical Sparse Indexer paragraphs of section 一 of the
// teardown "DeepSeek V4.1 Flash 拆解" (austincafe.tech): the Full layer scores
// every entry with its own indexer, keeps a Top-K and builds a pool of whole
// 8-position blocks; Reindex layers rescore only the pool with their own
// indexer query and keep their own Top-K.
//
// Score (reading; the pages give no formula):
//   s_j = sum_h w_h * max(0, q_h . k_j)      q, k in OCP E4M3
//
// Kernels
//   k_index_score  FP8 matrix-core scoring.  One v_mfma_scale_f32_16x16x128
//                  f8f6f4 per (16 heads x 16 entries x 128 dims); heads are the
//                  M dimension so the weighted ReLU sum over heads stays mostly
//                  inside a lane.  Full mode streams every visible key once
//                  (coalesced 32-byte lane loads) and writes the fp32 scores
//                  and the block maxima; Reindex mode gathers the pool's
//                  1 KiB key blocks and writes one score per pool slot.
//   k_select       One workgroup per query row: exact radix select (11-bit
//                  digits over order-preserving keys, histograms in LDS) and
//                  an ordered compaction, so the outputs come out sorted and
//                  ties resolve to the lowest index.  Full mode first reduces
//                  the candidates to the top-K blocks by block maximum (via
//                  the pool, which it also outputs), then selects the Top-K
//                  among those blocks' 8K entries: every Top-K entry lies in
//                  one of them, so the result equals a Top-K over all
//                  entries.  Reindex mode selects among all 8P pool
//                  positions at once (they fit in registers).
#include <mutex>

#include "csa2_device.h"
#include "csa2_host.h"

namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / CSA2_WAVE;
constexpr int kMaxK = 2048;
constexpr int kMaxP = 2048;
constexpr int kBins = 2048;
constexpr int kFullChunk = 1024;     // entries per Full-score workgroup
constexpr int kReChunkMax = 1024;    // pool slots per Reindex-score workgroup, at most (256, 512 or 1024)

// ------------------------------------------------------------------ scoring

// max(x, 0) for a finite x as one integer max: the sign bit makes every
// negative float (and -0) a negative integer, and non-negative floats keep
// their order as integers.  (A float max would first canonicalise x.)
__device__ __forceinline__ float relu(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// Maximum over the 8 lanes of each 8-lane group (lanes 8g .. 8g+7 of every
// row), as integer maxima of an order-preserving image of the float bits
// (negative floats have their magnitude bits flipped), which fold into DPP
// operands and need no canonicalisation.  Exact: the result is one of the
// inputs.  NaN inputs are not expected.
__device__ __forceinline__ float block_max8(float v)
{
    int k = __float_as_int(v);
    k ^= (k >> 31) & 0x7FFFFFFF;
    constexpr int kLow = (int)0x80000000;   // identity of max (every lane is written anyway)
    k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x141, 0xF, 0xF, false));   // row_half_mirror
    k ^= (k >> 31) & 0x7FFFFFFF;
    return __int_as_float(k);
}

// Paged cache addressing: entry j of sequence s lives in cache row
// bt[s * max_pages + (j >> shift)] * 2^shift + (j mod 2^shift).  A page id
// outside the cache (or a page past max_pages) makes the entry not visible.
struct PageMap {
    const int32_t* bt;
    int32_t max_pages;
    int32_t shift;
    int64_t cache_rows;
    // Page id of page `page` of sequence `seq` (-1 if past the table).
    __device__ __forceinline__ int32_t page_id(int seq, int64_t page) const
    {
        return page < max_pages ? bt[(int64_t)seq * max_pages + page] : -1;
    }
    // Cache row of entry j on page id pid, or -1 if not visible.
    __device__ __forceinline__ int64_t row_on(int32_t pid, int64_t j) const
    {
        const int64_t phys = ((int64_t)pid << shift) | (j & (((int64_t)1 << shift) - 1));
        return pid >= 0 && phys < cache_rows ? phys : -1;
    }
};

// Up to 4 query pieces (HT x KS) fit in 128 registers with no accumulation
// registers: four workgroups per compute unit, MFMA results in ordinary
// registers.  Larger queries (Di = 256 with 48 or more heads) keep the
// compiler's own budget.
template <int HT, int KS, bool REINDEX, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HT * KS <= 4 ? 4 : 1))) void k_index_score(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ ikeys,
    const int64_t* __restrict__ seq_start, PageMap pm, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, int32_t n_cap, const int32_t* __restrict__ pool, int32_t Hi,
    int32_t Di, int32_t P, float* __restrict__ scores, int64_t ld_scores, float* __restrict__ bmax,
    int64_t ld_bmax, int32_t re_chunk)
{
    const int r = blockIdx.y;
    const int n_raw = row_len[r];
    CSA2_DCHECK(blockIdx.x == 0 && threadIdx.x == 0 && (n_raw < 0 || n_raw > n_cap));
    const int n = n_raw < 0 ? 0 : (n_raw > n_cap ? n_cap : n_raw);   // row lengths are clamped to [0, n_cap]
    const int lane = lane_id();
    const int wave = threadIdx.x / CSA2_WAVE;
    const int col = lane & 15;       // entry within a 16-entry tile / head within a head tile
    const int grp = lane >> 4;       // 32-byte slice of a 128-byte k-step
    const int chunk = REINDEX ? re_chunk : kFullChunk;
    const int64_t first = (int64_t)blockIdx.x * chunk;
    if (!REINDEX && first >= n) return;
    const int nb = (n + 7) >> 3;
    const int seq = row_seq[r];
    const uint8_t* keys = PAGED ? ikeys : ikeys + seq_start[seq] * (int64_t)Di;

    // The workgroup's pool block ids (Reindex) and page ids (paged) are read
    // once into LDS, so the loop's key loads wait for one LDS read instead of
    // a dependent global load.  Reindex: per pool block of the chunk, the
    // block id (-1 if absent or out of range) and the id of the page that
    // holds it (a block never straddles pages).  Full, paged: the ids of the
    // pages its entries cover (at most chunk / 8: pages hold at least 8).
    constexpr int kPg = (REINDEX ? kReChunkMax : kFullChunk) / 8;
    __shared__ int32_t pg_id[PAGED ? kPg : 1];
    __shared__ int32_t pg_blk[REINDEX ? kPg : 1];
    if constexpr (PAGED || REINDEX) {
        for (int t = threadIdx.x; t < chunk / 8; t += blockDim.x) {
            if constexpr (REINDEX) {
                const int64_t ps = (first >> 3) + t;
                const int b = ps < P ? pool[(int64_t)r * P + ps] : -1;
                const bool in = b >= 0 && b < nb;
                CSA2_DCHECK(b != -1 && !in);
                pg_blk[t] = in ? b : -1;
                if constexpr (PAGED) pg_id[t] = in ? pm.page_id(seq, ((int64_t)b * 8) >> pm.shift) : -1;
            } else {
                pg_id[t] = pm.page_id(seq, (first >> pm.shift) + t);
            }
        }
        __syncthreads();
    }

    // Query fragments (A operand: row = head, 32 bytes of the k-step per lane)
    i32x8 qa[HT][KS];
    float wv[HT][4];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        const int h = t * 16 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = ks * 128 + grp * 32;
            i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
            if (h < Hi && d0 < Di) {
                const uint4* p = reinterpret_cast<const uint4*>(qI + ((int64_t)r * Hi + h) * Di + d0);
                uint4 a = p[0], b = p[1];
                v = (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
            }
            qa[t][ks] = v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = t * 16 + grp * 4 + i;
            wv[t][i] = hh < Hi ? w[(int64_t)r * Hi + hh] : 0.0f;
        }
    }

    const int iters = chunk / (4 * 16);
    const int64_t wbase = first + (int64_t)wave * (chunk / 4);
    constexpr int U = 4;
    for (int it0 = 0; it0 < iters; it0 += U) {
        i32x8 kb[U][KS];
        int64_t ent[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t slot = wbase + (int64_t)(it0 + u) * 16 + col;
            int64_t j;
            if (REINDEX) {
                const int b = pg_blk[(slot - first) >> 3];
                j = (int64_t)b * 8 + (slot & 7);
                ok[u] = b >= 0 && b < nb && j < n;
            } else {
                j = slot;
                ok[u] = j < n;
            }
            ent[u] = j;
            int64_t jc = ok[u] ? j : 0;
            if constexpr (PAGED) {
                const int32_t pid = REINDEX ? pg_id[(slot - first) >> 3] : pg_id[(j >> pm.shift) - (first >> pm.shift)];
                const int64_t ph = ok[u] ? pm.row_on(pid, j) : -1;
                ok[u] = ph >= 0;
                jc = ok[u] ? ph : 0;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int d0 = ks * 128 + grp * 32;
                i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
                if (ok[u] && d0 < Di) {
                    const uint4* p = reinterpret_cast<const uint4*>(keys + jc * Di + d0);
                    uint4 a = p[0], b = p[1];
                    v = (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
                }
                kb[u][ks] = v;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float part = 0.0f;
#pragma unroll
            for (int t = 0; t < HT; ++t) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[t][ks], kb[u][ks], acc,
                                                                           0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int i = 0; i < 4; ++i) part += wv[t][i] * relu(acc[i]);
            }
            part = sum_xor32(sum_xor16(part));
            const int64_t slot = wbase + (int64_t)(it0 + u) * 16 + col;
            // maximum over the visible entries of each 8-entry block (-inf if none)
            const float m = max_over8(ok[u] ? part : -INFINITY);
            const bool lead = grp == 0 && (col & 7) == 0;
            // a slot without a visible entry scores -inf (never selected)
            const float sv = ok[u] ? part : -INFINITY;
            if (REINDEX) {
                if (grp == 0 && slot < (int64_t)P * 8) scores[(int64_t)r * ld_scores + slot] = sv;
            } else {
                const int64_t j = ent[u];
                if (grp == 0 && j < n) scores[(int64_t)r * ld_scores + j] = sv;
                if (lead && j < n) bmax[(int64_t)r * ld_bmax + (j >> 3)] = m;
            }
        }
    }
}

// ------------------------------------------------------------------ prefill block maxima (GEMM)
// A prefill chunk has many query rows of one sequence that see (nearly) the
// same keys.  A workgroup takes kGemmRows consecutive rows (one per wave) and
// one range of at most kGemmSplitKeys keys, and stages each 64-key tile in LDS
// once for all its rows: the keys are read once per kGemmRows rows instead of
// once per row.  Per 16 keys a wave runs its row's HT x KS MFMAs and the same
// epilogue as k_index_score, in the same order (so an entry's score is
// bit-identical to the one k_index_score gives it), but keeps only the
// 8-entry block maxima: the Full selection needs the entries' own scores only
// within its candidate blocks, which are rescored afterwards.  A wave whose row
// belongs to another sequence than the tile's reads its keys directly.
constexpr int kGemmRows = 8;             // query rows per workgroup, one per wave
constexpr int kGemmTile = 128;           // keys per staged tile
static_assert(kGemmTile % 64 == 0, "a tile is groups of four 16-key steps, one per lane group in the block maxima");
constexpr int kGemmSplitKeys = 16384;    // keys per workgroup, about (whole tiles, ranges of equal size)
constexpr int32_t kGemmMinRows = 1024;   // Full calls with this many rows take this path
constexpr int32_t kGemmBatchRows = 2048; // rows per pass (bounds the block-maxima workspace)

template <int HT, int KS, bool PAGED>
__global__ __launch_bounds__(kGemmRows * CSA2_WAVE) void k_index_bmax(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ ikeys,
    const int64_t* __restrict__ seq_start, PageMap pm, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, int32_t n_cap, int32_t R, int32_t Hi, int32_t Di,
    float* __restrict__ bmax, int64_t ld_bmax, int32_t split_keys)
{
    constexpr int RS = KS * 128 + 16;   // LDS bytes per staged key: 32-byte lane reads of 16 keys hit distinct banks
    constexpr int CH = KS * 8;          // 16-byte chunks per key
    constexpr int NST = (kGemmTile * CH + kGemmRows * CSA2_WAVE - 1) / (kGemmRows * CSA2_WAVE);
    __shared__ __attribute__((aligned(16))) uint8_t kt[2][kGemmTile * RS];
    __shared__ int s_seq[kGemmRows], s_n[kGemmRows];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int r = (int)blockIdx.y * kGemmRows + wave;   // grid: x = key range, y = row tile
    const bool row_ok = r < R;
    const int n_raw = row_ok ? row_len[r] : 0;
    CSA2_DCHECK(blockIdx.x == 0 && lane == 0 && row_ok && (n_raw < 0 || n_raw > n_cap));
    const int n = n_raw < 0 ? 0 : (n_raw > n_cap ? n_cap : n_raw);   // clamped as k_index_score does
    const int seq = row_ok ? row_seq[r] : -1;
    if (lane == 0) {
        s_seq[wave] = seq;
        s_n[wave] = n;
    }
    // the row's query (A operand: row = head, 32 bytes of the k-step per lane) and weights
    i32x8 qa[HT][KS];
    float wv[HT][4];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        const int h = t * 16 + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = ks * 128 + grp * 32;
            i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
            if (row_ok && h < Hi && d0 < Di) {
                const uint4* p = reinterpret_cast<const uint4*>(qI + ((int64_t)r * Hi + h) * Di + d0);
                const uint4 a = p[0], b = p[1];
                v = (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
            }
            qa[t][ks] = v;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = t * 16 + grp * 4 + i;
            wv[t][i] = row_ok && hh < Hi ? w[(int64_t)r * Hi + hh] : 0.0f;
        }
    }
    __syncthreads();
    // The staged keys are those of the first row's sequence, up to the
    // longest of its rows here; the workgroup's range ends at its longest row.
    const int seq0 = s_seq[0];
    int n0 = 0, nmax = 0;
#pragma unroll
    for (int i = 0; i < kGemmRows; ++i) {
        nmax = max(nmax, s_n[i]);
        if (s_seq[i] == seq0) n0 = max(n0, s_n[i]);
    }
    const int64_t k_begin64 = (int64_t)blockIdx.x * split_keys;
    if (k_begin64 >= nmax) return;   // whole workgroup
    const int k_begin = (int)k_begin64;
    const int k_end = (int)min((int64_t)nmax, (int64_t)k_begin + split_keys);
    const int ntiles = (k_end - k_begin + kGemmTile - 1) / kGemmTile;
    const bool staged = seq == seq0;   // uniform in the wave
    const uint8_t* const keys0 = PAGED ? ikeys : ikeys + (seq0 >= 0 ? seq_start[seq0] : 0) * (int64_t)Di;
    const uint8_t* const keys_r = PAGED ? ikeys : ikeys + (seq >= 0 ? seq_start[seq] : 0) * (int64_t)Di;
    // cache row of entry j of sequence s (-1: not visible)
    auto key_row = [&](int s, int64_t j) -> int64_t {
        if constexpr (PAGED) return pm.row_on(pm.page_id(s, j >> pm.shift), j);
        else return j;
    };

    // Staging: thread t holds 16-byte chunks t, t + 512, ... of a tile (chunk
    // e: key e / CH, bytes 16 (e % CH)); zeros past the keys or past Di.
    uint4 stage[NST];
    auto fetch = [&](int tile) {
#pragma unroll
        for (int u = 0; u < NST; ++u) {
            const int e = (int)threadIdx.x + u * kGemmRows * CSA2_WAVE;
            const int key = e / CH, c = e % CH;
            const int j = k_begin + tile * kGemmTile + key;   // < max_len < 2^31
            stage[u] = make_uint4(0u, 0u, 0u, 0u);
            if (e < kGemmTile * CH && j < n0 && c * 16 < Di) {
                const int64_t row = key_row(seq0, j);
                if (row >= 0) stage[u] = *reinterpret_cast<const uint4*>(keys0 + row * Di + c * 16);
            }
        }
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NST; ++u) {
            const int e = (int)threadIdx.x + u * kGemmRows * CSA2_WAVE;
            if (e < kGemmTile * CH)
                *reinterpret_cast<uint4*>(&kt[buf][(e / CH) * RS + (e % CH) * 16]) = stage[u];
        }
    };
    // One 16-key step of the wave's row: scores of keys j0 + col from the B
    // operands kb, the sum over heads in the order k_index_score uses, and the
    // maxima of its two 8-entry blocks (by lanes grp 0, col 0 and 8).
    auto epilogue = [&](const f32x4 (&acc)[HT], int j0) {
        float part = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) part += wv[ht][i] * relu(acc[ht][i]);
        part = sum_xor32(sum_xor16(part));
        const int j = j0 + col;
        bool ok = j < n;
        if constexpr (PAGED) ok = ok && key_row(seq, j) >= 0;
        const float m = block_max8(ok ? part : -INFINITY);
        if (grp == 0 && (col & 7) == 0 && j < n) bmax[(int64_t)r * ld_bmax + (j >> 3)] = m;
    };
    auto products = [&](const i32x8 (&kb)[KS], f32x4 (&acc)[HT]) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            acc[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht][ks], kb[ks], acc[ht], 0, 0, 0, 127, 0,
                                                                          127);
        }
    };

    fetch(0);
    put(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) fetch(t + 1);   // in flight during the products
        const int tile0 = k_begin + t * kGemmTile;
        if (staged) {
            // The tile's four 16-key steps; lane (col, grp) sums its 16 heads
            // of key col of each.  One reduce-scatter over the lane groups
            // then leaves lane (col, g) with the whole score of key col of
            // step g, added in the pairs sum_xor16 then sum_xor32 use (the
            // same value), and the block maxima of all four steps come from
            // one 8-lane maximum.
#pragma unroll
          for (int g4 = 0; g4 < kGemmTile / 64; ++g4) {
            float ps[4];
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) {
                i32x8 kb[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint4* p =
                        reinterpret_cast<const uint4*>(&kt[buf][((g4 * 4 + sub) * 16 + col) * RS + ks * 128 + grp * 32]);
                    const uint4 a = p[0], b = p[1];
                    kb[ks] = (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
                }
                f32x4 acc[HT];
                products(kb, acc);
                float part = 0.0f;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                    for (int i = 0; i < 4; ++i) part += wv[ht][i] * relu(acc[ht][i]);
                ps[sub] = part;
            }
            // rows 2k, 2k+1: even rows get step 0 (2) summed over the pair,
            // odd rows step 1 (3); then the halves: row g gets step g
            const auto a01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps[0]), __float_as_uint(ps[1]), false, false);
            const auto a23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(ps[2]), __float_as_uint(ps[3]), false, false);
            const float q01 = __uint_as_float(a01[0]) + __uint_as_float(a01[1]);
            const float q23 = __uint_as_float(a23[0]) + __uint_as_float(a23[1]);
            const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(q01), __float_as_uint(q23), false, false);
            const float total = __uint_as_float(b[0]) + __uint_as_float(b[1]);
            const int j = tile0 + g4 * 64 + grp * 16 + col;
            bool ok = j < n;
            if constexpr (PAGED) ok = ok && key_row(seq, j) >= 0;
            const float m = block_max8(ok ? total : -INFINITY);
            if ((col & 7) == 0 && j < n) bmax[(int64_t)r * ld_bmax + (j >> 3)] = m;
          }
        } else {
#pragma unroll
            for (int sub = 0; sub < kGemmTile / 16; ++sub) {
                const int j = tile0 + sub * 16 + col;
                const int64_t row = j < n ? key_row(seq, j) : -1;
                i32x8 kb[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int d0 = ks * 128 + grp * 32;
                    i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
                    if (row >= 0 && d0 < Di) {
                        const uint4* p = reinterpret_cast<const uint4*>(keys_r + row * Di + d0);
                        const uint4 a = p[0], b = p[1];
                        v = (i32x8){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
                    }
                    kb[ks] = v;
                }
                f32x4 acc[HT];
                products(kb, acc);
                epilogue(acc, tile0 + sub * 16);
            }
        }
        if (t + 1 < ntiles) {
            put(buf ^ 1);   // the other buffer's last readers passed the previous barrier
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------ selection

struct SelState {
    uint32_t prefix;   // selected keys: (key & mask) > prefix, or == prefix among the first `need`
    uint32_t mask;
    int need;
};

// Published per-wave values and the digit search result.  The per-wave slots
// are double-buffered: every publish is followed by a barrier, so a slot set
// is only rewritten after every wave has passed the barrier that follows the
// reads of its previous contents.
constexpr int kHistSpan = kBins + kBins / 32;   // one digit histogram, bin b at b + b/32
struct SelShared {
    int hist[2 * kHistSpan + CSA2_WAVE];   // two histograms (two thresholds found in the same
                                           // passes), then one discard word per lane
    int wave_x[2][3][kSelWaves];
    int digit[2], above[2], in_bin[2];     // digit search results, one slot per threshold
};

__device__ __forceinline__ int hist_at(int b) { return b + (b >> 5); }
constexpr int kHistDiscard = 2 * kHistSpan;

// Wave-wide inclusive scan with DPP: Hillis-Steele steps inside each row of
// 16 lanes (row_shr 1, 2, 4, 8), then row 0's total to row 1 and row 2's to
// row 3 (row_bcast:15), then lane 31's running total to rows 2 and 3
// (row_bcast:31).  Lanes that receive nothing keep `id`, the identity of op.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op)
{
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xF, 0xF, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xF, 0xF, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xF, 0xF, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xF, 0xF, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xA, 0xF, false));
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xC, 0xF, false));
    return x;
}
__device__ __forceinline__ int wave_incl_sum(int v)
{
    return (int)wave_scan((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_last(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, CSA2_WAVE - 1); }

// Exclusive block-wide prefix sum of an int in thread order; returns the
// total.  `phase` selects the per-wave slot set and flips on every call.
__device__ __forceinline__ int block_excl_sum(SelShared& sh, int& phase, int v, int& excl)
{
    const int lane = lane_id(), wave = threadIdx.x / CSA2_WAVE;
    const int incl = wave_incl_sum(v);
    int* slot = sh.wave_x[phase][0];
    phase ^= 1;
    if (lane == CSA2_WAVE - 1) slot[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int x = slot[i];
        if (i < wave) before += x;
        total += x;
    }
    excl = before + incl - v;
    return total;
}

// The same for two ints at once (one barrier).
__device__ __forceinline__ void block_excl_sum2(SelShared& sh, int& phase, int v0, int v1, int& excl0, int& excl1,
                                                int& total0, int& total1)
{
    const int lane = lane_id(), wave = threadIdx.x / CSA2_WAVE;
    const int incl0 = wave_incl_sum(v0), incl1 = wave_incl_sum(v1);
    int (*slot)[kSelWaves] = sh.wave_x[phase];
    phase ^= 1;
    if (lane == CSA2_WAVE - 1) {
        slot[0][wave] = incl0;
        slot[1][wave] = incl1;
    }
    __syncthreads();
    int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int x0 = slot[0][i], x1 = slot[1][i];
        if (i < wave) { b0 += x0; b1 += x1; }
        t0 += x0;
        t1 += x1;
    }
    excl0 = b0 + incl0 - v0;
    excl1 = b1 + incl1 - v1;
    total0 = t0;
    total1 = t1;
}

// Items are processed in rounds of kRound; within a round thread t holds the
// kE consecutive items t*kE .. t*kE+kE-1 in registers (one 8-entry block of
// candidates, or eight block maxima: two 16-byte loads).  Key 0 marks an
// invalid item (order_key never maps a finite float to 0).  The first
// kRegRounds rounds stay in registers across all passes of a selection;
// later rounds are read again from their source on every pass.
constexpr int kE = 8;
constexpr int kRound = kSelThreads * kE;
constexpr int kRegRounds = 4;
// LDS key arrays: one spare word per 8 so that lane t reading word t*kE + e
// lands in bank 9t + e (all 64 lanes distinct).
__device__ __forceinline__ int padded(int i) { return i + (i >> 3); }
constexpr int padded_size(int n) { return n + n / 8; }

typedef uint32_t RegKeys[kRegRounds][kE];

__device__ __forceinline__ void keys8(const float* p, uint32_t (&key)[kE], int valid)
{
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    const float v[kE] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < kE; ++e) key[e] = e < valid && v[e] != -INFINITY ? order_key(v[e]) : 0u;
}

// Key sources.  Each gives rounds() and load(rd, key): the keys of items
// rd*kRound + threadIdx.x*kE + e; load is fetch (issue the reads into a Raw)
// followed by finish (turn the Raw into keys), and fetch may be issued for
// rounds past the end (they finish as invalid items).

// Block maxima of one Full row in global memory (item = block id).  The row
// holds a multiple of 8 floats, so the last thread's 32-byte read stays inside
// it; entries past `cnt` are masked.
struct BlockMaxSrc {
    const float* bm;
    int cnt;
    struct Raw { float4 a, b; };
    __device__ __forceinline__ int rounds() const { return (cnt + kRound - 1) / kRound; }
    // Unconditional: items past the end read the row's last 8 floats
    // (cnt >= 1 whenever there is a round), and finish() masks them.
    __device__ __forceinline__ void fetch(int rd, Raw& raw) const
    {
        const int i0 = rd * kRound + (int)threadIdx.x * kE;
        const int last = ((cnt + kE - 1) & ~(kE - 1)) - kE;
        const float4* p = reinterpret_cast<const float4*>(bm + (i0 < last ? i0 : last));
        raw.a = p[0];
        raw.b = p[1];
    }
    __device__ __forceinline__ void finish(int rd, const Raw& raw, uint32_t (&key)[kE]) const
    {
        const int i0 = rd * kRound + (int)threadIdx.x * kE;
        const float v[kE] = {raw.a.x, raw.a.y, raw.a.z, raw.a.w, raw.b.x, raw.b.y, raw.b.z, raw.b.w};
#pragma unroll
        for (int e = 0; e < kE; ++e) key[e] = i0 + e < cnt && v[e] != -INFINITY ? order_key(v[e]) : 0u;
    }
    __device__ __forceinline__ void load(int rd, uint32_t (&key)[kE]) const
    {
        Raw raw;
        fetch(rd, raw);
        finish(rd, raw, key);
    }
};

// Sources whose loads are cheap to repeat (LDS, or small gathers that always
// fit the register rounds) fetch by loading their keys directly.
template <class Src>
struct DirectFetch {
    struct Raw { uint32_t k[kE]; };
    __device__ __forceinline__ void fetch(int rd, Raw& raw) const { static_cast<const Src*>(this)->load(rd, raw.k); }
    __device__ __forceinline__ void finish(int, const Raw& raw, uint32_t (&key)[kE]) const
    {
#pragma unroll
        for (int e = 0; e < kE; ++e) key[e] = raw.k[e];
    }
};

// Keys already in an LDS array at padded positions.
struct LdsKeySrc : DirectFetch<LdsKeySrc> {
    const uint32_t* keys;
    int cnt;
    __device__ __forceinline__ int rounds() const { return (cnt + kRound - 1) / kRound; }
    __device__ __forceinline__ void load(int rd, uint32_t (&key)[kE]) const
    {
        const int i0 = rd * kRound + (int)threadIdx.x * kE;
#pragma unroll
        for (int e = 0; e < kE; ++e) key[e] = i0 + e < cnt ? keys[padded(i0 + e)] : 0u;
    }
};

// Pool positions of one Reindex row in slot order: item c is position c % 8
// of pool slot c / 8, whose score is sc[c] (-inf where the slot holds no
// visible entry), read as CandSrc reads a block.
struct SlotSrc : DirectFetch<SlotSrc> {
    const float* sc;
    int nslot;
    __device__ __forceinline__ int rounds() const { return (nslot + kSelThreads - 1) / kSelThreads; }
    __device__ __forceinline__ void load(int rd, uint32_t (&key)[kE]) const
    {
        const int ci = rd * kSelThreads + (int)threadIdx.x;
        keys8(sc + 8 * (int64_t)ci, key, ci < nslot ? kE : 0);
    }
};

// Candidate entries: item c is position c % 8 of candidate block c / 8, i.e.
// entry 8*blocks[c/8] + c%8, visible when below n (block -1: none).  Its
// score is at sc[8*blocks[c/8] + c%8] (Full: scores by entry id) or
// sc[8*slots[c/8] + c%8] (Reindex: scores by pool slot).  Thread t of round rd
// reads block rd*kSelThreads + t: two 16-byte loads.
struct CandSrc : DirectFetch<CandSrc> {
    const float* sc;
    const int* blocks;
    const int* slots;    // null in Full mode
    int nblk, n;
    __device__ __forceinline__ int rounds() const { return (nblk + kSelThreads - 1) / kSelThreads; }
    __device__ __forceinline__ void load(int rd, uint32_t (&key)[kE]) const
    {
        const int ci = rd * kSelThreads + (int)threadIdx.x;
        if (ci < nblk && blocks[ci] >= 0) {
            const int b = blocks[ci];
            const int64_t at = 8 * (int64_t)(slots ? slots[ci] : b);
            const int64_t vis = (int64_t)n - 8 * (int64_t)b;
            keys8(sc + at, key, vis < kE ? (int)vis : kE);
        } else {
#pragma unroll
            for (int e = 0; e < kE; ++e) key[e] = 0u;
        }
    }
};

// Evenly spaced block maxima of a long Full row (cnt > kRound): item s of the
// one round is block floor(s * cnt / kRound).
struct SampleSrc : DirectFetch<SampleSrc> {
    const float* bm;
    int cnt;
    __device__ __forceinline__ int rounds() const { return 1; }
    __device__ __forceinline__ void load(int, uint32_t (&key)[kE]) const
    {
        const int s0 = (int)threadIdx.x * kE;
        float v[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) v[e] = bm[(int)((int64_t)(s0 + e) * cnt / kRound)];
#pragma unroll
        for (int e = 0; e < kE; ++e) key[e] = v[e] != -INFINITY ? order_key(v[e]) : 0u;
    }
};

// Calls f(rd, keys) for every round: the register rounds first, then the
// rest read from the source with kPrefetch rounds in flight (their fetches
// are unconditional, so every wait is for the oldest round only).  Uniform
// across the block (f may synchronise).
constexpr int kPrefetch = 4;
template <class Src, class F>
__device__ __forceinline__ void for_rounds(const Src& src, const RegKeys& reg, F f)
{
    const int rounds = src.rounds();
#pragma unroll
    for (int rr = 0; rr < kRegRounds; ++rr)
        if (rr < rounds) f(rr, reg[rr]);
    if (rounds <= kRegRounds) return;
    typename Src::Raw buf[kPrefetch];
#pragma unroll
    for (int q = 0; q < kPrefetch; ++q) src.fetch(kRegRounds + q, buf[q]);
    for (int rd = kRegRounds; rd < rounds; rd += kPrefetch) {
#pragma unroll
        for (int q = 0; q < kPrefetch; ++q) {
            uint32_t key[kE];
            src.finish(rd + q, buf[q], key);
            // the next fetch reuses buf[q]'s registers only if it stays after
            // the finish; hoisted, it would land in other registers that the
            // loop then copies back, waiting for loads still in flight
            __builtin_amdgcn_sched_barrier(0);
            src.fetch(rd + q + kPrefetch, buf[q]);
            if (rd + q < rounds) f(rd + q, key);
        }
    }
}

template <class Src>
__device__ __forceinline__ void load_regs(const Src& src, RegKeys& reg)
{
    const int rounds = src.rounds();
#pragma unroll
    for (int rr = 0; rr < kRegRounds; ++rr) {
        if (rr < rounds) src.load(rr, reg[rr]);
        else
#pragma unroll
            for (int e = 0; e < kE; ++e) reg[rr][e] = 0u;
    }
}

// Finds the threshold of the k largest keys among the valid items.  The bits
// shared by every valid key are skipped first (an AND/OR reduction finds the
// highest and the lowest bit that differ: scores on a coarse grid leave their
// low bits zero in every key), then radix passes over 11-bit digits between
// them narrow to the digit holding the k-th largest key, stopping early once a
// whole digit bin is taken.  A pass is: LDS atomic histogram of the keys that
// match the prefix so far (the others add into a discard word of their own
// lane, so the loop has no branches), barrier, then wave 0 alone finds the
// digit: each lane sums 32 contiguous bins (highest first), a wave scan and a
// ballot pick the lane whose range holds the k-th key, a second scan over that
// lane's 32 bins (one per lane) picks the bin; wave 0 also clears the bins for
// the next pass and publishes the digit, barrier.  The histogram must be zero
// on entry and is zero again on return.

// Mask of the bits outside the varying range of the valid keys (diff: the bits
// in which some valid keys differ): above its highest and below its lowest
// bit.  Every valid key holds the same values there.
__device__ __forceinline__ uint32_t common_bits(uint32_t diff)
{
    if (diff == 0u) return 0xFFFFFFFFu;
    return ~((2u << (31 - __builtin_clz(diff))) - 1u) | ((1u << __builtin_ctz(diff)) - 1u);
}

// Run by one wave: the bin of histogram h holding the krem-th largest key
// (bins taken from the highest digit down), the count of keys in higher bins
// and the bin's own count go to result slot `res`.  Each lane sums 32 bins, a
// scan and a ballot pick the lane whose bins span rank krem, and a second
// scan over that lane's bins picks the bin.  With `clear` the wave zeroes the
// histogram after reading it.
__device__ __forceinline__ void digit_search(SelShared& sh, int h, int res, int krem, bool clear)
{
    const int lane = lane_id();
    int* const hist = sh.hist + h * kHistSpan;
    constexpr int BPL = kBins / CSA2_WAVE;    // bins per lane
    const int b0 = kBins - 1 - BPL * lane;    // this lane's highest bin
    int sum = 0;
#pragma unroll
    for (int m = 0; m < BPL; ++m) sum += hist[hist_at(b0 - m)];
    const int incl = wave_incl_sum(sum);
    const int excl = incl - sum;
    const uint64_t hit = __ballot(excl < krem && krem <= incl);   // exactly one lane
    const int L = hit ? __builtin_ctzll(hit) : 0;
    const int base = __builtin_amdgcn_readlane(excl, L);
    const int bL = kBins - 1 - BPL * L;
    const int v = lane < BPL ? hist[hist_at(bL - lane)] : 0;
    if (clear) {
#pragma unroll
        for (int m = 0; m < BPL; ++m) hist[hist_at(b0 - m)] = 0;
    }
    const int a = base + wave_incl_sum(v) - v;
    if (lane < BPL && a < krem && krem <= a + v) { sh.digit[res] = bL - lane; sh.above[res] = a; sh.in_bin[res] = v; }
}

template <class Src>
__device__ __forceinline__ SelState radix_select(SelShared& sh, int& phase, const Src& src, const RegKeys& reg,
                                                 int k)
{
    const int lane = lane_id(), wave = threadIdx.x / CSA2_WAVE;
    // population and common prefix of the valid keys
    uint32_t kand = 0xFFFFFFFFu, kor = 0u;
    int nv = 0;
    for_rounds(src, reg, [&](int, const uint32_t (&key)[kE]) {
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if (key[e]) { kand &= key[e]; kor |= key[e]; ++nv; }
    });
    kand = wave_last(wave_scan(kand, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a & b; }));
    kor = wave_last(wave_scan(kor, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
    nv = (int)wave_last((uint32_t)wave_incl_sum(nv));
    int (*slot)[kSelWaves] = sh.wave_x[phase];
    phase ^= 1;
    if (lane == 0) { slot[0][wave] = (int)kand; slot[1][wave] = (int)kor; slot[2][wave] = nv; }
    __syncthreads();
    kand = 0xFFFFFFFFu; kor = 0u; nv = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        kand &= (uint32_t)slot[0][w];
        kor |= (uint32_t)slot[1][w];
        nv += slot[2][w];
    }
    SelState st{0u, 0u, nv};
    if (nv <= k) return st;                       // everything valid is selected (mask 0)
    const uint32_t diff = kand ^ kor;             // bits that vary among valid keys
    st.mask = common_bits(diff);
    st.prefix = kand & st.mask;
    st.need = k;
    if (diff == 0u) return st;                    // all valid keys equal: ties only
    int top = 31 - __builtin_clz(diff);           // highest varying bit
    const int low = __builtin_ctz(diff);          // lowest varying bit
    int krem = k;
    while (top >= low) {
        const int width = top + 1 - low < 11 ? top + 1 - low : 11;
        const int shift = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        for_rounds(src, reg, [&](int, const uint32_t (&key)[kE]) {
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const bool hit = key[e] && (key[e] & st.mask) == st.prefix;
                atomicAdd(&sh.hist[hit ? hist_at((int)((key[e] >> shift) & dmask)) : kHistDiscard + lane], 1);
            }
        });
        __syncthreads();
        if (wave == 0) digit_search(sh, 0, 0, krem, true);
        __syncthreads();
        const int d = sh.digit[0];
        krem -= sh.above[0];
        const int in_bin = sh.in_bin[0];
        st.prefix |= (uint32_t)d << shift;
        st.mask |= dmask << shift;
        st.need = krem;
        if (in_bin == krem) break;   // the whole bin is taken: no tie to resolve
        top = shift - 1;
    }
    return st;
}

// Thresholds of the k1 and of the k2 largest keys (k1 >= k2) in the same
// passes.  Both searches take the same digit positions, so while their
// prefixes agree one histogram serves both; once they differ, a key can match
// at most one of them and counts in that one's histogram (the second half of
// the LDS histogram space), so a pass still costs one atomic per key.
template <class Src>
__device__ __forceinline__ void radix_select2(SelShared& sh, int& phase, const Src& src, const RegKeys& reg, int k1,
                                              int k2, SelState& s1, SelState& s2)
{
    const int lane = lane_id(), wave = threadIdx.x / CSA2_WAVE;
    uint32_t kand = 0xFFFFFFFFu, kor = 0u;
    int nv = 0;
    for_rounds(src, reg, [&](int, const uint32_t (&key)[kE]) {
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if (key[e]) { kand &= key[e]; kor |= key[e]; ++nv; }
    });
    kand = wave_last(wave_scan(kand, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a & b; }));
    kor = wave_last(wave_scan(kor, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
    nv = (int)wave_last((uint32_t)wave_incl_sum(nv));
    int (*slot)[kSelWaves] = sh.wave_x[phase];
    phase ^= 1;
    if (lane == 0) { slot[0][wave] = (int)kand; slot[1][wave] = (int)kor; slot[2][wave] = nv; }
    __syncthreads();
    kand = 0xFFFFFFFFu; kor = 0u; nv = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        kand &= (uint32_t)slot[0][w];
        kor |= (uint32_t)slot[1][w];
        nv += slot[2][w];
    }
    s1 = SelState{0u, 0u, nv};
    s2 = SelState{0u, 0u, nv};
    bool done1 = nv <= k1, done2 = nv <= k2;     // everything valid is selected (mask 0)
    if (done1 && done2) return;
    const uint32_t diff = kand ^ kor;
    const uint32_t mask0 = common_bits(diff);
    if (!done1) s1 = SelState{kand & mask0, mask0, k1};
    if (!done2) s2 = SelState{kand & mask0, mask0, k2};
    if (diff == 0u) return;                       // all valid keys equal: ties only
    int top = 31 - __builtin_clz(diff);
    const int low = __builtin_ctz(diff);
    int krem1 = k1, krem2 = k2;
    while (top >= low && !(done1 && done2)) {
        const int width = top + 1 - low < 11 ? top + 1 - low : 11;
        const int shift = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        const bool same = !done1 && !done2 && s1.prefix == s2.prefix;   // (the masks agree)
        for_rounds(src, reg, [&](int, const uint32_t (&key)[kE]) {
#pragma unroll
            for (int e = 0; e < kE; ++e) {
                const int dg = (int)((key[e] >> shift) & dmask);
                const bool h1 = !done1 && key[e] && (key[e] & s1.mask) == s1.prefix;
                const bool h2 = !done2 && !same && key[e] && (key[e] & s2.mask) == s2.prefix;
                atomicAdd(&sh.hist[h1 ? hist_at(dg) : h2 ? kHistSpan + hist_at(dg) : kHistDiscard + lane], 1);
            }
        });
        __syncthreads();
        if (same) {
            if (wave == 0) {
                digit_search(sh, 0, 0, krem1, false);
                digit_search(sh, 0, 1, krem2, true);
            }
        } else {
            if (wave == 0 && !done1) digit_search(sh, 0, 0, krem1, true);
            if (wave == 1 && !done2) digit_search(sh, 1, 1, krem2, true);
        }
        __syncthreads();
        if (!done1) {
            krem1 -= sh.above[0];
            s1.prefix |= (uint32_t)sh.digit[0] << shift;
            s1.mask |= dmask << shift;
            s1.need = krem1;
            done1 = sh.in_bin[0] == krem1;        // the whole bin is taken
        }
        if (!done2) {
            krem2 -= sh.above[1];
            s2.prefix |= (uint32_t)sh.digit[1] << shift;
            s2.mask |= dmask << shift;
            s2.need = krem2;
            done2 = sh.in_bin[1] == krem2;
        }
        top = shift - 1;
    }
}

// The lowest n set bits of m (n <= popcount(m)).
__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, int n)
{
    if (n >= __builtin_popcount(m)) return m;
    uint32_t r = 0u;
    for (int k = 0; k < n; ++k) {
        r |= m & (0u - m);
        m &= m - 1u;
    }
    return r;
}

// Ordered compaction: emit(pos, item, pre(round)) for the selected items in
// item order; pre(rd) is read once per thread and round, before the emits,
// so that no emit waits on a load of its own.  A thread marks the keys above
// the threshold and those equal to it among its items (two bit masks); one
// block scan of the packed counts per round gives every thread the number of
// selected items before its own (all keys above, plus the first `need` equal
// keys: ties go to the lowest item), and the thread then writes its selected
// items in order, visiting only the set bits (most threads of a round hold
// none).  Returns the number selected.
template <class Src, class Emit, class Pre>
__device__ __forceinline__ int select_compact(SelShared& sh, int& phase, const Src& src, const RegKeys& reg,
                                              SelState st, Emit emit, Pre pre)
{
    int gt_run = 0, eq_run = 0;
    for_rounds(src, reg, [&](int rd, const uint32_t (&key)[kE]) {
        const int pv = pre(rd);
        uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const uint32_t mk = key[e] & st.mask;
            gtm |= (key[e] && mk > st.prefix) ? 1u << e : 0u;
            eqm |= (key[e] && mk == st.prefix) ? 1u << e : 0u;
        }
        const int gt = __builtin_popcount(gtm), eq = __builtin_popcount(eqm);
        int before;
        const int total = block_excl_sum(sh, phase, (gt << 16) | eq, before);   // counts <= kRound < 2^15
        const int gt_before = gt_run + (before >> 16), eq_before = eq_run + (before & 0xFFFF);
        int out = gt_before + (eq_before < st.need ? eq_before : st.need);
        const int take = st.need - eq_before;   // equal keys this thread may still take
        uint32_t sel = gtm | (take <= 0 ? 0u : lowest_bits(eqm, take));
        const int i0 = rd * kRound + (int)threadIdx.x * kE;
        while (sel != 0u) {
            const int e = __builtin_ctz(sel);
            sel &= sel - 1u;
            emit(out++, i0 + e, pv);
        }
        gt_run += total >> 16;
        eq_run += total & 0xFFFF;
    });
    __syncthreads();
    return gt_run + (eq_run < st.need ? eq_run : st.need);
}

// Ordered compaction for two thresholds in the same rounds and scans:
// emit_a(pos, item) for the items of sa, emit_b(pos, item) for those of sb.
// Returns both counts (before any cap).
template <class Src, class EmitA, class EmitB>
__device__ __forceinline__ int2 select_compact2(SelShared& sh, int& phase, const Src& src, const RegKeys& reg,
                                                SelState sa, SelState sb, EmitA emit_a, EmitB emit_b)
{
    int gta_run = 0, eqa_run = 0, gtb_run = 0, eqb_run = 0;
    for_rounds(src, reg, [&](int rd, const uint32_t (&key)[kE]) {
        uint32_t gam = 0u, eam = 0u, gbm = 0u, ebm = 0u;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const uint32_t ma = key[e] & sa.mask, mb = key[e] & sb.mask;
            gam |= (key[e] && ma > sa.prefix) ? 1u << e : 0u;
            eam |= (key[e] && ma == sa.prefix) ? 1u << e : 0u;
            gbm |= (key[e] && mb > sb.prefix) ? 1u << e : 0u;
            ebm |= (key[e] && mb == sb.prefix) ? 1u << e : 0u;
        }
        const int gta = __builtin_popcount(gam), eqa = __builtin_popcount(eam);
        const int gtb = __builtin_popcount(gbm), eqb = __builtin_popcount(ebm);
        int bfa, bfb, tta, ttb;
        block_excl_sum2(sh, phase, (gta << 16) | eqa, (gtb << 16) | eqb, bfa, bfb, tta, ttb);   // counts < 2^15
        const int gta_b = gta_run + (bfa >> 16), eqa_b = eqa_run + (bfa & 0xFFFF);
        const int gtb_b = gtb_run + (bfb >> 16), eqb_b = eqb_run + (bfb & 0xFFFF);
        int outa = gta_b + (eqa_b < sa.need ? eqa_b : sa.need), outb = gtb_b + (eqb_b < sb.need ? eqb_b : sb.need);
        const int take_a = sa.need - eqa_b, take_b = sb.need - eqb_b;
        uint32_t sel_a = gam | (take_a <= 0 ? 0u : lowest_bits(eam, take_a));
        uint32_t sel_b = gbm | (take_b <= 0 ? 0u : lowest_bits(ebm, take_b));
        const int i0 = rd * kRound + (int)threadIdx.x * kE;
        while (sel_a != 0u) {
            const int e = __builtin_ctz(sel_a);
            sel_a &= sel_a - 1u;
            emit_a(outa++, i0 + e);
        }
        while (sel_b != 0u) {
            const int e = __builtin_ctz(sel_b);
            sel_b &= sel_b - 1u;
            emit_b(outb++, i0 + e);
        }
        gta_run += tta >> 16;
        eqa_run += tta & 0xFFFF;
        gtb_run += ttb >> 16;
        eqb_run += ttb & 0xFFFF;
    });
    __syncthreads();
    return make_int2(gta_run + (eqa_run < sa.need ? eqa_run : sa.need), gtb_run + (eqb_run < sb.need ? eqb_run : sb.need));
}

__device__ void bitonic_sort(unsigned long long* a, int n_pow2)
{
    for (int k = 2; k <= n_pow2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n_pow2; i += kSelThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long x = a[i], y = a[ixj];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) { a[i] = y; a[ixj] = x; }
                }
            }
            __syncthreads();
        }
    }
}

constexpr int kGatherCap = 8192;   // blocks a long Full row's pre-filter may keep

struct SelectLds {
    SelShared sh;
    int blocks[kMaxP];                   // Full: selected blocks; Reindex: block of each item
    int slots[kMaxP];                    // Reindex: pool slot of each item
    int cblk[kMaxK];                     // candidate blocks (when not `blocks` itself)
    int cslot[kMaxK];                    // Reindex: their pool slots
    unsigned long long sortbuf[kMaxP];   // Reindex: pool sorted by block id
    int flag;
};
struct SelectLdsFull : SelectLds {
    uint32_t gkey[padded_size(kGatherCap)];   // long rows: keys of the pre-filtered blocks
    int gid[kGatherCap];                      // and their block ids, ascending
};

// Threshold of the pre-filter of a long Full row (more block maxima than
// the registers hold): the key of the s-th largest of kRound evenly spaced
// block maxima, s chosen so that about 2 * big blocks are expected at or
// above it.  Deterministic, so every workgroup of the row finds the same one.
__device__ __forceinline__ uint32_t prefilter_threshold(SelShared& sh, int& phase, const float* bm, int nb, int big)
{
    const SampleSrc ssrc{{}, bm, nb};
    RegKeys reg;
    load_regs(ssrc, reg);
    int s_target = (int)(((int64_t)2 * big * kRound + nb - 1) / nb);
    s_target = s_target < 1 ? 1 : s_target;
    const uint32_t thr = radix_select(sh, phase, ssrc, reg, s_target).prefix;
    return thr > 1u ? thr : 1u;   // key 0 is an absent item
}

constexpr int kMaxSlices = 1024;    // slices of kRound block maxima a pre-filtered row may have
constexpr int kPrefilterRows = 128;  // the separate pre-filter runs below this many rows

// Pre-filter of long Full rows, one workgroup per (slice of kRound block
// maxima, row): the blocks of the slice whose key is at or above the row's
// threshold, in block order, go to gkey / gid at the slice's own offset, and
// their number to gcount.  Rows that fit the registers are left to k_select.
__global__ __launch_bounds__(kSelThreads) void k_prefilter(const float* __restrict__ bmax, int64_t ld_bmax,
                                                           const int32_t* __restrict__ row_len, int32_t n_cap,
                                                           int32_t big,
                                                           uint32_t* __restrict__ gkey, int32_t* __restrict__ gid,
                                                           int32_t* __restrict__ gcount, int32_t nslices)
{
    __shared__ SelShared sh;
    const int g = blockIdx.x, r = blockIdx.y;
    const int n = min(max(row_len[r], 0), n_cap);
    const int nb = (n + 7) >> 3;
    const int ns = (nb + kRound - 1) / kRound;
    if (nb <= kRegRounds * kRound || ns > kMaxSlices || g >= ns) return;   // uniform per workgroup
    for (int i = threadIdx.x; i < 2 * kHistSpan; i += kSelThreads) sh.hist[i] = 0;
    int phase = 0;
    const float* bm = bmax + (int64_t)r * ld_bmax;
    const uint32_t lo = prefilter_threshold(sh, phase, bm, nb, big);
    const BlockMaxSrc bsrc{bm, nb};
    uint32_t key[kE];
    bsrc.load(g, key);
    uint32_t hit = 0u;
#pragma unroll
    for (int e = 0; e < kE; ++e) hit |= (key[e] >= lo ? 1u : 0u) << e;
    int before;
    const int total = block_excl_sum(sh, phase, __builtin_popcount(hit), before);
    const int64_t base = (int64_t)r * ld_bmax + (int64_t)g * kRound;
    int pos = before;
    const int i0 = g * kRound + (int)threadIdx.x * kE;
#pragma unroll
    for (int e = 0; e < kE; ++e)
        if ((hit >> e) & 1u) {
            gkey[base + pos] = key[e];
            gid[base + pos] = i0 + e;
            ++pos;
        }
    if (threadIdx.x == 0) gcount[(int64_t)r * nslices + g] = total;
}

// Block-level reduction of the candidates.  Under the order (score desc,
// entry id asc) every Top-K entry lies in one of the top-K blocks under the
// order (block max desc, block id asc): if K blocks precede an entry's block,
// each holds an entry at its maximum that precedes the entry itself (a larger
// score, or an equal one at a lower id).  So the Top-K is taken among the
// 8*K entries of those blocks only.
template <bool FULL>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ scores, int64_t ld_scores, const float* __restrict__ bmax,
    int64_t ld_bmax, const int32_t* __restrict__ row_len, int32_t n_cap, const int32_t* __restrict__ pool_in,
    int32_t K, int32_t P, int32_t* __restrict__ topk, int32_t* __restrict__ pool_out,
    const uint32_t* __restrict__ gkey_g, const int32_t* __restrict__ gid_g, const int32_t* __restrict__ gcount,
    int32_t nslices, const int32_t* __restrict__ row_seq, PageMap pm, int32_t* __restrict__ rows_out,
    int32_t* __restrict__ cand_out)
{
    __shared__ typename std::conditional<FULL, SelectLdsFull, SelectLds>::type L;
    const int r = blockIdx.x;
    const int n = min(max(row_len[r], 0), n_cap);   // as the score kernel clamps it
    const int nb = (n + 7) >> 3;
    const float* sc = scores + (int64_t)r * ld_scores;
    const float* bm = FULL ? bmax + (int64_t)r * ld_bmax : nullptr;
    RegKeys reg;
    int phase = 0;
    for (int i = threadIdx.x; i < 2 * kHistSpan; i += kSelThreads) L.sh.hist[i] = 0;
    const int* cand;        // candidate blocks
    const int* cand_slot;   // their pool slots (Reindex)
    int ncb;                // number of candidate blocks
    bool preloaded = false; // reg already holds the candidates' keys
    int pool_late = -1;     // Full, pool = A: its size, the pool being written at the end

    if constexpr (FULL) {
        // A = the top max(P, K) blocks (all of them when nb is smaller) and B
        // = the top min(P, K) blocks (B lies in A); the pool and the
        // candidate blocks are A and B in the roles their sizes give.  Both
        // thresholds come from one two-target radix select (one target when
        // there is no pool); then A goes to L.blocks and B, when smaller, to
        // the pool output or L.cblk.
        const int big = K > P ? K : P;
        const int small = K < P ? K : P;
        const BlockMaxSrc bsrc{bm, nb};
        int na = -1, nsm = 0;
        // Selection of A and B over the items of `src` (block id of item i:
        // id(i)), whose keys `rg` holds.
        auto select_ab = [&](const auto& src, const RegKeys& rg, auto id) {
            SelState sa, sb;
            if (P > 0) {
                // A and B in the same rounds and scans (when A holds at most
                // `small` items, B selects all of them: B = A)
                radix_select2(L.sh, phase, src, rg, big, small, sa, sb);
                int32_t* po = pool_out + (int64_t)r * P;
                const int2 nn = select_compact2(L.sh, phase, src, rg, sa, sb,
                    [&](int pos, int i) { if (pos < big) L.blocks[pos] = id(i); },
                    [&](int pos, int i) {
                        if (pos < small) {
                            if (P >= K) L.cblk[pos] = id(i);
                            else po[pos] = id(i);
                        }
                    });
                na = nn.x < big ? nn.x : big;
                nsm = nn.y < small ? nn.y : small;
            } else {
                sa = radix_select(L.sh, phase, src, rg, big);
                na = select_compact(L.sh, phase, src, rg, sa, [&](int pos, int i, int) {
                    if (pos < big) L.blocks[pos] = id(i);
                }, [](int) { return 0; });
                na = na < big ? na : big;
                nsm = na;   // B = A
            }
        };
        const int ns = (nb + kRound - 1) / kRound;
        if (nb > kRegRounds * kRound && (!gcount || ns <= kMaxSlices)) {
            // Long row: every pass over all block maxima re-reads memory, so
            // the blocks whose key is at or above a sampled threshold are
            // gathered first, in block order: by k_prefilter, slice by slice
            // across many workgroups (when the rows are few), or here in one
            // pass.  When that set holds at least `big` blocks (so the big-th
            // largest key is at or above the threshold and every block of A is
            // in the set, ties included) and fits, A is selected from it;
            // otherwise the full selection below runs.
            int cnt = 0;
            if (gcount) {
                int* off = L.blocks;   // slice offsets, ns <= kMaxSlices <= kMaxP
                for (int c0 = 0; c0 < ns; c0 += kSelThreads) {
                    const int gi = c0 + (int)threadIdx.x;
                    const int c = gi < ns ? gcount[(int64_t)r * nslices + gi] : 0;
                    int before;
                    const int total = block_excl_sum(L.sh, phase, c, before);
                    if (gi < ns) off[gi] = cnt + before;
                    cnt += total;
                }
                __syncthreads();
                if (cnt >= big && cnt <= kGatherCap) {
                    for (int i = threadIdx.x; i < cnt; i += kSelThreads) {
                        int lo_s = 0, hi_s = ns - 1;   // last slice whose offset is <= i
                        while (lo_s < hi_s) {
                            const int mid = (lo_s + hi_s + 1) >> 1;
                            if (off[mid] <= i) lo_s = mid;
                            else hi_s = mid - 1;
                        }
                        const int64_t at = (int64_t)r * ld_bmax + (int64_t)lo_s * kRound + (i - off[lo_s]);
                        L.gkey[padded(i)] = gkey_g[at];
                        L.gid[i] = gid_g[at];
                    }
                }
            } else {
                const uint32_t lo = prefilter_threshold(L.sh, phase, bm, nb, big);
                load_regs(bsrc, reg);
                for_rounds(bsrc, reg, [&](int rd, const uint32_t (&key)[kE]) {
                    uint32_t hit = 0u;
#pragma unroll
                    for (int e = 0; e < kE; ++e) hit |= (key[e] >= lo ? 1u : 0u) << e;
                    int before;
                    const int total = block_excl_sum(L.sh, phase, __builtin_popcount(hit), before);
                    if (hit != 0u) {   // few blocks pass: most lanes and waves skip the writes
                        int pos = cnt + before;
                        const int i0 = rd * kRound + (int)threadIdx.x * kE;
#pragma unroll
                        for (int e = 0; e < kE; ++e)
                            if ((hit >> e) & 1u) {
                                if (pos < kGatherCap) { L.gkey[padded(pos)] = key[e]; L.gid[pos] = i0 + e; }
                                ++pos;
                            }
                    }
                    cnt += total;
                });
            }
            __syncthreads();
            if (cnt >= big && cnt <= kGatherCap) {
                const LdsKeySrc gsrc{{}, L.gkey, cnt};
                RegKeys greg;
                load_regs(gsrc, greg);
                select_ab(gsrc, greg, [&](int i) { return L.gid[i]; });
            }
            if (na < 0 && gcount) load_regs(bsrc, reg);
        } else {
            load_regs(bsrc, reg);
        }
        if (na < 0) select_ab(bsrc, reg, [](int i) { return i; });
        __syncthreads();
        cand = L.blocks;
        cand_slot = nullptr;
        ncb = na;
        if (P > 0) {
            int32_t* po = pool_out + (int64_t)r * P;
            if (P >= K) {   // pool = A, candidates = B
                // (written at the end, where no barrier follows the stores;
                // L.blocks is only read from here on)
                if (cand_out)
                    for (int i = threadIdx.x; i < P; i += kSelThreads) po[i] = i < na ? L.blocks[i] : -1;
                else
                    pool_late = na;
                if (na > K) {
                    cand = L.cblk;
                    ncb = nsm;
                }
            } else {        // candidates = A, pool = B
                if (na <= P)
                    for (int i = threadIdx.x; i < na; i += kSelThreads) po[i] = L.blocks[i];
                for (int i = nsm + threadIdx.x; i < P; i += kSelThreads) po[i] = -1;
            }
        }
        // Blocks only (the entries' scores are not at hand): the candidate
        // blocks, ascending, -1 padded to K, for rescoring.
        if (cand_out) {
            int32_t* co = cand_out + (int64_t)r * K;
            for (int i = threadIdx.x; i < K; i += kSelThreads) co[i] = i < ncb ? cand[i] : -1;
            return;   // uniform in the workgroup
        }
    } else {
        // Items are the pool slots in block-id order: the pool as given when
        // its valid ids already ascend, else sorted by id first, so that the
        // lowest-item tie rule of the selection is the lowest-id rule.  The
        // scores are stored by pool slot with -inf where a slot holds no
        // visible entry, so for a pool in order (the usual case: a Full
        // layer's pool) the keys are the scores in slot order; they are
        // requested before the order is checked.
        // (the pool ids are requested first, so that their latency and the
        // scores' overlap)
        const int32_t* pl = pool_in + (int64_t)r * P;
        constexpr int PPT = kMaxP / kSelThreads;
        int pb[PPT], pb2[PPT];
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + k * kSelThreads;
            pb[k] = i < P ? pl[i] : -1;
            pb2[k] = i + 1 < P ? pl[i + 1] : -1;
        }
        load_regs(SlotSrc{{}, sc, P}, reg);
        preloaded = true;
        if (threadIdx.x == 0) L.flag = 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + k * kSelThreads;
            if (i < P) {
                const int b = pb[k];
                const bool ok = b >= 0 && b < nb;
                L.blocks[i] = ok ? b : -1;
                L.slots[i] = i;
                if (i + 1 < P) {
                    const int b2 = pb2[k];
                    if (b2 >= 0 && b2 < nb && !(ok && b < b2)) L.flag = 1;
                }
            }
        }
        __syncthreads();
        if (L.flag) {
            int np2 = 1;
            while (np2 < P) np2 <<= 1;
            for (int i = threadIdx.x; i < np2; i += kSelThreads) {
                const unsigned hi = i < P && L.blocks[i] >= 0 ? (unsigned)L.blocks[i] : 0x7FFFFFFFu;
                L.sortbuf[i] = i < P ? ((unsigned long long)hi << 32) | (unsigned)i : ~0ull;
            }
            __syncthreads();
            bitonic_sort(L.sortbuf, np2);
            // a block listed more than once counts once: after the sort its
            // copies are adjacent, and only the first (lowest slot) is kept
            for (int i = threadIdx.x; i < P; i += kSelThreads) {
                const unsigned long long v = L.sortbuf[i];
                const unsigned hi = (unsigned)(v >> 32);
                const bool dup = i > 0 && hi != 0x7FFFFFFFu && (unsigned)(L.sortbuf[i - 1] >> 32) == hi;
                CSA2_DCHECK(dup);
                L.blocks[i] = hi == 0x7FFFFFFFu || dup ? -1 : (int)hi;
                L.slots[i] = (int)(unsigned)v;
            }
            __syncthreads();
            preloaded = false;   // keys in sorted order are read below
        }
        // The pool holds at most 2048 x 8 positions, which the registers
        // hold whole: the Top-K is selected among all of them at once.
        cand = L.blocks;
        cand_slot = L.slots;
        ncb = P;
    }
    __syncthreads();

    // The selected ids are kept in LDS (the sort buffer is free by now) and
    // written out after the compaction, so no barrier of the compaction waits
    // for global stores.  Paged caches: the cache row of each selected entry
    // is written too (-1 when beyond 32-bit row numbers), so attention needs
    // no separate translation.
    int32_t* tr = rows_out ? rows_out + (int64_t)r * K : nullptr;
    int* const sel_ids = reinterpret_cast<int*>(L.sortbuf);   // kMaxP 64-bit words hold kMaxK ids
    static_assert(sizeof(L.sortbuf) >= kMaxK * sizeof(int), "selected ids fit the sort buffer");

    // Top-K among the candidate blocks' entries, written in item order, which
    // is ascending entry order.
    const CandSrc csrc{{}, sc, cand, cand_slot, ncb, n};
    if (!preloaded) load_regs(csrc, reg);
    const SelState st = radix_select(L.sh, phase, csrc, reg, K);
    int32_t* to = topk + (int64_t)r * K;
    // (a thread's kE items of a round are the 8 positions of one candidate
    // block: its id is read once per round)
    static_assert(kE == 8, "one candidate block per thread and round");
    int nk = select_compact(L.sh, phase, csrc, reg, st, [&](int pos, int c, int blk) {
        if (pos < K) sel_ids[pos] = blk * 8 + (c & 7);
    }, [&](int rd) {
        const int cb = rd * kSelThreads + (int)threadIdx.x;
        return cb < ncb ? cand[cb] : 0;
    });
    nk = nk < K ? nk : K;
    for (int i = threadIdx.x; i < K; i += kSelThreads) {   // (select_compact ends with a barrier)
        to[i] = i < nk ? sel_ids[i] : -1;
        if (tr && i >= nk) tr[i] = -1;
    }
    if (tr) {   // (select_compact ends with a barrier: sel_ids is complete)
        const int seq = row_seq[r];
        for (int i = threadIdx.x; i < nk; i += kSelThreads) {
            const int j = sel_ids[i];
            const int64_t ph = pm.row_on(pm.page_id(seq, j >> pm.shift), j);
            tr[i] = ph <= 0x7FFFFFFF ? (int32_t)ph : -1;
        }
    }
    if (FULL && pool_late >= 0) {
        int32_t* po = pool_out + (int64_t)r * P;
        for (int i = threadIdx.x; i < P; i += kSelThreads) po[i] = i < pool_late ? L.blocks[i] : -1;
    }
}

template <bool REINDEX, bool PAGED>
void launch_score(int HT, int KS, dim3 grid, hipStream_t st, const uint8_t* qI, const float* w,
                  const uint8_t* ikeys, const int64_t* seq_start, const PageMap& pm, const int32_t* row_seq,
                  const int32_t* row_len, int32_t n_cap, const int32_t* pool, int32_t Hi, int32_t Di, int32_t P,
                  float* scores, int64_t lds, float* bm, int64_t ldb, int re_chunk)
{
#define CSA2_SCORE(ht, ks)                                                                                 \
    if (HT == ht && KS == ks) {                                                                            \
        hipLaunchKernelGGL((k_index_score<ht, ks, REINDEX, PAGED>), grid, dim3(256), 0, st, qI, w, ikeys,   \
                           seq_start, pm, row_seq, row_len, n_cap, pool, Hi, Di, P, scores, lds, bm, ldb,    \
                           re_chunk);                                                                      \
        return;                                                                                            \
    }
    CSA2_SCORE(1, 1) CSA2_SCORE(2, 1) CSA2_SCORE(3, 1) CSA2_SCORE(4, 1)
    CSA2_SCORE(1, 2) CSA2_SCORE(2, 2) CSA2_SCORE(3, 2) CSA2_SCORE(4, 2)
#undef CSA2_SCORE
}

template <bool REINDEX>
void launch_score(bool paged, int HT, int KS, dim3 grid, hipStream_t st, const uint8_t* qI, const float* w,
                  const uint8_t* ikeys, const int64_t* seq_start, const PageMap& pm, const int32_t* row_seq,
                  const int32_t* row_len, int32_t n_cap, const int32_t* pool, int32_t Hi, int32_t Di, int32_t P,
                  float* scores, int64_t lds, float* bm, int64_t ldb, int re_chunk = 0)
{
    if (paged)
        launch_score<REINDEX, true>(HT, KS, grid, st, qI, w, ikeys, seq_start, pm, row_seq, row_len, n_cap, pool,
                                    Hi, Di, P, scores, lds, bm, ldb, re_chunk);
    else
        launch_score<REINDEX, false>(HT, KS, grid, st, qI, w, ikeys, seq_start, pm, row_seq, row_len, n_cap, pool,
                                     Hi, Di, P, scores, lds, bm, ldb, re_chunk);
}

// Block-table arguments of the paged calls; shift = log2(page_rows).
csa2_status_t check_pages(const char* who, const int32_t* bt, int32_t max_pages, int32_t page_rows,
                          int64_t cache_rows, PageMap& pm)
{
    CSA2_REQUIRE(bt, CSA2_ERR_NULL, "%s: block_table is NULL", who);
    CSA2_REQUIRE(max_pages >= 1, CSA2_ERR_SHAPE, "%s: max_pages=%d < 1", who, max_pages);
    CSA2_REQUIRE(cache_rows >= 1, CSA2_ERR_SHAPE, "%s: cache_rows=%lld < 1", who, (long long)cache_rows);
    CSA2_REQUIRE(page_rows >= 8 && page_rows <= (1 << 20) && (page_rows & (page_rows - 1)) == 0,
                 CSA2_ERR_UNSUPPORTED, "%s: page_rows=%d must be a power of two in [8, 2^20]", who, page_rows);
    pm.bt = bt;
    pm.max_pages = max_pages;
    pm.shift = __builtin_ctz((unsigned)page_rows);
    pm.cache_rows = cache_rows;
    return CSA2_OK;
}

int64_t full_ld(int32_t max_len) { return ((int64_t)max_len + kFullChunk - 1) / kFullChunk * kFullChunk; }
// Slices of kRound block maxima per row, and whether rows this long use the
// pre-filter (then the workspace also holds its gathered keys, ids and counts).
int64_t full_slices(int64_t ld) { return (ld / 8 + kRound - 1) / kRound; }
bool full_prefilter(int64_t ld) { return ld / 8 > (int64_t)kRegRounds * kRound; }
int64_t reindex_ld(int32_t P) { return ((int64_t)P * 8 + kReChunkMax - 1) / kReChunkMax * kReChunkMax; }

// Pool slots per Reindex-score workgroup: the largest of 1024, 512 and 256
// that still gives at least two workgroups per compute unit (a few rows take
// smaller chunks, so that their pools spread over the whole GPU; many rows
// take larger ones, which load their keys with fewer, longer workgroups).
// Every choice divides reindex_ld(P).
int reindex_chunk(int32_t R, int64_t ld)
{
    for (int c = kReChunkMax; c > 256; c /= 2)
        if ((int64_t)R * (ld / c) >= 512) return c;
    return 256;
}

csa2_status_t check_indexer_dims(const char* who, int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t block)
{
    CSA2_REQUIRE(R >= 0, CSA2_ERR_SHAPE, "%s: R=%d < 0", who, R);
    CSA2_REQUIRE(Hi >= 1, CSA2_ERR_SHAPE, "%s: Hi=%d < 1", who, Hi);
    CSA2_REQUIRE(Hi <= 64, CSA2_ERR_UNSUPPORTED, "%s: Hi=%d > 64", who, Hi);
    CSA2_REQUIRE(Di >= 16 && Di % 16 == 0, CSA2_ERR_SHAPE, "%s: Di=%d must be a positive multiple of 16", who, Di);
    CSA2_REQUIRE(Di % 32 == 0 && Di <= 256, CSA2_ERR_UNSUPPORTED, "%s: Di=%d must be a multiple of 32 and <= 256", who, Di);
    CSA2_REQUIRE(K >= 1, CSA2_ERR_SHAPE, "%s: K=%d < 1", who, K);
    CSA2_REQUIRE(K <= kMaxK, CSA2_ERR_UNSUPPORTED, "%s: K=%d > %d", who, K, kMaxK);
    CSA2_REQUIRE(block >= 1, CSA2_ERR_SHAPE, "%s: block=%d < 1", who, block);
    CSA2_REQUIRE(block == 8, CSA2_ERR_UNSUPPORTED, "%s: block=%d (only 8 is supported)", who, block);
    return CSA2_OK;
}

}  // namespace

extern "C" size_t csa2_index_full_workspace_bytes(int32_t R, int32_t max_len, int32_t Hi, int32_t K, int32_t P,
                                                  int32_t block)
{
    (void)Hi; (void)P; (void)block;
    if (R < 0 || max_len < 0) return 0;
    const int64_t ld = full_ld(max_len);
    if (R >= kGemmMinRows && K >= 1 && K <= kMaxK) {
        // per batch of rows: the block maxima, the candidate blocks and their entries' scores
        const size_t rb = R < kGemmBatchRows ? (size_t)R : (size_t)kGemmBatchRows;
        return csa2::align_up(rb * (ld / 8) * 4, 256) + csa2::align_up(rb * K * 4, 256) +
               csa2::align_up(rb * reindex_ld(K) * 4, 256);
    }
    size_t b = csa2::align_up((size_t)R * ld * 4, 256) + csa2::align_up((size_t)R * (ld / 8) * 4, 256);
    if (full_prefilter(ld) && R < kPrefilterRows)
        b += 2 * csa2::align_up((size_t)R * (ld / 8) * 4, 256) + csa2::align_up((size_t)R * full_slices(ld) * 4, 256);
    return b;
}

namespace {
template <bool PAGED>
void launch_bmax(int HT, int KS, dim3 grid, hipStream_t st, const uint8_t* qI, const float* w, const uint8_t* ikeys,
                 const int64_t* seq_start, const PageMap& pm, const int32_t* row_seq, const int32_t* row_len,
                 int32_t n_cap, int32_t R, int32_t Hi, int32_t Di, float* bm, int64_t ldb, int32_t split_keys)
{
#define CSA2_BMAX(ht, ks)                                                                                   \
    if (HT == ht && KS == ks) {                                                                             \
        hipLaunchKernelGGL((k_index_bmax<ht, ks, PAGED>), grid, dim3(kGemmRows * CSA2_WAVE), 0, st, qI, w, ikeys, \
                           seq_start, pm, row_seq, row_len, n_cap, R, Hi, Di, bm, ldb, split_keys);       \
        return;                                                                                             \
    }
    CSA2_BMAX(1, 1) CSA2_BMAX(2, 1) CSA2_BMAX(3, 1) CSA2_BMAX(4, 1)
    CSA2_BMAX(1, 2) CSA2_BMAX(2, 2) CSA2_BMAX(3, 2) CSA2_BMAX(4, 2)
#undef CSA2_BMAX
}

// Full mode for many rows (a prefill chunk), in batches of kGemmBatchRows:
// block maxima by the GEMM kernel (key tiles shared by a workgroup's rows),
// the pool and the top-K candidate blocks from them (every Top-K entry lies
// in one of those blocks, see k_select), then the candidate blocks' entries
// rescored and the Top-K taken among them, as Reindex does for its pool.  No
// score of every entry is ever stored.  Arguments are validated by the caller.
csa2_status_t index_full_gemm(const uint8_t* qI, const float* w, const uint8_t* ikeys, const int64_t* seq_start,
                              const PageMap* pmp, const int32_t* row_seq, const int32_t* row_len, int32_t R,
                              int32_t Hi, int32_t Di, int32_t max_len, int32_t K, int32_t P, int32_t* topk_idx,
                              int32_t* topk_rows, int32_t* pool_blocks, void* workspace, void* stream)
{
    const int64_t ld = full_ld(max_len);
    const int32_t rb = R < kGemmBatchRows ? R : kGemmBatchRows;
    char* w8 = static_cast<char*>(workspace);
    float* bm = reinterpret_cast<float*>(w8);
    w8 += csa2::align_up((size_t)rb * (ld / 8) * 4, 256);
    int32_t* cand = reinterpret_cast<int32_t*>(w8);
    w8 += csa2::align_up((size_t)rb * K * 4, 256);
    float* resc = reinterpret_cast<float*>(w8);
    const int64_t rld = reindex_ld(K);
    const int chunk = reindex_chunk(rb, rld);
    hipStream_t st = csa2::as_stream(stream);
    const int HT = (Hi + 15) / 16, KS = (Di + 127) / 128;
    const PageMap pm = pmp ? *pmp : PageMap{nullptr, 0, 0, 0};
    // key ranges of about kGemmSplitKeys, all of one size in whole tiles (the
    // grid then comes to whole multiples of the row tiles, without a short last range)
    int64_t nsplit = max_len / kGemmSplitKeys;
    nsplit = nsplit < 1 ? (max_len > 0 ? 1 : 0) : nsplit;
    const int64_t tiles = ((int64_t)max_len + kGemmTile - 1) / kGemmTile;
    const int32_t split_keys = nsplit > 0 ? (int32_t)((tiles + nsplit - 1) / nsplit * kGemmTile) : 0;
    if (nsplit > 0) nsplit = (max_len + split_keys - 1) / split_keys;
    for (int32_t b0 = 0; b0 < R; b0 += rb) {
        const int32_t nr = R - b0 < rb ? R - b0 : rb;
        const uint8_t* q_b = qI + (int64_t)b0 * Hi * Di;
        const float* w_b = w + (int64_t)b0 * Hi;
        if (nsplit > 0) {
            const dim3 grid((unsigned)nsplit, (unsigned)((nr + kGemmRows - 1) / kGemmRows));
            if (pmp)
                launch_bmax<true>(HT, KS, grid, st, q_b, w_b, ikeys, seq_start, pm, row_seq + b0, row_len + b0, max_len,
                                  nr, Hi, Di, bm, ld / 8, split_keys);
            else
                launch_bmax<false>(HT, KS, grid, st, q_b, w_b, ikeys, seq_start, pm, row_seq + b0, row_len + b0,
                                   max_len, nr, Hi, Di, bm, ld / 8, split_keys);
        }
        hipLaunchKernelGGL(k_select<true>, dim3((unsigned)nr), dim3(kSelThreads), 0, st, nullptr, 0, bm, ld / 8,
                           row_len + b0, max_len, nullptr, K, P, topk_idx + (int64_t)b0 * K,
                           pool_blocks ? pool_blocks + (int64_t)b0 * P : nullptr, nullptr, nullptr, nullptr, 0,
                           row_seq + b0, pm, nullptr, cand);
        launch_score<true>(pmp != nullptr, HT, KS, dim3((unsigned)(rld / chunk), (unsigned)nr), st, q_b, w_b, ikeys,
                           seq_start, pm, row_seq + b0, row_len + b0, max_len, cand, Hi, Di, K, resc, rld, nullptr, 0,
                           chunk);
        hipLaunchKernelGGL(k_select<false>, dim3((unsigned)nr), dim3(kSelThreads), 0, st, resc, rld, nullptr, 0,
                           row_len + b0, max_len, cand, K, K, topk_idx + (int64_t)b0 * K, nullptr, nullptr, nullptr,
                           nullptr, 0, row_seq + b0, pm, pmp && topk_rows ? topk_rows + (int64_t)b0 * K : nullptr,
                           nullptr);
    }
    return CSA2_FINISH(st, "index_full");
}

csa2_status_t index_full_impl(const uint8_t* qI, const float* w, const uint8_t* ikeys, const int64_t* seq_start,
                              const PageMap* pmp, const int32_t* row_seq, const int32_t* row_len, int32_t R,
                              int32_t Hi, int32_t Di, int32_t max_len, int32_t K, int32_t P, int32_t block,
                              int32_t* topk_idx, int32_t* topk_rows, int32_t* pool_blocks, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    csa2_status_t s = check_indexer_dims("index_full", R, Hi, Di, K, block);
    if (s != CSA2_OK) return s;
    CSA2_REQUIRE(P >= 0, CSA2_ERR_SHAPE, "index_full: P=%d < 0", P);
    CSA2_REQUIRE(P <= kMaxP, CSA2_ERR_UNSUPPORTED, "index_full: P=%d > %d", P, kMaxP);
    CSA2_REQUIRE((P == 0) == (pool_blocks == nullptr), CSA2_ERR_SHAPE,
                 "index_full: pool_blocks must be NULL exactly when P == 0");
    CSA2_REQUIRE(max_len >= 0, CSA2_ERR_SHAPE, "index_full: max_len=%d < 0", max_len);
    CSA2_REQUIRE(max_len <= 0x7FFFFFFF - 2 * kFullChunk, CSA2_ERR_UNSUPPORTED, "index_full: max_len too large");
    if (R == 0) return CSA2_OK;
    CSA2_REQUIRE(qI && w && ikeys && (seq_start || pmp) && row_seq && row_len && topk_idx, CSA2_ERR_NULL,
                 "index_full: NULL pointer argument");
    CSA2_REQUIRE(R <= 65535, CSA2_ERR_UNSUPPORTED, "index_full: R=%d > 65535", R);
    const size_t need = csa2_index_full_workspace_bytes(R, max_len, Hi, K, P, block);
    CSA2_REQUIRE(workspace && workspace_bytes >= need && ((uintptr_t)workspace & 255) == 0,
                 CSA2_ERR_WORKSPACE, "index_full: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                 need, workspace_bytes);
    if (R >= kGemmMinRows)
        return index_full_gemm(qI, w, ikeys, seq_start, pmp, row_seq, row_len, R, Hi, Di, max_len, K, P, topk_idx,
                               topk_rows, pool_blocks, workspace, stream);
    const int64_t ld = full_ld(max_len);
    char* w8 = static_cast<char*>(workspace);
    float* scores = reinterpret_cast<float*>(w8);
    w8 += csa2::align_up((size_t)R * ld * 4, 256);
    float* bm = reinterpret_cast<float*>(w8);
    w8 += csa2::align_up((size_t)R * (ld / 8) * 4, 256);
    uint32_t* gkey = nullptr;
    int32_t* gid = nullptr;
    int32_t* gcount = nullptr;
    const int64_t nslices = full_slices(ld);
    // The separate pre-filter spreads long rows over many workgroups; with
    // enough rows to occupy the GPU the selector's own one-pass gather is
    // cheaper (it samples the threshold once per row instead of once per slice).
    if (full_prefilter(ld) && R < kPrefilterRows) {
        gkey = reinterpret_cast<uint32_t*>(w8);
        w8 += csa2::align_up((size_t)R * (ld / 8) * 4, 256);
        gid = reinterpret_cast<int32_t*>(w8);
        w8 += csa2::align_up((size_t)R * (ld / 8) * 4, 256);
        gcount = reinterpret_cast<int32_t*>(w8);
    }
    hipStream_t st = csa2::as_stream(stream);
    const int HT = (Hi + 15) / 16, KS = (Di + 127) / 128;
    const PageMap pm = pmp ? *pmp : PageMap{nullptr, 0, 0, 0};
    if (max_len > 0) {
        dim3 grid((unsigned)(ld / kFullChunk), (unsigned)R);
        launch_score<false>(pmp != nullptr, HT, KS, grid, st, qI, w, ikeys, seq_start, pm, row_seq, row_len,
                            max_len, nullptr, Hi, Di, 0, scores, ld, bm, ld / 8);
    }
    if (gcount) {
        const int32_t big = K > P ? K : P;
        hipLaunchKernelGGL(k_prefilter, dim3((unsigned)nslices, (unsigned)R), dim3(kSelThreads), 0, st, bm, ld / 8,
                           row_len, max_len, big, gkey, gid, gcount, (int32_t)nslices);
    }
    hipLaunchKernelGGL(k_select<true>, dim3((unsigned)R), dim3(kSelThreads), 0, st, scores, ld, bm, ld / 8,
                       row_len, max_len, nullptr, K, P, topk_idx, pool_blocks, gkey, gid, gcount, (int32_t)nslices, row_seq, pm,
                       pmp ? topk_rows : nullptr, nullptr);
    return CSA2_FINISH(st, "index_full");
}
}  // namespace

extern "C" csa2_status_t csa2_index_full(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                         const int64_t* seq_start, const int32_t* row_seq,
                                         const int32_t* row_len, int32_t R, int32_t Hi, int32_t Di,
                                         int32_t max_len, int32_t K, int32_t P, int32_t block,
                                         int32_t* topk_idx, int32_t* pool_blocks, void* workspace,
                                         size_t workspace_bytes, void* stream)
{
    if (!seq_start && R > 0) return csa2::fail(CSA2_ERR_NULL, "index_full: seq_start is NULL");
    return index_full_impl(qI, w, ikeys, seq_start, nullptr, row_seq, row_len, R, Hi, Di, max_len, K, P, block,
                           topk_idx, nullptr, pool_blocks, workspace, workspace_bytes, stream);
}

extern "C" csa2_status_t csa2_index_full_paged(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                               int64_t cache_rows, const int32_t* block_table, int32_t max_pages,
                                               int32_t page_rows, const int32_t* row_seq, const int32_t* row_len,
                                               int32_t R, int32_t Hi, int32_t Di, int32_t max_len, int32_t K,
                                               int32_t P, int32_t block, int32_t* topk_idx, int32_t* topk_rows,
                                               int32_t* pool_blocks, void* workspace, size_t workspace_bytes,
                                               void* stream)
{
    PageMap pm;
    if (R > 0) {
        const csa2_status_t s = check_pages("index_full_paged", block_table, max_pages, page_rows, cache_rows, pm);
        if (s != CSA2_OK) return s;
    }
    return index_full_impl(qI, w, ikeys, nullptr, &pm, row_seq, row_len, R, Hi, Di, max_len, K, P, block, topk_idx,
                           topk_rows, pool_blocks, workspace, workspace_bytes, stream);
}

extern "C" size_t csa2_index_reindex_workspace_bytes(int32_t R, int32_t Hi, int32_t K, int32_t P, int32_t block)
{
    (void)Hi; (void)K; (void)block;
    if (R < 0 || P < 0) return 0;
    return csa2::align_up((size_t)R * reindex_ld(P) * 4, 256);   // one score per pool slot
}

namespace {
csa2_status_t index_reindex_impl(const uint8_t* qI, const float* w, const uint8_t* ikeys, const int64_t* seq_start,
                                 const PageMap* pmp, const int32_t* row_seq, const int32_t* row_len,
                                 const int32_t* pool_blocks, int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t P,
                                 int32_t block, int32_t* topk_idx, int32_t* topk_rows, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    csa2_status_t s = check_indexer_dims("index_reindex", R, Hi, Di, K, block);
    if (s != CSA2_OK) return s;
    CSA2_REQUIRE(P >= 1, CSA2_ERR_SHAPE, "index_reindex: P=%d < 1", P);
    CSA2_REQUIRE(P <= kMaxP, CSA2_ERR_UNSUPPORTED, "index_reindex: P=%d > %d", P, kMaxP);
    if (R == 0) return CSA2_OK;
    CSA2_REQUIRE(qI && w && ikeys && (seq_start || pmp) && row_seq && row_len && pool_blocks && topk_idx,
                 CSA2_ERR_NULL, "index_reindex: NULL pointer argument");
    CSA2_REQUIRE(R <= 65535, CSA2_ERR_UNSUPPORTED, "index_reindex: R=%d > 65535", R);
    const size_t need = csa2_index_reindex_workspace_bytes(R, Hi, K, P, block);
    CSA2_REQUIRE(workspace && workspace_bytes >= need && ((uintptr_t)workspace & 255) == 0,
                 CSA2_ERR_WORKSPACE, "index_reindex: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                 need, workspace_bytes);
    const int64_t ld = reindex_ld(P);
    float* scores = static_cast<float*>(workspace);
    hipStream_t st = csa2::as_stream(stream);
    const int HT = (Hi + 15) / 16, KS = (Di + 127) / 128;
    const int chunk = reindex_chunk(R, ld);
    dim3 grid((unsigned)(ld / chunk), (unsigned)R);
    const PageMap pm = pmp ? *pmp : PageMap{nullptr, 0, 0, 0};
    launch_score<true>(pmp != nullptr, HT, KS, grid, st, qI, w, ikeys, seq_start, pm, row_seq, row_len, 0x7FFFFFFF,
                       pool_blocks, Hi, Di, P, scores, ld, nullptr, 0, chunk);
    hipLaunchKernelGGL(k_select<false>, dim3((unsigned)R), dim3(kSelThreads), 0, st, scores, ld, nullptr, 0,
                       row_len, 0x7FFFFFFF, pool_blocks, K, P, topk_idx, nullptr, nullptr, nullptr, nullptr, 0, row_seq, pm,
                       pmp ? topk_rows : nullptr, nullptr);
    return CSA2_FINISH(st, "index_reindex");
}
}  // namespace

extern "C" csa2_status_t csa2_index_reindex(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                            const int64_t* seq_start, const int32_t* row_seq,
                                            const int32_t* row_len, const int32_t* pool_blocks,
                                            int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t P,
                                            int32_t block, int32_t* topk_idx, void* workspace,
                                            size_t workspace_bytes, void* stream)
{
    if (!seq_start && R > 0 && P >= 1) return csa2::fail(CSA2_ERR_NULL, "index_reindex: seq_start is NULL");
    return index_reindex_impl(qI, w, ikeys, seq_start, nullptr, row_seq, row_len, pool_blocks, R, Hi, Di, K, P, block,
                              topk_idx, nullptr, workspace, workspace_bytes, stream);
}

extern "C" csa2_status_t csa2_index_reindex_paged(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                                  int64_t cache_rows, const int32_t* block_table, int32_t max_pages,
                                                  int32_t page_rows, const int32_t* row_seq, const int32_t* row_len,
                                                  const int32_t* pool_blocks, int32_t R, int32_t Hi, int32_t Di,
                                                  int32_t K, int32_t P, int32_t block, int32_t* topk_idx,
                                                  int32_t* topk_rows, void* workspace, size_t workspace_bytes,
                                                  void* stream)
{
    PageMap pm;
    if (R > 0) {
        const csa2_status_t s = check_pages("index_reindex_paged", block_table, max_pages, page_rows, cache_rows, pm);
        if (s != CSA2_OK) return s;
    }
    return index_reindex_impl(qI, w, ikeys, nullptr, &pm, row_seq, row_len, pool_blocks, R, Hi, Di, K, P, block,
                              topk_idx, topk_rows, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------ no-allocation Reindex
//
// csa2_index_reindex_noalloc runs the Reindex kernels with their score buffer
// in a fixed device array instead of a caller workspace, for callers that
// cannot allocate (code under graph capture, tight serving loops).  The array
// lives in this file's device code, one copy per GPU the library runs on, for
// the life of the process; host code never passes its name to a kernel (the
// name is a host-side stand-in): the device address of each GPU's copy is
// looked up once with hipGetSymbolAddress, with that GPU current, and kept.
// The kernels write every score slot they later read, so the array needs no
// clearing between calls; calls that overlap on one GPU share it and race.

static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];   // device address of `scratch`, per device id

// Device address of this GPU's `scratch` (the current device), looked up on
// the first call on that device.
csa2_status_t scratch_address(const char* who, void** out)
{
    int dev = -1;
    const hipError_t e0 = hipGetDevice(&dev);
    if (e0 != hipSuccess) return csa2::fail(CSA2_ERR_LAUNCH, "%s: hipGetDevice: %s", who, hipGetErrorString(e0));
    CSA2_REQUIRE(dev >= 0 && dev < kMaxScratchDevices, CSA2_ERR_UNSUPPORTED, "%s: device %d >= %d", who, dev,
                 kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return csa2::fail(CSA2_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", who, dev,
                              hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return CSA2_OK;
}

}  // namespace

extern "C" csa2_status_t csa2_index_reindex_noalloc(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                                    const int64_t* seq_start, const int32_t* row_seq,
                                                    const int32_t* row_len, const int32_t* pool_blocks, int32_t R,
                                                    int32_t Hi, int32_t Di, int32_t K, int32_t P, int32_t block,
                                                    int32_t* topk_idx, void* stream)
{
    // every argument check of the workspace form runs first (the workspace one
    // is met by construction), then the size limit, then the device lookup
    const size_t need = csa2_index_reindex_workspace_bytes(R, Hi, K, P, block);
    CSA2_REQUIRE(R >= 0 && P >= 1 && P <= kMaxP, R < 0 || P < 1 ? CSA2_ERR_SHAPE : CSA2_ERR_UNSUPPORTED,
                 "index_reindex_noalloc: R=%d, P=%d out of range", R, P);
    CSA2_REQUIRE(need <= (size_t)CSA2_NOALLOC_SCRATCH_BYTES, CSA2_ERR_UNSUPPORTED,
                 "index_reindex_noalloc: R=%d rows with P=%d pool blocks need %zu bytes of scratch, more than the "
                 "fixed %zu (call csa2_index_reindex with a workspace, or split the rows)",
                 R, P, need, (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
    if (R == 0) return index_reindex_impl(qI, w, ikeys, seq_start, nullptr, row_seq, row_len, pool_blocks, R, Hi,
                                          Di, K, P, block, topk_idx, nullptr, nullptr, 0, stream);
    if (!seq_start) return csa2::fail(CSA2_ERR_NULL, "index_reindex_noalloc: seq_start is NULL");
    void* ws = nullptr;
    const csa2_status_t s = scratch_address("index_reindex_noalloc", &ws);
    if (s != CSA2_OK) return s;
    return index_reindex_impl(qI, w, ikeys, seq_start, nullptr, row_seq, row_len, pool_blocks, R, Hi, Di, K, P,
                              block, topk_idx, nullptr, ws, (size_t)CSA2_NOALLOC_SCRATCH_BYTES, stream);
}
