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
//   k_select       One workgroup per query row: exact radix select (11/11/10
//                  bit digits over order-preserving keys, histograms in LDS)
//                  and an ordered compaction, so the outputs come out sorted
//                  and ties resolve to the lowest index.  Full mode selects the
//                  top max(P, K) blocks by block max, then the Top-K entries
//                  inside those blocks only: every Top-K entry lies in one of
//                  the top-K blocks under this order, so the result equals a
//                  Top-K over all entries.
#include "csa2_device.h"
#include "csa2_host.h"

namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / CSA2_WAVE;
constexpr int kMaxK = 2048;
constexpr int kMaxP = 2048;
constexpr int kBins = 2048;
constexpr int kLoadBatch = 16;      // global loads kept in flight per select thread
constexpr int kFullChunk = 1024;     // entries per Full-score workgroup
constexpr int kReChunk = 512;        // pool slots per Reindex-score workgroup

// ------------------------------------------------------------------ scoring

template <int HT, int KS, bool REINDEX>
__global__ __launch_bounds__(256) void k_index_score(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ ikeys,
    const int64_t* __restrict__ seq_start, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ pool, int32_t Hi, int32_t Di,
    int32_t P, float* __restrict__ scores, int64_t ld_scores, float* __restrict__ bmax,
    int64_t ld_bmax)
{
    const int r = blockIdx.y;
    const int n = row_len[r];
    const int lane = lane_id();
    const int wave = threadIdx.x / CSA2_WAVE;
    const int col = lane & 15;       // entry within a 16-entry tile / head within a head tile
    const int grp = lane >> 4;       // 32-byte slice of a 128-byte k-step
    const int chunk = REINDEX ? kReChunk : kFullChunk;
    const int64_t first = (int64_t)blockIdx.x * chunk;
    if (!REINDEX && first >= n) return;
    const int nb = (n + 7) >> 3;
    const uint8_t* keys = ikeys + seq_start[row_seq[r]] * (int64_t)Di;

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
                const int b = slot < (int64_t)P * 8 ? pool[(int64_t)r * P + (slot >> 3)] : -1;
                j = (int64_t)b * 8 + (slot & 7);
                ok[u] = b >= 0 && b < nb && j < n;
            } else {
                j = slot;
                ok[u] = j < n;
            }
            ent[u] = j;
            const int64_t jc = ok[u] ? j : 0;
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
                for (int i = 0; i < 4; ++i) part += wv[t][i] * fmaxf(acc[i], 0.0f);
            }
            part += shfl_xor_f(part, 16);
            part += shfl_xor_f(part, 32);
            const int64_t slot = wbase + (int64_t)(it0 + u) * 16 + col;
            if (REINDEX) {
                if (grp == 0 && slot < (int64_t)P * 8) scores[(int64_t)r * ld_scores + slot] = part;
            } else {
                const int64_t j = ent[u];
                if (grp == 0 && ok[u]) scores[(int64_t)r * ld_scores + j] = part;
                float m = ok[u] ? part : -INFINITY;
                m = fmaxf(m, shfl_xor_f(m, 1));
                m = fmaxf(m, shfl_xor_f(m, 2));
                m = fmaxf(m, shfl_xor_f(m, 4));
                if (grp == 0 && (col & 7) == 0 && j < n) bmax[(int64_t)r * ld_bmax + (j >> 3)] = m;
            }
        }
    }
}

// ------------------------------------------------------------------ selection

struct SelState {
    uint32_t prefix;   // selected keys: (key & mask) > prefix, or == prefix among the first `need`
    uint32_t mask;
    int need;
};

struct SelShared {
    int hist[kBins];
    int wave_a[kSelWaves];
    int wave_b[kSelWaves];
    int digit, above, nvalid;
};

__device__ __forceinline__ uint64_t lanes_below() { const int l = lane_id(); return l ? (~0ull >> (64 - l)) : 0ull; }

// Exclusive block-wide prefix sum of an int in thread order; returns the total.
__device__ __forceinline__ int block_excl_sum(SelShared& sh, int v, int& excl)
{
    const int lane = lane_id(), wave = threadIdx.x / CSA2_WAVE;
    int incl = v;
#pragma unroll
    for (int off = 1; off < CSA2_WAVE; off <<= 1) {
        const int y = __shfl_up(incl, off, CSA2_WAVE);
        if (lane >= off) incl += y;
    }
    __syncthreads();
    if (lane == CSA2_WAVE - 1) sh.wave_a[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int x = sh.wave_a[i];
        if (i < wave) before += x;
        total += x;
    }
    excl = before + incl - v;
    return total;
}

// Items are processed in rounds of kRound; within a round thread t holds the
// kE consecutive items t*kE .. t*kE+kE-1 in registers.  Key 0 marks an
// invalid item (order_key never maps a finite float to 0).  Keys live in LDS
// at padded positions (one spare word per 32) so that the 64 lanes reading
// word t*kE + e of their own run hit 64 different banks.
constexpr int kE = 32;
constexpr int kRound = kSelThreads * kE;
constexpr int kPadded = kRound + kRound / 32;
__device__ __forceinline__ int padded(int i) { return i + (i >> 5); }

// Where the keys come from: an LDS array holding all of them (cnt <= kRound),
// or global floats staged into the LDS array one round at a time.
struct KeySource {
    uint32_t* lds;
    const float* gsrc;   // null when the keys are already in lds
    int cnt;

    __device__ __forceinline__ int rounds() const { return (cnt + kRound - 1) / kRound; }

    __device__ __forceinline__ void stage(int rd) const
    {
        if (!gsrc) return;
        __syncthreads();
        const int base = rd * kRound;
        for (int c0 = 0; c0 < kRound; c0 += kSelThreads * kLoadBatch) {
            float v[kLoadBatch];
#pragma unroll
            for (int u = 0; u < kLoadBatch; ++u) {
                const int c = base + c0 + u * kSelThreads + threadIdx.x;
                v[u] = c < cnt ? gsrc[c] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kLoadBatch; ++u) {
                const int li = c0 + u * kSelThreads + threadIdx.x;
                lds[padded(li)] = base + li < cnt ? order_key(v[u]) : 0u;
            }
        }
        __syncthreads();
    }

    __device__ __forceinline__ void load(int rd, uint32_t (&key)[kE]) const
    {
        if (rounds() > 1) stage(rd);
        const int l0 = threadIdx.x * kE;
        const int i0 = rd * kRound + l0;
#pragma unroll
        for (int e = 0; e < kE; ++e) key[e] = (i0 + e < cnt) ? lds[padded(l0 + e)] : 0u;
    }
};

// Finds the threshold of the k largest keys among the valid items 0..cnt-1.
// The bits shared by every valid key are skipped first (an AND/OR reduction
// finds the highest bit that differs), then radix passes over 11-bit digits
// below it (LDS histograms) narrow to the digit holding the k-th largest key,
// stopping early once a whole digit bin is taken.  get(i) returns the key of
// item i, or 0 when the item is invalid.
__device__ __forceinline__ SelState radix_select(SelShared& sh, const KeySource& src, int k)
{
    constexpr int BPT = kBins / kSelThreads;      // bins per thread in the digit search
    const int lane = lane_id(), wave = threadIdx.x / CSA2_WAVE;
    const int rounds = src.rounds();
    uint32_t key[kE];
    if (rounds == 1) src.load(0, key);
    // population and common prefix of the valid keys
    uint32_t kand = 0xFFFFFFFFu, kor = 0u;
    int nv = 0;
    for (int rd = 0; rd < rounds; ++rd) {
        if (rounds > 1) src.load(rd, key);
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if (key[e]) { kand &= key[e]; kor |= key[e]; ++nv; }
    }
#pragma unroll
    for (int off = 1; off < CSA2_WAVE; off <<= 1) {
        kand &= (uint32_t)__shfl_xor((int)kand, off, CSA2_WAVE);
        kor |= (uint32_t)__shfl_xor((int)kor, off, CSA2_WAVE);
        nv += __shfl_xor(nv, off, CSA2_WAVE);
    }
    __syncthreads();
    if (lane == 0) { sh.hist[wave] = (int)kand; sh.hist[kSelWaves + wave] = (int)kor; sh.wave_b[wave] = nv; }
    __syncthreads();
    kand = 0xFFFFFFFFu; kor = 0u; nv = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        kand &= (uint32_t)sh.hist[w];
        kor |= (uint32_t)sh.hist[kSelWaves + w];
        nv += sh.wave_b[w];
    }
    __syncthreads();
    SelState st{0u, 0u, nv};
    if (nv <= k) return st;                       // everything valid is selected (mask 0)
    const uint32_t diff = kand ^ kor;             // bits that vary among valid keys
    st.mask = diff ? ~((2u << (31 - __builtin_clz(diff))) - 1u) : 0xFFFFFFFFu;
    st.prefix = kand & st.mask;
    st.need = k;
    if (diff == 0u) return st;                    // all valid keys equal: ties only
    int top = 31 - __builtin_clz(diff);           // highest varying bit
    int krem = k;
    while (top >= 0) {
        const int width = top + 1 < 11 ? top + 1 : 11;
        const int shift = top + 1 - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = threadIdx.x; i < kBins; i += kSelThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int rd = 0; rd < rounds; ++rd) {
            if (rounds > 1) src.load(rd, key);
#pragma unroll
            for (int e = 0; e < kE; ++e)
                if (key[e] && (key[e] & st.mask) == st.prefix) atomicAdd(&sh.hist[(key[e] >> shift) & dmask], 1);
        }
        __syncthreads();
        int h[BPT], sum = 0;
#pragma unroll
        for (int b = 0; b < BPT; ++b) { h[b] = sh.hist[kBins - 1 - BPT * threadIdx.x - b]; sum += h[b]; }
        int before;
        block_excl_sum(sh, sum, before);
        int acc = before;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
            if (acc < krem && krem <= acc + h[b]) { sh.digit = kBins - 1 - BPT * threadIdx.x - b; sh.above = acc; }
            acc += h[b];
        }
        __syncthreads();
        const int d = sh.digit;
        krem -= sh.above;
        const int in_bin = sh.hist[d];
        st.prefix |= (uint32_t)d << shift;
        st.mask |= dmask << shift;
        st.need = krem;
        __syncthreads();
        if (in_bin == krem) break;   // the whole bin is taken: no tie to resolve
        top = shift - 1;
    }
    return st;
}

// Ordered compaction: emit(pos, i) for the selected items in item order.  A
// thread counts the keys above the threshold and those equal to it among its
// items; one block scan of the packed counts gives every thread the number of
// selected items before its own (all keys above, plus the first `need` equal
// keys: ties go to the lowest index), and the thread then writes its items in
// order.  Returns the number selected.
template <class Emit>
__device__ __forceinline__ int select_compact(SelShared& sh, const KeySource& src, SelState st, Emit emit)
{
    const int rounds = src.rounds();
    int gt_run = 0, eq_run = 0;
    uint32_t key[kE];
    for (int rd = 0; rd < rounds; ++rd) {
        src.load(rd, key);
        int gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const uint32_t mk = key[e] & st.mask;
            gt += (key[e] && mk > st.prefix) ? 1 : 0;
            eq += (key[e] && mk == st.prefix) ? 1 : 0;
        }
        int before;
        const int total = block_excl_sum(sh, (gt << 16) | eq, before);   // counts < 2^15 per round
        const int gt_before = gt_run + (before >> 16), eq_before = eq_run + (before & 0xFFFF);
        int out = gt_before + (eq_before < st.need ? eq_before : st.need);
        int eq_seen = eq_before;
        const int i0 = rd * kRound + threadIdx.x * kE;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const uint32_t mk = key[e] & st.mask;
            const bool is_gt = key[e] && mk > st.prefix, is_eq = key[e] && mk == st.prefix;
            const bool sel = is_gt || (is_eq && eq_seen < st.need);
            if (sel) emit(out++, i0 + e);
            eq_seen += is_eq ? 1 : 0;
        }
        gt_run += total >> 16;
        eq_run += total & 0xFFFF;
    }
    __syncthreads();
    return gt_run + (eq_run < st.need ? eq_run : st.need);
}

// Bitonic sort (ascending) of n_pow2 ints in LDS.
__device__ void bitonic_sort(int* a, int n_pow2)
{
    for (int k = 2; k <= n_pow2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n_pow2; i += kSelThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const int x = a[i], y = a[ixj];
                    const bool up = (i & k) == 0;
                    if ((x > y) == up) { a[i] = y; a[ixj] = x; }
                }
            }
            __syncthreads();
        }
    }
}

struct SelectLds {
    SelShared sh;
    uint32_t keys[kPadded];     // block-max keys (Full), then candidate keys; padded positions
    int blocks[kMaxP];
    int outbuf[kMaxK];
    int flag;
};

template <bool FULL>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ scores, int64_t ld_scores, const float* __restrict__ bmax,
    int64_t ld_bmax, const int32_t* __restrict__ row_len, const int32_t* __restrict__ pool_in,
    int32_t K, int32_t P, int32_t* __restrict__ topk, int32_t* __restrict__ pool_out)
{
    __shared__ SelectLds L;
    const int r = blockIdx.x;
    const int n = row_len[r];
    const int nb = (n + 7) >> 3;
    const float* sc = scores + (int64_t)r * ld_scores;
    int ncand_blocks;   // candidate blocks listed in L.blocks

    if (FULL) {
        const float* bm = bmax + (int64_t)r * ld_bmax;
        // Block maxima: staged into LDS once when they fit in one round, else
        // round by round inside each pass.
        KeySource bsrc{L.keys, bm, nb};
        if (nb <= kRound) {
            bsrc.stage(0);
            bsrc.gsrc = nullptr;
        }
        const int pint = K > P ? K : P;   // blocks that must hold the Top-K (and the pool)
        if (pool_out && P < K && nb > P) {   // pool smaller than the Top-K block set: select it first
            int32_t* po = pool_out + (int64_t)r * P;
            SelState st = radix_select(L.sh, bsrc, P);
            int np = select_compact(L.sh, bsrc, st, [&](int pos, int i) { if (pos < P) po[pos] = i; });
            np = np < P ? np : P;
            for (int i = np + threadIdx.x; i < P; i += kSelThreads) po[i] = -1;
        }
        if (nb <= pint) {
            for (int i = threadIdx.x; i < nb; i += kSelThreads) L.blocks[i] = i;
            ncand_blocks = nb;
        } else {
            SelState st = radix_select(L.sh, bsrc, pint);
            ncand_blocks = select_compact(L.sh, bsrc, st, [&](int pos, int i) { if (pos < pint) L.blocks[pos] = i; });
            ncand_blocks = ncand_blocks < pint ? ncand_blocks : pint;
        }
        __syncthreads();
        if (pool_out && (P >= K || nb <= P)) {
            int32_t* po = pool_out + (int64_t)r * P;
            const int np = ncand_blocks < P ? ncand_blocks : P;
            for (int i = threadIdx.x; i < P; i += kSelThreads) po[i] = i < np ? L.blocks[i] : -1;
        }
    } else {
        const int32_t* pl = pool_in + (int64_t)r * P;
        if (threadIdx.x == 0) L.flag = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < P; i += kSelThreads) {
            L.blocks[i] = pl[i];
            if (i + 1 < P) {
                const int a = pl[i], b = pl[i + 1];
                if (b >= 0 && (a < 0 || a >= b)) L.flag = 1;   // not strictly ascending
            }
        }
        ncand_blocks = P;
    }
    __syncthreads();

    // Candidate entries: slot c -> block L.blocks[c/8], position 8*block + c%8
    const int ncand = ncand_blocks * 8;
    // Key 0 marks a slot without a visible entry (every finite score maps above
    // it).  Loads are batched so that many are in flight per thread.
    for (int c0 = 0; c0 < ncand; c0 += kSelThreads * kLoadBatch) {
        float v[kLoadBatch];
        bool ok[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int c = c0 + u * kSelThreads + threadIdx.x;
            const int b = c < ncand ? L.blocks[c >> 3] : -1;
            const int64_t j = (int64_t)b * 8 + (c & 7);
            ok[u] = b >= 0 && b < nb && j < n;
            v[u] = ok[u] ? (FULL ? sc[j] : sc[c]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int c = c0 + u * kSelThreads + threadIdx.x;
            if (c < ncand) L.keys[padded(c)] = ok[u] ? order_key(v[u]) : 0u;
        }
    }
    __syncthreads();
    const KeySource csrc{L.keys, nullptr, ncand};
    int32_t* to = topk + (int64_t)r * K;
    SelState st = radix_select(L.sh, csrc, K);
    if (FULL) {
        int nk = select_compact(L.sh, csrc, st,
                                [&](int pos, int c) { if (pos < K) to[pos] = L.blocks[c >> 3] * 8 + (c & 7); });
        nk = nk < K ? nk : K;
        for (int i = nk + threadIdx.x; i < K; i += kSelThreads) to[i] = -1;
    } else {
        int nk = select_compact(L.sh, csrc, st,
                                [&](int pos, int c) { if (pos < K) L.outbuf[pos] = L.blocks[c >> 3] * 8 + (c & 7); });
        nk = nk < K ? nk : K;
        __syncthreads();
        if (L.flag) {   // pool not ascending: sort the selected ids
            int np2 = 1;
            while (np2 < nk) np2 <<= 1;
            for (int i = nk + threadIdx.x; i < np2; i += kSelThreads) L.outbuf[i] = 0x7FFFFFFF;
            __syncthreads();
            bitonic_sort(L.outbuf, np2);
        }
        for (int i = threadIdx.x; i < K; i += kSelThreads) to[i] = i < nk ? L.outbuf[i] : -1;
    }
}

template <bool REINDEX>
void launch_score(int HT, int KS, dim3 grid, hipStream_t st, const uint8_t* qI, const float* w,
                  const uint8_t* ikeys, const int64_t* seq_start, const int32_t* row_seq,
                  const int32_t* row_len, const int32_t* pool, int32_t Hi, int32_t Di, int32_t P,
                  float* scores, int64_t lds, float* bm, int64_t ldb)
{
#define CSA2_SCORE(ht, ks)                                                                          \
    if (HT == ht && KS == ks) {                                                                     \
        hipLaunchKernelGGL((k_index_score<ht, ks, REINDEX>), grid, dim3(256), 0, st, qI, w, ikeys,   \
                           seq_start, row_seq, row_len, pool, Hi, Di, P, scores, lds, bm, ldb);     \
        return;                                                                                     \
    }
    CSA2_SCORE(1, 1) CSA2_SCORE(2, 1) CSA2_SCORE(3, 1) CSA2_SCORE(4, 1)
    CSA2_SCORE(1, 2) CSA2_SCORE(2, 2) CSA2_SCORE(3, 2) CSA2_SCORE(4, 2)
#undef CSA2_SCORE
}

int64_t full_ld(int32_t max_len) { return ((int64_t)max_len + kFullChunk - 1) / kFullChunk * kFullChunk; }

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

extern "C" size_t csa2_index_full_workspace_bytes(int32_t R, int32_t max_len, int32_t K, int32_t P,
                                                  int32_t block)
{
    (void)K; (void)P; (void)block;
    if (R < 0 || max_len < 0) return 0;
    const int64_t ld = full_ld(max_len);
    return csa2::align_up((size_t)R * ld * 4, 256) + csa2::align_up((size_t)R * (ld / 8) * 4, 256);
}

extern "C" csa2_status_t csa2_index_full(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                         const int64_t* seq_start, const int32_t* row_seq,
                                         const int32_t* row_len, int32_t R, int32_t Hi, int32_t Di,
                                         int32_t max_len, int32_t K, int32_t P, int32_t block,
                                         int32_t* topk_idx, int32_t* pool_blocks, void* workspace,
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
    CSA2_REQUIRE(qI && w && ikeys && seq_start && row_seq && row_len && topk_idx, CSA2_ERR_NULL,
                 "index_full: NULL pointer argument");
    const size_t need = csa2_index_full_workspace_bytes(R, max_len, K, P, block);
    CSA2_REQUIRE(workspace && workspace_bytes >= need && ((uintptr_t)workspace & 255) == 0,
                 CSA2_ERR_WORKSPACE, "index_full: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                 need, workspace_bytes);
    CSA2_REQUIRE(R <= 65535, CSA2_ERR_UNSUPPORTED, "index_full: R=%d > 65535", R);
    const int64_t ld = full_ld(max_len);
    float* scores = static_cast<float*>(workspace);
    float* bm = reinterpret_cast<float*>(static_cast<char*>(workspace) + csa2::align_up((size_t)R * ld * 4, 256));
    hipStream_t st = csa2::as_stream(stream);
    const int HT = (Hi + 15) / 16, KS = (Di + 127) / 128;
    if (max_len > 0) {
        dim3 grid((unsigned)(ld / kFullChunk), (unsigned)R);
        launch_score<false>(HT, KS, grid, st, qI, w, ikeys, seq_start, row_seq, row_len, nullptr, Hi, Di,
                            0, scores, ld, bm, ld / 8);
    }
    hipLaunchKernelGGL(k_select<true>, dim3((unsigned)R), dim3(kSelThreads), 0, st, scores, ld, bm, ld / 8,
                       row_len, nullptr, K, P, topk_idx, pool_blocks);
    return csa2::check_launch("index_full");
}

extern "C" size_t csa2_index_reindex_workspace_bytes(int32_t R, int32_t K, int32_t P, int32_t block)
{
    (void)K; (void)block;
    if (R < 0 || P < 0) return 0;
    const int64_t ld = ((int64_t)P * 8 + kReChunk - 1) / kReChunk * kReChunk;
    return csa2::align_up((size_t)R * ld * 4, 256);
}

extern "C" csa2_status_t csa2_index_reindex(const uint8_t* qI, const float* w, const uint8_t* ikeys,
                                            const int64_t* seq_start, const int32_t* row_seq,
                                            const int32_t* row_len, const int32_t* pool_blocks,
                                            int32_t R, int32_t Hi, int32_t Di, int32_t K, int32_t P,
                                            int32_t block, int32_t* topk_idx, void* workspace,
                                            size_t workspace_bytes, void* stream)
{
    csa2_status_t s = check_indexer_dims("index_reindex", R, Hi, Di, K, block);
    if (s != CSA2_OK) return s;
    CSA2_REQUIRE(P >= 1, CSA2_ERR_SHAPE, "index_reindex: P=%d < 1", P);
    CSA2_REQUIRE(P <= kMaxP, CSA2_ERR_UNSUPPORTED, "index_reindex: P=%d > %d", P, kMaxP);
    if (R == 0) return CSA2_OK;
    CSA2_REQUIRE(qI && w && ikeys && seq_start && row_seq && row_len && pool_blocks && topk_idx,
                 CSA2_ERR_NULL, "index_reindex: NULL pointer argument");
    const size_t need = csa2_index_reindex_workspace_bytes(R, K, P, block);
    CSA2_REQUIRE(workspace && workspace_bytes >= need && ((uintptr_t)workspace & 255) == 0,
                 CSA2_ERR_WORKSPACE, "index_reindex: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                 need, workspace_bytes);
    CSA2_REQUIRE(R <= 65535, CSA2_ERR_UNSUPPORTED, "index_reindex: R=%d > 65535", R);
    const int64_t ld = ((int64_t)P * 8 + kReChunk - 1) / kReChunk * kReChunk;
    float* scores = static_cast<float*>(workspace);
    hipStream_t st = csa2::as_stream(stream);
    const int HT = (Hi + 15) / 16, KS = (Di + 127) / 128;
    dim3 grid((unsigned)(ld / kReChunk), (unsigned)R);
    launch_score<true>(HT, KS, grid, st, qI, w, ikeys, seq_start, row_seq, row_len, pool_blocks, Hi, Di, P,
                       scores, ld, nullptr, 0);
    hipLaunchKernelGGL(k_select<false>, dim3((unsigned)R), dim3(kSelThreads), 0, st, scores, ld, nullptr, 0,
                       row_len, pool_blocks, K, P, topk_idx, nullptr);
    return csa2::check_launch("index_reindex");
}
