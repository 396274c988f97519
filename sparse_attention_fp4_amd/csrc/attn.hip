// Sparse MQA attention over gathered FP4 main-KV entries plus the FP8 SWA
// window (every CSA2 layer; the only step of a Reuse layer).
//
// CSA2 modes paragraph (Reuse mode attends sparsely with inherited Top-K
// indices) and FP4 KV cache paragraph (main KV in E2M1 + E4M3 per 16 channels,
// SWA KV in FP8) of section 一 of the teardown "DeepSeek V4.1 Flash 拆解"
// (austincafe.tech).  Readings: one latent per entry is both key and value and
// is shared by all query heads; the selected entries and the SWA rows form one
// key set under one softmax.
//
// Work decomposition (one workgroup = 4 waves = one query row x NH heads x a
// contiguous range of 64-key tiles):
//   * Each wave owns 16 keys of a tile.  A lane loads the raw bytes of one
//     key's quarter of the channels straight from the cache, dequantises them
//     to fp16 in registers (E2M1 -> fp16 by the hardware converter, times the
//     E4M3 scale; the product is exact in fp16) and feeds them as the A operand
//     of S^T = K Q^T on v_mfma_f32_16x16x32_f16, with the NH query heads held
//     in registers as the B operand.  Because the contraction order is the
//     same for both operands, each lane can hold a contiguous quarter of the
//     channels.
//   * The same fp16 values are stored once into an LDS tile [64 keys][D].
//   * Softmax statistics are exchanged through LDS (online softmax across
//     tiles, log2 domain); probabilities are written to LDS as fp16.
//   * PV: each wave produces D/4 output channels for all NH heads.  The B
//     operand (keys x channels) is read transposed with ds_read_b64_tr_b16,
//     whose 16-lane 4x4 block transpose delivers 4 keys of one channel per
//     lane per instruction.
//   * When a row's tiles are split across several workgroups, each writes its
//     unnormalised partial output and (max, sum) and k_attn_combine merges
//     them with the usual log-sum-exp weights.
#include "csa2_device.h"
#include "csa2_host.h"

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kTile = 64;
constexpr float kLazy = 8.0f;   // log2-domain slack before a running max is raised

template <int NB>
__device__ __forceinline__ void load_bytes(uint32_t* dst, const uint8_t* src)
{
    if constexpr (NB >= 16) {
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            uint4 v = reinterpret_cast<const uint4*>(src)[i];
            dst[4 * i] = v.x; dst[4 * i + 1] = v.y; dst[4 * i + 2] = v.z; dst[4 * i + 3] = v.w;
        }
    } else if constexpr (NB == 8) {
        uint2 v = *reinterpret_cast<const uint2*>(src);
        dst[0] = v.x; dst[1] = v.y;
    } else if constexpr (NB == 4) {
        dst[0] = *reinterpret_cast<const uint32_t*>(src);
    } else if constexpr (NB == 2) {
        dst[0] = *reinterpret_cast<const uint16_t*>(src);
    } else {
        dst[0] = *src;
    }
}


// Scale words / fp16 scale pairs held per lane (one scale per 16 channels).
template <int DW> constexpr int kScaleWords = (DW / 16 + 3) / 4;
template <int DW> constexpr int kScalePairs = (DW / 32) > 0 ? (DW / 32) : 1;

// Raw bytes of one lane's quarter-key for one tile: FP4 codes and E4M3 scales
// of a selected main entry, or FP8 bytes of an SWA row; zeros when the slot
// holds no valid key (which dequantise to zeros on either path).
template <int DW>
struct TileRaw {
    uint32_t raw[DW / 4];
    uint32_t sraw[kScaleWords<DW>];
    bool valid, is_main;

    // j: the Top-K entry of a main slot (ignored for SWA slots); slot: the
    // lane's key slot (main slots first, then SWA rows).
    __device__ __forceinline__ void load(int j, int slot, int K, int n, int64_t base, int nsw, int64_t swa0,
                                         const uint8_t* codes, const uint8_t* scales, const uint8_t* swa, int D,
                                         int grp)
    {
        int64_t row;
        if (slot < K) {
            valid = j >= 0 && j < n;
            is_main = true;
            row = base + (valid ? j : 0);
        } else {
            const int i = slot - K;
            valid = i < nsw;
            is_main = false;
            row = swa0 + (valid ? i : 0);
        }
#pragma unroll
        for (int i = 0; i < DW / 4; ++i) raw[i] = 0u;
#pragma unroll
        for (int i = 0; i < kScaleWords<DW>; ++i) sraw[i] = 0u;
        if (valid) {
            if (is_main) {
                load_bytes<DW / 2>(raw, codes + row * (D / 2) + grp * (DW / 2));
                load_bytes<DW / 16>(sraw, scales + row * (D / 16) + grp * (DW / 16));
            } else {
                load_bytes<DW>(raw, swa + row * D + grp * DW);
            }
        }
    }
};

// Dequantise k-step t (8 channels) of this lane's key to fp16.
//   MODE 0: FP4 codes (one 32-bit word per step) times the group's E4M3 scale;
//   MODE 1: FP8 E4M3 bytes (two words per step), unscaled;
//   MODE 2: either, chosen per lane by is_main.
template <int MODE>
__device__ __forceinline__ f16x8 dequant_step(const uint32_t* raw, const f16x2* sc, bool is_main, int t)
{
    f16x8 a, b;
    if (MODE != 1) {
        const uint32_t c = raw[t];
        const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
        const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
        const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
        const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
        const _Float16 s = sc[t >> 2][(t >> 1) & 1];
        a = (f16x8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]} * s;
    }
    if (MODE != 0) {
        const uint32_t c0 = raw[2 * t], c1 = raw[2 * t + 1];
        const f16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false);
        const f16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true);
        const f16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false);
        const f16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true);
        b = (f16x8){b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
    }
    if (MODE == 0) return a;
    if (MODE == 1) return b;
    return is_main ? a : b;
}

// S^T for this wave's 16 keys: dequantise each k-step, store it to the V tile
// and accumulate K Q^T (plain fp32 accumulation, or fresh partials folded by
// TwoSum when PRECISE).
template <int MODE, bool PRECISE, int HT, int KST>
__device__ __forceinline__ void s_tile(const uint32_t* raw, const f16x2* sc, bool is_main,
                                       const f16x8 (&qf)[HT][KST], _Float16* vrow, f32x4 (&sacc)[HT],
                                       f32x4 (&slo)[HT])
{
#pragma unroll
    for (int t = 0; t < KST; ++t) {
        const f16x8 kf = dequant_step<MODE>(raw, sc, is_main, t);
        *reinterpret_cast<f16x8*>(vrow + 8 * t) = kf;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            if (PRECISE) {
                const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ht][t],
                                                                          (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // TwoSum: hi + part == s + err exactly
                    const float a = sacc[ht][i], b = part[i];
                    const float s2 = a + b;
                    const float bb = s2 - a;
                    const float err = (a - (s2 - bb)) + (b - bb);
                    sacc[ht][i] = s2;
                    slo[ht][i] += err;
                }
            } else {
                sacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ht][t], sacc[ht], 0, 0, 0);
            }
        }
    }
}

// O[heads x this wave's channels] += P V for one 64-key tile.  The B operand
// is read with ds_read_b64_tr_b16: within each 16-lane group, lane l receives
// element l%4 of the 8-byte rows addressed by lanes 4i + l/4, so addressing
// row (key 4g + l/4, channels c0 + 4(l%4)) hands lane l the 4 keys 4g + 0..3
// of channel c0 + l, matching the probability fragment's key order.
template <bool SPLIT, int HT, int NDT, int VST, int PST>
__device__ __forceinline__ void pv_tile(const _Float16* Pt, const _Float16* Plo, const _Float16* V, int col,
                                        int grp, int c0, f32x4 (&o)[HT][NDT])
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        f16x8 pa[HT], pl[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int off = (ht * 16 + col) * PST + 32 * kk + 4 * grp;
            const f16x4 a0 = *reinterpret_cast<const f16x4*>(&Pt[off]);
            const f16x4 a1 = *reinterpret_cast<const f16x4*>(&Pt[off + 16]);
            pa[ht] = (f16x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            if (SPLIT) {
                const f16x4 b0 = *reinterpret_cast<const f16x4*>(&Plo[off]);
                const f16x4 b1 = *reinterpret_cast<const f16x4*>(&Plo[off + 16]);
                pl[ht] = (f16x8){b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            }
        }
        const _Float16* v1 = V + (32 * kk + 4 * grp + (col >> 2)) * VST + c0 + 4 * (col & 3);
        const _Float16* v2 = v1 + 16 * VST;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const lds_f16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                (lds_f16x4 __attribute__((address_space(3)))*)(v1 + 16 * dt));
            const lds_f16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                (lds_f16x4 __attribute__((address_space(3)))*)(v2 + 16 * dt));
            const f16x8 vb8 = {(_Float16)b1[0], (_Float16)b1[1], (_Float16)b1[2], (_Float16)b1[3],
                               (_Float16)b2[0], (_Float16)b2[1], (_Float16)b2[2], (_Float16)b2[3]};
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[ht], vb8, o[ht][dt], 0, 0, 0);
                if (SPLIT) o[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[ht], vb8, o[ht][dt], 0, 0, 0);
            }
        }
    }
}

template <int HT, int D>
__global__ __launch_bounds__(256, 1) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int64_t* __restrict__ seq_start, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ topk, int32_t K,
    const uint8_t* __restrict__ swa, const int64_t* __restrict__ swa_row_start,
    const int32_t* __restrict__ swa_len, int32_t H, int32_t W, float scale_log2e, int32_t HG, int32_t S,
    int32_t ntiles, float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml)
{
    constexpr int DW = D / 4;        // channels per lane (S^T) and per wave (PV)
    constexpr int KST = D / 32;      // k-steps of 8 channels per lane
    constexpr int NDT = DW / 16;     // 16-channel output tiles per wave
    constexpr int VST = D + 16;      // V tile row stride in halves (bank spread)
    constexpr int PST = kTile + 8;   // P row stride in halves
    constexpr int NH = HT * 16;

    __shared__ __attribute__((aligned(16))) _Float16 Vt[2][kTile * VST];
    __shared__ __attribute__((aligned(16))) _Float16 Pt[NH * PST];
    __shared__ __attribute__((aligned(16))) _Float16 Plo[NH * PST];
    __shared__ float wmax[4][NH];
    __shared__ uint32_t wvmax[4];   // per wave: its keys may exceed |v| = 8
    __shared__ float wl[4][NH];

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int r = blockIdx.x / HG, hg = blockIdx.x % HG, s = blockIdx.y;
    const int h0 = hg * NH;
    const int n = row_len[r];
    const int64_t base = seq_start[row_seq[r]];
    int nsw = W > 0 ? swa_len[r] : 0;
    nsw = nsw < 0 ? 0 : (nsw > W ? W : nsw);
    const int64_t swa0 = W > 0 ? swa_row_start[r] : 0;
    const int t_begin = (int)((int64_t)ntiles * s / S), t_end = (int)((int64_t)ntiles * (s + 1) / S);

    // Query heads as fp16 B-operand fragments: lane (head col, grp) holds
    // channels grp*DW + 8t .. +8 of its head for k-step t.
    f16x8 qf[HT][KST];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + ht * 16 + col;
        uint32_t raw[DW / 2];
        if (h < H) load_bytes<DW * 2>(raw, reinterpret_cast<const uint8_t*>(q + ((int64_t)r * H + h) * D + grp * DW));
        else {
#pragma unroll
            for (int i = 0; i < DW / 2; ++i) raw[i] = 0;
        }
#pragma unroll
        for (int t = 0; t < KST; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = raw[4 * t + e];
                qf[ht][t][2 * e] = (_Float16)__uint_as_float(w << 16);
                qf[ht][t][2 * e + 1] = (_Float16)__uint_as_float(w & 0xFFFF0000u);
            }
        }
    }

    // Online softmax state (log2 domain).  The reference max of a head is
    // raised only when a tile's max exceeds it by more than kLazy, so the
    // accumulated output is rarely rescaled; probabilities stay <= 2^kLazy.
    float m_p[HT], l_p[HT], m_o[HT][4];
    f32x4 o[HT][NDT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        m_p[ht] = -INFINITY;
        l_p[ht] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) m_o[ht][i] = -INFINITY;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[ht][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }

    // Software pipeline over tiles: while tile t is processed, the raw bytes
    // of tile t+1 and the index of tile t+2 are already in flight, so the
    // dependent index -> row loads never stall the matrix work.
    auto slot_index = [&](int tile) -> int {     // Top-K entry of this lane's slot (or -2)
        const int slot = tile * kTile + wave * 16 + col;
        return (tile < t_end && slot < K) ? topk[(int64_t)r * K + slot] : -2;
    };
    TileRaw<DW> cur, nxt;
    int idx_next = slot_index(t_begin + 1);
    cur.load(slot_index(t_begin), t_begin * kTile + wave * 16 + col, K, n, base, nsw, swa0, codes, scales, swa, D,
             grp);

    for (int tile = t_begin; tile < t_end; ++tile) {
        const int buf = (tile - t_begin) & 1;
        _Float16* V = Vt[buf];
        if (tile + 1 < t_end) {
            const int idx_after = slot_index(tile + 2);
            nxt.load(idx_next, (tile + 1) * kTile + wave * 16 + col, K, n, base, nsw, swa0, codes, scales, swa, D,
                     grp);
            idx_next = idx_after;
        }
        const bool valid = cur.valid, is_main = cur.is_main;
        const uint32_t* raw = cur.raw;
        const uint32_t* sraw = cur.sraw;

        // Large values (|v| > 8) make the output sensitive to logit rounding:
        // a logit error e moves the output by about e * |v - out|.  A wave whose
        // keys may hold such values accumulates S^T with one fresh MFMA result
        // per k-step folded into an fp32 (hi, lo) pair by an exact TwoSum, and
        // the tile uses two-part probabilities in PV.  The test is on the
        // stored bytes: an FP4 group holds |v| <= 6 * scale, so a scale byte of
        // 0x3B (1.375) or more; an FP8 SWA byte of magnitude 0x50 (8.0) or more.
        // Adding 0x45 (resp. 0x30) to a 7-bit magnitude sets bit 7 exactly
        // when the magnitude reaches 0x3B (resp. 0x50), with no carry between
        // bytes (missing bytes are zero).
        uint32_t bigbits = 0u;
        if (is_main) {
#pragma unroll
            for (int i = 0; i < kScaleWords<DW>; ++i) bigbits |= ((sraw[i] & 0x7F7F7F7Fu) + 0x45454545u) & 0x80808080u;
            // bytes past the lane's DW/16 scales are zero and read as 0x45 < 0x80
        } else {
#pragma unroll
            for (int i = 0; i < DW / 4; ++i) bigbits |= ((raw[i] & 0x7F7F7F7Fu) + 0x30303030u) & 0x80808080u;
        }
        const bool precise = __ballot(bigbits != 0u) != 0ull;
        const uint64_t bmain = __ballot(valid && is_main), bswa = __ballot(valid && !is_main);

        f16x2 sc[kScalePairs<DW>];
#pragma unroll
        for (int i = 0; i < kScalePairs<DW>; i += 2) {
            sc[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw[i >> 1], 1.0f, false);
            if (i + 1 < kScalePairs<DW>) sc[i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw[i >> 1], 1.0f, true);
        }

        f32x4 sacc[HT], slo[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            sacc[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            slo[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
        _Float16* vrow = V + (wave * 16 + col) * VST + grp * DW;
        if (bswa == 0ull) {
            if (precise) s_tile<0, true, HT, KST>(raw, sc, is_main, qf, vrow, sacc, slo);
            else s_tile<0, false, HT, KST>(raw, sc, is_main, qf, vrow, sacc, slo);
        } else if (bmain == 0ull) {
            if (precise) s_tile<1, true, HT, KST>(raw, sc, is_main, qf, vrow, sacc, slo);
            else s_tile<1, false, HT, KST>(raw, sc, is_main, qf, vrow, sacc, slo);
        } else {
            if (precise) s_tile<2, true, HT, KST>(raw, sc, is_main, qf, vrow, sacc, slo);
            else s_tile<2, false, HT, KST>(raw, sc, is_main, qf, vrow, sacc, slo);
        }
        if (lane == 0) wvmax[wave] = precise ? 1u : 0u;

        // S^T lane layout: head (h0 + 16 ht + col), keys wave*16 + 4 grp + i
        const uint64_t vb = __ballot(valid);
        float x[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kv = (vb >> (4 * grp + i)) & 1ull;
                x[ht][i] = kv ? (sacc[ht][i] + slo[ht][i]) * scale_log2e : -INFINITY;
                mx = fmaxf(mx, x[ht][i]);
            }
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            if (grp == 0) wmax[wave][ht * 16 + col] = mx;
        }
        __syncthreads();

        // Probabilities enter PV as fp16, whose rounding (relative 2^-12) moves
        // the output by up to 2^-12 * |v - out|.  For tiles whose keys may hold
        // |v| > 8 the probability is split into fp16 hi + lo parts and PV runs
        // twice, which brings the rounding to ~2^-23.
        const bool split = (wvmax[0] | wvmax[1] | wvmax[2] | wvmax[3]) != 0u;
        float alpha[HT][4];
        bool rescale = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int hh = ht * 16 + col;
            const float mt = fmaxf(fmaxf(wmax[0][hh], wmax[1][hh]), fmaxf(wmax[2][hh], wmax[3][hh]));
            const float mn = (mt > m_p[ht] + kLazy) ? mt : m_p[ht];
            const bool live = mn != -INFINITY;
            const float ap = live ? exp2f(m_p[ht] - mn) : 1.0f;
            float ps = 0.0f;
            f16x4 p4, q4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the exponent's argument is formed with one rounding at its own
                // (small) magnitude; the reference itself only has to be consistent
                const float d = fmaf(sacc[ht][i], scale_log2e, -mn) + slo[ht][i] * scale_log2e;
                const float pf = (live && x[ht][i] != -INFINITY) ? exp2f(d) : 0.0f;
                const _Float16 p = (_Float16)pf;
                p4[i] = p;
                q4[i] = (_Float16)(pf - (float)p);
                ps += split ? pf : (float)p;   // normalise by what PV actually weights
            }
            l_p[ht] = l_p[ht] * ap + ps;
            m_p[ht] = mn;
            *reinterpret_cast<f16x4*>(&Pt[hh * PST + wave * 16 + 4 * grp]) = p4;
            if (split) *reinterpret_cast<f16x4*>(&Plo[hh * PST + wave * 16 + 4 * grp]) = q4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ho = ht * 16 + 4 * grp + i;
                const float mto = fmaxf(fmaxf(wmax[0][ho], wmax[1][ho]), fmaxf(wmax[2][ho], wmax[3][ho]));
                const float mno = (mto > m_o[ht][i] + kLazy) ? mto : m_o[ht][i];
                alpha[ht][i] = (m_o[ht][i] != -INFINITY) ? exp2f(m_o[ht][i] - mno) : 1.0f;
                rescale |= mno != m_o[ht][i] && m_o[ht][i] != -INFINITY;
                m_o[ht][i] = mno;
            }
        }
        __syncthreads();

        if (__ballot(rescale) != 0ull) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[ht][dt][i] *= alpha[ht][i];
        }

        if (split) pv_tile<true, HT, NDT, VST, PST>(Pt, Plo, V, col, grp, wave * DW, o);
        else pv_tile<false, HT, NDT, VST, PST>(Pt, Plo, V, col, grp, wave * DW, o);
        cur = nxt;
    }

    // Row sums over the four waves' keys.
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float lt = l_p[ht];
        lt += shfl_xor_f(lt, 16);
        lt += shfl_xor_f(lt, 32);
        if (grp == 0) wl[wave][ht * 16 + col] = lt;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = ht * 16 + 4 * grp + i;
            const int h = h0 + hh;
            if (h >= H) continue;
            const float L = wl[0][hh] + wl[1][hh] + wl[2][hh] + wl[3][hh];
            const float M = m_o[ht][i];
            if (S == 1) {
                const float inv = L > 0.0f ? 1.0f / L : 0.0f;
                float* op = out + ((int64_t)r * H + h) * D + wave * DW + col;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) op[16 * dt] = o[ht][dt][i] * inv;
                if (lse && wave == 0 && col == 0)
                    lse[(int64_t)r * H + h] = L > 0.0f ? M * kLn2 + logf(L) : -INFINITY;
            } else {
                float* op = part_o + (((int64_t)r * S + s) * H + h) * D + wave * DW + col;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) op[16 * dt] = o[ht][dt][i];
                if (wave == 0 && col == 0) {
                    float* ml = part_ml + (((int64_t)r * S + s) * H + h) * 2;
                    ml[0] = M;
                    ml[1] = L;
                }
            }
        }
    }
}

// Merge of split partials: o = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// One workgroup per (row, head); each thread owns four consecutive channels.
constexpr int kMaxSplits = 64;
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int32_t H,
                                                      int32_t D, int32_t S, float* __restrict__ out,
                                                      float* __restrict__ lse)
{
    const int rh = blockIdx.x;          // r * H + h
    const int r = rh / H, h = rh % H;
    __shared__ float wgt[kMaxSplits];
    __shared__ float Ls;
    if (threadIdx.x == 0) {
        float M = -INFINITY;
        for (int s = 0; s < S; ++s) {
            const float* ml = part_ml + (((int64_t)r * S + s) * H + h) * 2;
            if (ml[1] > 0.0f) M = fmaxf(M, ml[0]);
        }
        float L = 0.0f;
        for (int s = 0; s < S; ++s) {
            const float* ml = part_ml + (((int64_t)r * S + s) * H + h) * 2;
            const float w = ml[1] > 0.0f ? exp2f(ml[0] - M) : 0.0f;
            wgt[s] = w;
            L += ml[1] * w;
        }
        Ls = L;
        if (lse) lse[rh] = L > 0.0f ? M * kLn2 + logf(L) : -INFINITY;
    }
    __syncthreads();
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    for (int d = 4 * threadIdx.x; d < D; d += 4 * blockDim.x) {
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int s = 0; s < S; ++s) {
            const float w = wgt[s];
            const float4 v = *reinterpret_cast<const float4*>(part_o + (((int64_t)r * S + s) * H + h) * D + d);
            acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
        }
        *reinterpret_cast<float4*>(out + (int64_t)rh * D + d) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}

struct AttnPlan {
    int HT, HG, S, ntiles;
};

AttnPlan plan_attn(int32_t R, int32_t H, int32_t K, int32_t W)
{
    AttnPlan p;
    p.ntiles = (K + W + kTile - 1) / kTile;
    if (p.ntiles < 1) p.ntiles = 1;
    const int hg2 = (H + 31) / 32;
    p.HT = (H > 16 && (int64_t)R * hg2 * p.ntiles >= 256) ? 2 : 1;
    p.HG = (H + 16 * p.HT - 1) / (16 * p.HT);
    const int64_t base = (int64_t)R * p.HG;
    int64_t S = base >= 256 ? 1 : (256 + base - 1) / base;
    if (S > p.ntiles) S = p.ntiles;
    if (S > kMaxSplits) S = kMaxSplits;
    p.S = (int)S;
    return p;
}

template <int HT, int D>
void launch_attn(dim3 grid, hipStream_t st, const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                 const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len, const int32_t* topk,
                 int32_t K, const uint8_t* swa, const int64_t* swa_row_start, const int32_t* swa_len, int32_t H,
                 int32_t W, float sl2e, int HG, int S, int ntiles, float* out, float* lse, float* po, float* pml)
{
    hipLaunchKernelGGL((k_sparse_attn<HT, D>), grid, dim3(256), 0, st, q, codes, scales, seq_start, row_seq,
                       row_len, topk, K, swa, swa_row_start, swa_len, H, W, sl2e, HG, S, ntiles, out, lse, po,
                       pml);
}

}  // namespace

extern "C" size_t csa2_sparse_attn_workspace_bytes(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W)
{
    if (R <= 0 || H <= 0 || D <= 0 || K < 0 || W < 0) return 0;
    const AttnPlan p = plan_attn(R, H, K, W);
    if (p.S <= 1) return 0;
    return csa2::align_up((size_t)R * p.S * H * D * 4, 256) + csa2::align_up((size_t)R * p.S * H * 2 * 4, 256);
}

extern "C" csa2_status_t csa2_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                          const int64_t* seq_start, const int32_t* row_seq,
                                          const int32_t* row_len, const int32_t* topk_idx, int32_t K,
                                          const uint8_t* swa, const int64_t* swa_row_start,
                                          const int32_t* swa_len, int32_t R, int32_t H, int32_t D, int32_t W,
                                          float softmax_scale, float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream)
{
    CSA2_REQUIRE(R >= 0, CSA2_ERR_SHAPE, "sparse_attn: R=%d < 0", R);
    CSA2_REQUIRE(H >= 1, CSA2_ERR_SHAPE, "sparse_attn: H=%d < 1", H);
    CSA2_REQUIRE(D >= 16 && D % 16 == 0, CSA2_ERR_SHAPE, "sparse_attn: D=%d must be a positive multiple of 16", D);
    CSA2_REQUIRE(D == 64 || D == 128 || D == 256 || D == 512, CSA2_ERR_UNSUPPORTED,
                 "sparse_attn: D=%d (supported: 64, 128, 256, 512)", D);
    CSA2_REQUIRE(K >= 0 && W >= 0, CSA2_ERR_SHAPE, "sparse_attn: K=%d, W=%d must be >= 0", K, W);
    CSA2_REQUIRE(K <= 4096 && W <= 4096, CSA2_ERR_UNSUPPORTED, "sparse_attn: K=%d or W=%d > 4096", K, W);
    if (R == 0) return CSA2_OK;
    CSA2_REQUIRE(q && codes && scales && seq_start && row_seq && row_len && out, CSA2_ERR_NULL,
                 "sparse_attn: NULL pointer argument");
    CSA2_REQUIRE(K == 0 || topk_idx, CSA2_ERR_NULL, "sparse_attn: topk_idx is NULL with K > 0");
    CSA2_REQUIRE(W == 0 || (swa && swa_row_start && swa_len), CSA2_ERR_NULL,
                 "sparse_attn: SWA pointers are NULL with W > 0");
    const AttnPlan p = plan_attn(R, H, K, W);
    CSA2_REQUIRE((int64_t)R * p.HG <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED, "sparse_attn: grid too large");
    const size_t need = csa2_sparse_attn_workspace_bytes(R, H, D, K, W);
    CSA2_REQUIRE(need == 0 || (workspace && workspace_bytes >= need && ((uintptr_t)workspace & 255) == 0),
                 CSA2_ERR_WORKSPACE, "sparse_attn: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                 workspace_bytes);
    float* po = nullptr;
    float* pml = nullptr;
    if (p.S > 1) {
        po = static_cast<float*>(workspace);
        pml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       csa2::align_up((size_t)R * p.S * H * D * 4, 256));
    }
    // With W == 0 or K == 0 the kernels never dereference the unused pointers.
    hipStream_t st = csa2::as_stream(stream);
    const float sl2e = softmax_scale * 1.44269504088896340736f;
    dim3 grid((unsigned)(R * p.HG), (unsigned)p.S);
#define CSA2_ATTN(ht, d)                                                                               \
    if (p.HT == ht && D == d) {                                                                         \
        launch_attn<ht, d>(grid, st, q, codes, scales, seq_start, row_seq, row_len, topk_idx, K, swa,   \
                           swa_row_start, swa_len, H, W, sl2e, p.HG, p.S, p.ntiles, out, lse, po, pml); \
    }
    CSA2_ATTN(1, 64) CSA2_ATTN(1, 128) CSA2_ATTN(1, 256) CSA2_ATTN(1, 512)
    CSA2_ATTN(2, 64) CSA2_ATTN(2, 128) CSA2_ATTN(2, 256) CSA2_ATTN(2, 512)
#undef CSA2_ATTN
    if (p.S > 1)
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(R * H)), dim3(128), 0, st, po, pml, H, D, p.S, out, lse);
    return csa2::check_launch("sparse_attn");
}
