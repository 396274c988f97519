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
// Work decomposition.  One workgroup (4 waves) = one query row x NH = 16*HT
// heads x a contiguous range of 64-key tiles.  Wave w owns the channel slice
// [w*D/4, (w+1)*D/4) in both products, so every key is dequantised once per
// workgroup and the query registers hold only a quarter of the channels:
//   * S^T = K Q^T: each lane dequantises D/16 channels of 4 keys (one per
//     16-key fragment) straight from the cache to fp16 in registers (E2M1 ->
//     fp16 by the hardware converter, times the E4M3 scale; the product is
//     exact in fp16) and feeds them as the A operand of
//     v_mfma_f32_16x16x32_f16 against the NH query heads (B operand).  The
//     contraction order only has to agree between the two operands; it is
//     chosen so that in every MFMA lanes 0-31 carry the two halves of one
//     16-channel scale group and lanes 32-63 those of another (see below).
//     The same fp16 values go once into an LDS tile [64 keys][D].
//   * The four channel-slice partials of S^T are summed through LDS; wave w
//     keeps the 16 keys of fragment w.
//   * Online softmax across tiles (log2 domain, lazily raised reference max);
//     probabilities go to LDS as fp16.
//   * PV: wave w produces its D/4 output channels for all NH heads; the B
//     operand (keys x channels) is read with ds_read_b64_tr_b16.
//   * Rows whose tiles are split across workgroups write unnormalised partial
//     outputs plus (max, sums); k_attn_combine merges them.
//
// Exact scores for keys with large values.  The matrix cores sum products
// with errors of a few units in the last place of the largest addend, and
// with |v| in the hundreds a near tie between two keys turns such a score
// error into an output error far above the tolerance.  Where a wave's keys
// may hold |v| > 8 it computes S exactly instead: each query head is split as
// q = a + b, a being q rounded to a multiple of 2^(E-11) with 2^E > max|q| of
// the head (11 bits, exact in fp16), b the small remainder.  Within one scale
// group every a*k product is then an integer multiple of one quantum and the
// 16 products sum to less than 2^24 quanta, so an MFMA restricted to one group
// (the other lane half masked to zero) returns the group sum exactly; the
// group sums are accumulated in fp64, and K b^T (small, nonzero only for
// channels with |q| < max|q|/16) is added from an ordinary MFMA chain.
#include "csa2_device.h"
#include "csa2_host.h"

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kTile = 64;           // keys per tile: 4 fragments of 16
constexpr float kLazy = 8.0f;       // log2-domain slack before a running max is raised
constexpr int kMaxPlanSplits = 8;     // key splits per row, at most

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

// Channel layout of a lane (col, grp) in wave w, with p = grp / 2 and
// h = grp % 2: k-step t (t < KT = D/128) covers the 8 channels
//   w*D/4 + 16*(p*KT + t) + 8*h .. + 8,
// i.e. half h of scale group p*KT + t of the wave's slice.  In each MFMA the
// lanes with p = 0 thus hold one whole scale group and those with p = 1 another.
template <int D>
__device__ __forceinline__ int lane_ch0(int wave, int grp)
{
    constexpr int KT = D / 128;
    return wave * (D / 4) + 16 * ((grp >> 1) * KT) + 8 * (grp & 1);
}

// Local unit holding piece t after TileRaw::unpair(): {0, 2, 1, 3} for four
// pieces, identity otherwise.
template <int D>
__device__ __forceinline__ constexpr int kperm(int t)
{
    return D / 128 == 4 ? ((t & 1) << 1 | (t >> 1)) : t;
}

// Raw bytes of one tile held by one lane: for each of the 4 key fragments, the
// lane's key (16 f + col) restricted to its channels: FP4 codes (one word per
// k-step) and its KT E4M3 scale bytes of a selected main entry, or FP8 bytes
// (two words per k-step) of an SWA row.  A slot without a valid key gets a
// zero scale (main; its code bytes are left as they are, any E2M1 code times
// zero is zero) or zero bytes (SWA), so it dequantises to zeros.
template <int D>
struct TileRaw {
    static constexpr int KT = D / 128;
    uint32_t raw[4][2 * KT];
    uint32_t sc[4];
    bool valid[4], is_main[4];

    // idx: the Top-K entries of the lane's 4 slots (fetched a tile earlier;
    // only read for Top-K slots).  crow / srow / wrow: code, scale and SWA
    // pointers of the row's first entry, already offset to the lane's
    // channels.  One straight-line path for every kind of slot: each load is
    // predicated and writes its registers in place, so the loads stay in
    // flight until the bytes are used a tile later.  FP4 piece t lands in word
    // 2t, FP8 piece t in words 2t and 2t+1.
    __device__ __forceinline__ void load(int tile, const int (&idx)[4], int col, int h, int K, int n, int nsw,
                                         const uint8_t* crow, const uint8_t* srow, const uint8_t* wrow)
    {
        // SWA slots without a row must read as zero bytes (a main slot without
        // an entry gets a zero scale instead); only tiles that reach past the
        // Top-K slots can have them.
        const bool any_swa = (tile + 1) * kTile > K;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int slot = tile * kTile + 16 * f + col;
            const bool m = slot < K;
            const int j = idx[f], i = slot - K;
            const bool vm = m && j >= 0 && j < n;
            const bool vs = !m && i < nsw;
            valid[f] = vm || vs;
            is_main[f] = m;
            sc[f] = 0u;
            // The lane pair (p, 0), (p, 1) of a key needs one contiguous block
            // (codes: 4*KT bytes, SWA: 16*KT bytes); each lane loads its half,
            // into consecutive words, and unpair() exchanges the halves a tile
            // later.  The first access serves both kinds (its address is chosen
            // per lane), so no two loads in flight write the same registers.
            const uint8_t* ca = crow + (size_t)j * (D / 2) + (KT == 4 ? 12 : (KT == 2 ? 4 : 0)) * h;
            const uint8_t* sa = wrow + (size_t)i * D + (KT == 4 ? 24 : (KT == 2 ? 8 : 0)) * h;
            const uint8_t* a1 = vm ? ca : sa;
            if (any_swa) {
#pragma unroll
                for (int w = 0; w < 2 * KT; ++w) raw[f][w] = 0u;
            }
            if (vm || vs) {
                if constexpr (KT == 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(a1);
                    raw[f][0] = v.x; raw[f][1] = v.y; raw[f][2] = v.z; raw[f][3] = v.w;
                } else if constexpr (KT == 2) {
                    const uint2 v = *reinterpret_cast<const uint2*>(a1);
                    raw[f][0] = v.x; raw[f][1] = v.y;
                } else {
                    raw[f][0] = *reinterpret_cast<const uint32_t*>(a1);
                }
            }
            if (vs) {                 // the second half of an SWA lane's bytes
                if constexpr (KT == 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(sa + 16);
                    raw[f][4] = v.x; raw[f][5] = v.y; raw[f][6] = v.z; raw[f][7] = v.w;
                } else if constexpr (KT == 2) {
                    const uint2 v = *reinterpret_cast<const uint2*>(sa + 8);
                    raw[f][2] = v.x; raw[f][3] = v.y;
                } else {
                    raw[f][1] = *reinterpret_cast<const uint32_t*>(sa + 4);
                }
            }
            if (vm) load_bytes<KT>(&sc[f], srow + (size_t)j * (D / 16));
        }
    }

    // Unit u of a pair's block (a code word, or 8 FP8 bytes) is piece u/2 of
    // half u%2; after load() lane h holds units 2h, 2h+1 (KT = 2) or 4h .. 4h+3
    // (KT = 4) in consecutive words.  v_permlane16_swap(x, y) exchanges row 1
    // of x with row 0 of y (rows are the 16-lane groups: rows 0/1 are the
    // halves h = 0/1 of p = 0, rows 2/3 those of p = 1).  Swapping local units
    // (0, 1) and, for KT = 4, (2, 3) leaves the lane's own half of piece t in
    // local unit kPerm[t]: code word kPerm[t], or FP8 words 2 kPerm[t] and
    // 2 kPerm[t] + 1.  KIND as for the tile (main, SWA, or both per lane).
    template <int KIND>
    __device__ __forceinline__ void unpair()
    {
        if constexpr (KT >= 2) {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                uint32_t c[KT], w[2 * KT];
#pragma unroll
                for (int u = 0; u < KT / 2; ++u) {
                    if (KIND != 1) {      // code words 2u <-> 2u+1
                        const auto r = __builtin_amdgcn_permlane16_swap(raw[f][2 * u], raw[f][2 * u + 1], false, false);
                        c[2 * u] = r[0];
                        c[2 * u + 1] = r[1];
                    }
                    if (KIND != 0) {      // FP8 units 2u <-> 2u+1, both words
                        const auto ra = __builtin_amdgcn_permlane16_swap(raw[f][4 * u], raw[f][4 * u + 2], false, false);
                        const auto rb = __builtin_amdgcn_permlane16_swap(raw[f][4 * u + 1], raw[f][4 * u + 3], false, false);
                        w[4 * u] = ra[0];
                        w[4 * u + 2] = ra[1];
                        w[4 * u + 1] = rb[0];
                        w[4 * u + 3] = rb[1];
                    }
                }
                if (KIND == 0) {
#pragma unroll
                    for (int k = 0; k < KT; ++k) raw[f][k] = c[k];
                } else if (KIND == 1) {
#pragma unroll
                    for (int k = 0; k < 2 * KT; ++k) raw[f][k] = w[k];
                } else {
                    const bool mm = is_main[f];
#pragma unroll
                    for (int k = 0; k < 2 * KT; ++k) raw[f][k] = mm ? (k < KT ? c[k] : 0u) : w[k];
                }
            }
        }
    }

    // Whether this lane's keys may hold |v| > 8: an FP4 group holds
    // |v| <= 6 * scale, so a scale byte of 0x3B (1.375) or more; an FP8 byte
    // of magnitude 0x50 (8.0) or more.  Adding 0x45 (resp. 0x30) to a 7-bit
    // magnitude sets bit 7 exactly at that threshold, with no carry between
    // bytes; the unused high bytes of sc are zero and stay below bit 7.
    __device__ __forceinline__ bool big() const
    {
        uint32_t bits = 0u;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            if (!valid[f]) continue;
            if (is_main[f]) {
                bits |= ((sc[f] & 0x7F7F7F7Fu) + 0x45454545u) & 0x80808080u;
            } else {
#pragma unroll
                for (int i = 0; i < 2 * KT; ++i) bits |= ((raw[f][i] & 0x7F7F7F7Fu) + 0x30303030u) & 0x80808080u;
            }
        }
        return bits != 0u;
    }
};

// Dequantise k-step t (8 channels) of fragment f to fp16.
//   MODE 0: FP4 codes (word kperm(t)) times the group's E4M3 scale
//           (scale byte t of the lane's KT scale bytes);
//   MODE 1: FP8 E4M3 bytes (words 2 kperm(t), +1), unscaled;
//   MODE 2: either, chosen per lane.
template <int MODE, int D>
__device__ __forceinline__ f16x8 dequant_step(const TileRaw<D>& tr, int f, int t)
{
    f16x8 a, b;
    if (MODE != 1) {
        const uint32_t c = tr.raw[f][kperm<D>(t)];
        const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
        const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
        const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
        const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
        const f16x2 sp = (t & 2) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(tr.sc[f], 1.0f, true)
                                 : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(tr.sc[f], 1.0f, false);
        const _Float16 s = sp[t & 1];
        a = (f16x8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]} * s;
    }
    if (MODE != 0) {
        const uint32_t c0 = tr.raw[f][2 * kperm<D>(t)], c1 = tr.raw[f][2 * kperm<D>(t) + 1];
        const f16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false);
        const f16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true);
        const f16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false);
        const f16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true);
        b = (f16x8){b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
    }
    if (MODE == 0) return a;
    if (MODE == 1) return b;
    return tr.is_main[f] ? a : b;
}

// TwoSum, elementwise: (hi, lo) += b, where hi + b == new hi + its rounding
// error exactly and the error is added to lo.
__device__ __forceinline__ void two_sum_into(f32x4& hi, f32x4& lo, f32x4 b)
{
    const f32x4 s = hi + b;
    const f32x4 bb = s - hi;
    lo += (hi - (s - bb)) + (b - bb);
    hi = s;
}

// One fragment of S^T over this lane's channels, fp32 MFMA chain; the
// dequantised keys also go to the V tile (piece t at channel offset 16 t).
template <int MODE, int HT, int KT, int D>
__device__ __forceinline__ void s_frag(const TileRaw<D>& tr, int f, const f16x8 (&qf)[HT][KT], _Float16* vrow,
                                       f32x4 (&acc)[HT])
{
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const f16x8 kf = dequant_step<MODE, D>(tr, f, t);
        *reinterpret_cast<f16x8*>(vrow + 16 * t) = kf;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ht][t], acc[ht], 0, 0, 0);
    }
}

// The same fragment with S computed exactly as (hi, lo) = K a^T + K b^T
// (split of q described at the top of the file).  qa: this lane's a-part
// pieces in LDS, [HT * KT][256 lanes]; upper: lane >= 32.
template <int MODE, int HT, int KT, int D>
__device__ __forceinline__ void s_frag_exact(const TileRaw<D>& tr, int f, const f16x8 (&qf)[HT][KT],
                                             const f16x8* qa, bool upper, _Float16* vrow, f32x4 (&acc)[HT],
                                             f32x4 (&lo)[HT])
{
    double ex[HT][4];
    f32x4 sb[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        sb[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) ex[ht][i] = 0.0;
    }
    const f16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const f16x8 kf = dequant_step<MODE, D>(tr, f, t);
        *reinterpret_cast<f16x8*>(vrow + 16 * t) = kf;
        const f16x8 k_lo = upper ? zero : kf;     // scale group p*KT + t with p = 0
        const f16x8 k_hi = upper ? kf : zero;     // and with p = 1
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const f16x8 a = qa[(ht * KT + t) * 256];
            const f16x8 b = qf[ht][t] - a;        // exact: the low bits of q
            sb[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, b, sb[ht], 0, 0, 0);
            const f32x4 g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_lo, a, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const f32x4 g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_hi, a, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) ex[ht][i] += (double)g0[i] + (double)g1[i];
        }
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double v = ex[ht][i] + (double)sb[ht][i];
            const float h = (float)v;
            acc[ht][i] = h;
            lo[ht][i] = (float)(v - (double)h);
        }
}

// S^T partials of all 4 fragments over this lane's channels.  vbase: V tile
// at (key col of fragment 0, this lane's first channel).  KIND as in
// TileRaw::load; the exact path uses one general dequantisation for all kinds.
template <bool EXACT, int KIND, int HT, int KT, int D, int VST>
__device__ __forceinline__ void s_tile(const TileRaw<D>& tr, const f16x8 (&qf)[HT][KT], const f16x8* qa,
                                       bool upper, _Float16* vbase, f32x4 (&acc)[4][HT], f32x4 (&lo)[4][HT])
{
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        _Float16* vrow = vbase + 16 * f * VST;
        if (EXACT) s_frag_exact<2, HT, KT, D>(tr, f, qf, qa, upper, vrow, acc[f], lo[f]);
        else s_frag<KIND, HT, KT, D>(tr, f, qf, vrow, acc[f]);
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

// Workgroups are handed to the 8 XCDs of the chip round-robin by linear id,
// and each XCD has its own L2.  All G workgroups of a row are placed on one
// XCD (row r on XCD r % 8, at consecutive slots there), so the head groups and
// key splits of a row share its key bytes in one L2 and the merge kernel finds
// the row's partial outputs there.
constexpr int kXcds = 8;
__host__ __device__ inline int64_t xcd_grid(int64_t R, int64_t G) { return (R + kXcds - 1) / kXcds * kXcds * G; }
// workgroup id -> (row, index g < G within the row)
__device__ __forceinline__ int xcd_slot(unsigned id, int G, int& r)
{
    const int xcd = (int)(id % kXcds), slot = (int)(id / kXcds);
    r = slot / G * kXcds + xcd;
    return slot % G;
}

// Kind of a 64-key tile (uniform): 0 all Top-K slots, 1 all SWA rows, 2 both.
__device__ __forceinline__ int tile_kind(int tile, int K)
{
    return (tile + 1) * kTile <= K ? 0 : (tile * kTile >= K ? 1 : 2);
}

// LDS slot of the partial S^T that wave `src` computed for fragment f != src.
__device__ __forceinline__ int red_slot(int f, int src) { return f * 3 + (src < f ? src : src - 1); }

template <int HT>
__device__ __forceinline__ void pick_own(const f32x4 (&a)[4][HT], int wave, f32x4 (&dst)[HT])
{
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const f32x4 x01 = wave == 0 ? a[0][ht] : a[1][ht];
        const f32x4 x23 = wave == 2 ? a[2][ht] : a[3][ht];
        dst[ht] = wave < 2 ? x01 : x23;
    }
}

template <int HT, int D>
__global__ __launch_bounds__(256, 1) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int64_t* __restrict__ seq_start, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ topk, int32_t K,
    const uint8_t* __restrict__ swa, const int64_t* __restrict__ swa_row_start,
    const int32_t* __restrict__ swa_len, int32_t R, int32_t H, int32_t W, float scale_log2e, int32_t HG,
    int32_t S, int32_t ntiles, float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml)
{
    constexpr int DW = D / 4;        // channels per wave
    constexpr int KT = D / 128;      // k-steps per fragment
    constexpr int NDT = DW / 16;     // 16-channel output tiles per wave
    constexpr int VST = D + 16;      // V tile row stride in halves (bank spread)
    constexpr int PST = kTile + 8;   // P row stride in halves
    constexpr int NH = HT * 16;

    __shared__ __attribute__((aligned(16))) _Float16 Vt[kTile * VST];
    __shared__ __attribute__((aligned(16))) f32x4 red[12][HT][CSA2_WAVE];
    __shared__ __attribute__((aligned(16))) _Float16 Pt[NH * PST];
    __shared__ __attribute__((aligned(16))) _Float16 Plo[NH * PST];
    __shared__ __attribute__((aligned(16))) f16x8 qa_s[HT * KT][256];
    __shared__ float wmax[4][NH];
    __shared__ __attribute__((aligned(16))) float alpha_s[NH];
    __shared__ float wl[4][NH];
    __shared__ float wle[4][NH];
    __shared__ float mfin[NH];
    __shared__ uint32_t wbig[4];
    __shared__ uint32_t wraise[4];

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    int r, hg, s;
    {
        const int g = xcd_slot(blockIdx.x, HG * S, r);
        hg = g % HG;
        s = g / HG;
    }
    if (r >= R) return;   // padding of the XCD mapping (whole workgroup, before any barrier)
    const int h0 = hg * NH;
    const int ch0 = lane_ch0<D>(wave, grp);     // channel of this lane's k-step 0
    const bool upper = lane >= 32;
    const int t_begin = (int)((int64_t)ntiles * s / S), t_end = (int)((int64_t)ntiles * (s + 1) / S);
    const int32_t* topk_row = topk + (int64_t)r * K;

    // Loads are issued in dependency order so that waiting for one never waits
    // for a later chain: the query first, then the row's metadata and the
    // first two tiles' Top-K entries, then (after the sequence's first row is
    // known) the first tile's key bytes.  The query is converted while those
    // are in flight.
    uint4 qraw[HT][KT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int h = h0 + ht * 16 + col;
#pragma unroll
        for (int t = 0; t < KT; ++t)
            qraw[ht][t] = h < H ? *reinterpret_cast<const uint4*>(q + ((int64_t)r * H + h) * D + ch0 + 16 * t)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
    // Top-K entries of the lane's 4 slots of a tile.  SWA slots are left as
    // they are (TileRaw::load never reads them); no select on the loaded
    // value, so nothing waits for the load here.
    auto load_idx = [&](int tile, int (&idx)[4]) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int slot = tile * kTile + 16 * f + col;
            if (slot < K) idx[f] = topk_row[slot];
        }
    };
    int idx0[4] = {0, 0, 0, 0}, idx_n[4] = {0, 0, 0, 0};
    const int n = row_len[r];
    const int seq = row_seq[r];
    int nsw = W > 0 ? swa_len[r] : 0;
    const int64_t swa0 = W > 0 ? swa_row_start[r] : 0;
    load_idx(t_begin, idx0);
    if (t_begin + 1 < t_end) load_idx(t_begin + 1, idx_n);
    nsw = nsw < 0 ? 0 : (nsw > W ? W : nsw);
    const int64_t base = seq_start[seq];
    const uint8_t* const crow = codes + base * (D / 2) + ch0 / 2;
    const uint8_t* const srow = scales + base * (D / 16) + ch0 / 16;
    const uint8_t* const wrow = swa + swa0 * D + ch0;   // not dereferenced when W == 0
    TileRaw<D> cur, nxt;   // cur is unpaired in place at the start of its tile
    cur.load(t_begin, idx0, col, grp & 1, K, n, nsw, crow, srow, wrow);

    // Query heads (B operand): lane (head col, grp) holds channels ch0 + 16 t
    // .. +8 for k-step t.  bf16 -> fp16 is exact for |q| in [2^-14, 65504].
    f16x8 qf[HT][KT];
    float q32[HT][KT][8];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const uint32_t ws[4] = {qraw[ht][t].x, qraw[ht][t].y, qraw[ht][t].z, qraw[ht][t].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                q32[ht][t][2 * e] = __uint_as_float(ws[e] << 16);
                q32[ht][t][2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qf[ht][t][e] = (_Float16)q32[ht][t][e];
                m = fmaxf(m, fabsf(q32[ht][t][e]));
            }
        }
        m = fmaxf(m, shfl_xor_f(m, 16));
        m = fmaxf(m, shfl_xor_f(m, 32));
        if (grp == 0) wmax[wave][ht * 16 + col] = m;
    }
    __syncthreads();
    // a-part of each head: q rounded to a multiple of 2^(E-11), 2^E > max|q|
    // (E >= -13 keeps the quantum within fp16's subnormal grid).  Adding and
    // subtracting 1.5 * 2^(E+12) rounds to that multiple in fp32.
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int hh = ht * 16 + col;
        const float m = fmaxf(fmaxf(wmax[0][hh], wmax[1][hh]), fmaxf(wmax[2][hh], wmax[3][hh]));
        int E = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 126 : -13;
        E = E < -13 ? -13 : E;
        const float C = __uint_as_float((uint32_t)(E + 12 + 127) << 23 | 0x400000u);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            f16x8 av;
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = (_Float16)((q32[ht][t][e] + C) - C);
            qa_s[ht * KT + t][threadIdx.x] = av;
        }
    }
    // (qa_s and wmax are next touched after the first barrier of the tile loop)

    // Online softmax state (log2 domain).  The reference max of a head is
    // raised only when a tile's max exceeds it by more than kLazy, so the
    // accumulated output is rarely rescaled; probabilities stay <= 2^kLazy.
    // Every wave tracks the same reference (from the workgroup-wide tile max)
    // and its own keys' part of the row sum.
    // l_p: sum of the probabilities as PV weights them (normalises the
    // output); l_e: sum of the unrounded probabilities (for lse).
    float m_p[HT], l_p[HT], l_e[HT];
    f32x4 o[HT][NDT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        m_p[ht] = -INFINITY;
        l_p[ht] = 0.0f;
        l_e[ht] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[ht][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }
    _Float16* const vbase = Vt + col * VST + ch0;
    const f16x8* const qa_lane = &qa_s[0][threadIdx.x];

    for (int tile = t_begin; tile < t_end; ++tile) {
        __syncthreads();   // (A) LDS buffers of the previous tile are free
        // Large values (|v| > 8) make the output sensitive to logit rounding:
        // a logit error e moves the output by about e * |v - out|.  A wave whose
        // keys may hold such values computes its score slice exactly as a
        // (hi, lo) pair; the whole tile then sums the slices with TwoSum and
        // uses two-part probabilities in PV.
        const bool my_big = __ballot(cur.big()) != 0ull;
        const int kind = tile_kind(tile, K);
        if (kind == 0) cur.template unpair<0>();
        else if (kind == 1) cur.template unpair<1>();
        else cur.template unpair<2>();
        // prefetch: raw bytes of the next tile, Top-K entries of the one after
        if (tile + 1 < t_end) {
            nxt.load(tile + 1, idx_n, col, grp & 1, K, n, nsw, crow, srow, wrow);
            if (tile + 2 < t_end) load_idx(tile + 2, idx_n);
        }

        f32x4 acc[4][HT], lo[4][HT];
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                acc[f][ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
                lo[f][ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            }
        if (my_big) s_tile<true, 2, HT, KT, D, VST>(cur, qf, qa_lane, upper, vbase, acc, lo);
        else if (kind == 0) s_tile<false, 0, HT, KT, D, VST>(cur, qf, qa_lane, upper, vbase, acc, lo);
        else if (kind == 1) s_tile<false, 1, HT, KT, D, VST>(cur, qf, qa_lane, upper, vbase, acc, lo);
        else s_tile<false, 2, HT, KT, D, VST>(cur, qf, qa_lane, upper, vbase, acc, lo);

        // ---- sum the four channel slices: wave w keeps fragment w
#pragma unroll
        for (int f = 0; f < 4; ++f)
            if (f != wave)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) red[red_slot(f, wave)][ht][lane] = acc[f][ht];
        if (lane == 0) wbig[wave] = my_big ? 1u : 0u;
        __syncthreads();   // (B)
        const bool precise = (wbig[0] | wbig[1] | wbig[2] | wbig[3]) != 0u;
        f32x4 sh[HT], sl[HT];
        pick_own<HT>(acc, wave, sh);
        pick_own<HT>(lo, wave, sl);
        if (precise) {
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const int src = (wave + k) & 3;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    two_sum_into(sh[ht], sl[ht], red[red_slot(wave, src)][ht][lane]);
                }
            }
            __syncthreads();   // all high parts read; the buffer takes the low parts
#pragma unroll
            for (int f = 0; f < 4; ++f)
                if (f != wave)
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) red[red_slot(f, wave)][ht][lane] = lo[f][ht];
            __syncthreads();
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const int src = (wave + k) & 3;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) sl[ht] += red[red_slot(wave, src)][ht][lane];
            }
        } else {
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const int src = (wave + k) & 3;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) sh[ht] += red[red_slot(wave, src)][ht][lane];
            }
        }

        // S^T lane layout: head h0 + 16 ht + col, keys 16 wave + 4 grp + i
        const bool v0 = wave == 0 ? cur.valid[0] : cur.valid[1];
        const bool v1 = wave == 2 ? cur.valid[2] : cur.valid[3];
        const uint64_t vb = __ballot(wave < 2 ? v0 : v1);
        float x[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kv = (vb >> (4 * grp + i)) & 1ull;
                x[ht][i] = kv ? (sh[ht][i] + sl[ht][i]) * scale_log2e : -INFINITY;
                mx = fmaxf(mx, x[ht][i]);
            }
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            if (grp == 0) wmax[wave][ht * 16 + col] = mx;
        }

        // Probabilities enter PV as fp16, whose rounding (relative 2^-12) moves
        // the output by up to 2^-12 * |v - out|; in a precise tile they are
        // split into fp16 hi + lo parts and PV runs twice (rounding ~2^-23).
        // They are first formed against the current reference m_p, which is
        // right unless some key of the tile exceeds it by more than kLazy; a
        // wave that sees such a key flags it, and after the barrier all waves
        // redo the tile's probabilities against the raised reference (the
        // first tile of a workgroup, and rarely later ones).
        auto probs = [&](int ht, float mn, float& ps, float& pe) {
            const int hh = ht * 16 + col;
            const bool live = mn != -INFINITY;
            ps = 0.0f;
            pe = 0.0f;
            f16x4 p4, q4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the exponent's argument is formed with one rounding at its own
                // (small) magnitude; the reference itself only has to be consistent
                const float d = fmaf(sh[ht][i], scale_log2e, -mn) + sl[ht][i] * scale_log2e;
                const float pf = (live && x[ht][i] != -INFINITY) ? exp2f(d) : 0.0f;
                const _Float16 p = (_Float16)pf;
                p4[i] = p;
                q4[i] = (_Float16)(pf - (float)p);
                ps += precise ? pf : (float)p;   // normalise by what PV actually weights
                pe += pf;
            }
            *reinterpret_cast<f16x4*>(&Pt[hh * PST + wave * 16 + 4 * grp]) = p4;
            if (precise) *reinterpret_cast<f16x4*>(&Plo[hh * PST + wave * 16 + 4 * grp]) = q4;
        };
        bool raise = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) raise |= x[ht][i] > m_p[ht] + kLazy;
        const bool wave_raise = __ballot(raise) != 0ull;
        float ps[HT], pe[HT];
        if (!wave_raise) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) probs(ht, m_p[ht], ps[ht], pe[ht]);
        }
        if (lane == 0) wraise[wave] = wave_raise ? 1u : 0u;
        __syncthreads();   // (C) P against the old reference, raise flags

        if ((wraise[0] | wraise[1] | wraise[2] | wraise[3]) != 0u) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const int hh = ht * 16 + col;
                const float mt = fmaxf(fmaxf(wmax[0][hh], wmax[1][hh]), fmaxf(wmax[2][hh], wmax[3][hh]));
                const float mn = (mt > m_p[ht] + kLazy) ? mt : m_p[ht];
                const float ap = mn != -INFINITY ? exp2f(m_p[ht] - mn) : 1.0f;
                probs(ht, mn, ps[ht], pe[ht]);
                l_p[ht] = l_p[ht] * ap + ps[ht];
                l_e[ht] = l_e[ht] * ap + pe[ht];
                if (wave == 0 && grp == 0) alpha_s[hh] = (m_p[ht] != -INFINITY && mn != m_p[ht]) ? ap : 1.0f;
                m_p[ht] = mn;
            }
            __syncthreads();   // (D) rewritten P, rescale factors

            // O lane layout: channel c0 + 16 dt + col, heads 16 ht + 4 grp + i
            bool rescale = false;
            f32x4 al[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                al[ht] = *reinterpret_cast<const f32x4*>(&alpha_s[ht * 16 + 4 * grp]);
#pragma unroll
                for (int i = 0; i < 4; ++i) rescale |= al[ht][i] != 1.0f;
            }
            if (__ballot(rescale) != 0ull) {
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) o[ht][dt] *= al[ht];
            }
        } else {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                l_p[ht] += ps[ht];
                l_e[ht] += pe[ht];
            }
        }
        if (precise) pv_tile<true, HT, NDT, VST, PST>(Pt, Plo, Vt, col, grp, wave * DW, o);
        else pv_tile<false, HT, NDT, VST, PST>(Pt, Plo, Vt, col, grp, wave * DW, o);
        cur = nxt;
    }

    // Row sums over the four waves' keys; the reference max is the same in
    // every wave.
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        float lt = l_p[ht], le = l_e[ht];
        lt += shfl_xor_f(lt, 16);
        lt += shfl_xor_f(lt, 32);
        le += shfl_xor_f(le, 16);
        le += shfl_xor_f(le, 32);
        if (grp == 0) {
            wl[wave][ht * 16 + col] = lt;
            wle[wave][ht * 16 + col] = le;
        }
        if (wave == 0 && grp == 0) mfin[ht * 16 + col] = m_p[ht];
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
            const float Le = wle[0][hh] + wle[1][hh] + wle[2][hh] + wle[3][hh];
            const float M = mfin[hh];
            if (S == 1) {
                const float inv = L > 0.0f ? 1.0f / L : 0.0f;
                float* op = out + ((int64_t)r * H + h) * D + wave * DW + col;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) op[16 * dt] = o[ht][dt][i] * inv;
                if (lse && wave == 0 && col == 0)
                    lse[(int64_t)r * H + h] = L > 0.0f ? M * kLn2 + logf(Le) : -INFINITY;
            } else {
                float* op = part_o + (((int64_t)r * S + s) * H + h) * D + wave * DW + col;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) op[16 * dt] = o[ht][dt][i];
                if (wave == 0 && col == 0) {
                    *reinterpret_cast<float4*>(part_ml + (((int64_t)r * S + s) * H + h) * 4) =
                        make_float4(M, L, Le, 0.0f);
                }
            }
        }
    }
}

// Merge of split partials: o = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// lse from the unrounded sums.  Partial statistics per (row, split, head):
// (m, l, l_exact, 0).  One workgroup per (row, head), placed on the row's XCD;
// each thread owns four consecutive channels and requests all splits at once.
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int32_t R, int32_t H,
                                                      int32_t D, int32_t S, float* __restrict__ out,
                                                      float* __restrict__ lse)
{
    int r;
    const int h = xcd_slot(blockIdx.x, H, r);
    if (r >= R) return;
    const int64_t rh = (int64_t)r * H + h;
    float4 st[kMaxPlanSplits];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxPlanSplits; ++k) {
        st[k] = k < S ? *reinterpret_cast<const float4*>(part_ml + (((int64_t)r * S + k) * H + h) * 4)
                      : make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
        if (st[k].y > 0.0f) M = fmaxf(M, st[k].x);
    }
    float L = 0.0f, Le = 0.0f, w[kMaxPlanSplits];
#pragma unroll
    for (int k = 0; k < kMaxPlanSplits; ++k) {
        w[k] = st[k].y > 0.0f ? exp2f(st[k].x - M) : 0.0f;
        L += st[k].y * w[k];
        Le += st[k].z * w[k];
    }
    if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? M * kLn2 + logf(Le) : -INFINITY;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int d = 4 * threadIdx.x; d < D; d += 4 * blockDim.x) {
        float4 v[kMaxPlanSplits];
#pragma unroll
        for (int k = 0; k < kMaxPlanSplits; ++k)
            v[k] = k < S ? *reinterpret_cast<const float4*>(part_o + (((int64_t)r * S + k) * H + h) * D + d)
                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int k = 0; k < kMaxPlanSplits; ++k) {
            acc.x += w[k] * v[k].x; acc.y += w[k] * v[k].y; acc.z += w[k] * v[k].z; acc.w += w[k] * v[k].w;
        }
        *reinterpret_cast<float4*>(out + rh * D + d) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}

struct AttnPlan {
    int HT, HG, S, ntiles;
};

// Heads per workgroup (16 HT) and key splits per row.  A workgroup's cost is
// dominated by per-tile latency (loads, four barriers) rather than by its
// MFMA work, so the head count per group only grows (sharing each key's
// dequantisation among more heads) once the rows alone give every compute
// unit a workgroup; otherwise rows are spread over head groups and, as far as
// needed to reach about one workgroup per compute unit, over key splits
// (each split adds a partial output for the merge kernel).  Measured on
// MI355X at 64 heads, D = 512, 640 keys per row: 32 rows -> 16 heads x 2
// splits; 256 rows -> 32 heads, no split; 4 rows -> 16 heads x 8 splits.
AttnPlan plan_attn(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W)
{
    constexpr int64_t kTargetGroups = 256;
    AttnPlan p;
    p.ntiles = (K + W + kTile - 1) / kTile;
    if (p.ntiles < 1) p.ntiles = 1;
    const int64_t rows_x_32 = (int64_t)R * ((H + 31) / 32);
    const int64_t rows_x_64 = (int64_t)R * ((H + 63) / 64);
    if (D <= 128 && H > 32 && rows_x_64 >= kTargetGroups) p.HT = 4;
    else if (H > 16 && rows_x_32 >= kTargetGroups) p.HT = 2;
    else p.HT = 1;
    p.HG = (H + 16 * p.HT - 1) / (16 * p.HT);
    const int64_t base = (int64_t)R * p.HG;
    int64_t S = base >= kTargetGroups ? 1 : (kTargetGroups + base - 1) / base;
    if (S > kMaxPlanSplits) S = kMaxPlanSplits;
    if (S > p.ntiles) S = p.ntiles;
    p.S = (int)S;
    return p;
}

template <int HT, int D>
void launch_attn(dim3 grid, hipStream_t st, const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                 const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len, const int32_t* topk,
                 int32_t K, const uint8_t* swa, const int64_t* swa_row_start, const int32_t* swa_len, int32_t H,
                 int32_t R, int32_t W, float sl2e, int HG, int S, int ntiles, float* out, float* lse, float* po,
                 float* pml)
{
    hipLaunchKernelGGL((k_sparse_attn<HT, D>), grid, dim3(256), 0, st, q, codes, scales, seq_start, row_seq,
                       row_len, topk, K, swa, swa_row_start, swa_len, R, H, W, sl2e, HG, S, ntiles, out, lse, po,
                       pml);
}

}  // namespace

extern "C" size_t csa2_sparse_attn_workspace_bytes(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W)
{
    if (R <= 0 || H <= 0 || D <= 0 || K < 0 || W < 0) return 0;
    const AttnPlan p = plan_attn(R, H, D, K, W);
    if (p.S <= 1) return 0;
    return csa2::align_up((size_t)R * p.S * H * D * 4, 256) + csa2::align_up((size_t)R * p.S * H * 4 * 4, 256);
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
    CSA2_REQUIRE(D == 128 || D == 256 || D == 512, CSA2_ERR_UNSUPPORTED,
                 "sparse_attn: D=%d (supported: 128, 256, 512)", D);
    CSA2_REQUIRE(K >= 0 && W >= 0, CSA2_ERR_SHAPE, "sparse_attn: K=%d, W=%d must be >= 0", K, W);
    CSA2_REQUIRE(K <= 4096 && W <= 4096, CSA2_ERR_UNSUPPORTED, "sparse_attn: K=%d or W=%d > 4096", K, W);
    if (R == 0) return CSA2_OK;
    CSA2_REQUIRE(q && codes && scales && seq_start && row_seq && row_len && out, CSA2_ERR_NULL,
                 "sparse_attn: NULL pointer argument");
    CSA2_REQUIRE(K == 0 || topk_idx, CSA2_ERR_NULL, "sparse_attn: topk_idx is NULL with K > 0");
    CSA2_REQUIRE(W == 0 || (swa && swa_row_start && swa_len), CSA2_ERR_NULL,
                 "sparse_attn: SWA pointers are NULL with W > 0");
    const AttnPlan p = plan_attn(R, H, D, K, W);
    CSA2_REQUIRE(xcd_grid(R, (int64_t)p.HG * p.S) <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED, "sparse_attn: grid too large");
    CSA2_REQUIRE(xcd_grid(R, H) <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED, "sparse_attn: grid too large");
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
    const dim3 grid((unsigned)xcd_grid(R, p.HG * p.S));
#define CSA2_ATTN(ht, d)                                                                               \
    if (p.HT == ht && D == d) {                                                                         \
        launch_attn<ht, d>(grid, st, q, codes, scales, seq_start, row_seq, row_len, topk_idx, K, swa,   \
                           swa_row_start, swa_len, H, R, W, sl2e, p.HG, p.S, p.ntiles, out, lse, po, pml); \
    }
    CSA2_ATTN(1, 128) CSA2_ATTN(1, 256) CSA2_ATTN(1, 512)
    CSA2_ATTN(2, 128) CSA2_ATTN(2, 256) CSA2_ATTN(2, 512)
    CSA2_ATTN(4, 128)
#undef CSA2_ATTN
    if (p.S > 1)
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)xcd_grid(R, H)), dim3(128), 0, st, po, pml, R, H, D, p.S,
                           out, lse);
    return csa2::check_launch("sparse_attn");
}
