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
// Work decomposition.  One workgroup (8 waves, two per SIMD) = one query row
// x NH = 16*HT heads x a contiguous range of 16-key fragments, taken in rounds
// of 8 fragments, fragment f0 + w of a round by wave w:
//   * scores: wave w dequantises its fragment's 16 keys straight from the
//     cache to fp16 in registers (E2M1 -> fp16 by the hardware converter,
//     times the E4M3 scale; the product is exact in fp16) and feeds them as the
//     A operand of v_mfma_f32_16x16x32_f16 against the NH query heads (B
//     operand, all D channels held in registers): S^T of the fragment.  The
//     same fp16 values go to the wave's V tile in LDS.
//   * softmax: the waves publish each fragment's per-head maximum; every wave
//     derives the same reference maximum per head from them (raised lazily,
//     log2 domain, so the output is rarely rescaled), and the owner turns its
//     scores into fp16 probabilities, published in the A operand layout of
//     v_mfma_f32_16x16x16_f16 (the S^T accumulator already has it).
//   * PV: output channels are split between the waves (D/8 each); every wave
//     multiplies the probabilities of all 8 fragments of the round into its
//     channels, reading its columns of the 8 V tiles transposed
//     (ds_read_b64_tr_b16).
// So each key is dequantised once per workgroup, a wave's accumulators hold
// only its channels (two waves fit one SIMD and hide each other's latency),
// and the end needs no merge of outputs between waves.  With many rows
// (prefill chunks) the same scheme runs with four waves and rounds of four
// fragments: half the LDS, so two workgroups share each compute unit and
// their phases interleave.  Rows whose fragments
// are split across workgroups write unnormalised partial outputs plus (max,
// sums): with two splits the second workgroup of the pair to finish merges
// the first's partial into its own output; with more, k_attn_combine merges
// them.
//
// Exact scores for keys with large values.  The matrix cores sum products
// with errors of a few units in the last place of the largest addend, and
// with |v| in the hundreds a near tie between two keys turns such a score
// error into an output error far above the tolerance.  Where a fragment's
// keys may hold |v| > 8 its scores are computed exactly instead: each query
// head is split as q = a + b, a being q rounded to a multiple of 2^(E-11) with
// 2^E > max|q| of the head (11 bits, exact in fp16), b the small remainder.
// Within one scale group every a*k product is then an integer multiple of one
// quantum and the 16 products sum to less than 2^24 quanta, so MFMAs
// restricted to one group (a lane group's two k-steps over it, the other lane
// groups masked to zero) return the group sum exactly; the group sums are
// accumulated in fp64, and K b^T (small, nonzero only for channels with
// |q| < max|q|/16) is added from an ordinary MFMA chain.
#include "csa2_device.h"
#include "csa2_host.h"

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kFrag = 16;           // keys per fragment (one MFMA row block)
constexpr int kWaves = 8;           // waves per workgroup (two per SIMD), fragments per round
constexpr int kWavesMany = 4;       // the same with many rows: half the LDS, two workgroups per compute unit
constexpr float kLazy = 8.0f;       // log2-domain slack before a running max is raised
constexpr int kMaxPlanSplits = 8;   // key splits per row, at most

// Channel layout of a lane (col, grp): k-step t (t < KS = D/32) covers the
// 8 channels
//   D/4*grp + 8*t .. +8,
// so each lane's k-steps run through one contiguous quarter of the channels,
// which is the block of a key's bytes it loads (no exchange between lanes),
// and k-steps 2u, 2u+1 of a lane share scale group D/64*grp + u.  In each
// MFMA the four lane groups hold 8 channels of four different scale groups.
template <int D>
__device__ __forceinline__ int step_ch(int grp, int t)
{
    return (D / 4) * grp + 8 * t;
}

// Main entries are read through 64-bit addresses once the slot's entry is
// checked against the row (FragRaw::load_row).  A row's SWA window is read
// with buffer loads: one descriptor spans exactly the window's valid bytes,
// and the hardware returns zeros for any dword outside it.  A slot without an
// SWA row gets the offset kNoKey, beyond the descriptor's range (kept below
// 2^31 bytes), so those loads are unconditional and a missing row reads as
// zero bytes.
constexpr uint32_t kNoKey = 0x80000000u;
constexpr int32_t kBufConfig = 0x00020000;   // raw 32-bit buffer, as for gfx9 data loads
// Descriptor of a buffer whose base and size are the same in every lane; the
// values are passed through readfirstlane so that the compiler keeps the
// descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int32_t bytes)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b), hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void* const ub = reinterpret_cast<void*>((uint64_t)hi << 32 | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufConfig);
}

// Raw bytes of one fragment held by one lane: the lane's channels of its key
// (col): FP4 codes (one word per k-step) and the KS E4M3 scale bytes of a
// selected main entry, or FP8 bytes (two words per k-step) of an SWA row.  A
// slot without a valid key reads zero bytes, so it dequantises to zeros.
template <int D>
struct FragRaw {
    static constexpr int KS = D / 32;
    static constexpr int NSC = KS / 8 > 1 ? KS / 8 : 1;   // words of the lane's KS/2 scale bytes (D = 128: one
                                                        // word, its two bytes in the low half)
    uint32_t raw[2 * KS];
    uint32_t sc[NSC];
    _Float16 sp[KS / 2];   // the lane's scale groups as fp16 (set by scales_f16())
    bool valid;

    // SWA row i of the lane's slot (vs: the slot holds one) through rw, the
    // buffer over the row's window: the lane's quarter of the row (D/4
    // contiguous bytes) into consecutive words.  An absent row gets the offset
    // kNoKey and reads as zeros; the loads are unconditional.
    __device__ __forceinline__ void load_swa(bool vs, int i, int grp, __amdgpu_buffer_rsrc_t rw)
    {
        valid = vs;
        const uint32_t off1 = vs ? (uint32_t)i * D + (D / 4) * grp : kNoKey;
#pragma unroll
        for (int u = 0; u < KS / 2; ++u) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off1 + 16 * u, 0, 0);
            raw[4 * u] = v[0]; raw[4 * u + 1] = v[1]; raw[4 * u + 2] = v[2]; raw[4 * u + 3] = v[3];
        }
        // (the scale words are loaded too, as zeros from past the buffer's
        // end, so that on either kind of fragment every raw register is
        // written by a load: the loop then waits on loads in issue order)
        if constexpr (NSC == 2) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, kNoKey, 0, 0);
            sc[0] = v[0]; sc[1] = v[1];
        } else {
            sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, kNoKey, 0, 0);
        }
    }

    // The lane's bytes of main entry j (vm: the slot holds a visible entry)
    // from codes / scales, which start at the row's first entry (or at the
    // cache's first row in the cache-row form): the codes of its quarter of
    // the channels (D/8 bytes) and the KS/2 scale bytes of their groups,
    // through 64-bit addresses, so entries anywhere in a cache of any size are
    // reachable; an absent slot loads nothing and keeps zeros.
    __device__ __forceinline__ void load_row(bool vm, int j, int grp, const uint8_t* codes, const uint8_t* scales)
    {
        valid = vm;
        // (words KS .. 2 KS - 1 hold FP8 bytes of window rows only: nothing
        // reads them for a main entry)
#pragma unroll
        for (int k = 0; k < KS; ++k) raw[k] = 0u;
#pragma unroll
        for (int w = 0; w < NSC; ++w) sc[w] = 0u;
        if (vm) {
            const uint8_t* pc = codes + (uint64_t)(uint32_t)j * (D / 2) + (D / 8) * grp;
#pragma unroll
            for (int u = 0; u < KS / 4; ++u) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(pc + 16 * u);
                raw[4 * u] = v[0]; raw[4 * u + 1] = v[1]; raw[4 * u + 2] = v[2]; raw[4 * u + 3] = v[3];
            }
            const uint8_t* ps = scales + (uint64_t)(uint32_t)j * (D / 16);
            if constexpr (KS / 2 == 8) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(ps + 8 * grp);
                sc[0] = v[0]; sc[1] = v[1];
            } else if constexpr (KS / 2 == 4) {
                sc[0] = *reinterpret_cast<const uint32_t*>(ps + 4 * grp);
            } else {   // two bytes: the word of the lane pair, the lane's half shifted down
                sc[0] = *reinterpret_cast<const uint32_t*>(ps + 4 * (grp >> 1)) >> (16 * (grp & 1));
            }
        }
    }

    // The scale bytes as fp16, converted before the next fragment's loads are
    // issued, so that nothing after those loads reads the raw scale words.
    // KIND: 0 Top-K slots only, 1 SWA rows only (no scales).
    template <int KIND>
    __device__ __forceinline__ void scales_f16()
    {
        if (KIND != 1) {
#pragma unroll
            for (int u = 0; u < KS / 4; ++u) {
                const f16x2 v = (u & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[u >> 1], 1.0f, true)
                                        : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[u >> 1], 1.0f, false);
                sp[2 * u] = v[0];
                sp[2 * u + 1] = v[1];
            }
        }
    }

    // Whether this lane's key may hold |v| > 8: an FP4 group holds
    // |v| <= 6 * scale, so a scale byte of 0x3B (1.375) or more; an FP8 byte
    // of magnitude 0x50 (8.0) or more.  Adding 0x45 (resp. 0x30) to a 7-bit
    // magnitude sets bit 7 exactly at that threshold, with no carry between
    // bytes.
    template <int KIND>
    __device__ __forceinline__ bool big() const
    {
        static_assert(KIND == 0 || KIND == 1, "a fragment holds one kind of slot");
        uint32_t bm = 0u, bs = 0u;
        if (KIND == 0) {
#pragma unroll
            for (int w = 0; w < NSC; ++w) bm |= ((sc[w] & 0x7F7F7F7Fu) + 0x45454545u) & 0x80808080u;
        }
        if (KIND == 1) {
#pragma unroll
            for (int w = 0; w < 2 * KS; ++w) bs |= ((raw[w] & 0x7F7F7F7Fu) + 0x30303030u) & 0x80808080u;
        }
        const uint32_t bits = KIND == 0 ? bm : bs;
        return valid && bits != 0u;
    }
};

// Dequantise k-step t (8 channels) of the lane's key to fp16.
//   MODE 0: FP4 codes (word t) times the group's E4M3 scale (scale byte t/2
//           of the lane's KS/2 scale bytes);
//   MODE 1: FP8 E4M3 bytes (words 2t, 2t+1), unscaled.
template <int MODE, int D>
__device__ __forceinline__ f16x8 dequant_step(const FragRaw<D>& fr, int t)
{
    static_assert(MODE == 0 || MODE == 1, "a fragment holds one kind of slot");
    f16x8 a, b;
    if (MODE == 0) {
        const uint32_t c = fr.raw[t];
        const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
        const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
        const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
        const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
        const _Float16 s = fr.sp[t >> 1];
        a = (f16x8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]} * s;
    }
    if (MODE == 1) {
        const uint32_t c0 = fr.raw[2 * t], c1 = fr.raw[2 * t + 1];
        const f16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false);
        const f16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true);
        const f16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false);
        const f16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true);
        b = (f16x8){b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
    }
    if constexpr (MODE == 0) return a;
    else return b;
}

// Store k-step t of the lane's key to its row (vrow) of the wave's V tile.
template <int D>
__device__ __forceinline__ void v_store(_Float16* vrow, int grp, int t, f16x8 kf)
{
    *reinterpret_cast<f16x8*>(vrow + step_ch<D>(grp, t)) = kf;
}

// Query pieces (B operand of the score MFMAs; piece (ht, t) = k-step t of head
// tile ht, this lane's column) and their a-parts for exact scores (split of q
// described at the top of the file).
template <int HT, int D>
struct QueryRegs {   // the query in registers, the a-parts in LDS ([HT * KS][64])
    static constexpr bool kPackedSub = true;   // b-parts by packed adds (eight waves: registers to spare)
    const f16x8 (&qf)[HT][D / 32];
    const f16x8* qa;
    __device__ __forceinline__ f16x8 q(int ht, int t) const { return qf[ht][t]; }
    __device__ __forceinline__ f16x8 a(int ht, int t) const { return qa[(ht * (D / 32) + t) * CSA2_WAVE]; }
};
// Rounding constant of a head's a-parts from its largest magnitude m:
// 1.5 * 2^(E+12) with 2^E > m, E >= -13.
__device__ __forceinline__ float a_part_const(float m)
{
    int E = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 126 : -13;
    E = E < -13 ? -13 : E;
    return __uint_as_float((uint32_t)(E + 12 + 127) << 23 | 0x400000u);
}
template <int HT, int D>
struct QueryRegsC {   // the query in registers, the a-parts formed from it
    static constexpr bool kPackedSub = false;   // (four waves: the compiler's form schedules better at their budget)
    const f16x8 (&qf)[HT][D / 32];
    const float (&C)[HT];   // per head tile: the rounding constant 1.5 * 2^(E + 12) of the a-part
    __device__ __forceinline__ f16x8 q(int ht, int t) const { return qf[ht][t]; }
    __device__ __forceinline__ f16x8 a(int ht, int t) const
    {
        // formed where it is used: kept from being hoisted out of the
        // fragment loop, where all of them would hold registers throughout
        u32x4 w = __builtin_bit_cast(u32x4, qf[ht][t]);
        asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
        const f16x8 v = __builtin_bit_cast(f16x8, w);
        f16x8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)(((float)v[e] + C[ht]) - C[ht]);
        return r;
    }
};
template <int HT, int D>
struct QueryLds {    // the query in LDS ([HT * KS][64]); a-parts formed from it
    static constexpr bool kPackedSub = true;
    const f16x8* qs;
    const float (&C)[HT];   // per head tile: the rounding constant 1.5 * 2^(E + 12) of the a-part
    __device__ __forceinline__ f16x8 q(int ht, int t) const { return qs[(ht * (D / 32) + t) * CSA2_WAVE]; }
    __device__ __forceinline__ f16x8 a(int ht, int t) const
    {
        const f16x8 v = q(ht, t);
        f16x8 r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)(((float)v[e] + C[ht]) - C[ht]);
        return r;
    }
};

// S^T of one fragment, fp32 MFMA chain; the dequantised keys also go to the
// wave's V tile.
template <int MODE, int HT, int D, class QS>
__device__ __forceinline__ void s_frag(const FragRaw<D>& fr, const QS& qs, _Float16* vrow, int grp, f32x4 (&acc)[HT])
{
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
        const f16x8 kf = dequant_step<MODE, D>(fr, t);
        v_store<D>(vrow, grp, t, kf);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qs.q(ht, t), acc[ht], 0, 0, 0);
    }
}

// Only the V tile of a fragment (its scores came from the native FP4 products).
template <int MODE, int D>
__device__ __forceinline__ void v_frag(const FragRaw<D>& fr, _Float16* vrow, int grp)
{
#pragma unroll
    for (int t = 0; t < D / 32; ++t) v_store<D>(vrow, grp, t, dequant_step<MODE, D>(fr, t));
}

// x - y on eight fp16 values as four packed adds of x and -y (the compiler
// splits a vector fp16 subtraction into single-half subtractions and packs).
__device__ __forceinline__ f16x8 sub_f16x8(f16x8 x, f16x8 y)
{
    const u32x4 xw = __builtin_bit_cast(u32x4, x), yw = __builtin_bit_cast(u32x4, y);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        asm("v_pk_add_f16 %0, %1, %2 neg_lo:[0,1] neg_hi:[0,1]" : "=v"(r[i]) : "v"(xw[i]), "v"(yw[i]));
    return __builtin_bit_cast(f16x8, r);
}

// The same fragment with S computed exactly as (hi, lo) = K a^T + K b^T
// (split of q described at the top of the file); b = q - a is an exact fp16
// subtraction (the difference is q's bits below the quantum of a).  MODE: the
// fragment's kind, as in dequant_step.

template <int MODE, int HT, int D, class QS>
__device__ __forceinline__ void s_frag_exact(const FragRaw<D>& fr, const QS& qs, _Float16* vrow, int grp,
                                             f32x4 (&acc)[HT], f32x4 (&lo)[HT])
{
    constexpr int KS = D / 32;
    double ex[HT][4];
    f32x4 sb[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        sb[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) ex[ht][i] = 0.0;
    }
    const f16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
    // k-steps 2u and 2u + 1 of a lane hold the two halves of one scale group
    // (D/64 grp + u).  One head tile: two products chained per lane group sum
    // its 16 channels; more (fewer registers to spare): one product per
    // k-step and lane group, 8 channels.
    if constexpr (HT == 1) {
#pragma unroll
        for (int t = 0; t < KS; t += 2) {
            const f16x8 kf0 = dequant_step<MODE, D>(fr, t), kf1 = dequant_step<MODE, D>(fr, t + 1);
            v_store<D>(vrow, grp, t, kf0);
            v_store<D>(vrow, grp, t + 1, kf1);
            const f16x8 a0 = qs.a(0, t), a1 = qs.a(0, t + 1);
            const f16x8 b0 = QS::kPackedSub ? sub_f16x8(qs.q(0, t), a0) : qs.q(0, t) - a0;
            const f16x8 b1 = QS::kPackedSub ? sub_f16x8(qs.q(0, t + 1), a1) : qs.q(0, t + 1) - a1;
            sb[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf0, b0, sb[0], 0, 0, 0);
            sb[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf1, b1, sb[0], 0, 0, 0);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // lane group g's channels of its scale group, the others zero
                const f16x8 k0 = grp == g ? kf0 : zero, k1 = grp == g ? kf1 : zero;
                f32x4 gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, a0, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, a1, gs, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) ex[0][i] += (double)gs[i];
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const f16x8 kf = dequant_step<MODE, D>(fr, t);
            v_store<D>(vrow, grp, t, kf);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const f16x8 a = qs.a(ht, t);
                const f16x8 b = QS::kPackedSub ? sub_f16x8(qs.q(ht, t), a) : qs.q(ht, t) - a;
                sb[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, b, sb[ht], 0, 0, 0);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f16x8 kg = grp == g ? kf : zero;
                    const f32x4 gs =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(kg, a, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) ex[ht][i] += (double)gs[i];
                }
            }
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

// Native FP4 scores (the scaled FP4 matrix-core product, no dequantisation).
// v_mfma_scale_f32_16x16x128_f8f6f4 takes the keys' E2M1 codes as the A
// operand and the query as E4M3 (B operand), each lane block of 32 values with
// one power-of-two (E8M0) scale.  Lane (key, g) holds, for k-step T < D/128,
// the 32 channels g*D/4 + 32T .. +31: exactly the 16 code bytes it loaded as
// words 4T .. 4T+3, whose two E4M3 scale bytes are those of groups
// g*D/64 + 2T and + 1 (bytes 2T and 2T + 1 of the lane's scale bytes).  The
// products equal the dequantised ones only where both bytes
// are the same power of two, which nat_key_scales() checks; the query side is
// checked once per workgroup, where the query's operand layout (which pairs
// each lane's values with the keys' in a fixed interleave) is built.  An
// absent key has zero codes, so any scale gives it zero products.
template <int D>
__device__ __forceinline__ bool nat_key_scales(const FragRaw<D>& f, uint32_t& e8)
{
    bool ok = true;
    e8 = 0u;
#pragma unroll
    for (int T = 0; T < D / 128; ++T) {
        const int b = 2 * T;   // the pair's first byte among the lane's (even: one word holds both)
        const uint32_t w = f.sc[b >> 2] >> (8 * (b & 3));
        const uint32_t s0 = w & 0xFFu, s1 = (w >> 8) & 0xFFu;
        // E4M3 2^(e - 7) with e = bits 6..3, positive, mantissa zero -> E8M0 e + 120
        ok = ok && s0 == s1 && (s0 & 0x87u) == 0u && s0 != 0u;
        e8 |= ((s0 >> 3) + 120u) << (8 * T);
    }
    return ok || !f.valid;
}

// S^T of a fragment from the native products: one MFMA per k-step and head
// tile, each lane's scales taken from byte T of the packed words.
template <int HT, int D>
__device__ __forceinline__ void s_frag_nat(const FragRaw<D>& fr, uint32_t ke8, const i32x8 (&qn)[HT][D / 128],
                                           const uint32_t (&qe8)[HT], f32x4 (&acc)[HT])
{
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        acc[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int T = 0; T < D / 128; ++T) {
            const i32x8 a = {(int)fr.raw[4 * T], (int)fr.raw[4 * T + 1], (int)fr.raw[4 * T + 2], (int)fr.raw[4 * T + 3],
                             0, 0, 0, 0};
            acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qn[ht][T], acc[ht], 4, 0, 0,
                                                                      (int)(ke8 >> (8 * T)), 0,
                                                                      (int)(qe8[ht] >> (8 * T)));
        }
    }
}

// O[heads x the wave's channels] += P V for G fragment slots of the round,
// all of whose LDS reads are issued before the first product.  The B operand
// is read with ds_read_b64_tr_b16: within each 16-lane group, lane l receives
// element l%4 of the 8-byte rows addressed by lanes 4i + l/4, so addressing
// row (key 4g + l/4, channels c0 + 4(l%4)) hands lane l the 4 keys 4g + 0..3
// of channel c0 + l, the key order of the probability operand.
// pp: this lane's probabilities of the first slot, [HT][64] apart by head
// tile, pstride apart by slot; vr: this lane's address in the first slot's
// tile at the wave's first channel, vstride apart by slot.
constexpr int kPvGroup = 4;
template <int G, int HT, int NDT>
__device__ __forceinline__ void pv_slots(const f16x4* pp, int pstride, const _Float16* vr, int vstride,
                                         f32x4 (&o)[HT][NDT])
{
    f16x4 pa[G][HT];
    lds_f16x4 b[G][NDT];
#pragma unroll
    for (int u = 0; u < G; ++u) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) pa[u][ht] = pp[u * pstride + ht * CSA2_WAVE];
#pragma unroll
        for (int k = 0; k < NDT; ++k)
            b[u][k] = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                (lds_f16x4 __attribute__((address_space(3)))*)(vr + u * vstride + 16 * k));
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
        for (int k = 0; k < NDT; ++k) {
            const f16x4 vb = {(_Float16)b[u][k][0], (_Float16)b[u][k][1], (_Float16)b[u][k][2], (_Float16)b[u][k][3]};
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                o[ht][k] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa[u][ht], vb, o[ht][k], 0, 0, 0);
        }
}

// Workgroups are handed to the 8 XCDs of the chip round-robin by linear id,
// and each XCD has its own L2.  All G workgroups of a row are placed on one
// XCD (row r on XCD r % 8, at consecutive slots there), so the head groups and
// key splits of a row share its key bytes in one L2.
constexpr int kXcds = 8;
__host__ __device__ inline int64_t xcd_grid(int64_t R, int64_t G) { return (R + kXcds - 1) / kXcds * kXcds * G; }
// workgroup id -> (row, index g < G within the row)
__device__ __forceinline__ int xcd_slot(unsigned id, int G, int& r)
{
    const int xcd = (int)(id % kXcds), slot = (int)(id / kXcds);
    r = slot / G * kXcds + xcd;
    return slot % G;
}

// Relaxed device-scope store: written through to the device's coherence point,
// so that a workgroup on any XCD reads it with a device-scope load once the
// store has completed.
__device__ __forceinline__ void store_coherent(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Rows with exactly two key splits have fewer than 256 (row, head group)
// pairs (the plan splits only below 256 groups): the arrival words of the
// pair merge fit in the first 1 KiB of the workspace.
constexpr int kPairWords = 256;
// Bound of a wait that always ends; running into it is counted as a device check.
constexpr int kSpinLimit = 1 << 22;

// Slot layout of a row: the Top-K slots padded to Kp = a multiple of 16, then
// the SWA rows, so that a fragment holds one kind of slot only.
__host__ __device__ inline int pad_topk(int K) { return (K + kFrag - 1) / kFrag * kFrag; }
// Kind of a fragment (uniform): 0 Top-K slots, 1 SWA rows.
__device__ __forceinline__ int frag_kind(int fr, int Kp) { return fr * kFrag >= Kp ? 1 : 0; }

// LDS of one workgroup: one V tile per fragment slot of a round (slot w
// filled by wave w), the a-parts of the query (exact scores, eight waves) and
// the round's probabilities; before the loop the query is staged where the
// tiles go.
template <int HT, int D, int NW>
struct AttnSmem {
    static constexpr int KS = D / 32;
    static constexpr int NH = HT * 16;
    static constexpr int CW = D / NW;              // output channels of a wave
    static constexpr int NDT = CW / 16;            // its output tiles per head tile
    static constexpr int VS = D + 8;               // V row stride in halves (conflict-free rows and transposes)
    static constexpr int kTile = kFrag * VS;       // halves per V tile
    static constexpr int kVBytes = NW * kTile * 2;
    // [HT * KS][64] f16x8: the a-parts of the query (eight waves) or, in the
    // native-FP4 form, the query itself; four waves form the a-parts from
    // the query registers instead, which halves the LDS per workgroup
    static constexpr int kQaBytes = NW == kWaves ? HT * KS * CSA2_WAVE * 16 : 0;
    static constexpr int kPBytes = NW * 2 * HT * CSA2_WAVE * 8;       // [slot][hi, lo][HT][64] f16x4
    static constexpr int kBytes = kVBytes + kQaBytes + kPBytes;
    static_assert(HT * KS * CSA2_WAVE * 16 <= kVBytes, "the query staging fits the V tiles");
    static_assert(D % (16 * NW) == 0 && NDT >= 1, "whole output tiles per wave");
};

// PG: the index lists hold cache rows (paged caches) and the SWA window may be
// a ring; the packed form is a separate instantiation so that it carries none
// of that addressing.  NAT: scores of Top-K fragments from the native FP4
// products wherever they are exact (s_frag_nat); the query then lives in LDS
// as fp16 for the other fragments and as E4M3 in registers, and nat_count (if
// not null) counts the fragments scored natively.
// NW: waves per workgroup, kWaves (one workgroup per compute unit) or
// kWavesMany (rows enough for two per compute unit: half the fragments per
// round, no LDS copy of the a-parts).
template <int HT, int D, bool PG, bool NAT, int NW>
__global__ __launch_bounds__(CSA2_WAVE * NW, NW == kWaves ? 1 : 2) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int64_t* __restrict__ seq_start, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ topk, int32_t K,
    const uint8_t* __restrict__ swa, const int64_t* __restrict__ swa_row_start,
    const int32_t* __restrict__ swa_len, const int32_t* __restrict__ swa_head, int64_t phys_rows, int32_t R,
    int32_t H, int32_t W, float scale_log2e, int32_t HG, int32_t S, int32_t nfrag, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml, int32_t* __restrict__ pair_sync,
    int32_t* __restrict__ nat_count)
{
    static_assert(NW == kWaves || (NW == kWavesMany && !NAT), "the native form runs with eight waves");
    using SM = AttnSmem<HT, D, NW>;
    constexpr int KS = SM::KS;
    constexpr int NH = SM::NH;
    constexpr int NDT = SM::NDT;
    constexpr int VS = SM::VS;

    __shared__ __attribute__((aligned(16))) char smem[SM::kBytes];
    __shared__ float4 fmx[NH][NW / 4];   // per head: each slot's largest logit of the head
    __shared__ float wsum[2][NW][NH];    // at the end: each wave's sums (PV weights, unrounded)
    __shared__ uint32_t wqm[NW][NH];     // per wave: bf16 bits of the max |q| of each head over its pieces
    __shared__ __attribute__((aligned(16))) uint32_t fprec[NW];   // per slot: its bit if the slot is precise (exact
                                                                  // scores, two-part probabilities), else 0
    _Float16* const vtiles = reinterpret_cast<_Float16*>(smem);
    f16x8* const qa_s = reinterpret_cast<f16x8*>(smem + SM::kVBytes);                  // [HT * KS][64]
    f16x4* const p_s = reinterpret_cast<f16x4*>(smem + SM::kVBytes + SM::kQaBytes);   // [slot][2][HT][64]
    f16x8* const qf_s = reinterpret_cast<f16x8*>(smem);                                // staging (before the loop)

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: branches on it are scalar
    const int col = lane & 15, grp = lane >> 4;
    int r, hg, s;   // row, head group, key split
    bool g_first;   // the row's first workgroup
    {
        const int g = xcd_slot(blockIdx.x, HG * S, r);
        hg = g % HG;
        s = g / HG;
        g_first = g == 0;
    }
    (void)g_first;
    if (r >= R) return;   // padding of the XCD mapping (whole workgroup, before any barrier)
    const int h0 = hg * NH;
    // Key splits take contiguous fragment ranges.  Two splits divide whole
    // rounds, the first taking half of them rounded up: with an odd number of
    // rounds the second finishes a round earlier and has published its partial
    // when the first needs it, instead of both finishing a half-filled last
    // round together with the merger then waiting for the publication.
    int f_begin = (int)((int64_t)nfrag * s / S), f_end = (int)((int64_t)nfrag * (s + 1) / S);
    if (S == 2) {
        const int rounds = (nfrag + NW - 1) / NW;
        const int mid = (rounds + 1) / 2 * NW < nfrag ? (rounds + 1) / 2 * NW : nfrag;
        f_begin = s == 0 ? 0 : mid;
        f_end = s == 0 ? mid : nfrag;
    }
    const int32_t* topk_row = topk + (int64_t)r * K;

    // Loads are issued in dependency order so that waiting for one never waits
    // for a later chain: the row's metadata (scalar) and the wave's first two
    // fragments' Top-K entries, the wave's pieces of the query, then the first
    // fragment's key bytes, which arrive during the barriers that share the
    // query.
    // PG: the index lists hold cache rows directly (paged caches),
    // checked against the cache size; otherwise entries of the row's sequence.
    const int n = PG ? (int)(phys_rows < 0x7FFFFFFF ? phys_rows : 0x7FFFFFFF) : row_len[r];
    const int seq = PG ? 0 : row_seq[r];
    int nsw = W > 0 ? swa_len[r] : 0;
    // SWA ring: window row i sits in slot (head + i) mod W of the row's W slots
    int head = 0;
    if constexpr (PG) {
        head = W > 0 && swa_head ? swa_head[r] % W : 0;
        head = head < 0 ? head + W : head;
    }
    const int64_t swa0 = W > 0 ? swa_row_start[r] : 0;
    // Top-K entry of the lane's key in a fragment; SWA slots are left as they
    // are (the key loads never read them), and no select on the loaded value
    // so nothing waits for the load here.
    auto load_idx = [&](int fr_, int& idx) {
        const int slot = fr_ * kFrag + col;
        if (slot < K) idx = topk_row[slot];
    };
    const int fw = f_begin + wave;   // the wave's fragment in the first round
    int idx_c = 0, idx_n = 0;
    if (fw < f_end) load_idx(fw, idx_c);
    if (fw + NW < f_end) load_idx(fw + NW, idx_n);
    // The query, as NQP pieces (piece P = ht * KS + t: k-step t of head tile
    // ht, the B operand layout); wave w loads and converts pieces w, w + 8, ...,
    // which go to LDS; every wave reads the whole query back after the
    // barrier.  The query is read through a buffer over its H heads: heads past
    // H read as zeros.
    constexpr int NQP = HT * KS;
    constexpr int NPW = (NQP + NW - 1) / NW;
    uint4 qraw[NPW];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + (int64_t)r * H * D, H * D * 2);
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int P = k * NW + wave;
            qraw[k] = make_uint4(0u, 0u, 0u, 0u);
            if (P < NQP) {
                const uint32_t hoff = (uint32_t)(h0 + (P / KS) * 16 + col) * (D * 2);
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, hoff + 2 * step_ch<D>(grp, P % KS), 0, 0);
                qraw[k] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    }
    CSA2_DCHECK(g_first && threadIdx.x == 0 && (nsw < 0 || nsw > W));
    nsw = nsw < 0 ? 0 : (nsw > W ? W : nsw);
    const int64_t base = PG ? 0 : seq_start[seq];
    // Query heads (B operand): lane (head col, grp) holds channels
    // step_ch(grp, t) .. +8 for k-step t.  bf16 -> fp16 is exact for |q| in
    // [2^-14, 65504].  a-part of a head: q rounded to a multiple of 2^(E-11),
    // 2^E > max|q| (E >= -13 keeps the quantum within fp16's subnormal grid).
    // Adding and subtracting Cq = 1.5 * 2^(E+12) rounds to that multiple in
    // fp32.  The a-parts are formed from the fp16 query where they are used,
    // and E from the largest fp16 magnitude of the head: below 2^-13, where
    // fp16 may round a bf16 value, E is -13 either way.
    float Cq[HT];
    if constexpr (NAT) {
        // the native form needs Cq before the query goes to LDS: the maximum
        // of each head over the waves' pieces (integer max of bf16 magnitudes)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            u16x2 mx = {0, 0};
#pragma unroll
            for (int k = 0; k < NPW; ++k) {
                const int P = k * NW + wave;
                if (P < NQP && P / KS == ht) {
                    const uint32_t ws[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, ws[e] & 0x7FFF7FFFu));
                }
            }
            uint32_t mb = mx[0] > mx[1] ? mx[0] : mx[1];
            mb = umax_xor32(umax_xor16(mb));
            if (grp == 0) wqm[wave][ht * 16 + col] = mb;
        }
        __syncthreads();
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            uint32_t mb = 0u;
#pragma unroll
            for (int w = 0; w < NW; ++w) mb = max(mb, wqm[w][ht * 16 + col]);
            Cq[ht] = a_part_const(__uint_as_float(mb << 16));
        }
    }
    // Staging: wave w converts pieces w, w + NW, ... to fp16 and stores them
    // in LDS, in the V tiles' space (the native form: in its query region,
    // where the query stays).
    f16x8* const stage = NAT ? qa_s : qf_s;
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
        const int P = k * NW + wave;
        if (P >= NQP) continue;
        const uint32_t ws[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
        f16x8 qv;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qv[e] = (_Float16)__uint_as_float(e & 1 ? ws[e >> 1] & 0xFFFF0000u : ws[e >> 1] << 16);
        stage[P * CSA2_WAVE + lane] = qv;   // (the native form keeps the query there)
    }
    // The row's SWA rows through a buffer (reads outside it return zeros);
    // main entries are read through 64-bit addresses (FragRaw::load_row),
    // so entry ids are bounded only by the row's length.
    const int nb = n < 0 ? 0 : n;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W > 0 ? swa + swa0 * D : swa, (PG && swa_head ? W : nsw) * D);   // empty when W == 0
    const int Kp = pad_topk(K);
    auto load_frag = [&](FragRaw<D>& f, int fr_, int j) {
        const int slot = fr_ * kFrag + col, i = slot - Kp;
        const bool vm = slot < K && j >= 0 && j < nb;
        CSA2_DCHECK(hg == 0 && slot < K && j != -1 && !vm);
        const bool vs = i >= 0 && i < nsw;
        const int iw = PG ? (head + i >= W ? head + i - W : head + i) : i;
        if (frag_kind(fr_, Kp) == 0)
            f.load_row(vm, j, grp, codes + base * (D / 2), scales + base * (D / 16));
        else
            f.load_swa(vs, iw, grp, rw);
    };
    FragRaw<D> cur, nxt;   // cur's scales are converted at the start of its round
    if (fw < f_end) load_frag(cur, fw, idx_c);

    // Native form: the query as E4M3 with one power-of-two scale per lane
    // block (B operand of s_frag_nat), and whether every value is exact in
    // it.  In the product an E2M1 value of A lane group g, nibble e meets the
    // E4M3 byte 16 (g >> 1) + (e & 15) of B lane group 2 (g & 1) + (e >> 4)
    // (measured on gfx950), so B lane (head, g), k-step T, holds the 16
    // channels from c0 = (g >> 1) D/4 + 32T + 16 (g & 1) in bytes 0 .. 15 and
    // the 16 from c0 + D/2 in bytes 16 .. 31.  Every wave converts the whole
    // query of its head group, so all waves agree.
    constexpr int NT = D / 128;
    i32x8 qn[NAT ? HT : 1][NAT ? NT : 1];
    uint32_t qe8[NAT ? HT : 1];
    bool nat_q = false;
    if constexpr (NAT) {
        typedef short s16x2 __attribute__((ext_vector_type(2)));
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + (int64_t)r * H * D, H * D * 2);
        bool exact = true;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            qe8[ht] = 0u;
#pragma unroll
            for (int T = 0; T < NT; ++T) {
                const int c0 = (grp >> 1) * (D / 4) + 32 * T + 16 * (grp & 1);
                const uint32_t off = (uint32_t)(h0 + ht * 16 + col) * (D * 2) + 2 * c0;
                uint32_t wq[16];
#pragma unroll
                for (int u = 0; u < 4; ++u) {   // 32 bytes at c0, then 32 at c0 + D/2
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, off + (u >> 1) * D + 16 * (u & 1), 0, 0);
                    wq[4 * u] = v[0]; wq[4 * u + 1] = v[1]; wq[4 * u + 2] = v[2]; wq[4 * u + 3] = v[3];
                }
                float x[32];
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    x[e] = __uint_as_float(e & 1 ? wq[e >> 1] & 0xFFFF0000u : wq[e >> 1] << 16);
                    m = fmaxf(m, fabsf(x[e]));
                }
                // scale 2^sx puts the block's largest magnitude in [128, 256)
                int sx = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 134 : 0;
                sx = sx < -127 ? -127 : sx;
                const float down = __uint_as_float((uint32_t)(127 - sx) << 23);   // 2^-sx, exact
                const float up = sx > -127 ? __uint_as_float((uint32_t)(127 + sx) << 23) : 0x1p-127f;
                i32x8 pk;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const s16x2 z = {0, 0};
                    const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, x[4 * k] * down, x[4 * k + 1] * down,
                                                                              1.0f, false);
                    const s16x2 both = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[4 * k + 2] * down,
                                                                                x[4 * k + 3] * down, 1.0f, true);
                    const uint32_t wv = __builtin_bit_cast(uint32_t, both);
                    pk[k] = (int)wv;
                    // exact iff each E4M3 value times 2^sx gives the bf16 value back
                    const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wv, 1.0f, false);
                    const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wv, 1.0f, true);
                    exact = exact && b0[0] * up == x[4 * k] && b0[1] * up == x[4 * k + 1] &&
                            b1[0] * up == x[4 * k + 2] && b1[1] * up == x[4 * k + 3];
                }
                qn[ht][T] = pk;
                qe8[ht] |= (uint32_t)(sx + 127) << (8 * T);
            }
        }
        nat_q = __ballot(!exact) == 0ull;
    }

    __syncthreads();   // the query is staged
    f16x8 qf[NAT ? 1 : HT][NAT ? 1 : KS];
    if constexpr (!NAT) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            u16x2 mx = {0, 0};
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                qf[ht][t] = stage[(ht * KS + t) * CSA2_WAVE + lane];
                const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ht][t]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w4[e] & 0x7FFF7FFFu));
            }
            uint32_t mb = mx[0] > mx[1] ? mx[0] : mx[1];
            mb = umax_xor32(umax_xor16(mb));   // over the head's lanes
            Cq[ht] = a_part_const((float)__builtin_bit_cast(_Float16, (uint16_t)mb));
        }
    }
    if constexpr (!NAT && NW == kWaves) {
        // eight waves: the a-parts of the wave's pieces go to LDS once (the
        // exact-score path reads them there)
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int P = k * NW + wave;
            if (P >= NQP) continue;
            float C = Cq[0];
#pragma unroll
            for (int ht = 1; ht < HT; ++ht) C = P / KS == ht ? Cq[ht] : C;
            const f16x8 v = stage[P * CSA2_WAVE + lane];
            f16x8 av;
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = (_Float16)(((float)v[e] + C) - C);
            qa_s[P * CSA2_WAVE + lane] = av;
        }
    }
    // every wave holds the query and the a-parts are in LDS: the V tiles' space is free
    if constexpr (!NAT) __syncthreads();

    // Softmax state (log2 domain), per head in the S^T layout (lane col =
    // head).  m_run, the reference maximum, is the same in every wave.  l_p:
    // sum of the probabilities as PV weights them (normalises the output);
    // l_e: sum of the unrounded probabilities (for lse).  Both are per-lane
    // partial sums over the keys of the fragments this wave scored.
    float m_run[HT], l_p[HT], l_e[HT];
    f32x4 o[HT][NDT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        m_run[ht] = -INFINITY;
        l_p[ht] = 0.0f;
        l_e[ht] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[ht][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }
    _Float16* const vrow = vtiles + wave * SM::kTile + col * VS;   // the lane's key row of the wave's tile
    const f16x8* const qa_lane = qa_s + lane;
    const auto qsrc = [&]() {
        if constexpr (NAT) return QueryLds<HT, D>{qa_lane, Cq};
        else if constexpr (NW == kWaves) return QueryRegs<HT, D>{qf, qa_lane};
        else return QueryRegsC<HT, D>{qf, Cq};
    }();
    // the lane's PV operand address in slot 0's tile, at the wave's first channel
    const _Float16* const vr0 = vtiles + (4 * grp + (col >> 2)) * VS + 4 * (col & 3) + wave * SM::CW;

    // Registers: this file is compiled with the matrix-core operands and
    // accumulators in ordinary VGPRs (-amdgpu-mfma-vgpr-form), so that the
    // query (64 registers at HT * D = 512), the output and the fragment bytes
    // share one budget of 256 per wave, two waves per SIMD.
    for (int f0 = f_begin; f0 < f_end; f0 += NW) {
        const int fr = f0 + wave;
        const bool has = fr < f_end;                               // uniform in the wave
        const int nslot = f_end - f0 < NW ? f_end - f0 : NW;   // uniform in the workgroup
        // ---- the wave's fragment: scores, V tile, per-head maximum.
        // Large values (|v| > 8) make the output sensitive to logit rounding:
        // a logit error e moves the output by about e * |v - out|.  Such a
        // fragment gets exact scores and two-part probabilities.
        f32x4 sh[HT], sl[HT];
        float x[HT][4];
        bool precise = false;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            sh[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            sl[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < 4; ++i) x[ht][i] = -INFINITY;
        }
        if (has) {
            const int kind = frag_kind(fr, Kp);
            precise = __ballot(kind == 0 ? cur.template big<0>() : cur.template big<1>()) != 0ull;
            // native products first: they read the code words as loaded
            bool nat = false;
            if constexpr (NAT) {
                if (kind == 0 && nat_q) {
                    uint32_t ke8;
                    const bool ok = nat_key_scales<D>(cur, ke8);
                    nat = __ballot(!ok) == 0ull;
                    if (nat) {
                        s_frag_nat<HT, D>(cur, ke8, qn, qe8, sh);
                        if (nat_count && lane == 0) atomicAdd(nat_count, 1);
                    }
                }
            }
            if (kind == 0) cur.template scales_f16<0>();
            const uint64_t vb = __ballot(cur.valid);   // bit k: key k of the fragment (lanes 0..15)
            // prefetch: raw bytes of the wave's next fragment, Top-K entry of the one after
            {
                const int f1 = fr + NW;
                if (f1 < f_end) {
                    load_frag(nxt, f1, idx_n);
                    if (f1 + NW < f_end) load_idx(f1 + NW, idx_n);
                }
            }
            if (nat) v_frag<0, D>(cur, vrow, grp);
            else if (precise && kind == 0) s_frag_exact<0, HT, D>(cur, qsrc, vrow, grp, sh, sl);
            else if (precise) s_frag_exact<1, HT, D>(cur, qsrc, vrow, grp, sh, sl);
            else if (kind == 0) s_frag<0, HT, D>(cur, qsrc, vrow, grp, sh);
            else s_frag<1, HT, D>(cur, qsrc, vrow, grp, sh);
            // S^T lane layout: head h0 + 16 ht + col, keys 4 grp + i.
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if ((vb >> (4 * grp + i)) & 1ull) x[ht][i] = (sh[ht][i] + sl[ht][i]) * scale_log2e;
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float mx = fmaxf(fmaxf(x[ht][0], x[ht][1]), fmaxf(x[ht][2], x[ht][3]));
            mx = max_xor32(max_xor16(mx));
            if (grp == 0) reinterpret_cast<float*>(fmx[ht * 16 + col])[wave] = mx;
        }
        if (lane == 0) fprec[wave] = precise ? 1u << wave : 0u;
        __syncthreads();   // the round's V tiles, maxima and flags
        // The round's precise slots as one mask, their flags read together
        // (a read per slot ahead of its branch would chain the LDS latencies).
        uint32_t pmask = 0u;
#pragma unroll
        for (int w4 = 0; w4 < NW / 4; ++w4) {
            const uint4 f = reinterpret_cast<const uint4*>(fprec)[w4];
            pmask |= f.x | f.y | f.z | f.w;
        }
        pmask = __builtin_amdgcn_readfirstlane(pmask) & ((1u << nslot) - 1u);

        // ---- reference maximum of each head (the same in every wave): raised
        // to the round's maximum when that exceeds it by more than kLazy (a
        // head without any key so far has l = 0 and o = 0: nothing to
        // rescale).  Then the wave's own probabilities.
        // Probabilities enter PV as fp16, whose rounding (relative 2^-12)
        // moves the output by up to 2^-12 * |v - out|; in a precise fragment
        // they are split into fp16 hi + lo parts and PV runs twice (rounding
        // ~2^-23).
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float rm = -INFINITY;
#pragma unroll
            for (int w4 = 0; w4 < NW / 4; ++w4) {
                const float4 v = fmx[ht * 16 + col][w4];
                rm = fmaxf(rm, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
            }
            const bool raise = rm > m_run[ht] + kLazy;
            if (__ballot(raise) != 0ull) {
                const float al = (raise && m_run[ht] != -INFINITY) ? __builtin_amdgcn_exp2f(m_run[ht] - rm) : 1.0f;
                l_p[ht] *= al;
                l_e[ht] *= al;
                if (raise) m_run[ht] = rm;
                // O lane layout: channel 16 dt + col, heads 4 grp + i; the
                // factor of head 4 grp + i sits in lane 4 grp + i.
                float ai[4];
                bool rescale = false;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ai[i] = __shfl(al, 4 * grp + i, CSA2_WAVE);
                    rescale |= ai[i] != 1.0f;
                }
                if (__ballot(rescale) != 0ull) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[ht][dt][i] *= ai[i];
                }
            }
            if (has) {
                const float mn = m_run[ht];
                float ps = 0.0f, pe = 0.0f;
                f16x4 pa, pl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // the exponent's argument is formed with one rounding at its own
                    // (small) magnitude; the reference itself only has to be consistent
                    const float d = fmaf(sh[ht][i], scale_log2e, -mn) + sl[ht][i] * scale_log2e;
                    const float pf = x[ht][i] != -INFINITY ? __builtin_amdgcn_exp2f(d) : 0.0f;
                    const _Float16 ph = (_Float16)pf;
                    pa[i] = ph;
                    pl[i] = (_Float16)(pf - (float)ph);
                    ps += precise ? pf : (float)ph;   // normalise by what PV actually weights
                    pe += pf;
                }
                l_p[ht] += ps;
                l_e[ht] += pe;
                p_s[((wave * 2 + 0) * HT + ht) * CSA2_WAVE + lane] = pa;
                if (precise) p_s[((wave * 2 + 1) * HT + ht) * CSA2_WAVE + lane] = pl;
            }
        }
        __syncthreads();   // the round's probabilities

        // ---- PV: the probabilities of every slot into the wave's channels
        // (then the low parts of precise slots).
        // (four waves hold twice the output channels each: two slots' operands at a time)
        constexpr int PVG = NW == kWaves ? kPvGroup : (HT * D >= 512 ? 1 : 2);
        for (int j0 = 0; j0 < nslot; j0 += PVG) {
            if (j0 + PVG <= nslot)
                pv_slots<PVG, HT, NDT>(p_s + (j0 * 2 * HT) * CSA2_WAVE + lane, 2 * HT * CSA2_WAVE,
                                            vr0 + j0 * SM::kTile, SM::kTile, o);
            else
                for (int j = j0; j < nslot; ++j)
                    pv_slots<1, HT, NDT>(p_s + (j * 2 * HT) * CSA2_WAVE + lane, 0, vr0 + j * SM::kTile, 0, o);
        }
        for (uint32_t m = pmask; m != 0u; m &= m - 1u) {
            const int j = __builtin_ctz(m);
            pv_slots<1, HT, NDT>(p_s + ((j * 2 + 1) * HT) * CSA2_WAVE + lane, 0, vr0 + j * SM::kTile, 0, o);
        }
        cur = nxt;
        __syncthreads();   // the round's tiles and probabilities are consumed
    }

    // ---- the end: per-head sums over the waves; each wave writes its
    // channels (normalised when the row is not split, else as this split's
    // partial output with its statistics).
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float lt = sum_xor32(sum_xor16(l_p[ht])), le = sum_xor32(sum_xor16(l_e[ht]));
        if (grp == 0) {
            wsum[0][wave][ht * 16 + col] = lt;
            wsum[1][wave][ht * 16 + col] = le;
        }
    }
    __syncthreads();
    float Lh[HT], Leh[HT], Mh[HT];   // per head (S^T layout): the workgroup's statistics
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        Lh[ht] = 0.0f;
        Leh[ht] = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            Lh[ht] += wsum[0][w][ht * 16 + col];
            Leh[ht] += wsum[1][w][ht * 16 + col];
        }
        Mh[ht] = m_run[ht];
    }
    if (S == 2) {
        // Two splits: the first of the pair to get here publishes its partial
        // (device-coherent stores, in this register layout) and leaves; the
        // second merges it into its own registers and writes the output.  The
        // arrival word of the (row, head group) counts arrivals (+1) and the
        // published partial (+4); the second resets it to zero.  The second
        // waits only for a workgroup that has arrived and waits for nothing,
        // so the wait ends (it is bounded all the same).
        __shared__ int second;
        int32_t* const sync = pair_sync + (r * HG + hg);
        CSA2_DCHECK(threadIdx.x == 0 && r * HG + hg >= kPairWords);
        constexpr int NE = HT * NDT * 4;   // output values per lane
        float* const po = part_o + ((int64_t)r * HG + hg) * (NW * CSA2_WAVE * NE) + wave * CSA2_WAVE + lane;
        float* const pml = part_ml + ((int64_t)r * HG + hg) * (NH * 4);
        int prev = 0;   // thread 0: the word before this workgroup's arrival
        if (threadIdx.x == 0) {
            prev = __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            second = prev == 0 ? 0 : 1;
        }
        __syncthreads();
        if (!second) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        store_coherent(po + ((ht * NDT + dt) * 4 + i) * (NW * CSA2_WAVE), o[ht][dt][i]);
                if (wave == 0 && grp == 0) {
                    float* const ml = pml + (ht * 16 + col) * 4;
                    store_coherent(ml + 0, Mh[ht]);
                    store_coherent(ml + 1, Lh[ht]);
                    store_coherent(ml + 2, Leh[ht]);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial is complete
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_fetch_add(sync, 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (threadIdx.x == 0) {
            // The first publishes about a microsecond after it arrives (its
            // device-coherent stores complete first).  Device-coherent loads
            // of the word slow each other down, so the second waits about
            // that long (2,560 cycles) before its first look and then looks
            // at short intervals; nothing to wait for if the first had
            // already published when this one arrived.
            if ((prev & 4) == 0) {
                __builtin_amdgcn_s_sleep(40);
                int n = 0;
                while ((__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 4) == 0 &&
                       n < kSpinLimit) {
                    __builtin_amdgcn_s_sleep(4);
                    ++n;
                }
                CSA2_DCHECK(n >= kSpinLimit);
            }
            __hip_atomic_store(sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        // merge: o = (o_a 2^(m_a - M) + o_b 2^(m_b - M)) / L, per head; each
        // product is rounded on its own (no contraction into an fma) and the
        // sum commutes, so the result does not depend on which split arrived
        // first.  The partial's statistics and values are requested together
        // (one round trip).
        float mlb[HT][3], obv[HT][NDT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const float* const ml = pml + (ht * 16 + col) * 4;
#pragma unroll
            for (int k = 0; k < 3; ++k) mlb[ht][k] = __hip_atomic_load(ml + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    obv[ht][dt][i] = __hip_atomic_load(po + ((ht * NDT + dt) * 4 + i) * (NW * CSA2_WAVE),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
#pragma clang fp contract(off)
            const float Mb = mlb[ht][0], Lb = mlb[ht][1], Leb = mlb[ht][2];
            float M = -INFINITY;
            if (Lh[ht] > 0.0f) M = Mh[ht];
            if (Lb > 0.0f) M = fmaxf(M, Mb);
            const float wa = Lh[ht] > 0.0f ? exp2f(Mh[ht] - M) : 0.0f;
            const float wb = Lb > 0.0f ? exp2f(Mb - M) : 0.0f;
            Lh[ht] = Lh[ht] * wa + Lb * wb;
            Leh[ht] = Leh[ht] * wa + Leb * wb;
            Mh[ht] = M;
            float wai[4], wbi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wai[i] = __shfl(wa, 4 * grp + i, CSA2_WAVE);
                wbi[i] = __shfl(wb, 4 * grp + i, CSA2_WAVE);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[ht][dt][i] = o[ht][dt][i] * wai[i] + obv[ht][dt][i] * wbi[i];
        }
    }
    const bool whole = S <= 2;   // this workgroup writes the normalised output
    float inv_o[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int hh = ht * 16 + col;
        const float L = Lh[ht], Le = Leh[ht], M = Mh[ht];
        const int h = h0 + hh;
        if (wave == 0 && grp == 0 && h < H) {
            if (whole) {
                if (lse) lse[(int64_t)r * H + h] = L > 0.0f ? M * kLn2 + logf(Le) : -INFINITY;
            } else {
                *reinterpret_cast<float4*>(part_ml + (((int64_t)r * S + s) * H + h) * 4) = make_float4(M, L, Le, 0.0f);
            }
        }
        const float inv = whole ? (L > 0.0f ? 1.0f / L : 0.0f) : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) inv_o[ht][i] = __shfl(inv, 4 * grp + i, CSA2_WAVE);
    }
    float* const dst = (whole ? out + ((int64_t)r * H + h0) * D : part_o + (((int64_t)r * S + s) * H + h0) * D) +
                       wave * SM::CW;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hh = ht * 16 + 4 * grp + i;
                if (h0 + hh < H) dst[(int64_t)hh * D + 16 * dt + col] = o[ht][dt][i] * inv_o[ht][i];
            }
}

// Merge of split partials: o = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// lse from the unrounded sums.  Partial statistics per (row, split, head):
// (m, l, l_exact, 0).  One workgroup per (row, head), placed on the row's XCD;
// each thread owns four consecutive channels and requests the statistics and
// its channels of every split at once, so the merge waits for one round trip.
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int32_t R, int32_t H,
                                                      int32_t D, int32_t S, float* __restrict__ out,
                                                      float* __restrict__ lse)
{
    int r;
    const int h = xcd_slot(blockIdx.x, H, r);
    if (r >= R) return;
    const int64_t rh = (int64_t)r * H + h;
    const int d = 4 * threadIdx.x;   // D <= 4 * blockDim.x
    const bool has_d = d < D;
    float4 st[kMaxPlanSplits], v[kMaxPlanSplits];
#pragma unroll
    for (int k = 0; k < kMaxPlanSplits; ++k) {
        st[k] = k < S ? *reinterpret_cast<const float4*>(part_ml + (((int64_t)r * S + k) * H + h) * 4)
                      : make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
        v[k] = k < S && has_d ? *reinterpret_cast<const float4*>(part_o + (((int64_t)r * S + k) * H + h) * D + d)
                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxPlanSplits; ++k)
        if (st[k].y > 0.0f) M = fmaxf(M, st[k].x);
    float L = 0.0f, Le = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int k = 0; k < kMaxPlanSplits; ++k) {
        const float w = st[k].y > 0.0f ? exp2f(st[k].x - M) : 0.0f;
        L += st[k].y * w;
        Le += st[k].z * w;
        acc.x += w * v[k].x; acc.y += w * v[k].y; acc.z += w * v[k].z; acc.w += w * v[k].w;
    }
    if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? M * kLn2 + logf(Le) : -INFINITY;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (has_d)
        *reinterpret_cast<float4*>(out + rh * D + d) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

struct AttnPlan {
    int HT, HG, S, nfrag, NW;
};

// Workgroup shape: heads per workgroup (16 HT) and key splits S per row.  A
// workgroup dequantises and stages each of its keys once and computes full
// scores, whatever its head count, so:
//   * the head count per group is as large as the registers allow (each wave
//     holds all D query channels of every head: HT <= 512 / D) while the rows
//     alone give about one workgroup per compute unit;
//   * otherwise HT = 1 and a row's keys are split over up to kMaxPlanSplits
//     workgroups, keeping at least one fragment per wave (each split adds a
//     partial output to the merge);
//   * with at least eight workgroups per compute unit (prefill chunks), they
//     take four waves each (half the LDS), so two run on each compute unit at
//     once.  (Four waves form the exact-score a-parts from the query
//     registers, which costs VALU work on large-valued keys: with fewer rows,
//     e.g. a 256-row ragged batch of heavy-tailed values, eight waves are
//     faster.)
AttnPlan plan_attn(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W)
{
    constexpr int64_t kTargetGroups = 256;
    AttnPlan p;
    p.nfrag = (pad_topk(K) + W + kFrag - 1) / kFrag;
    if (p.nfrag < 1) p.nfrag = 1;
    const int heads16 = (H + 15) / 16;
    int ht = 512 / D < heads16 ? 512 / D : heads16;
    if (ht == 3) ht = 2;
    p.HT = ht;
    p.HG = (H + 16 * ht - 1) / (16 * ht);
    if ((int64_t)R * p.HG < kTargetGroups) {
        p.HT = 1;
        p.HG = heads16;
    }
    const int64_t smax = p.nfrag / kWaves > 1 ? p.nfrag / kWaves : 1;
    const int64_t base = (int64_t)R * p.HG;
    // no more workgroups than compute units: each holds a whole one (LDS)
    int64_t S = base >= kTargetGroups ? 1 : kTargetGroups / base;
    if (S > kMaxPlanSplits) S = kMaxPlanSplits;
    if (S > smax) S = smax;
    p.S = (int)S;
    p.NW = base >= 8 * kTargetGroups ? kWavesMany : kWaves;
    return p;
}

template <int HT, int D, bool PG, bool NAT, int NW>
void launch_attn(dim3 grid, hipStream_t st, const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                 const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len, const int32_t* topk,
                 int32_t K, const uint8_t* swa, const int64_t* swa_row_start, const int32_t* swa_len,
                 const int32_t* swa_head, int64_t phys_rows, int32_t H, int32_t R, int32_t W, float sl2e, int HG,
                 int S, int nfrag, float* out, float* lse, float* po, float* pml, int32_t* sync, int32_t* nat_count)
{
    hipLaunchKernelGGL((k_sparse_attn<HT, D, PG, NAT, NW>), grid, dim3(CSA2_WAVE * NW), 0, st, q, codes, scales,
                       seq_start, row_seq, row_len, topk, K, swa, swa_row_start, swa_len, swa_head, phys_rows, R, H, W,
                       sl2e, HG, S, nfrag, out, lse, po, pml, sync, nat_count);
}

// Cache rows of the entries of index lists over a paged cache: entry j of the
// row's sequence is in row bt[s * max_pages + j / page] * page + j % page;
// -1 for absent entries, entries outside [0, row_len) and pages outside the
// cache.
__global__ __launch_bounds__(256) void k_paged_rows(const int32_t* __restrict__ bt, int32_t max_pages, int32_t shift,
                                                    int64_t cache_rows, const int32_t* __restrict__ row_seq,
                                                    const int32_t* __restrict__ row_len,
                                                    const int32_t* __restrict__ idx, int32_t R, int32_t K,
                                                    int32_t* __restrict__ phys)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)R * K) return;
    const int r = (int)(e / K);
    const int j = idx[e];
    int32_t out = -1;
    CSA2_DCHECK(j != -1 && !(j >= 0 && j < row_len[r]));
    if (j >= 0 && j < row_len[r]) {
        const int page = j >> shift;
        if (page < max_pages) {
            const int64_t pid = bt[(int64_t)row_seq[r] * max_pages + page];
            const int64_t row = (pid << shift) | (j & ((1 << shift) - 1));
            if (pid >= 0 && row < cache_rows && row <= 0x7FFFFFFF) out = (int32_t)row;
        }
    }
    phys[e] = out;
}

csa2_status_t sparse_attn_impl(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                               const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                               int64_t phys_rows, const int32_t* topk_idx, int32_t K, const uint8_t* swa,
                               const int64_t* swa_row_start, const int32_t* swa_len, const int32_t* swa_head,
                               int32_t R, int32_t H, int32_t D, int32_t W, float softmax_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream, bool nat = false,
                               int32_t* nat_count = nullptr);

}  // namespace

extern "C" size_t csa2_sparse_attn_workspace_bytes(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W)
{
    // arguments the call rejects need no workspace
    if (R <= 0 || H <= 0 || H > 65536 || (D != 128 && D != 256 && D != 512) || K < 0 || K > 4096 || W < 0 ||
        W > 4096)
        return 0;
    const AttnPlan p = plan_attn(R, H, D, K, W);
    if (p.S <= 1) return 0;
    // the pair-merge arrival words, then the partial outputs and statistics
    const size_t head = (size_t)kPairWords * 4;
    if (p.S == 2) {
        const size_t nh = (size_t)16 * p.HT;
        return head + csa2::align_up((size_t)R * p.HG * nh * D * 4, 256) + csa2::align_up((size_t)R * p.HG * nh * 16, 256);
    }
    return head + csa2::align_up((size_t)R * p.S * H * D * 4, 256) + csa2::align_up((size_t)R * p.S * H * 4 * 4, 256);
}

namespace {
csa2_status_t sparse_attn_impl(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                               const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                               int64_t phys_rows, const int32_t* topk_idx, int32_t K, const uint8_t* swa,
                               const int64_t* swa_row_start, const int32_t* swa_len, const int32_t* swa_head,
                               int32_t R, int32_t H, int32_t D, int32_t W, float softmax_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream, bool nat,
                               int32_t* nat_count)
{
    CSA2_REQUIRE(R >= 0, CSA2_ERR_SHAPE, "sparse_attn: R=%d < 0", R);
    CSA2_REQUIRE(H >= 1, CSA2_ERR_SHAPE, "sparse_attn: H=%d < 1", H);
    CSA2_REQUIRE(H <= 65536, CSA2_ERR_UNSUPPORTED, "sparse_attn: H=%d > 65536", H);
    CSA2_REQUIRE(D >= 16 && D % 16 == 0, CSA2_ERR_SHAPE, "sparse_attn: D=%d must be a positive multiple of 16", D);
    CSA2_REQUIRE(D == 128 || D == 256 || D == 512, CSA2_ERR_UNSUPPORTED,
                 "sparse_attn: D=%d (supported: 128, 256, 512)", D);
    CSA2_REQUIRE(K >= 0 && W >= 0, CSA2_ERR_SHAPE, "sparse_attn: K=%d, W=%d must be >= 0", K, W);
    CSA2_REQUIRE(K <= 4096 && W <= 4096, CSA2_ERR_UNSUPPORTED, "sparse_attn: K=%d or W=%d > 4096", K, W);
    if (R == 0) return CSA2_OK;
    CSA2_REQUIRE(q && codes && scales && out && (phys_rows > 0 || (seq_start && row_seq && row_len)), CSA2_ERR_NULL,
                 "sparse_attn: NULL pointer argument");
    CSA2_REQUIRE(K == 0 || topk_idx, CSA2_ERR_NULL, "sparse_attn: topk_idx is NULL with K > 0");
    CSA2_REQUIRE(W == 0 || (swa && swa_row_start && swa_len), CSA2_ERR_NULL,
                 "sparse_attn: SWA pointers are NULL with W > 0");
    CSA2_REQUIRE((((uintptr_t)q | (uintptr_t)codes | (uintptr_t)scales | (uintptr_t)(W > 0 ? swa : nullptr)) & 15) == 0,
                 CSA2_ERR_UNSUPPORTED, "sparse_attn: q, codes, scales and swa must be 16-byte aligned");
    const AttnPlan p = plan_attn(R, H, D, K, W);
    CSA2_REQUIRE(xcd_grid(R, (int64_t)p.HG * p.S) <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED,
                 "sparse_attn: grid too large");
    CSA2_REQUIRE(xcd_grid(R, H) <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED, "sparse_attn: grid too large");
    const size_t need = csa2_sparse_attn_workspace_bytes(R, H, D, K, W);
    CSA2_REQUIRE(need == 0 || (workspace && workspace_bytes >= need && ((uintptr_t)workspace & 255) == 0),
                 CSA2_ERR_WORKSPACE, "sparse_attn: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                 workspace_bytes);
    float* po = nullptr;
    float* pml = nullptr;
    int32_t* sync = nullptr;
    if (p.S > 1) {
        char* w8 = static_cast<char*>(workspace);
        sync = reinterpret_cast<int32_t*>(w8);
        w8 += (size_t)kPairWords * 4;
        po = reinterpret_cast<float*>(w8);
        const size_t po_bytes = p.S == 2 ? (size_t)R * p.HG * 16 * p.HT * D * 4 : (size_t)R * p.S * H * D * 4;
        pml = reinterpret_cast<float*>(w8 + csa2::align_up(po_bytes, 256));
    }
    // With W == 0 or K == 0 the kernels never dereference the unused pointers.
    hipStream_t st = csa2::as_stream(stream);
    const float sl2e = softmax_scale * 1.44269504088896340736f;
    const dim3 grid((unsigned)xcd_grid(R, p.HG * p.S));
#define CSA2_ATTN(ht, d)                                                                                    \
    if (p.HT == ht && D == d)                                                                               \
        (nat                      ? launch_attn<ht, d, false, true, kWaves>                                 \
         : p.NW == kWavesMany     ? (phys_rows > 0 ? launch_attn<ht, d, true, false, kWavesMany>            \
                                                   : launch_attn<ht, d, false, false, kWavesMany>)          \
         : phys_rows > 0 ? launch_attn<ht, d, true, false, kWaves> : launch_attn<ht, d, false, false, kWaves>)( \
            grid, st, q, codes, scales, seq_start, row_seq, row_len, topk_idx, K, swa, swa_row_start, swa_len, \
            swa_head, phys_rows, H, R, W, sl2e, p.HG, p.S, p.nfrag, out, lse, po, pml, sync, nat_count);
    CSA2_ATTN(1, 128) CSA2_ATTN(2, 128) CSA2_ATTN(4, 128)
    CSA2_ATTN(1, 256) CSA2_ATTN(2, 256)
    CSA2_ATTN(1, 512)
#undef CSA2_ATTN
    if (p.S > 2)
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)xcd_grid(R, H)), dim3(128), 0, st, po, pml, R, H, D, p.S,
                           out, lse);
    return CSA2_FINISH(st, "sparse_attn");
}
}  // namespace

extern "C" csa2_status_t csa2_sparse_attn(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                          const int64_t* seq_start, const int32_t* row_seq,
                                          const int32_t* row_len, const int32_t* topk_idx, int32_t K,
                                          const uint8_t* swa, const int64_t* swa_row_start,
                                          const int32_t* swa_len, int32_t R, int32_t H, int32_t D, int32_t W,
                                          float softmax_scale, float* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream)
{
    return sparse_attn_impl(q, codes, scales, seq_start, row_seq, row_len, 0, topk_idx, K, swa, swa_row_start, swa_len,
                            nullptr, R, H, D, W, softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

extern "C" csa2_status_t csa2_sparse_attn_fp4mma(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                                const int64_t* seq_start, const int32_t* row_seq,
                                                const int32_t* row_len, const int32_t* topk_idx, int32_t K,
                                                const uint8_t* swa, const int64_t* swa_row_start,
                                                const int32_t* swa_len, int32_t R, int32_t H, int32_t D, int32_t W,
                                                float softmax_scale, float* out, float* lse, int32_t* native_fragments,
                                                void* workspace, size_t workspace_bytes, void* stream)
{
    return sparse_attn_impl(q, codes, scales, seq_start, row_seq, row_len, 0, topk_idx, K, swa, swa_row_start, swa_len,
                            nullptr, R, H, D, W, softmax_scale, out, lse, workspace, workspace_bytes, stream, true,
                            native_fragments);
}

extern "C" csa2_status_t csa2_sparse_attn_phys(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                                               int64_t cache_rows, const int32_t* phys_idx, int32_t K,
                                               const uint8_t* swa, const int64_t* swa_row_start,
                                               const int32_t* swa_len, const int32_t* swa_head, int32_t R, int32_t H,
                                               int32_t D, int32_t W, float softmax_scale, float* out, float* lse,
                                               void* workspace, size_t workspace_bytes, void* stream)
{
    CSA2_REQUIRE(cache_rows >= 1, CSA2_ERR_SHAPE, "sparse_attn_phys: cache_rows=%lld < 1", (long long)cache_rows);
    return sparse_attn_impl(q, codes, scales, nullptr, nullptr, nullptr, cache_rows, phys_idx, K, swa, swa_row_start,
                            swa_len, swa_head, R, H, D, W, softmax_scale, out, lse, workspace, workspace_bytes,
                            stream);
}

extern "C" csa2_status_t csa2_paged_rows(const int32_t* block_table, int32_t max_pages, int32_t page_rows,
                                         int64_t cache_rows, const int32_t* row_seq, const int32_t* row_len,
                                         const int32_t* idx, int32_t R, int32_t K, int32_t* phys, void* stream)
{
    CSA2_REQUIRE(R >= 0 && K >= 0, CSA2_ERR_SHAPE, "paged_rows: R=%d, K=%d must be >= 0", R, K);
    CSA2_REQUIRE(max_pages >= 1, CSA2_ERR_SHAPE, "paged_rows: max_pages=%d < 1", max_pages);
    CSA2_REQUIRE(cache_rows >= 1, CSA2_ERR_SHAPE, "paged_rows: cache_rows=%lld < 1", (long long)cache_rows);
    CSA2_REQUIRE(page_rows >= 8 && page_rows <= (1 << 20) && (page_rows & (page_rows - 1)) == 0,
                 CSA2_ERR_UNSUPPORTED, "paged_rows: page_rows=%d must be a power of two in [8, 2^20]", page_rows);
    if ((int64_t)R * K == 0) return CSA2_OK;
    CSA2_REQUIRE(block_table && row_seq && row_len && idx && phys, CSA2_ERR_NULL, "paged_rows: NULL pointer argument");
    const int64_t total = (int64_t)R * K;
    CSA2_REQUIRE((total + 255) / 256 <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED, "paged_rows: too many entries");
    hipLaunchKernelGGL(k_paged_rows, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, csa2::as_stream(stream),
                       block_table, max_pages, __builtin_ctz((unsigned)page_rows), cache_rows, row_seq, row_len, idx, R,
                       K, phys);
    return CSA2_FINISH(csa2::as_stream(stream), "paged_rows");
}
