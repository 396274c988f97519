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
// heads x a contiguous range of 16-key fragments.  The waves take the range's
// fragments in turn and each runs a complete online softmax over its own
// fragments, so no wave waits for another before the final merge:
//   * S^T = K Q^T: lane (key col, grp) dequantises D/4 channels of key col
//     straight from the cache to fp16 in registers (E2M1 -> fp16 by the
//     hardware converter, times the E4M3 scale; the product is exact in fp16)
//     and feeds them as the A operand of v_mfma_f32_16x16x32_f16 against the
//     NH query heads (B operand, all D channels held in registers).  The
//     contraction order only has to agree between the two operands; it is
//     chosen so that in every MFMA lanes 0-31 carry the two halves of one
//     16-channel scale group and lanes 32-63 those of another (see below).
//   * The same fp16 values go to the wave's own LDS tile [16 keys][D] and come
//     back transposed (ds_read_b64_tr_b16) as the B operand of PV.
//   * The S^T accumulator (lane = head, 4 keys) is already the A operand
//     layout of v_mfma_f32_16x16x16_f16, so probabilities never leave the
//     registers.  Online softmax in the log2 domain with a lazily raised
//     reference max.
//   * At the end the four waves' (max, sums, O) are merged through LDS; wave w
//     writes output channels [w*D/4, (w+1)*D/4).  Rows whose fragments are
//     split across workgroups write unnormalised partial outputs plus (max,
//     sums); k_attn_combine merges them.
//
// Exact scores for keys with large values.  The matrix cores sum products
// with errors of a few units in the last place of the largest addend, and
// with |v| in the hundreds a near tie between two keys turns such a score
// error into an output error far above the tolerance.  Where a fragment's
// keys may hold |v| > 8 its scores are computed exactly instead: each query
// head is split as q = a + b, a being q rounded to a multiple of 2^(E-11) with
// 2^E > max|q| of the head (11 bits, exact in fp16), b the small remainder.
// Within one scale group every a*k product is then an integer multiple of one
// quantum and the 16 products sum to less than 2^24 quanta, so an MFMA
// restricted to one group (the other lane half masked to zero) returns the
// group sum exactly; the group sums are accumulated in fp64, and K b^T (small,
// nonzero only for channels with |q| < max|q|/16) is added from an ordinary
// MFMA chain.
#include "csa2_device.h"
#include "csa2_host.h"

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kFrag = 16;           // keys per fragment (one MFMA row block)
constexpr int kWaves = 4;           // waves per workgroup
constexpr float kLazy = 8.0f;       // log2-domain slack before a running max is raised
constexpr int kMaxPlanSplits = 8;   // key splits per row, at most

// Channel layout of a lane (col, grp), p = grp / 2, hf = grp % 2: k-step t
// (t < KS = D/32) covers the 8 channels
//   D/2*p + 16*t + 8*hf .. +8,
// i.e. half hf of scale group KS*p + t.  In each MFMA the lanes with p = 0
// thus hold one whole scale group and those with p = 1 another.
template <int D>
__device__ __forceinline__ int step_ch(int grp, int t)
{
    return (D / 2) * (grp >> 1) + 16 * t + 8 * (grp & 1);
}

// Local unit holding piece t after FragRaw::unpair(): pieces 0 .. KS/2-1 sit
// at even units, the rest at odd ones.
template <int D>
__device__ __forceinline__ constexpr int kperm(int t)
{
    constexpr int KS = D / 32;
    return t < KS / 2 ? 2 * t : 2 * t - KS + 1;
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
    static constexpr int NSC = KS / 4;
    uint32_t raw[2 * KS];
    uint32_t sc[NSC];
    f16x2 sp[KS / 2];   // scales of pieces 2u, 2u+1 as fp16 (set by unpair())
    bool valid, is_main;

    // SWA row i of the lane's slot (vs: the slot holds one) through rw, the
    // buffer over the row's window.  The lane pair (p, 0), (p, 1) of a row
    // needs one contiguous block of D/2 bytes; each lane loads its half into
    // consecutive words and unpair() exchanges the halves.  An absent row
    // gets the offset kNoKey and reads as zeros; the loads are unconditional.
    __device__ __forceinline__ void load_swa(bool vs, int i, int p, int hf, __amdgpu_buffer_rsrc_t rw)
    {
        valid = vs;
        is_main = false;
        const uint32_t off1 = vs ? (uint32_t)i * D + (D / 2) * p + (D / 4) * hf : kNoKey;
#pragma unroll
        for (int u = 0; u < KS / 4; ++u) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off1 + 16 * u, 0, 0);
            raw[4 * u] = v[0]; raw[4 * u + 1] = v[1]; raw[4 * u + 2] = v[2]; raw[4 * u + 3] = v[3];
        }
#pragma unroll
        for (int u = 0; u < KS / 4; ++u) {   // second half of the lane's bytes
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, off1 + D / 8 + 16 * u, 0, 0);
            raw[KS + 4 * u] = v[0]; raw[KS + 4 * u + 1] = v[1]; raw[KS + 4 * u + 2] = v[2]; raw[KS + 4 * u + 3] = v[3];
        }
        // (the scale words are loaded too, as zeros from past the buffer's
        // end, so that on either kind of fragment every raw register is
        // written by a load: the loop then waits on loads in issue order)
        if constexpr (NSC == 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, kNoKey, 0, 0);
            sc[0] = v[0]; sc[1] = v[1]; sc[2] = v[2]; sc[3] = v[3];
        } else if constexpr (NSC == 2) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, kNoKey, 0, 0);
            sc[0] = v[0]; sc[1] = v[1];
        } else {
            sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, kNoKey, 0, 0);
        }
    }

    // The lane's bytes of main entry j (vm: the slot holds a visible entry)
    // from codes / scales, which start at the row's first entry (or at the
    // cache's first row in the cache-row form): its D/4-byte half-block of
    // codes (the lane pair exchanges halves in unpair()) and its KS scale
    // bytes, through 64-bit addresses, so entries anywhere in a cache of any
    // size are reachable; an absent slot loads nothing and keeps zeros.
    __device__ __forceinline__ void load_row(bool vm, int j, int p, int hf, const uint8_t* codes,
                                             const uint8_t* scales)
    {
        valid = vm;
        is_main = true;
#pragma unroll
        for (int k = 0; k < 2 * KS; ++k) raw[k] = 0u;
#pragma unroll
        for (int w = 0; w < NSC; ++w) sc[w] = 0u;
        if (vm) {
            const uint8_t* pc = codes + (uint64_t)(uint32_t)j * (D / 2) + (D / 4) * p + (D / 8) * hf;
#pragma unroll
            for (int u = 0; u < KS / 4; ++u) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(pc + 16 * u);
                raw[4 * u] = v[0]; raw[4 * u + 1] = v[1]; raw[4 * u + 2] = v[2]; raw[4 * u + 3] = v[3];
            }
            const uint8_t* ps = scales + (uint64_t)(uint32_t)j * (D / 16) + KS * p;
            if constexpr (NSC == 4) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(ps);
                sc[0] = v[0]; sc[1] = v[1]; sc[2] = v[2]; sc[3] = v[3];
            } else if constexpr (NSC == 2) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(ps);
                sc[0] = v[0]; sc[1] = v[1];
            } else {
                sc[0] = *reinterpret_cast<const uint32_t*>(ps);
            }
        }
    }

    // Unit u of a pair's block (a code word, or 8 FP8 bytes) is piece u/2 of
    // half u%2; after load() lane hf holds units KS*hf .. KS*hf + KS-1 in
    // consecutive words.  v_permlane16_swap(x, y) exchanges row 1 of x with
    // row 0 of y (rows are the 16-lane groups: rows 0/1 are the halves hf =
    // 0/1 of p = 0, rows 2/3 those of p = 1).  Swapping local units 2v and
    // 2v+1 leaves the lane's own half of piece t in local unit kperm(t): code
    // word kperm(t), or FP8 words 2 kperm(t) and 2 kperm(t) + 1.  KIND: 0
    // Top-K slots only, 1 SWA rows only, 2 either (chosen per lane).
    template <int KIND>
    __device__ __forceinline__ void unpair()
    {
        // The scales are converted here, before the next fragment's loads are
        // issued, so that nothing after those loads reads the raw scale words.
        if (KIND != 1) {
#pragma unroll
            for (int u = 0; u < KS / 2; ++u)
                sp[u] = (u & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[u >> 1], 1.0f, true)
                                : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc[u >> 1], 1.0f, false);
        }
        uint32_t c[KS], w[2 * KS];
#pragma unroll
        for (int v = 0; v < KS / 2; ++v) {
            if (KIND != 1) {
                const auto r = __builtin_amdgcn_permlane16_swap(raw[2 * v], raw[2 * v + 1], false, false);
                c[2 * v] = r[0];
                c[2 * v + 1] = r[1];
            }
            if (KIND != 0) {
                const auto ra = __builtin_amdgcn_permlane16_swap(raw[4 * v], raw[4 * v + 2], false, false);
                const auto rb = __builtin_amdgcn_permlane16_swap(raw[4 * v + 1], raw[4 * v + 3], false, false);
                w[4 * v] = ra[0];
                w[4 * v + 2] = ra[1];
                w[4 * v + 1] = rb[0];
                w[4 * v + 3] = rb[1];
            }
        }
        if (KIND == 0) {
#pragma unroll
            for (int k = 0; k < KS; ++k) raw[k] = c[k];
        } else if (KIND == 1) {
#pragma unroll
            for (int k = 0; k < 2 * KS; ++k) raw[k] = w[k];
        } else {
#pragma unroll
            for (int k = 0; k < 2 * KS; ++k) raw[k] = is_main ? (k < KS ? c[k] : 0u) : w[k];
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
        uint32_t bm = 0u, bs = 0u;   // both reductions in full, then one select
        if (KIND != 1) {
#pragma unroll
            for (int w = 0; w < NSC; ++w) bm |= ((sc[w] & 0x7F7F7F7Fu) + 0x45454545u) & 0x80808080u;
        }
        if (KIND != 0) {
#pragma unroll
            for (int w = 0; w < 2 * KS; ++w) bs |= ((raw[w] & 0x7F7F7F7Fu) + 0x30303030u) & 0x80808080u;
        }
        const uint32_t bits = KIND == 0 ? bm : (KIND == 1 ? bs : (is_main ? bm : bs));
        return valid && bits != 0u;
    }
};

// Dequantise k-step t (8 channels) of the lane's key to fp16.
//   MODE 0: FP4 codes (word kperm(t)) times the group's E4M3 scale (scale
//           byte t of the lane's KS scale bytes);
//   MODE 1: FP8 E4M3 bytes (words 2 kperm(t), +1), unscaled;
//   MODE 2: either, chosen per lane.
template <int MODE, int D>
__device__ __forceinline__ f16x8 dequant_step(const FragRaw<D>& fr, int t)
{
    f16x8 a, b;
    if (MODE != 1) {
        const uint32_t c = fr.raw[kperm<D>(t)];
        const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
        const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
        const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
        const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
        const _Float16 s = fr.sp[t >> 1][t & 1];
        a = (f16x8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]} * s;
    }
    if (MODE != 0) {
        const uint32_t c0 = fr.raw[2 * kperm<D>(t)], c1 = fr.raw[2 * kperm<D>(t) + 1];
        const f16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false);
        const f16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true);
        const f16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false);
        const f16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true);
        b = (f16x8){b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
    }
    if (MODE == 0) return a;
    if (MODE == 1) return b;
    return fr.is_main ? a : b;
}

// The workgroup's output channels are part c of CS equal parts of D; its V
// tile holds only those.  k-step t of lane group grp falls in part
// (D/2 * p + 16 t) / (D/CS), p = grp / 2.
template <int D, int CS>
__device__ __forceinline__ bool in_part(int grp, int t, int c)
{
    return step_ch<D>(grp, t) / (D / CS) == c;
}

// Store k-step t of the lane's key to the V tile (vrow: the lane's key row of
// the tile, already offset by -c D/CS) if it belongs to the part.
template <int D, int CS>
__device__ __forceinline__ void v_store(_Float16* vrow, int grp, int t, int c, f16x8 kf)
{
    if (in_part<D, CS>(grp, t, c)) *reinterpret_cast<f16x8*>(vrow + step_ch<D>(grp, t)) = kf;
}

// S^T of one fragment, fp32 MFMA chain; the dequantised keys of the
// workgroup's channel part also go to the wave's V tile.
template <int MODE, int HT, int D, int CS>
__device__ __forceinline__ void s_frag(const FragRaw<D>& fr, const f16x8 (&qf)[HT][D / 32], _Float16* vrow, int grp,
                                       int c, f32x4 (&acc)[HT])
{
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
        const f16x8 kf = dequant_step<MODE, D>(fr, t);
        v_store<D, CS>(vrow, grp, t, c, kf);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ht][t], acc[ht], 0, 0, 0);
    }
}

// The same fragment with S computed exactly as (hi, lo) = K a^T + K b^T
// (split of q described at the top of the file).  qab: this lane's a- and
// b-part pieces in LDS, [2][HT * KS][64 lanes]; upper: lane >= 32.
template <int HT, int D, int CS>
__device__ __forceinline__ void s_frag_exact(const FragRaw<D>& fr, const f16x8* qab, bool upper, _Float16* vrow,
                                             int grp, int c, f32x4 (&acc)[HT], f32x4 (&lo)[HT])
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
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        const f16x8 kf = dequant_step<2, D>(fr, t);
        v_store<D, CS>(vrow, grp, t, c, kf);
        const f16x8 k_lo = upper ? zero : kf;     // scale group t (p = 0)
        const f16x8 k_hi = upper ? kf : zero;     // and scale group KS + t (p = 1)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const f16x8 a = qab[(ht * KS + t) * CSA2_WAVE];
            const f16x8 b = qab[((HT + ht) * KS + t) * CSA2_WAVE];
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

// O[heads x the part's channels] += P V for one fragment.  The B operand is read with
// ds_read_b64_tr_b16: within each 16-lane group, lane l receives element l%4
// of the 8-byte rows addressed by lanes 4i + l/4, so addressing row (key
// 4g + l/4, channels c0 + 4(l%4)) hands lane l the 4 keys 4g + 0..3 of channel
// c0 + l, the key order of the probability operand.
template <int HT, int NDT, int VS>
__device__ __forceinline__ void pv_frag(const f16x4 (&pa)[HT], const _Float16* vt, int col, int grp,
                                        f32x4 (&o)[HT][NDT])
{
    const _Float16* vr = vt + (4 * grp + (col >> 2)) * VS + 4 * (col & 3);
    constexpr int B = NDT < 16 ? NDT : 16;   // reads in flight
#pragma unroll
    for (int d0 = 0; d0 < NDT; d0 += B) {
        lds_f16x4 b[B];
#pragma unroll
        for (int k = 0; k < B; ++k)
            b[k] = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4 __attribute__((address_space(3)))*)(vr + 16 * (d0 + k)));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < B; ++k) {
            const f16x4 vb = {(_Float16)b[k][0], (_Float16)b[k][1], (_Float16)b[k][2], (_Float16)b[k][3]};
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                o[ht][d0 + k] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa[ht], vb, o[ht][d0 + k], 0, 0, 0);
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

// Slot layout of a row: the Top-K slots padded to Kp = a multiple of 16, then
// the SWA rows, so that a fragment holds one kind of slot only.
__host__ __device__ inline int pad_topk(int K) { return (K + kFrag - 1) / kFrag * kFrag; }
// Kind of a fragment (uniform): 0 Top-K slots, 1 SWA rows.
__device__ __forceinline__ int frag_kind(int fr, int Kp) { return fr * kFrag >= Kp ? 1 : 0; }

// LDS of one workgroup: the waves' V tiles and the query (fp16, and its a-
// and b-parts) during the key loop, then the merge buffers.
template <int HT, int D, int CS>
struct AttnSmem {
    static constexpr int KS = D / 32;
    static constexpr int DP = D / CS;              // channels of the workgroup's part
    static constexpr int NDT = DP / 16;            // output tiles per head tile
    static constexpr int VS = DP + 8;              // V row stride in halves (conflict-free rows and transposes)
    static constexpr int kVBytes = kWaves * kFrag * VS * 2;
    static constexpr int kQaBytes = 2 * HT * KS * CSA2_WAVE * 16;   // a and b parts
    static constexpr int kQfBytes = HT * KS * CSA2_WAVE * 16;       // the query as fp16
    static constexpr int kLoop = kVBytes + kQaBytes + kQfBytes;
    // Merge: rounds over RT output tiles at a time (a multiple of the wave
    // count); per round every wave stores its RT tiles per head tile,
    // [wave][HT][RT][64] f32x4.  One round when that fits in 128 KB.
    static constexpr int RT = HT * NDT <= 32 ? NDT : 32 / HT;
    static_assert(RT % kWaves == 0 && NDT % RT == 0, "merge rounds");
    static constexpr int kMerge = kWaves * HT * RT * CSA2_WAVE * 16;
    static constexpr int kBytes = kLoop > kMerge ? kLoop : kMerge;
};

// PG: the index lists hold cache rows (paged caches) and the SWA window may be
// a ring; the packed form is a separate instantiation so that it carries none
// of that addressing.
template <int HT, int D, int CS, bool PG>
__global__ __launch_bounds__(256, 1) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int64_t* __restrict__ seq_start, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_len, const int32_t* __restrict__ topk, int32_t K,
    const uint8_t* __restrict__ swa, const int64_t* __restrict__ swa_row_start,
    const int32_t* __restrict__ swa_len, const int32_t* __restrict__ swa_head, int64_t phys_rows, int32_t R,
    int32_t H, int32_t W, float scale_log2e, int32_t HG, int32_t S, int32_t nfrag, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml)
{
    using SM = AttnSmem<HT, D, CS>;
    constexpr int KS = SM::KS;
    constexpr int NDT = SM::NDT;
    constexpr int VS = SM::VS;
    constexpr int NH = HT * 16;

    __shared__ __attribute__((aligned(16))) char smem[SM::kBytes];
    __shared__ float wm[kWaves][NH];
    __shared__ float wl[kWaves][NH];
    __shared__ float wle[kWaves][NH];
    __shared__ uint32_t wqm[kWaves][NH];   // per wave: bf16 bits of the max |q| of each head over its pieces
    _Float16* const vt = reinterpret_cast<_Float16*>(smem) + (threadIdx.x >> 6) * (kFrag * VS);
    f16x8* const qa_s = reinterpret_cast<f16x8*>(smem + SM::kVBytes);   // [2][HT * KS][64]: a, b
    f16x8* const qf_s = reinterpret_cast<f16x8*>(smem + SM::kVBytes + SM::kQaBytes);   // [HT * KS][64]
    f32x4* const xo = reinterpret_cast<f32x4*>(smem);                    // merge buffers (after the loop)

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: branches on it are scalar
    const int col = lane & 15, grp = lane >> 4, hf = grp & 1;
    int r, hg, c, s;   // row, head group, channel part, key split
    {
        const int g = xcd_slot(blockIdx.x, HG * CS * S, r);
        hg = g % HG;
        c = g / HG % CS;
        s = g / (HG * CS);
    }
    if (r >= R) return;   // padding of the XCD mapping (whole workgroup, before any barrier)
    const int h0 = hg * NH;
    const bool upper = lane >= 32;
    const int f_begin = (int)((int64_t)nfrag * s / S), f_end = (int)((int64_t)nfrag * (s + 1) / S);
    const int32_t* topk_row = topk + (int64_t)r * K;

    // Loads are issued in dependency order so that waiting for one never waits
    // for a later chain: the row's metadata (scalar) and the wave's first two
    // fragments' Top-K entries, the wave's quarter of the query, then the
    // first fragment's key bytes, which arrive during the barriers that share
    // the query.
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
    auto load_idx = [&](int fr, int& idx) {
        const int slot = fr * kFrag + col;
        if (slot < K) idx = topk_row[slot];
    };
    int fr = f_begin + wave;
    int idx_c = 0, idx_n = 0;
    if (fr < f_end) load_idx(fr, idx_c);
    if (fr + kWaves < f_end) load_idx(fr + kWaves, idx_n);
    // The query is shared by the four waves: wave w loads and converts the
    // pieces (ht, t) with (ht * KS + t) % 4 == w, i.e. piece k < NP of the
    // wave is ht = k / (KS/4), t = 4k % KS + w; the pieces go to LDS and every
    // wave reads the whole query back after the barrier.  The query is read
    // through a buffer over its H heads: heads past H read as zeros.
    constexpr int NP = HT * KS / kWaves;
    static_assert(KS % kWaves == 0, "query pieces per wave");
    uint4 qraw[NP];
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + (int64_t)r * H * D, H * D * 2);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int ht = k / (KS / kWaves), t = (kWaves * k) % KS + wave;
            const uint32_t hoff = (uint32_t)(h0 + ht * 16 + col) * (D * 2);
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, hoff + 2 * step_ch<D>(grp, t), 0, 0);
            qraw[k] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
    nsw = nsw < 0 ? 0 : (nsw > W ? W : nsw);
    const int64_t base = PG ? 0 : seq_start[seq];
    // Max |q| of each head over the wave's pieces: an integer max of the bf16
    // magnitude bits (two per instruction), then over the lane groups.
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        u16x2 mx = {0, 0};
#pragma unroll
        for (int k = ht * (KS / kWaves); k < (ht + 1) * (KS / kWaves); ++k) {
            const uint32_t ws[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, ws[e] & 0x7FFF7FFFu));
        }
        uint32_t mb = mx[0] > mx[1] ? mx[0] : mx[1];
        mb = umax_xor32(umax_xor16(mb));
        if (grp == 0) wqm[wave][ht * 16 + col] = mb;
    }
    __syncthreads();
    // Query heads (B operand): lane (head col, grp) holds channels
    // step_ch(grp, t) .. +8 for k-step t.  bf16 -> fp16 is exact for |q| in
    // [2^-14, 65504].  a-part of a head: q rounded to a multiple of 2^(E-11),
    // 2^E > max|q| (E >= -13 keeps the quantum within fp16's subnormal grid).
    // Adding and subtracting 1.5 * 2^(E+12) rounds to that multiple in fp32.
    float Cq[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        uint32_t mb = 0u;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mb = max(mb, wqm[w][ht * 16 + col]);
        const float m = __uint_as_float(mb << 16);
        int E = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 126 : -13;
        E = E < -13 ? -13 : E;
        Cq[ht] = __uint_as_float((uint32_t)(E + 12 + 127) << 23 | 0x400000u);
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int ht = k / (KS / kWaves), t = (kWaves * k) % KS + wave;
        const uint32_t ws[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
        f16x8 qv, av, bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q32 = __uint_as_float(e & 1 ? ws[e >> 1] & 0xFFFF0000u : ws[e >> 1] << 16);
            const float a = (q32 + Cq[ht]) - Cq[ht];
            qv[e] = (_Float16)q32;
            av[e] = (_Float16)a;
            bv[e] = (_Float16)(q32 - a);   // exact: the low bits of q
        }
        qf_s[(ht * KS + t) * CSA2_WAVE + lane] = qv;
        qa_s[(ht * KS + t) * CSA2_WAVE + lane] = av;
        qa_s[((HT + ht) * KS + t) * CSA2_WAVE + lane] = bv;
    }
    const int p = grp >> 1;
    // The row's SWA rows through a buffer (reads outside it return zeros);
    // main entries are read through 64-bit addresses (FragRaw::load_row),
    // so entry ids are bounded only by the row's length.
    const int nb = n < 0 ? 0 : n;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W > 0 ? swa + swa0 * D : swa, (PG && swa_head ? W : nsw) * D);   // empty when W == 0
    const int Kp = pad_topk(K);
    auto load_frag = [&](FragRaw<D>& f, int fr_, int j) {
        const int slot = fr_ * kFrag + col, i = slot - Kp;
        const bool vm = slot < K && j >= 0 && j < nb;
        const bool vs = i >= 0 && i < nsw;
        const int iw = PG ? (head + i >= W ? head + i - W : head + i) : i;
        if (frag_kind(fr_, Kp) == 0)
            f.load_row(vm, j, p, hf, codes + base * (D / 2), scales + base * (D / 16));
        else
            f.load_swa(vs, iw, p, hf, rw);
    };
    FragRaw<D> cur, nxt;   // cur is unpaired in place at the start of its fragment
    if (fr < f_end) load_frag(cur, fr, idx_c);

    __syncthreads();
    f16x8 qf[HT][KS];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            qf[ht][t] = qf_s[(ht * KS + t) * CSA2_WAVE + lane];
            asm volatile("" : "+a"(qf[ht][t]));
        }

    // Online softmax state (log2 domain), per head in the S^T layout (lane
    // col = head).  The reference max of a head is raised only when a
    // fragment's max exceeds it by more than kLazy, so the accumulated output
    // is rarely rescaled; probabilities stay <= 2^kLazy.
    // l_p: sum of the probabilities as PV weights them (normalises the
    // output); l_e: sum of the unrounded probabilities (for lse).  Both are
    // per-lane partial sums over the lane's keys.
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
    _Float16* const vrow = vt + col * VS - c * SM::DP;   // indexed by the key's channel
    const f16x8* const qa_lane = qa_s + lane;

    // Register classes: the query pieces (MFMA B operands) and the output
    // accumulators stay in the matrix-core registers (AGPRs) for the whole
    // loop, leaving the VGPRs to the raw bytes and the dequantisation.  The
    // empty asm statements only name that class for the compiler.
    for (; fr < f_end; fr += kWaves) {
        // Large values (|v| > 8) make the output sensitive to logit rounding:
        // a logit error e moves the output by about e * |v - out|.  Such a
        // fragment gets exact scores and two-part probabilities.
        const int kind = frag_kind(fr, Kp);
        const bool precise = __ballot(kind == 0 ? cur.template big<0>() : cur.template big<1>()) != 0ull;
        if (kind == 0) cur.template unpair<0>();
        else cur.template unpair<1>();
        const uint64_t vb = __ballot(cur.valid);   // bit k: key k of the fragment (lanes 0..15)
        // prefetch: raw bytes of the wave's next fragment, Top-K entry of the one after
        {
            const int f1 = fr + kWaves;
            if (f1 < f_end) {
                load_frag(nxt, f1, idx_n);
                if (f1 + kWaves < f_end) load_idx(f1 + kWaves, idx_n);
            }
        }

        f32x4 sh[HT], sl[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            sh[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            sl[ht] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (precise) s_frag_exact<HT, D, CS>(cur, qa_lane, upper, vrow, grp, c, sh, sl);
        else if (kind == 0) s_frag<0, HT, D, CS>(cur, qf, vrow, grp, c, sh);
        else s_frag<1, HT, D, CS>(cur, qf, vrow, grp, c, sh);

        // S^T lane layout: head h0 + 16 ht + col, keys 4 grp + i.
        // Probabilities enter PV as fp16, whose rounding (relative 2^-12)
        // moves the output by up to 2^-12 * |v - out|; in a precise fragment
        // they are split into fp16 hi + lo parts and PV runs twice (rounding
        // ~2^-23).
        f16x4 pa[HT], pl[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            float x[4];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kv = (vb >> (4 * grp + i)) & 1ull;
                x[i] = kv ? (sh[ht][i] + sl[ht][i]) * scale_log2e : -INFINITY;
                mx = fmaxf(mx, x[i]);
            }
            mx = max_xor32(max_xor16(mx));
            // Raise the head's reference when the fragment's max exceeds it by
            // more than kLazy (a head without any key so far has l = 0 and
            // o = 0: nothing to rescale).
            const bool raise = mx > m_p[ht] + kLazy;
            if (__ballot(raise) != 0ull) {
                const float al = (raise && m_p[ht] != -INFINITY) ? __builtin_amdgcn_exp2f(m_p[ht] - mx) : 1.0f;
                l_p[ht] *= al;
                l_e[ht] *= al;
                if (raise) m_p[ht] = mx;
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
                    for (int dt = 0; dt < NDT; ++dt) {
                        asm volatile("" : "+a"(o[ht][dt]));   // copies out of the AGPRs happen only here
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[ht][dt][i] *= ai[i];
                        asm volatile("" : "+a"(o[ht][dt]));
                    }
                }
            }
            const float mn = m_p[ht];
            float ps = 0.0f, pe = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the exponent's argument is formed with one rounding at its own
                // (small) magnitude; the reference itself only has to be consistent
                const float d = fmaf(sh[ht][i], scale_log2e, -mn) + sl[ht][i] * scale_log2e;
                const float pf = x[i] != -INFINITY ? __builtin_amdgcn_exp2f(d) : 0.0f;
                const _Float16 ph = (_Float16)pf;
                pa[ht][i] = ph;
                pl[ht][i] = (_Float16)(pf - (float)ph);
                ps += precise ? pf : (float)ph;   // normalise by what PV actually weights
                pe += pf;
            }
            l_p[ht] += ps;
            l_e[ht] += pe;
        }
        pv_frag<HT, NDT, VS>(pa, vt, col, grp, o);
        if (precise) pv_frag<HT, NDT, VS>(pl, vt, col, grp, o);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) asm volatile("" : "+a"(o[ht][dt]));
#pragma unroll
            for (int t = 0; t < KS; ++t) asm volatile("" : "+a"(qf[ht][t]));
        }
        cur = nxt;
    }

    // ---- merge the four waves.  Per-head statistics first.
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const float lt = sum_xor32(sum_xor16(l_p[ht])), le = sum_xor32(sum_xor16(l_e[ht]));
        if (grp == 0) {
            wm[wave][ht * 16 + col] = m_p[ht];
            wl[wave][ht * 16 + col] = lt;
            wle[wave][ht * 16 + col] = le;
        }
    }
    __syncthreads();   // statistics visible; every wave is done with its V tile and qa
    // Per head (S^T layout, lane col = head): the merged max M, the sums and
    // this wave's weight 2^(m_w - M).  The O layout (lane (col, grp) holds
    // heads 4 grp + i) takes the weight and 1 / L of head 4 grp + i from lane
    // 4 grp + i.
    float own_o[HT][4], inv_o[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const int hh = ht * 16 + col;
        float m4[kWaves], l4[kWaves], e4[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            m4[w] = wm[w][hh];
            l4[w] = wl[w][hh];
            e4[w] = wle[w][hh];
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            if (l4[w] > 0.0f) M = fmaxf(M, m4[w]);
        float L = 0.0f, Le = 0.0f, own = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = l4[w] > 0.0f ? exp2f(m4[w] - M) : 0.0f;
            L += l4[w] * f;
            Le += e4[w] * f;
            own = w == wave ? f : own;
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int h = h0 + hh;
        if (wave == 0 && grp == 0 && c == 0 && h < H) {
            if (S == 1) {
                if (lse) lse[(int64_t)r * H + h] = L > 0.0f ? M * kLn2 + logf(Le) : -INFINITY;
            } else {
                *reinterpret_cast<float4*>(part_ml + (((int64_t)r * S + s) * H + h) * 4) = make_float4(M, L, Le, 0.0f);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            own_o[ht][i] = __shfl(own, 4 * grp + i, CSA2_WAVE);
            inv_o[ht][i] = S == 1 ? __shfl(inv, 4 * grp + i, CSA2_WAVE) : 1.0f;
        }
    }
    // Rounds over RT output tiles at a time: every wave stores its weighted
    // tiles of the round, then wave w sums the four waves' tiles
    // [w RT/4, (w+1) RT/4) of it and writes them out (normalised when the row
    // is not split, else as this split's partial output).
    constexpr int RT = SM::RT;
    constexpr int QW = RT / kWaves;
    float* const dst = (S == 1 ? out + ((int64_t)r * H + h0) * D : part_o + (((int64_t)r * S + s) * H + h0) * D) +
                       c * SM::DP;
#pragma unroll
    for (int rd = 0; rd < NDT / RT; ++rd) {
        if (rd > 0) __syncthreads();   // the previous round's tiles are read
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int k = 0; k < RT; ++k) {
                f32x4 v = o[ht][rd * RT + k];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] *= own_o[ht][i];
                xo[((wave * HT + ht) * RT + k) * CSA2_WAVE + lane] = v;
            }
        __syncthreads();
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int k = 0; k < QW; ++k) {
                const int tk = wave * QW + k;   // tile rd * RT + tk of the output
                f32x4 acc = xo[((0 * HT + ht) * RT + tk) * CSA2_WAVE + lane];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) acc += xo[((w * HT + ht) * RT + tk) * CSA2_WAVE + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int hh = ht * 16 + 4 * grp + i;
                    if (h0 + hh < H) dst[(int64_t)hh * D + 16 * (rd * RT + tk) + col] = acc[i] * inv_o[ht][i];
                }
            }
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
    int HT, HG, CS, S, nfrag;
};

// Workgroup shape: heads per workgroup (16 HT), channel parts CS and key
// splits S per row.  A workgroup dequantises and stages each of its keys once
// and computes full scores, whatever its head count and channel part, so:
//   * the head count per group is as large as the registers allow (each wave
//     holds all D query channels and its part of the output of every head:
//     HT <= 512 / D) while the rows alone give about one workgroup per
//     compute unit;
//   * otherwise HT = 1 and a row's keys are split over up to kMaxPlanSplits
//     workgroups (each split adds a partial output for the merge kernel).
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
    p.CS = 1;
    if ((int64_t)R * p.HG < kTargetGroups) {
        p.HT = 1;
        p.HG = heads16;
    }
    const int64_t smax = p.nfrag / kWaves > 1 ? p.nfrag / kWaves : 1;   // at least one fragment per wave
    const int64_t base = (int64_t)R * p.HG;
    int64_t S = base >= kTargetGroups ? 1 : (kTargetGroups + base - 1) / base;
    if (S > kMaxPlanSplits) S = kMaxPlanSplits;
    if (S > smax) S = smax;
    // Channel parts repeat the whole score computation, which costs more
    // than the merge of further key splits at every measured shape (4 to 256
    // rows, 64 heads, D = 512), so they are not planned; the kernels support
    // them (CS = 2, and 4 for D = 512).
    p.S = (int)S;
    return p;
}

template <int HT, int D, int CS, bool PG>
void launch_attn(dim3 grid, hipStream_t st, const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                 const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len, const int32_t* topk,
                 int32_t K, const uint8_t* swa, const int64_t* swa_row_start, const int32_t* swa_len,
                 const int32_t* swa_head, int64_t phys_rows, int32_t H, int32_t R, int32_t W, float sl2e, int HG,
                 int S, int nfrag, float* out, float* lse, float* po, float* pml)
{
    hipLaunchKernelGGL((k_sparse_attn<HT, D, CS, PG>), grid, dim3(64 * kWaves), 0, st, q, codes, scales, seq_start, row_seq,
                       row_len, topk, K, swa, swa_row_start, swa_len, swa_head, phys_rows, R, H, W, sl2e, HG, S,
                       nfrag, out, lse, po, pml);
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
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace

extern "C" size_t csa2_sparse_attn_workspace_bytes(int32_t R, int32_t H, int32_t D, int32_t K, int32_t W)
{
    if (R <= 0 || H <= 0 || D <= 0 || K < 0 || W < 0) return 0;
    const AttnPlan p = plan_attn(R, H, D, K, W);
    if (p.S <= 1) return 0;
    return csa2::align_up((size_t)R * p.S * H * D * 4, 256) + csa2::align_up((size_t)R * p.S * H * 4 * 4, 256);
}

namespace {
csa2_status_t sparse_attn_impl(const uint16_t* q, const uint8_t* codes, const uint8_t* scales,
                               const int64_t* seq_start, const int32_t* row_seq, const int32_t* row_len,
                               int64_t phys_rows, const int32_t* topk_idx, int32_t K, const uint8_t* swa,
                               const int64_t* swa_row_start, const int32_t* swa_len, const int32_t* swa_head,
                               int32_t R, int32_t H, int32_t D, int32_t W, float softmax_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream)
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
    CSA2_REQUIRE(xcd_grid(R, (int64_t)p.HG * p.CS * p.S) <= 0x7FFFFFFF, CSA2_ERR_UNSUPPORTED,
                 "sparse_attn: grid too large");
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
    const dim3 grid((unsigned)xcd_grid(R, p.HG * p.CS * p.S));
#define CSA2_ATTN(ht, d, cs)                                                                               \
    if (p.HT == ht && D == d && p.CS == cs) {                                                               \
        (phys_rows > 0 ? launch_attn<ht, d, cs, true> : launch_attn<ht, d, cs, false>)(grid, st, q, codes, scales, seq_start, row_seq, row_len, topk_idx, K, swa,   \
                               swa_row_start, swa_len, swa_head, phys_rows, H, R, W, sl2e, p.HG, p.S, p.nfrag, \
                               out, lse, po, pml);                                                          \
    }
    CSA2_ATTN(1, 128, 1) CSA2_ATTN(2, 128, 1) CSA2_ATTN(4, 128, 1) CSA2_ATTN(1, 128, 2)
    CSA2_ATTN(1, 256, 1) CSA2_ATTN(2, 256, 1) CSA2_ATTN(1, 256, 2)
    CSA2_ATTN(1, 512, 1) CSA2_ATTN(1, 512, 2) CSA2_ATTN(1, 512, 4)
#undef CSA2_ATTN
    if (p.S > 1)
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)xcd_grid(R, H)), dim3(128), 0, st, po, pml, R, H, D, p.S,
                           out, lse);
    return csa2::check_launch("sparse_attn");
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
    return csa2::check_launch("paged_rows");
}
