// Device-side building blocks for the gfx950 (CDNA4) KDA kernels: bf16 packing,
// 16-lane DPP scans and the 16x16 matrix-core (MFMA) tile products.
//
// Fragment convention used by every MFMA product in this library
// -----------------------------------------------------------------
// A 16x16 output tile lives in the MFMA accumulator layout: lane l holds rows
// 4*(l/16)+j (j = 0..3) of column l%16.  Contractions are cut into 16-wide k tiles.
// For one k tile, lane l supplies the four k indices 4*(l/16) .. 4*(l/16)+3:
//   A operand (16 x k):  A[m = l%16][k = 4*(l/16) + j]
//   B operand (k x 16):  B[k = 4*(l/16) + j][n = l%16]
// so an accumulator tile can be fed back as a B operand without moving data between
// lanes, and operands stored row-major by their non-contracted index (A as [m][k],
// B as [n][k]) are read as 4 consecutive elements per lane.  The sum over k does not
// depend on which hardware k slot a value occupies, only that A and B agree, so the
// same fragments drive v_mfma_f32_16x16x4_f32 (4 slots of 1) and v_mfma_f32_16x16x32_bf16
// (two tiles, or one tile with the other half zero).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
    __bf16 h = (__bf16)a;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until at most N of this wave's vector memory loads are outstanding (they complete in
// issue order); the other counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// lds + 16 l (lds is the same for every lane of the wave).  The write is complete once this
// wave's vmcnt has counted the load; other waves may read it after a barrier that follows.
__device__ __forceinline__ void load_lds16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
// 4 bytes per lane likewise: lane l's bytes land at lds + 4 l
__device__ __forceinline__ void load_lds4(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 4, 0, 0);
}

// Value from the lane n places lower in the same row of 16 lanes; 0 for the first n lanes.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}
// Value from the lane n places higher in the same row of 16 lanes; 0 for the last n lanes.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xf, 0xf, true));
}
// One operand-type element as fp32.
__device__ __forceinline__ float elem_f32(float x) { return x; }
__device__ __forceinline__ float elem_f32(uint16_t x) { return bf16_to_f32(x); }
// Inclusive prefix sum over each row of 16 lanes (Hillis-Steele, 4 DPP steps).
__device__ __forceinline__ float scan16_add(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// ------------------------------------------ diagonal blocks under strong decay --
// Inside one 16-token sub-chunk the gated products need e^{G_r - G_i} (i <= r) per channel.  With
// one anchor per sub-chunk one factor of that split grows like e^{-(total decay)} and overflows
// once a channel decays by more than about e^{-88} within 16 tokens.  The exact alternative used
// there splits the 16 tokens in halves, quarters, eighths and pairs: tokens r > i lie in the same
// block but in different halves at exactly one of these four levels, and at that level the anchor
// a = G at the last token of the first half gives e^{G_r - G_i} = e^{G_r - a} e^{a - G_i} with both
// factors <= 1.  Per level, the row operand keeps only second-half tokens and the column operand
// only first-half tokens, so every product pairs tokens split at that level and the four level
// products sum to the strictly lower part of the block (the diagonal, factor 1, is added apart).

// True when the lane's token (l16, in its row of 16 lanes) lies in the second half of its block at
// level LVL (block sizes 16, 8, 4, 2 for LVL 0..3).
template <int LVL>
__device__ __forceinline__ bool split_second(int l16) {
    return (l16 >> (3 - LVL)) & 1;
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// G at the anchor token of the lane's block at level LVL: the last token of the block's first half
// (tokens 7 | 3, 11 | 1, 5, 9, 13 | 0, 2, ..., 14), gathered within each row of 16 lanes by DPP
// (quad_perm 0xA0 = [0,0,2,2], 0x55 = [1,1,1,1], 0xFF = [3,3,3,3]; row_half_mirror 0x141 takes
// lane 7 - x of each half row, row_mirror 0x140 lane 15 - x of the row).
template <int LVL>
__device__ __forceinline__ float split_anchor(float G, int l16) {
    if constexpr (LVL == 3) {
        return dpp_mov<0xA0>(G);
    } else if constexpr (LVL == 2) {
        return dpp_mov<0x55>(G);
    } else {
        const float t = dpp_mov<0xFF>(G);        // quad q: G of token 4q + 3
        const float u = dpp_mov<0x141>(t);       // lane x: t of lane 7 - x in its half row
        if constexpr (LVL == 1) {
            return (l16 & 4) ? u : t;            // tokens 3 (lanes 0-7) and 11 (lanes 8-15)
        } else {
            const float v = (l16 & 4) ? t : u;   // lanes 0-7: token 7
            const float w = dpp_mov<0x140>(v);   // lanes 8-15: lane 15 - x, i.e. lanes 7-0
            return (l16 & 8) ? w : v;
        }
    }
}

// Factor of a token at level LVL: e^{G - a} for a second-half token, e^{a - G} for a first-half one
// (both <= 1 since the cumulative log-gate G does not increase along the tokens).
template <int LVL>
__device__ __forceinline__ float split_factor(float G, int l16) {
    return __builtin_amdgcn_exp2f(-fabsf(G - split_anchor<LVL>(G, l16)));
}

// ---------------------------------------------------------------- fragments --
// One lane's share of one 16-wide k tile: 4 values, as packed bf16 or fp32.
template <bool BF16>
struct Frag;
template <>
struct Frag<true> {
    uint2 v;
};
template <>
struct Frag<false> {
    float4 v;
};

template <bool BF16>
__device__ __forceinline__ Frag<BF16> make_frag(float a, float b, float c, float d);
template <>
__device__ __forceinline__ Frag<true> make_frag<true>(float a, float b, float c, float d) {
    Frag<true> f;
    f.v.x = pack_bf16x2(a, b);
    f.v.y = pack_bf16x2(c, d);
    return f;
}
template <>
__device__ __forceinline__ Frag<false> make_frag<false>(float a, float b, float c, float d) {
    Frag<false> f;
    f.v = make_float4(a, b, c, d);
    return f;
}
template <bool BF16>
__device__ __forceinline__ Frag<BF16> frag_from_acc(const f32x4 &x, float s = 1.0f) {
    return make_frag<BF16>(x[0] * s, x[1] * s, x[2] * s, x[3] * s);
}

// 4 consecutive operand values from LDS (bf16 bits or fp32).
__device__ __forceinline__ Frag<true> lds_frag(const uint16_t *p) {
    Frag<true> f;
    f.v = *reinterpret_cast<const uint2 *>(p);
    return f;
}
__device__ __forceinline__ Frag<false> lds_frag(const float *p) {
    Frag<false> f;
    f.v = *reinterpret_cast<const float4 *>(p);
    return f;
}
// 4 consecutive fp32 values from LDS, converted to the operand type and multiplied by s.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> lds_frag_f32(const float *p, float s = 1.0f) {
    const float4 x = *reinterpret_cast<const float4 *>(p);
    return make_frag<BF16>(x.x * s, x.y * s, x.z * s, x.w * s);
}

// acc += A * B over one 16-wide k tile.  bf16 uses the K=32 instruction with a zero second
// half: code built for gfx950 with v_mfma_f32_16x16x16_bf16 computed wrong results that varied
// from run to run where its result was read back soon after (the backward reverse scan at
// d_k = 64), and the same code with the K=32 instruction is exact and repeatable.
__device__ __forceinline__ void mma16(f32x4 &acc, const Frag<true> &a, const Frag<true> &b) {
    const uint4 av = make_uint4(a.v.x, a.v.y, 0u, 0u);
    const uint4 bv = make_uint4(b.v.x, b.v.y, 0u, 0u);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc,
                                                  0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4 &acc, const Frag<false> &a, const Frag<false> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.x, b.v.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.y, b.v.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.z, b.v.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.w, b.v.w, acc, 0, 0, 0);
}
// acc += A * B over two 16-wide k tiles (k tile 0 from a0/b0, k tile 1 from a1/b1).
__device__ __forceinline__ void mma32(f32x4 &acc, const Frag<true> &a0, const Frag<true> &a1, const Frag<true> &b0,
                                      const Frag<true> &b1) {
    const uint4 av = make_uint4(a0.v.x, a0.v.y, a1.v.x, a1.v.y);
    const uint4 bv = make_uint4(b0.v.x, b0.v.y, b1.v.x, b1.v.y);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc,
                                                  0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x4 &acc, const Frag<false> &a0, const Frag<false> &a1, const Frag<false> &b0,
                                      const Frag<false> &b1) {
    mma16(acc, a0, b0);
    mma16(acc, a1, b1);
}

// Wait states between matrix-core products and reads of their results that may sit in another basic
// block.  A VALU read (or v_accvgpr_read) of an MFMA result needs 11 wait states after an 8-pass
// instruction (16x16x32 bf16, 16x16x4 f32 on gfx950) and 19 after a 16-pass one.  The compiler
// inserts them within a block, but across a join was seen to leave none: the last product of a chain
// ended its block, a branch led to a block reached also from a path that did have the wait states,
// and the first instruction there read the accumulator's stale value (wrong results, no fault).
// The accumulators pass through this asm as operands, so it sits after their last product and before
// every read, and its three s_nop 7 give 24 wait states.  Used where a chain's results are consumed
// after a branch or a loop exit.
__device__ __forceinline__ void mfma_settle(f32x4 &a) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a)); }
__device__ __forceinline__ void mfma_settle(f32x4 &a, f32x4 &b) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// Orders LDS accesses between the lanes of one wave: a wave barrier (convergent, so code around
// it cannot be duplicated into divergent branches) and a wavefront-scope fence (no LDS access is
// moved across it).  A wave's LDS operations execute in order, so no instruction is emitted; it
// is needed wherever lanes read what other lanes of the same wave wrote without a workgroup
// barrier in between.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Writes a ROWS x WC fp32 tile held in LDS (row stride LDK floats) to dst (row stride ld
// elements, element type OT: bf16 bits or fp32) as 16-byte row segments spread over the lanes of
// one wave.  Used to turn accumulator fragments (4 rows of one column per lane) into few wide
// stores; a tile of many rows keeps all of its LDS reads in flight at once.  The tile is written
// by other lanes of the same wave just before and rewritten just after, so the read-back is
// bracketed by wave_lds_sync (without it the compiler duplicated the code after the partial-wave
// read-back into its divergent branches, and the lanes with no segment wrote the next tile before
// the other lanes had read this one).
template <typename OT, int WC, int LDK, int ROWS = 16>
__device__ __forceinline__ void keep_rows(OT *dst, int64_t ld, const float *tile, int lane) {
    constexpr int EPS = 16 / (int)sizeof(OT), SPR = WC / EPS, NSEG = ROWS * SPR;
    static_assert(WC % EPS == 0 && LDK % 4 == 0, "whole 16-byte segments");
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < (NSEG + 63) / 64; ++i) {
        const int sg = lane + 64 * i;
        if (NSEG % 64 == 0 || sg < NSEG) {
            const int row = sg / SPR, c0 = (sg % SPR) * EPS;
            const float *src = tile + row * LDK + c0;
            if constexpr (sizeof(OT) == 2) {
                const float4 a = *reinterpret_cast<const float4 *>(src);
                const float4 b = *reinterpret_cast<const float4 *>(src + 4);
                const uint2 lo = make_frag<true>(a.x, a.y, a.z, a.w).v, hi = make_frag<true>(b.x, b.y, b.z, b.w).v;
                *reinterpret_cast<uint4 *>(dst + row * ld + c0) = make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
                *reinterpret_cast<float4 *>(dst + row * ld + c0) = *reinterpret_cast<const float4 *>(src);
            }
        }
    }
    wave_lds_sync();
}

template <typename IO>
struct IoTraits;  // fp32 / bf16 io element access, below

// ------------------------------------------------- split-level diagonal blocks --
// A wave's own 16 x 16 diagonal block of the chunk matrices for one sub-chunk, exact under any
// decay: per split level (see split_anchor), row operands keep the second-half tokens scaled by
// e^{G - a} and column operands the first-half tokens scaled by e^{a - G}, all factors <= 1.  A
// level's product also pairs tokens of different blocks (with each other's anchors, so still
// bounded by 1); those entries are dropped before the level is added.
//   accA [j] = sum_c k_rc k_ic e^{G_rc - G_ic}   for r = 4*q4 + j, i = l16, i < r (else 0)
//   accPt[j] = sum_c q_rc k_ic e^{G_rc - G_ic}   for r = l16, i = 4*q4 + j, i <= r (else 0)
// i.e. the accumulator layouts of the strictly lower part of K K^T and of the transpose of the
// lower part (with diagonal) of Q K^T, before beta.  kqg(ct, k, q, G) gives the lane's raw k and q
// for channels 16 ct + 4 q4 .. + 3 of its token (zero past the chunk end) and the in-sub-chunk
// cumulative log2 gate G of the same channels; it is called once per channel tile.
template <bool BF, int LVL, int KT, bool WA, bool WP, typename KQG>
__device__ __forceinline__ void split_level_add(f32x4 &accA, f32x4 &accPt, const KQG &kqg, int l16, int q4) {
    const bool sec = split_second<LVL>(l16);
    f32x4 tA = zero4(), tPt = zero4();
    // one 16-channel tile per product keeps few operands live at a time (a rare path)
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
        float4 kv, qv, gv;
        kqg(ct, kv, qv, gv);
        const float kx[4] = {kv.x, kv.y, kv.z, kv.w}, qx[4] = {qv.x, qv.y, qv.z, qv.w};
        const float gx[4] = {gv.x, gv.y, gv.z, gv.w};
        float a[4], b[4], c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float f = split_factor<LVL>(gx[j], l16);
            a[j] = sec ? kx[j] * f : 0.f;
            b[j] = sec ? qx[j] * f : 0.f;
            c[j] = sec ? 0.f : kx[j] * f;
        }
        const Frag<BF> ck = make_frag<BF>(c[0], c[1], c[2], c[3]);
        if constexpr (WA) mma16(tA, make_frag<BF>(a[0], a[1], a[2], a[3]), ck);
        if constexpr (WP) mma16(tPt, ck, make_frag<BF>(b[0], b[1], b[2], b[3]));
    }
    mfma_settle(tA, tPt);
    // keep the pairs of tokens in the same block of 16 >> LVL (an entry's two token indices are
    // 4*q4 + j and l16 in both layouts)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool same = ((4 * q4 + j) >> (4 - LVL)) == (l16 >> (4 - LVL));
        if constexpr (WA) accA[j] += same ? tA[j] : 0.f;
        if constexpr (WP) accPt[j] += same ? tPt[j] : 0.f;
    }
}

// WA / WP select the blocks to form (both by default; one at a time where registers are short).
template <bool BF, int KT, typename KQG, bool WA = true, bool WP = true>
__device__ __forceinline__ void diag_block_split(f32x4 &accA, f32x4 &accPt, const KQG &kqg, int l16, int q4) {
    accA = zero4();
    accPt = zero4();
    split_level_add<BF, 0, KT, WA, WP>(accA, accPt, kqg, l16, q4);
    split_level_add<BF, 1, KT, WA, WP>(accA, accPt, kqg, l16, q4);
    split_level_add<BF, 2, KT, WA, WP>(accA, accPt, kqg, l16, q4);
    split_level_add<BF, 3, KT, WA, WP>(accA, accPt, kqg, l16, q4);
    if constexpr (WP) {
        float dot = 0.f;  // q_r . k_r of the lane's token over its channels (the diagonal, factor 1)
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            float4 kv, qv, gv;
            kqg(ct, kv, qv, gv);
            dot += kv.x * qv.x + kv.y * qv.y + kv.z * qv.z + kv.w * qv.w;
        }
        // the four lanes of a token (q4 = 0..3) hold disjoint channels
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        if (q4 == (l16 >> 2)) {  // P_RR[r][r] sits at r = l16, i = 4*q4 + j with j = l16 % 4
            const int jd = l16 & 3;
            accPt[0] += jd == 0 ? dot : 0.f;
            accPt[1] += jd == 1 ? dot : 0.f;
            accPt[2] += jd == 2 ? dot : 0.f;
            accPt[3] += jd == 3 ? dot : 0.f;
        }
    }
}

// The same blocks with every loop rolled and the operands reloaded from memory: a few hundred
// instructions and few live registers, for kernels whose common path already uses every register
// (there the unrolled form's code and temporaries slow the common path down).  k, q and g point at
// the lane's token row (channels 4*q4 ...: tile ct at + 16 ct), valid is false past the chunk end.
template <typename IO>
__device__ __forceinline__ void diag_block_split_rolled(f32x4 &accA, f32x4 &accPt, const IO *k, const IO *q,
                                                        const float *g, bool valid, int KT, int l16, int q4,
                                                        int lane) {
    constexpr bool BF = IoTraits<IO>::kBf16;
    accA = zero4();
    accPt = zero4();
    float dot = 0.f;
#pragma unroll 1
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int hs = 8 >> lvl;
        const bool sec = (l16 & hs) != 0;
        const int src = (lane & ~15) | ((l16 & ~(2 * hs - 1)) + hs - 1);  // the level's anchor token
        f32x4 tA = zero4(), tPt = zero4();
#pragma unroll 1
        for (int ct = 0; ct < KT; ++ct) {
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 kv = valid ? IoTraits<IO>::load4(k + 16 * ct) : z;
            const float4 qv = valid ? IoTraits<IO>::load4(q + 16 * ct) : z;
            const float4 gr = *reinterpret_cast<const float4 *>(g + 16 * ct);
            const float m = valid ? kLog2e : 0.f;
            const float G[4] = {scan16_add(gr.x * m), scan16_add(gr.y * m), scan16_add(gr.z * m),
                                scan16_add(gr.w * m)};
            const float kx[4] = {kv.x, kv.y, kv.z, kv.w}, qx[4] = {qv.x, qv.y, qv.z, qv.w};
            float a[4], b[4], c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = __builtin_amdgcn_exp2f(-fabsf(G[j] - __shfl(G[j], src)));
                a[j] = sec ? kx[j] * f : 0.f;
                b[j] = sec ? qx[j] * f : 0.f;
                c[j] = sec ? 0.f : kx[j] * f;
                if (lvl == 0) dot += kx[j] * qx[j];
            }
            const Frag<BF> ck = make_frag<BF>(c[0], c[1], c[2], c[3]);
            mma16(tA, make_frag<BF>(a[0], a[1], a[2], a[3]), ck);
            mma16(tPt, ck, make_frag<BF>(b[0], b[1], b[2], b[3]));
        }
        mfma_settle(tA, tPt);  // read after the loop's exit
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool same = ((4 * q4 + j) >> (4 - lvl)) == (l16 >> (4 - lvl));
            accA[j] += same ? tA[j] : 0.f;
            accPt[j] += same ? tPt[j] : 0.f;
        }
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    if (q4 == (l16 >> 2)) {
        const int jd = l16 & 3;
        accPt[0] += jd == 0 ? dot : 0.f;
        accPt[1] += jd == 1 ? dot : 0.f;
        accPt[2] += jd == 2 ? dot : 0.f;
        accPt[3] += jd == 3 ? dot : 0.f;
    }
}

// diag_block_split_rolled with the lane's k, q (as the operator sees them; zero for tokens past the
// chunk end) and its scanned log2 gate G already in registers: the fused prologue has no memory copy
// of the transformed operands to reload.  The level loop stays rolled.
template <typename IO, int KT>
__device__ __forceinline__ void diag_block_split_regs(f32x4 &accA, f32x4 &accPt, const float (&kr)[KT][4],
                                                      const float (&qr)[KT][4], const float (&G)[KT][4], int l16,
                                                      int q4, int lane) {
    constexpr bool BF = IoTraits<IO>::kBf16;
    accA = zero4();
    accPt = zero4();
    float dot = 0.f;
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) dot += kr[ct][j] * qr[ct][j];
#pragma unroll 1
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int hs = 8 >> lvl;
        const bool sec = (l16 & hs) != 0;
        const int src = (lane & ~15) | ((l16 & ~(2 * hs - 1)) + hs - 1);  // the level's anchor token
        f32x4 tA = zero4(), tPt = zero4();
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            float a[4], b[4], c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = __builtin_amdgcn_exp2f(-fabsf(G[ct][j] - __shfl(G[ct][j], src)));
                a[j] = sec ? kr[ct][j] * f : 0.f;
                b[j] = sec ? qr[ct][j] * f : 0.f;
                c[j] = sec ? 0.f : kr[ct][j] * f;
            }
            const Frag<BF> ck = make_frag<BF>(c[0], c[1], c[2], c[3]);
            mma16(tA, make_frag<BF>(a[0], a[1], a[2], a[3]), ck);
            mma16(tPt, ck, make_frag<BF>(b[0], b[1], b[2], b[3]));
        }
        mfma_settle(tA, tPt);  // read after the loop's exit
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool same = ((4 * q4 + j) >> (4 - lvl)) == (l16 >> (4 - lvl));
            accA[j] += same ? tA[j] : 0.f;
            accPt[j] += same ? tPt[j] : 0.f;
        }
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    if (q4 == (l16 >> 2)) {
        const int jd = l16 & 3;
        accPt[0] += jd == 0 ? dot : 0.f;
        accPt[1] += jd == 1 ? dot : 0.f;
        accPt[2] += jd == 2 ? dot : 0.f;
        accPt[3] += jd == 3 ? dot : 0.f;
    }
}

// 4 packed io values (bf16 pair words or fp32) -> fp32
template <bool BF, typename KQ>
__device__ __forceinline__ float4 unpack4(const KQ &x) {
    if constexpr (BF) return make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
    else return x;
}

// ---------------------------------------------------------- fused prologue ----
// The activations of the prologue (Kimi Linear summary page, "Kimi Linear model composition";
// the readings: Swish(c) = c sigmoid(c), g = -softplus(g_raw), beta = sigmoid(beta_raw)), in the
// same fp32 forms as the standalone prologue kernels.
__device__ __forceinline__ float swish_f(float c) { return c * __builtin_amdgcn_rcpf(1.0f + __expf(-c)); }
__device__ __forceinline__ float neg_softplus_f(float x) { return -(fmaxf(x, 0.f) + __logf(1.0f + __expf(-fabsf(x)))); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Filter taps of one channel as a 4-tap window over tokens t-3 .. t: tap i < W of the W-tap filter
// (tap W-1 on the current token) lands at position 4 - W + i, the front is zero.
__device__ __forceinline__ void conv_taps4(const float *w, int W, float (&w4)[4]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) w4[d] = d >= 4 - W ? w[d - (4 - W)] : 0.f;
}

// Largest in-sub-chunk decay (log2 units) for which the single-anchor diagonal blocks stay exact:
// their column factor e^{b_R - G_i} is then at most 2^96 and the row factor at least 2^-96, far
// inside the normal range of fp32 and bf16.  Waves whose sub-chunk decays further in some channel
// use diag_block_split.
constexpr float kDiagAnchorMaxDecay = 96.f;

// True (uniformly across the wave) when some channel of the lanes' sub-chunks has an in-sub-chunk
// cumulative log2 gate below -kDiagAnchorMaxDecay.
template <int KT>
__device__ __forceinline__ bool diag_needs_split(const float (&G)[KT][4]) {
    bool big = false;
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) big |= G[ct][j] < -kDiagAnchorMaxDecay;
    return __builtin_amdgcn_ballot_w64(big) != 0;
}

// ------------------------------------------------------------ io element types --
// q, k, v and out are fp32 or bf16 in memory; g, beta and states are fp32.
template <typename IO>
struct IoTraits;
template <>
struct IoTraits<float> {
    static constexpr bool kBf16 = false;
    // 4 consecutive io values -> fp32
    __device__ static __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    __device__ static __forceinline__ float load1(const float *p) { return *p; }
    __device__ static __forceinline__ float to_float(float x) { return x; }
    __device__ static __forceinline__ void store1(float *p, float x) { *p = x; }
    __device__ static __forceinline__ void store4(float *p, float4 x) { *reinterpret_cast<float4 *>(p) = x; }
};
template <>
struct IoTraits<uint16_t> {
    static constexpr bool kBf16 = true;
    __device__ static __forceinline__ float4 load4(const uint16_t *p) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    }
    __device__ static __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ float to_float(uint16_t x) { return bf16_to_f32(x); }
    __device__ static __forceinline__ void store1(uint16_t *p, float x) { *p = f32_to_bf16(x); }
    __device__ static __forceinline__ void store4(uint16_t *p, float4 x) {
        uint2 w;
        w.x = pack_bf16x2(x.x, x.y);
        w.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<uint2 *>(p) = w;
    }
};

// Workgroup -> logical work item.  Workgroups are dealt to the 8 XCDs round robin
// (block b runs on XCD b % 8); this remaps block ids so that consecutive logical items
// land on the same XCD and share its L2 (used to keep the d_v tiles of one (sequence,
// head) together).  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int64_t xcd_grouped_block(int64_t b, int64_t nblocks) {
    if ((nblocks & 7) != 0) return b;
    const int64_t per = nblocks >> 3;
    return (b & 7) * per + (b >> 3);
}

// Workgroup -> (sequence, head, d_v tile) for the kernels that walk one sequence's chunks in order.
// A unit is a (sequence rank, head) pair; its ntile d_v tiles run next to each other on one XCD,
// since they read the same per-chunk inputs through its L2.  When the unit count is a multiple of 8
// the units are dealt to the XCDs in turn, in rank order: workgroups start in id order, so with
// `order` listing the sequences most chunks first the longest chains start first and every XCD
// gets every 8th of them.  Without `order` the rank is the sequence index.
struct SeqItem {
    int n, h, tile;
};
__device__ __forceinline__ SeqItem seq_item(int64_t b, int num_seqs, int H, int ntile, const int32_t *order) {
    const int64_t units = (int64_t)num_seqs * H;
    int64_t u;
    int tile;
    if ((units & 7) == 0) {
        const int64_t j = b >> 3;  // position on XCD b % 8
        u = (j / ntile) * 8 + (b & 7);
        tile = (int)(j % ntile);
    } else {
        const int64_t item = xcd_grouped_block(b, units * ntile);
        u = item / ntile;
        tile = (int)(item % ntile);
    }
    const int r = (int)(u / H);
    return SeqItem{order ? order[r] : r, (int)(u % H), tile};
}

}  // namespace kda
