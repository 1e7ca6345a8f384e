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

// Value from the lane n places lower in the same row of 16 lanes; 0 for the first n lanes.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}
// Inclusive prefix sum over each row of 16 lanes (Hillis-Steele, 4 DPP steps).
__device__ __forceinline__ float scan16_add(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
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

}  // namespace kda
