// General-DPLR chunk forward for gfx950: the comparator KDA is measured against.
//
// Recurrence (Kimi Linear summary page, "Less compute than general DPLR" section: general
// DPLR keeps two independent low-rank vectors, KDA ties both to the key):
//
//   S_t = (Diag(e^{g_t}) + a_t b_t^T) S_{t-1} + k_t v_t^T,    o_t = scale * S_t^T q_t
//
// Chunk form (one chunk, initial state S, G = in-chunk cumulative gate, G_{-1} = 0):
//   B~ = b e^{G_{r-1}}, Q~ = q e^{G}, A^ = a e^{-G}, K^ = k e^{-G}, A- = a e^{G_C-G}, K- = k e^{G_C-G}
//   M_ba = strictly_lower(B~ A^T)   M_bk = strictly_lower(B~ K^T)        (from b)
//   M_qa = lower_incl(Q~ A^T)       M_qk = lower_incl(Q~ K^T)            (from q)
//   U  = (I - M_ba)^{-1} (B~ S + M_bk V)
//   O  = scale (Q~ S + M_qa U + M_qk V)
//   S <- Diag(e^{G_C}) S + A-^T U + K-^T V
// Four C x C matrices where KDA has two, and three more matrix products per state slice
// (M_bk V, M_qk V, K-^T V).  The kernel keeps the structure of the fused KDA forward
// (kda_chunk_impl.h) so that the two are compared like for like: one workgroup per
// (sequence, head, d_v tile), four waves, wave R owns 16-token sub-chunk R, the state tile
// in registers, bf16 matrix-core products with fp32 accumulation.
//
// Numerics as in KDA: log2-domain gates, e^{G_r - G_i} split at sub-chunk boundaries;
// the row operand of block (R, I) carries e^{b_R - b_{I+1}} (so every off-diagonal factor is
// <= 1), the diagonal block's column operand carries e^{b_R - G_i} >= 1.  The b-rows use
// the exclusive prefix G_{r-1}.
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename IO, int DK, int DVT, int C>
struct DplrLayout {
    static constexpr bool BF = IoTraits<IO>::kBf16;
    using OT = typename std::conditional<BF, uint16_t, float>::type;
    static constexpr int NW = 4;
    static constexpr int NSUB = C / 16;
    static constexpr int KT = DK / 16;
    static constexpr int NSL = DVT / 16;
    static constexpr int SPW = NSL > NW ? NSL / NW : 1;
    static constexpr int PADO = 16 / (int)sizeof(OT);
    static constexpr int LDO = DK + PADO;
    static constexpr int LDT = C + PADO;
    static constexpr int LDM = C + PADO;
    static constexpr int LDD = 16 + 4;
    static constexpr int LDV = DVT + PADO;
    static constexpr int NSHIFT = NSUB >= 3 ? (NSUB - 1) * (NSUB - 2) / 2 : 0;
    static_assert(C % 16 == 0 && NSUB >= 1 && NSUB <= NW, "chunk must be 16, 32 or 64");
    static_assert(DK % 32 == 0 && DVT % 16 == 0, "head dims");
    static_assert(NSL <= NW || NSL % NW == 0, "d_v tile");

    static constexpr int V_PIECES = C * DVT * (int)sizeof(IO) / 16;
    static constexpr int V_PER_THREAD = (V_PIECES + kChunkThreads - 1) / kChunkThreads;
    static constexpr int V_ELEMS = 16 / (int)sizeof(IO);

    static constexpr size_t kOp = (size_t)C * LDO * sizeof(OT);
    static constexpr size_t kOpT = (size_t)DK * LDT * sizeof(OT);
    // region shared by the block products' column operands (A^, K^ of each sub-chunk)
    // and, after them, the inter-chunk operands (Q~, B~, A-^T, K-^T)
    static constexpr size_t kRegA = 2 * kOp;
    static constexpr size_t kRegB = 2 * kOp + 2 * kOpT;
    static constexpr size_t oAb = 0, oKb = kOp;
    static constexpr size_t oQt = 0, oBt = kOp, oAbT = 2 * kOp, oKbT = 2 * kOp + kOpT;
    static constexpr size_t oM = kRegA > kRegB ? kRegA : kRegB;
    static constexpr size_t kMat = (size_t)C * LDM * sizeof(OT);
    static constexpr size_t oMba = oM, oMbk = oM + kMat, oMqa = oM + 2 * kMat, oMqk = oM + 3 * kMat;
    static constexpr size_t oAd = oM + 4 * kMat;
    static constexpr size_t oV = oAd + (size_t)NSUB * 16 * LDD * 4;
    static constexpr size_t oTot = oV + (size_t)C * LDV * sizeof(OT);
    static constexpr size_t oEB = oTot + (size_t)NSUB * DK * 4;
    static constexpr size_t oED = oEB + (size_t)NSUB * DK * 4;
    static constexpr size_t oEC = oED + (size_t)NSUB * DK * 4;
    static constexpr size_t oSH = oEC + (size_t)NSUB * DK * 4;
    static constexpr size_t oGam = oSH + (size_t)(NSHIFT > 0 ? NSHIFT : 1) * DK * 4;
    static constexpr size_t kBytes = oGam + (size_t)DK * 4;
    static constexpr bool kFits = kBytes <= 160 * 1024;

    __host__ __device__ static constexpr int shift_slot(int R, int I) { return (R - 2) * (R - 1) / 2 + I; }
};

template <typename IO, int DK, int DVT, int C>
struct DplrRaw {
    using L = DplrLayout<IO, DK, DVT, C>;
    using KQ = typename std::conditional<L::BF, uint2, float4>::type;
    float4 g[L::KT];
    KQ k[L::KT], q[L::KT], a[L::KT], b[L::KT];
    uint4 v[L::V_PER_THREAD];
};

template <typename IO, int DK, int DVT, int C>
__device__ __forceinline__ void dplr_load_chunk(DplrRaw<IO, DK, DVT, C> &raw, const DplrParams &dp, int64_t tok0,
                                                int clen, int h, int col0, int tid) {
    using L = DplrLayout<IO, DK, DVT, C>;
    using KQ = typename DplrRaw<IO, DK, DVT, C>::KQ;
    const FwdParams &p = dp.f;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    const int H = p.H;
    if (wave < L::NSUB) {
        const int r = min(16 * wave + l16, clen - 1);
        const int64_t row = ((tok0 + r) * H + h) * (int64_t)DK + 4 * q4;
#pragma unroll
        for (int ct = 0; ct < L::KT; ++ct) {
            raw.g[ct] = *reinterpret_cast<const float4 *>(p.g + row + 16 * ct);
            raw.k[ct] = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.k) + row + 16 * ct);
            raw.q[ct] = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.q) + row + 16 * ct);
            raw.a[ct] = *reinterpret_cast<const KQ *>(static_cast<const IO *>(dp.a) + row + 16 * ct);
            raw.b[ct] = *reinterpret_cast<const KQ *>(static_cast<const IO *>(dp.b) + row + 16 * ct);
        }
    }
    constexpr int PPR = DVT / L::V_ELEMS;
#pragma unroll
    for (int i = 0; i < L::V_PER_THREAD; ++i) {
        const int piece = tid + kChunkThreads * i;
        if (L::V_PIECES % kChunkThreads == 0 || piece < L::V_PIECES) {
            const int r = min(piece / PPR, clen - 1);
            const int cc = (piece % PPR) * L::V_ELEMS;
            raw.v[i] = *reinterpret_cast<const uint4 *>(static_cast<const IO *>(p.v) +
                                                        ((tok0 + r) * H + h) * (int64_t)p.dv + col0 + cc);
        }
    }
}

template <typename KQ, bool BF>
__device__ __forceinline__ float4 dplr_unpack(const KQ &x) {
    if constexpr (BF) return make_float4(bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y));
    else return x;
}

// One of the four chunk matrices' diagonal 16 x 16 blocks of a sub-chunk, exact under any decay:
// the split levels of kda_device.h (split_anchor) with the loops rolled, the operands reloaded from
// memory and the matrix chosen at run time (one copy of this rare path's code: the kernel's common
// path uses every register).  ROWB: the row vector is b with the
// exclusive gate G_{r-1}, else q with G_r; COLA: the column vector is a, else k.  For a second-half
// row token the level's anchor token is at or before r - 1, so e^{G_{r-1} - a} and e^{G_r - a} are
// both <= 1.  Returns the accumulator layout (rows r = 4*q4 + j, column i = l16) of the strictly
// lower part plus, for q rows, the diagonal (factor 1).  q, k, a, b, g point at the lane's token row
// (channels 4*q4 ...: tile ct at + 16 ct); valid is false past the chunk end.
template <typename IO>
__device__ __forceinline__ f32x4 dplr_diag_split(const IO *q, const IO *k, const IO *a, const IO *b, const float *g,
                                                 bool valid, int KT, int l16, int q4, int lane, bool ROWB, bool COLA) {
    using Tr = IoTraits<IO>;
    constexpr bool BF = Tr::kBf16;
    f32x4 acc = zero4();
    float d = 0.f;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 1
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int hs = 8 >> lvl;
        const bool sec = (l16 & hs) != 0;
        const int src = (lane & ~15) | ((l16 & ~(2 * hs - 1)) + hs - 1);  // the level's anchor token
        f32x4 t = zero4();
#pragma unroll 1
        for (int ct = 0; ct < KT; ++ct) {
            const float4 rv = valid ? Tr::load4((ROWB ? b : q) + 16 * ct) : z;
            const float4 cv = valid ? Tr::load4((COLA ? a : k) + 16 * ct) : z;
            const float4 gr = valid ? *reinterpret_cast<const float4 *>(g + 16 * ct) : z;
            const float G[4] = {scan16_add(gr.x * kLog2e), scan16_add(gr.y * kLog2e), scan16_add(gr.z * kLog2e),
                                scan16_add(gr.w * kLog2e)};
            const float gx[4] = {gr.x, gr.y, gr.z, gr.w};
            const float rx[4] = {rv.x, rv.y, rv.z, rv.w}, cx[4] = {cv.x, cv.y, cv.z, cv.w};
            float ro[4], co[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float an = __shfl(G[j], src);
                const float Gr = ROWB ? G[j] - gx[j] * kLog2e : G[j];
                ro[j] = sec ? rx[j] * fast_exp2(fminf(Gr - an, 0.f)) : 0.f;     // e^{G_{r(-1)} - a}
                co[j] = sec ? 0.f : cx[j] * fast_exp2(fminf(an - G[j], 0.f));  // e^{a - G_i}
                if (!ROWB && lvl == 0) d += rx[j] * cx[j];
            }
            mma16(t, make_frag<BF>(ro[0], ro[1], ro[2], ro[3]), make_frag<BF>(co[0], co[1], co[2], co[3]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += ((4 * q4 + j) >> (4 - lvl)) == (l16 >> (4 - lvl)) ? t[j] : 0.f;
    }
    if (!ROWB) {  // diagonal of the q rows: q_r . (a_r or k_r) of the lane's token
        d += __shfl_xor(d, 16);
        d += __shfl_xor(d, 32);
        if (q4 == (l16 >> 2)) {  // entry [r = l16][i = l16] sits at j = l16 % 4
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += (l16 & 3) == j ? d : 0.f;
        }
    }
    return acc;
}

template <typename IO, int DK, int DVT, int C>
__global__ void __launch_bounds__(kChunkThreads) kda_dplr_fwd_kernel(DplrParams dp) {
    using L = DplrLayout<IO, DK, DVT, C>;
    using OT = typename L::OT;
    using KQ = typename DplrRaw<IO, DK, DVT, C>::KQ;
    constexpr bool BF = L::BF;
    constexpr int NSUB = L::NSUB, KT = L::KT, NSL = L::NSL, SPW = L::SPW;
    constexpr int LDO = L::LDO, LDT = L::LDT, LDM = L::LDM, LDD = L::LDD, LDV = L::LDV;
    using Tr = IoTraits<IO>;
    const FwdParams &p = dp.f;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OT *sAb = reinterpret_cast<OT *>(smem + L::oAb);
    OT *sKb = reinterpret_cast<OT *>(smem + L::oKb);
    OT *sQt = reinterpret_cast<OT *>(smem + L::oQt);
    OT *sBt = reinterpret_cast<OT *>(smem + L::oBt);
    OT *sAbT = reinterpret_cast<OT *>(smem + L::oAbT);
    OT *sKbT = reinterpret_cast<OT *>(smem + L::oKbT);
    OT *sMba = reinterpret_cast<OT *>(smem + L::oMba);
    OT *sMbk = reinterpret_cast<OT *>(smem + L::oMbk);
    OT *sMqa = reinterpret_cast<OT *>(smem + L::oMqa);
    OT *sMqk = reinterpret_cast<OT *>(smem + L::oMqk);
    float *sAd = reinterpret_cast<float *>(smem + L::oAd);
    OT *sV = reinterpret_cast<OT *>(smem + L::oV);
    float *sTot = reinterpret_cast<float *>(smem + L::oTot);
    float *sEB = reinterpret_cast<float *>(smem + L::oEB);
    float *sED = reinterpret_cast<float *>(smem + L::oED);
    float *sEC = reinterpret_cast<float *>(smem + L::oEC);
    float *sSH = reinterpret_cast<float *>(smem + L::oSH);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    IO *__restrict__ O = static_cast<IO *>(p.out);
    const int H = p.H, DV = p.dv;

    const int ntile = DV / DVT;
    const int64_t nblocks = (int64_t)p.num_seqs * H * ntile;
    const int64_t item = xcd_grouped_block(blockIdx.x, nblocks);
    const int tile = (int)(item % ntile);
    const int64_t nh = item / ntile;
    const int h = (int)(nh % H);
    const int n = (int)(nh / H);
    int64_t start;
    int len;
    if (p.cu) {
        start = p.cu[n];
        len = p.cu[n + 1] - p.cu[n];
    } else {
        start = (int64_t)n * p.T;
        len = p.T;
    }
    const int col0 = tile * DVT;

    f32x4 S[SPW][KT];
    const int64_t state_base = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int sl = wave + L::NW * s;
        const int col = col0 + 16 * sl + l16;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ct + 4 * q4 + j;
                S[s][ct][j] = (p.s0 && sl < NSL) ? p.s0[state_base + (int64_t)row * DV + col] : 0.f;
            }
    }
    __builtin_amdgcn_s_waitcnt(0);

    DplrRaw<IO, DK, DVT, C> raw;
    if (len > 0) dplr_load_chunk<IO, DK, DVT, C>(raw, dp, start, min(C, len), h, col0, tid);

    for (int c0 = 0; c0 < len; c0 += C) {
        const int clen = min(C, len - c0);
        const int64_t tok0 = start + c0;

        // ================= 1: gate scan (log2), stage V
        float G[KT][4];
        const bool valid = 16 * wave + l16 < clen;
        bool split = false;  // the sub-chunk decays too strongly for a single-anchor diagonal block
        if (wave < NSUB) {
            const int R = wave;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const int c = 16 * ct + 4 * q4;
                const float m = valid ? kLog2e : 0.f;
                G[ct][0] = scan16_add(raw.g[ct].x * m);
                G[ct][1] = scan16_add(raw.g[ct].y * m);
                G[ct][2] = scan16_add(raw.g[ct].z * m);
                G[ct][3] = scan16_add(raw.g[ct].w * m);
                if (l16 == 15)
                    *reinterpret_cast<float4 *>(sTot + R * DK + c) = make_float4(G[ct][0], G[ct][1], G[ct][2], G[ct][3]);
            }
            split = diag_needs_split<KT>(G);
        }
        {
            constexpr int PPR = DVT / L::V_ELEMS;
#pragma unroll
            for (int i = 0; i < L::V_PER_THREAD; ++i) {
                const int piece = tid + kChunkThreads * i;
                if (L::V_PIECES % kChunkThreads == 0 || piece < L::V_PIECES) {
                    const int r = piece / PPR;
                    const int cc = (piece % PPR) * L::V_ELEMS;
                    *reinterpret_cast<uint4 *>(sV + r * LDV + cc) = r < clen ? raw.v[i] : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
        if (split) {
            // Decay beyond 2^-96 inside the sub-chunk: the diagonal blocks from the split levels (all
            // factors <= 1), written to their LDS places here; phase 4a discards its own products.
            const int R = wave;
            const int64_t row = ((tok0 + min(16 * R + l16, clen - 1)) * H + h) * (int64_t)DK + 4 * q4;
            const IO *qp = static_cast<const IO *>(p.q) + row, *kp = static_cast<const IO *>(p.k) + row;
            const IO *ap = static_cast<const IO *>(dp.a) + row, *bp = static_cast<const IO *>(dp.b) + row;
            const float *gp = p.g + row;
            // matrices 0..3: M_ba (fp32 to sAd for the inverse), M_bk, M_qa, M_qk
#pragma unroll 1
            for (int mi = 0; mi < 4; ++mi) {
                const bool rowb = mi < 2, cola = (mi & 1) == 0;
                const f32x4 v = dplr_diag_split<IO>(qp, kp, ap, bp, gp, valid, KT, l16, q4, lane, rowb, cola);
                OT *m = mi == 1 ? sMbk : mi == 2 ? sMqa : sMqk;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * q4 + j;
                    const float x = (rowb ? l16 < rr : l16 <= rr) ? v[j] : 0.f;
                    if (mi == 0) {
                        sAd[(R * 16 + rr) * LDD + l16] = x;
                    } else {
                        if constexpr (BF) m[(16 * R + rr) * LDM + 16 * R + l16] = f32_to_bf16(x);
                        else m[(16 * R + rr) * LDM + 16 * R + l16] = x;
                    }
                }
            }
        }
        __syncthreads();

        // ================= 2: per-channel boundary factors
        if (tid < DK) {
            const int c = tid;
            float tot[NSUB], bnd[NSUB + 1];
            bnd[0] = 0.f;
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                tot[R] = sTot[R * DK + c];
                bnd[R + 1] = bnd[R] + tot[R];
            }
            const float gc = bnd[NSUB];
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                sEB[R * DK + c] = fast_exp2(bnd[R]);
                sED[R * DK + c] = fast_exp2(-tot[R]);
                sEC[R * DK + c] = fast_exp2(gc - bnd[R + 1]);
#pragma unroll
                for (int I = 0; I + 2 <= R; ++I) sSH[L::shift_slot(R, I) * DK + c] = fast_exp2(bnd[R] - bnd[I + 1]);
            }
            sGam[c] = fast_exp2(gc);
        }
        __syncthreads();

        // ================= 3: column operands of sub-chunk R: a, k * e^{b_{R+1} - G} (<= 1)
        Frag<BF> adiag[KT], kdiag[KT];  // a, k * e^{b_R - G} (>= 1): the diagonal block's columns
        if (wave < NSUB) {
            const int R = wave;
            const int r = 16 * R + l16;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const int c = 16 * ct + 4 * q4;
                const float4 tot = *reinterpret_cast<const float4 *>(sTot + R * DK + c);
                const float4 ed = *reinterpret_cast<const float4 *>(sED + R * DK + c);
                const float tv[4] = {tot.x, tot.y, tot.z, tot.w};
                const float edv[4] = {ed.x, ed.y, ed.z, ed.w};
                const float4 av = dplr_unpack<KQ, BF>(raw.a[ct]), kv = dplr_unpack<KQ, BF>(raw.k[ct]);
                const float ax[4] = {av.x, av.y, av.z, av.w}, kx[4] = {kv.x, kv.y, kv.z, kv.w};
                float ab[4], kb[4], ad[4], kd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fb = valid ? fast_exp2(tv[j] - G[ct][j]) : 0.f;
                    ab[j] = ax[j] * fb;
                    kb[j] = kx[j] * fb;
                    ad[j] = ab[j] * edv[j];
                    kd[j] = kb[j] * edv[j];
                }
                adiag[ct] = make_frag<BF>(ad[0], ad[1], ad[2], ad[3]);
                kdiag[ct] = make_frag<BF>(kd[0], kd[1], kd[2], kd[3]);
                const Frag<BF> fa = make_frag<BF>(ab[0], ab[1], ab[2], ab[3]);
                const Frag<BF> fk = make_frag<BF>(kb[0], kb[1], kb[2], kb[3]);
                *reinterpret_cast<decltype(fa.v) *>(sAb + r * LDO + c) = fa.v;
                *reinterpret_cast<decltype(fk.v) *>(sKb + r * LDO + c) = fk.v;
            }
        }
        __syncthreads();

        // ================= 4a: row-R blocks of the four chunk matrices; diagonal inverse
        if (wave < NSUB) {
            const int R = wave;
            // row operands: q e^{G_r - b_R}, b e^{G_{r-1} - b_R} (both <= 1)
            float qrow[KT][4], brow[KT][4];
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const float4 qv = dplr_unpack<KQ, BF>(raw.q[ct]), bv = dplr_unpack<KQ, BF>(raw.b[ct]);
                const float qx[4] = {qv.x, qv.y, qv.z, qv.w}, bx[4] = {bv.x, bv.y, bv.z, bv.w};
                const float gx[4] = {raw.g[ct].x, raw.g[ct].y, raw.g[ct].z, raw.g[ct].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    qrow[ct][j] = valid ? qx[j] * fast_exp2(G[ct][j]) : 0.f;
                    brow[ct][j] = valid ? bx[j] * fast_exp2(G[ct][j] - gx[j] * kLog2e) : 0.f;
                }
            }
#pragma unroll
            for (int I = 0; I < NSUB; ++I) {
                if (I > R) break;
                Frag<BF> qa[KT], ba[KT];
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) {
                    float4 sh = make_float4(1.f, 1.f, 1.f, 1.f);
                    if (I + 2 <= R) sh = *reinterpret_cast<const float4 *>(sSH + L::shift_slot(R, I) * DK + 16 * ct + 4 * q4);
                    qa[ct] = make_frag<BF>(qrow[ct][0] * sh.x, qrow[ct][1] * sh.y, qrow[ct][2] * sh.z, qrow[ct][3] * sh.w);
                    ba[ct] = make_frag<BF>(brow[ct][0] * sh.x, brow[ct][1] * sh.y, brow[ct][2] * sh.z, brow[ct][3] * sh.w);
                }
                f32x4 mba = zero4(), mbk = zero4(), mqa = zero4(), mqk = zero4();
                const OT *ca = sAb + (16 * I + l16) * LDO + 4 * q4;
                const OT *ck = sKb + (16 * I + l16) * LDO + 4 * q4;
#pragma unroll
                for (int ct = 0; ct < KT; ct += 2) {
                    Frag<BF> a0, a1, k0, k1;
                    if (I == R) {
                        a0 = adiag[ct];
                        a1 = adiag[ct + 1];
                        k0 = kdiag[ct];
                        k1 = kdiag[ct + 1];
                    } else {
                        a0 = lds_frag(ca + 16 * ct);
                        a1 = lds_frag(ca + 16 * ct + 16);
                        k0 = lds_frag(ck + 16 * ct);
                        k1 = lds_frag(ck + 16 * ct + 16);
                    }
                    mma32(mba, ba[ct], ba[ct + 1], a0, a1);
                    mma32(mbk, ba[ct], ba[ct + 1], k0, k1);
                    mma32(mqa, qa[ct], qa[ct + 1], a0, a1);
                    mma32(mqk, qa[ct], qa[ct + 1], k0, k1);
                }
                // accumulator: rows rr = 4 q4 + j of block R, column ii = l16 of block I (with `split`
                // the diagonal block was written in phase 1 and this product is discarded)
                if (!(I == R && split))
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * q4 + j, ii = l16;
                    float vba = mba[j], vbk = mbk[j], vqa = mqa[j], vqk = mqk[j];
                    if (I == R) {
                        if (ii >= rr) vba = vbk = 0.f;
                        if (ii > rr) vqa = vqk = 0.f;
                    }
                    const int e = (16 * R + rr) * LDM + 16 * I + l16;
                    if constexpr (BF) {
                        sMbk[e] = f32_to_bf16(vbk);
                        sMqa[e] = f32_to_bf16(vqa);
                        sMqk[e] = f32_to_bf16(vqk);
                        if (I != R) sMba[e] = f32_to_bf16(vba);
                    } else {
                        sMbk[e] = vbk;
                        sMqa[e] = vqa;
                        sMqk[e] = vqk;
                        if (I != R) sMba[e] = vba;
                    }
                    if (I == R) sAd[(R * 16 + rr) * LDD + l16] = vba;
                }
            }
            // X_RR = (I - M_ba,RR)^{-1}: lane l16 computes column l16 by forward substitution
            wave_lds_sync();  // this wave's lanes wrote the block
            float *Ab = sAd + R * 16 * LDD;
            const int jc = l16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == jc) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s += Ab[r * LDD + m] * x[m];
                x[r] = s;
            }
            if (q4 == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Ab[r * LDD + jc] = x[r];
            }
        }
        __syncthreads();  // the column operands are dead from here on

        // ================= 4b: inter-chunk operands Q~, B~ (rows), A-^T, K-^T (columns)
        if (wave < NSUB) {
            const int R = wave;
            const int r = 16 * R + l16;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const int c = 16 * ct + 4 * q4;
                const float4 tot = *reinterpret_cast<const float4 *>(sTot + R * DK + c);
                const float4 eb = *reinterpret_cast<const float4 *>(sEB + R * DK + c);
                const float4 ec = *reinterpret_cast<const float4 *>(sEC + R * DK + c);
                const float tv[4] = {tot.x, tot.y, tot.z, tot.w};
                const float ebv[4] = {eb.x, eb.y, eb.z, eb.w};
                const float ecv[4] = {ec.x, ec.y, ec.z, ec.w};
                const float4 qv = dplr_unpack<KQ, BF>(raw.q[ct]), bv = dplr_unpack<KQ, BF>(raw.b[ct]);
                const float4 av = dplr_unpack<KQ, BF>(raw.a[ct]), kv = dplr_unpack<KQ, BF>(raw.k[ct]);
                const float qx[4] = {qv.x, qv.y, qv.z, qv.w}, bx[4] = {bv.x, bv.y, bv.z, bv.w};
                const float ax[4] = {av.x, av.y, av.z, av.w}, kx[4] = {kv.x, kv.y, kv.z, kv.w};
                const float gx[4] = {raw.g[ct].x, raw.g[ct].y, raw.g[ct].z, raw.g[ct].w};
                float qt[4], bt[4], abar[4], kbar[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fb = valid ? fast_exp2(tv[j] - G[ct][j]) * ecv[j] : 0.f;  // e^{G_C - G}
                    qt[j] = valid ? qx[j] * fast_exp2(G[ct][j]) * ebv[j] : 0.f;
                    bt[j] = valid ? bx[j] * fast_exp2(G[ct][j] - gx[j] * kLog2e) * ebv[j] : 0.f;
                    abar[j] = ax[j] * fb;
                    kbar[j] = kx[j] * fb;
                }
                const Frag<BF> fq = make_frag<BF>(qt[0], qt[1], qt[2], qt[3]);
                *reinterpret_cast<decltype(fq.v) *>(sQt + r * LDO + c) = fq.v;
                *reinterpret_cast<decltype(fq.v) *>(sBt + r * LDO + c) = make_frag<BF>(bt[0], bt[1], bt[2], bt[3]).v;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (BF) {
                        sAbT[(c + j) * LDT + r] = f32_to_bf16(abar[j]);
                        sKbT[(c + j) * LDT + r] = f32_to_bf16(kbar[j]);
                    } else {
                        sAbT[(c + j) * LDT + r] = abar[j];
                        sKbT[(c + j) * LDT + r] = kbar[j];
                    }
                }
            }
        }
        if (c0 + C < len) dplr_load_chunk<IO, DK, DVT, C>(raw, dp, tok0 + C, min(C, len - c0 - C), h, col0, tid);
        __syncthreads();

        // ================= 5: state slices
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int sl = wave + L::NW * s;
            if (sl >= NSL) break;
            const int col = col0 + 16 * sl + l16;
            Frag<BF> Sb[KT];
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) Sb[ct] = frag_from_acc<BF>(S[s][ct]);
            // V as B operands: rows 16I + 4q4 + j, column l16 of the slice
            Frag<BF> Vf[NSUB];
#pragma unroll
            for (int I = 0; I < NSUB; ++I) {
                float t[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const OT x = sV[(16 * I + 4 * q4 + j) * LDV + 16 * sl + l16];
                    if constexpr (BF) t[j] = bf16_to_f32(x);
                    else t[j] = x;
                }
                Vf[I] = make_frag<BF>(t[0], t[1], t[2], t[3]);
            }
            Frag<BF> Uf[NSUB];
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                // Y_R = B~_R S + sum_{I<=R} M_bk(R,I) V_I;  U_R = X_RR (Y_R + sum_{I<R} M_ba(R,I) U_I)
                f32x4 y = zero4(), o = zero4();
                const OT *bt = sBt + (16 * R + l16) * LDO + 4 * q4;
                const OT *qt = sQt + (16 * R + l16) * LDO + 4 * q4;
#pragma unroll
                for (int ct = 0; ct < KT; ct += 2) {
                    mma32(y, lds_frag(bt + 16 * ct), lds_frag(bt + 16 * ct + 16), Sb[ct], Sb[ct + 1]);
                    mma32(o, lds_frag(qt + 16 * ct), lds_frag(qt + 16 * ct + 16), Sb[ct], Sb[ct + 1]);
                }
                const int mrow = (16 * R + l16) * LDM + 4 * q4;
#pragma unroll
                for (int I = 0; I <= R; ++I) mma16(y, lds_frag(sMbk + mrow + 16 * I), Vf[I]);
#pragma unroll
                for (int I = 0; I < R; ++I) mma16(y, lds_frag(sMba + mrow + 16 * I), Uf[I]);
                f32x4 u = zero4();
                mma16(u, lds_frag_f32<BF>(sAd + (16 * R + l16) * LDD + 4 * q4), frag_from_acc<BF>(y));
                Uf[R] = frag_from_acc<BF>(u);
                // O_R = scale (Q~_R S + sum_{I<=R} M_qa(R,I) U_I + M_qk(R,I) V_I)
#pragma unroll
                for (int I = 0; I <= R; ++I) {
                    mma16(o, lds_frag(sMqa + mrow + 16 * I), Uf[I]);
                    mma16(o, lds_frag(sMqk + mrow + 16 * I), Vf[I]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * q4 + j;
                    if (O && r < clen) Tr::store1(O + ((tok0 + r) * H + h) * (int64_t)DV + col, o[j] * p.scale);
                }
            }
            // S <- Diag(e^{G_C}) S + A-^T U + K-^T V
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const float4 gm = *reinterpret_cast<const float4 *>(sGam + 16 * ct + 4 * q4);
                S[s][ct][0] *= gm.x;
                S[s][ct][1] *= gm.y;
                S[s][ct][2] *= gm.z;
                S[s][ct][3] *= gm.w;
                const OT *ab = sAbT + (16 * ct + l16) * LDT + 4 * q4;
                const OT *kb = sKbT + (16 * ct + l16) * LDT + 4 * q4;
#pragma unroll
                for (int I = 0; I + 1 < NSUB; I += 2) {
                    mma32(S[s][ct], lds_frag(ab + 16 * I), lds_frag(ab + 16 * (I + 1)), Uf[I], Uf[I + 1]);
                    mma32(S[s][ct], lds_frag(kb + 16 * I), lds_frag(kb + 16 * (I + 1)), Vf[I], Vf[I + 1]);
                }
                if constexpr (NSUB % 2 == 1) {
                    mma16(S[s][ct], lds_frag(ab + 16 * (NSUB - 1)), Uf[NSUB - 1]);
                    mma16(S[s][ct], lds_frag(kb + 16 * (NSUB - 1)), Vf[NSUB - 1]);
                }
            }
        }
        __syncthreads();
    }

    if (p.sf) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int sl = wave + L::NW * s;
            if (sl >= NSL) break;
            const int col = col0 + 16 * sl + l16;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) p.sf[state_base + (int64_t)(16 * ct + 4 * q4 + j) * DV + col] = S[s][ct][j];
        }
    }
}

template <typename IO, int DK, int DVT, int C>
hipError_t launch_dplr_variant(const DplrParams &dp, hipStream_t stream) {
    if constexpr (!DplrLayout<IO, DK, DVT, C>::kFits) {
        return hipErrorInvalidConfiguration;
    } else {
        const int64_t blocks = (int64_t)dp.f.num_seqs * dp.f.H * (dp.f.dv / DVT);
        if (blocks <= 0) return hipSuccess;
        hipLaunchKernelGGL((kda_dplr_fwd_kernel<IO, DK, DVT, C>), dim3((unsigned)blocks), dim3(kChunkThreads), 0,
                           stream, dp);
        return hipGetLastError();
    }
}

#define KDA_DPLR_VARIANTS(F) \
    F(64, 32, 16) F(64, 32, 32) F(64, 32, 64) F(128, 32, 16) F(128, 32, 32) F(128, 32, 64) \
    F(64, 64, 64) F(128, 64, 64)

template <typename IO>
bool dplr_supported(int dk, int dvt, int chunk) {
#define KDA_DPLR_FIT(DK_, DVT_, C_) \
    if (dk == DK_ && dvt == DVT_ && chunk == C_) return DplrLayout<IO, DK_, DVT_, C_>::kFits;
    KDA_DPLR_VARIANTS(KDA_DPLR_FIT)
#undef KDA_DPLR_FIT
    return false;
}

template <typename IO>
hipError_t launch_dplr(const DplrParams &dp, int dvt, int chunk, hipStream_t stream) {
#define KDA_DPLR_CASE(DK_, DVT_, C_) \
    if (dp.f.dk == DK_ && dvt == DVT_ && chunk == C_) return launch_dplr_variant<IO, DK_, DVT_, C_>(dp, stream);
    KDA_DPLR_VARIANTS(KDA_DPLR_CASE)
#undef KDA_DPLR_CASE
    return hipErrorInvalidConfiguration;
}

}  // namespace kda
