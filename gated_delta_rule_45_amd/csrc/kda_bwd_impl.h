// Chunkwise KDA backward for gfx950.
//
// Gradients of L = <dO, O> + <dS_final, S_T> with respect to q, k, v, g, beta and the
// initial state, by reverse-mode differentiation of the chunk equations (Kimi Linear
// summary page, "Chunkwise parallel algorithm": chunk-level state passing, the WY/UT
// transform with one triangular inverse per chunk, and the inter/intra-chunk output
// split; the UT form exists for training throughput).  Per chunk, with its initial
// state S, D = X Diag(beta)(V - K~ S), X = (I + A)^{-1}, and dS the gradient of the
// state the chunk hands on:
//
//   dD = scale P^T dO + K- dS        dU = X^T dD        dY = beta * dU   (= dv)
//   dS <- Diag(e^{G_C}) dS + scale Q~^T dO - K~^T dY                      (reverse scan)
//
//   dP = scale lower_incl(dO D^T)    dA = -strictly_lower(dU D^T)    dL = beta * dA
//   dq_r = scale e^{G_r} (S dO_r) + sum_i dP_ri k_i e^{G_r - G_i}
//   dk_r = beta_r [ sum_i dA_ri k_i e^{G_r - G_i} - e^{G_r} (S dU_r) ]           (via K~)
//        + sum_r' (dP_r'r q_r' + dL_r'r k_r') e^{G_r' - G_r}                      (via K^)
//        + e^{G_C - G_r} (dS D_r)                                                 (via K-)
//   dG   = q dq + k (dk via K~) - k (dk via K^) - k (dk via K-), and at the chunk's last
//          token also sum_i k_i (dk_i via K-) + e^{G_C} rowsum(dS .* S);  dg = reverse
//          cumulative sum of dG over the chunk
//   dbeta_r = sum_j dU_rj V_rj - sum_c e^{G_rc} k_rc (S dU_r)_c + sum_c k_rc W_rc,
//          W_rc = sum_i dA_ri k_ic e^{G_rc - G_ic}
//
// Four launches:
//   1. kda_bwd_prep_kernel: one workgroup per (chunk, head), all chunks in parallel; builds
//      the chunk's gated operands, A^T, P^T and the diagonal blocks of X^T as one record, and
//      (two-pass forward) the forward's record of the chunk from the same operands: K~, K-^T,
//      T = X Diag(beta) and e^{G_C}, the same values the forward's prep kernel writes;
//   2. the forward again (its scan only on those records, or the fused kernel where no two-pass
//      variant exists, launched before the prep kernel) keeps each chunk's initial state S and D;
//   3. kda_bwd_scan_kernel: one workgroup per (sequence, head, d_v tile), chunks in
//      reverse order; streams the records, keeps dS in registers, writes dv, dU and the
//      chunk-end dS of every chunk, and d(initial state);
//   4. kda_bwd_grad_kernel: one workgroup per (chunk, head), all chunks in parallel;
//      each wave owns 16 key channels for every token of the chunk, so the gate
//      factors stay in registers and no cross-wave reduction over channels is needed
//      except for dbeta (a sum over channels).
//
// The exponentials e^{G_r - G_i} inside the C x C products are split at 16-token
// sub-chunk boundaries b_R (as in the forward): e^{G_r - G_i} = e^{G_r - b_R} *
// e^{b_R - b_{I+1}} * e^{b_{I+1} - G_i} for r in sub-chunk R >= I, i in I; the outer two
// factors are <= 1 and the middle one is a per-channel constant of the block pair.
#pragma once

#include <algorithm>
#include <type_traits>

#include "kda_chunk_impl.h"
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_split_record.h"

namespace kda {


__device__ __forceinline__ int64_t bwd_slot0(const FwdParams &p, int n, int C) {
    return p.cu ? (int64_t)p.chunk_off[n] : (int64_t)n * ((p.T + C - 1) / C);
}

// Sequence and chunk of a chunk slot (the inverse of bwd_slot0); false past the last chunk.
__device__ __forceinline__ bool bwd_slot_chunk(const FwdParams &p, int C, int64_t slot, int &n, int &ci) {
    if (p.cu) {
        if (slot >= p.chunk_off[p.num_seqs]) return false;
        int lo = 0, hi = p.num_seqs - 1;  // last n with chunk_off[n] <= slot
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.chunk_off[mid] <= slot) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        ci = (int)(slot - p.chunk_off[lo]);
        return true;
    }
    const int64_t per = (p.T + C - 1) / C;
    if (per == 0 || slot >= per * p.num_seqs) return false;
    n = (int)(slot / per);
    ci = (int)(slot % per);
    return true;
}

constexpr int kBwdScanTile = 32;  // d_v columns per reverse-scan workgroup (two 16-column compute waves)
constexpr int kBwdScanCopyWaves = 4;
constexpr int kBwdScanThreads = 64 * (kBwdScanTile / 16 + kBwdScanCopyWaves);

// ==================================================================== record ====
// Per-chunk operands of the reverse scan, built by kda_bwd_prep_kernel for every (chunk, head)
// in parallel and streamed by kda_bwd_scan_kernel.  With X = (I + A)^{-1} the chunk's part of
// the reverse chain is
//     dU = M dS + N (scale dO),        M = X^T K-,  N = X^T P^T,
//     dS <- Diag(e^{G_C}) dS + Q~^T (scale dO) - (Diag(beta) K~)^T dU,
// so the only products left in the sequential chain are against dS and dU.  The record holds
// M [C][DK], N [C][C], Q~^T and (Diag(beta) K~)^T [DK][C] (operand type), e^{G_C} [DK] and
// beta [C] (fp32).  It is stored exactly as the scan keeps it in LDS, every row padded by 16
// bytes so that the fragment reads spread over the banks, and the scan copies it verbatim; the
// size is rounded up to whole KB (the copy waves move 1 KB per wave instruction).  Padding bytes
// are not written.
template <typename IO, int DK, int C>
struct BwdRec {
    static constexpr bool BF = IoTraits<IO>::kBf16;
    using OT = typename std::conditional<BF, uint16_t, float>::type;
    static constexpr int S = (int)sizeof(OT);
    static constexpr int NSUB = C / 16, KT = DK / 16;
    static constexpr int PAD = 16 / S;
    static constexpr int LDO = DK + PAD;  // [C][DK] rows
    static constexpr int LDT = C + PAD;   // [DK][C] rows
    static constexpr int LDM = C + PAD;   // [C][C] rows
    static constexpr size_t oM = 0;
    static constexpr size_t oN = oM + (size_t)C * LDO * S;
    static constexpr size_t oQtT = oN + (size_t)C * LDM * S;
    static constexpr size_t oBKtT = oQtT + (size_t)DK * LDT * S;
    static constexpr size_t oGam = oBKtT + (size_t)DK * LDT * S;
    static constexpr size_t oBeta = oGam + (size_t)DK * 4;
    static constexpr size_t kUsed = oBeta + (size_t)C * 4;
    static constexpr size_t kBytes = (kUsed + 1023) / 1024 * 1024;
    static_assert(C % 16 == 0 && NSUB >= 1 && NSUB <= 4, "chunk must be 16, 32 or 64");
    static_assert(DK % 64 == 0, "d_k must be 64 or 128");
};

// ====================================================================== prep ====
// LDS of the prep kernel.  M and N are formed in LDS at their record offsets and copied out
// with e^{G_C} and beta; Q~^T and (Diag(beta) K~)^T go from registers straight to the record.
// The K_b rows take M's place (dead before M is formed), and the per-channel gate tables take
// X's place (dead before A is written there).
template <typename IO, int DK, int C>
struct BwdPrepLayout {
    using Rec = BwdRec<IO, DK, C>;
    using OT = typename Rec::OT;
    static constexpr bool BF = Rec::BF;
    static constexpr int S = Rec::S;
    static constexpr int NSUB = C / 16, KT = DK / 16;
    static constexpr int LDO = Rec::LDO, LDT = Rec::LDT, LDM = Rec::LDM;
    static constexpr int LDX = C + 4;  // fp32 [C][C]: A, then X in place
    static constexpr int NSHIFT = NSUB >= 3 ? (NSUB - 1) * (NSUB - 2) / 2 : 0;
    static constexpr size_t oKb = Rec::oM;
    static constexpr size_t oKbarT = Rec::oQtT;  // right after M and N
    static constexpr size_t kXBytes = (size_t)C * LDX * 4;
    static constexpr size_t kTabBytes = (size_t)4 * NSUB * DK * 4;  // Tot, EB, ED, EC
    static constexpr size_t oX = oKbarT + (size_t)DK * LDT * S;
    static constexpr size_t oTot = oX;
    static constexpr size_t oEB = oTot + (size_t)NSUB * DK * 4;
    static constexpr size_t oED = oEB + (size_t)NSUB * DK * 4;
    static constexpr size_t oEC = oED + (size_t)NSUB * DK * 4;
    static constexpr size_t oP = oX + (kXBytes > kTabBytes ? kXBytes : kTabBytes);
    static constexpr size_t oSH = oP + (size_t)C * LDM * S;
    static constexpr size_t oGam = oSH + (size_t)(NSHIFT > 0 ? NSHIFT : 1) * DK * 4;  // e^{G_C} then beta, as in the record
    static constexpr size_t oBeta = oGam + (size_t)DK * 4;
    static constexpr size_t kBytes = oBeta + (size_t)C * 4;
    static constexpr bool kFits = kBytes <= 160 * 1024;
    static_assert(Rec::oBeta == Rec::oGam + (size_t)DK * 4, "e^{G_C} and beta are one run in the record");

    __host__ __device__ static constexpr int shift_slot(int R, int I) { return (R - 2) * (R - 1) / 2 + I; }
};

// Raw key side of one chunk: q, k, g of sub-chunk R = wave, and beta.
template <typename IO, int DK>
struct BwdRaw {
    using KQ = typename std::conditional<IoTraits<IO>::kBf16, uint2, float4>::type;
    float4 g[DK / 16];
    KQ k[DK / 16], q[DK / 16];
    float beta;
};

template <typename IO, int DK, int C>
__device__ __forceinline__ void bwd_load_keys(BwdRaw<IO, DK> &raw, const FwdParams &p, int64_t tok0, int clen, int h,
                                              int tid) {
    using KQ = typename BwdRaw<IO, DK>::KQ;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    if (wave < C / 16) {
        const int r = min(16 * wave + l16, clen - 1);
        const int64_t row = ((tok0 + r) * p.H + h) * (int64_t)DK + 4 * q4;
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct) {
            raw.g[ct] = *reinterpret_cast<const float4 *>(p.g + row + 16 * ct);
            raw.k[ct] = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.k) + row + 16 * ct);
            raw.q[ct] = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.q) + row + 16 * ct);
        }
    }
    if (tid < C) raw.beta = p.beta[(tok0 + min(tid, clen - 1)) * p.H + h];
}

// X_IR (I >= R) as a B operand: rows 4*q4 + j, column l16.  X is kept with its diagonal blocks
// in place and the blocks below the diagonal transposed in the unused upper blocks:
// X_IR[a][b] at sX[(16R + b) * LDX + 16I + a] for I > R.
template <bool BF, int LDX>
__device__ __forceinline__ Frag<BF> bwd_x_frag(const float *sX, int I, int R, int l16, int q4) {
    float4 x;
    if (I == R) {
        const float *d = sX + (16 * R + 4 * q4) * LDX + 16 * R + l16;
        x = make_float4(d[0], d[LDX], d[2 * LDX], d[3 * LDX]);
    } else {
        x = *reinterpret_cast<const float4 *>(sX + (16 * R + l16) * LDX + 16 * I + 4 * q4);
    }
    return make_frag<BF>(x.x, x.y, x.z, x.w);
}

// A 16x16 tile given as an A operand (row l16, columns 4*q4 + j) turned into the accumulator
// layout (rows 4*q4 + j, column l16), i.e. each lane then holds 4 consecutive rows of one column:
// an exact product with the identity.
template <bool BF>
__device__ __forceinline__ Frag<BF> bwd_turn(const Frag<BF> &a, const Frag<BF> &eye) {
    f32x4 t = zero4();
    mma16(t, a, eye);
    return frag_from_acc<BF>(t);
}

// Diagonal-block terms of one sub-chunk for the gradient kernel, exact under any decay: the split
// levels of kda_device.h (split_anchor), here in products that contract over the tokens.  The lane
// holds token l16 of the sub-chunk and channels 4*q4 + j of its wave's 16: raw k and q (kk, qq) and
// the in-sub-chunk cumulative log2 gate G.  P, A (rows r) and PT, LT (rows i) point at the
// sub-chunk's diagonal 16 x 16 tiles of dP, dA, dP^T and dL^T (row stride LDC); without TRANS
// there are no transposed tiles and the column side gathers dP^T and dL^T = (beta_r dA)^T from
// the columns of P and A, with beta the sub-chunk's 16 betas:
//   ROW: rowP[j] += sum_{i <= r} k_i dP_ri e^{G_r - G_i},  rowA[j] += sum_{i < r} k_i dA_ri e^{G_r - G_i}
//        (r the lane's token)
//   COL: col[j]  += sum_{r >= i} (q_r dP_ri + k_r dL_ri) e^{G_r - G_i}  (i the lane's token)
// Per level, the tiles are masked to the pairs with both tokens in one block, the row-side token in
// its second half and the column-side token in its first half, and the token operands carry
// e^{-|G - a|} <= 1 (a the level's anchor); the diagonal pairs (factor 1) are added apart.
template <bool BF, bool ROW, bool COL, bool TRANS, typename OT>
__device__ __forceinline__ void grad_diag_split(f32x4 &rowP, f32x4 &rowA, f32x4 &col, const float (&kk)[4],
                                                const float (&qq)[4], const float (&G)[4], const OT *P, const OT *A,
                                                const OT *PT, const OT *LT, const float *beta, int LDC,
                                                const Frag<BF> &eye, int l16, int q4, int lane) {
    // the level loop stays rolled (anchors by lane shuffle): the common path of this kernel uses
    // every register, and an unrolled rare path would add code and temporaries to it
#pragma unroll 1
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int hs = 8 >> lvl;
        const int src = (lane & ~15) | ((l16 & ~(2 * hs - 1)) + hs - 1);  // the level's anchor token
        float f[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = fast_exp2(-fabsf(G[j] - __shfl(G[j], src)));
        // B fragment of tokens x = 4*q4 + j (contracted) against the lane's token l16: keep x where
        // both lie in one block and the lane's token is in the half `lane_second`, x in the other
        auto masked_vals = [&](const float (&x)[4], bool lane_second) {
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tx = 4 * q4 + j;
                const bool same = (tx >> (4 - lvl)) == (l16 >> (4 - lvl));
                const bool lane_sec = (l16 & hs) != 0, x_sec = (tx & hs) != 0;
                o[j] = (same && lane_sec == lane_second && x_sec != lane_second) ? x[j] : 0.f;
            }
            return make_frag<BF>(o[0], o[1], o[2], o[3]);
        };
        auto masked = [&](const OT *t, bool lane_second) {  // rows of t: tile element [l16][4 q4 + j]
            const float4 v = unpack4<BF>(lds_frag(t + l16 * LDC + 4 * q4).v);
            const float x[4] = {v.x, v.y, v.z, v.w};
            return masked_vals(x, lane_second);
        };
        // the transposed tiles' element [l16][4 q4 + j] from the columns of P and A
        auto masked_pt = [&](bool lane_second) {
            if constexpr (TRANS) {
                return masked(PT, lane_second);
            } else {
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = elem_f32(P[(4 * q4 + j) * LDC + l16]);
                return masked_vals(x, lane_second);
            }
        };
        auto masked_lt = [&](bool lane_second) {
            if constexpr (TRANS) {
                return masked(LT, lane_second);
            } else {
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = beta[4 * q4 + j] * elem_f32(A[(4 * q4 + j) * LDC + l16]);
                return masked_vals(x, lane_second);
            }
        };
        const Frag<BF> kT = bwd_turn<BF>(make_frag<BF>(kk[0] * f[0], kk[1] * f[1], kk[2] * f[2], kk[3] * f[3]), eye);
        if constexpr (ROW) {
            f32x4 tp = zero4(), ta = zero4();
            mma16(tp, kT, masked(P, true));
            mma16(ta, kT, masked(A, true));
            mfma_settle(tp, ta);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rowP[j] += f[j] * tp[j];
                rowA[j] += f[j] * ta[j];
            }
        }
        if constexpr (COL) {
            const Frag<BF> qT =
                bwd_turn<BF>(make_frag<BF>(qq[0] * f[0], qq[1] * f[1], qq[2] * f[2], qq[3] * f[3]), eye);
            f32x4 tc = zero4();
            mma16(tc, qT, masked_pt(false));
            mma16(tc, kT, masked_lt(false));
            mfma_settle(tc);
#pragma unroll
            for (int j = 0; j < 4; ++j) col[j] += f[j] * tc[j];
        }
    }
    // diagonal pairs: dP_rr (dA and dL are strictly lower)
    OT d = P[l16 * LDC + l16];
    float dpp;
    if constexpr (BF) dpp = bf16_to_f32(d);
    else dpp = d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (ROW) rowP[j] += kk[j] * dpp;
        if constexpr (COL) col[j] += qq[j] * dpp;
    }
}

template <typename IO, int DK, int C>
__global__ void __launch_bounds__(kChunkThreads) kda_bwd_prep_kernel(BwdParams bp, char *__restrict__ records) {
    using L = BwdPrepLayout<IO, DK, C>;
    using Rec = typename L::Rec;
    using OT = typename L::OT;
    constexpr bool BF = L::BF;
    constexpr int NSUB = L::NSUB, KT = L::KT;
    constexpr int LDO = L::LDO, LDT = L::LDT, LDM = L::LDM, LDX = L::LDX;
    static_assert(KT % 4 == 0 && NSUB <= 4, "four waves share the d_k tiles of M");
    const FwdParams &p = bp.f;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OT *sKb = reinterpret_cast<OT *>(smem + L::oKb);
    OT *sKbarT = reinterpret_cast<OT *>(smem + L::oKbarT);
    float *sX = reinterpret_cast<float *>(smem + L::oX);
    OT *sP = reinterpret_cast<OT *>(smem + L::oP);
    float *sTot = reinterpret_cast<float *>(smem + L::oTot);
    float *sEB = reinterpret_cast<float *>(smem + L::oEB);
    float *sED = reinterpret_cast<float *>(smem + L::oED);
    float *sEC = reinterpret_cast<float *>(smem + L::oEC);
    float *sSH = reinterpret_cast<float *>(smem + L::oSH);
    OT *sM = reinterpret_cast<OT *>(smem + Rec::oM);
    OT *sN = reinterpret_cast<OT *>(smem + Rec::oN);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int H = p.H;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int n, ci;
    if (!bwd_slot_chunk(p, C, slot, n, ci)) return;
    const int64_t start = p.cu ? (int64_t)p.cu[n] : (int64_t)n * p.T;
    const int len = p.cu ? p.cu[n + 1] - p.cu[n] : p.T;
    const int clen = min(C, len - ci * C);
    char *rec = records + (size_t)(slot * H + h) * Rec::kBytes;
    // the forward's record of this chunk (BwdParams::frec): written alongside, from the same operands
    using FRec = SplitRecord<IO, DK, C>;
    char *frec = bp.frec ? bp.frec + (size_t)(slot * H + h) * FRec::kBytes : nullptr;

    BwdRaw<IO, DK> raw;
    bwd_load_keys<IO, DK, C>(raw, p, start + (int64_t)ci * C, clen, h, tid);
    const Frag<BF> eye = make_frag<BF>(4 * q4 == l16 ? 1.f : 0.f, 4 * q4 + 1 == l16 ? 1.f : 0.f,
                                       4 * q4 + 2 == l16 ? 1.f : 0.f, 4 * q4 + 3 == l16 ? 1.f : 0.f);

    // ================= 1: gate scan (log2 domain), stage beta
    // (k and q stay packed in the raw registers; phases 3 and 4 unpack them where used)
    float G[KT][4];
    const bool valid = 16 * wave + l16 < clen;
    bool split = false;  // the sub-chunk decays too strongly for a single-anchor diagonal block
    if (wave < NSUB) {
        const int R = wave;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            const int c = 16 * ct + 4 * q4;
            const float4 gv = raw.g[ct];
            const float m = valid ? kLog2e : 0.f;
            G[ct][0] = scan16_add(gv.x * m);
            G[ct][1] = scan16_add(gv.y * m);
            G[ct][2] = scan16_add(gv.z * m);
            G[ct][3] = scan16_add(gv.w * m);
            if (l16 == 15)
                *reinterpret_cast<float4 *>(sTot + R * DK + c) = make_float4(G[ct][0], G[ct][1], G[ct][2], G[ct][3]);
        }
        split = diag_needs_split<KT>(G);
    }
    if (tid < C) sBeta[tid] = tid < clen ? raw.beta : 0.f;
    // the gradient kernel handles this chunk in its split-capable instantiation when any sub-chunk
    // needs the split levels
    const int any_split = __syncthreads_or(split ? 1 : 0);
    if (tid == 0) bp.split_flag[slot * H + h] = any_split;

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
        const float gam = fast_exp2(gc);
        sGam[c] = gam;
        if (frec) reinterpret_cast<float *>(frec + FRec::oGam)[c] = gam;
    }
    __syncthreads();

    // ================= 3: gated operands of sub-chunk R: K_b rows, and K-^T, Q~^T,
    // (Diag(beta) K~)^T turned through the identity so that a lane holds 4 consecutive tokens of
    // one channel (8-byte pieces of their [DK][C] rows: K-^T to LDS, the other two to the record)
    Frag<BF> kdiag[KT];
    if (wave < NSUB) {
        const int R = wave;
        const float br = sBeta[16 * R + l16];
        OT *rq = reinterpret_cast<OT *>(rec + Rec::oQtT);
        OT *rk = reinterpret_cast<OT *>(rec + Rec::oBKtT);
        Frag<BF> fk_even;  // forward record: the even channel tile's K~ fragment, stored with the odd one's
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            const int c = 16 * ct + 4 * q4;
            const float4 tot = *reinterpret_cast<const float4 *>(sTot + R * DK + c);
            const float4 eb = *reinterpret_cast<const float4 *>(sEB + R * DK + c);
            const float4 ed = *reinterpret_cast<const float4 *>(sED + R * DK + c);
            const float4 ec = *reinterpret_cast<const float4 *>(sEC + R * DK + c);
            const float tv[4] = {tot.x, tot.y, tot.z, tot.w};
            const float ebv[4] = {eb.x, eb.y, eb.z, eb.w};
            const float edv[4] = {ed.x, ed.y, ed.z, ed.w};
            const float ecv[4] = {ec.x, ec.y, ec.z, ec.w};
            const float4 kv = unpack4<BF>(raw.k[ct]), qv = unpack4<BF>(raw.q[ct]);
            const float kx[4] = {kv.x, kv.y, kv.z, kv.w}, qx[4] = {qv.x, qv.y, qv.z, qv.w};
            float kb[4], kt[4], qt[4], kbar[4], kd[4], kf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fr = valid ? fast_exp2(G[ct][j]) : 0.f;
                const float fb = valid ? fast_exp2(tv[j] - G[ct][j]) : 0.f;
                kb[j] = kx[j] * fb;
                kd[j] = kb[j] * edv[j];
                kf[j] = kx[j] * fr * ebv[j];  // the forward's K~
                kt[j] = kf[j] * br;
                qt[j] = qx[j] * fr * ebv[j];
                kbar[j] = kb[j] * ecv[j];
            }
            kdiag[ct] = make_frag<BF>(kd[0], kd[1], kd[2], kd[3]);
            const Frag<BF> fkb = make_frag<BF>(kb[0], kb[1], kb[2], kb[3]);
            *reinterpret_cast<decltype(fkb.v) *>(sKb + (16 * R + l16) * LDO + c) = fkb.v;
            // turned: lane holds tokens 16R + 4q4 .. +3 of channel 16ct + l16
            const int64_t toff = (int64_t)(16 * ct + l16) * LDT + 16 * R + 4 * q4;
            const Frag<BF> tb = bwd_turn<BF>(make_frag<BF>(kbar[0], kbar[1], kbar[2], kbar[3]), eye);
            *reinterpret_cast<decltype(tb.v) *>(sKbarT + toff) = tb.v;
            const Frag<BF> tq = bwd_turn<BF>(make_frag<BF>(qt[0], qt[1], qt[2], qt[3]), eye);
            *reinterpret_cast<decltype(tq.v) *>(rq + toff) = tq.v;
            const Frag<BF> tk = bwd_turn<BF>(make_frag<BF>(kt[0], kt[1], kt[2], kt[3]), eye);
            *reinterpret_cast<decltype(tk.v) *>(rk + toff) = tk.v;
            if (frec) {
                // K~ in 16 x 32 operand tiles (row tile R, channel tile pair ct / 2); K-^T: the turned
                // fragment is this sub-chunk's half of operand tile (ct, R / 2)
                const Frag<BF> fk = make_frag<BF>(kf[0], kf[1], kf[2], kf[3]);
                if (ct % 2 == 0) fk_even = fk;
                else store_pair<BF>(frec + FRec::oKt + (size_t)(R * (KT / 2) + ct / 2) * FRec::TILE_BYTES, lane, fk_even, fk);
                *reinterpret_cast<decltype(tb.v) *>(frec + FRec::oKbT + ((size_t)ct * FRec::NPAIR + R / 2) * FRec::TILE_BYTES +
                                                    lane * FRec::PAIR_BYTES + (R % 2) * FRec::FRAG_BYTES) = tb.v;
            }
        }
        if (frec && NSUB % 2 == 1 && R == NSUB - 1) {  // odd sub-chunk count: the unused half of the last pair
            const Frag<BF> z = make_frag<BF>(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
                *reinterpret_cast<decltype(z.v) *>(frec + FRec::oKbT + ((size_t)ct * FRec::NPAIR + R / 2) * FRec::TILE_BYTES +
                                                   lane * FRec::PAIR_BYTES + FRec::FRAG_BYTES) = z.v;
        }
    }
    __syncthreads();

    // ================= 4: row-R blocks of A (fp32, to sX) and P (to sP, zero above the block
    // diagonal), then X_RR = (I + A_RR)^{-1} in place.  Block (R, I) pairs the row operands
    // k_r e^{G_r - b_R} (and the same for q) with the column operand K_b of sub-chunk I; for
    // I <= R - 2 the row operands take the extra factor e^{b_R - b_{I+1}} (all factors <= 1), and
    // for I = R the column operand is k_i e^{b_R - G_i}.
    if (wave < NSUB) {
        const int R = wave;
        float kr[KT][4], qr[KT][4];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            const float4 kv = unpack4<BF>(raw.k[ct]), qv = unpack4<BF>(raw.q[ct]);
            const float kx[4] = {kv.x, kv.y, kv.z, kv.w}, qx[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fr = valid ? fast_exp2(G[ct][j]) : 0.f;
                kr[ct][j] = kx[j] * fr;
                qr[ct][j] = qx[j] * fr;
            }
        }
#pragma unroll
        for (int I = 0; I < NSUB; ++I) {
            if (I > R) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sP[(16 * R + 4 * q4 + j) * LDM + 16 * I + l16] = OT(0);
                continue;
            }
            const OT *colp = sKb + (16 * I + l16) * LDO + 4 * q4;
            const float *shp = sSH + (I + 2 <= R ? L::shift_slot(R, I) : 0) * DK + 4 * q4;
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int ct = 0; ct < KT; ct += 2) {
                Frag<BF> b0, b1, ka0, ka1, qa0, qa1;
                if (I == R) {
                    b0 = kdiag[ct];
                    b1 = kdiag[ct + 1];
                } else {
                    b0 = lds_frag(colp + 16 * ct);
                    b1 = lds_frag(colp + 16 * (ct + 1));
                }
                if (I + 2 <= R) {
                    const float4 s0 = *reinterpret_cast<const float4 *>(shp + 16 * ct);
                    const float4 s1 = *reinterpret_cast<const float4 *>(shp + 16 * (ct + 1));
                    ka0 = make_frag<BF>(kr[ct][0] * s0.x, kr[ct][1] * s0.y, kr[ct][2] * s0.z, kr[ct][3] * s0.w);
                    ka1 = make_frag<BF>(kr[ct + 1][0] * s1.x, kr[ct + 1][1] * s1.y, kr[ct + 1][2] * s1.z,
                                        kr[ct + 1][3] * s1.w);
                    qa0 = make_frag<BF>(qr[ct][0] * s0.x, qr[ct][1] * s0.y, qr[ct][2] * s0.z, qr[ct][3] * s0.w);
                    qa1 = make_frag<BF>(qr[ct + 1][0] * s1.x, qr[ct + 1][1] * s1.y, qr[ct + 1][2] * s1.z,
                                        qr[ct + 1][3] * s1.w);
                } else {
                    ka0 = make_frag<BF>(kr[ct][0], kr[ct][1], kr[ct][2], kr[ct][3]);
                    ka1 = make_frag<BF>(kr[ct + 1][0], kr[ct + 1][1], kr[ct + 1][2], kr[ct + 1][3]);
                    qa0 = make_frag<BF>(qr[ct][0], qr[ct][1], qr[ct][2], qr[ct][3]);
                    qa1 = make_frag<BF>(qr[ct + 1][0], qr[ct + 1][1], qr[ct + 1][2], qr[ct + 1][3]);
                }
                mma32(accA, ka0, ka1, b0, b1);
                mma32(accP, qa0, qa1, b0, b1);
            }
            // accumulator: rows rr = 4*q4 + j of block R, column ii = l16 of block I
            if (I == R && split) {
                // Decay beyond 2^-96 inside the sub-chunk: the diagonal block from the split levels
                // (all factors <= 1), operands reloaded; this wave's product above is discarded.
                const int64_t tok0 = start + (int64_t)ci * C;
                const int64_t row = ((tok0 + min(16 * R + l16, clen - 1)) * H + h) * (int64_t)DK + 4 * q4;
                f32x4 dA, dPt;
                diag_block_split_rolled<IO>(dA, dPt, static_cast<const IO *>(p.k) + row,
                                            static_cast<const IO *>(p.q) + row, p.g + row, valid, KT, l16, q4, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * q4 + j;
                    sX[(16 * R + rr) * LDX + 16 * R + l16] = l16 < rr ? dA[j] * sBeta[16 * R + rr] : 0.f;
                    // dPt holds P_RR[l16][4 q4 + j]
                    if constexpr (BF) sP[(16 * R + l16) * LDM + 16 * R + rr] = f32_to_bf16(dPt[j]);
                    else sP[(16 * R + l16) * LDM + 16 * R + rr] = dPt[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * q4 + j, ii = l16;
                    float av = accA[j] * sBeta[16 * R + rr], pv = accP[j];
                    if (I == R) {
                        if (ii >= rr) av = 0.f;
                        if (ii > rr) pv = 0.f;
                    }
                    sX[(16 * R + rr) * LDX + 16 * I + ii] = av;
                    if constexpr (BF) sP[(16 * R + rr) * LDM + 16 * I + ii] = f32_to_bf16(pv);
                    else sP[(16 * R + rr) * LDM + 16 * I + ii] = pv;
                }
            }
        }
    }
    __syncthreads();  // A is complete in sX (the gate tables that shared its place are dead)
    if (wave < NSUB) {
        // X_RR = (I + A_RR)^{-1}: lane l16 computes column l16 by forward substitution
        const int R = wave;
        float *Ab = sX + (16 * R) * LDX + 16 * R;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float s = (rr == l16) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < rr; ++m) s -= Ab[rr * LDX + m] * x[m];
            x[rr] = s;
        }
        if (q4 == 0) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) Ab[rr * LDX + l16] = x[rr];
        }
    }
    __syncthreads();

    // ================= 5: blocks of X below the diagonal, one block diagonal at a time:
    // X_RI = -X_RR sum_{J=I}^{R-1} A_RJ X_JI (fp32 matrix-core products), stored transposed in
    // the upper block (I, R).
#pragma unroll
    for (int lvl = 1; lvl < NSUB; ++lvl) {
        const int R = wave;
        if (R >= lvl && R < NSUB) {
            const int I = R - lvl;
            f32x4 m = zero4();
#pragma unroll
            for (int J = 0; J < NSUB; ++J) {
                if (J < I || J >= R) continue;
                const Frag<false> a = lds_frag(sX + (16 * R + l16) * LDX + 16 * J + 4 * q4);  // A_RJ rows
                mma16(m, a, bwd_x_frag<false, LDX>(sX, J, I, l16, q4));
            }
            f32x4 xo = zero4();
            const Frag<false> xrr = lds_frag(sX + (16 * R + l16) * LDX + 16 * R + 4 * q4);
            Frag<false> mb;
            mb.v = make_float4(-m[0], -m[1], -m[2], -m[3]);
            mma16(xo, xrr, mb);
            // xo holds X_RI rows 4*q4 + j, column l16
            *reinterpret_cast<float4 *>(sX + (16 * I + l16) * LDX + 16 * R + 4 * q4) = make_float4(xo[0], xo[1], xo[2], xo[3]);
        }
        __syncthreads();
    }
    // forward record: T = X Diag(beta) in its half tiles (X_RR in place, X_RI stored transposed in
    // block (I, R); rows l16, columns 4 q4 + j of each 16 x 16 block)
    if (frec && wave < NSUB) {
        const int R = wave;
#pragma unroll
        for (int pp = 0; pp < FRec::NPAIR; ++pp) {
            if (2 * pp > R) break;
            Frag<BF> f[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int I = 2 * pp + u;
                float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (I == R) {
                    xv = *reinterpret_cast<const float4 *>(sX + (16 * R + l16) * LDX + 16 * R + 4 * q4);
                } else if (I < R) {
                    const float *xt = sX + (16 * I + 4 * q4) * LDX + 16 * R + l16;
                    xv = make_float4(xt[0], xt[LDX], xt[2 * LDX], xt[3 * LDX]);
                }
                const float4 bv = I < NSUB ? *reinterpret_cast<const float4 *>(sBeta + 16 * I + 4 * q4)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
                f[u] = make_frag<BF>(xv.x * bv.x, xv.y * bv.y, xv.z * bv.z, xv.w * bv.w);
            }
            if (FRec::tp_half(R, pp)) store_frag<BF>(frec + FRec::oT + FRec::tp_off(R, pp), lane, f[0]);
            else store_pair<BF>(frec + FRec::oT + FRec::tp_off(R, pp), lane, f[0], f[1]);
        }
    }

    // ================= 6: M^T = K-^T X in tiles (16 channels x 16 tokens), each accumulator
    // holding 4 consecutive channels of one token, i.e. a 4-element piece of a row of M.  Wave w
    // takes d_k tiles w*KT/4 ...; sub-chunk R of X's columns needs its rows I >= R.
    {
        constexpr int CPW = KT / 4;
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) {
            const int ct = wave * CPW + cc;
            const OT *kr = sKbarT + (16 * ct + l16) * LDT + 4 * q4;
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                f32x4 acc = zero4();
#pragma unroll
                for (int I = R; I < NSUB; ++I) mma16(acc, lds_frag(kr + 16 * I), bwd_x_frag<BF, LDX>(sX, I, R, l16, q4));
                const Frag<BF> f = make_frag<BF>(acc[0], acc[1], acc[2], acc[3]);
                *reinterpret_cast<decltype(f.v) *>(sM + (16 * R + l16) * LDO + 16 * ct + 4 * q4) = f.v;
            }
        }
    }
    // N^T = P X: wave I forms the tiles of row block I, (P X)_IR = sum_{J=R}^{I} P_IJ X_JR, and
    // stores them as rows of N (zero for R > I)
    if (wave < NSUB) {
        const int I = wave;
        const OT *pr = sP + (16 * I + l16) * LDM + 4 * q4;
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            f32x4 acc = zero4();
#pragma unroll
            for (int J = 0; J < NSUB; ++J) {
                if (J < R || J > I) continue;
                mma16(acc, lds_frag(pr + 16 * J), bwd_x_frag<BF, LDX>(sX, J, R, l16, q4));
            }
            const Frag<BF> f = make_frag<BF>(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<decltype(f.v) *>(sN + (16 * R + l16) * LDM + 16 * I + 4 * q4) = f.v;
        }
    }
    __syncthreads();

    // ================= 7: M and N (the record's first bytes, formed in place), then e^{G_C} and beta
    for (int pc = tid; pc < (int)(Rec::oQtT / 16); pc += kChunkThreads)
        reinterpret_cast<u32x4 *>(rec)[pc] = reinterpret_cast<const u32x4 *>(smem)[pc];
    for (int pc = tid; pc < (int)((DK + C) * 4 / 16); pc += kChunkThreads)
        reinterpret_cast<u32x4 *>(rec + Rec::oGam)[pc] = reinterpret_cast<const u32x4 *>(smem + L::oGam)[pc];
}

// ====================================================================== scan ====
// Workgroup = two compute waves (16 state columns each, dS in registers) + four copy waves
// that stage each chunk's record and dO tile in LDS, in two pairs that take turns, each pair
// loading its chunk two chunks ahead (the forward scan's arrangement).  Copy waves keep their
// own memory counters, so the compute waves' stores never delay a load being waited for.
// The compute waves keep their stores few and wide (a wave stalls once it has 63 memory
// operations in flight): dU is formed transposed, dU^T = dS^T M^T + (scale dO)^T N^T, so that a
// lane holds 4 consecutive columns of one token (one 8-byte dv and dU store per 16x16 tile;
// the accumulator fragments of dS and dO are the operand fragments of their transposes), an
// exact product with the identity turns it back for the dS update, and dS leaves through a
// per-wave LDS tile as 16-byte row segments.
template <typename IO, int DK, int C>
struct BwdScanLayout {
    using Rec = BwdRec<IO, DK, C>;
    using OT = typename Rec::OT;
    static constexpr bool BF = Rec::BF;
    static constexpr int S = Rec::S;
    static constexpr int DVT = kBwdScanTile;
    static constexpr int NW = DVT / 16;  // compute waves
    static constexpr int NCW = kBwdScanCopyWaves;
    static constexpr int NT = kBwdScanThreads;
    static constexpr int LDV = DVT + Rec::PAD;  // staged dO [C][LDV]
    static constexpr int EP = 16 / S;           // elements per 16-byte piece
    static constexpr int PPR = DVT / EP;        // pieces per dO row
    static constexpr int V_PIECES = C * PPR;
    static constexpr int REC_UNITS = (int)(Rec::kBytes / 1024);
    static constexpr int V_UNITS = V_PIECES / 64;
    static_assert(V_PIECES % 64 == 0, "dO tile is copied in whole wave units");
    static_assert(sizeof(IO) == sizeof(OT), "operand type follows the io type");
    static constexpr int LDH = 16 + 4;  // per-wave fp32 [DK][LDH] tile that turns dS around for its stores
    static constexpr size_t kVBytes = (size_t)C * LDV * S;
    static constexpr size_t kHBytes = (size_t)NW * DK * LDH * 4;
    // Two record buffers where they fit, else one (fp32 records at d_k = 128, chunk 64: 119 KB):
    // then each chunk has a second barrier, after which the copy waves write the next one.
    static constexpr bool SINGLE = 2 * (Rec::kBytes + kVBytes) + kHBytes > 160 * 1024;
    static constexpr int GROUP = SINGLE ? NCW : 2;  // copy waves that share one chunk
    static constexpr size_t oRec0 = 0;
    static constexpr size_t oRec1 = SINGLE ? 0 : Rec::kBytes;
    static constexpr size_t oV0 = (SINGLE ? 1 : 2) * Rec::kBytes;
    static constexpr size_t oV1 = SINGLE ? oV0 : oV0 + kVBytes;
    static constexpr size_t oH = oV1 + kVBytes;
    static constexpr size_t kBytes = oH + kHBytes;
    static constexpr int UNITS_PER_WAVE = (REC_UNITS + V_UNITS + GROUP - 1) / GROUP;
    static constexpr bool kFits = kBytes <= 160 * 1024 && UNITS_PER_WAVE <= 40;
};

// One copy wave's share of a chunk (record units and dO pieces dealt in turn to the GROUP waves
// that share a chunk; IDX is this wave's place among them), held in registers between its loads
// and its LDS writes.
template <typename IO, int DK, int C, int IDX>
struct BwdStager {
    using L = BwdScanLayout<IO, DK, C>;
    using OT = typename L::OT;
    static constexpr int UNITS = L::REC_UNITS + L::V_UNITS;
    static constexpr int G = L::GROUP;
    static constexpr int PER = (UNITS - IDX + G - 1) / G;
    u32x4 r[PER];

    __device__ __forceinline__ void load(const char *rec, const IO *orow0, int clen, int64_t ostride, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = IDX + G * i;
            if (u < L::REC_UNITS) {
                r[i] = *reinterpret_cast<const u32x4 *>(rec + (size_t)u * 1024 + lane * 16);
            } else {
                const int piece = (u - L::REC_UNITS) * 64 + lane;
                const int row = min(piece / L::PPR, clen - 1);  // rows past the end re-read the last row
                r[i] = *reinterpret_cast<const u32x4 *>(orow0 + row * ostride + (piece % L::PPR) * L::EP);
            }
        }
    }
    __device__ __forceinline__ void store(char *lds_rec, OT *lds_o, int lane) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = IDX + G * i;
            if (u < L::REC_UNITS) {
                *reinterpret_cast<u32x4 *>(lds_rec + u * 1024 + lane * 16) = r[i];
            } else {
                const int piece = (u - L::REC_UNITS) * 64 + lane;
                *reinterpret_cast<u32x4 *>(lds_o + (piece / L::PPR) * L::LDV + (piece % L::PPR) * L::EP) = r[i];
            }
        }
    }
};

// Copy wave CW.  Stream element j is chunk nchunks - 1 - j.  With two buffers, pair CW / 2
// stages the elements with j % 2 == CW / 2; barrier j hands element j to the compute waves, and
// passing it also means that both compute waves are done with element j - 1, whose buffer may take
// element j + 1.  With one buffer the four copy waves load element j + 1 after barrier j and
// write it after the second barrier of element j, when the compute waves are done reading.
template <typename IO, int DK, int C, int CW>
__device__ __forceinline__ void bwd_copy_wave(char *smem, const char *records, int64_t slot0, int H, int h,
                                              const IO *obase, int64_t ostride, int len, int nchunks, int lane) {
    using L = BwdScanLayout<IO, DK, C>;
    using Rec = typename L::Rec;
    using OT = typename L::OT;
    constexpr int NPAIR = L::NCW / L::GROUP, PAIR = CW / L::GROUP;
    BwdStager<IO, DK, C, CW % L::GROUP> st;
    auto load = [&](int j) {
        const int c = nchunks - 1 - j;
        st.load(records + (size_t)((slot0 + c) * H + h) * Rec::kBytes, obase + (int64_t)c * C * ostride,
                min(C, len - c * C), ostride, lane);
    };
    auto store = [&](int j) {
        st.store(smem + ((j & 1) ? L::oRec1 : L::oRec0), reinterpret_cast<OT *>(smem + ((j & 1) ? L::oV1 : L::oV0)),
                 lane);
    };
    if constexpr (L::SINGLE) {
        if (nchunks > 0) {
            load(0);
            store(0);
        }
        for (int j = 0; j < nchunks; ++j) {
            __syncthreads();  // barrier j: element j is in the buffer
            if (j + 1 < nchunks) load(j + 1);
            __syncthreads();  // the compute waves are done reading element j
            if (j + 1 < nchunks) store(j + 1);
        }
    } else {
        if (PAIR < nchunks) {
            load(PAIR);
            if (PAIR == 0) {
                store(0);
                if (NPAIR < nchunks) load(NPAIR);
            }
        }
        for (int j = 0; j < nchunks; ++j) {
            __syncthreads();  // barrier j: the buffer of element j + 1 is free
            if ((j + 1) % NPAIR == PAIR && j + 1 < nchunks) {
                store(j + 1);
                if (j + 1 + NPAIR < nchunks) load(j + 1 + NPAIR);
            }
        }
    }
}

template <typename IO, int DK, int C>
__global__ void __launch_bounds__(kBwdScanThreads) kda_bwd_scan_kernel(BwdParams bp, const char *__restrict__ records) {
    using L = BwdScanLayout<IO, DK, C>;
    using Rec = typename L::Rec;
    using OT = typename L::OT;
    constexpr bool BF = L::BF;
    constexpr int NSUB = Rec::NSUB, KT = Rec::KT, NW = L::NW, DVT = L::DVT;
    constexpr int LDO = Rec::LDO, LDT = Rec::LDT, LDM = Rec::LDM, LDV = L::LDV, LDH = L::LDH;
    using Tr = IoTraits<IO>;
    const FwdParams &p = bp.f;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int H = p.H, DV = p.dv;

    const int ntile = DV / DVT;
    const SeqItem item = seq_item(blockIdx.x, p.num_seqs, H, ntile, p.order);
    const int tile = item.tile, h = item.h, n = item.n;
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
    const int64_t slot0 = bwd_slot0(p, n, C);
    const int nchunks = (len + C - 1) / C;
    const int64_t ostride = (int64_t)H * DV;  // elements between consecutive tokens of one head
    const IO *obase = static_cast<const IO *>(bp.d_out) + (start * H + h) * (int64_t)DV + col0;

    if (wave >= NW) {
        switch (wave - NW) {
            case 0: bwd_copy_wave<IO, DK, C, 0>(smem, records, slot0, H, h, obase, ostride, len, nchunks, lane); break;
            case 1: bwd_copy_wave<IO, DK, C, 1>(smem, records, slot0, H, h, obase, ostride, len, nchunks, lane); break;
            case 2: bwd_copy_wave<IO, DK, C, 2>(smem, records, slot0, H, h, obase, ostride, len, nchunks, lane); break;
            default: bwd_copy_wave<IO, DK, C, 3>(smem, records, slot0, H, h, obase, ostride, len, nchunks, lane); break;
        }
        return;
    }

    // ---- compute wave: state columns col0 + 16*wave + l16; dS in the accumulator layout
    const int col = col0 + 16 * wave + l16;
    f32x4 dS[KT];
    const int64_t state_base = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dS[ct][j] = bp.d_sf ? bp.d_sf[state_base + (int64_t)(16 * ct + 4 * q4 + j) * DV + col] : 0.f;
    __builtin_amdgcn_s_waitcnt(0);

    float *sH = reinterpret_cast<float *>(smem + L::oH) + wave * DK * LDH;
    // identity as a B operand: rows 4q4 + jj, column l16
    const Frag<BF> ident = make_frag<BF>(4 * q4 == l16 ? 1.f : 0.f, 4 * q4 + 1 == l16 ? 1.f : 0.f,
                                         4 * q4 + 2 == l16 ? 1.f : 0.f, 4 * q4 + 3 == l16 ? 1.f : 0.f);

    for (int j = 0; j < nchunks; ++j) {
        const int ci = nchunks - 1 - j;
        const int clen = min(C, len - ci * C);
        const int64_t tok0 = start + (int64_t)ci * C;
        __syncthreads();  // element j is in its buffer
        const char *rb = smem + ((j & 1) ? L::oRec1 : L::oRec0);
        const OT *sO = reinterpret_cast<const OT *>(smem + ((j & 1) ? L::oV1 : L::oV0));
        const OT *sM = reinterpret_cast<const OT *>(rb + Rec::oM);
        const OT *sN = reinterpret_cast<const OT *>(rb + Rec::oN);
        const OT *sQtT = reinterpret_cast<const OT *>(rb + Rec::oQtT);
        const OT *sBKtT = reinterpret_cast<const OT *>(rb + Rec::oBKtT);
        const float *sGam = reinterpret_cast<const float *>(rb + Rec::oGam);
        const float *sBeta = reinterpret_cast<const float *>(rb + Rec::oBeta);
        const int64_t slot_base = (slot0 + ci) * H + h;

        // gradient of the state this chunk hands on, kept for the gradient kernel (operand type):
        // written to the wave's LDS tile in the accumulator layout, read back as row segments
        {
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sH[(16 * ct + 4 * q4 + jj) * LDH + l16] = dS[ct][jj];
            OT *dh = static_cast<OT *>(bp.dhs) + slot_base * DK * DV + col0 + 16 * wave;
            keep_rows<OT, 16, LDH, DK>(dh, DV, sH, lane);  // all d_k rows: every read in flight together
        }
        Frag<BF> Sb[KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) Sb[ct] = frag_from_acc<BF>(dS[ct]);

        // scale * dO: rows 16I + 4q4 + jj (zero past the chunk's end), column l16
        Frag<BF> dOf[NSUB];
#pragma unroll
        for (int I = 0; I < NSUB; ++I) {
            float t[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * I + 4 * q4 + jj;
                const OT x = sO[r * LDV + 16 * wave + l16];
                float v;
                if constexpr (BF) v = bf16_to_f32(x);
                else v = x;
                t[jj] = r < clen ? v * p.scale : 0.f;
            }
            dOf[I] = make_frag<BF>(t[0], t[1], t[2], t[3]);
        }

        // dU^T = dS^T M^T + (scale dO)^T N^T; N is zero left of its block diagonal.  Lane holds
        // dU[16R + l16][16*wave + 4q4 + jj].
        f32x4 dUt[NSUB];
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            f32x4 z = zero4();
            const OT *mr = sM + (16 * R + l16) * LDO + 4 * q4;
#pragma unroll
            for (int kp = 0; kp < KT; kp += 2) mma32(z, Sb[kp], Sb[kp + 1], lds_frag(mr + 16 * kp), lds_frag(mr + 16 * kp + 16));
            const OT *nr = sN + (16 * R + l16) * LDM + 4 * q4;
#pragma unroll
            for (int I = R & ~1; I + 1 < NSUB; I += 2)
                mma32(z, dOf[I], dOf[I + 1], lds_frag(nr + 16 * I), lds_frag(nr + 16 * I + 16));
            if constexpr (NSUB % 2 == 1) mma16(z, dOf[NSUB - 1], lds_frag(nr + 16 * (NSUB - 1)));
            // fp32: the dv store branches below put joins between these products and later writes
            // of their registers, where the compiler leaves too few wait states
            if constexpr (!BF) mfma_settle(z);
            dUt[R] = z;
        }

        // dv = beta * dU and dU (kept per chunk for the gradient kernel): one store each per tile;
        // -dU back in the accumulator layout (rows 16R + 4q4 + jj, column l16) for the dS update
        Frag<BF> nU[NSUB];
        {
            const int cq = col0 + 16 * wave + 4 * q4;
            OT *du = static_cast<OT *>(bp.duch) + slot_base * C * DV + cq;
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                const int r = 16 * R + l16;
                const float b = sBeta[r];
                if (r < clen)
                    Tr::store4(static_cast<IO *>(bp.dv) + ((tok0 + r) * H + h) * (int64_t)DV + cq,
                               make_float4(b * dUt[R][0], b * dUt[R][1], b * dUt[R][2], b * dUt[R][3]));
                const Frag<BF> u = make_frag<BF>(dUt[R][0], dUt[R][1], dUt[R][2], dUt[R][3]);
                *reinterpret_cast<decltype(u.v) *>(du + (int64_t)r * DV) = u.v;
                f32x4 t = zero4();
                mma16(t, make_frag<BF>(-dUt[R][0], -dUt[R][1], -dUt[R][2], -dUt[R][3]), ident);
                // fp32: the next tile's store branch puts a join between these products and a later
                // write of their registers, where the compiler leaves too few wait states
                if constexpr (!BF) mfma_settle(t);
                nU[R] = frag_from_acc<BF>(t);
            }
        }

        // dS <- Diag(e^{G_C}) dS + Q~^T (scale dO) - (Diag(beta) K~)^T dU
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            const float4 gm = *reinterpret_cast<const float4 *>(sGam + 16 * ct + 4 * q4);
            dS[ct][0] *= gm.x;
            dS[ct][1] *= gm.y;
            dS[ct][2] *= gm.z;
            dS[ct][3] *= gm.w;
            const OT *qt = sQtT + (16 * ct + l16) * LDT + 4 * q4;
            const OT *kt = sBKtT + (16 * ct + l16) * LDT + 4 * q4;
#pragma unroll
            for (int R = 0; R + 1 < NSUB; R += 2) {
                mma32(dS[ct], lds_frag(qt + 16 * R), lds_frag(qt + 16 * (R + 1)), dOf[R], dOf[R + 1]);
                mma32(dS[ct], lds_frag(kt + 16 * R), lds_frag(kt + 16 * (R + 1)), nU[R], nU[R + 1]);
            }
            if constexpr (NSUB % 2 == 1) {
                mma16(dS[ct], lds_frag(qt + 16 * (NSUB - 1)), dOf[NSUB - 1]);
                mma16(dS[ct], lds_frag(kt + 16 * (NSUB - 1)), nU[NSUB - 1]);
            }
        }
        if constexpr (L::SINGLE) __syncthreads();  // one buffer: done reading this element
    }

    if (bp.ds0) {
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                bp.ds0[state_base + (int64_t)(16 * ct + 4 * q4 + jj) * DV + col] = dS[ct][jj];
    }
}

// ================================================================== gradients ====
template <typename IO, int DK, int DV, int C>
struct BwdGradLayout {
    static constexpr bool BF = IoTraits<IO>::kBf16;
    using OT = typename std::conditional<BF, uint16_t, float>::type;
    static constexpr int NW = DK / 16;  // one 16-channel key tile per wave
    static constexpr int NT = 64 * NW;
    static constexpr int NSUB = C / 16;
    static constexpr int NPAIR = NSUB * (NSUB + 1) / 2;  // sub-chunk pairs R >= I
    static constexpr int PADO = 16 / (int)sizeof(OT);
    static constexpr int LDV = DV + PADO;  // [C][DV] staged dO, dU, D
    static constexpr int LDC = C + PADO;   // [C][C] gradient blocks
    static constexpr int PIECES = C * DV * (int)sizeof(OT) / 16;  // 16-byte pieces of one [C][DV] tile
    static constexpr int PPR = DV * (int)sizeof(OT) / 16;         // pieces per row
    static constexpr int ELEMS = 16 / (int)sizeof(OT);
    static_assert(sizeof(IO) == sizeof(OT), "operand type follows the io type");
    static_assert(NT % PPR == 0 && PIECES % PPR == 0 && PPR <= 64, "staging split: whole rows per lane group");
    static_assert(DV % 32 == 0 && C % 16 == 0 && NSUB <= 4, "tile sizes");

    static constexpr size_t kTile = (size_t)C * LDV * sizeof(OT);
    static constexpr size_t kBlk = (size_t)C * LDC * sizeof(OT);
    static constexpr size_t kSmall = (size_t)C * 4 * 2 + (size_t)DK * 4 + (size_t)NW * C * 4;
    // The transposed blocks dP^T and dL^T are kept where they fit (one wide read per fragment);
    // otherwise (fp32 at d_k = d_v = 128, chunk 64) their fragments are gathered from the
    // columns of dP and dA (dL = beta_r dA).
    static constexpr bool TRANS = 3 * kTile + 4 * kBlk + kSmall <= 160 * 1024;
    static constexpr size_t oO = 0;
    static constexpr size_t oU = oO + kTile;
    static constexpr size_t oD = oU + kTile;
    static constexpr size_t oP = oD + kTile;                     // dP   [r][i]
    static constexpr size_t oPT = oP + kBlk;                     // dP   [i][r]  (TRANS)
    static constexpr size_t oA = oPT + (TRANS ? kBlk : 0);       // dA   [r][i]
    static constexpr size_t oLT = oA + kBlk;                     // dL   [i][r]  (TRANS; dL = beta_r dA)
    static constexpr size_t oBeta = oLT + (TRANS ? kBlk : 0);
    static constexpr size_t oUV = oBeta + (size_t)C * 4;
    static constexpr size_t oGam = oUV + (size_t)C * 4;
    static constexpr size_t oDb = oGam + (size_t)DK * 4;
    static constexpr size_t kBytes = oDb + (size_t)NW * C * 4;
    static constexpr bool kFits = kBytes <= 160 * 1024;

    __host__ __device__ static constexpr int pair_r(int pi) {
        int R = 0;
        while ((R + 1) * (R + 2) / 2 <= pi) ++R;
        return R;
    }
    __host__ __device__ static constexpr int pair_i(int pi) { return pi - pair_r(pi) * (pair_r(pi) + 1) / 2; }
};


// Advances `item` to the first (slot, head) pair among item, item + gridDim.x, ... that
// kda_bwd_prep_kernel flagged (thread t checks the t-th candidate, the first flagged one wins); false
// when there is none.  Every thread of the workgroup calls it and gets the same answer.
template <int C, int NT>
__device__ __forceinline__ bool next_flagged_pair(const BwdParams &bp, int64_t &item) {
    __shared__ int s_first;
    const int64_t items = bp.slots * bp.f.H;
    const int tid = threadIdx.x;
    for (; item < items; item += (int64_t)gridDim.x * NT) {
        if (tid == 0) s_first = NT;
        __syncthreads();
        const int64_t cand = item + (int64_t)gridDim.x * tid;
        int n, ci;
        if (cand < items && bwd_slot_chunk(bp.f, C, cand / bp.f.H, n, ci) && bp.split_flag[cand] != 0)
            atomicMin(&s_first, tid);
        __syncthreads();
        const int first = s_first;
        __syncthreads();  // every thread has read s_first before the next round resets it
        if (first < NT) {
            item += (int64_t)gridDim.x * first;
            return true;
        }
    }
    return false;
}

// SPLIT: this instantiation takes the chunks kda_bwd_prep_kernel flagged (some sub-chunk decays beyond
// the single-anchor limit of the diagonal blocks) and forms their diagonal-block terms from the split
// levels; the other instantiation takes every other chunk with no trace of that path in its code.  Such
// chunks are rare, so the SPLIT grid has about one workgroup per CU, and each walks the (slot, head)
// pairs blockIdx.x, + gridDim.x, ... and takes the flagged ones: in the common case the launch costs a
// few flag reads instead of one empty 92 KB workgroup per pair.
template <typename IO, int DK, int DV, int C, bool SPLIT>
__global__ void __launch_bounds__(64 * (DK / 16)) kda_bwd_grad_kernel(BwdParams bp) {
    using L = BwdGradLayout<IO, DK, DV, C>;
    using OT = typename L::OT;
    constexpr bool BF = L::BF;
    constexpr int NSUB = L::NSUB, NW = L::NW, NT = L::NT, LDV = L::LDV, LDC = L::LDC;
    using Tr = IoTraits<IO>;
    const FwdParams &p = bp.f;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OT *sO = reinterpret_cast<OT *>(smem + L::oO);
    OT *sU = reinterpret_cast<OT *>(smem + L::oU);
    OT *sD = reinterpret_cast<OT *>(smem + L::oD);
    OT *sP = reinterpret_cast<OT *>(smem + L::oP);
    OT *sPT = reinterpret_cast<OT *>(smem + L::oPT);
    OT *sA = reinterpret_cast<OT *>(smem + L::oA);
    OT *sLT = reinterpret_cast<OT *>(smem + L::oLT);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);
    float *sUV = reinterpret_cast<float *>(smem + L::oUV);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);
    float *sDb = reinterpret_cast<float *>(smem + L::oDb);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    const int H = p.H;

    // SPLIT: the (slot, head) pair this pass takes; a workgroup with no flagged pair leaves here,
    // before anything the pass keeps across pairs is formed
    [[maybe_unused]] int64_t item = blockIdx.x;
    if constexpr (SPLIT) {
        if (!next_flagged_pair<C, NT>(bp, item)) return;
    }
next_item:
    const int64_t slot = SPLIT ? item / H : blockIdx.x / H;
    const int h = SPLIT ? (int)(item % H) : (int)(blockIdx.x % H);
    int n, ci;
    if (!bwd_slot_chunk(p, C, slot, n, ci)) return;
    if ((bp.split_flag[slot * H + h] != 0) != SPLIT) return;  // the other instantiation's chunk
    const int64_t start = p.cu ? (int64_t)p.cu[n] : (int64_t)n * p.T;
    const int len = p.cu ? p.cu[n + 1] - p.cu[n] : p.T;
    const int clen = min(C, len - ci * C);
    const int64_t tok0 = start + (int64_t)ci * C;
    const int64_t base = slot * H + h;
    const int cw = 16 * wave;  // first key channel of this wave

    // ---- key side of the wave's channels for every token: lane (token 16R + l16, channels cw + 4q4 + j)
    // (k and q stay packed as loaded and are unpacked where used)
    using KQ = typename std::conditional<BF, uint2, float4>::type;
    float G[NSUB][4];
    KQ kraw[NSUB], qraw[NSUB];
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
        const int r = 16 * R + l16;
        const bool valid = r < clen;
        const int64_t row = ((tok0 + min(r, clen - 1)) * H + h) * (int64_t)DK + cw + 4 * q4;
        const float4 gv = *reinterpret_cast<const float4 *>(p.g + row);
        const KQ kv = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.k) + row);
        const KQ qv = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.q) + row);
        const float m = valid ? kLog2e : 0.f;
        G[R][0] = scan16_add(gv.x * m);
        G[R][1] = scan16_add(gv.y * m);
        G[R][2] = scan16_add(gv.z * m);
        G[R][3] = scan16_add(gv.w * m);
        kraw[R] = valid ? kv : KQ{};
        qraw[R] = valid ? qv : KQ{};
    }
    // sub-chunks whose decay (in this wave's channels) is too strong for the single-anchor split of
    // the diagonal blocks
    bool split[NSUB];
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
        bool big = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) big |= G[R][j] < -kDiagAnchorMaxDecay;
        split[R] = SPLIT && __builtin_amdgcn_ballot_w64(big) != 0;
    }
    auto unpk = [](const KQ &x, float (&o)[4]) {
        const float4 v = unpack4<BF>(x);
        o[0] = v.x;
        o[1] = v.y;
        o[2] = v.z;
        o[3] = v.w;
    };

    // ---- stage dO, dU, D ([C][DV]); sum_j dU_rj V_rj per token
    if (tid < C) sBeta[tid] = tid < clen ? p.beta[(tok0 + tid) * H + h] : 0.f;
    {
        const IO *dO = static_cast<const IO *>(bp.d_out);
        const OT *dU = static_cast<const OT *>(bp.duch) + base * C * DV;
        const OT *Dc = static_cast<const OT *>(bp.dch) + base * C * DV;
        const IO *V = static_cast<const IO *>(p.v);
#pragma unroll
        for (int i = 0; i < (L::PIECES + NT - 1) / NT; ++i) {
            const int piece = tid + NT * i;
            // a row's PPR pieces sit in PPR consecutive lanes, all inside or all outside
            if (L::PIECES % NT != 0 && piece >= L::PIECES) break;
            const int r = piece / L::PPR;
            const int cc = (piece % L::PPR) * L::ELEMS;
            const bool valid = r < clen;
            const int64_t grow = ((tok0 + min(r, clen - 1)) * H + h) * (int64_t)DV + cc;
            const uint4 xo = valid ? *reinterpret_cast<const uint4 *>(dO + grow) : make_uint4(0u, 0u, 0u, 0u);
            const uint4 xu = *reinterpret_cast<const uint4 *>(dU + (int64_t)r * DV + cc);
            const uint4 xd = *reinterpret_cast<const uint4 *>(Dc + (int64_t)r * DV + cc);
            const uint4 xv = *reinterpret_cast<const uint4 *>(V + grow);
            *reinterpret_cast<uint4 *>(sO + r * LDV + cc) = xo;
            *reinterpret_cast<uint4 *>(sU + r * LDV + cc) = xu;
            *reinterpret_cast<uint4 *>(sD + r * LDV + cc) = xd;
            float uv = 0.f;
            if constexpr (BF) {
                const uint32_t a[4] = {xu.x, xu.y, xu.z, xu.w}, b[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) uv += bf16_lo(a[e]) * bf16_lo(b[e]) + bf16_hi(a[e]) * bf16_hi(b[e]);
            } else {
                uv = __uint_as_float(xu.x) * __uint_as_float(xv.x) + __uint_as_float(xu.y) * __uint_as_float(xv.y) +
                     __uint_as_float(xu.z) * __uint_as_float(xv.z) + __uint_as_float(xu.w) * __uint_as_float(xv.w);
            }
            // the PPR pieces of a row sit in PPR consecutive lanes of one wave
#pragma unroll
            for (int o = 1; o < L::PPR; o <<= 1) uv += __shfl_xor(uv, o);
            if (piece % L::PPR == 0) sUV[r] = valid ? uv : 0.f;
        }
    }
    __syncthreads();

    // rows c = cw + l16 of S and dS (A operands straight from the chunk states, operand type: 4
    // consecutive columns are an A fragment), loaded here so that they arrive during the dP / dA products
    Frag<BF> sf[DV / 16], dsf[DV / 16];
    {
        const OT *Sr = static_cast<const OT *>(bp.hs) + base * DK * DV + (int64_t)(cw + l16) * DV + 4 * q4;
        const OT *dSr = static_cast<const OT *>(bp.dhs) + base * DK * DV + (int64_t)(cw + l16) * DV + 4 * q4;
#pragma unroll
        for (int kt = 0; kt < DV / 16; ++kt) {
            sf[kt] = lds_frag(Sr + 16 * kt);
            dsf[kt] = lds_frag(dSr + 16 * kt);
        }
    }

    // ---- dP = scale lower_incl(dO D^T), dA = -strictly_lower(dU D^T), block pairs R >= I
#pragma unroll
    for (int pi0 = 0; pi0 < L::NPAIR; pi0 += NW) {
        const int pi = pi0 + wave;
        if (pi >= L::NPAIR) break;
        const int R = L::pair_r(pi), I = L::pair_i(pi);
        f32x4 accP = zero4(), accA = zero4();
        const OT *ao = sO + (16 * R + l16) * LDV + 4 * q4;
        const OT *au = sU + (16 * R + l16) * LDV + 4 * q4;
        const OT *bd = sD + (16 * I + l16) * LDV + 4 * q4;
#pragma unroll
        for (int kt = 0; kt < DV; kt += 32) {
            const Frag<BF> b0 = lds_frag(bd + kt), b1 = lds_frag(bd + kt + 16);
            mma32(accP, lds_frag(ao + kt), lds_frag(ao + kt + 16), b0, b1);
            mma32(accA, lds_frag(au + kt), lds_frag(au + kt + 16), b0, b1);
        }
        // accumulator: row r = 16R + 4q4 + j, column i = 16I + l16
        float vp[4], va[4], vl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 4 * q4 + j;
            vp[j] = (R == I && l16 > rr) ? 0.f : accP[j] * p.scale;
            va[j] = (R == I && l16 >= rr) ? 0.f : -accA[j];
            vl[j] = va[j] * sBeta[16 * R + rr];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * R + 4 * q4 + j;
            if constexpr (BF) {
                sP[r * LDC + 16 * I + l16] = f32_to_bf16(vp[j]);
                sA[r * LDC + 16 * I + l16] = f32_to_bf16(va[j]);
            } else {
                sP[r * LDC + 16 * I + l16] = vp[j];
                sA[r * LDC + 16 * I + l16] = va[j];
            }
        }
        if constexpr (L::TRANS) {
            const Frag<BF> fp = make_frag<BF>(vp[0], vp[1], vp[2], vp[3]);
            const Frag<BF> fl = make_frag<BF>(vl[0], vl[1], vl[2], vl[3]);
            *reinterpret_cast<decltype(fp.v) *>(sPT + (16 * I + l16) * LDC + 16 * R + 4 * q4) = fp.v;
            *reinterpret_cast<decltype(fl.v) *>(sLT + (16 * I + l16) * LDC + 16 * R + 4 * q4) = fl.v;
        } else {
            (void)vl;
        }
    }

    // ---- rowsum(dS .* S) over the rows c = cw + l16 of S and dS, and dS D^T; S dO^T and S dU^T are
    //      formed later, just before the row side needs them
    f32x4 Zs[NSUB];
    {
        float gam = 0.f;
#pragma unroll
        for (int kt = 0; kt < DV / 16; ++kt) {
            const float4 a = unpack4<BF>(sf[kt].v), b = unpack4<BF>(dsf[kt].v);
            gam += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
        }
        gam += __shfl_xor(gam, 16);
        gam += __shfl_xor(gam, 32);
        if (q4 == 0) sGam[cw + l16] = gam;
        __syncthreads();  // dP / dA blocks complete
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            Zs[R] = zero4();
            const OT *bdd = sD + (16 * R + l16) * LDV + 4 * q4;
#pragma unroll
            for (int kt = 0; kt < DV / 16; kt += 2)
                mma32(Zs[R], dsf[kt], dsf[kt + 1], lds_frag(bdd + 16 * kt), lds_frag(bdd + 16 * kt + 16));
        }
    }

    // ---- gate factors (log2 domain; per lane and channel j): b_R sub-chunk boundaries
    float bnd[NSUB + 1][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bnd[0][j] = 0.f;
#pragma unroll
    for (int R = 0; R < NSUB; ++R)
#pragma unroll
        for (int j = 0; j < 4; ++j) bnd[R + 1][j] = bnd[R][j] + __shfl(G[R][j], 16 * q4 + 15);

    // transposed operands through the identity: A operands with rows = channels
    const Frag<BF> eye = make_frag<BF>(4 * q4 == l16 ? 1.f : 0.f, 4 * q4 + 1 == l16 ? 1.f : 0.f,
                                       4 * q4 + 2 == l16 ? 1.f : 0.f, 4 * q4 + 3 == l16 ? 1.f : 0.f);
    Frag<BF> kbT[NSUB];
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
        float kb[4], kk[4];
        unpk(kraw[R], kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[j] = kk[j] * fast_exp2(bnd[R + 1][j] - bnd[R][j] - G[R][j]);  // k e^{b_{R+1} - G}
        f32x4 t = zero4();
        mma16(t, make_frag<BF>(kb[0], kb[1], kb[2], kb[3]), eye);
        if constexpr (SPLIT) mfma_settle(t);  // the split path's branches put joins before some reads
        kbT[R] = frag_from_acc<BF>(t);
    }

    // ---- column side (tokens of I): Col_I = sum_{R >= I} e^{b_R - b_{I+1}} (q_r dP_ri + k_r dL_ri),
    //      finished into the parts of dk that do not need the row side (via K^ and via K-)
    float dkc[NSUB][4], dG[NSUB][4], gcs[4] = {0.f, 0.f, 0.f, 0.f};
    {
        Frag<BF> qrT[NSUB], krT[NSUB];
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            float kr[4], qr[4], kk[4], qq[4];
            unpk(kraw[R], kk);
            unpk(qraw[R], qq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fr = fast_exp2(G[R][j]);  // e^{G - b_R} (<= 1)
                kr[j] = kk[j] * fr;
                qr[j] = qq[j] * fr;
            }
            f32x4 t = zero4();
            mma16(t, make_frag<BF>(kr[0], kr[1], kr[2], kr[3]), eye);
            if constexpr (SPLIT) mfma_settle(t);
            krT[R] = frag_from_acc<BF>(t);
            t = zero4();
            mma16(t, make_frag<BF>(qr[0], qr[1], qr[2], qr[3]), eye);
            if constexpr (SPLIT) mfma_settle(t);
            qrT[R] = frag_from_acc<BF>(t);
        }
        // fragments of dP^T and dL^T (row i, the 4 columns r .. r + 3): read whole from their own
        // blocks, or gathered from the columns of dP and dA (dL = beta_r dA)
        auto pt_frag = [&](int i, int r) {
            if constexpr (L::TRANS) {
                return lds_frag(sPT + i * LDC + r);
            } else {
                return make_frag<BF>(elem_f32(sP[r * LDC + i]), elem_f32(sP[(r + 1) * LDC + i]),
                                     elem_f32(sP[(r + 2) * LDC + i]), elem_f32(sP[(r + 3) * LDC + i]));
            }
        };
        auto lt_frag = [&](int i, int r) {
            if constexpr (L::TRANS) {
                return lds_frag(sLT + i * LDC + r);
            } else {
                return make_frag<BF>(sBeta[r] * elem_f32(sA[r * LDC + i]), sBeta[r + 1] * elem_f32(sA[(r + 1) * LDC + i]),
                                     sBeta[r + 2] * elem_f32(sA[(r + 2) * LDC + i]),
                                     sBeta[r + 3] * elem_f32(sA[(r + 3) * LDC + i]));
            }
        };
        f32x4 Col[NSUB];
#pragma unroll
        for (int I = 0; I < NSUB; ++I) Col[I] = zero4();
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
#pragma unroll
            for (int I = 0; I <= R; ++I) {
                if (I == R && split[R]) continue;  // the diagonal block comes from the split levels below
                f32x4 tc = zero4();
                mma16(tc, qrT[R], pt_frag(16 * I + l16, 16 * R + 4 * q4));
                mma16(tc, krT[R], lt_frag(16 * I + l16, 16 * R + 4 * q4));
#pragma unroll
                for (int j = 0; j < 4; ++j) Col[I][j] += fast_exp2(bnd[R][j] - bnd[I + 1][j]) * tc[j];
            }
        }
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            float kk[4];
            unpk(kraw[R], kk);
            f32x4 colD = zero4();  // diagonal-block part with its whole factor (split sub-chunks)
            if (split[R]) {
                float qq[4];
                unpk(qraw[R], qq);
                f32x4 unused = zero4();
                grad_diag_split<BF, false, true, L::TRANS>(unused, unused, colD, kk, qq, G[R],
                                                           sP + 16 * R * LDC + 16 * R, sA + 16 * R * LDC + 16 * R,
                                                           sPT + 16 * R * LDC + 16 * R, sLT + 16 * R * LDC + 16 * R,
                                                           sBeta + 16 * R, LDC, eye, l16, q4, lane);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float fb = fast_exp2(bnd[R + 1][j] - bnd[R][j] - G[R][j]);
                const float ekb = fast_exp2(bnd[NSUB][j] - bnd[R][j] - G[R][j]);
                const float dk2 = fb * Col[R][j] + colD[j];
                const float dk3 = ekb * Zs[R][j];
                dkc[R][j] = dk2 + dk3;
                dG[R][j] = -kk[j] * (dk2 + dk3);
                gcs[j] += kk[j] * dk3;
            }
        }
    }

    // ---- row side (tokens of R), one token tile at a time, and the outputs dq, dk:
    //      RowP_R = sum_{I <= R} e^{b_R - b_{I+1}} kb_i dP_ri, RowA_R likewise with dA
    float dbp[NSUB];
    IO *dqo = static_cast<IO *>(bp.dq);
    IO *dko = static_cast<IO *>(bp.dk);
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
        f32x4 Zq = zero4(), Zu = zero4();
        {
            const OT *bo = sO + (16 * R + l16) * LDV + 4 * q4;
            const OT *bu = sU + (16 * R + l16) * LDV + 4 * q4;
#pragma unroll
            for (int kt = 0; kt < DV / 16; kt += 2) {
                mma32(Zq, sf[kt], sf[kt + 1], lds_frag(bo + 16 * kt), lds_frag(bo + 16 * kt + 16));
                mma32(Zu, sf[kt], sf[kt + 1], lds_frag(bu + 16 * kt), lds_frag(bu + 16 * kt + 16));
            }
        }
        f32x4 RowP = zero4(), RowA = zero4(), RowPD = zero4(), RowAD = zero4();
        if (split[R]) {  // diagonal-block part with its whole factor
            float kk[4], qq[4];
            unpk(kraw[R], kk);
            unpk(qraw[R], qq);
            f32x4 unused = zero4();
            grad_diag_split<BF, true, false, L::TRANS>(RowPD, RowAD, unused, kk, qq, G[R],
                                                       sP + 16 * R * LDC + 16 * R, sA + 16 * R * LDC + 16 * R,
                                                       sPT + 16 * R * LDC + 16 * R, sLT + 16 * R * LDC + 16 * R,
                                                       sBeta + 16 * R, LDC, eye, l16, q4, lane);
        }
#pragma unroll
        for (int I = 0; I <= R; ++I) {
            if (I == R && split[R]) continue;
            f32x4 tp = zero4(), ta = zero4();
            mma16(tp, kbT[I], lds_frag(sP + (16 * R + l16) * LDC + 16 * I + 4 * q4));
            mma16(ta, kbT[I], lds_frag(sA + (16 * R + l16) * LDC + 16 * I + 4 * q4));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sh = fast_exp2(bnd[R][j] - bnd[I + 1][j]);  // e^{b_R - b_{I+1}}
                RowP[j] += sh * tp[j];
                RowA[j] += sh * ta[j];
            }
        }
        const int r = 16 * R + l16;
        const float b = sBeta[r];
        float dq4[4], dk4[4], kk[4], qq[4];
        unpk(kraw[R], kk);
        unpk(qraw[R], qq);
        dbp[R] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float fr = fast_exp2(G[R][j]);
            const float eG = fast_exp2(bnd[R][j] + G[R][j]);
            const float W = fr * RowA[j] + RowAD[j];
            const float dq = p.scale * eG * Zq[j] + fr * RowP[j] + RowPD[j];
            const float dk1 = b * (W - eG * Zu[j]);
            dq4[j] = dq;
            dk4[j] = dk1 + dkc[R][j];
            dG[R][j] += qq[j] * dq + kk[j] * dk1;
            dbp[R] += kk[j] * (W - eG * Zu[j]);
        }
        if (r < clen) {
            const int64_t row = ((tok0 + r) * H + h) * (int64_t)DK + cw + 4 * q4;
            Tr::store4(dqo + row, make_float4(dq4[0], dq4[1], dq4[2], dq4[3]));
            Tr::store4(dko + row, make_float4(dk4[0], dk4[1], dk4[2], dk4[3]));
        }
    }
    // gradient of the chunk's total gate G_C: sum over tokens, plus e^{G_C} rowsum(dS .* S)
    const int rl = clen - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x = gcs[j];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        x += fast_exp2(bnd[NSUB][j]) * sGam[cw + 4 * q4 + j];
#pragma unroll
        for (int R = 0; R < NSUB; ++R)
            if (16 * R + l16 == rl) dG[R][j] += x;
    }
    // dg = reverse cumulative sum of dG over the chunk's tokens
    float carry[4] = {0.f, 0.f, 0.f, 0.f};
    float *dgo = bp.dg;
#pragma unroll
    for (int R = NSUB - 1; R >= 0; --R) {
        float out4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float incl = scan16_add(dG[R][j]);
            const float tot = __shfl(incl, 16 * q4 + 15);
            out4[j] = tot - incl + dG[R][j] + carry[j];
            carry[j] += tot;
        }
        const int r = 16 * R + l16;
        if (r < clen)
            *reinterpret_cast<float4 *>(dgo + ((tok0 + r) * H + h) * (int64_t)DK + cw + 4 * q4) =
                make_float4(out4[0], out4[1], out4[2], out4[3]);
    }
    // dbeta: this wave's channels, then the sum over waves and the value term
#pragma unroll
    for (int R = 0; R < NSUB; ++R) {
        float x = dbp[R];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (q4 == 0) sDb[wave * C + 16 * R + l16] = x;
    }
    __syncthreads();
    if (tid < clen) {
        float x = sUV[tid];
#pragma unroll
        for (int w = 0; w < NW; ++w) x += sDb[w * C + tid];
        bp.dbeta[(tok0 + tid) * H + h] = x;
    }
    if constexpr (SPLIT) {
        __syncthreads();  // the next pair restages the LDS this one still reads
        item += gridDim.x;
        if (next_flagged_pair<C, NT>(bp, item)) goto next_item;
    }
}

// ================================================================== launch ====

template <typename IO, int DK, int DV, int C>
constexpr bool bwd_fits() {
    return BwdPrepLayout<IO, DK, C>::kFits && BwdScanLayout<IO, DK, C>::kFits && BwdGradLayout<IO, DK, DV, C>::kFits;
}

template <typename IO, int DK, int DV, int C>
hipError_t launch_bwd_variant(const BwdParams &bp, hipStream_t stream) {
    if constexpr (!bwd_fits<IO, DK, DV, C>()) {
        return hipErrorInvalidConfiguration;
    } else {
        const FwdParams &p = bp.f;
        const int64_t prep_blocks = bp.slots * p.H;
        if (prep_blocks > 0 && (bp.phases & 1)) {
            hipLaunchKernelGGL((kda_bwd_prep_kernel<IO, DK, C>), dim3((unsigned)prep_blocks), dim3(kChunkThreads), 0,
                               stream, bp, bp.brec);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (!(bp.phases & 2)) return hipSuccess;
        const int64_t scan_blocks = (int64_t)p.num_seqs * p.H * (DV / kBwdScanTile);
        if (scan_blocks > 0) {
            hipLaunchKernelGGL((kda_bwd_scan_kernel<IO, DK, C>), dim3((unsigned)scan_blocks),
                               dim3(BwdScanLayout<IO, DK, C>::NT), 0, stream, bp, (const char *)bp.brec);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int64_t grad_blocks = bp.slots * p.H;
        if (grad_blocks > 0) {
            hipLaunchKernelGGL((kda_bwd_grad_kernel<IO, DK, DV, C, false>), dim3((unsigned)grad_blocks),
                               dim3(BwdGradLayout<IO, DK, DV, C>::NT), 0, stream, bp);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            // chunks with strong decay (flagged by the prep kernel), walked by about one workgroup per CU
            const int64_t split_blocks = std::min<int64_t>(grad_blocks, std::max(1, bp.cus));
            hipLaunchKernelGGL((kda_bwd_grad_kernel<IO, DK, DV, C, true>), dim3((unsigned)split_blocks),
                               dim3(BwdGradLayout<IO, DK, DV, C>::NT), 0, stream, bp);
            return hipGetLastError();
        }
        return hipSuccess;
    }
}

// F(DK, DV, C)
#define KDA_BWD_VARIANTS(F)                                                                \
    F(64, 64, 16) F(64, 64, 32) F(64, 64, 64) F(64, 128, 16) F(64, 128, 32) F(64, 128, 64) \
    F(128, 64, 16) F(128, 64, 32) F(128, 64, 64) F(128, 128, 16) F(128, 128, 32) F(128, 128, 64)

template <typename IO>
size_t bwd_record_bytes(int dk, int chunk) {
#define KDA_BWD_REC_CASE(DK_, DV_, C_) \
    if (dk == DK_ && chunk == C_) return BwdRec<IO, DK_, C_>::kBytes;
    KDA_BWD_VARIANTS(KDA_BWD_REC_CASE)
#undef KDA_BWD_REC_CASE
    return 0;
}

template <typename IO>
bool bwd_supported(int dk, int dv, int chunk) {
#define KDA_BWD_FIT_CASE(DK_, DV_, C_) \
    if (dk == DK_ && dv == DV_ && chunk == C_) return bwd_fits<IO, DK_, DV_, C_>();
    KDA_BWD_VARIANTS(KDA_BWD_FIT_CASE)
#undef KDA_BWD_FIT_CASE
    return false;
}

template <typename IO>
hipError_t launch_bwd(const BwdParams &bp, int chunk, hipStream_t stream) {
#define KDA_BWD_CASE(DK_, DV_, C_) \
    if (bp.f.dk == DK_ && bp.f.dv == DV_ && chunk == C_) return launch_bwd_variant<IO, DK_, DV_, C_>(bp, stream);
    KDA_BWD_VARIANTS(KDA_BWD_CASE)
#undef KDA_BWD_CASE
    return hipErrorInvalidConfiguration;
}

}  // namespace kda
