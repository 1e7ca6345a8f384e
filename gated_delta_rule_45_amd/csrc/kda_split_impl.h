// Two-pass chunkwise KDA forward for gfx950.
//
// Pass 1 (kda_prep_kernel): one workgroup per (chunk, head), all in parallel.  It does
// every step that does not depend on the recurrent state (Kimi Linear summary page,
// "Chunkwise parallel algorithm" and "Less compute than general DPLR" sections):
// in-chunk cumulative gate, gated operands, the two C x C matrices A (from k, k) and
// P (from q, k), and the UT transform T = (I + A)^{-1} Diag(beta) with the
// lower-triangular inverse computed by forward substitution (16 x 16 diagonal blocks row
// by row, off-diagonal blocks block by block).  It writes one record per chunk-head:
//
//   K~ = k e^{G},  Q~ = q e^{G}   [C x d_k]   A operands of K~ S and Q~ S
//   K-^T, K- = k e^{G_C - G}     [d_k x C]   A operand of K-^T D
//   T, P                          [C x C]     lower-triangular, A operands of T Y and P D
//   Gamma = e^{G_C}               [d_k]       per-channel chunk decay
//
// in matrix-core fragment order: each 16 x 32 operand tile is 64 lanes x 8 values, so the
// scan reads every fragment with one 16-byte load per lane.
//
// Pass 2 (kda_scan_kernel): one workgroup per (sequence, head, d_v tile); each compute wave
// owns 16 or 32 columns of the fp32 state, kept in registers.  Per chunk, with the record
// staged in LDS by copy waves that load it one to three chunks ahead:
//
//   Y = V - K~ S        D = T Y         O = scale (Q~ S + P D)        S <- Gamma S + K-^T D
//
// (D = T (V - K~ S) equals the WY form U - W S with W = T K~ and U = T V.)  Where LDS allows,
// kda_scan_ow_kernel runs the same algebra with the state chain and the output on separate
// waves (its KEEP instantiation, for the backward pass, writes each chunk's initial state and
// D instead of the output); shapes whose extra LDS slots do not fit use kda_scan_kernel.
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_plan.h"
#include "kda_split_record.h"

namespace kda {

template <bool BF>
__device__ __forceinline__ void load_pair(const char *tile, int lane, Frag<BF> &a, Frag<BF> &b) {
    if constexpr (BF) {
        const uint4 x = *reinterpret_cast<const uint4 *>(tile + lane * 16);
        a.v = make_uint2(x.x, x.y);
        b.v = make_uint2(x.z, x.w);
    } else {
        a.v = *reinterpret_cast<const float4 *>(tile + lane * 32);
        b.v = *reinterpret_cast<const float4 *>(tile + lane * 32 + 16);
    }
}

template <bool BF>
struct FragPair {
    Frag<BF> a, b;
};
template <bool BF>
__device__ __forceinline__ FragPair<BF> ld_pair(const char *tile, int lane) {
    FragPair<BF> f;
    load_pair<BF>(tile, lane, f.a, f.b);
    return f;
}
// tile (R, pp) of T or P at `base`: a full pair, or a half tile's left fragment (b is zero)
template <bool BF, typename Rec>
__device__ __forceinline__ FragPair<BF> ld_tp(const char *base, int R, int pp, int lane) {
    if (Rec::tp_half(R, pp)) {
        FragPair<BF> f;
        f.a.v = *reinterpret_cast<const decltype(f.a.v) *>(base + Rec::tp_off(R, pp) + lane * (int)sizeof(f.a.v));
        f.b = make_frag<BF>(0.f, 0.f, 0.f, 0.f);
        return f;
    }
    return ld_pair<BF>(base + Rec::tp_off(R, pp), lane);
}
// acc += (tile (R, pp) of T or P) x (the matching two 16-token operand fragments), and its
// transpose-side twin; a half tile contracts over its left 16 tokens only
template <bool BF, typename Rec>
__device__ __forceinline__ void mma_tp_left(f32x4 &acc, const FragPair<BF> &t, const Frag<BF> &y0, const Frag<BF> &y1,
                                            int R, int pp) {
    if (Rec::tp_half(R, pp)) mma16(acc, t.a, y0);
    else mma32(acc, t.a, t.b, y0, y1);
}
template <bool BF, typename Rec>
__device__ __forceinline__ void mma_tp_right(f32x4 &acc, const Frag<BF> &x0, const Frag<BF> &x1, const FragPair<BF> &t,
                                             int R, int pp) {
    if (Rec::tp_half(R, pp)) mma16(acc, x0, t.a);
    else mma32(acc, x0, x1, t.a, t.b);
}

// Sequence n and chunk c of global chunk index gidx; false if gidx is past the last chunk.
__device__ __forceinline__ bool locate_chunk(const FwdParams &p, const int32_t *chunk_off, int C, int64_t gidx,
                                             int &n, int &c, int64_t &start, int &len) {
    if (p.cu) {
        if (gidx >= chunk_off[p.num_seqs]) return false;
        int lo = 0, hi = p.num_seqs - 1;  // largest n with chunk_off[n] <= gidx
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_off[mid] <= gidx) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        c = (int)(gidx - chunk_off[n]);
        start = p.cu[n];
        len = p.cu[n + 1] - p.cu[n];
    } else {
        const int per = (p.T + C - 1) / C;
        if (per == 0 || gidx >= (int64_t)p.num_seqs * per) return false;
        n = (int)(gidx / per);
        c = (int)(gidx % per);
        start = (int64_t)n * p.T;
        len = p.T;
    }
    return true;
}

__device__ __forceinline__ int64_t first_chunk(const FwdParams &p, const int32_t *chunk_off, int C, int n) {
    if (p.cu) return chunk_off[n];
    return (int64_t)n * ((p.T + C - 1) / C);
}

// ------------------------------------------------------------------- prep ----
template <typename IO, int DK, int C, bool PRO = false>
struct PrepLayout {
    using Rec = SplitRecord<IO, DK, C>;
    static constexpr bool BF = Rec::BF;
    using OT = typename std::conditional<BF, uint16_t, float>::type;
    static constexpr int NSUB = C / 16, KT = DK / 16;
    // one wave per sub-chunk, and at least d_k threads for the per-channel factors
    static constexpr int NT = 64 * (NSUB > DK / 64 ? NSUB : DK / 64);
    static constexpr int PADO = 16 / (int)sizeof(OT);
    static constexpr int LDO = DK + PADO;
    static constexpr int LDX = C + 4;
    static constexpr int NSHIFT = NSUB >= 3 ? (NSUB - 1) * (NSUB - 2) / 2 : 0;
    // K_b rows of every sub-chunk but the last, whose K_b is never a column operand
    static constexpr int KB_ROWS = C - 16;
    static constexpr size_t oKb = 0;
    static constexpr size_t oX = oKb + (size_t)KB_ROWS * LDO * sizeof(OT);
    static constexpr size_t oTot = oX + (size_t)C * LDX * 4;
    static constexpr size_t oEB = oTot + (size_t)NSUB * DK * 4;
    static constexpr size_t oEC = oEB + (size_t)NSUB * DK * 4;
    static constexpr size_t oSH = oEC + (size_t)NSUB * DK * 4;
    static constexpr size_t oBeta = oSH + (size_t)(NSHIFT > 0 ? NSHIFT : 1) * DK * 4;
    static constexpr size_t oTap = oBeta + (size_t)C * 4;  // the fused prologue's q and k filter taps
    static constexpr size_t kBytes = oTap + (PRO ? (size_t)2 * DK * 16 : 0);
    __host__ __device__ static constexpr int shift_slot(int R, int I) { return (R - 2) * (R - 1) / 2 + I; }
};

// Several workgroups per CU (4 waves each; see kPrepWaves): each spends much of its time waiting
// for its loads, and the waves of the other workgroups hide it.
// PRO: the inputs are the raw projections and phase 1 applies the prologue as it loads them (see
// FwdParams::conv): each lane's raw k and q for its token, the three tokens before it from its row
// neighbours by DPP row shifts (the first three lanes of a row of 16 tokens also load the three
// tokens before the row, zero before the sequence start), the 4-tap causal convolution and Swish
// in fp32, then the L2 norm over the token's d_k channels (the four lanes of a token);
// g = -softplus(g_raw) and beta = sigmoid(beta_raw) where read.
// Waves per SIMD the prep kernel is compiled for: four for bf16 io up to chunk 32 (128 registers;
// eight two-wave workgroups per CU at d_k = 128, chunk 32), three at chunk 64 (the row operands of
// phase 1 are kept for phase 3 instead of recomputed) and with the fused prologue, two for fp32 io.
template <typename IO, int C, bool PRO>
constexpr int kPrepWaves = std::is_same<IO, float>::value ? 2 : (PRO || C >= 64) ? 3 : 4;
template <typename IO, int DK, int C, bool PRO = false>
__global__ void __launch_bounds__((PrepLayout<IO, DK, C, PRO>::NT), (kPrepWaves<IO, C, PRO>)) kda_prep_kernel(FwdParams p, const int32_t *__restrict__ chunk_off,
                                                       char *__restrict__ records) {
    using L = PrepLayout<IO, DK, C, PRO>;
    using Rec = typename L::Rec;
    using OT = typename L::OT;
    constexpr bool BF = L::BF;
    constexpr int NSUB = L::NSUB, KT = L::KT, NPAIR = Rec::NPAIR;
    constexpr int LDO = L::LDO, LDX = L::LDX;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OT *sKb = reinterpret_cast<OT *>(smem + L::oKb);
    float *sX = reinterpret_cast<float *>(smem + L::oX);
    float *sTot = reinterpret_cast<float *>(smem + L::oTot);
    float *sEB = reinterpret_cast<float *>(smem + L::oEB);
    float *sEC = reinterpret_cast<float *>(smem + L::oEC);
    float *sSH = reinterpret_cast<float *>(smem + L::oSH);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    const int H = p.H;
    const int h = (int)(blockIdx.x % H);
    const int64_t gidx = blockIdx.x / H;
    int n, c;
    int64_t start;
    int len;
    if (!locate_chunk(p, chunk_off, C, gidx, n, c, start, len)) return;
    const int clen = min(C, len - c * C);
    const int64_t tok0 = start + (int64_t)c * C;
    char *rec = records + (size_t)(gidx * H + h) * Rec::kBytes;

    // fused prologue: the head's q and k filter taps as 4-tap windows: [q | k][channel]
    [[maybe_unused]] const float4 *sTap = reinterpret_cast<const float4 *>(smem + L::oTap);
    if constexpr (PRO) {
        for (int i = tid; i < 2 * DK; i += L::NT) {
            float w4[4];
            conv_taps4(p.conv[i / DK] + ((int64_t)h * DK + i % DK) * p.conv_w, p.conv_w, w4);
            reinterpret_cast<float4 *>(smem + L::oTap)[i] = make_float4(w4[0], w4[1], w4[2], w4[3]);
        }
        __syncthreads();
    }

    // beta of the chunk's tokens to sBeta, issued before the sub-chunk loads: straight into LDS
    // (tokens past the chunk end are zeroed in phase 2), or, for the fused prologue, through a
    // register that phase 1 passes through the sigmoid
    [[maybe_unused]] float bta = 0.f;
    if (tid < C) {
        const float *bp = p.beta + (tok0 + min(tid, clen - 1)) * H + h;
        if constexpr (PRO) bta = *bp;
        else load_lds4(bp, sBeta);
    }

    // ================= 1: load sub-chunk, scan the gate (log2 domain)
    // The lane's k and q stay packed as loaded until they are used (bf16 pairs: exact, and half
    // the registers); fp32 io and the fused prologue, which forms them in fp32, keep fp32.
    constexpr bool PACKED = BF && !PRO;
    using KQ = typename std::conditional<PACKED, uint2, float4>::type;
    float G[KT][4];
    KQ kin[KT], qin[KT];
    // chunk 64: phase 1's k e^{G_r - b_R}, q e^{G_r - b_R} and k e^{b_{R+1} - G_r} stay in registers
    // for phase 3 (at three waves per SIMD); smaller chunks recompute them there (four waves)
    constexpr bool KEEPROW = NSUB >= 4;
    [[maybe_unused]] float krs[KEEPROW ? KT : 1][4], qrs[KEEPROW ? KT : 1][4], kbs[KEEPROW ? KT : 1][4];
    bool split = false;  // the sub-chunk decays too strongly for a single-anchor diagonal block
    if (wave < NSUB) {
        const int R = wave;
        const bool valid = 16 * R + l16 < clen;
        const int r = min(16 * R + l16, clen - 1);
        const int64_t row = ((tok0 + r) * H + h) * (int64_t)DK + 4 * q4;
        const float m = valid ? kLog2e : 0.f;
        if constexpr (PRO) {
            // token three back: inside the sequence (this or the previous chunk) or zero; loaded by
            // the first three lanes of each row only, the others take it from the lane three below
            const bool has3 = (int64_t)c * C + 16 * R + l16 - 3 >= 0 && l16 < 3;
            const int64_t row3 = ((tok0 + min(16 * R + l16 - 3, clen - 1)) * H + h) * (int64_t)DK + 4 * q4;
            // every load in flight first, packed as loaded
            using RKQ = typename std::conditional<BF, uint2, float4>::type;
            RKQ rk0[KT], rq0[KT], rk3[KT], rq3[KT];
            float4 rg[KT];
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const IO *kp = static_cast<const IO *>(p.k), *qp = static_cast<const IO *>(p.q);
                rg[ct] = *reinterpret_cast<const float4 *>(p.g + row + 16 * ct);
                rk0[ct] = *reinterpret_cast<const RKQ *>(kp + row + 16 * ct);
                rq0[ct] = *reinterpret_cast<const RKQ *>(qp + row + 16 * ct);
                rk3[ct] = has3 ? *reinterpret_cast<const RKQ *>(kp + row3 + 16 * ct) : RKQ{};
                rq3[ct] = has3 ? *reinterpret_cast<const RKQ *>(qp + row3 + 16 * ct) : RKQ{};
            }
            float kr[KT][4], qr[KT][4];
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                // one channel tile at a time: only its taps and temporaries are live
                __builtin_amdgcn_sched_barrier(0);
                const float4 k0 = unpack4<BF>(rk0[ct]), q0 = unpack4<BF>(rq0[ct]);
                const float4 k3 = unpack4<BF>(rk3[ct]), q3 = unpack4<BF>(rq3[ct]);
                const float gx[4] = {rg[ct].x, rg[ct].y, rg[ct].z, rg[ct].w};
                const float kx0[4] = {k0.x, k0.y, k0.z, k0.w}, kx3[4] = {k3.x, k3.y, k3.z, k3.w};
                const float qx0[4] = {q0.x, q0.y, q0.z, q0.w}, qx3[4] = {q3.x, q3.y, q3.z, q3.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ch = 16 * ct + 4 * q4 + j;
                    G[ct][j] = neg_softplus_f(gx[j]) * m;
                    const float4 tq = sTap[ch], tk = sTap[DK + ch];
                    // raw inputs of tokens t-3, t-2 and t-1: row neighbours, or (first lanes of the
                    // row) the token-three-back loads of lanes 0, 1 and 2
                    const float ka = row_shr<1>(kx0[j]), kb = row_shl<2>(kx3[j]);
                    const float kc = row_shr<2>(kx0[j]), kd = row_shl<1>(kx3[j]);
                    const float ke = row_shr<3>(kx0[j]);
                    const float qa = row_shr<1>(qx0[j]), qb = row_shl<2>(qx3[j]);
                    const float qc = row_shr<2>(qx0[j]), qd = row_shl<1>(qx3[j]);
                    const float qe = row_shr<3>(qx0[j]);
                    const float k1 = l16 >= 1 ? ka : kb, k2 = l16 >= 2 ? kc : kd, k3 = l16 >= 3 ? ke : kx3[j];
                    const float q1 = l16 >= 1 ? qa : qb, q2 = l16 >= 2 ? qc : qd, q3 = l16 >= 3 ? qe : qx3[j];
                    float ck = 0.f, cq = 0.f;
                    ck = fmaf(tk.x, k3, ck); ck = fmaf(tk.y, k2, ck);
                    ck = fmaf(tk.z, k1, ck); ck = fmaf(tk.w, kx0[j], ck);
                    cq = fmaf(tq.x, q3, cq); cq = fmaf(tq.y, q2, cq);
                    cq = fmaf(tq.z, q1, cq); cq = fmaf(tq.w, qx0[j], cq);
                    kr[ct][j] = swish_f(ck);
                    qr[ct][j] = swish_f(cq);
                    sk = fmaf(kr[ct][j], kr[ct][j], sk);
                    sq = fmaf(qr[ct][j], qr[ct][j], sq);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // L2 norm over the token's channels: the four lanes 16 apart hold a quarter each
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            const float rk = valid ? rsqrtf(sk + p.norm_eps) : 0.f, rq = valid ? rsqrtf(sq + p.norm_eps) : 0.f;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                kin[ct] = make_float4(kr[ct][0] * rk, kr[ct][1] * rk, kr[ct][2] * rk, kr[ct][3] * rk);
                qin[ct] = make_float4(qr[ct][0] * rq, qr[ct][1] * rq, qr[ct][2] * rq, qr[ct][3] * rq);
            }
        } else {
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            const float4 gv = *reinterpret_cast<const float4 *>(p.g + row + 16 * ct);
            const KQ kv = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.k) + row + 16 * ct);
            const KQ qv = *reinterpret_cast<const KQ *>(static_cast<const IO *>(p.q) + row + 16 * ct);
            G[ct][0] = gv.x * m; G[ct][1] = gv.y * m; G[ct][2] = gv.z * m; G[ct][3] = gv.w * m;
            kin[ct] = valid ? kv : KQ{};
            qin[ct] = valid ? qv : KQ{};
        }
        }
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
            for (int j = 0; j < 4; ++j) G[ct][j] = scan16_add(G[ct][j]);
            if (l16 == 15)
                *reinterpret_cast<float4 *>(sTot + R * DK + 16 * ct + 4 * q4) =
                    make_float4(G[ct][0], G[ct][1], G[ct][2], G[ct][3]);
        }
        split = diag_needs_split<KT>(G);
        f32x4 dA = zero4(), dPt = zero4();
        if (split) {
            // This sub-chunk decays by more than 2^-96 in some channel: its diagonal blocks of A and
            // P come from the split levels (all factors <= 1, operands reloaded).
            if constexpr (PRO) {
                float kr[KT][4], qr[KT][4];
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) {
                    kr[ct][0] = kin[ct].x; kr[ct][1] = kin[ct].y; kr[ct][2] = kin[ct].z; kr[ct][3] = kin[ct].w;
                    qr[ct][0] = qin[ct].x; qr[ct][1] = qin[ct].y; qr[ct][2] = qin[ct].z; qr[ct][3] = qin[ct].w;
                }
                diag_block_split_regs<IO, KT>(dA, dPt, kr, qr, G, l16, q4, lane);
            } else {
                diag_block_split_rolled<IO>(dA, dPt, static_cast<const IO *>(p.k) + row,
                                            static_cast<const IO *>(p.q) + row, p.g + row, valid, KT, l16, q4, lane);
            }
        }
        // Per channel-tile pair: K_b = k e^{b_{R+1} - G} (the column operand of the later sub-chunks'
        // off-diagonal blocks) to LDS, and the diagonal blocks, which pair the row operands
        // k_r e^{G_r - b_R} (and the same for q) with the column operand k_i e^{b_R - G_i} (at most
        // 2^96 unless `split`, when the blocks above replace them).  The sub-chunk total of each
        // channel is in sTot (lane 15 of each row wrote it above).
        wave_lds_sync();
        f32x4 accA = zero4(), accPt = zero4();
#pragma unroll
        for (int kp = 0; kp < KT / 2; ++kp) {
            Frag<BF> fk[2], fq[2], fd[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ct = 2 * kp + u;
                const int ch = 16 * ct + 4 * q4;
                const float4 tot = *reinterpret_cast<const float4 *>(sTot + R * DK + ch);
                const float tv[4] = {tot.x, tot.y, tot.z, tot.w};
                const float4 kf = unpack4<PACKED>(kin[ct]), qf = unpack4<PACKED>(qin[ct]);
                const float kx[4] = {kf.x, kf.y, kf.z, kf.w}, qx[4] = {qf.x, qf.y, qf.z, qf.w};
                float kb[4], kd[4], kr[4], qr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fr = fast_exp2(G[ct][j]);          // e^{G_r - b_R}     <= 1
                    const float fb = fast_exp2(tv[j] - G[ct][j]);  // e^{b_{R+1} - G_r} <= 1
                    kr[j] = kx[j] * fr;
                    qr[j] = qx[j] * fr;
                    kb[j] = kx[j] * fb;
                    kd[j] = kb[j] * fast_exp2(-tv[j]);
                    if constexpr (KEEPROW) {
                        krs[ct][j] = kr[j];
                        qrs[ct][j] = qr[j];
                        kbs[ct][j] = kb[j];
                    }
                }
                fk[u] = make_frag<BF>(kr[0], kr[1], kr[2], kr[3]);
                fq[u] = make_frag<BF>(qr[0], qr[1], qr[2], qr[3]);
                fd[u] = make_frag<BF>(kd[0], kd[1], kd[2], kd[3]);
                if (R < NSUB - 1) {
                    const Frag<BF> fkb = make_frag<BF>(kb[0], kb[1], kb[2], kb[3]);
                    *reinterpret_cast<decltype(fkb.v) *>(sKb + (16 * R + l16) * LDO + ch) = fkb.v;
                }
            }
            mma32(accA, fk[0], fk[1], fd[0], fd[1]);   // A_RR:  rows r, columns i
            mma32(accPt, fd[0], fd[1], fq[0], fq[1]);  // P_RR^T: rows i, columns r
        }
        mfma_settle(accA, accPt);
        if (split) {
            accA = dA;
            accPt = dPt;
        }
        // A_RR (strictly lower, beta not yet applied) to its place in sX (lane: rows rr = 4*q4 + j,
        // column l16); P_RR to its fragment of the record (the P_RR^T accumulator is the P_RR
        // operand fragment: row l16, columns 4*q4 + j)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 4 * q4 + j;
            sX[(16 * R + rr) * LDX + 16 * R + l16] = l16 < rr ? accA[j] : 0.f;
        }
        {
            float pv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[j] = 4 * q4 + j > l16 ? 0.f : accPt[j];
            const Frag<BF> fp = make_frag<BF>(pv[0], pv[1], pv[2], pv[3]);
            char *tile = rec + Rec::oP + Rec::tp_off(R, R / 2);
            // even R: the half tile is this fragment alone; odd R: the right fragment of the pair
            if (Rec::tp_half(R, R / 2)) store_frag<BF>(tile, lane, fp);
            else *reinterpret_cast<decltype(fp.v) *>(tile + lane * Rec::PAIR_BYTES + Rec::FRAG_BYTES) = fp.v;
        }
    }
    if constexpr (PRO) {
        if (tid < C) sBeta[tid] = tid < clen ? sigmoid_f(bta) : 0.f;
    } else if (wave == 0) {
        wait_vmcnt<0>();  // the beta loads into LDS are complete
    }
    __syncthreads();

    // ================= 2: per-channel boundary factors; Gamma = e^{G_C}
    if constexpr (!PRO) {
        if (tid < C && tid >= clen) sBeta[tid] = 0.f;
    }
    if (tid < DK) {
        const int ch = tid;
        float tot[NSUB], bnd[NSUB + 1];
        bnd[0] = 0.f;
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            tot[R] = sTot[R * DK + ch];
            bnd[R + 1] = bnd[R] + tot[R];
        }
        const float gc = bnd[NSUB];
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            sEB[R * DK + ch] = fast_exp2(bnd[R]);
            sEC[R * DK + ch] = fast_exp2(gc - bnd[R + 1]);
#pragma unroll
            for (int I = 0; I + 2 <= R; ++I) sSH[L::shift_slot(R, I) * DK + ch] = fast_exp2(bnd[R] - bnd[I + 1]);
        }
        reinterpret_cast<float *>(rec + Rec::oGam)[ch] = fast_exp2(gc);
    }
    __syncthreads();

    // ================= 3: gated operands and the off-diagonal blocks of A and P.
    // K~ and Q~ go straight to the record; K- is transposed in registers by a product with the
    // identity (exact: every term is the operand times 1 or 0), which leaves this sub-chunk's half
    // of each K-^T operand tile in fragment layout.  Block (R, I), I < R, pairs the row operands
    // k_r e^{G_r - b_{I+1}} (and the same for q) with the column operand K_b of sub-chunk I (in
    // LDS since phase 1); for I <= R - 2 the row operands take the extra factor
    // e^{b_R - b_{I+1}} <= 1.  Each channel-tile pair adds its part to every block as soon as its
    // row operands exist, so no row operand outlives its pair.
    if (wave < NSUB) {
        const int R = wave;
        Frag<BF> eye;  // identity as a B operand: rows 4*q4 + j, column l16
        {
            float e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = (4 * q4 + j == l16) ? 1.f : 0.f;
            eye = make_frag<BF>(e[0], e[1], e[2], e[3]);
        }
        char *kbt_half = rec + Rec::oKbT + (size_t)(R / 2) * Rec::TILE_BYTES + lane * Rec::PAIR_BYTES +
                         (R % 2) * Rec::FRAG_BYTES;
        constexpr int NOFF = NSUB > 1 ? NSUB - 1 : 1;
        f32x4 accA[NOFF], accPt[NOFF];
#pragma unroll
        for (int I = 0; I < NOFF; ++I) {
            accA[I] = zero4();
            accPt[I] = zero4();
        }
#pragma unroll
        for (int kp = 0; kp < KT / 2; ++kp) {
            Frag<BF> fkt[2], fqt[2];
            float kr[2][4], qr[2][4];  // k and q times e^{G_r - b_R}
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ct = 2 * kp + u;
                const int ch = 16 * ct + 4 * q4;
                const float4 eb = *reinterpret_cast<const float4 *>(sEB + R * DK + ch);
                const float4 ec = *reinterpret_cast<const float4 *>(sEC + R * DK + ch);
                const float ebv[4] = {eb.x, eb.y, eb.z, eb.w};
                const float ecv[4] = {ec.x, ec.y, ec.z, ec.w};
                float kb[4];
                if constexpr (KEEPROW) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kr[u][j] = krs[ct][j];
                        qr[u][j] = qrs[ct][j];
                        kb[j] = kbs[ct][j];
                    }
                } else {  // the same values as phase 1's
                    const float4 tot = *reinterpret_cast<const float4 *>(sTot + R * DK + ch);
                    const float tv[4] = {tot.x, tot.y, tot.z, tot.w};
                    const float4 kf = unpack4<PACKED>(kin[ct]), qf = unpack4<PACKED>(qin[ct]);
                    const float kx[4] = {kf.x, kf.y, kf.z, kf.w}, qx[4] = {qf.x, qf.y, qf.z, qf.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float fr = fast_exp2(G[ct][j]);          // e^{G_r - b_R}     <= 1
                        const float fb = fast_exp2(tv[j] - G[ct][j]);  // e^{b_{R+1} - G_r} <= 1
                        kr[u][j] = kx[j] * fr;
                        qr[u][j] = qx[j] * fr;
                        kb[j] = kx[j] * fb;
                    }
                }
                float kt[4], qt[4], kbar[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kt[j] = kr[u][j] * ebv[j];
                    qt[j] = qr[u][j] * ebv[j];
                    kbar[j] = kb[j] * ecv[j];
                }
                fkt[u] = make_frag<BF>(kt[0], kt[1], kt[2], kt[3]);
                fqt[u] = make_frag<BF>(qt[0], qt[1], qt[2], qt[3]);
                f32x4 kbt = zero4();
                mma16(kbt, make_frag<BF>(kbar[0], kbar[1], kbar[2], kbar[3]), eye);
                const Frag<BF> fkbt = frag_from_acc<BF>(kbt);
                *reinterpret_cast<decltype(fkbt.v) *>(kbt_half + (size_t)ct * NPAIR * Rec::TILE_BYTES) = fkbt.v;
            }
            store_pair<BF>(rec + Rec::oKt + (size_t)(R * (KT / 2) + kp) * Rec::TILE_BYTES, lane, fkt[0], fkt[1]);
            store_pair<BF>(rec + Rec::oQt + (size_t)(R * (KT / 2) + kp) * Rec::TILE_BYTES, lane, fqt[0], fqt[1]);
            const int ct = 2 * kp;
#pragma unroll
            for (int I = 0; I < NSUB - 1; ++I) {
                if (I >= R) break;
                const OT *colp = sKb + (16 * I + l16) * LDO;
                const Frag<BF> b0 = lds_frag(colp + 16 * ct + 4 * q4);
                const Frag<BF> b1 = lds_frag(colp + 16 * (ct + 1) + 4 * q4);
                Frag<BF> ka0, ka1, qa0, qa1;
                if (I + 2 <= R) {
                    const float *shp = sSH + L::shift_slot(R, I) * DK + 4 * q4;
                    const float4 s0 = *reinterpret_cast<const float4 *>(shp + 16 * ct);
                    const float4 s1 = *reinterpret_cast<const float4 *>(shp + 16 * (ct + 1));
                    ka0 = make_frag<BF>(kr[0][0] * s0.x, kr[0][1] * s0.y, kr[0][2] * s0.z, kr[0][3] * s0.w);
                    ka1 = make_frag<BF>(kr[1][0] * s1.x, kr[1][1] * s1.y, kr[1][2] * s1.z, kr[1][3] * s1.w);
                    qa0 = make_frag<BF>(qr[0][0] * s0.x, qr[0][1] * s0.y, qr[0][2] * s0.z, qr[0][3] * s0.w);
                    qa1 = make_frag<BF>(qr[1][0] * s1.x, qr[1][1] * s1.y, qr[1][2] * s1.z, qr[1][3] * s1.w);
                } else {
                    ka0 = make_frag<BF>(kr[0][0], kr[0][1], kr[0][2], kr[0][3]);
                    ka1 = make_frag<BF>(kr[1][0], kr[1][1], kr[1][2], kr[1][3]);
                    qa0 = make_frag<BF>(qr[0][0], qr[0][1], qr[0][2], qr[0][3]);
                    qa1 = make_frag<BF>(qr[1][0], qr[1][1], qr[1][2], qr[1][3]);
                }
                mma32(accA[I], ka0, ka1, b0, b1);   // A_RI:  rows r, columns i
                mma32(accPt[I], b0, b1, qa0, qa1);  // P_RI^T: rows i, columns r
            }
        }
        if (NSUB % 2 == 1 && R == NSUB - 1) {  // odd sub-chunk count: zero the unused half of the last pair
            const Frag<BF> z = make_frag<BF>(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
                *reinterpret_cast<decltype(z.v) *>(kbt_half + Rec::FRAG_BYTES + (size_t)ct * NPAIR * Rec::TILE_BYTES) = z.v;
        }
        // A_RI (times beta) to sX: lane holds rows rr = 4*q4 + j, column l16; P_RI^T accumulator =
        // P_RI operand fragment: row l16, columns 4*q4 + j
        Frag<BF> pf[2 * NPAIR];
#pragma unroll
        for (int I = 0; I < NSUB - 1; ++I) {
            if (I >= R) break;
            mfma_settle(accA[I], accPt[I]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 4 * q4 + j;
                sX[(16 * R + rr) * LDX + 16 * I + l16] = accA[I][j] * sBeta[16 * R + rr];
            }
            pf[I] = make_frag<BF>(accPt[I][0], accPt[I][1], accPt[I][2], accPt[I][3]);
        }
        // P tiles of row R; the fragment P_RR came from phase 1
#pragma unroll
        for (int pp = 0; pp < NPAIR; ++pp)
            if (2 * pp + 1 < R) {
                store_pair<BF>(rec + Rec::oP + Rec::tp_off(R, pp), lane, pf[2 * pp], pf[2 * pp + 1]);
            } else if (2 * pp + 1 == R) {  // odd R: the left fragment P_R,R-1 of the tile holding P_RR
                *reinterpret_cast<decltype(pf[0].v) *>(rec + Rec::oP + Rec::tp_off(R, pp) + lane * Rec::PAIR_BYTES) =
                    pf[2 * pp].v;
            }

        // X_RR = (I + Diag(beta) A_RR)^{-1}, row by row (phase 1 left A_RR without beta); lane l16
        // owns column l16
        float *Ab = sX + (16 * R) * LDX + 16 * R;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float br = sBeta[16 * R + r];
            float s = (r == l16) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) {
                const float a = Ab[r * LDX + m] * br;
                s -= a * x[m];
            }
            x[r] = s;
        }
        if (q4 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Ab[r * LDX + l16] = x[r];
        }
    }
    __syncthreads();

    // ================= 4: off-diagonal blocks of X, one block diagonal at a time:
    // X_RI = -X_RR sum_{J=I}^{R-1} A_RJ X_JI  (fp32 matrix-core products).
    // sX holds A_RI below the diagonal (kept), X_RR on the diagonal, and X_RI transposed in
    // the otherwise unused upper block (I, R): X_RI[a][b] at sX[(16I + b) * LDX + 16R + a].
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
                Frag<false> b;  // X_JI: rows 4*q4 + j, column l16
                if (J == I) {
                    const float *xd = sX + (16 * I + 4 * q4) * LDX + 16 * I + l16;
                    b.v = make_float4(xd[0], xd[LDX], xd[2 * LDX], xd[3 * LDX]);
                } else {
                    b = lds_frag(sX + (16 * I + l16) * LDX + 16 * J + 4 * q4);
                }
                mma16(m, a, b);
            }
            f32x4 xo = zero4();
            const Frag<false> xrr = lds_frag(sX + (16 * R + l16) * LDX + 16 * R + 4 * q4);
            Frag<false> mb;
            mb.v = make_float4(-m[0], -m[1], -m[2], -m[3]);
            mma16(xo, xrr, mb);
            // xo holds X_RI rows 4*q4 + j, column l16: store transposed in block (I, R)
            *reinterpret_cast<float4 *>(sX + (16 * I + l16) * LDX + 16 * R + 4 * q4) = make_float4(xo[0], xo[1], xo[2], xo[3]);
        }
        __syncthreads();
    }

    // ================= 5: T = X Diag(beta) to the record
    if (wave < NSUB) {
        const int R = wave;
#pragma unroll
        for (int pp = 0; pp < NPAIR; ++pp) {
            if (2 * pp > R) break;
            Frag<BF> f[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int I = 2 * pp + u;
                float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (I == R) {
                    xv = *reinterpret_cast<const float4 *>(sX + (16 * R + l16) * LDX + 16 * R + 4 * q4);
                } else if (I < R) {  // X_RI[l16][4*q4 + j], stored transposed
                    const float *xt = sX + (16 * I + 4 * q4) * LDX + 16 * R + l16;
                    xv = make_float4(xt[0], xt[LDX], xt[2 * LDX], xt[3 * LDX]);
                }
                const float4 bv = I < NSUB ? *reinterpret_cast<const float4 *>(sBeta + 16 * I + 4 * q4)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
                f[u] = make_frag<BF>(xv.x * bv.x, xv.y * bv.y, xv.z * bv.z, xv.w * bv.w);
            }
            if (Rec::tp_half(R, pp)) store_frag<BF>(rec + Rec::oT + Rec::tp_off(R, pp), lane, f[0]);
            else store_pair<BF>(rec + Rec::oT + Rec::tp_off(R, pp), lane, f[0], f[1]);
        }
    }
}

// ------------------------------------------------------------------- scan ----
// Workgroup = NW compute waves, each owning SPW 16-column slices of the state (with two
// slices every operand fragment read from LDS feeds two matrix-core products), plus the
// copy waves that stage each chunk's record and V tile in LDS.
//
// The output is produced transposed, O^T = S^T Q~^T + D^T P^T: the state's accumulator
// fragments are exactly the operand fragments of S^T, D's accumulator fragments those of
// D^T, and the record's Q~ and P fragments serve unchanged as Q~^T and P^T.  Each lane then
// holds 4 consecutive output columns of one token and stores them with one 8-byte write.
// Copy waves per scan workgroup with two or more record buffers (see ScanLayout).
constexpr int scan_copy_waves(int spw) { return spw == 1 ? 4 : 2; }

template <typename IO, int DK, int C, int SPW, int NW>
struct ScanLayout {
    using Rec = SplitRecord<IO, DK, C>;
    static constexpr int WCOLS = 16 * SPW;      // state columns per compute wave (SPW 16-column slices)
    static constexpr int DVT = WCOLS * NW;      // state columns per workgroup
    static constexpr size_t kVBytes = (size_t)C * DVT * sizeof(IO);  // V tile [C][DVT]
    static constexpr int V_PIECES = (int)(kVBytes / 16);
    // KEEP only: a per-compute-wave fp32 tile [16][LDK] through which the kept state and D leave
    // as 16-byte row segments (a few wide stores instead of one per accumulator element)
    static constexpr int LDK = WCOLS + 4;
    static constexpr size_t kKeepBytes = (size_t)NW * 16 * LDK * 4;
    // One record buffer holds a chunk's record and its V tile.  At least two (chunk c + 1 is
    // written while chunk c is read) where they fit with the kept-state tile; otherwise one (fp32
    // records at d_k = 128, chunk 64: 117 KB each), and the next chunk is written after a second
    // barrier per chunk, once every wave is done reading.
    static constexpr size_t kBufBytes = Rec::kBytes + kVBytes;
    static constexpr bool SINGLE = 2 * kBufBytes + kKeepBytes > 160 * 1024;
    // LDS that the output-wave scan places after the buffers: its S and D slots, two per compute
    // wave (SPW 16-column slices of the state in KT k tiles, and of D in 2 NPAIR row tiles).
    static constexpr size_t kOwSlotBytes =
        (size_t)2 * NW * SPW * (Rec::KT + 2 * Rec::NPAIR) * Rec::FRAG_BYTES * 64;
    static constexpr bool buffers_fit(int n) { return n * kBufBytes + kOwSlotBytes + kKeepBytes <= 160 * 1024; }
    // Buffers: as many as fit up to four, so that small records are loaded up to three chunks ahead.
    static constexpr int NBUF = SINGLE ? 1 : buffers_fit(4) ? 4 : buffers_fit(3) ? 3 : 2;
    // DIRECT (three or four buffers): the copy waves load each chunk from global memory straight
    // into its LDS buffer (16 bytes per lane), NBUF - 1 chunks ahead.  Otherwise they load into
    // registers and write LDS at the barrier that frees the buffer, which lets two buffers run two
    // chunks ahead.  Measured on bf16, d_k = 128: one 131,072-token sequence x 32 heads at chunk 32
    // (four buffers) 4.18 instead of 4.38 ms per forward call, 4 x 4,096 tokens x 16 heads at chunk
    // 32 with 64-column tiles (three) 0.234 instead of 0.299 ms; with two buffers the direct copy
    // (one chunk ahead) was slower, 0.246 instead of 0.219 ms at chunk 64.
    static constexpr bool DIRECT = !SINGLE && NBUF >= 3;
    // Copy waves.  Direct: every copy wave takes a share of every chunk.  Registers, two buffers:
    // pairs that hold one chunk each (two pairs take turns with 16-column compute waves, so each
    // chunk's loads are issued two chunks ahead; the wider compute waves need every register of
    // their SIMD and keep a single pair, one chunk ahead).  One buffer: a group of four holds the
    // next chunk.
    static constexpr int NCW = SINGLE ? 4 : scan_copy_waves(SPW);
    static constexpr int GROUP = SINGLE ? 4 : DIRECT ? NCW : 2;  // copy waves that share one chunk
    static constexpr int NT = 64 * (NW + NCW);  // threads (compute waves + copy waves)
    // [record 0 .. record NBUF-1][V 0 .. V NBUF-1]
    static constexpr size_t oV = (size_t)NBUF * Rec::kBytes;
    __host__ __device__ static constexpr size_t rec_off(int c) { return (size_t)(NBUF == 1 ? 0 : c % NBUF) * Rec::kBytes; }
    __host__ __device__ static constexpr size_t v_off(int c) { return oV + (size_t)(NBUF == 1 ? 0 : c % NBUF) * kVBytes; }
    static constexpr size_t kBytes = (size_t)NBUF * kBufBytes;
    static constexpr int UNITS_PER_WAVE = ((int)(Rec::kBytes / 1024) + V_PIECES / 64 + GROUP - 1) / GROUP;
    // (the V tile is copied in whole wave units: a 16-column bf16 tile needs C >= 32; register
    // copies hold at most 40 units per lane, direct ones at most 63 loads in flight per wave)
    static constexpr bool kFits = kBytes <= 160 * 1024 && (!SINGLE || SPW == 1) && V_PIECES % 64 == 0 &&
                                  (DIRECT ? (NBUF - 1) * UNITS_PER_WAVE <= 63 : UNITS_PER_WAVE <= 40);
    static_assert(Rec::kBytes % (64 * 16) == 0, "record is copied in whole wave units");
    static constexpr bool kFitsKeep = kFits && kBytes + kKeepBytes <= 160 * 1024;
};

// One copy wave's share of a chunk's record and V tile (1 KB units dealt in turn to the GROUP
// waves that share a chunk; IDX is this wave's place in its group), 16 bytes per lane, either
// loaded into registers and later written to LDS (load, store) or loaded straight into LDS
// (issue; the layouts with ScanLayout::DIRECT).  With SKIP_QP the Q~ and P sections, which only
// the output uses, are not copied (their LDS stays stale and unread).
template <typename IO, int DK, int C, int SPW, int NW, int IDX, bool SKIP_QP = false>
struct ChunkStager {
    using S = ScanLayout<IO, DK, C, SPW, NW>;
    using Rec = typename S::Rec;
    static constexpr int REC_UNITS = (int)(Rec::kBytes / 1024);
    static constexpr int Q0 = (int)(Rec::oQt / 1024), Q1 = (int)(Rec::oKbT / 1024);
    static constexpr int P0 = (int)(Rec::oP / 1024), P1 = (int)(Rec::oGam / 1024);
    static_assert(Rec::oQt % 1024 == 0 && Rec::oKbT % 1024 == 0 && Rec::oP % 1024 == 0 && Rec::oGam % 1024 == 0,
                  "record sections start on copy units");
    static constexpr int USED = REC_UNITS - (SKIP_QP ? (Q1 - Q0) + (P1 - P0) : 0);  // record units copied
    static constexpr int UNITS = USED + S::V_PIECES / 64;
    // record unit of the j-th copied unit: the sections in order, Q~ and P left out with SKIP_QP
    __device__ static constexpr int rec_unit(int j) {
        if (SKIP_QP) {
            if (j >= Q0) j += Q1 - Q0;
            if (j >= P0) j += P1 - P0;
        }
        return j;
    }
    static constexpr int G = S::GROUP;
    static constexpr int PER = (UNITS - IDX + G - 1) / G;  // units of this wave
    static constexpr int EP = 16 / (int)sizeof(IO);
    static constexpr int PPR = S::DVT / EP;  // 16-byte pieces per V row
    // A native vector type: HIP's uint4 is a union that the compiler leaves in scratch
    // memory when it stays live across the copy loop.
    u32x4 r[PER];

    __device__ __forceinline__ void load(const char *rec, const IO *vrow0, int clen, int64_t vstride, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = IDX + G * i;
            if (u < USED) {
                r[i] = *reinterpret_cast<const u32x4 *>(rec + (size_t)rec_unit(u) * 1024 + lane * 16);
            } else {
                const int piece = (u - USED) * 64 + lane;
                const int row = min(piece / PPR, clen - 1);  // rows past the end re-read the last row
                r[i] = *reinterpret_cast<const u32x4 *>(vrow0 + row * vstride + (piece % PPR) * EP);
            }
        }
    }
    __device__ __forceinline__ void issue(const char *rec, const IO *vrow0, int clen, int64_t vstride, char *lds_rec,
                                          char *lds_v, int lane) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = IDX + G * i;
            if (u < USED) {
                load_lds16(rec + (size_t)rec_unit(u) * 1024 + lane * 16, lds_rec + rec_unit(u) * 1024);
            } else {
                const int piece = (u - USED) * 64 + lane;
                const int row = min(piece / PPR, clen - 1);  // rows past the end re-read the last row
                load_lds16(vrow0 + row * vstride + (piece % PPR) * EP, lds_v + (u - USED) * 1024);
            }
        }
    }
    __device__ __forceinline__ void store(char *lds_rec, char *lds_v, int lane) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = IDX + G * i;
            char *dst = u < USED ? lds_rec + rec_unit(u) * 1024 : lds_v + (u - USED) * 1024;
            *reinterpret_cast<u32x4 *>(dst + lane * 16) = r[i];
        }
    }
};

// Copy wave CW.  Barrier c hands chunk c to the compute waves; passing it also means every
// compute wave has finished chunk c - 1, so that buffer may take the next chunk.  DIRECT: the
// loads of chunk c + NBUF - 1 go into that buffer, and before barrier c + 1 each copy wave waits
// until its share of chunk c + 1 has landed (the newer chunks may still be in flight).  Registers,
// two buffers: group CW / GROUP stages the chunks j with j % NPAIR == CW / GROUP; the freed buffer
// takes chunk c + 1 from the registers of its group, which then load their next chunk.  One
// buffer: every chunk has a second barrier, after which every wave is done reading chunk c and
// chunk c + 1 (loaded while c was read) is written.
template <typename IO, int DK, int C, int SPW, int NW, int CW, bool SKIP_QP = false>
__device__ __forceinline__ void copy_wave(char *smem, const char *rec0, size_t rec_stride, const IO *vbase,
                                          int64_t vstride, int len, int nchunks, int lane) {
    using S = ScanLayout<IO, DK, C, SPW, NW>;
    constexpr int NPAIR = S::NCW / S::GROUP, PAIR = CW / S::GROUP;
    static_assert(!S::SINGLE || NPAIR == 1, "one buffer: one group of copy waves");
    ChunkStager<IO, DK, C, SPW, NW, CW % S::GROUP, SKIP_QP> st;
#define KDA_STAGE_LOAD(j) \
    st.load(rec0 + (size_t)(j) * rec_stride, vbase + (int64_t)(j) * C * vstride, min(C, len - (j) * C), vstride, lane)
#define KDA_STAGE_STORE(j) st.store(smem + S::rec_off(j), smem + S::v_off(j), lane)
#define KDA_STAGE_ISSUE(j)                                                                                \
    st.issue(rec0 + (size_t)(j) * rec_stride, vbase + (int64_t)(j) * C * vstride, min(C, len - (j) * C), \
             vstride, smem + S::rec_off(j), smem + S::v_off(j), lane)
    if constexpr (S::DIRECT) {
        constexpr int NB = S::NBUF;
        for (int j = 0; j < NB - 1 && j < nchunks; ++j) KDA_STAGE_ISSUE(j);
        wait_vmcnt<0>();
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();  // barrier c: chunk c is in LDS, the buffer of chunk c - 1 is free
            if (c + NB - 1 < nchunks) {
                KDA_STAGE_ISSUE(c + NB - 1);
                wait_vmcnt<(NB - 2) * decltype(st)::PER>();  // this wave's share of chunk c + 1 has landed
            } else {
                wait_vmcnt<0>();
            }
        }
    } else if constexpr (S::SINGLE) {
        if (nchunks > 0) {
            KDA_STAGE_LOAD(0);
            KDA_STAGE_STORE(0);
        }
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();  // barrier c: chunk c is in LDS
            if (c + 1 < nchunks) KDA_STAGE_LOAD(c + 1);
            __syncthreads();  // every wave is done reading chunk c
            if (c + 1 < nchunks) KDA_STAGE_STORE(c + 1);
        }
    } else if constexpr (NPAIR == 1) {
        if (nchunks > 0) {
            KDA_STAGE_LOAD(0);
            KDA_STAGE_STORE(0);
        }
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();
            if (c + 1 < nchunks) {
                KDA_STAGE_LOAD(c + 1);
                KDA_STAGE_STORE(c + 1);
            }
        }
    } else {
        // pair p stages the chunks j with j % NPAIR == p, each loaded NPAIR chunks ahead
        if (PAIR < nchunks) {
            KDA_STAGE_LOAD(PAIR);
            if (PAIR == 0) {
                KDA_STAGE_STORE(0);
                if (NPAIR < nchunks) KDA_STAGE_LOAD(NPAIR);
            }
        }
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();  // barrier c: the buffer of chunk c + 1 is free
            if ((c + 1) % NPAIR == PAIR && c + 1 < nchunks) {
                KDA_STAGE_STORE(c + 1);
                if (c + 1 + NPAIR < nchunks) KDA_STAGE_LOAD(c + 1 + NPAIR);
            }
        }
    }
#undef KDA_STAGE_LOAD
#undef KDA_STAGE_STORE
#undef KDA_STAGE_ISSUE
}

// Fused prologue (PRO) in the scans: V rows 16 r2 + 4 q4 + j (j < 4) of one column as the operator
// sees them: Swish of the 4-tap causal convolution (taps w4, FwdParams::conv[2]) of the raw rows
// staged in vb, the rows before the chunk from prev (that column's last three raw rows of the
// previous chunk; zero at the sequence start).
template <typename IO, int DVT>
__device__ __forceinline__ void conv_v4(const IO *vb, int col, int base, const float (&w4)[4], const float (&prev)[3],
                                        float (&out)[4]) {
    float x[7];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const int row = base - 3 + i;
        const float xv = elem_f32(vb[max(row, 0) * DVT + col]);
        x[i] = row >= 0 ? xv : (row == -3 ? prev[0] : (row == -2 ? prev[1] : prev[2]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float c = 0.f;
        c = fmaf(w4[0], x[j], c);
        c = fmaf(w4[1], x[j + 1], c);
        c = fmaf(w4[2], x[j + 2], c);
        c = fmaf(w4[3], x[j + 3], c);
        out[j] = swish_f(c);
    }
}

// KEEP: write each chunk's initial state and D (FwdParams::hs / dch) for the backward pass and
// no output (Q~ and P are neither staged nor used); a separate instantiation so the forward's
// register allocation is not affected.
template <typename IO, int DK, int C, int SPW, int NW, bool KEEP, bool PRO = false>
__global__ void __launch_bounds__((ScanLayout<IO, DK, C, SPW, NW>::NT)) kda_scan_kernel(FwdParams p, const int32_t *__restrict__ chunk_off,
                                                                  const char *__restrict__ records) {
    using S = ScanLayout<IO, DK, C, SPW, NW>;
    using Rec = typename S::Rec;
    constexpr bool BF = Rec::BF;
    constexpr int NSUB = Rec::NSUB, KT = Rec::KT, NPAIR = Rec::NPAIR, DVT = S::DVT, WC = S::WCOLS;
    using Tr = IoTraits<IO>;

    __shared__ __attribute__((aligned(16))) char smem[S::kBytes + (KEEP ? S::kKeepBytes : 0)];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
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
    const int nchunks = (len + C - 1) / C;
    const int64_t g0 = first_chunk(p, chunk_off, C, n);
    const int col0 = tile * DVT;
    const int64_t vstride = (int64_t)H * DV;  // elements between consecutive tokens of one head
    const IO *vbase = static_cast<const IO *>(p.v) + (start * H + h) * (int64_t)DV + col0;
    IO *obase = static_cast<IO *>(p.out) + (start * H + h) * (int64_t)DV + col0;
    const char *rec0 = records + (size_t)(g0 * H + h) * Rec::kBytes;
    const size_t rec_stride = (size_t)H * Rec::kBytes;

    if (wave >= NW) {
        switch (wave - NW) {
            case 0: copy_wave<IO, DK, C, SPW, NW, 0, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane); break;
            case 1: copy_wave<IO, DK, C, SPW, NW, 1, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane); break;
            case 2:
                if constexpr (S::NCW > 2)
                    copy_wave<IO, DK, C, SPW, NW, 2, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane);
                break;
            case 3:
                if constexpr (S::NCW > 3)
                    copy_wave<IO, DK, C, SPW, NW, 3, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane);
                break;
            case 4:
                if constexpr (S::NCW > 4)
                    copy_wave<IO, DK, C, SPW, NW, 4, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane);
                break;
            default:
                if constexpr (S::NCW > 5)
                    copy_wave<IO, DK, C, SPW, NW, 5, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane);
                break;
        }
        return;
    }

    // ---------------- compute waves: slice s holds state columns col0 + WC*wave + 16*s + l16
    f32x4 St[SPW][KT];
    [[maybe_unused]] float *keep_tile = KEEP ? reinterpret_cast<float *>(smem + S::kBytes) + wave * 16 * S::LDK : nullptr;
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int col = col0 + WC * wave + 16 * s + l16;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                St[s][ct][j] = p.s0 ? p.s0[sbase + (int64_t)(16 * ct + 4 * q4 + j) * DV + col] : 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);

    // The state as matrix-core B operand (bf16 or fp32), refreshed at the end of every chunk.
    Frag<BF> Sb[SPW][KT];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) Sb[s][ct] = frag_from_acc<BF>(St[s][ct]);

    // Record fragments are read from LDS in groups issued ahead of the products that use them:
    // the K~ and Q~ tiles of row tile rt two row tiles ahead, T after the first row tile, P and
    // the first half of K-^T after the second-to-last, the rest of K-^T after the last, and
    // Gamma before the state products.  Scheduling fences keep the compiler from sinking the
    // reads next to their uses.
    constexpr int KP = KT / 2;                        // 32-wide k pairs of d_k
    // fused prologue: V's filter taps for this lane's columns and the previous chunk's last raw rows
    [[maybe_unused]] float vw4[SPW][4], vprev[SPW][3];
    if constexpr (PRO) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            conv_taps4(p.conv[2] + ((int64_t)h * DV + col0 + WC * wave + 16 * s + l16) * p.conv_w, p.conv_w, vw4[s]);
            vprev[s][0] = vprev[s][1] = vprev[s][2] = 0.f;
        }
    }
    constexpr int GP = NSUB >= 2 ? NSUB - 2 : 0;      // row tile after which P and K-^T reads start
    constexpr int KT_H = (KT + 1) / 2;                // K-^T row tiles read at GP

    for (int c = 0; c < nchunks; ++c) {
        const int clen = min(C, len - c * C);
        __syncthreads();  // chunk c is in LDS
        // optional: the state entering this chunk, kept for the backward pass
        const int64_t slot_base = (g0 + c) * H + h;
        if constexpr (KEEP) {
            using OT = typename std::conditional<BF, uint16_t, float>::type;
            OT *hs = static_cast<OT *>(p.hs) + slot_base * DK * DV + col0 + WC * wave;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
                for (int s = 0; s < SPW; ++s)
#pragma unroll
                    for (int j = 0; j < 4; ++j) keep_tile[(4 * q4 + j) * S::LDK + 16 * s + l16] = St[s][ct][j];
                keep_rows<OT, WC, S::LDK>(hs + (int64_t)16 * ct * DV, DV, keep_tile, lane);
            }
        }
        const char *rb = smem + S::rec_off(c);
        const IO *vb = reinterpret_cast<const IO *>(smem + S::v_off(c));

        FragPair<BF> Kf[NSUB][KP], Qf[NSUB][KP], Tf[NSUB][NPAIR], Pf[NSUB][NPAIR], Bf[KT][NPAIR];
        // V as stored (converted where Y is formed), or with the fused prologue already applied
        typename std::conditional<PRO, float, IO>::type vv[SPW][NSUB][4];
        auto read_kq = [&](int rt) {
#pragma unroll
            for (int kp = 0; kp < KP; ++kp) {
                Kf[rt][kp] = ld_pair<BF>(rb + Rec::oKt + (size_t)(rt * KP + kp) * Rec::TILE_BYTES, lane);
                if constexpr (!KEEP)  // the kept forward computes no output: Q~ and P are not staged
                    Qf[rt][kp] = ld_pair<BF>(rb + Rec::oQt + (size_t)(rt * KP + kp) * Rec::TILE_BYTES, lane);
            }
        };
        auto read_kbt = [&](int ct0, int ct1) {
#pragma unroll
            for (int ct = ct0; ct < ct1; ++ct)
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    Bf[ct][pp] = ld_pair<BF>(rb + Rec::oKbT + (size_t)(ct * NPAIR + pp) * Rec::TILE_BYTES, lane);
        };
        read_kq(0);
        if constexpr (NSUB > 1) read_kq(1);
        __builtin_amdgcn_sched_barrier(0);

        // K~ S (for Y = V - K~ S) and O^T = S^T Q~^T, one row tile at a time
        f32x4 AK[SPW][NSUB], Ot[SPW][NSUB];
#pragma unroll
        for (int rt = 0; rt < NSUB; ++rt) {
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                AK[s][rt] = zero4();
                Ot[s][rt] = zero4();
            }
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
#pragma unroll
                for (int s = 0; s < SPW; ++s) {
                    mma32(AK[s][rt], Kf[rt][kp].a, Kf[rt][kp].b, Sb[s][2 * kp], Sb[s][2 * kp + 1]);
                    if constexpr (!KEEP) mma32(Ot[s][rt], Sb[s][2 * kp], Sb[s][2 * kp + 1], Qf[rt][kp].a, Qf[rt][kp].b);
                }
            __builtin_amdgcn_sched_barrier(0);
            if (rt + 2 < NSUB) read_kq(rt + 2);
            if (rt == 0) {
                if constexpr (PRO) {
#pragma unroll
                    for (int s = 0; s < SPW; ++s) {
                        const int vc = WC * wave + 16 * s + l16;
#pragma unroll
                        for (int r2 = 0; r2 < NSUB; ++r2) conv_v4<IO, DVT>(vb, vc, 16 * r2 + 4 * q4, vw4[s], vprev[s], vv[s][r2]);
#pragma unroll
                        for (int i = 0; i < 3; ++i) vprev[s][i] = elem_f32(vb[(C - 3 + i) * DVT + vc]);
                    }
                } else {
#pragma unroll
                for (int s = 0; s < SPW; ++s)
#pragma unroll
                    for (int r2 = 0; r2 < NSUB; ++r2)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            vv[s][r2][j] = vb[(16 * r2 + 4 * q4 + j) * DVT + WC * wave + 16 * s + l16];
                }
#pragma unroll
                for (int R = 0; R < NSUB; ++R)
#pragma unroll
                    for (int pp = 0; pp < NPAIR; ++pp)
                        if (2 * pp <= R)
                            Tf[R][pp] = ld_tp<BF, Rec>(rb + Rec::oT, R, pp, lane);
            }
            if (rt == GP) {
                if constexpr (!KEEP)
#pragma unroll
                    for (int R = 0; R < NSUB; ++R)
#pragma unroll
                        for (int pp = 0; pp < NPAIR; ++pp)
                            if (2 * pp <= R)
                                Pf[R][pp] = ld_tp<BF, Rec>(rb + Rec::oP, R, pp, lane);
                read_kbt(0, KT_H);
            }
            if (rt == NSUB - 1) read_kbt(KT_H, KT);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Y = V - K~ S as B fragments (rows past the chunk end hold finite filler; T zeroes them),
        // then D = T Y
        Frag<BF> Db[SPW][2 * NPAIR];
        {
            Frag<BF> Yb[SPW][2 * NPAIR];
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int rt = 0; rt < 2 * NPAIR; ++rt)
                    Yb[s][rt] = rt < NSUB ? make_frag<BF>(elem_f32(vv[s][rt][0]) - AK[s][rt][0],
                                                          elem_f32(vv[s][rt][1]) - AK[s][rt][1],
                                                          elem_f32(vv[s][rt][2]) - AK[s][rt][2],
                                                          elem_f32(vv[s][rt][3]) - AK[s][rt][3])
                                          : make_frag<BF>(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                f32x4 d[SPW];
#pragma unroll
                for (int s = 0; s < SPW; ++s) d[s] = zero4();
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    if (2 * pp <= R)
#pragma unroll
                        for (int s = 0; s < SPW; ++s) mma_tp_left<BF, Rec>(d[s], Tf[R][pp], Yb[s][2 * pp], Yb[s][2 * pp + 1], R, pp);
#pragma unroll
                for (int s = 0; s < SPW; ++s) Db[s][R] = frag_from_acc<BF>(d[s]);
                if constexpr (KEEP) {  // D of this chunk for the backward pass (operand type)
                    using OT = typename std::conditional<BF, uint16_t, float>::type;
#pragma unroll
                    for (int s = 0; s < SPW; ++s)
#pragma unroll
                        for (int j = 0; j < 4; ++j) keep_tile[(4 * q4 + j) * S::LDK + 16 * s + l16] = d[s][j];
                    keep_rows<OT, WC, S::LDK>(static_cast<OT *>(p.dch) + slot_base * C * DV + (int64_t)16 * R * DV +
                                                  col0 + WC * wave,
                                              DV, keep_tile, lane);
                }
            }
            if constexpr (NSUB % 2 == 1)
#pragma unroll
                for (int s = 0; s < SPW; ++s) Db[s][NSUB] = make_frag<BF>(0.f, 0.f, 0.f, 0.f);
        }

        // M = K-^T D (fresh accumulators) and O^T += D^T P^T; the state itself stays in plain
        // registers and is updated as S <- Gamma * S + M once the products are done
        float4 gm[KT];
        {
            const float *gam = reinterpret_cast<const float *>(rb + Rec::oGam);
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) gm[ct] = *reinterpret_cast<const float4 *>(gam + 16 * ct + 4 * q4);
        }
        // one record buffer: the last read of this chunk's record is done; the copy waves may
        // write the next chunk while the products below run
        if constexpr (S::SINGLE) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        f32x4 M[SPW][KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
            for (int s = 0; s < SPW; ++s) M[s][ct] = zero4();
#pragma unroll
            for (int pp = 0; pp < NPAIR; ++pp)
#pragma unroll
                for (int s = 0; s < SPW; ++s) mma32(M[s][ct], Bf[ct][pp].a, Bf[ct][pp].b, Db[s][2 * pp], Db[s][2 * pp + 1]);
        }
        if constexpr (!KEEP)
#pragma unroll
            for (int R = 0; R < NSUB; ++R)
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    if (2 * pp <= R)
#pragma unroll
                        for (int s = 0; s < SPW; ++s) mma_tp_right<BF, Rec>(Ot[s][R], Db[s][2 * pp], Db[s][2 * pp + 1], Pf[R][pp], R, pp);

#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                St[s][ct][0] = fmaf(gm[ct].x, St[s][ct][0], M[s][ct][0]);
                St[s][ct][1] = fmaf(gm[ct].y, St[s][ct][1], M[s][ct][1]);
                St[s][ct][2] = fmaf(gm[ct].z, St[s][ct][2], M[s][ct][2]);
                St[s][ct][3] = fmaf(gm[ct].w, St[s][ct][3], M[s][ct][3]);
                Sb[s][ct] = frag_from_acc<BF>(St[s][ct]);
            }

        // O rows of this chunk; lane holds columns 16 s + 4 q4 .. +3 of token 16 R + l16
        IO *oc = obase + (int64_t)c * C * vstride + WC * wave + 4 * q4;
#pragma unroll
        for (int R = 0; R < NSUB; ++R) {
            const int r = 16 * R + l16;
            if (!KEEP && r < clen) {
#pragma unroll
                for (int s = 0; s < SPW; ++s)
                    Tr::store4(oc + r * vstride + 16 * s, make_float4(Ot[s][R][0] * p.scale, Ot[s][R][1] * p.scale,
                                                                    Ot[s][R][2] * p.scale, Ot[s][R][3] * p.scale));
            }
        }
    }

    if (p.sf) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int col = col0 + WC * wave + 16 * s + l16;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) p.sf[sbase + (int64_t)(16 * ct + 4 * q4 + j) * DV + col] = St[s][ct][j];
        }
    }
}

// ------------------------------------------------ scan with output waves ----
// The same per-chunk algebra as kda_scan_kernel with the work split by what the recurrence
// needs: NW chain waves carry the state (Y = V - K~ S, D = T Y, S <- Gamma S + K-^T D), and NW
// output waves, one chunk behind, form O = scale (Q~ S + P D) for the same columns.  The chain
// waves hand S (at the start of each chunk) and D over through LDS slots that alternate with
// the chunk parity; an output wave reads Q~ and P of chunk c while chunk c is staged, keeps P in
// registers, and finishes O of chunk c after the next barrier, once D of chunk c is in its slot.
// The chain's share of each chunk drops from 5 to 3 products per 16-column slice and it issues
// no output stores.  The KEEP instantiation (the forward pass of the backward) has no output:
// its second group of waves writes each chunk's initial state and D to the workspace instead,
// from the same slots, and the copy waves leave Q~ and P out.
template <typename IO, int DK, int C, int SPW, int NW>
struct ScanOwLayout {
    using S = ScanLayout<IO, DK, C, SPW, NW>;
    using Rec = typename S::Rec;
    static constexpr int FB = Rec::FRAG_BYTES;
    static constexpr int SB_UNITS = SPW * Rec::KT * FB / 16;           // 16-byte units per lane: S operand
    static constexpr int DB_UNITS = SPW * 2 * Rec::NPAIR * FB / 16;    // 16-byte units per lane: D operand
    static constexpr int NT = 64 * (2 * NW + S::NCW);
    static constexpr size_t oSb = S::kBytes;                                     // [parity][wave][unit][lane]
    static constexpr size_t oDb = oSb + (size_t)2 * NW * SB_UNITS * 64 * 16;
    static constexpr size_t kBytes = oDb + (size_t)2 * NW * DB_UNITS * 64 * 16;
    static_assert(kBytes - S::kBytes == S::kOwSlotBytes, "slot bytes counted when choosing the buffers");
    static constexpr bool kFits = S::kFits && !S::SINGLE && kBytes <= 160 * 1024;
    // KEEP: after the slots, one fp32 [KROWS][LDK] tile per writer wave (kept rows leave through
    // it): 64 rows where they fit, so a chunk's state and D leave in 3 read-backs, else 16
    static constexpr int KROWS = kBytes + (size_t)NW * 64 * S::LDK * 4 <= 160 * 1024 ? 64 : 16;
    static constexpr size_t kKeepBytes = (size_t)NW * KROWS * S::LDK * 4;
    static constexpr bool kFitsKeep = S::kFits && !S::SINGLE && kBytes + kKeepBytes <= 160 * 1024;
    static_assert((Rec::KT * FB) % 16 == 0 && (2 * Rec::NPAIR * FB) % 16 == 0, "slot units");
};

// N operand fragments of one lane to / from an LDS slot laid out as [unit][lane] 16-byte units
template <bool BF, int N>
__device__ __forceinline__ void slot_put(char *slot, int lane, const Frag<BF> *f) {
    if constexpr (BF) {
#pragma unroll
        for (int u = 0; u < N / 2; ++u)
            *reinterpret_cast<uint4 *>(slot + (u * 64 + lane) * 16) =
                make_uint4(f[2 * u].v.x, f[2 * u].v.y, f[2 * u + 1].v.x, f[2 * u + 1].v.y);
    } else {
#pragma unroll
        for (int u = 0; u < N; ++u) *reinterpret_cast<float4 *>(slot + (u * 64 + lane) * 16) = f[u].v;
    }
}
template <bool BF, int N>
__device__ __forceinline__ void slot_get(const char *slot, int lane, Frag<BF> *f) {
    if constexpr (BF) {
#pragma unroll
        for (int u = 0; u < N / 2; ++u) {
            const uint4 x = *reinterpret_cast<const uint4 *>(slot + (u * 64 + lane) * 16);
            f[2 * u].v = make_uint2(x.x, x.y);
            f[2 * u + 1].v = make_uint2(x.z, x.w);
        }
    } else {
#pragma unroll
        for (int u = 0; u < N; ++u) f[u].v = *reinterpret_cast<const float4 *>(slot + (u * 64 + lane) * 16);
    }
}

template <typename IO, int DK, int C, int SPW, int NW, bool KEEP, bool PRO = false>
__global__ void __launch_bounds__((ScanOwLayout<IO, DK, C, SPW, NW>::NT)) kda_scan_ow_kernel(FwdParams p, const int32_t *__restrict__ chunk_off,
                                                                     const char *__restrict__ records) {
    using S = ScanLayout<IO, DK, C, SPW, NW>;
    using SO = ScanOwLayout<IO, DK, C, SPW, NW>;
    using Rec = typename S::Rec;
    constexpr bool BF = Rec::BF;
    constexpr int NSUB = Rec::NSUB, KT = Rec::KT, NPAIR = Rec::NPAIR, DVT = S::DVT, WC = S::WCOLS;
    using Tr = IoTraits<IO>;

    __shared__ __attribute__((aligned(16))) char smem[SO::kBytes + (KEEP ? SO::kKeepBytes : 0)];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
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
    const int nchunks = (len + C - 1) / C;
    const int64_t g0 = first_chunk(p, chunk_off, C, n);
    const int col0 = tile * DVT;
    const int64_t vstride = (int64_t)H * DV;
    const IO *vbase = static_cast<const IO *>(p.v) + (start * H + h) * (int64_t)DV + col0;
    const char *rec0 = records + (size_t)(g0 * H + h) * Rec::kBytes;
    const size_t rec_stride = (size_t)H * Rec::kBytes;
    constexpr int KP = KT / 2;
    constexpr int SBN = SPW * KT, DBN = SPW * 2 * NPAIR;  // fragments per lane in the S / D slots
    // Every wave passes nchunks + 1 barriers: one per chunk and a last one after which the
    // output waves finish the final chunk.
    if (wave >= 2 * NW) {
        switch (wave - 2 * NW) {
            case 0: copy_wave<IO, DK, C, SPW, NW, 0, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane); break;
            case 1: copy_wave<IO, DK, C, SPW, NW, 1, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane); break;
            case 2:
                if constexpr (S::NCW > 2)
                    copy_wave<IO, DK, C, SPW, NW, 2, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane);
                break;
            default:
                if constexpr (S::NCW > 3)
                    copy_wave<IO, DK, C, SPW, NW, 3, KEEP>(smem, rec0, rec_stride, vbase, vstride, len, nchunks, lane);
                break;
        }
        __syncthreads();
        return;
    }
    static_assert(S::NCW <= 4, "copy wave count");

    if (KEEP && wave >= NW) {
        // ---------------- writer waves (KEEP): the state entering chunk c and D of chunk c, in
        // the operand type, as 16-byte row segments of [slot, H, d_k, d_v] and [slot, H, C, d_v]
        using OT = typename std::conditional<BF, uint16_t, float>::type;
        const int ow = wave - NW;
        constexpr int KR = SO::KROWS, TPR = KR / 16;  // tile rows, 16-row fragments per read-back
        float *tile = reinterpret_cast<float *>(smem + SO::kBytes) + ow * KR * S::LDK;
        const int64_t cbase = g0 * H + h;  // slot of chunk 0
        // one 16 x 16 fragment per slice into 16-row block b of the tile (rows 16 b + 4 q4 + j,
        // column 16 s + l16); every TPR blocks the tile goes out as row segments
        auto put = [&](const Frag<BF> &f, int s, int b) {
            float x[4];
            if constexpr (BF) {
                x[0] = __uint_as_float(f.v.x << 16);
                x[1] = __uint_as_float(f.v.x & 0xffff0000u);
                x[2] = __uint_as_float(f.v.y << 16);
                x[3] = __uint_as_float(f.v.y & 0xffff0000u);
            } else {
                x[0] = f.v.x; x[1] = f.v.y; x[2] = f.v.z; x[3] = f.v.w;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) tile[(16 * b + 4 * q4 + j) * S::LDK + 16 * s + l16] = x[j];
        };
        auto write_d = [&](int cp) {
            Frag<BF> Db[SPW * 2 * NPAIR];
            slot_get<BF, DBN>(smem + SO::oDb + (size_t)(((cp & 1) * NW + ow) * SO::DB_UNITS) * 64 * 16, lane, Db);
            OT *dd = static_cast<OT *>(p.dch) + (cbase + (int64_t)cp * H) * C * DV + col0 + WC * ow;
            constexpr int DG = NSUB < TPR ? NSUB : TPR;  // 16-row blocks of D per read-back (divides NSUB)
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
#pragma unroll
                for (int s = 0; s < SPW; ++s) put(Db[s * 2 * NPAIR + R], s, R % DG);
                if (R % DG == DG - 1)
                    keep_rows<OT, WC, S::LDK, 16 * DG>(dd + (int64_t)16 * (R - DG + 1) * DV, DV, tile, lane);
            }
        };
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();  // S of chunk c and D of chunk c - 1 are in their slots
            if (c > 0) write_d(c - 1);
            Frag<BF> Sb[SPW * KT];
            slot_get<BF, SBN>(smem + SO::oSb + (size_t)(((c & 1) * NW + ow) * SO::SB_UNITS) * 64 * 16, lane, Sb);
            OT *hs = static_cast<OT *>(p.hs) + (cbase + (int64_t)c * H) * DK * DV + col0 + WC * ow;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
                for (int s = 0; s < SPW; ++s) put(Sb[s * KT + ct], s, ct % TPR);
                if (ct % TPR == TPR - 1)  // d_k / 16 is a multiple of TPR (d_k is 64 or 128)
                    keep_rows<OT, WC, S::LDK, KR>(hs + (int64_t)16 * (ct - TPR + 1) * DV, DV, tile, lane);
            }
        }
        __syncthreads();  // D of the last chunk is in its slot
        if (nchunks > 0) write_d(nchunks - 1);
        return;
    }
    if (!KEEP && wave >= NW) {
        // ---------------- output waves: slice s holds columns col0 + WC*ow + 16*s + l16
        const int ow = wave - NW;
        IO *obase = static_cast<IO *>(p.out) + (start * H + h) * (int64_t)DV + col0 + WC * ow + 4 * q4;
        f32x4 Ot[SPW][NSUB];
        FragPair<BF> Pf[NSUB][NPAIR];
        // O of chunk cp: add P D (D from its slot), scale, store; lane holds 4 columns of a token
        auto finish = [&](int cp) {
            Frag<BF> Db[SPW * 2 * NPAIR];
            slot_get<BF, DBN>(smem + SO::oDb + (size_t)(((cp & 1) * NW + ow) * SO::DB_UNITS) * 64 * 16, lane, Db);
#pragma unroll
            for (int R = 0; R < NSUB; ++R)
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    if (2 * pp <= R)
#pragma unroll
                        for (int s = 0; s < SPW; ++s)
                            mma_tp_right<BF, Rec>(Ot[s][R], Db[s * 2 * NPAIR + 2 * pp], Db[s * 2 * NPAIR + 2 * pp + 1],
                                                  Pf[R][pp], R, pp);
            const int clen = min(C, len - cp * C);
            IO *oc = obase + (int64_t)cp * C * vstride;
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                const int r = 16 * R + l16;
                if (r < clen) {
#pragma unroll
                    for (int s = 0; s < SPW; ++s)
                        Tr::store4(oc + r * vstride + 16 * s, make_float4(Ot[s][R][0] * p.scale, Ot[s][R][1] * p.scale,
                                                                        Ot[s][R][2] * p.scale, Ot[s][R][3] * p.scale));
                }
            }
        };
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();  // chunk c is in LDS; S of chunk c and D of chunk c - 1 are in their slots
            if (c > 0) finish(c - 1);
            const char *rb = smem + S::rec_off(c);
            Frag<BF> Sb[SPW * KT];
            slot_get<BF, SBN>(smem + SO::oSb + (size_t)(((c & 1) * NW + ow) * SO::SB_UNITS) * 64 * 16, lane, Sb);
            FragPair<BF> Qf[NSUB][KP];
#pragma unroll
            for (int rt = 0; rt < NSUB; ++rt)
#pragma unroll
                for (int kp = 0; kp < KP; ++kp)
                    Qf[rt][kp] = ld_pair<BF>(rb + Rec::oQt + (size_t)(rt * KP + kp) * Rec::TILE_BYTES, lane);
#pragma unroll
            for (int R = 0; R < NSUB; ++R)
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    if (2 * pp <= R)
                        Pf[R][pp] = ld_tp<BF, Rec>(rb + Rec::oP, R, pp, lane);
            // O^T = S^T Q~^T, one row tile at a time
#pragma unroll
            for (int rt = 0; rt < NSUB; ++rt) {
#pragma unroll
                for (int s = 0; s < SPW; ++s) Ot[s][rt] = zero4();
#pragma unroll
                for (int kp = 0; kp < KP; ++kp)
#pragma unroll
                    for (int s = 0; s < SPW; ++s)
                        mma32(Ot[s][rt], Sb[s * KT + 2 * kp], Sb[s * KT + 2 * kp + 1], Qf[rt][kp].a, Qf[rt][kp].b);
            }
        }
        __syncthreads();  // D of the last chunk is in its slot
        if (nchunks > 0) finish(nchunks - 1);
        return;
    }

    // ---------------- chain waves: slice s holds state columns col0 + WC*wave + 16*s + l16
    f32x4 St[SPW][KT];
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int col = col0 + WC * wave + 16 * s + l16;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                St[s][ct][j] = p.s0 ? p.s0[sbase + (int64_t)(16 * ct + 4 * q4 + j) * DV + col] : 0.f;
    }
    Frag<BF> Sb[SPW * KT];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) Sb[s * KT + ct] = frag_from_acc<BF>(St[s][ct]);
    slot_put<BF, SBN>(smem + SO::oSb + (size_t)(wave * SO::SB_UNITS) * 64 * 16, lane, Sb);

    constexpr int GP = NSUB >= 2 ? NSUB - 2 : 0;  // row tile after which the K-^T reads start
    // fused prologue: V's filter taps for this lane's columns and the previous chunk's last raw rows
    [[maybe_unused]] float vw4[SPW][4], vprev[SPW][3];
    if constexpr (PRO) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            conv_taps4(p.conv[2] + ((int64_t)h * DV + col0 + WC * wave + 16 * s + l16) * p.conv_w, p.conv_w, vw4[s]);
            vprev[s][0] = vprev[s][1] = vprev[s][2] = 0.f;
        }
    }
    constexpr int KT_H = (KT + 1) / 2;
    for (int c = 0; c < nchunks; ++c) {
        __syncthreads();  // chunk c is in LDS
        const char *rb = smem + S::rec_off(c);
        const IO *vb = reinterpret_cast<const IO *>(smem + S::v_off(c));

        FragPair<BF> Kf[NSUB][KP], Tf[NSUB][NPAIR], Bf[KT][NPAIR];
        typename std::conditional<PRO, float, IO>::type vv[SPW][NSUB][4];  // see kda_scan_kernel
        auto read_k = [&](int rt) {
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
                Kf[rt][kp] = ld_pair<BF>(rb + Rec::oKt + (size_t)(rt * KP + kp) * Rec::TILE_BYTES, lane);
        };
        auto read_kbt = [&](int ct0, int ct1) {
#pragma unroll
            for (int ct = ct0; ct < ct1; ++ct)
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    Bf[ct][pp] = ld_pair<BF>(rb + Rec::oKbT + (size_t)(ct * NPAIR + pp) * Rec::TILE_BYTES, lane);
        };
        read_k(0);
        if constexpr (NSUB > 1) read_k(1);
        __builtin_amdgcn_sched_barrier(0);

        // K~ S for Y = V - K~ S, one row tile at a time
        f32x4 AK[SPW][NSUB];
#pragma unroll
        for (int rt = 0; rt < NSUB; ++rt) {
#pragma unroll
            for (int s = 0; s < SPW; ++s) AK[s][rt] = zero4();
#pragma unroll
            for (int kp = 0; kp < KP; ++kp)
#pragma unroll
                for (int s = 0; s < SPW; ++s)
                    mma32(AK[s][rt], Kf[rt][kp].a, Kf[rt][kp].b, Sb[s * KT + 2 * kp], Sb[s * KT + 2 * kp + 1]);
            __builtin_amdgcn_sched_barrier(0);
            if (rt + 2 < NSUB) read_k(rt + 2);
            if (rt == 0) {
                if constexpr (PRO) {
#pragma unroll
                    for (int s = 0; s < SPW; ++s) {
                        const int vc = WC * wave + 16 * s + l16;
#pragma unroll
                        for (int r2 = 0; r2 < NSUB; ++r2) conv_v4<IO, DVT>(vb, vc, 16 * r2 + 4 * q4, vw4[s], vprev[s], vv[s][r2]);
#pragma unroll
                        for (int i = 0; i < 3; ++i) vprev[s][i] = elem_f32(vb[(C - 3 + i) * DVT + vc]);
                    }
                } else {
#pragma unroll
                for (int s = 0; s < SPW; ++s)
#pragma unroll
                    for (int r2 = 0; r2 < NSUB; ++r2)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            vv[s][r2][j] = vb[(16 * r2 + 4 * q4 + j) * DVT + WC * wave + 16 * s + l16];
                }
#pragma unroll
                for (int R = 0; R < NSUB; ++R)
#pragma unroll
                    for (int pp = 0; pp < NPAIR; ++pp)
                        if (2 * pp <= R)
                            Tf[R][pp] = ld_tp<BF, Rec>(rb + Rec::oT, R, pp, lane);
            }
            if (rt == GP) read_kbt(0, KT_H);
            if (rt == NSUB - 1) read_kbt(KT_H, KT);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Y = V - K~ S as B fragments (rows past the chunk end hold finite filler; T zeroes them),
        // then D = T Y, handed to the output waves
        Frag<BF> Db[SPW * 2 * NPAIR];
        {
            Frag<BF> Yb[SPW][2 * NPAIR];
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int rt = 0; rt < 2 * NPAIR; ++rt)
                    Yb[s][rt] = rt < NSUB ? make_frag<BF>(elem_f32(vv[s][rt][0]) - AK[s][rt][0],
                                                          elem_f32(vv[s][rt][1]) - AK[s][rt][1],
                                                          elem_f32(vv[s][rt][2]) - AK[s][rt][2],
                                                          elem_f32(vv[s][rt][3]) - AK[s][rt][3])
                                          : make_frag<BF>(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                f32x4 d[SPW];
#pragma unroll
                for (int s = 0; s < SPW; ++s) d[s] = zero4();
#pragma unroll
                for (int pp = 0; pp < NPAIR; ++pp)
                    if (2 * pp <= R)
#pragma unroll
                        for (int s = 0; s < SPW; ++s) mma_tp_left<BF, Rec>(d[s], Tf[R][pp], Yb[s][2 * pp], Yb[s][2 * pp + 1], R, pp);
#pragma unroll
                for (int s = 0; s < SPW; ++s) Db[s * 2 * NPAIR + R] = frag_from_acc<BF>(d[s]);
            }
            if constexpr (NSUB % 2 == 1)
#pragma unroll
                for (int s = 0; s < SPW; ++s) Db[s * 2 * NPAIR + NSUB] = make_frag<BF>(0.f, 0.f, 0.f, 0.f);
        }
        slot_put<BF, DBN>(smem + SO::oDb + (size_t)(((c & 1) * NW + wave) * SO::DB_UNITS) * 64 * 16, lane, Db);

        // M = K-^T D, then S <- Gamma * S + M; the new S goes to the output waves' next slot
        float4 gm[KT];
        {
            const float *gam = reinterpret_cast<const float *>(rb + Rec::oGam);
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) gm[ct] = *reinterpret_cast<const float4 *>(gam + 16 * ct + 4 * q4);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 M[SPW][KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
            for (int s = 0; s < SPW; ++s) M[s][ct] = zero4();
#pragma unroll
            for (int pp = 0; pp < NPAIR; ++pp)
#pragma unroll
                for (int s = 0; s < SPW; ++s)
                    mma32(M[s][ct], Bf[ct][pp].a, Bf[ct][pp].b, Db[s * 2 * NPAIR + 2 * pp], Db[s * 2 * NPAIR + 2 * pp + 1]);
        }
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                St[s][ct][0] = fmaf(gm[ct].x, St[s][ct][0], M[s][ct][0]);
                St[s][ct][1] = fmaf(gm[ct].y, St[s][ct][1], M[s][ct][1]);
                St[s][ct][2] = fmaf(gm[ct].z, St[s][ct][2], M[s][ct][2]);
                St[s][ct][3] = fmaf(gm[ct].w, St[s][ct][3], M[s][ct][3]);
                Sb[s * KT + ct] = frag_from_acc<BF>(St[s][ct]);
            }
        slot_put<BF, SBN>(smem + SO::oSb + (size_t)((((c + 1) & 1) * NW + wave) * SO::SB_UNITS) * 64 * 16, lane, Sb);
    }
    __syncthreads();  // matches the output waves' last barrier

    if (p.sf) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int col = col0 + WC * wave + 16 * s + l16;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) p.sf[sbase + (int64_t)(16 * ct + 4 * q4 + j) * DV + col] = St[s][ct][j];
        }
    }
}

// ----------------------------------------------------------------- launch ----
template <typename IO, int DK, int C>
constexpr size_t split_record_bytes() {
    return SplitRecord<IO, DK, C>::kBytes;
}

template <typename IO, int DK, int C, int SPW, int NW>
constexpr bool split_fits() {
    return ScanLayout<IO, DK, C, SPW, NW>::kFits && PrepLayout<IO, DK, C, true>::kBytes <= 160 * 1024;
}

// Workspace: [plan: chunk offsets and longest-first order, split_plan_bytes][records]
template <typename IO, int DK, int C, int SPW, int NW>
hipError_t launch_split_variant(const FwdParams &params, char *workspace, int64_t chunk_upper, hipStream_t stream) {
    FwdParams p = params;
    if (p.cu) p.order = plan_order(workspace, p.num_seqs);  // the scan runs the longest sequences first
    const bool keep = p.hs != nullptr;
    const bool pro = p.conv[0] != nullptr;  // fused prologue: the inputs are raw projections
    if constexpr (!split_fits<IO, DK, C, SPW, NW>()) {
        return hipErrorInvalidConfiguration;
    } else {
        if (keep && (!ScanLayout<IO, DK, C, SPW, NW>::kFitsKeep || p.out != nullptr || pro))
            return hipErrorInvalidConfiguration;  // the kept forward writes S and D, never O
        int32_t *chunk_off = reinterpret_cast<int32_t *>(workspace);
        char *records = workspace + split_plan_bytes(p.num_seqs);
        if (p.cu && !p.skip_prep) {
            hipError_t e = launch_plan(p.cu, p.num_seqs, C, workspace, stream);
            if (e != hipSuccess) return e;
        }
        const int64_t prep_blocks = chunk_upper * p.H;
        if (prep_blocks > 0 && !p.skip_prep) {
            if (pro)
                hipLaunchKernelGGL((kda_prep_kernel<IO, DK, C, true>), dim3((unsigned)prep_blocks),
                                   dim3(PrepLayout<IO, DK, C, true>::NT), 0, stream,
                                   p, chunk_off, records);
            else
                hipLaunchKernelGGL((kda_prep_kernel<IO, DK, C>), dim3((unsigned)prep_blocks),
                                   dim3(PrepLayout<IO, DK, C>::NT), 0, stream, p,
                                   chunk_off, records);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int64_t scan_blocks = (int64_t)p.num_seqs * p.H * (p.dv / ScanLayout<IO, DK, C, SPW, NW>::DVT);
        if (scan_blocks > 0) {
            if (keep) {
                if constexpr (ScanOwLayout<IO, DK, C, SPW, NW>::kFitsKeep)
                    hipLaunchKernelGGL((kda_scan_ow_kernel<IO, DK, C, SPW, NW, true>), dim3((unsigned)scan_blocks),
                                       dim3(ScanOwLayout<IO, DK, C, SPW, NW>::NT), 0, stream, p, chunk_off, records);
                else
                    hipLaunchKernelGGL((kda_scan_kernel<IO, DK, C, SPW, NW, true>), dim3((unsigned)scan_blocks),
                                       dim3(ScanLayout<IO, DK, C, SPW, NW>::NT), 0, stream, p, chunk_off, records);
            } else if constexpr (ScanOwLayout<IO, DK, C, SPW, NW>::kFits) {
                if (pro)
                    hipLaunchKernelGGL((kda_scan_ow_kernel<IO, DK, C, SPW, NW, false, true>), dim3((unsigned)scan_blocks),
                                       dim3(ScanOwLayout<IO, DK, C, SPW, NW>::NT), 0, stream, p, chunk_off, records);
                else
                    hipLaunchKernelGGL((kda_scan_ow_kernel<IO, DK, C, SPW, NW, false>), dim3((unsigned)scan_blocks),
                                       dim3(ScanOwLayout<IO, DK, C, SPW, NW>::NT), 0, stream, p, chunk_off, records);
            } else {
                if (pro)
                    hipLaunchKernelGGL((kda_scan_kernel<IO, DK, C, SPW, NW, false, true>), dim3((unsigned)scan_blocks),
                                       dim3(ScanLayout<IO, DK, C, SPW, NW>::NT), 0, stream, p, chunk_off, records);
                else
                    hipLaunchKernelGGL((kda_scan_kernel<IO, DK, C, SPW, NW, false>), dim3((unsigned)scan_blocks),
                                       dim3(ScanLayout<IO, DK, C, SPW, NW>::NT), 0, stream, p, chunk_off, records);
            }
            return hipGetLastError();
        }
        return hipSuccess;
    }
}

// F(DK, C, SPW, NW): NW compute waves of 16 * SPW state columns each (d_v tile 16 * SPW * NW)
#define KDA_SPLIT_SHAPES(F, DK_, C_) F(DK_, C_, 1, 1) F(DK_, C_, 1, 2) F(DK_, C_, 2, 2)
#define KDA_SPLIT_VARIANTS(F)                                                                          \
    KDA_SPLIT_SHAPES(F, 64, 16) KDA_SPLIT_SHAPES(F, 64, 32) KDA_SPLIT_SHAPES(F, 64, 64)                \
    KDA_SPLIT_SHAPES(F, 128, 16) KDA_SPLIT_SHAPES(F, 128, 32) KDA_SPLIT_SHAPES(F, 128, 64)

template <typename IO>
size_t split_record_size(int dk, int chunk) {
#define KDA_REC_CASE(DK_, C_, SPW_, NW_) \
    if (dk == DK_ && chunk == C_) return split_record_bytes<IO, DK_, C_>();
    KDA_SPLIT_VARIANTS(KDA_REC_CASE)
#undef KDA_REC_CASE
    return 0;
}

template <typename IO>
bool split_supported(int dk, int chunk, int spw, int nw, bool keep) {
#define KDA_FIT_CASE(DK_, C_, SPW_, NW_)                                       \
    if (dk == DK_ && chunk == C_ && spw == SPW_ && nw == NW_)                 \
        return split_fits<IO, DK_, C_, SPW_, NW_>() &&                        \
               (!keep || ScanLayout<IO, DK_, C_, SPW_, NW_>::kFitsKeep);
    KDA_SPLIT_VARIANTS(KDA_FIT_CASE)
#undef KDA_FIT_CASE
    return false;
}

// Workgroup size and LDS of the scan kernel the forward launches for a shape (the output-wave
// scan where its slots fit, else the single-role scan); false if the shape is not compiled.
template <typename IO>
bool split_scan_shape(int dk, int chunk, int spw, int nw, int &threads, int &lds) {
#define KDA_SHAPE_CASE(DK_, C_, SPW_, NW_)                                                   \
    if (dk == DK_ && chunk == C_ && spw == SPW_ && nw == NW_) {                              \
        if (!split_fits<IO, DK_, C_, SPW_, NW_>()) return false;                             \
        using SO = ScanOwLayout<IO, DK_, C_, SPW_, NW_>;                                     \
        using SL = ScanLayout<IO, DK_, C_, SPW_, NW_>;                                       \
        threads = SO::kFits ? SO::NT : SL::NT;                                               \
        lds = (int)(SO::kFits ? SO::kBytes : SL::kBytes);                                    \
        return true;                                                                         \
    }
    KDA_SPLIT_VARIANTS(KDA_SHAPE_CASE)
#undef KDA_SHAPE_CASE
    return false;
}

template <typename IO>
hipError_t launch_split(const FwdParams &p, int chunk, int spw, int nw, char *workspace, int64_t chunk_upper,
                        hipStream_t stream) {
#define KDA_SPLIT_CASE(DK_, C_, SPW_, NW_)                     \
    if (p.dk == DK_ && chunk == C_ && spw == SPW_ && nw == NW_) \
        return launch_split_variant<IO, DK_, C_, SPW_, NW_>(p, workspace, chunk_upper, stream);
    KDA_SPLIT_VARIANTS(KDA_SPLIT_CASE)
#undef KDA_SPLIT_CASE
    return hipErrorInvalidConfiguration;
}

}  // namespace kda
