// Chunkwise KDA forward for gfx950: one workgroup per (sequence, head, d_v tile),
// walking the sequence chunk by chunk with the state tile resident in registers.
//
// Method (Kimi Linear summary page, "Chunkwise parallel algorithm" and "Less compute
// than general DPLR" sections).  For a chunk of C tokens with in-chunk cumulative
// log-gate G_r = sum_{i<=r} g_i (per channel) and chunk-initial state S:
//
//   A  = Diag(beta) strictly_lower(K~ K^T)   K~ = k*e^{G}, K^ = k*e^{-G}  (from k and k)
//   P  = lower_incl_diag(Q~ K^T)             Q~ = q*e^{G}                 (from q and k)
//   D  = (I + A)^{-1} Diag(beta) (V - K~ S)  -- the UT transform T = (I+A)^{-1} Diag(beta)
//                                              applied to the residual (one inverse per
//                                              chunk, by forward substitution)
//   O  = scale (Q~ S + P D)                  -- inter-chunk part + intra-chunk part
//   S <- Diag(e^{G_C}) S + K-^T D            K- = k*e^{G_C - G}
//
// Only two C x C matrices exist (A and P): both DPLR vectors are tied to the key.
// The WY factors of the pages are W = T K~ and U = T V; D = U - W S is evaluated here as
// T (V - K~ S), which gives the same D but costs C*d_k*dvt instead of C^2*d_k per tile.
//
// Numerics.  Gates are handled in the log2 domain.  Inside A and P the factor
// e^{G_r - G_i} is split at 16-token sub-chunk boundaries b_R (G before sub-chunk R):
//   off-diagonal block (R > I):  [k_r e^{G_r-b_R}] [e^{b_R-b_{I+1}}] [k_i e^{b_{I+1}-G_i}]
//                                 every factor <= 1;
//   diagonal block (R == I):     [k_r e^{G_r-b_R} e^{-(b_{R+1}-b_R)}] [k_i e^{b_{R+1}-G_i}]
//                                 the row factor is >= 1 and overflows only when one
//                                 16-token sub-chunk decays a channel by more than e^-88.
// The operands of the inter-chunk products (K~, Q~, K-) carry factors <= 1.
//
// Work split inside the workgroup (4 waves):
//   wave R < C/16 owns sub-chunk R for the key-side work (loads, gate scan, operands,
//   the row-R blocks of A and P, and the diagonal inverse X_RR = (I + A_RR)^{-1});
//   every wave owns 16-column slices of the state tile for the state-side work.
// Operands are staged in LDS; all contractions run on the matrix cores (bf16 inputs
// with fp32 accumulation, or fp32 inputs for fp32 io).
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename IO, int DK, int DVT, int C>
struct ChunkLayout {
    static constexpr bool BF = IoTraits<IO>::kBf16;
    using OT = typename std::conditional<BF, uint16_t, float>::type;  // operand element in LDS
    static constexpr int NW = 4;
    static constexpr int NSUB = C / 16;
    static constexpr int KT = DK / 16;
    static constexpr int NSL = DVT / 16;
    static constexpr int SPW = NSL > NW ? NSL / NW : 1;
    static constexpr int PADO = 16 / (int)sizeof(OT);  // 16-byte row padding
    static constexpr int LDO = DK + PADO;               // [C][DK] operand tiles
    static constexpr int LDT = C + PADO;                // [DK][C] transposed K-bar
    static constexpr int LDA = C + 4;                   // fp32 [C][C]
    static_assert(C % 16 == 0 && NSUB >= 1 && NSUB <= NW, "chunk must be 16, 32 or 64");
    static_assert(DK % 32 == 0 && DVT % 16 == 0, "head dims");
    static_assert(NSL <= NW || NSL % NW == 0, "d_v tile");

    static constexpr size_t kOp = (size_t)C * LDO * sizeof(OT);
    static constexpr size_t oKb = 0;
    static constexpr size_t oKt = oKb + kOp;
    static constexpr size_t oQt = oKt + kOp;
    static constexpr size_t oKbT = oQt + kOp;
    static constexpr size_t oA = oKbT + (size_t)DK * LDT * sizeof(OT);
    static constexpr size_t oP = oA + (size_t)C * LDA * 4;
    static constexpr size_t oTot = oP + (size_t)C * LDA * 4;
    static constexpr size_t oEB = oTot + (size_t)NSUB * DK * 4;
    static constexpr size_t oED = oEB + (size_t)NSUB * DK * 4;
    static constexpr size_t oEC = oED + (size_t)NSUB * DK * 4;
    static constexpr size_t oSH = oEC + (size_t)NSUB * DK * 4;
    static constexpr size_t oGam = oSH + (size_t)NSUB * NSUB * DK * 4;
    static constexpr size_t oBeta = oGam + (size_t)DK * 4;
    static constexpr size_t kBytes = oBeta + (size_t)C * 4;
    static constexpr bool kFits = kBytes <= 160 * 1024;
};

template <typename IO, int DK, int DVT, int C>
__global__ void __launch_bounds__(kChunkThreads) kda_chunk_fwd_kernel(FwdParams p) {
    using L = ChunkLayout<IO, DK, DVT, C>;
    using OT = typename L::OT;
    constexpr bool BF = L::BF;
    constexpr int NSUB = L::NSUB, KT = L::KT, NSL = L::NSL, SPW = L::SPW;
    constexpr int LDO = L::LDO, LDT = L::LDT, LDA = L::LDA;
    using Tr = IoTraits<IO>;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OT *sKb = reinterpret_cast<OT *>(smem + L::oKb);
    OT *sKt = reinterpret_cast<OT *>(smem + L::oKt);
    OT *sQt = reinterpret_cast<OT *>(smem + L::oQt);
    OT *sKbT = reinterpret_cast<OT *>(smem + L::oKbT);
    float *sA = reinterpret_cast<float *>(smem + L::oA);
    float *sP = reinterpret_cast<float *>(smem + L::oP);
    float *sTot = reinterpret_cast<float *>(smem + L::oTot);
    float *sEB = reinterpret_cast<float *>(smem + L::oEB);
    float *sED = reinterpret_cast<float *>(smem + L::oED);
    float *sEC = reinterpret_cast<float *>(smem + L::oEC);
    float *sSH = reinterpret_cast<float *>(smem + L::oSH);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;

    const IO *__restrict__ Q = static_cast<const IO *>(p.q);
    const IO *__restrict__ K = static_cast<const IO *>(p.k);
    const IO *__restrict__ V = static_cast<const IO *>(p.v);
    IO *__restrict__ O = static_cast<IO *>(p.out);
    const int H = p.H, DV = p.dv;

    // ---- which (sequence, head, d_v tile) this workgroup owns
    const int ntile = DV / DVT;
    const int64_t nblocks = (int64_t)p.num_seqs * H * ntile;
    const int64_t item = xcd_grouped_block(blockIdx.x, nblocks);
    const int tile = (int)(item % ntile);
    const int64_t nh = item / ntile;
    const int h = (int)(nh % H);
    int n = (int)(nh / H);
    if (p.order) n = p.order[n];
    int64_t start;
    int len;
    if (p.cu) {
        start = p.cu[n];
        len = p.cu[n + 1] - p.cu[n];
    } else {
        start = (int64_t)n * p.T;
        len = p.T;
    }

    // ---- state slices owned by this wave: S[s][ct] holds rows 16ct+4q4+j of column col(s)
    f32x4 S[SPW][KT];
    const int64_t state_base = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int sl = wave + L::NW * s;
        const int col = tile * DVT + 16 * sl + l16;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ct + 4 * q4 + j;
                S[s][ct][j] = (p.s0 && sl < NSL) ? p.s0[state_base + (int64_t)row * DV + col] : 0.f;
            }
        }
    }

    for (int c0 = 0; c0 < len; c0 += C) {
        const int clen = min(C, len - c0);
        const int64_t tok0 = start + c0;

        // ================= phase 1: load the sub-chunk, scan the gate (log2 domain)
        float G[KT][4], kr[KT][4], qr[KT][4];
        if (wave < NSUB) {
            const int R = wave;
            const int r = 16 * R + l16;
            const bool valid = r < clen;
            const int64_t rowk = ((tok0 + r) * H + h) * (int64_t)DK;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const int c = 16 * ct + 4 * q4;
                float4 gv = make_float4(0.f, 0.f, 0.f, 0.f), kv = gv, qv = gv;
                if (valid) {
                    gv = *reinterpret_cast<const float4 *>(p.g + rowk + c);
                    kv = Tr::load4(K + rowk + c);
                    qv = Tr::load4(Q + rowk + c);
                }
                G[ct][0] = scan16_add(gv.x * kLog2e);
                G[ct][1] = scan16_add(gv.y * kLog2e);
                G[ct][2] = scan16_add(gv.z * kLog2e);
                G[ct][3] = scan16_add(gv.w * kLog2e);
                kr[ct][0] = kv.x; kr[ct][1] = kv.y; kr[ct][2] = kv.z; kr[ct][3] = kv.w;
                qr[ct][0] = qv.x; qr[ct][1] = qv.y; qr[ct][2] = qv.z; qr[ct][3] = qv.w;
                if (l16 == 15)
                    *reinterpret_cast<float4 *>(sTot + R * DK + c) = make_float4(G[ct][0], G[ct][1], G[ct][2], G[ct][3]);
            }
            if (q4 == 0) sBeta[r] = valid ? p.beta[(tok0 + r) * H + h] : 0.f;
        }
        __syncthreads();

        // ================= phase 2: per-channel boundary factors
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
                for (int I = 0; I + 1 < R; ++I) sSH[(R * NSUB + I) * DK + c] = fast_exp2(bnd[R] - bnd[I + 1]);
            }
            sGam[c] = fast_exp2(gc);
        }
        __syncthreads();

        // ================= phase 3: gated operands
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
                float kb[4], kt[4], qt[4], kbar[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fr = fast_exp2(G[ct][j]);          // e^{G_r - b_R}     <= 1
                    const float fb = fast_exp2(tv[j] - G[ct][j]);  // e^{b_{R+1} - G_r} <= 1
                    const float krow = kr[ct][j] * fr;
                    const float qrow = qr[ct][j] * fr;
                    kb[j] = kr[ct][j] * fb;
                    kt[j] = krow * ebv[j];
                    qt[j] = qrow * ebv[j];
                    kbar[j] = kb[j] * ecv[j];
                    kr[ct][j] = krow;  // keep the row operands for the A / P blocks
                    qr[ct][j] = qrow;
                }
                if constexpr (BF) {
                    *reinterpret_cast<uint2 *>(sKb + r * LDO + c) = make_frag<true>(kb[0], kb[1], kb[2], kb[3]).v;
                    *reinterpret_cast<uint2 *>(sKt + r * LDO + c) = make_frag<true>(kt[0], kt[1], kt[2], kt[3]).v;
                    *reinterpret_cast<uint2 *>(sQt + r * LDO + c) = make_frag<true>(qt[0], qt[1], qt[2], qt[3]).v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) sKbT[(c + j) * LDT + r] = f32_to_bf16(kbar[j]);
                } else {
                    *reinterpret_cast<float4 *>(sKb + r * LDO + c) = make_float4(kb[0], kb[1], kb[2], kb[3]);
                    *reinterpret_cast<float4 *>(sKt + r * LDO + c) = make_float4(kt[0], kt[1], kt[2], kt[3]);
                    *reinterpret_cast<float4 *>(sQt + r * LDO + c) = make_float4(qt[0], qt[1], qt[2], qt[3]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) sKbT[(c + j) * LDT + r] = kbar[j];
                }
            }
        }
        __syncthreads();

        // ================= phase 4: row-R blocks of A and P (MFMA)
        if (wave < NSUB) {
            const int R = wave;
#pragma unroll
            for (int I = 0; I < NSUB; ++I) {
                if (I > R) break;
                f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                for (int ct = 0; ct < KT; ct += 2) {
                    Frag<BF> ka[2], qa[2], kb[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int c = 16 * (ct + u) + 4 * q4;
                        float sh[4] = {1.f, 1.f, 1.f, 1.f};
                        if (I == R) {
                            const float4 e = *reinterpret_cast<const float4 *>(sED + R * DK + c);
                            sh[0] = e.x; sh[1] = e.y; sh[2] = e.z; sh[3] = e.w;
                        } else if (I + 1 < R) {
                            const float4 e = *reinterpret_cast<const float4 *>(sSH + (R * NSUB + I) * DK + c);
                            sh[0] = e.x; sh[1] = e.y; sh[2] = e.z; sh[3] = e.w;
                        }
                        const float *kk = kr[ct + u];
                        const float *qq = qr[ct + u];
                        ka[u] = make_frag<BF>(kk[0] * sh[0], kk[1] * sh[1], kk[2] * sh[2], kk[3] * sh[3]);
                        qa[u] = make_frag<BF>(qq[0] * sh[0], qq[1] * sh[1], qq[2] * sh[2], qq[3] * sh[3]);
                        kb[u] = lds_frag(sKb + (16 * I + l16) * LDO + c);
                    }
                    mma32(accA, ka[0], ka[1], kb[0], kb[1]);
                    mma32(accP, qa[0], qa[1], kb[0], kb[1]);
                }
                // accumulator: rows rr = 4*q4 + j of block R, column ii = l16 of block I
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * q4 + j, ii = l16;
                    float a = accA[j] * sBeta[16 * R + rr];
                    float pp = accP[j];
                    if (I == R) {
                        if (ii >= rr) a = 0.f;
                        if (ii > rr) pp = 0.f;
                    }
                    sA[(16 * R + rr) * LDA + 16 * I + ii] = a;
                    sP[(16 * R + rr) * LDA + 16 * I + ii] = pp;
                }
            }
        }
        __syncthreads();

        // ================= phase 5: diagonal inverses X_RR = (I + A_RR)^{-1}, row by row
        if (wave < NSUB) {
            const int R = wave;
            float *Ab = sA + (16 * R) * LDA + 16 * R;
            const int jc = l16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == jc) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s -= Ab[r * LDA + m] * x[m];
                x[r] = s;
            }
            if (q4 == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Ab[r * LDA + jc] = x[r];
            }
        }
        __syncthreads();

        // ================= phase 6: state slices (each wave: 16-column slices of the tile)
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int sl = wave + L::NW * s;
            if (sl >= NSL) break;
            const int col = tile * DVT + 16 * sl + l16;

            Frag<BF> Sb[KT];
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) Sb[ct] = frag_from_acc<BF>(S[s][ct]);

            f32x4 Y[NSUB], Oa[NSUB];
#pragma unroll
            for (int rt = 0; rt < NSUB; ++rt) {
                f32x4 ak = zero4(), ao = zero4();
#pragma unroll
                for (int ct = 0; ct < KT; ct += 2) {
                    const int cA = 16 * ct + 4 * q4, cB = cA + 16;
                    const OT *kt = sKt + (16 * rt + l16) * LDO;
                    const OT *qt = sQt + (16 * rt + l16) * LDO;
                    mma32(ak, lds_frag(kt + cA), lds_frag(kt + cB), Sb[ct], Sb[ct + 1]);
                    mma32(ao, lds_frag(qt + cA), lds_frag(qt + cB), Sb[ct], Sb[ct + 1]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * q4 + j;
                    const float vv = (r < clen) ? Tr::load1(V + ((tok0 + r) * H + h) * (int64_t)DV + col) : 0.f;
                    Y[rt][j] = sBeta[r] * (vv - ak[j]);
                }
                Oa[rt] = ao;
            }

            // D_R = X_RR (Y_R - sum_{I<R} A_RI D_I): block forward substitution
            Frag<BF> D[NSUB];
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
                f32x4 z = Y[R];
#pragma unroll
                for (int I = 0; I < R; ++I)
                    mma16(z, lds_frag_f32<BF>(sA + (16 * R + l16) * LDA + 16 * I + 4 * q4, -1.f), D[I]);
                f32x4 d = zero4();
                mma16(d, lds_frag_f32<BF>(sA + (16 * R + l16) * LDA + 16 * R + 4 * q4), frag_from_acc<BF>(z));
                D[R] = frag_from_acc<BF>(d);
            }

            // O = scale (Q~ S + P D)
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
#pragma unroll
                for (int I = 0; I <= R; ++I)
                    mma16(Oa[R], lds_frag_f32<BF>(sP + (16 * R + l16) * LDA + 16 * I + 4 * q4), D[I]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * q4 + j;
                    if (r < clen) Tr::store1(O + ((tok0 + r) * H + h) * (int64_t)DV + col, Oa[R][j] * p.scale);
                }
            }

            // S <- Diag(e^{G_C}) S + K-^T D
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const float4 gm = *reinterpret_cast<const float4 *>(sGam + 16 * ct + 4 * q4);
                S[s][ct][0] *= gm.x;
                S[s][ct][1] *= gm.y;
                S[s][ct][2] *= gm.z;
                S[s][ct][3] *= gm.w;
                const OT *kb = sKbT + (16 * ct + l16) * LDT + 4 * q4;
#pragma unroll
                for (int I = 0; I + 1 < NSUB; I += 2) mma32(S[s][ct], lds_frag(kb + 16 * I), lds_frag(kb + 16 * (I + 1)), D[I], D[I + 1]);
                if constexpr (NSUB % 2 == 1) mma16(S[s][ct], lds_frag(kb + 16 * (NSUB - 1)), D[NSUB - 1]);
            }
        }
        __syncthreads();
    }

    if (p.sf) {
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int sl = wave + L::NW * s;
            if (sl >= NSL) break;
            const int col = tile * DVT + 16 * sl + l16;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * ct + 4 * q4 + j;
                    p.sf[state_base + (int64_t)row * DV + col] = S[s][ct][j];
                }
            }
        }
    }
}

template <typename IO, int DK, int DVT, int C>
constexpr int chunk_lds_bytes() {
    using L = ChunkLayout<IO, DK, DVT, C>;
    return L::kFits ? (int)L::kBytes : 0;
}

template <typename IO, int DK, int DVT, int C>
hipError_t launch_chunk_variant(const FwdParams &p, hipStream_t stream) {
    if constexpr (!ChunkLayout<IO, DK, DVT, C>::kFits) {
        return hipErrorInvalidConfiguration;
    } else {
        const int64_t blocks = (int64_t)p.num_seqs * p.H * (p.dv / DVT);
        if (blocks <= 0) return hipSuccess;
        hipLaunchKernelGGL((kda_chunk_fwd_kernel<IO, DK, DVT, C>), dim3((unsigned)blocks), dim3(kChunkThreads), 0,
                           stream, p);
        return hipGetLastError();
    }
}

// Expands F(DK, DVT, C) over every compiled variant.
#define KDA_CHUNK_VARIANTS(F) \
    F(64, 32, 16) F(64, 32, 32) F(64, 32, 64) F(64, 64, 16) F(64, 64, 32) F(64, 64, 64) \
    F(128, 32, 16) F(128, 32, 32) F(128, 32, 64) F(128, 64, 16) F(128, 64, 32) F(128, 64, 64) \
    F(128, 128, 16) F(128, 128, 32) F(128, 128, 64)

template <typename IO>
int chunk_variant_lds(int dk, int dvt, int chunk) {
#define KDA_LDS_CASE(DK_, DVT_, C_) \
    if (dk == DK_ && dvt == DVT_ && chunk == C_) return chunk_lds_bytes<IO, DK_, DVT_, C_>();
    KDA_CHUNK_VARIANTS(KDA_LDS_CASE)
#undef KDA_LDS_CASE
    return 0;
}

template <typename IO>
hipError_t launch_chunk(const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream) {
#define KDA_LAUNCH_CASE(DK_, DVT_, C_) \
    if (p.dk == DK_ && cfg.dv_tile == DVT_ && cfg.chunk == C_) return launch_chunk_variant<IO, DK_, DVT_, C_>(p, stream);
    KDA_CHUNK_VARIANTS(KDA_LAUNCH_CASE)
#undef KDA_LAUNCH_CASE
    return hipErrorInvalidConfiguration;
}

}  // namespace kda
