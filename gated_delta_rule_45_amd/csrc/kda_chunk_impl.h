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
// Numerics.  Gates are handled in the log2 domain.  With b_R the cumulative gate before
// 16-token sub-chunk R, the factor e^{G_r - G_i} inside A and P is split as
//   off-diagonal block (R > I):  [k_r e^{G_r-b_R}] [k_i e^{b_{I+1}-G_i} e^{b_R-b_{I+1}}]
//                                 (row factor and both column factors <= 1);
//   diagonal block (R == I):     [k_r e^{G_r-b_R}] [k_i e^{b_R-G_i}]
//                                 (the column factor is >= 1 and overflows only when one
//                                 16-token sub-chunk decays a channel by more than e^-88).
// The operands of the inter-chunk products (K~, Q~, K-) carry factors <= 1.
//
// Work split inside the workgroup (4 waves, 4 barriers per chunk):
//   1. wave R < C/16 takes its 16-token sub-chunk from registers (prefetched during the
//      previous chunk), scans the gate with DPP; all threads stage V and beta in LDS;
//   2. per-channel boundary factors from the sub-chunk totals;
//   3. wave R builds the gated operands of its sub-chunk (K~, Q~, K-^T, column operands);
//   4. wave R computes the row-R blocks of A and P on the matrix cores and inverts its
//      diagonal block A_RR by forward substitution; the next chunk's loads are issued;
//   5. every wave updates its 16-column slices of the state tile (matrix cores).
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
    static constexpr int LDM = C + PADO;                // [C][C] A and P in operand type
    static constexpr int LDD = 16 + 4;                  // fp32 diagonal blocks [16][16]
    static constexpr int LDV = DVT + PADO;              // [C][DVT] staged V (io type == operand type)
    static constexpr int NSHIFT = NSUB >= 3 ? (NSUB - 1) * (NSUB - 2) / 2 : 0;  // pairs R >= I + 2
    static_assert(C % 16 == 0 && NSUB >= 1 && NSUB <= NW, "chunk must be 16, 32 or 64");
    static_assert(DK % 32 == 0 && DVT % 16 == 0, "head dims");
    static_assert(NSL <= NW || NSL % NW == 0, "d_v tile");

    // raw-input prefetch: V tile in 16-byte pieces spread over the workgroup
    static constexpr int V_PIECES = C * DVT * (int)sizeof(IO) / 16;
    static constexpr int V_PER_THREAD = (V_PIECES + kChunkThreads - 1) / kChunkThreads;
    static constexpr int V_ELEMS = 16 / (int)sizeof(IO);  // io elements per piece

    static constexpr size_t kOp = (size_t)C * LDO * sizeof(OT);
    static constexpr size_t oKb = 0;
    static constexpr size_t oKs = oKb + kOp;
    static constexpr size_t oKt = oKs + (size_t)NSHIFT * 16 * LDO * sizeof(OT);
    static constexpr size_t oQt = oKt + kOp;
    static constexpr size_t oKbT = oQt + kOp;
    static constexpr size_t oA = oKbT + (size_t)DK * LDT * sizeof(OT);
    static constexpr size_t oP = oA + (size_t)C * LDM * sizeof(OT);
    static constexpr size_t oAd = oP + (size_t)C * LDM * sizeof(OT);
    static constexpr size_t oV = oAd + (size_t)NSUB * 16 * LDD * 4;
    static constexpr size_t oTot = oV + (size_t)C * LDV * sizeof(OT);
    static constexpr size_t oEB = oTot + (size_t)NSUB * DK * 4;
    static constexpr size_t oED = oEB + (size_t)NSUB * DK * 4;
    static constexpr size_t oEC = oED + (size_t)NSUB * DK * 4;
    static constexpr size_t oSH = oEC + (size_t)NSUB * DK * 4;
    static constexpr size_t oGam = oSH + (size_t)(NSHIFT > 0 ? NSHIFT : 1) * DK * 4;
    static constexpr size_t oBeta = oGam + (size_t)DK * 4;
    static constexpr size_t kBytes = oBeta + (size_t)C * 4;
    static constexpr bool kFits = kBytes <= 160 * 1024;

    // index of the shifted column operand for block (R, I), R >= I + 2
    __host__ __device__ static constexpr int shift_slot(int R, int I) { return (R - 2) * (R - 1) / 2 + I; }
};

// Raw inputs of one chunk, held in registers between the load and their use.
template <typename IO, int DK, int DVT, int C>
struct ChunkRaw {
    using L = ChunkLayout<IO, DK, DVT, C>;
    using KQ = typename std::conditional<L::BF, uint2, float4>::type;  // 4 io values
    float4 g[L::KT];
    KQ k[L::KT], q[L::KT];
    uint4 v[L::V_PER_THREAD];
    float beta;
};

template <typename IO, int DK, int DVT, int C>
__device__ __forceinline__ void load_chunk(ChunkRaw<IO, DK, DVT, C> &raw, const FwdParams &p, int64_t tok0, int clen,
                                           int h, int col0, int tid) {
    using L = ChunkLayout<IO, DK, DVT, C>;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    const int H = p.H;
    // key side: wave R < NSUB reads its sub-chunk (rows past the end re-read the last row;
    // their values are masked to zero when used)
    if (wave < L::NSUB) {
        const int r = min(16 * wave + l16, clen - 1);
        const int64_t row = ((tok0 + r) * H + h) * (int64_t)DK + 4 * q4;
        const float *gp = p.g + row;
        const IO *kp = static_cast<const IO *>(p.k) + row;
        const IO *qp = static_cast<const IO *>(p.q) + row;
#pragma unroll
        for (int ct = 0; ct < L::KT; ++ct) {
            raw.g[ct] = *reinterpret_cast<const float4 *>(gp + 16 * ct);
            using KQ = typename ChunkRaw<IO, DK, DVT, C>::KQ;
            raw.k[ct] = *reinterpret_cast<const KQ *>(kp + 16 * ct);
            raw.q[ct] = *reinterpret_cast<const KQ *>(qp + 16 * ct);
        }
    }
    // V tile [C][DVT] in 16-byte pieces
    constexpr int PPR = DVT / L::V_ELEMS;  // pieces per row
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
    if (tid < C) raw.beta = p.beta[(tok0 + min(tid, clen - 1)) * H + h];
}

// bf16 at d_k = 64 with chunk 16 fits two workgroups' registers per CU without spilling; the other
// shapes take every register of one.
template <typename IO, int DK, int C>
constexpr int fused_min_waves() { return IoTraits<IO>::kBf16 && DK == 64 && C == 16 ? 2 : 1; }

template <typename IO, int DK, int DVT, int C>
__global__ void __launch_bounds__(kChunkThreads, (fused_min_waves<IO, DK, C>())) kda_chunk_fwd_kernel(FwdParams p) {
    using L = ChunkLayout<IO, DK, DVT, C>;
    using OT = typename L::OT;
    constexpr bool BF = L::BF;
    constexpr int NSUB = L::NSUB, KT = L::KT, NSL = L::NSL, SPW = L::SPW;
    constexpr int LDO = L::LDO, LDT = L::LDT, LDM = L::LDM, LDD = L::LDD, LDV = L::LDV;
    using Tr = IoTraits<IO>;

    __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
    OT *sKb = reinterpret_cast<OT *>(smem + L::oKb);
    OT *sKs = reinterpret_cast<OT *>(smem + L::oKs);
    OT *sKt = reinterpret_cast<OT *>(smem + L::oKt);
    OT *sQt = reinterpret_cast<OT *>(smem + L::oQt);
    OT *sKbT = reinterpret_cast<OT *>(smem + L::oKbT);
    OT *sA = reinterpret_cast<OT *>(smem + L::oA);
    OT *sP = reinterpret_cast<OT *>(smem + L::oP);
    float *sAd = reinterpret_cast<float *>(smem + L::oAd);
    OT *sV = reinterpret_cast<OT *>(smem + L::oV);
    float *sTot = reinterpret_cast<float *>(smem + L::oTot);
    float *sEB = reinterpret_cast<float *>(smem + L::oEB);
    float *sED = reinterpret_cast<float *>(smem + L::oED);
    float *sEC = reinterpret_cast<float *>(smem + L::oEC);
    float *sSH = reinterpret_cast<float *>(smem + L::oSH);
    float *sGam = reinterpret_cast<float *>(smem + L::oGam);
    float *sBeta = reinterpret_cast<float *>(smem + L::oBeta);

    const int tid = threadIdx.x;
    // wave index as a scalar: every branch on it is uniform across the wave
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;

    IO *__restrict__ O = static_cast<IO *>(p.out);
    const int H = p.H, DV = p.dv;

    // ---- which (sequence, head, d_v tile) this workgroup owns
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
    // first chunk slot of this sequence in the optional per-chunk outputs
    int64_t slot0 = 0;
    if (p.hs || p.dch) slot0 = p.cu ? (int64_t)p.chunk_off[n] : (int64_t)n * ((p.T + C - 1) / C);

    // ---- state slices owned by this wave: S[s][ct] holds rows 16ct+4q4+j of column col(s)
    f32x4 S[SPW][KT];
    const int64_t state_base = ((int64_t)n * H + h) * DK * DV;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int sl = wave + L::NW * s;
        const int col = col0 + 16 * sl + l16;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ct + 4 * q4 + j;
                S[s][ct][j] = (p.s0 && sl < NSL) ? p.s0[state_base + (int64_t)row * DV + col] : 0.f;
            }
        }
    }

    // The state loads above must land before the chunk loop: otherwise the wait-count
    // bookkeeping at the loop header still sees them pending and makes the state phase wait
    // for every outstanding load, including the next chunk's prefetch.
    __builtin_amdgcn_s_waitcnt(0);

    ChunkRaw<IO, DK, DVT, C> raw;
    if (len > 0) load_chunk<IO, DK, DVT, C>(raw, p, start, min(C, len), h, col0, tid);

    for (int c0 = 0; c0 < len; c0 += C) {
        const int clen = min(C, len - c0);
        const int64_t tok0 = start + c0;

        // ================= 1: gate scan (log2 domain), stage V and beta
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
        {
            constexpr int PPR = DVT / L::V_ELEMS;
#pragma unroll
            for (int i = 0; i < L::V_PER_THREAD; ++i) {
                const int piece = tid + kChunkThreads * i;
                if (L::V_PIECES % kChunkThreads == 0 || piece < L::V_PIECES) {
                    const int r = piece / PPR;
                    const int cc = (piece % PPR) * L::V_ELEMS;
                    const uint4 x = r < clen ? raw.v[i] : make_uint4(0u, 0u, 0u, 0u);
                    *reinterpret_cast<uint4 *>(sV + r * LDV + cc) = x;
                }
            }
            if (tid < C) sBeta[tid] = tid < clen ? raw.beta : 0.f;
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

        // Decay beyond 2^-96 inside the sub-chunk: A_RR and P_RR from the split levels (all factors
        // <= 1), written to their LDS places here (phase 4 writes only the other blocks of these rows)
        if (split) {
            const int R = wave;
            const int64_t row = ((tok0 + min(16 * R + l16, clen - 1)) * H + h) * (int64_t)DK + 4 * q4;
            f32x4 dA, dPt;
            diag_block_split_rolled<IO>(dA, dPt, static_cast<const IO *>(p.k) + row, static_cast<const IO *>(p.q) + row,
                                        p.g + row, valid, KT, l16, q4, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 4 * q4 + j;
                const float b = 16 * R + rr < clen ? p.beta[(tok0 + 16 * R + rr) * H + h] : 0.f;
                sAd[(R * 16 + rr) * LDD + l16] = l16 < rr ? dA[j] * b : 0.f;
                // dPt holds P_RR[l16][4 q4 + j]
                if constexpr (BF) sP[(16 * R + l16) * LDM + 16 * R + rr] = f32_to_bf16(dPt[j]);
                else sP[(16 * R + l16) * LDM + 16 * R + rr] = dPt[j];
            }
        }

        // ================= 3: gated operands of sub-chunk R
        Frag<BF> kdiag[KT];  // k * e^{b_R - G} (>= 1): column operand of the diagonal block
        if (wave < NSUB) {
            const int R = wave;
            const int r = 16 * R + l16;
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
                float kb[4], kt[4], qt[4], kbar[4], kd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float fr = valid ? fast_exp2(G[ct][j]) : 0.f;          // e^{G_r - b_R}     <= 1
                    const float fb = valid ? fast_exp2(tv[j] - G[ct][j]) : 0.f;  // e^{b_{R+1} - G_r} <= 1
                    kb[j] = kx[j] * fb;
                    kd[j] = kb[j] * edv[j];
                    kt[j] = kx[j] * fr * ebv[j];
                    qt[j] = qx[j] * fr * ebv[j];
                    kbar[j] = kb[j] * ecv[j];
                }
                kdiag[ct] = make_frag<BF>(kd[0], kd[1], kd[2], kd[3]);
                const Frag<BF> fkb = make_frag<BF>(kb[0], kb[1], kb[2], kb[3]);
                *reinterpret_cast<decltype(fkb.v) *>(sKb + r * LDO + c) = fkb.v;
                *reinterpret_cast<decltype(fkb.v) *>(sKt + r * LDO + c) = make_frag<BF>(kt[0], kt[1], kt[2], kt[3]).v;
                *reinterpret_cast<decltype(fkb.v) *>(sQt + r * LDO + c) = make_frag<BF>(qt[0], qt[1], qt[2], qt[3]).v;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (BF) sKbT[(c + j) * LDT + r] = f32_to_bf16(kbar[j]);
                    else sKbT[(c + j) * LDT + r] = kbar[j];
                }
                // column operands of blocks (R2, R) with R2 >= R + 2: k e^{b_{R2} - G}
#pragma unroll
                for (int R2 = 2; R2 < NSUB; ++R2) {
                    if (R2 < R + 2) continue;
                    const float4 sh = *reinterpret_cast<const float4 *>(sSH + L::shift_slot(R2, R) * DK + c);
                    const Frag<BF> f = make_frag<BF>(kb[0] * sh.x, kb[1] * sh.y, kb[2] * sh.z, kb[3] * sh.w);
                    *reinterpret_cast<decltype(f.v) *>(sKs + (L::shift_slot(R2, R) * 16 + l16) * LDO + c) = f.v;
                }
            }
        }
        __syncthreads();

        // ================= 4: row-R blocks of A and P, diagonal inverse; prefetch next chunk
        if (wave < NSUB) {
            const int R = wave;
            // row operands k, q * e^{G_r - b_R} (<= 1)
            Frag<BF> ka[KT], qa[KT];
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                const float4 kv = unpack4<BF>(raw.k[ct]), qv = unpack4<BF>(raw.q[ct]);
                float fr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) fr[j] = valid ? fast_exp2(G[ct][j]) : 0.f;
                ka[ct] = make_frag<BF>(kv.x * fr[0], kv.y * fr[1], kv.z * fr[2], kv.w * fr[3]);
                qa[ct] = make_frag<BF>(qv.x * fr[0], qv.y * fr[1], qv.z * fr[2], qv.w * fr[3]);
            }
#pragma unroll
            for (int I = 0; I < NSUB; ++I) {
                if (I > R) break;
                f32x4 accA = zero4(), accP = zero4();
                const OT *colp = (I == R - 1) ? sKb + (16 * I + l16) * LDO
                                              : sKs + (L::shift_slot(R < 2 ? 2 : R, I) * 16 + l16) * LDO;
#pragma unroll
                for (int ct = 0; ct < KT; ct += 2) {
                    Frag<BF> b0, b1;
                    if (I == R) {
                        b0 = kdiag[ct];
                        b1 = kdiag[ct + 1];
                    } else {
                        b0 = lds_frag(colp + 16 * ct + 4 * q4);
                        b1 = lds_frag(colp + 16 * (ct + 1) + 4 * q4);
                    }
                    mma32(accA, ka[ct], ka[ct + 1], b0, b1);
                    mma32(accP, qa[ct], qa[ct + 1], b0, b1);
                }
                // accumulator: rows rr = 4*q4 + j of block R, column ii = l16 of block I
                float av[4], pv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 4 * q4 + j, ii = l16;
                    av[j] = accA[j] * sBeta[16 * R + rr];
                    pv[j] = accP[j];
                    if (I == R) {
                        if (ii >= rr) av[j] = 0.f;
                        if (ii > rr) pv[j] = 0.f;
                    }
                }
                // with `split` the diagonal block was written in phase 1 (this product is discarded)
                if (!(I == R && split)) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rr = 4 * q4 + j;
                        if constexpr (BF) {
                            sP[(16 * R + rr) * LDM + 16 * I + l16] = f32_to_bf16(pv[j]);
                            if (I != R) sA[(16 * R + rr) * LDM + 16 * I + l16] = f32_to_bf16(av[j]);
                        } else {
                            sP[(16 * R + rr) * LDM + 16 * I + l16] = pv[j];
                            if (I != R) sA[(16 * R + rr) * LDM + 16 * I + l16] = av[j];
                        }
                        if (I == R) sAd[(R * 16 + rr) * LDD + l16] = av[j];
                    }
                }
            }
            // X_RR = (I + A_RR)^{-1}, row by row: lane l16 owns column l16 (same wave wrote A_RR)
            wave_lds_sync();
            float *Ab = sAd + R * 16 * LDD;
            const int jc = l16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == jc) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s -= Ab[r * LDD + m] * x[m];
                x[r] = s;
            }
            if (q4 == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Ab[r * LDD + jc] = x[r];
            }
        }
        if (c0 + C < len) load_chunk<IO, DK, DVT, C>(raw, p, tok0 + C, min(C, len - c0 - C), h, col0, tid);
        __syncthreads();

        // ================= 5: state slices (each wave: 16-column slices of the tile)
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int sl = wave + L::NW * s;
            if (sl >= NSL) break;
            const int col = col0 + 16 * sl + l16;
            const int64_t slot_base = ((slot0 + c0 / C) * H + h);
            if (p.hs) {  // operand type, as the backward reads it
                OT *hs = static_cast<OT *>(p.hs) + slot_base * DK * DV + col;
#pragma unroll
                for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (BF) hs[(int64_t)(16 * ct + 4 * q4 + j) * DV] = f32_to_bf16(S[s][ct][j]);
                        else hs[(int64_t)(16 * ct + 4 * q4 + j) * DV] = S[s][ct][j];
                    }
            }

            Frag<BF> Sb[KT];
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) Sb[ct] = frag_from_acc<BF>(S[s][ct]);

            f32x4 Y[NSUB], Oa[NSUB];
#pragma unroll
            for (int rt = 0; rt < NSUB; ++rt) {
                f32x4 ak = zero4(), ao = zero4();
                const OT *kt = sKt + (16 * rt + l16) * LDO + 4 * q4;
                const OT *qt = sQt + (16 * rt + l16) * LDO + 4 * q4;
#pragma unroll
                for (int ct = 0; ct < KT; ct += 2) {
                    mma32(ak, lds_frag(kt + 16 * ct), lds_frag(kt + 16 * ct + 16), Sb[ct], Sb[ct + 1]);
                    mma32(ao, lds_frag(qt + 16 * ct), lds_frag(qt + 16 * ct + 16), Sb[ct], Sb[ct + 1]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * q4 + j;
                    float vv;
                    if constexpr (BF) vv = bf16_to_f32(sV[r * LDV + 16 * sl + l16]);
                    else vv = sV[r * LDV + 16 * sl + l16];
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
                for (int I = 0; I < R; ++I) {
                    Frag<BF> a = lds_frag(sA + (16 * R + l16) * LDM + 16 * I + 4 * q4);
                    if constexpr (BF) {
                        a.v.x ^= 0x80008000u;
                        a.v.y ^= 0x80008000u;
                    } else {
                        a.v = make_float4(-a.v.x, -a.v.y, -a.v.z, -a.v.w);
                    }
                    mma16(z, a, D[I]);
                }
                f32x4 d = zero4();
                mma16(d, lds_frag_f32<BF>(sAd + (16 * R + l16) * LDD + 4 * q4), frag_from_acc<BF>(z));
                D[R] = frag_from_acc<BF>(d);
                if (p.dch) {
                    OT *dc = static_cast<OT *>(p.dch) + slot_base * C * DV + (int64_t)(16 * R + 4 * q4) * DV + col;
                    if constexpr (BF) {
                        dc[0] = (uint16_t)(D[R].v.x & 0xffffu);
                        dc[DV] = (uint16_t)(D[R].v.x >> 16);
                        dc[2 * DV] = (uint16_t)(D[R].v.y & 0xffffu);
                        dc[3 * DV] = (uint16_t)(D[R].v.y >> 16);
                    } else {
                        dc[0] = D[R].v.x;
                        dc[DV] = D[R].v.y;
                        dc[2 * DV] = D[R].v.z;
                        dc[3 * DV] = D[R].v.w;
                    }
                }
            }

            // O = scale (Q~ S + P D)
#pragma unroll
            for (int R = 0; R < NSUB; ++R) {
#pragma unroll
                for (int I = 0; I <= R; ++I) mma16(Oa[R], lds_frag(sP + (16 * R + l16) * LDM + 16 * I + 4 * q4), D[I]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * R + 4 * q4 + j;
                    if (O && r < clen) Tr::store1(O + ((tok0 + r) * H + h) * (int64_t)DV + col, Oa[R][j] * p.scale);
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
                for (int I = 0; I + 1 < NSUB; I += 2)
                    mma32(S[s][ct], lds_frag(kb + 16 * I), lds_frag(kb + 16 * (I + 1)), D[I], D[I + 1]);
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
            const int col = col0 + 16 * sl + l16;
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
