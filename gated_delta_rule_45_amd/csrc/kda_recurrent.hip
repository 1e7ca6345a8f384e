// Token-serial KDA kernels for gfx950: the decode step (one token per sequence, state
// updated in place in HBM) and the recurrent reference mode (a whole sequence, state
// kept in registers).  Both run the same per-token update (Kimi Linear summary page,
// "Kimi Delta Attention: fine-grained memory control"):
//
//   S' = Diag(e^{g}) S        p = S'^T k        d = beta (v - p)
//   S  = S' + k d^T           o = scale S^T q = scale (S'^T q + (k.q) d)
//
// Every column j of S evolves on its own given (q, k, g, beta, v_j), so the state tile
// is spread over the workgroup as 4-column groups (16-byte, coalesced row segments)
// times row groups; the two column reductions (p and S'^T q) cross row groups through
// LDS.  The decode step is bound by HBM: the 64 KB fp32 state of a (sequence, head) is
// read once and written once, everything else is a few hundred bytes.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV>
struct SerialLayout {
    static constexpr int CG = DV / 4;             // 4-column groups
    static constexpr int RG = kSerialThreads / CG; // row groups
    static constexpr int RPT = DK / RG;           // rows per thread: rg, rg+RG, ...
    static_assert(kSerialThreads % CG == 0 && DK % RG == 0, "layout");
};

// Per-token inputs staged in LDS (double-buffered across tokens).
template <int DK, int DV>
struct TokenSmem {
    float alpha[DK], k[DK], q[DK], v[DV];
    float beta, qk;
    float red_p[SerialLayout<DK, DV>::RG][DV];
    float red_a[SerialLayout<DK, DV>::RG][DV];
};

// Stage token inputs: threads < DK load q, k, g; threads < DV load v.  Also reduces k.q.
template <typename IO, int DK, int DV>
__device__ __forceinline__ void stage_token(TokenSmem<DK, DV> &ts, float *qk_part, const IO *q, const IO *k,
                                            const IO *v, const float *g, const float *beta, int tid) {
    using Tr = IoTraits<IO>;
    float kq = 0.f;
    if (tid < DK) {
        const float kk = Tr::load1(k + tid), qq = Tr::load1(q + tid);
        ts.alpha[tid] = expf(g[tid]);
        ts.k[tid] = kk;
        ts.q[tid] = qq;
        kq = kk * qq;
    }
    if (tid < DV) ts.v[tid] = Tr::load1(v + tid);
    if (tid == 0) ts.beta = *beta;
    // wave-level sum of k.q (waves with tid < DK), then one partial per wave
    if (tid < DK) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off, 64);
        if ((tid & 63) == 0) qk_part[tid >> 6] = kq;
    }
}

// One token: S (this thread's RPT x 4 block) is updated in place; returns o for the thread's
// 4 columns in `o4` (valid for every thread; only row group 0 stores it).
template <int DK, int DV, int RPT = SerialLayout<DK, DV>::RPT>
__device__ __forceinline__ void token_update(float (&S)[RPT][4], TokenSmem<DK, DV> &ts, const float *qk_part, int cg,
                                             int rg, float4 &o4) {
    using L = SerialLayout<DK, DV>;
    float pp[4] = {0.f, 0.f, 0.f, 0.f}, aa[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < L::RPT; ++m) {
        const int i = rg + L::RG * m;
        const float al = ts.alpha[i], kk = ts.k[i], qq = ts.q[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            S[m][j] *= al;
            pp[j] += kk * S[m][j];
            aa[j] += qq * S[m][j];
        }
    }
    *reinterpret_cast<float4 *>(&ts.red_p[rg][4 * cg]) = make_float4(pp[0], pp[1], pp[2], pp[3]);
    *reinterpret_cast<float4 *>(&ts.red_a[rg][4 * cg]) = make_float4(aa[0], aa[1], aa[2], aa[3]);
    __syncthreads();
    float p4[4] = {0.f, 0.f, 0.f, 0.f}, a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < L::RG; ++r) {
        const float4 x = *reinterpret_cast<const float4 *>(&ts.red_p[r][4 * cg]);
        const float4 y = *reinterpret_cast<const float4 *>(&ts.red_a[r][4 * cg]);
        p4[0] += x.x; p4[1] += x.y; p4[2] += x.z; p4[3] += x.w;
        a4[0] += y.x; a4[1] += y.y; a4[2] += y.z; a4[3] += y.w;
    }
    float qk = 0.f;
#pragma unroll
    for (int w = 0; w < (DK + 63) / 64; ++w) qk += qk_part[w];
    const float b = ts.beta;
    float d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = b * (ts.v[4 * cg + j] - p4[j]);
#pragma unroll
    for (int m = 0; m < L::RPT; ++m) {
        const float kk = ts.k[rg + L::RG * m];
#pragma unroll
        for (int j = 0; j < 4; ++j) S[m][j] += kk * d[j];
    }
    o4 = make_float4(a4[0] + qk * d[0], a4[1] + qk * d[1], a4[2] + qk * d[2], a4[3] + qk * d[3]);
}

// Decode: one 256-thread workgroup per (sequence, head, 32-column block).  The state block
// (d_k x 32 fp32, 16 KB at d_k = 128) is read once and written once with nontemporal
// 16-byte accesses, 4 per thread: thread t owns columns 4*(t % 8) .. +3 of the block and
// rows t/8 + 32*m.  Small per-thread footprints and many workgroups keep HBM busy.
constexpr int kDecodeCols = 32;

typedef float kda_v4f __attribute__((ext_vector_type(4)));

template <typename IO, int DK, int DV>
__global__ void __launch_bounds__(256) kda_decode_kernel(int32_t H, float scale, const IO *__restrict__ q,
                                                         const IO *__restrict__ k, const IO *__restrict__ v,
                                                         const float *__restrict__ g, const float *__restrict__ beta,
                                                         float *state, IO *__restrict__ out) {
    constexpr int NCB = DV / kDecodeCols;  // column blocks per (sequence, head)
    constexpr int RG = 256 / 8;            // row groups
    constexpr int RPT = DK / RG;           // rows per thread
    __shared__ float s_alpha[DK], s_k[DK], s_q[DK], s_v[kDecodeCols];
    __shared__ float s_beta, s_qk[4];
    __shared__ kda_v4f s_part[2][4][8];  // per-wave partial p and S'^T q per column group

    const int tid = threadIdx.x;
    const int cg = tid & 7, rg = tid >> 3, wv = tid >> 6;
    // the NCB column blocks of one (sequence, head) run on one XCD, so their shared q, k and
    // gate reads come from HBM once and from that XCD's L2 after
    const int64_t item = xcd_grouped_block(blockIdx.x, (int64_t)gridDim.x);
    const int64_t nh = item / NCB;
    const int cb = (int)(item % NCB);
    const int col0 = cb * kDecodeCols;
    kda_v4f *Sg = reinterpret_cast<kda_v4f *>(state + nh * DK * DV + col0) + cg;

    kda_v4f S[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) S[m] = __builtin_nontemporal_load(Sg + (int64_t)(rg + RG * m) * (DV / 4));

    using Tr = IoTraits<IO>;
    float kq = 0.f;
    if (tid < DK) {
        const float kk = Tr::load1(k + nh * DK + tid), qq = Tr::load1(q + nh * DK + tid);
        s_alpha[tid] = expf(g[nh * DK + tid]);
        s_k[tid] = kk;
        s_q[tid] = qq;
        kq = kk * qq;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off, 64);
        if ((tid & 63) == 0) s_qk[tid >> 6] = kq;
    }
    if (tid < kDecodeCols) s_v[tid] = Tr::load1(v + nh * DV + col0 + tid);
    if (tid == 0) s_beta = beta[nh];
    __syncthreads();

    // S' = Diag(alpha) S;  partial p = S'^T k and a = S'^T q over this thread's rows, then
    // summed over the 8 row groups of the wave (lanes 8 apart) and, through LDS, the 4 waves
    kda_v4f pp = {0.f, 0.f, 0.f, 0.f}, aa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        S[m] *= s_alpha[i];
        pp += s_k[i] * S[m];
        aa += s_q[i] * S[m];
    }
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pp[j] += __shfl_xor(pp[j], off, 64);
            aa[j] += __shfl_xor(aa[j], off, 64);
        }
    }
    if ((tid & 63) < 8) {
        s_part[0][wv][cg] = pp;
        s_part[1][wv][cg] = aa;
    }
    __syncthreads();
    kda_v4f ps = s_part[0][0][cg] + s_part[0][1][cg] + s_part[0][2][cg] + s_part[0][3][cg];

    // d = beta (v - p);  S = S' + k d^T;  o = a + (k.q) d
    const float b = s_beta;
    kda_v4f d;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = b * (s_v[4 * cg + j] - ps[j]);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        S[m] += s_k[rg + RG * m] * d;
        __builtin_nontemporal_store(S[m], Sg + (int64_t)(rg + RG * m) * (DV / 4));
    }
    if (rg == 0) {
        float qk = 0.f;
#pragma unroll
        for (int w = 0; w < (DK + 63) / 64; ++w) qk += s_qk[w];
        const kda_v4f as = s_part[1][0][cg] + s_part[1][1][cg] + s_part[1][2][cg] + s_part[1][3][cg];
        float4 o;
        o.x = (as[0] + qk * d[0]) * scale;
        o.y = (as[1] + qk * d[1]) * scale;
        o.z = (as[2] + qk * d[2]) * scale;
        o.w = (as[3] + qk * d[3]) * scale;
        Tr::store4(out + nh * DV + col0 + 4 * cg, o);
    }
}

// Decode step with the output epilogue fused in (Kimi Linear summary page: the per-token update
// of "Kimi Delta Attention: fine-grained memory control", then the per-head RMSNorm and output
// gate of "Kimi Linear model composition"; the page gives no formula for the latter, the reading is
// out = o * rsqrt(mean(o^2) + eps) * w * sigmoid(z) over the d_v values of one head).
//
// The norm needs the whole d_v row of o, so one workgroup (NT threads) owns one (sequence, head): the
// d_k x d_v fp32 state (64 KB at d = 128) is read and written once with 16-byte nontemporal
// accesses, thread t holding columns 4 (t % CG) .. + 3 of rows t / CG + RG m.  The column sums
// p = S'^T k and a = S'^T q cross the row groups of a wave with lane shuffles and the waves
// through LDS; every thread then has o for its 4 columns, and the lanes of one row group (a
// contiguous run of CG lanes) reduce sum(o^2) among themselves.  1024 threads (4 state rows of
// 4 columns per thread at d = 128) measured at least as fast as 256 or 512 on the decode
// workload; the kernel is bound by HBM like the plain decode step.
#ifndef KDA_DECODE_GATED_THREADS
#define KDA_DECODE_GATED_THREADS 1024
#endif
constexpr int kDecodeGatedThreads = KDA_DECODE_GATED_THREADS;

template <typename IO, int DK, int DV, int NT>
__global__ void __launch_bounds__(NT) kda_decode_gated_kernel(float scale, float eps, const IO *__restrict__ q,
                                                               const IO *__restrict__ k, const IO *__restrict__ v,
                                                               const float *__restrict__ g,
                                                               const float *__restrict__ beta, float *state,
                                                               const IO *__restrict__ gate,
                                                               const float *__restrict__ weight, IO *__restrict__ out) {
    constexpr int CG = DV / 4;      // 4-column groups (lanes of one row group)
    constexpr int RG = NT / CG;     // row groups
    constexpr int RPT = DK / RG;    // rows per thread
    constexpr int WRG = 64 / CG;    // row groups per wave
    constexpr int NWV = NT / 64;    // waves
    static_assert(CG <= 64 && 64 % CG == 0 && DK % RG == 0 && RPT >= 1, "layout");
    __shared__ float s_alpha[DK], s_k[DK], s_q[DK], s_v[DV];
    __shared__ float s_beta, s_qk[(DK + 63) / 64];
    __shared__ kda_v4f s_part[2][NWV][CG];  // per-wave partial p and S'^T q per column group

    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG, wv = tid >> 6;
    const int64_t nh = blockIdx.x;
    kda_v4f *Sg = reinterpret_cast<kda_v4f *>(state + nh * DK * DV) + cg;

    kda_v4f S[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) S[m] = __builtin_nontemporal_load(Sg + (int64_t)(rg + RG * m) * (DV / 4));

    using Tr = IoTraits<IO>;
    if (tid < DK) {
        const float kk = Tr::load1(k + nh * DK + tid), qq = Tr::load1(q + nh * DK + tid);
        s_alpha[tid] = expf(g[nh * DK + tid]);
        s_k[tid] = kk;
        s_q[tid] = qq;
        float kq = kk * qq;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off, 64);
        if ((tid & 63) == 0) s_qk[tid >> 6] = kq;
    }
    if (tid < DV) s_v[tid] = Tr::load1(v + nh * DV + tid);
    if (tid == 0) s_beta = beta[nh];
    // gate and weight of this thread's 4 columns, needed only at the end
    float zc[4], wc[4];
    {
        const f32x4 ww = *reinterpret_cast<const f32x4 *>(weight + 4 * cg);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            zc[j] = Tr::load1(gate + nh * DV + 4 * cg + j);
            wc[j] = ww[j];
        }
    }
    __syncthreads();

    // S' = Diag(alpha) S;  partial p = S'^T k and a = S'^T q over this thread's rows, summed over
    // the row groups of the wave (lanes CG apart) and then, through LDS, over the 4 waves
    kda_v4f pp = {0.f, 0.f, 0.f, 0.f}, aa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        S[m] *= s_alpha[i];
        pp += s_k[i] * S[m];
        aa += s_q[i] * S[m];
    }
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pp[j] += __shfl_xor(pp[j], off, 64);
            aa[j] += __shfl_xor(aa[j], off, 64);
        }
    }
    if ((tid & 63) < CG) {
        s_part[0][wv][cg] = pp;
        s_part[1][wv][cg] = aa;
    }
    __syncthreads();
    kda_v4f ps = s_part[0][0][cg], as = s_part[1][0][cg];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
        ps += s_part[0][w][cg];
        as += s_part[1][w][cg];
    }

    // d = beta (v - p);  S = S' + k d^T;  o = scale (a + (k.q) d)
    const float b = s_beta;
    kda_v4f d;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = b * (s_v[4 * cg + j] - ps[j]);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        S[m] += s_k[rg + RG * m] * d;
        __builtin_nontemporal_store(S[m], Sg + (int64_t)(rg + RG * m) * (DV / 4));
    }
    float qk = 0.f;
#pragma unroll
    for (int w = 0; w < (DK + 63) / 64; ++w) qk += s_qk[w];
    float o[4], ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j] = (as[j] + qk * d[j]) * scale;
        ss = fmaf(o[j], o[j], ss);
    }
    // sum of o^2 over the CG lanes of this row group (xor offsets below CG stay inside it)
#pragma unroll
    for (int off = CG / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    static_assert(WRG >= 1, "a row group lives inside one wave");
    if (rg == 0) {
        const float r = rsqrtf(ss * (1.0f / DV) + eps);
        float4 y;
        y.x = o[0] * r * wc[0] / (1.0f + __expf(-zc[0]));
        y.y = o[1] * r * wc[1] / (1.0f + __expf(-zc[1]));
        y.z = o[2] * r * wc[2] / (1.0f + __expf(-zc[2]));
        y.w = o[3] * r * wc[3] / (1.0f + __expf(-zc[3]));
        Tr::store4(out + nh * DV + 4 * cg, y);
    }
}

template <typename IO, int DK, int DV>
__global__ void __launch_bounds__(kSerialThreads) kda_recurrent_kernel(FwdParams p) {
    using L = SerialLayout<DK, DV>;
    __shared__ TokenSmem<DK, DV> ts[2];
    __shared__ float qk_part[2][4];
    const int tid = threadIdx.x;
    const int cg = tid % L::CG, rg = tid / L::CG;
    const int H = p.H;
    const int h = blockIdx.x % H;
    const int n = blockIdx.x / H;
    int64_t start;
    int len;
    if (p.cu) {
        start = p.cu[n];
        len = p.cu[n + 1] - p.cu[n];
    } else {
        start = (int64_t)n * p.T;
        len = p.T;
    }
    const IO *Q = static_cast<const IO *>(p.q);
    const IO *K = static_cast<const IO *>(p.k);
    const IO *V = static_cast<const IO *>(p.v);
    IO *O = static_cast<IO *>(p.out);
    const int64_t sbase = ((int64_t)n * H + h) * DK * DV;

    float S[L::RPT][4];
#pragma unroll
    for (int m = 0; m < L::RPT; ++m) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.s0) x = *reinterpret_cast<const float4 *>(p.s0 + sbase + (int64_t)(rg + L::RG * m) * DV + 4 * cg);
        S[m][0] = x.x; S[m][1] = x.y; S[m][2] = x.z; S[m][3] = x.w;
    }
    for (int t = 0; t < len; ++t) {
        const int64_t th = (start + t) * H + h;
        TokenSmem<DK, DV> &cur = ts[t & 1];
        stage_token<IO, DK, DV>(cur, qk_part[t & 1], Q + th * DK, K + th * DK, V + th * DV, p.g + th * DK, p.beta + th,
                                tid);
        __syncthreads();
        float4 o4;
        token_update<DK, DV>(S, cur, qk_part[t & 1], cg, rg, o4);
        if (rg == 0)
            IoTraits<IO>::store4(O + th * DV + 4 * cg,
                                 make_float4(o4.x * p.scale, o4.y * p.scale, o4.z * p.scale, o4.w * p.scale));
    }
    if (p.sf) {
#pragma unroll
        for (int m = 0; m < L::RPT; ++m)
            *reinterpret_cast<float4 *>(p.sf + sbase + (int64_t)(rg + L::RG * m) * DV + 4 * cg) =
                make_float4(S[m][0], S[m][1], S[m][2], S[m][3]);
    }
}

#define KDA_SERIAL_DIMS(F) F(64, 64) F(64, 128) F(128, 64) F(128, 128)

template <typename IO>
static hipError_t recurrent_dispatch(const FwdParams &p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.num_seqs * p.H;
    if (blocks <= 0) return hipSuccess;
#define KDA_REC_CASE(DK_, DV_)                                                                                       \
    if (p.dk == DK_ && p.dv == DV_) {                                                                                \
        hipLaunchKernelGGL((kda_recurrent_kernel<IO, DK_, DV_>), dim3((unsigned)blocks), dim3(kSerialThreads), 0, \
                           stream, p);                                                                               \
        return hipGetLastError();                                                                                    \
    }
    KDA_SERIAL_DIMS(KDA_REC_CASE)
#undef KDA_REC_CASE
    return hipErrorInvalidConfiguration;
}

template <typename IO>
static hipError_t decode_dispatch(int32_t N, int32_t H, int32_t dk, int32_t dv, float scale, const void *q,
                                  const void *k, const void *v, const float *g, const float *beta, float *state,
                                  void *out, hipStream_t stream) {
    const int64_t blocks = (int64_t)N * H * (dv / kDecodeCols);
    if (blocks <= 0) return hipSuccess;
#define KDA_DEC_CASE(DK_, DV_)                                                                                      \
    if (dk == DK_ && dv == DV_) {                                                                                   \
        hipLaunchKernelGGL((kda_decode_kernel<IO, DK_, DV_>), dim3((unsigned)blocks), dim3(256), 0,              \
                           stream, H, scale, static_cast<const IO *>(q), static_cast<const IO *>(k),                \
                           static_cast<const IO *>(v), g, beta, state, static_cast<IO *>(out));                     \
        return hipGetLastError();                                                                                   \
    }
    KDA_SERIAL_DIMS(KDA_DEC_CASE)
#undef KDA_DEC_CASE
    return hipErrorInvalidConfiguration;
}

template <typename IO>
static hipError_t decode_gated_dispatch(int32_t N, int32_t H, int32_t dk, int32_t dv, float scale, float eps,
                                        const void *q, const void *k, const void *v, const float *g,
                                        const float *beta, float *state, const void *gate, const float *weight,
                                        void *out, hipStream_t stream) {
    const int64_t blocks = (int64_t)N * H;
    if (blocks <= 0) return hipSuccess;
#define KDA_DECG_CASE(DK_, DV_)                                                                                  \
    if (dk == DK_ && dv == DV_) {                                                                                \
        hipLaunchKernelGGL((kda_decode_gated_kernel<IO, DK_, DV_, kDecodeGatedThreads>), dim3((unsigned)blocks),      \
                           dim3(kDecodeGatedThreads), 0, stream,                                                 \
                           scale, eps, static_cast<const IO *>(q), static_cast<const IO *>(k),                   \
                           static_cast<const IO *>(v), g, beta, state, static_cast<const IO *>(gate), weight,   \
                           static_cast<IO *>(out));                                                              \
        return hipGetLastError();                                                                                \
    }
    KDA_SERIAL_DIMS(KDA_DECG_CASE)
#undef KDA_DECG_CASE
    return hipErrorInvalidConfiguration;
}

hipError_t launch_decode_gated(kda_dtype_t io, int32_t N, int32_t H, int32_t dk, int32_t dv, float scale, float eps,
                               const void *q, const void *k, const void *v, const float *g, const float *beta,
                               float *state, const void *gate, const float *weight, void *out, hipStream_t stream) {
    return io == KDA_BF16
               ? decode_gated_dispatch<uint16_t>(N, H, dk, dv, scale, eps, q, k, v, g, beta, state, gate, weight, out,
                                                 stream)
               : decode_gated_dispatch<float>(N, H, dk, dv, scale, eps, q, k, v, g, beta, state, gate, weight, out,
                                              stream);
}

hipError_t launch_recurrent_fwd(kda_dtype_t io, const FwdParams &p, hipStream_t stream) {
    return io == KDA_BF16 ? recurrent_dispatch<uint16_t>(p, stream) : recurrent_dispatch<float>(p, stream);
}

hipError_t launch_decode_step(kda_dtype_t io, int32_t N, int32_t H, int32_t dk, int32_t dv, float scale,
                              const void *q, const void *k, const void *v, const float *g, const float *beta,
                              float *state, void *out, hipStream_t stream) {
    return io == KDA_BF16 ? decode_dispatch<uint16_t>(N, H, dk, dv, scale, q, k, v, g, beta, state, out, stream)
                          : decode_dispatch<float>(N, H, dk, dv, scale, q, k, v, g, beta, state, out, stream);
}

}  // namespace kda
