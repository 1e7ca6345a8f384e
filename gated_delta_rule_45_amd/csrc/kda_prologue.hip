// Prologue: raw projections -> the operator's inputs (Kimi Linear summary page, section "Kimi
// Linear model composition": query, key and value pass a short convolution and Swish, query and
// key an L2 normalisation; the decay gate uses a GDN / Mamba-like decay function).  Readings:
//
//   c_t  = sum_{i<W} w[i] x_{t-W+1+i}     causal depthwise convolution over time, per channel;
//                                          inputs before a sequence's first token come from the
//                                          carried-in state, or are zero
//   y    = c * sigmoid(c)                 Swish
//   q, k = y / sqrt(sum y^2 + eps)        over the head dimension;  v = y
//   g    = -softplus(g_raw),  beta = sigmoid(beta_raw)
//
// Bound: HBM.  Each lane owns one 16-byte segment of a head's rows and walks 8 consecutive
// tokens, so every raw input is read once.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <typename IO>
struct Seg16;
template <>
struct Seg16<uint16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ void unpack(const u32x4 &w, float (&v)[N]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static __forceinline__ u32x4 pack(const float (&v)[N]) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        return w;
    }
};
template <>
struct Seg16<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ void unpack(const u32x4 &w, float (&v)[N]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    }
    __device__ static __forceinline__ u32x4 pack(const float (&v)[N]) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(v[i]);
        return w;
    }
};

struct PrologueArgs {
    int64_t tokens;
    int32_t num_seqs, seq_len, H, dk, dv, W;
    const int32_t *cu;  // [num_seqs + 1] or null (sequence n = tokens [n * seq_len, (n + 1) * seq_len))
    float eps;
};

// Sequence holding token t: its index, first token and end.
__device__ __forceinline__ void find_seq(const PrologueArgs &a, int64_t t, int &n, int64_t &start, int64_t &end) {
    if (!a.cu) {
        n = (int)(t / a.seq_len);
        start = (int64_t)n * a.seq_len;
        end = start + a.seq_len;
        return;
    }
    int lo = 0, hi = a.num_seqs - 1;  // last n with cu[n] <= t (empty sequences skipped by taking the last)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    start = a.cu[lo];
    end = a.cu[lo + 1];
}

constexpr int kConvTokensPerStream = 8;

// One tensor (q, k or v): rows of D values at column offset `col` of the state's concatenated
// q | k | v rows.  NORM: L2-normalise each row.  Workgroup `bid` of the tensor takes one head
// and TT consecutive tokens; each group of LPR lanes streams L of them in order, so a lane
// keeps its filter taps and the last W-1 raw inputs of its channels in registers and loads
// each input once.
template <typename IO, int D>
constexpr int conv_tokens_per_block() { return 256 / (D / Seg16<IO>::N) * kConvTokensPerStream; }

template <typename IO, int D, bool NORM, int W>
__device__ __forceinline__ void conv_swish_rows(const PrologueArgs &a, int64_t bid, const IO *__restrict__ x,
                                                const float *__restrict__ w, const IO *__restrict__ st_in,
                                                IO *__restrict__ st_out, int col, IO *__restrict__ y) {
    constexpr int N = Seg16<IO>::N;
    constexpr int LPR = D / N;      // lanes per row
    constexpr int L = kConvTokensPerStream;
    constexpr int TT = conv_tokens_per_block<IO, D>();  // tokens per workgroup
    static_assert(LPR <= 64 && 64 % LPR == 0, "a row lives inside one wave");
    const int seg = threadIdx.x % LPR;
    const int stream = threadIdx.x / LPR;
    const int h = (int)(bid % a.H);
    const int64_t t0 = (bid / a.H) * TT + (int64_t)stream * L;
    const int SD = 2 * a.dk + a.dv;  // state row width per head

    float wc[N * W];  // taps of this lane's N channels: N * W consecutive floats
    {
        const float *wp = w + ((int64_t)h * D + seg * N) * W;
#pragma unroll
        for (int i = 0; i < N * W; i += 4) {
            const f32x4 t4 = *reinterpret_cast<const f32x4 *>(wp + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) wc[i + j] = t4[j];
        }
    }
    // all of this stream's inputs in flight at once (tokens past the end re-read the last one)
    const int64_t tlast = a.tokens - 1;
    u32x4 raw[L];
#pragma unroll
    for (int u = 0; u < L; ++u)
        raw[u] = *reinterpret_cast<const u32x4 *>(x + (min(t0 + u, tlast) * a.H + h) * D + seg * N);

    int n;
    int64_t start, end;
    find_seq(a, min(t0, tlast), n, start, end);
    // window[i]: raw input of token t - (W - 1) + i for the token t being processed
    float win[W][N];
    auto fill_window = [&](int64_t t) {  // the W-1 inputs before token t, at a sequence start or the stream start
#pragma unroll
        for (int i = 0; i < W - 1; ++i) {
            const int64_t p = t - (W - 1) + i;
            u32x4 r = {0u, 0u, 0u, 0u};
            if (p >= start) {
                r = *reinterpret_cast<const u32x4 *>(x + (p * a.H + h) * D + seg * N);
            } else if (st_in) {
                const int64_t sr = (W - 1) - (start - p);
                r = *reinterpret_cast<const u32x4 *>(st_in + (((int64_t)n * (W - 1) + sr) * a.H + h) * SD + col + seg * N);
            }
            Seg16<IO>::unpack(r, win[i]);
        }
    };
    if (t0 <= tlast) fill_window(t0);
#pragma unroll
    for (int u = 0; u < L; ++u) {
        const int64_t t = t0 + u;
        if (t > tlast) break;
        if (t >= end) {  // next sequence (skipping empty ones): restart the window from its state
            do {
                ++n;
                start = a.cu ? (int64_t)a.cu[n] : (int64_t)n * a.seq_len;
                end = a.cu ? (int64_t)a.cu[n + 1] : start + a.seq_len;
            } while (t >= end);
            fill_window(t);
        }
        Seg16<IO>::unpack(raw[u], win[W - 1]);
        float acc[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float c = 0.f;
#pragma unroll
            for (int i = 0; i < W; ++i) c = fmaf(wc[j * W + i], win[i][j], c);
            acc[j] = c * __builtin_amdgcn_rcpf(1.0f + __expf(-c));  // Swish; reciprocal to 1 ulp
        }
        if constexpr (NORM) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < N; ++j) ss = fmaf(acc[j], acc[j], ss);
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
            const float rn = rsqrtf(ss + a.eps);
#pragma unroll
            for (int j = 0; j < N; ++j) acc[j] *= rn;
        }
        *reinterpret_cast<u32x4 *>(y + (t * a.H + h) * D + seg * N) = Seg16<IO>::pack(acc);
        if (st_out && t >= end - (W - 1)) {  // the last W-1 raw inputs of the sequence are handed on
            const int64_t sr = (W - 1) - (end - t);
            *reinterpret_cast<u32x4 *>(st_out + (((int64_t)n * (W - 1) + sr) * a.H + h) * SD + col + seg * N) = raw[u];
        }
#pragma unroll
        for (int i = 0; i + 1 < W; ++i)
#pragma unroll
            for (int j = 0; j < N; ++j) win[i][j] = win[i + 1][j];
    }
}

// q, k and v in one launch: workgroups [0, nb_k) take q, [nb_k, 2 nb_k) take k and the rest v,
// so that the loads of some workgroups overlap the stores of others across the three tensors.
template <typename IO>
struct ConvQkv {
    const IO *x[3];
    const float *w[3];
    IO *y[3];
    const IO *st_in;
    IO *st_out;
    int64_t nb_k;  // workgroups per key-width tensor (q, k)
};

template <typename IO, int DK, int DV, int W>
__global__ void __launch_bounds__(256) kda_conv_swish_kernel(PrologueArgs a, ConvQkv<IO> j) {
    const int64_t b = blockIdx.x;
    if (b < 2 * j.nb_k) {
        const int t = b < j.nb_k ? 0 : 1;
        conv_swish_rows<IO, DK, true, W>(a, b - t * j.nb_k, j.x[t], j.w[t], j.st_in, j.st_out, t * DK, j.y[t]);
    } else {
        conv_swish_rows<IO, DV, false, W>(a, b - 2 * j.nb_k, j.x[2], j.w[2], j.st_in, j.st_out, 2 * DK, j.y[2]);
    }
}

// State rows of sequences shorter than W - 1: positions before the first token are carried over
// from the incoming state (or zero).  One thread per (sequence, state row, head, 16-byte piece).
template <typename IO>
__global__ void __launch_bounds__(256) kda_conv_state_carry_kernel(PrologueArgs a, const IO *__restrict__ st_in,
                                                                  IO *__restrict__ st_out) {
    constexpr int N = Seg16<IO>::N;
    const int SD = 2 * a.dk + a.dv;
    const int pieces = SD / N;
    const int64_t total = (int64_t)a.num_seqs * (a.W - 1) * a.H * pieces;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int piece = (int)(i % pieces);
    const int64_t rest = i / pieces;
    const int h = (int)(rest % a.H);
    const int sr = (int)((rest / a.H) % (a.W - 1));
    const int n = (int)(rest / ((int64_t)a.H * (a.W - 1)));
    const int64_t len = a.cu ? (int64_t)(a.cu[n + 1] - a.cu[n]) : (int64_t)a.seq_len;
    // state row sr holds position end - (W - 1) + sr; it precedes the sequence when the
    // sequence has fewer than W - 1 - sr tokens, and then it is incoming state row sr + len
    if (sr + len >= a.W - 1) return;
    const int64_t off = (((int64_t)n * (a.W - 1) + sr) * a.H + h) * SD + piece * N;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (st_in) v = *reinterpret_cast<const u32x4 *>(st_in + (((int64_t)n * (a.W - 1) + sr + len) * a.H + h) * SD + piece * N);
    *reinterpret_cast<u32x4 *>(st_out + off) = v;
}

__global__ void __launch_bounds__(256) kda_gate_beta_kernel(int64_t gcount, int64_t bcount, const float *__restrict__ g_raw,
                                                           const float *__restrict__ b_raw, float *__restrict__ g,
                                                           float *__restrict__ b) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < gcount / 4) {  // -softplus in a form that neither overflows nor loses more than 1e-8 absolute
        const f32x4 x = *reinterpret_cast<const f32x4 *>(g_raw + 4 * i);
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = -(fmaxf(x[j], 0.f) + __logf(1.0f + __expf(-fabsf(x[j]))));
        *reinterpret_cast<f32x4 *>(g + 4 * i) = o;
    }
    if (i < bcount) b[i] = 1.0f / (1.0f + __expf(-b_raw[i]));
}

template <typename IO, int DK, int DV>
hipError_t launch_conv(const PrologueArgs &a, const void *const raw[3], const float *const w[3], const void *st_in,
                       void *st_out, void *const out[3], hipStream_t s) {
    constexpr int TK = conv_tokens_per_block<IO, DK>(), TV = conv_tokens_per_block<IO, DV>();
    const int64_t nb_k = (a.tokens + TK - 1) / TK * a.H;
    const int64_t blocks = 2 * nb_k + (a.tokens + TV - 1) / TV * a.H;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ConvQkv<IO> j;
    for (int i = 0; i < 3; ++i) {
        j.x[i] = static_cast<const IO *>(raw[i]);
        j.w[i] = w[i];
        j.y[i] = static_cast<IO *>(out[i]);
    }
    j.st_in = static_cast<const IO *>(st_in);
    j.st_out = static_cast<IO *>(st_out);
    j.nb_k = nb_k;
    const dim3 g((unsigned)blocks), b(256);
    switch (a.W) {
        case 1: hipLaunchKernelGGL((kda_conv_swish_kernel<IO, DK, DV, 1>), g, b, 0, s, a, j); break;
        case 2: hipLaunchKernelGGL((kda_conv_swish_kernel<IO, DK, DV, 2>), g, b, 0, s, a, j); break;
        case 3: hipLaunchKernelGGL((kda_conv_swish_kernel<IO, DK, DV, 3>), g, b, 0, s, a, j); break;
        default: hipLaunchKernelGGL((kda_conv_swish_kernel<IO, DK, DV, 4>), g, b, 0, s, a, j); break;
    }
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_prologue_t(const PrologueArgs &a, const void *const raw[3], const float *const w[3],
                             const float *g_raw, const float *b_raw, const void *st_in, void *st_out, void *const out[3],
                             float *g, float *b, hipStream_t s) {
    hipError_t e;
    if (a.dk == 128) e = a.dv == 128 ? launch_conv<IO, 128, 128>(a, raw, w, st_in, st_out, out, s)
                                     : launch_conv<IO, 128, 64>(a, raw, w, st_in, st_out, out, s);
    else e = a.dv == 128 ? launch_conv<IO, 64, 128>(a, raw, w, st_in, st_out, out, s)
                         : launch_conv<IO, 64, 64>(a, raw, w, st_in, st_out, out, s);
    if (e != hipSuccess) return e;
    if (st_out && a.W > 1 && a.num_seqs > 0) {
        const int64_t total = (int64_t)a.num_seqs * (a.W - 1) * a.H * ((2 * a.dk + a.dv) / Seg16<IO>::N);
        hipLaunchKernelGGL(kda_conv_state_carry_kernel<IO>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a,
                           static_cast<const IO *>(st_in), static_cast<IO *>(st_out));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t gcount = a.tokens * a.H * a.dk, bcount = a.tokens * a.H;
    const int64_t n = std::max(gcount / 4, bcount);
    if (n > 0) {
        hipLaunchKernelGGL(kda_gate_beta_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gcount, bcount,
                           g_raw, b_raw, g, b);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_prologue(kda_dtype_t io, int64_t tokens, int32_t num_seqs, int32_t seq_len, int32_t H, int32_t dk,
                           int32_t dv, int32_t W, const int32_t *cu, float eps, const void *const raw[3],
                           const float *const w[3], const float *g_raw, const float *b_raw, const void *st_in,
                           void *st_out, void *const out[3], float *g, float *b, hipStream_t s) {
    PrologueArgs a{tokens, num_seqs, seq_len, H, dk, dv, W, cu, eps};
    return io == KDA_BF16 ? launch_prologue_t<uint16_t>(a, raw, w, g_raw, b_raw, st_in, st_out, out, g, b, s)
                          : launch_prologue_t<float>(a, raw, w, g_raw, b_raw, st_in, st_out, out, g, b, s);
}

}  // namespace kda
