// Output epilogue: per-head RMSNorm followed by the data-dependent output gate (Kimi Linear
// summary page, section "Kimi Linear model composition"; the page gives no formula, the
// reading is out = o * rsqrt(mean(o^2) + eps) * w * sigmoid(z) for every (token, head) row
// of d values).
//
// Bound: HBM (reads o and z once, writes out once).  Each lane moves one 16-byte segment of
// a row; the lanes of a row sit next to each other in the wave and sum the squares with
// lane shuffles, so a 256-thread workgroup covers 256 * 16 / (d * sizeof) rows.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <typename IO>
struct Seg;  // one 16-byte segment of a row as fp32 values
template <>
struct Seg<uint16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ void load(const uint16_t *p, float (&v)[N]) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static __forceinline__ void store(uint16_t *p, const float (&v)[N]) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        *reinterpret_cast<u32x4 *>(p) = w;
    }
};
template <>
struct Seg<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ void load(const float *p, float (&v)[N]) {
        const f32x4 w = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = w[i];
    }
    __device__ static __forceinline__ void store(float *p, const float (&v)[N]) {
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = v[i];
        *reinterpret_cast<f32x4 *>(p) = w;
    }
};

// o and out may be the same buffer: every lane reads its segment before writing it back.
template <typename IO, int D>
__global__ void __launch_bounds__(256) kda_norm_gate_kernel(int64_t rows, float eps, const IO *o, const IO *z,
                                                           const float *__restrict__ w, IO *out) {
    constexpr int N = Seg<IO>::N;      // values per lane
    constexpr int LPR = D / N;         // lanes per row
    constexpr int RPB = 256 / LPR;     // rows per workgroup
    static_assert(LPR <= 64 && 64 % LPR == 0, "a row lives inside one wave");
    const int t = threadIdx.x;
    const int seg = t % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + t / LPR;
    const bool live = row < rows;
    const int64_t off = (live ? row : 0) * D + seg * N;

    float ov[N], zv[N], wv[N];
    Seg<IO>::load(o + off, ov);
    Seg<IO>::load(z + off, zv);
#pragma unroll
    for (int i = 0; i < N; i += 4) {
        const f32x4 ww = *reinterpret_cast<const f32x4 *>(w + seg * N + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[i + j] = ww[j];
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) ss = fmaf(ov[i], ov[i], ss);
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = rsqrtf(ss * (1.0f / D) + eps);
#pragma unroll
    for (int i = 0; i < N; ++i) ov[i] = ov[i] * r * wv[i] / (1.0f + __expf(-zv[i]));
    if (live) Seg<IO>::store(out + off, ov);
}

template <typename IO, int D>
hipError_t launch_norm_gate_t(int64_t rows, float eps, const void *o, const void *z, const float *w, void *out,
                              hipStream_t stream) {
    constexpr int RPB = 256 / (D / Seg<IO>::N);
    const int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((kda_norm_gate_kernel<IO, D>), dim3((unsigned)blocks), dim3(256), 0, stream, rows, eps,
                       static_cast<const IO *>(o), static_cast<const IO *>(z), w, static_cast<IO *>(out));
    return hipGetLastError();
}

}  // namespace

int64_t norm_gate_blocks(kda_dtype_t io, int64_t rows, int d) {
    const int n = io == KDA_BF16 ? 8 : 4;
    const int rpb = 256 / (d / n);
    return rows / rpb + (rows % rpb != 0);  // no rows + rpb - 1: rows may be as large as INT64_MAX
}

hipError_t launch_norm_gate(kda_dtype_t io, int64_t rows, int d, float eps, const void *o, const void *z,
                            const float *w, void *out, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (io == KDA_BF16)
        return d == 128 ? launch_norm_gate_t<uint16_t, 128>(rows, eps, o, z, w, out, stream)
                        : launch_norm_gate_t<uint16_t, 64>(rows, eps, o, z, w, out, stream);
    return d == 128 ? launch_norm_gate_t<float, 128>(rows, eps, o, z, w, out, stream)
                    : launch_norm_gate_t<float, 64>(rows, eps, o, z, w, out, stream);
}

}  // namespace kda
