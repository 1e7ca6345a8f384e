// Chunk-offset table of a packed batch, shared by the two-pass forward and the backward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// ------------------------------------------------------------------- plan ----
// chunk_off[n] = sum_{m<n} ceil(len_m / C) for a packed batch (one workgroup).
static __global__ void __launch_bounds__(256) kda_plan_kernel(const int32_t *__restrict__ cu, int32_t num_seqs, int32_t C,
                                                       int32_t *__restrict__ chunk_off) {
    __shared__ int32_t part[256];
    const int t = threadIdx.x;
    const int per = (num_seqs + 255) / 256;
    const int n0 = min(t * per, num_seqs), n1 = min(n0 + per, num_seqs);
    int32_t s = 0;
    for (int n = n0; n < n1; ++n) s += (cu[n + 1] - cu[n] + C - 1) / C;
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive scan of the partial sums
        const int32_t x = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int32_t run = part[t] - s;
    for (int n = n0; n < n1; ++n) {
        chunk_off[n] = run;
        run += (cu[n + 1] - cu[n] + C - 1) / C;
    }
    if (t == 255) chunk_off[num_seqs] = part[255];
}

}  // namespace kda
