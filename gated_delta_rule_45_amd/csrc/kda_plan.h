// Plan of a packed batch, shared by the two-pass forward and the backward: the chunk-offset
// table and the longest-first order in which the per-sequence workgroups run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

// ------------------------------------------------------------------- plan ----
inline unsigned plan_blocks(int32_t num_seqs) { return (unsigned)(num_seqs > 256 ? (num_seqs + 255) / 256 : 1); }

// Launched with plan_blocks(num_seqs) workgroups of 256 threads; the layout in the workspace is
// plan_offsets_bytes / plan_order.
//  chunk_off[n] = sum_{m<n} ceil(len_m / C)            (workgroup 0)
//  order[r]     = the sequence of rank r when the sequences are sorted by chunk count, most
//                 chunks first, equal counts in batch order (every workgroup ranks 256 of them)
static __global__ void __launch_bounds__(256) kda_plan_kernel(const int32_t *__restrict__ cu, int32_t num_seqs, int32_t C,
                                                              int32_t *__restrict__ chunk_off, int32_t *__restrict__ order) {
    __shared__ int32_t part[256];
    const int t = threadIdx.x;
    if (blockIdx.x == 0) {
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
        __syncthreads();  // part is reused below
    }
    // rank of sequence i = #{j : nc_j > nc_i} + #{j < i : nc_j == nc_i}, a permutation of 0..n-1
    const int i = blockIdx.x * 256 + t;
    const int32_t nci = i < num_seqs ? (cu[i + 1] - cu[i] + C - 1) / C : 0;
    int32_t rank = 0;
    for (int j0 = 0; j0 < num_seqs; j0 += 256) {
        const int j = j0 + t;
        part[t] = j < num_seqs ? (cu[j + 1] - cu[j] + C - 1) / C : -1;
        __syncthreads();
        const int m = min(256, num_seqs - j0);
        for (int jj = 0; jj < m; ++jj) {
            const int32_t ncj = part[jj];
            rank += (ncj > nci) || (ncj == nci && j0 + jj < i);
        }
        __syncthreads();
    }
    if (i < num_seqs) order[rank] = i;
}

inline hipError_t launch_plan(const int32_t *cu, int32_t num_seqs, int32_t chunk, void *plan, hipStream_t stream) {
    hipLaunchKernelGGL(kda_plan_kernel, dim3(plan_blocks(num_seqs)), dim3(256), 0, stream, cu, num_seqs, chunk,
                       static_cast<int32_t *>(plan), plan_order(plan, num_seqs));
    return hipGetLastError();
}

}  // namespace kda
