// kda_chunk_fwd_noalloc: the two-pass chunkwise forward with its scratch memory (chunk-offset table
// and per-chunk records) in a fixed device array of this library instead of a caller's workspace,
// for callers that cannot allocate device memory.  Calls on one device share the array: calls that
// overlap on a device race, and the array keeps the last call's contents (the two-pass kernels
// write every byte they later read, so nothing needs clearing between calls).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB on every device the library runs on

// The array itself.  In host code this name is a host-side stand-in, not a device address: every
// use below goes through the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of the array, looked up on the first call on that
// device (with it current) and kept; hipSuccess or the lookup's error.
hipError_t scratch_address(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t kda_noalloc_scratch_bytes(void) { return kScratchBytes; }

kda_status_t kda_chunk_fwd_noalloc(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, const float *initial_state,
                                   const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                                   float *final_state, void *stream) {
    try {
        if (!problem) return kda::set_error(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
        kda_problem_t p = *problem;
        p.algo = KDA_ALGO_TWO_PASS;
        // every argument is checked on the host before the device is touched
        int64_t num_seqs = 0;
        kda_status_t st = kda::check_chunk_fwd(&p, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
                                               out, final_state, &num_seqs);
        if (st != KDA_OK) return st;
        if (num_seqs == 0) return KDA_OK;  // no sequence: nothing to compute, no scratch used
        kda_problem_t pq = p;
        if (!cu_seqlens) pq.num_seqs = 0;  // kda_query: a plain batch
        kda_query_result_t r;
        st = kda_query(&pq, 0, &r);
        if (st != KDA_OK) return st;
        if (r.workspace_bytes > kScratchBytes)
            return kda::set_error(KDA_ERR_WORKSPACE,
                                  "kda_chunk_fwd_noalloc: this problem needs %zu bytes of scratch, the library's "
                                  "fixed array holds %zu (call kda_chunk_fwd with a workspace)",
                                  r.workspace_bytes, kScratchBytes);
        void *ptr = nullptr;
        const hipError_t e = scratch_address(&ptr);
        if (e != hipSuccess)
            return kda::set_error(KDA_ERR_HIP, "kda_chunk_fwd_noalloc: scratch address: %s", hipGetErrorString(e));
        return kda_chunk_fwd(&p, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, out, final_state, ptr,
                             kScratchBytes, stream);
    } catch (...) {
        return kda::set_error(KDA_ERR_HIP, "unexpected exception in kda_chunk_fwd_noalloc");
    }
}

}  // extern "C"
