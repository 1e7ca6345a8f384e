// bf16-io backward variants (bf16 matrix-core operands, fp32 accumulation and states),
// and the chunk-offset plan launch used by the backward.
#include "kda_bwd_impl.h"
#include "kda_plan.h"

namespace kda {

bool bwd_supported_bf16(int dk, int dv, int chunk) { return bwd_supported<uint16_t>(dk, dv, chunk); }
size_t bwd_record_bytes_bf16(int dk, int chunk) { return bwd_record_bytes<uint16_t>(dk, chunk); }
hipError_t launch_bwd_bf16(const BwdParams &bp, int chunk, hipStream_t stream) {
    return launch_bwd<uint16_t>(bp, chunk, stream);
}

hipError_t launch_chunk_plan(const int32_t *cu, int32_t num_seqs, int32_t chunk, void *plan, hipStream_t stream) {
    return launch_plan(cu, num_seqs, chunk, plan, stream);
}

}  // namespace kda
