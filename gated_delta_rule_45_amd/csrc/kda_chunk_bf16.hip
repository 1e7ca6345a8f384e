// bf16-io chunk-forward variants (bf16 matrix-core operands, fp32 accumulation and state).
#include "kda_chunk_impl.h"

namespace kda {

int chunk_variant_lds_bytes_bf16(int dk, int dv_tile, int chunk) { return chunk_variant_lds<uint16_t>(dk, dv_tile, chunk); }

hipError_t launch_chunk_fwd_bf16(const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream) {
    return launch_chunk<uint16_t>(p, cfg, stream);
}

}  // namespace kda
