// fp32-io chunk-forward variants (fp32 matrix-core operands and accumulation).
#include "kda_chunk_impl.h"

namespace kda {

int chunk_variant_lds_bytes_f32(int dk, int dv_tile, int chunk) { return chunk_variant_lds<float>(dk, dv_tile, chunk); }

hipError_t launch_chunk_fwd_f32(const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream) {
    return launch_chunk<float>(p, cfg, stream);
}

}  // namespace kda
