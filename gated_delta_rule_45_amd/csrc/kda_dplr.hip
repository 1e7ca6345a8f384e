// General-DPLR comparator variants (bf16 and fp32 io).
#include "kda_dplr_impl.h"

namespace kda {

bool dplr_variant_supported(kda_dtype_t io, int dk, int dvt, int chunk) {
    return io == KDA_BF16 ? dplr_supported<uint16_t>(dk, dvt, chunk) : dplr_supported<float>(dk, dvt, chunk);
}

hipError_t launch_dplr_fwd(kda_dtype_t io, const DplrParams &dp, int dvt, int chunk, hipStream_t stream) {
    return io == KDA_BF16 ? launch_dplr<uint16_t>(dp, dvt, chunk, stream) : launch_dplr<float>(dp, dvt, chunk, stream);
}

}  // namespace kda
