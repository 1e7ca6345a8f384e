// fp32-io backward variants (fp32 matrix-core operands and accumulation).
#include "kda_bwd_impl.h"

namespace kda {

bool bwd_supported_f32(int dk, int dv, int chunk) { return bwd_supported<float>(dk, dv, chunk); }
size_t bwd_record_bytes_f32(int dk, int chunk) { return bwd_record_bytes<float>(dk, chunk); }
hipError_t launch_bwd_f32(const BwdParams &bp, int chunk, hipStream_t stream) {
    return launch_bwd<float>(bp, chunk, stream);
}

}  // namespace kda
