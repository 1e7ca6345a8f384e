// fp32-io two-pass variants (fp32 matrix-core operands and accumulation).
#include "kda_split_impl.h"

namespace kda {

size_t split_record_size_f32(int dk, int chunk) { return split_record_size<float>(dk, chunk); }
bool split_scan_shape_f32(int dk, int chunk, int spw, int nw, int &threads, int &lds) {
    return split_scan_shape<float>(dk, chunk, spw, nw, threads, lds);
}
bool split_supported_f32(int dk, int chunk, int spw, int nw, bool keep) {
    return split_supported<float>(dk, chunk, spw, nw, keep);
}
hipError_t launch_split_f32(const FwdParams &p, int chunk, int spw, int nw, char *workspace, int64_t chunk_upper,
                            hipStream_t stream) {
    return launch_split<float>(p, chunk, spw, nw, workspace, chunk_upper, stream);
}

}  // namespace kda
