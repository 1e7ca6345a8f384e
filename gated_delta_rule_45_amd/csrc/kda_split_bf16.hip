// bf16-io two-pass variants (bf16 matrix-core operands, fp32 accumulation and state).
#include "kda_split_impl.h"

namespace kda {

size_t split_record_size_bf16(int dk, int chunk) { return split_record_size<uint16_t>(dk, chunk); }
bool split_scan_shape_bf16(int dk, int chunk, int spw, int nw, int &threads, int &lds) {
    return split_scan_shape<uint16_t>(dk, chunk, spw, nw, threads, lds);
}
bool split_supported_bf16(int dk, int chunk, int spw, int nw, bool keep) {
    return split_supported<uint16_t>(dk, chunk, spw, nw, keep);
}
hipError_t launch_split_bf16(const FwdParams &p, int chunk, int spw, int nw, char *workspace, int64_t chunk_upper,
                             hipStream_t stream) {
    return launch_split<uint16_t>(p, chunk, spw, nw, workspace, chunk_upper, stream);
}

}  // namespace kda
