// Internal (non-ABI) declarations shared by the host dispatch and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// The host-side argument checks of kda_chunk_fwd (problem, pointers, alignment, aliasing and
// cu_seqlens_host), without the workspace; KDA_OK clears the error and reports the sequence count.
kda_status_t check_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *initial_state,
                             const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, const void *out,
                             const float *final_state, int64_t *num_seqs);
// Records a status message readable with kda_last_error() (this thread) and returns the status.
kda_status_t set_error(kda_status_t st, const char *fmt, ...);

// Everything a forward launch needs; pointers are device pointers.
struct FwdParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *s0;     // [num_seqs, H, DK, DV] or null
    const int32_t *cu;   // [num_seqs + 1] or null (then sequence n is tokens [n*T, (n+1)*T))
    const int32_t *order;// optional schedule: order[r] = sequence of rank r, most chunks first
    void *out;
    float *sf;           // [num_seqs, H, DK, DV] or null
    int32_t num_seqs, T, H, dk, dv;
    float scale;
    // Optional per-chunk outputs of the forward, kept for the backward pass:
    // hs [slot, H, DK, DV] the state entering each chunk, dch [slot, H, C, DV] the
    // chunk's delta-rule corrections D (both in the operand type: bf16 for bf16 io).  slot = chunk_off[n] + chunk index
    // for a packed batch (chunk_off from the plan kernel), n * ceil(T / C) + chunk index
    // otherwise.
    void *hs = nullptr;
    void *dch = nullptr;
    const int32_t *chunk_off = nullptr;
    // Fused prologue (two-pass forward only): q, k, v, g and beta hold the raw projections, and the
    // kernels apply the short convolution (taps conv[0..2] for q, k, v: fp32 [H, d, conv_w]) with
    // Swish, the L2 normalisation of q and k (norm_eps) and the gate and beta activations as they
    // read them.  Null conv[0]: the inputs are the operator's own.
    const float *conv[3] = {nullptr, nullptr, nullptr};
    int32_t conv_w = 0;
    float norm_eps = 0.f;
    // two-pass forward without its plan and prep launches: the chunk offsets and the records are
    // already in the workspace (the backward's prep kernel writes them)
    bool skip_prep = false;
};

// Chunk-forward configuration chosen by the host.
struct ChunkConfig {
    int chunk;
    int dv_tile;
};

// Compiled chunk-forward variants (per io dtype) and their LDS footprint; 0 = not built.
int chunk_variant_lds_bytes(kda_dtype_t io, int dk, int dv_tile, int chunk);
hipError_t launch_chunk_fwd(kda_dtype_t io, const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream);
// one entry per io dtype (the two kernel files)
int chunk_variant_lds_bytes_f32(int dk, int dv_tile, int chunk);
int chunk_variant_lds_bytes_bf16(int dk, int dv_tile, int chunk);
hipError_t launch_chunk_fwd_f32(const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream);
hipError_t launch_chunk_fwd_bf16(const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream);

// Token-serial kernels (recurrent reference mode and the decode step).
hipError_t launch_recurrent_fwd(kda_dtype_t io, const FwdParams &p, hipStream_t stream);
hipError_t launch_decode_step(kda_dtype_t io, int32_t N, int32_t H, int32_t dk, int32_t dv, float scale,
                              const void *q, const void *k, const void *v, const float *g, const float *beta,
                              float *state, void *out, hipStream_t stream);

// Decode step with the output epilogue (RMSNorm and gate) fused in: one workgroup per (sequence, head).
hipError_t launch_decode_gated(kda_dtype_t io, int32_t N, int32_t H, int32_t dk, int32_t dv, float scale, float eps,
                               const void *q, const void *k, const void *v, const float *g, const float *beta,
                               float *state, const void *gate, const float *weight, void *out, hipStream_t stream);

constexpr int kChunkThreads = 256;

// Plan of a packed batch at the start of the two-pass forward's and the backward's workspace:
// [chunk offsets: num_seqs + 1 int32][longest-first order: num_seqs int32], each padded to 256 bytes.
inline size_t plan_offsets_bytes(int64_t num_seqs) { return (size_t)(((num_seqs + 1) * 4 + 255) / 256 * 256); }
inline size_t split_plan_bytes(int64_t num_seqs) {
    return plan_offsets_bytes(num_seqs) + (size_t)((num_seqs * 4 + 255) / 256 * 256);
}
inline int32_t *plan_order(void *plan, int64_t num_seqs) {
    return reinterpret_cast<int32_t *>(static_cast<char *>(plan) + plan_offsets_bytes(num_seqs));
}
size_t split_workspace_bytes(kda_dtype_t io, int dk, int chunk, int64_t chunk_upper, int H, int64_t num_seqs);
bool split_variant_supported(kda_dtype_t io, int dk, int chunk, int spw, int nw, bool keep = false);
// workgroup size and LDS of the forward's scan kernel for a shape; false if not compiled
bool split_scan_shape(kda_dtype_t io, int dk, int chunk, int spw, int nw, int &threads, int &lds);
hipError_t launch_split_fwd(kda_dtype_t io, const FwdParams &p, int chunk, int spw, int nw, char *workspace,
                            int64_t chunk_upper, hipStream_t stream);
// one entry per io dtype
size_t split_record_size_f32(int dk, int chunk);
size_t split_record_size_bf16(int dk, int chunk);
bool split_supported_f32(int dk, int chunk, int spw, int nw, bool keep);
bool split_scan_shape_f32(int dk, int chunk, int spw, int nw, int &threads, int &lds);
bool split_scan_shape_bf16(int dk, int chunk, int spw, int nw, int &threads, int &lds);
bool split_supported_bf16(int dk, int chunk, int spw, int nw, bool keep);
hipError_t launch_split_f32(const FwdParams &p, int chunk, int spw, int nw, char *workspace, int64_t chunk_upper,
                            hipStream_t stream);
hipError_t launch_split_bf16(const FwdParams &p, int chunk, int spw, int nw, char *workspace, int64_t chunk_upper,
                             hipStream_t stream);
constexpr int kSerialThreads = 256;

// Backward: reverse chunk scan + per-chunk gradients (kda_bwd_*.hip); the forward pass
// that keeps the chunk states is the fused forward with FwdParams::hs / dch set.
struct BwdParams {
    FwdParams f;          // forward inputs and sizes (f.out, f.sf unused)
    const void *d_out;    // dO [tokens, H, DV] io dtype
    const float *d_sf;    // [num_seqs, H, DK, DV] or null (zero)
    void *dq, *dk, *dv;   // [tokens, H, DK|DV] io dtype
    float *dg;            // [tokens, H, DK]
    float *dbeta;         // [tokens, H]
    float *ds0;           // [num_seqs, H, DK, DV] or null
    const void *hs;       // [slot, H, DK, DV] chunk initial states (operand type; forward pass)
    void *dhs;            // [slot, H, DK, DV] gradient of each chunk's final state (operand type)
    const void *dch;      // [slot, H, C, DV] D per chunk (operand type)
    void *duch;           // [slot, H, C, DV] dU per chunk (operand type)
    char *brec;           // [slot, H] reverse-scan records (kda_bwd_prep_kernel)
    int32_t *split_flag;  // [slot, H] 1 where a sub-chunk of the chunk decays beyond the single-anchor
                          // limit of the diagonal blocks (kda_bwd_prep_kernel writes every entry)
    int64_t slots;        // upper bound on the number of chunk slots
    // [slot, H] two-pass forward records for the forward pass that keeps S and D (K~, K-^T, T and
    // e^{G_C}; the output's Q~ and P are left out), written by kda_bwd_prep_kernel; null: not written
    char *frec = nullptr;
    int phases = 3;  // launches: 1 = the prep kernel, 2 = the reverse scan and the gradients
    int cus = 256;   // compute units of the device (grid of the strong-decay gradient pass)
};
bool bwd_supported_bf16(int dk, int dv, int chunk);
size_t bwd_record_bytes_bf16(int dk, int chunk);
size_t bwd_record_bytes_f32(int dk, int chunk);
bool bwd_supported_f32(int dk, int dv, int chunk);
hipError_t launch_bwd_bf16(const BwdParams &bp, int chunk, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdParams &bp, int chunk, hipStream_t stream);
// writes the plan (chunk offsets and order) of a packed batch to `plan`
hipError_t launch_chunk_plan(const int32_t *cu, int32_t num_seqs, int32_t chunk, void *plan, hipStream_t stream);

// General-DPLR comparator (kda_dplr.hip).
struct DplrParams {
    FwdParams f;        // q, k (write key), v, g, s0, cu, out, sf, sizes, scale (f.beta unused)
    const void *a, *b;  // [tokens, H, DK] io dtype
};
bool dplr_variant_supported(kda_dtype_t io, int dk, int dvt, int chunk);
hipError_t launch_dplr_fwd(kda_dtype_t io, const DplrParams &dp, int dvt, int chunk, hipStream_t stream);

// Prologue (short convolution + Swish, q/k L2 normalisation, gate and beta activations).
hipError_t launch_prologue(kda_dtype_t io, int64_t tokens, int32_t num_seqs, int32_t seq_len, int32_t H, int32_t dk,
                           int32_t dv, int32_t W, const int32_t *cu, float eps, const void *const raw[3],
                           const float *const w[3], const float *g_raw, const float *b_raw, const void *st_in,
                           void *st_out, void *const out[3], float *g, float *b, hipStream_t s);

// Output epilogue (per-head RMSNorm and output gate) over rows of d values.
int64_t norm_gate_blocks(kda_dtype_t io, int64_t rows, int d);
hipError_t launch_norm_gate(kda_dtype_t io, int64_t rows, int d, float eps, const void *o, const void *z,
                            const float *w, void *out, hipStream_t stream);

}  // namespace kda
