// Host side of libkda.so: argument validation, launch configuration and the C ABI.
// Every entry point validates on the host before touching HIP, so invalid calls
// return a status without launching anything (and work on machines without a GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status_t fail(kda_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kda_status_t ok() {
    g_last_error.clear();
    return KDA_OK;
}

}  // namespace

kda_status_t kda::set_error(kda_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// An element type that has passed validation (KDA_F32 or KDA_BF16), as the enum.
kda_dtype_t dtype_of(int32_t io) { return io == KDA_BF16 ? KDA_BF16 : KDA_F32; }

// a * b for a, b >= 0, saturating at INT64_MAX: size checks on caller-given dimensions never overflow
int64_t sat_mul(int64_t a, int64_t b) { return (a != 0 && b > INT64_MAX / a) ? INT64_MAX : a * b; }
int64_t sat_mul(int64_t a, int64_t b, int64_t c) { return sat_mul(sat_mul(a, b), c); }

// Published MI355X peaks used for roofline fractions.
constexpr double kPeakBf16Tflops = 2500.0;
constexpr double kPeakHbmGBps = 8000.0;

// Compute units of the current device, read once per device (256 on MI355X; also the value used
// when no device is visible, as for the host-only queries).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

struct Resolved {
    int64_t tokens = 0;     // flattened token count
    int32_t num_seqs = 0;   // sequences (batch rows or cu_seqlens segments)
    kda::ChunkConfig cfg{64, 128};  // fused algorithm: chunk and d_v tile
    int lds = 0;                    // fused algorithm: LDS per workgroup (0 = not supported)
    bool two_pass_ok = false;       // two-pass algorithm supports the problem
    int spw = 1, nw = 2;            // two-pass: scan workgroup = nw compute waves x 16*spw state columns
    int64_t chunk_upper = 0;        // two-pass: upper bound on the number of chunks
    size_t ws_bytes = 0;            // two-pass: workspace bytes
};

// Default chunk: 32.  Measured with d_k = d_v = 128 in bf16, against chunk 64: 4 x 4,096 tokens x
// 16 heads 0.208 vs 0.220 ms, 64 packed sequences x 32 heads 5.60 vs 5.77 ms, one 131,072-token
// sequence x 32 heads 4.14 vs 4.47 ms.  The prep kernel does less block work per token (three
// 16 x 16 blocks of A and P per 32 tokens instead of ten per 64) with four workgroups of two
// waves per SIMD pair, and the scan's records are small enough for direct staging.
int default_chunk(const kda_problem_t &, int64_t) { return 32; }

// d_v tile: whole rows of the state per workgroup when there are enough (sequence, head)
// chains to fill the GPU, otherwise narrower tiles so more workgroups run side by side
// (each tile redoes the key-side work of its chunk).
int default_dv_tile(int64_t chains, int dv) {
    int t = dv;
    while (t > 32 && chains * (dv / t) < device_cus()) t /= 2;
    return t;
}

// Shape checks common to the chunked and recurrent forward.
kda_status_t check_problem(const kda_problem_t *p, Resolved &r, bool chunked) {
    if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
    if (p->batch < 0 || p->seq_len < 0 || p->num_heads < 1)
        return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes: batch=%d seq_len=%d num_heads=%d", p->batch, p->seq_len,
                    p->num_heads);
    if (p->io_dtype != KDA_F32 && p->io_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not KDA_F32 or KDA_BF16", (int)p->io_dtype);
    if (!supported_head_dim(p->head_dim_k) || !supported_head_dim(p->head_dim_v))
        return fail(KDA_ERR_UNSUPPORTED, "head dims d_k=%d d_v=%d: supported are 64 and 128", p->head_dim_k,
                    p->head_dim_v);
    if (!std::isfinite(p->scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
    if (chunked) {
        if (p->chunk_size != 0 && p->chunk_size != 16 && p->chunk_size != 32 && p->chunk_size != 64)
            return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: supported are 16, 32, 64 (0 = default)", p->chunk_size);
        if (p->dv_tile != 0 && p->dv_tile != 16 && p->dv_tile != 32 && p->dv_tile != 64 && p->dv_tile != 128)
            return fail(KDA_ERR_UNSUPPORTED, "dv_tile %d: supported are 16, 32, 64, 128 (0 = default)", p->dv_tile);
        if (p->dv_tile > p->head_dim_v)
            return fail(KDA_ERR_INVALID_ARGUMENT, "dv_tile %d exceeds d_v %d", p->dv_tile, p->head_dim_v);
        if (p->algo != KDA_ALGO_AUTO && p->algo != KDA_ALGO_FUSED && p->algo != KDA_ALGO_TWO_PASS)
            return fail(KDA_ERR_INVALID_ARGUMENT, "algo %d is not a kda_algo_t", (int)p->algo);
    }
    return KDA_OK;
}

kda_status_t resolve(const kda_problem_t *p, bool varlen, Resolved &r, bool chunked) {
    kda_status_t st = check_problem(p, r, chunked);
    if (st != KDA_OK) return st;
    if (varlen) {
        if (p->batch != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens needs batch == 1 (got %d)", p->batch);
        if (p->num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", p->num_seqs);
        r.num_seqs = p->num_seqs;
        r.tokens = p->seq_len;
    } else {
        r.num_seqs = p->batch;
        r.tokens = (int64_t)p->batch * p->seq_len;
    }
    const int64_t blocks_max = sat_mul(r.num_seqs, p->num_heads, 4);
    if (blocks_max > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
    if (sat_mul(r.tokens, p->num_heads, std::max(p->head_dim_k, p->head_dim_v)) >= (1LL << 62))
        return fail(KDA_ERR_UNSUPPORTED, "tensor too large");
    if (chunked) {
        const int64_t chains = (int64_t)r.num_seqs * p->num_heads;
        const int C = p->chunk_size ? p->chunk_size : default_chunk(*p, chains);
        r.cfg.chunk = C;
        r.cfg.dv_tile = p->dv_tile ? p->dv_tile : default_dv_tile((int64_t)r.num_seqs * p->num_heads, p->head_dim_v);
        r.lds = kda::chunk_variant_lds_bytes(dtype_of(p->io_dtype), p->head_dim_k, r.cfg.dv_tile, r.cfg.chunk);
        // two-pass: scan workgroups of two compute waves, each owning 16 (32-column tiles) or 32
        // (64-column tiles) state columns, or of one 16-column wave.  By default 64-column tiles
        // once they still give every CU two workgroups: each record is then staged half as often
        // (measured on 64 packed sequences x 32 heads: 7.01 vs 8.71 ms, and 5.78 vs 6.62 ms with
        // 16-column tiles at 9.1 ms); 16-column tiles where 32-column ones leave CUs idle (one
        // 131,072-token sequence x 32 heads: 4.37 vs 4.52 ms); otherwise 32-column tiles.
        int scan_cols = p->dv_tile == 64 ? 64 : p->dv_tile == 16 ? 16 : 32;
        const int cus = device_cus();
        if (p->dv_tile == 0 && p->head_dim_v >= 64 && chains * (p->head_dim_v / 64) >= 2 * cus &&
            kda::split_variant_supported(dtype_of(p->io_dtype), p->head_dim_k, C, 2, 2))
            scan_cols = 64;
        else if (p->dv_tile == 0 && chains * (p->head_dim_v / 32) < cus &&
                 kda::split_variant_supported(dtype_of(p->io_dtype), p->head_dim_k, C, 1, 1))
            scan_cols = 16;
        r.spw = scan_cols == 64 ? 2 : 1;
        r.nw = scan_cols == 16 ? 1 : 2;
        r.two_pass_ok = p->dv_tile != 128 && scan_cols <= p->head_dim_v &&
                        kda::split_variant_supported(dtype_of(p->io_dtype), p->head_dim_k, C, r.spw, r.nw);
        if (r.two_pass_ok) {
            const int64_t per = ((int64_t)p->seq_len + C - 1) / C;
            r.chunk_upper = varlen ? per + r.num_seqs : (int64_t)r.num_seqs * per;
            r.ws_bytes = kda::split_workspace_bytes(dtype_of(p->io_dtype), p->head_dim_k, C, r.chunk_upper, p->num_heads,
                                                    r.num_seqs);
        }
        const bool fused_ok = r.lds > 0;
        if (p->algo == KDA_ALGO_FUSED && !fused_ok)
            return fail(KDA_ERR_UNSUPPORTED, "fused: no compiled variant for io=%s d_k=%d dv_tile=%d chunk=%d (LDS)",
                        p->io_dtype == KDA_BF16 ? "bf16" : "fp32", p->head_dim_k, r.cfg.dv_tile, r.cfg.chunk);
        if (p->algo == KDA_ALGO_TWO_PASS && !r.two_pass_ok)
            return fail(KDA_ERR_UNSUPPORTED, "two-pass: no compiled variant for io=%s d_k=%d chunk=%d dv_tile=%d",
                        p->io_dtype == KDA_BF16 ? "bf16" : "fp32", p->head_dim_k, C, p->dv_tile);
        if (!fused_ok && !r.two_pass_ok)
            return fail(KDA_ERR_UNSUPPORTED, "no compiled variant for io=%s d_k=%d dv_tile=%d chunk=%d",
                        p->io_dtype == KDA_BF16 ? "bf16" : "fp32", p->head_dim_k, r.cfg.dv_tile, C);
    }
    return KDA_OK;
}

// Algorithm for this call given the caller's workspace.
kda_status_t pick_algo(const kda_problem_t *p, const Resolved &r, const void *ws, size_t ws_bytes, int &algo) {
    const bool ws_ok = ws != nullptr && ws_bytes >= r.ws_bytes && aligned(ws, 256);
    if (p->algo == KDA_ALGO_TWO_PASS) {
        if (!ws_ok)
            return fail(KDA_ERR_WORKSPACE, "two-pass needs a 256-byte aligned workspace of %zu bytes (got %zu at %p)",
                        r.ws_bytes, ws_bytes, ws);
        algo = KDA_ALGO_TWO_PASS;
    } else if (p->algo == KDA_ALGO_FUSED) {
        algo = KDA_ALGO_FUSED;
    } else {
        algo = (r.two_pass_ok && ws_ok) ? KDA_ALGO_TWO_PASS : KDA_ALGO_FUSED;
        if (algo == KDA_ALGO_FUSED && r.lds <= 0)
            return fail(KDA_ERR_WORKSPACE, "this problem needs the two-pass algorithm and a workspace of %zu bytes",
                        r.ws_bytes);
    }
    return KDA_OK;
}

kda_status_t check_tensors(const kda_problem_t *p, const Resolved &r, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *s0, const int32_t *cu,
                           const int32_t *cu_host, const void *out, const float *sf) {
    if (r.tokens > 0) {
        const void *req[] = {q, k, v, g, beta, out};
        const char *names[] = {"q", "k", "v", "g", "beta", "out"};
        for (int i = 0; i < 6; ++i)
            if (!req[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        const void *al16[] = {q, k, v, g, out};
        const char *n16[] = {"q", "k", "v", "g", "out"};
        for (int i = 0; i < 5; ++i)
            if (!aligned(al16[i], 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
        if (!aligned(beta, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "beta is not 4-byte aligned");
    }
    if (s0 && !aligned(s0, 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "initial_state is not 16-byte aligned");
    if (sf && !aligned(sf, 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "final_state is not 16-byte aligned");
    const bool varlen = cu != nullptr;
    if (varlen && !aligned(cu, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    if (!varlen && cu_host) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host given without cu_seqlens");
    if (cu_host) {
        if (cu_host[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d, expected 0", cu_host[0]);
        for (int32_t i = 0; i < r.num_seqs; ++i)
            if (cu_host[i + 1] < cu_host[i])
                return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d (%d -> %d)", i, cu_host[i],
                            cu_host[i + 1]);
        if (cu_host[r.num_seqs] != p->seq_len)
            return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[%d] = %d, expected seq_len %d", r.num_seqs,
                        cu_host[r.num_seqs], p->seq_len);
    }
    // aliasing: only initial_state == final_state is allowed among the written buffers
    const void *outs[] = {out, sf};
    const void *ins[] = {q, k, v, g, beta};
    for (const void *o : outs) {
        if (!o) continue;
        for (const void *i : ins)
            if (o == i) return fail(KDA_ERR_INVALID_ARGUMENT, "an output aliases an input tensor");
    }
    if (out && (out == s0 || out == sf)) return fail(KDA_ERR_INVALID_ARGUMENT, "out aliases a state buffer");
    return KDA_OK;
}

kda_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

kda::FwdParams make_params(const kda_problem_t *p, const Resolved &r, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *s0, const int32_t *cu, void *out,
                           float *sf) {
    kda::FwdParams fp;
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.g = g;
    fp.beta = beta;
    fp.s0 = s0;
    fp.cu = cu;
    fp.order = nullptr;
    fp.out = out;
    fp.sf = sf;
    fp.num_seqs = r.num_seqs;
    fp.T = p->seq_len;
    fp.H = p->num_heads;
    fp.dk = p->head_dim_k;
    fp.dv = p->head_dim_v;
    fp.scale = p->scale;
    return fp;
}

// ----------------------------------------------------------------- backward --
struct BwdResolved {
    Resolved r;
    int chunk = 64;
    bool two_pass = false;  // the forward pass that keeps the chunk states: two-pass (64-column
                            // scan tiles) when compiled for the problem, else fused
    int fwd_dv_tile = 32;   // fused: d_v tile
    int64_t slots = 0;      // chunk slots (upper bound for a packed batch)
    size_t off_hs = 0, off_dhs = 0, off_dch = 0, off_duch = 0, off_brec = 0, off_flag = 0, ws_bytes = 0;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool bwd_variant_supported(kda_dtype_t io, int dk, int dv, int chunk) {
    return io == KDA_BF16 ? kda::bwd_supported_bf16(dk, dv, chunk) : kda::bwd_supported_f32(dk, dv, chunk);
}

kda_status_t resolve_bwd(const kda_problem_t *p, bool varlen, BwdResolved &b) {
    kda_status_t st = resolve(p, varlen, b.r, false);
    if (st != KDA_OK) return st;
    if (p->chunk_size != 0 && p->chunk_size != 16 && p->chunk_size != 32 && p->chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "chunk_size %d: supported are 16, 32, 64 (0 = default)", p->chunk_size);
    const int dk = p->head_dim_k, dv = p->head_dim_v;
    if (p->chunk_size) {
        b.chunk = p->chunk_size;
    } else {  // largest chunk with a compiled variant
        b.chunk = 0;
        for (int c : {64, 32, 16})
            if (bwd_variant_supported(dtype_of(p->io_dtype), dk, dv, c) &&
                kda::chunk_variant_lds_bytes(dtype_of(p->io_dtype), dk, 32, c) > 0) {
                b.chunk = c;
                break;
            }
        if (b.chunk == 0) return fail(KDA_ERR_UNSUPPORTED, "backward: no compiled variant for d_k=%d d_v=%d", dk, dv);
    }
    if (!bwd_variant_supported(dtype_of(p->io_dtype), dk, dv, b.chunk))
        return fail(KDA_ERR_UNSUPPORTED, "backward: no compiled variant for io=%s d_k=%d d_v=%d chunk=%d (LDS)",
                    p->io_dtype == KDA_BF16 ? "bf16" : "fp32", dk, dv, b.chunk);
    // the forward again with the 32-column scan (twice the workgroups of the 64-column one)
    b.two_pass = dv % 32 == 0 && kda::split_variant_supported(dtype_of(p->io_dtype), dk, b.chunk, 1, 2, true);
    b.fwd_dv_tile = 0;
    if (!b.two_pass) {
        for (int t : {default_dv_tile((int64_t)b.r.num_seqs * p->num_heads, dv), 32})
            if (t <= dv && kda::chunk_variant_lds_bytes(dtype_of(p->io_dtype), dk, t, b.chunk) > 0) {
                b.fwd_dv_tile = t;
                break;
            }
        if (b.fwd_dv_tile == 0)
            return fail(KDA_ERR_UNSUPPORTED, "backward: no forward variant keeps the states for d_k=%d chunk=%d", dk,
                        b.chunk);
    }
    const int64_t per = ((int64_t)p->seq_len + b.chunk - 1) / b.chunk;
    b.slots = varlen ? per + b.r.num_seqs : (int64_t)b.r.num_seqs * per;
    if (b.slots * p->num_heads > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many chunks");
    const size_t s_io = p->io_dtype == KDA_BF16 ? 2 : 4;
    const size_t states = align256((size_t)b.slots * p->num_heads * dk * dv * s_io);  // operand type
    const size_t tiles = align256((size_t)b.slots * p->num_heads * b.chunk * dv * s_io);
    // [chunk offsets][two-pass records (when two-pass)][states][state gradients][D][dU][records][flags]
    b.off_hs = b.two_pass ? align256(kda::split_workspace_bytes(dtype_of(p->io_dtype), dk, b.chunk, b.slots, p->num_heads,
                                                                b.r.num_seqs))
                          : kda::split_plan_bytes(b.r.num_seqs);
    b.off_dhs = b.off_hs + states;
    b.off_dch = b.off_dhs + states;
    b.off_duch = b.off_dch + tiles;
    b.off_brec = b.off_duch + tiles;
    const size_t rec = p->io_dtype == KDA_BF16 ? kda::bwd_record_bytes_bf16(dk, b.chunk)
                                               : kda::bwd_record_bytes_f32(dk, b.chunk);
    b.off_flag = b.off_brec + align256((size_t)b.slots * p->num_heads * rec);
    b.ws_bytes = b.off_flag + align256((size_t)b.slots * p->num_heads * sizeof(int32_t));
    return KDA_OK;
}

kda_status_t check_bwd_tensors(const BwdResolved &b, const void *const in[], const char *const in_names[], int n_in,
                               const void *const outs[], const char *const out_names[], int n_out) {
    for (int i = 0; i < n_out; ++i) {
        if (!outs[i]) continue;
        for (int j = 0; j < n_in; ++j)
            if (outs[i] == in[j])
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s aliases input %s", out_names[i], in_names[j]);
        for (int j = 0; j < i; ++j)
            if (outs[i] == outs[j])
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s aliases %s", out_names[i], out_names[j]);
    }
    (void)b;
    return KDA_OK;
}

}  // namespace

namespace kda {

size_t split_workspace_bytes(kda_dtype_t io, int dk, int chunk, int64_t chunk_upper, int H, int64_t num_seqs) {
    const size_t rec = io == KDA_BF16 ? split_record_size_bf16(dk, chunk) : split_record_size_f32(dk, chunk);
    return split_plan_bytes(num_seqs) + (size_t)chunk_upper * H * rec;
}

bool split_scan_shape(kda_dtype_t io, int dk, int chunk, int spw, int nw, int &threads, int &lds) {
    return io == KDA_BF16 ? split_scan_shape_bf16(dk, chunk, spw, nw, threads, lds)
                          : split_scan_shape_f32(dk, chunk, spw, nw, threads, lds);
}
bool split_variant_supported(kda_dtype_t io, int dk, int chunk, int spw, int nw, bool keep) {
    return io == KDA_BF16 ? split_supported_bf16(dk, chunk, spw, nw, keep) : split_supported_f32(dk, chunk, spw, nw, keep);
}

hipError_t launch_split_fwd(kda_dtype_t io, const FwdParams &p, int chunk, int spw, int nw, char *workspace,
                            int64_t chunk_upper, hipStream_t stream) {
    return io == KDA_BF16 ? launch_split_bf16(p, chunk, spw, nw, workspace, chunk_upper, stream)
                          : launch_split_f32(p, chunk, spw, nw, workspace, chunk_upper, stream);
}

int chunk_variant_lds_bytes(kda_dtype_t io, int dk, int dv_tile, int chunk) {
    return io == KDA_BF16 ? chunk_variant_lds_bytes_bf16(dk, dv_tile, chunk)
                          : chunk_variant_lds_bytes_f32(dk, dv_tile, chunk);
}

hipError_t launch_chunk_fwd(kda_dtype_t io, const FwdParams &p, const ChunkConfig &cfg, hipStream_t stream) {
    return io == KDA_BF16 ? launch_chunk_fwd_bf16(p, cfg, stream) : launch_chunk_fwd_f32(p, cfg, stream);
}

}  // namespace kda

namespace kda {

kda_status_t check_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *initial_state,
                             const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, const void *out,
                             const float *final_state, int64_t *num_seqs) {
    try {
        Resolved r;
        kda_status_t st = resolve(problem, cu_seqlens != nullptr, r, true);
        if (st != KDA_OK) return st;
        st = check_tensors(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, out,
                           final_state);
        if (st != KDA_OK) return st;
        if (num_seqs) *num_seqs = r.num_seqs;
        return ok();
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in argument checks");
    }
}

}  // namespace kda

extern "C" {

kda_status_t kda_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *initial_state,
                           const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                           float *final_state, void *workspace, size_t workspace_bytes, void *stream) {
    try {
        Resolved r;
        kda_status_t st = resolve(problem, cu_seqlens != nullptr, r, true);
        if (st != KDA_OK) return st;
        st = check_tensors(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, out,
                           final_state);
        if (st != KDA_OK) return st;
        int algo = KDA_ALGO_FUSED;
        st = pick_algo(problem, r, workspace, workspace_bytes, algo);
        if (st != KDA_OK) return st;
        if (r.num_seqs == 0) return ok();
        const kda::FwdParams fp =
            make_params(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state);
        if (algo == KDA_ALGO_TWO_PASS)
            return hip_status(kda::launch_split_fwd(dtype_of(problem->io_dtype), fp, r.cfg.chunk, r.spw, r.nw,
                                                    static_cast<char *>(workspace), r.chunk_upper,
                                                    static_cast<hipStream_t>(stream)),
                              "kda_chunk_fwd (two-pass) launch");
        return hip_status(kda::launch_chunk_fwd(dtype_of(problem->io_dtype), fp, r.cfg, static_cast<hipStream_t>(stream)),
                          "kda_chunk_fwd (fused) launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_chunk_fwd");
    }
}

kda_status_t kda_chunk_fwd_prologue(const kda_problem_t *problem, int32_t conv_width, float norm_eps,
                                    const void *q_raw, const void *k_raw, const void *v_raw, const float *conv_q,
                                    const float *conv_k, const float *conv_v, const float *g_raw,
                                    const float *beta_raw, const float *initial_state, const int32_t *cu_seqlens,
                                    const int32_t *cu_seqlens_host, void *out, float *final_state, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    try {
        Resolved r;
        kda_status_t st = resolve(problem, cu_seqlens != nullptr, r, true);
        if (st != KDA_OK) return st;
        if (problem->algo == KDA_ALGO_FUSED || !r.two_pass_ok)
            return fail(KDA_ERR_UNSUPPORTED, "fused prologue: runs in the two-pass algorithm, which has no variant for "
                                             "io=%s d_k=%d chunk=%d dv_tile=%d",
                        problem->io_dtype == KDA_BF16 ? "bf16" : "fp32", problem->head_dim_k, r.cfg.chunk,
                        problem->dv_tile);
        if (conv_width < 1 || conv_width > 4)
            return fail(KDA_ERR_UNSUPPORTED, "conv_width %d: supported are 1..4", conv_width);
        if (!std::isfinite(norm_eps) || norm_eps < 0.f)
            return fail(KDA_ERR_INVALID_ARGUMENT, "norm_eps must be finite and >= 0");
        // raw projections in the places of q, k, v, g and beta
        st = check_tensors(problem, r, q_raw, k_raw, v_raw, g_raw, beta_raw, initial_state, cu_seqlens,
                           cu_seqlens_host, out, final_state);
        if (st != KDA_OK) return st;
        if (r.tokens > 0) {
            const float *taps[] = {conv_q, conv_k, conv_v};
            const char *names[] = {"conv_q", "conv_k", "conv_v"};
            for (int i = 0; i < 3; ++i) {
                if (!taps[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
                if (!aligned(taps[i], 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", names[i]);
                if ((const void *)taps[i] == out || taps[i] == final_state)
                    return fail(KDA_ERR_INVALID_ARGUMENT, "an output aliases %s", names[i]);
            }
        }
        if (!workspace || workspace_bytes < r.ws_bytes || !aligned(workspace, 256))
            return fail(KDA_ERR_WORKSPACE, "fused prologue: needs a 256-byte aligned workspace of %zu bytes (got %zu at %p)",
                        r.ws_bytes, workspace_bytes, workspace);
        if (r.num_seqs == 0) return ok();
        kda::FwdParams fp = make_params(problem, r, q_raw, k_raw, v_raw, g_raw, beta_raw, initial_state, cu_seqlens,
                                        out, final_state);
        fp.conv[0] = conv_q;
        fp.conv[1] = conv_k;
        fp.conv[2] = conv_v;
        fp.conv_w = conv_width;
        fp.norm_eps = norm_eps;
        return hip_status(kda::launch_split_fwd(dtype_of(problem->io_dtype), fp, r.cfg.chunk, r.spw, r.nw,
                                                static_cast<char *>(workspace), r.chunk_upper,
                                                static_cast<hipStream_t>(stream)),
                          "kda_chunk_fwd_prologue launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_chunk_fwd_prologue");
    }
}

kda_status_t kda_chunk_bwd_workspace(const kda_problem_t *problem, size_t *bytes) {
    try {
        if (!bytes) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
        *bytes = 0;
        BwdResolved b;
        kda_status_t st = resolve_bwd(problem, problem && problem->num_seqs > 0, b);
        if (st != KDA_OK) return st;
        *bytes = b.ws_bytes;
        return ok();
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_chunk_bwd_workspace");
    }
}

kda_status_t kda_chunk_bwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *initial_state,
                           const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, const void *d_out,
                           const float *d_final_state, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                           float *d_initial_state, void *workspace, size_t workspace_bytes, void *stream) {
    try {
        BwdResolved b;
        const bool varlen = cu_seqlens != nullptr;
        kda_status_t st = resolve_bwd(problem, varlen, b);
        if (st != KDA_OK) return st;
        const Resolved &r = b.r;
        if (r.tokens > 0) {
            const void *req[] = {d_out, dq, dk, dv, dg, dbeta};
            const char *names[] = {"d_out", "dq", "dk", "dv", "dg", "dbeta"};
            for (int i = 0; i < 6; ++i)
                if (!req[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
            const void *al16[] = {d_out, dq, dk, dv, dg};
            const char *n16[] = {"d_out", "dq", "dk", "dv", "dg"};
            for (int i = 0; i < 5; ++i)
                if (!aligned(al16[i], 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
            if (!aligned(dbeta, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "dbeta is not 4-byte aligned");
        }
        // the forward-side checks (inputs, alignment, cu_seqlens), dq in the place of out
        st = check_tensors(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, dq, nullptr);
        if (st != KDA_OK) return st;
        if (d_final_state && !aligned(d_final_state, 16))
            return fail(KDA_ERR_INVALID_ARGUMENT, "d_final_state is not 16-byte aligned");
        if (d_initial_state && !aligned(d_initial_state, 16))
            return fail(KDA_ERR_INVALID_ARGUMENT, "d_initial_state is not 16-byte aligned");
        const void *ins[] = {q, k, v, g, beta, initial_state, d_out, d_final_state, cu_seqlens};
        const char *in_names[] = {"q", "k", "v", "g", "beta", "initial_state", "d_out", "d_final_state", "cu_seqlens"};
        const void *outs[] = {dq, dk, dv, dg, dbeta, d_initial_state};
        const char *out_names[] = {"dq", "dk", "dv", "dg", "dbeta", "d_initial_state"};
        st = check_bwd_tensors(b, ins, in_names, 9, outs, out_names, 6);
        if (st != KDA_OK) return st;
        if (!workspace || workspace_bytes < b.ws_bytes || !aligned(workspace, 256))
            return fail(KDA_ERR_WORKSPACE, "kda_chunk_bwd needs a 256-byte aligned workspace of %zu bytes (got %zu at %p)",
                        b.ws_bytes, workspace_bytes, workspace);
        if (r.num_seqs == 0) return ok();
        hipStream_t s = static_cast<hipStream_t>(stream);
        char *ws = static_cast<char *>(workspace);
        int32_t *chunk_off = reinterpret_cast<int32_t *>(ws);
        kda::FwdParams fp = make_params(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, nullptr, nullptr);
        fp.hs = ws + b.off_hs;
        fp.dch = ws + b.off_dch;
        fp.chunk_off = varlen ? chunk_off : nullptr;
        fp.order = varlen ? kda::plan_order(ws, r.num_seqs) : nullptr;  // longest sequences first
        kda::BwdParams bp;
        bp.f = fp;
        bp.d_out = d_out;
        bp.d_sf = d_final_state;
        bp.dq = dq;
        bp.dk = dk;
        bp.dv = dv;
        bp.dg = dg;
        bp.dbeta = dbeta;
        bp.ds0 = d_initial_state;
        bp.hs = fp.hs;
        bp.dhs = ws + b.off_dhs;
        bp.dch = fp.dch;
        bp.duch = ws + b.off_duch;
        bp.brec = ws + b.off_brec;
        bp.split_flag = reinterpret_cast<int32_t *>(ws + b.off_flag);
        bp.slots = b.slots;
        bp.cus = device_cus();
        auto launch_bwd = [&](int phases) {
            bp.phases = phases;
            return problem->io_dtype == KDA_BF16 ? kda::launch_bwd_bf16(bp, b.chunk, s) : kda::launch_bwd_f32(bp, b.chunk, s);
        };
        if (varlen) {
            st = hip_status(kda::launch_chunk_plan(cu_seqlens, r.num_seqs, b.chunk, ws, s), "kda_chunk_bwd plan launch");
            if (st != KDA_OK) return st;
        }
        if (b.two_pass) {
            // the backward's prep kernel also writes the two-pass forward's records (one pass over
            // q, k, g and beta serves both); the forward then launches its scan only
            bp.frec = ws + kda::split_plan_bytes(r.num_seqs);
            st = hip_status(launch_bwd(1), "kda_chunk_bwd prep launch");
            if (st != KDA_OK) return st;
            kda::FwdParams fk = fp;
            fk.skip_prep = true;
            st = hip_status(kda::launch_split_fwd(dtype_of(problem->io_dtype), fk, b.chunk, 1, 2, ws, b.slots, s),
                            "kda_chunk_bwd forward launch");
            if (st != KDA_OK) return st;
            return hip_status(launch_bwd(2), "kda_chunk_bwd launch");
        }
        st = hip_status(kda::launch_chunk_fwd(dtype_of(problem->io_dtype), fp, kda::ChunkConfig{b.chunk, b.fwd_dv_tile}, s),
                        "kda_chunk_bwd forward launch");
        if (st != KDA_OK) return st;
        return hip_status(launch_bwd(3), "kda_chunk_bwd launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_chunk_bwd");
    }
}

kda_status_t kda_dplr_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                                const void *a, const void *b, const float *g, const float *initial_state,
                                const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                                float *final_state, void *stream) {
    try {
        Resolved r;
        kda_status_t st = resolve(problem, cu_seqlens != nullptr, r, false);
        if (st != KDA_OK) return st;
        const int C = problem->chunk_size ? problem->chunk_size : 64;
        const int dvt = problem->dv_tile ? problem->dv_tile : 32;
        if (dvt > problem->head_dim_v)
            return fail(KDA_ERR_INVALID_ARGUMENT, "dv_tile %d exceeds d_v %d", dvt, problem->head_dim_v);
        if (!kda::dplr_variant_supported(dtype_of(problem->io_dtype), problem->head_dim_k, dvt, C))
            return fail(KDA_ERR_UNSUPPORTED, "dplr: no compiled variant for io=%s d_k=%d dv_tile=%d chunk=%d",
                        problem->io_dtype == KDA_BF16 ? "bf16" : "fp32", problem->head_dim_k, dvt, C);
        // q, k, v, g, out checks as the forward (beta is not an input here: g stands in for it)
        st = check_tensors(problem, r, q, k, v, g, g, initial_state, cu_seqlens, cu_seqlens_host, out, final_state);
        if (st != KDA_OK) return st;
        if (r.tokens > 0) {
            if (!a || !b) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", !a ? "a" : "b");
            if (!aligned(a, 16) || !aligned(b, 16))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", !aligned(a, 16) ? "a" : "b");
        }
        const void *outs[] = {out, final_state};
        for (const void *o : outs)
            if (o && (o == a || o == b)) return fail(KDA_ERR_INVALID_ARGUMENT, "an output aliases a or b");
        if (r.num_seqs == 0) return ok();
        kda::DplrParams dp;
        dp.f = make_params(problem, r, q, k, v, g, nullptr, initial_state, cu_seqlens, out, final_state);
        dp.a = a;
        dp.b = b;
        return hip_status(kda::launch_dplr_fwd(dtype_of(problem->io_dtype), dp, dvt, C, static_cast<hipStream_t>(stream)),
                          "kda_dplr_chunk_fwd launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_dplr_chunk_fwd");
    }
}

kda_status_t kda_tune(const kda_problem_t *problem, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                      const int32_t *cu_seqlens_host, void *out, float *final_state, void *workspace,
                      size_t workspace_bytes, void *stream, kda_query_result_t *best) {
    try {
        if (!best) return fail(KDA_ERR_INVALID_ARGUMENT, "best is NULL");
        if (!problem) return fail(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
        if (initial_state && (const void *)initial_state == (const void *)final_state)
            return fail(KDA_ERR_INVALID_ARGUMENT, "initial_state aliases final_state (candidates run repeatedly)");
        {  // the problem as given must be valid (fields left at 0 are tuned)
            Resolved r;
            kda_status_t st = resolve(problem, cu_seqlens != nullptr, r, true);
            if (st != KDA_OK) return st;
            st = check_tensors(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, out,
                               final_state);
            if (st != KDA_OK) return st;
        }
        const hipStream_t s = static_cast<hipStream_t>(stream);
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
            if (e0) (void)hipEventDestroy(e0);
            return fail(KDA_ERR_HIP, "hipEventCreate failed");
        }
        const int chunks[3] = {16, 32, 64}, tiles[4] = {16, 32, 64, 128}, algos[2] = {KDA_ALGO_FUSED, KDA_ALGO_TWO_PASS};
        kda_problem_t winner{};
        float best_ms = -1.f;
        kda_status_t err = KDA_OK;
        for (int ci = 0; ci < 3 && err == KDA_OK; ++ci) {
            if (problem->chunk_size && chunks[ci] != problem->chunk_size) continue;
            for (int ai = 0; ai < 2 && err == KDA_OK; ++ai) {
                if (problem->algo != KDA_ALGO_AUTO && algos[ai] != problem->algo) continue;
                for (int ti = 0; ti < 4 && err == KDA_OK; ++ti) {
                    if (problem->dv_tile && tiles[ti] != problem->dv_tile) continue;
                    kda_problem_t c = *problem;
                    c.chunk_size = chunks[ci];
                    c.algo = algos[ai];
                    c.dv_tile = tiles[ti];
                    Resolved r;
                    if (resolve(&c, cu_seqlens != nullptr, r, true) != KDA_OK) continue;  // variant not built
                    if (c.algo == KDA_ALGO_TWO_PASS &&
                        (workspace == nullptr || workspace_bytes < r.ws_bytes || !aligned(workspace, 256)))
                        continue;
                    auto call = [&]() {
                        return kda_chunk_fwd(&c, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, out,
                                             final_state, workspace, workspace_bytes, stream);
                    };
                    if ((err = call()) != KDA_OK) break;
                    if (hipEventRecord(e0, s) != hipSuccess) { err = fail(KDA_ERR_HIP, "hipEventRecord failed"); break; }
                    for (int rep = 0; rep < 3 && err == KDA_OK; ++rep) err = call();
                    if (err != KDA_OK) break;
                    float ms = 0.f;
                    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
                        err = fail(KDA_ERR_HIP, "timing the candidate failed");
                        break;
                    }
                    ms /= 3.f;
                    if (best_ms < 0.f || ms < best_ms) {
                        best_ms = ms;
                        winner = c;
                    }
                }
            }
        }
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
        if (err != KDA_OK) return err;
        if (best_ms < 0.f) return fail(KDA_ERR_UNSUPPORTED, "no candidate configuration runs this problem");
        kda_status_t st = kda_query(&winner, KDA_QUERY_DEVICE, best);
        if (st != KDA_OK) return st;
        best->tuned_ms = best_ms;
        return ok();
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_tune");
    }
}

kda_status_t kda_recurrent_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *initial_state,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                               float *final_state, void *stream) {
    try {
        Resolved r;
        kda_status_t st = resolve(problem, cu_seqlens != nullptr, r, false);
        if (st != KDA_OK) return st;
        st = check_tensors(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host, out,
                           final_state);
        if (st != KDA_OK) return st;
        if (r.num_seqs == 0) return ok();
        const kda::FwdParams fp =
            make_params(problem, r, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state);
        return hip_status(kda::launch_recurrent_fwd(dtype_of(problem->io_dtype), fp, static_cast<hipStream_t>(stream)),
                          "kda_recurrent_fwd launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_recurrent_fwd");
    }
}

kda_status_t kda_decode_step(int32_t num_seqs, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                             int32_t io_dtype, float scale, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, float *state, void *out, void *stream) {
    try {
        if (num_seqs < 0 || num_heads < 1)
            return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes: num_seqs=%d num_heads=%d", num_seqs, num_heads);
        if (io_dtype != KDA_F32 && io_dtype != KDA_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not KDA_F32 or KDA_BF16", (int)io_dtype);
        if (!supported_head_dim(head_dim_k) || !supported_head_dim(head_dim_v))
            return fail(KDA_ERR_UNSUPPORTED, "head dims d_k=%d d_v=%d: supported are 64 and 128", head_dim_k,
                        head_dim_v);
        if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
        if (sat_mul(num_seqs, num_heads, head_dim_v / 32) > 0x7fffffffLL)
            return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
        if (num_seqs == 0) return ok();
        const void *req[] = {q, k, v, g, beta, state, out};
        const char *names[] = {"q", "k", "v", "g", "beta", "state", "out"};
        for (int i = 0; i < 7; ++i)
            if (!req[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        const void *al16[] = {q, k, v, g, state, out};
        const char *n16[] = {"q", "k", "v", "g", "state", "out"};
        for (int i = 0; i < 6; ++i)
            if (!aligned(al16[i], 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
        if (!aligned(beta, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "beta is not 4-byte aligned");
        if (out == state || out == q || out == k || out == v || (const void *)state == (const void *)g ||
            (const void *)state == q || (const void *)state == k || (const void *)state == v)
            return fail(KDA_ERR_INVALID_ARGUMENT, "state or out aliases another tensor");
        return hip_status(kda::launch_decode_step(dtype_of(io_dtype), num_seqs, num_heads, head_dim_k, head_dim_v, scale, q, k,
                                                  v, g, beta, state, out, static_cast<hipStream_t>(stream)),
                          "kda_decode_step launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_decode_step");
    }
}

kda_status_t kda_decode_step_gated(int32_t num_seqs, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                                   int32_t io_dtype, float scale, const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, float *state, const void *gate,
                                   const float *weight, float eps, void *out, void *stream) {
    try {
        if (num_seqs < 0 || num_heads < 1)
            return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes: num_seqs=%d num_heads=%d", num_seqs, num_heads);
        if (io_dtype != KDA_F32 && io_dtype != KDA_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not KDA_F32 or KDA_BF16", (int)io_dtype);
        if (!supported_head_dim(head_dim_k) || !supported_head_dim(head_dim_v))
            return fail(KDA_ERR_UNSUPPORTED, "head dims d_k=%d d_v=%d: supported are 64 and 128", head_dim_k,
                        head_dim_v);
        if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
        if (!std::isfinite(eps) || eps < 0.f) return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
        if (sat_mul(num_seqs, num_heads) > 0x7fffffffLL)
            return fail(KDA_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
        if (num_seqs == 0) return ok();
        const void *req[] = {q, k, v, g, beta, state, gate, weight, out};
        const char *names[] = {"q", "k", "v", "g", "beta", "state", "gate", "weight", "out"};
        for (int i = 0; i < 9; ++i)
            if (!req[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        const void *al16[] = {q, k, v, g, state, gate, weight, out};
        const char *n16[] = {"q", "k", "v", "g", "state", "gate", "weight", "out"};
        for (int i = 0; i < 8; ++i)
            if (!aligned(al16[i], 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
        if (!aligned(beta, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "beta is not 4-byte aligned");
        // the written buffers (state, out) alias nothing
        const void *ins[] = {q, k, v, g, beta, gate, weight};
        for (const void *i : ins)
            if (i == out || i == (const void *)state)
                return fail(KDA_ERR_INVALID_ARGUMENT, "state or out aliases another tensor");
        if (out == (const void *)state) return fail(KDA_ERR_INVALID_ARGUMENT, "out aliases state");
        return hip_status(kda::launch_decode_gated(dtype_of(io_dtype), num_seqs, num_heads, head_dim_k, head_dim_v,
                                                   scale, eps, q, k, v, g, beta, state, gate, weight, out,
                                                   static_cast<hipStream_t>(stream)),
                          "kda_decode_step_gated launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_decode_step_gated");
    }
}

kda_status_t kda_prologue(const kda_prologue_t *p, const void *q_raw, const void *k_raw, const void *v_raw,
                          const float *conv_q, const float *conv_k, const float *conv_v, const float *g_raw,
                          const float *beta_raw, const int32_t *cu_seqlens, const void *conv_state,
                          void *conv_state_out, void *q, void *k, void *v, float *g, float *beta, void *stream) {
    try {
        if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "problem is NULL");
        if (p->batch < 0 || p->seq_len < 0 || p->num_seqs < 0 || p->num_heads < 1)
            return fail(KDA_ERR_INVALID_ARGUMENT, "bad sizes: batch=%d seq_len=%d num_seqs=%d num_heads=%d", p->batch,
                        p->seq_len, p->num_seqs, p->num_heads);
        if (p->io_dtype != KDA_F32 && p->io_dtype != KDA_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not KDA_F32 or KDA_BF16", (int)p->io_dtype);
        if (!supported_head_dim(p->head_dim_k) || !supported_head_dim(p->head_dim_v))
            return fail(KDA_ERR_UNSUPPORTED, "head dims d_k=%d d_v=%d: supported are 64 and 128", p->head_dim_k,
                        p->head_dim_v);
        if (p->conv_width < 1 || p->conv_width > 4)
            return fail(KDA_ERR_UNSUPPORTED, "conv_width %d: supported are 1..4", p->conv_width);
        if (!std::isfinite(p->norm_eps) || p->norm_eps < 0.f)
            return fail(KDA_ERR_INVALID_ARGUMENT, "norm_eps must be finite and >= 0");
        const bool varlen = p->num_seqs > 0;
        if (varlen && p->batch != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens needs batch == 1");
        if (varlen && !cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs > 0 needs cu_seqlens");
        const int64_t tokens = varlen ? (int64_t)p->seq_len : (int64_t)p->batch * p->seq_len;
        const int32_t nseq = varlen ? p->num_seqs : p->batch;
        if (sat_mul(tokens, p->num_heads, std::max(p->head_dim_k, p->head_dim_v)) >= (1LL << 40))
            return fail(KDA_ERR_UNSUPPORTED, "tensor too large");
        if (tokens == 0 && !conv_state_out) return ok();
        const void *req[] = {q_raw, k_raw, v_raw, conv_q, conv_k, conv_v, g_raw, beta_raw, q, k, v, g, beta};
        const char *names[] = {"q_raw", "k_raw", "v_raw", "conv_q", "conv_k", "conv_v", "g_raw", "beta_raw",
                               "q", "k", "v", "g", "beta"};
        for (int i = 0; i < 13 && tokens > 0; ++i)  // with no tokens only the state is touched
            if (!req[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
        const void *al16[] = {q_raw, k_raw, v_raw, g_raw, q, k, v, g, conv_state, conv_state_out, conv_q, conv_k, conv_v};
        const char *n16[] = {"q_raw", "k_raw", "v_raw", "g_raw", "q", "k", "v", "g", "conv_state", "conv_state_out",
                             "conv_q", "conv_k", "conv_v"};
        for (int i = 0; i < 13; ++i)
            if (!aligned(al16[i], 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n16[i]);
        const void *al4[] = {beta_raw, beta};
        for (int i = 0; i < 2; ++i)
            if (!aligned(al4[i], 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "a 4-byte argument is misaligned");
        const void *outs[] = {q, k, v, g, beta, conv_state_out};
        const void *ins[] = {q_raw, k_raw, v_raw, g_raw, beta_raw, conv_state, conv_q, conv_k, conv_v};
        for (const void *o : outs)
            for (const void *i : ins)
                if (o && o == i) return fail(KDA_ERR_INVALID_ARGUMENT, "an output aliases an input");
        if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens misaligned");
        const void *raw[3] = {q_raw, k_raw, v_raw};
        const float *w[3] = {conv_q, conv_k, conv_v};
        void *out[3] = {q, k, v};
        return hip_status(kda::launch_prologue(dtype_of(p->io_dtype), tokens, nseq, varlen ? 0 : p->seq_len, p->num_heads,
                                               p->head_dim_k, p->head_dim_v, p->conv_width,
                                               varlen ? cu_seqlens : nullptr, p->norm_eps, raw, w, g_raw, beta_raw,
                                               conv_state, conv_state_out, out, g, beta,
                                               static_cast<hipStream_t>(stream)),
                          "kda_prologue launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_prologue");
    }
}

kda_status_t kda_norm_gate(int64_t rows, int32_t d, int32_t io_dtype, float eps, const void *o,
                           const void *gate, const float *weight, void *out, void *stream) {
    try {
        if (rows < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "rows %lld < 0", (long long)rows);
        if (io_dtype != KDA_F32 && io_dtype != KDA_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "io_dtype %d is not KDA_F32 or KDA_BF16", (int)io_dtype);
        if (!supported_head_dim(d)) return fail(KDA_ERR_UNSUPPORTED, "d=%d: supported are 64 and 128", d);
        if (!std::isfinite(eps) || eps < 0.f) return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
        if (kda::norm_gate_blocks(dtype_of(io_dtype), rows, d) > 0x7fffffffLL) return fail(KDA_ERR_UNSUPPORTED, "too many rows");
        if (rows == 0) return ok();
        const void *req[] = {o, gate, weight, out};
        const char *names[] = {"o", "gate", "weight", "out"};
        for (int i = 0; i < 4; ++i) {
            if (!req[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
            if (!aligned(req[i], 16)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
        }
        if (out == gate || (const void *)weight == out || (const void *)weight == o || (const void *)weight == gate)
            return fail(KDA_ERR_INVALID_ARGUMENT, "out may alias o only");
        return hip_status(kda::launch_norm_gate(dtype_of(io_dtype), rows, d, eps, o, gate, weight, out,
                                                static_cast<hipStream_t>(stream)),
                          "kda_norm_gate launch");
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_norm_gate");
    }
}

kda_status_t kda_query(const kda_problem_t *problem, uint32_t flags, kda_query_result_t *res) {
    try {
        if (!res) return fail(KDA_ERR_INVALID_ARGUMENT, "result is NULL");
        std::memset(res, 0, sizeof *res);
        res->version = KDA_VERSION;
        res->peak_bf16_tflops = kPeakBf16Tflops;
        res->peak_hbm_gbps = kPeakHbmGBps;
        Resolved r;
        const bool varlen = problem && problem->num_seqs > 0;
        kda_status_t st = resolve(problem, varlen, r, true);
        if (st == KDA_OK) {
            const kda_problem_t &p = *problem;
            res->supported = 1;
            const bool two = r.two_pass_ok && p.algo != KDA_ALGO_FUSED;
            res->algo = two ? KDA_ALGO_TWO_PASS : KDA_ALGO_FUSED;
            res->workspace_bytes = two ? r.ws_bytes : 0;
            res->chunk_size = r.cfg.chunk;
            if (two) {  // the scan pass: one workgroup per (sequence, head, 16*spw*nw columns)
                res->dv_tile = 16 * r.spw * r.nw;
                int threads = 0, lds = 0;
                kda::split_scan_shape(dtype_of(p.io_dtype), p.head_dim_k, r.cfg.chunk, r.spw, r.nw, threads, lds);
                res->threads_per_block = threads;
                res->lds_bytes = lds;
                res->grid_blocks = (int64_t)r.num_seqs * p.num_heads * (p.head_dim_v / res->dv_tile);
            } else {
                res->dv_tile = r.cfg.dv_tile;
                res->threads_per_block = kda::kChunkThreads;
                res->lds_bytes = r.lds;
                res->grid_blocks = (int64_t)r.num_seqs * p.num_heads * (p.head_dim_v / r.cfg.dv_tile);
            }
            const double C = r.cfg.chunk, dk = p.head_dim_k, dv = p.head_dim_v;
            const double head_tokens = (double)r.tokens * p.num_heads;
            // per head-token, as computed chunk by chunk: A and P (C^2 dk each per chunk, triangular),
            // forward substitution (C^3/3), T applied to the residual and P D (C^2 dv each),
            // K~ S, Q~ S and K-^T D (2 C dk dv each)
            res->flops = head_tokens * (2.0 * C * (dk + dv) + C * C / 3.0 + 6.0 * dk * dv);
            const double s_io = p.io_dtype == KDA_BF16 ? 2.0 : 4.0;
            res->hbm_bytes = head_tokens * ((2.0 * dk + 2.0 * dv) * s_io + 4.0 * dk + 4.0) +
                             2.0 * 4.0 * dk * dv * (double)r.num_seqs * p.num_heads;
        } else if (st != KDA_ERR_UNSUPPORTED) {
            return st;
        }
        if (flags & KDA_QUERY_DEVICE) {
            int dev = 0;
            hipDeviceProp_t prop;
            if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess) {
                res->device_ok = 1;
                res->compute_units = prop.multiProcessorCount;
                std::snprintf(res->arch, sizeof res->arch, "%s", prop.gcnArchName);
            } else {
                (void)hipGetLastError();
            }
        }
        if (st == KDA_OK) return ok();
        return st;
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected exception in kda_query");
    }
}

const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
