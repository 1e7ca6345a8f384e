// Host-side checks of libkda's C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// around the library's host code (argument validation, sizing, error messages).  Every call here
// is refused by validation before any device work, or describes an empty problem that launches
// nothing, so the program needs no GPU and never reaches a kernel.  Host arrays (cu_seqlens_host)
// are allocated at their exact sizes so that a read past the end is reported.
//
// Exit status 0 when every expectation holds (and no sanitizer report aborted the run).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <memory>
#include <vector>

#include "kda.h"

namespace {

int g_failures = 0, g_checks = 0;

void expect(bool ok, const char *what, int line) {
    ++g_checks;
    if (!ok) {
        ++g_failures;
        std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, kda_last_error());
    }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

// Fake device addresses: aligned, never dereferenced on the host.
void *dev(uintptr_t i, uintptr_t misalign = 0) { return reinterpret_cast<void *>(0x100000 * (i + 1) + misalign); }
float *devf(uintptr_t i, uintptr_t misalign = 0) { return static_cast<float *>(dev(i, misalign)); }

kda_problem_t prefill() {
    kda_problem_t p;
    std::memset(&p, 0, sizeof p);
    p.batch = 4;
    p.seq_len = 4096;
    p.num_heads = 16;
    p.head_dim_k = 128;
    p.head_dim_v = 128;
    p.io_dtype = KDA_BF16;
    p.chunk_size = 64;
    p.scale = 1.f;
    return p;
}

// exact-size heap copy of cu_seqlens for the host
std::unique_ptr<int32_t[]> host_cu(const std::vector<int32_t> &v) {
    std::unique_ptr<int32_t[]> a(new int32_t[v.size()]);
    for (size_t i = 0; i < v.size(); ++i) a[i] = v[i];
    return a;
}

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // xorshift64*
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return g_rng * 0x2545F4914F6CDD1Dull;
}
template <typename T, size_t N>
T pick(const T (&a)[N]) {
    return a[next_u64() % N];
}

void status_strings() {
    for (int s = -2; s < 8; ++s) {
        const char *m = kda_status_string(static_cast<kda_status_t>(s));
        EXPECT(m != nullptr && std::strlen(m) > 0);
    }
}

void query_cases() {
    kda_query_result_t r;
    kda_problem_t p = prefill();
    EXPECT(kda_query(nullptr, 0, &r) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(std::strlen(kda_last_error()) > 0);
    EXPECT(kda_query(&p, 0, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_query(&p, 0, &r) == KDA_OK && r.supported == 1 && r.workspace_bytes > 0);
    p.chunk_size = 48;
    EXPECT(kda_query(&p, 0, &r) == KDA_ERR_UNSUPPORTED && r.supported == 0);
    p = prefill();
    p.head_dim_k = 96;
    EXPECT(kda_query(&p, 0, &r) == KDA_ERR_UNSUPPORTED);
    p = prefill();
    p.scale = std::numeric_limits<float>::quiet_NaN();
    EXPECT(kda_query(&p, 0, &r) == KDA_ERR_INVALID_ARGUMENT);
    p = prefill();
    p.batch = 2;
    p.num_seqs = 3;  // a packed batch needs batch == 1
    EXPECT(kda_query(&p, 0, &r) == KDA_ERR_INVALID_ARGUMENT);
    // sizes at the edges of int32 must be refused without overflowing the size arithmetic
    const int32_t big[] = {std::numeric_limits<int32_t>::max(), 1 << 30, 1 << 28, 1 << 20};
    for (int32_t b : big)
        for (int32_t t : big)
            for (int32_t h : big) {
                p = prefill();
                p.batch = b;
                p.seq_len = t;
                p.num_heads = h;
                const kda_status_t st = kda_query(&p, 0, &r);
                EXPECT(st == KDA_ERR_UNSUPPORTED || st == KDA_ERR_INVALID_ARGUMENT || st == KDA_OK);
                p.batch = 1;
                p.num_seqs = 0;
                EXPECT(kda_query(&p, 0, &r) != KDA_ERR_HIP);
                size_t n = 1;
                const kda_status_t sb = kda_chunk_bwd_workspace(&p, &n);
                EXPECT(sb != KDA_OK ? n == 0 : n > 0);
            }
}

// Random problems from edge values: every call returns one of the documented statuses, and a
// supported problem reports a consistent configuration.
void fuzz_query(int iters) {
    const int32_t sizes[] = {std::numeric_limits<int32_t>::min(), -1, 0, 1, 2, 3, 15, 16, 17, 63, 64, 65, 100,
                             4096, 1 << 20, 1 << 28, std::numeric_limits<int32_t>::max()};
    const int32_t dims[] = {-64, 0, 1, 32, 64, 96, 128, 256};
    const int32_t chunks[] = {-16, 0, 8, 16, 32, 48, 64, 128};
    const int32_t tiles[] = {-32, 0, 16, 32, 64, 96, 128, 256};
    const int32_t dtypes[] = {-1, 0, 1, 2};
    const int32_t algos[] = {-1, 0, 1, 2, 3};
    const float scales[] = {0.f, 1.f, -2.5f, std::numeric_limits<float>::infinity(),
                            std::numeric_limits<float>::quiet_NaN()};
    for (int it = 0; it < iters; ++it) {
        kda_problem_t p;
        p.batch = pick(sizes);
        p.seq_len = pick(sizes);
        p.num_heads = pick(sizes);
        p.head_dim_k = pick(dims);
        p.head_dim_v = pick(dims);
        p.num_seqs = next_u64() % 2 ? pick(sizes) : 0;
        p.io_dtype = static_cast<kda_dtype_t>(pick(dtypes));
        p.chunk_size = pick(chunks);
        p.scale = pick(scales);
        p.dv_tile = pick(tiles);
        p.algo = pick(algos);
        kda_query_result_t r;
        const kda_status_t st = kda_query(&p, 0, &r);
        EXPECT(st == KDA_OK || st == KDA_ERR_INVALID_ARGUMENT || st == KDA_ERR_UNSUPPORTED);
        if (st == KDA_OK) {
            EXPECT(r.supported == 1 && r.grid_blocks >= 0 && r.flops >= 0.0 && r.hbm_bytes >= 0.0);
            EXPECT(r.chunk_size == 16 || r.chunk_size == 32 || r.chunk_size == 64);
            EXPECT(r.algo == KDA_ALGO_FUSED || r.algo == KDA_ALGO_TWO_PASS);
        }
        size_t n = 7;
        const kda_status_t sb = kda_chunk_bwd_workspace(&p, &n);
        EXPECT(sb == KDA_OK || sb == KDA_ERR_INVALID_ARGUMENT || sb == KDA_ERR_UNSUPPORTED);
        EXPECT(sb == KDA_OK || n == 0);
    }
}

void forward_validation() {
    kda_problem_t p = prefill();
    void *q = dev(0), *k = dev(1), *v = dev(2), *out = dev(5), *ws = dev(8);
    float *g = devf(3), *beta = devf(4), *s0 = devf(6), *sf = devf(7);
    const size_t ws_bytes = size_t(1) << 30;
    // one defect at a time
    EXPECT(kda_chunk_fwd(nullptr, q, k, v, g, beta, s0, nullptr, nullptr, out, sf, ws, ws_bytes, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_fwd(&p, nullptr, k, v, g, beta, s0, nullptr, nullptr, out, sf, ws, ws_bytes, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_fwd(&p, q, dev(1, 2), v, g, beta, s0, nullptr, nullptr, out, sf, ws, ws_bytes, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, devf(4, 2), s0, nullptr, nullptr, out, sf, ws, ws_bytes, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, q, sf, ws, ws_bytes, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);  // out aliases q
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, out, static_cast<float *>(out), ws, ws_bytes,
                         nullptr) == KDA_ERR_INVALID_ARGUMENT);  // final_state aliases out
    p.algo = KDA_ALGO_TWO_PASS;
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, out, sf, ws, 1024, nullptr) ==
           KDA_ERR_WORKSPACE);
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, out, sf, dev(8, 128), ws_bytes, nullptr) ==
           KDA_ERR_WORKSPACE);
    EXPECT(kda_chunk_fwd_noalloc(&p, q, k, v, g, beta, s0, nullptr, nullptr, out, sf, nullptr) == KDA_ERR_WORKSPACE);
    // cu_seqlens_host without cu_seqlens
    p = prefill();
    auto cu_ok = host_cu({0, 5, 9, 12});
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, nullptr, cu_ok.get(), out, sf, ws, ws_bytes, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    // packed batches with bad offsets (host copy at its exact size)
    p.batch = 1;
    p.seq_len = 12;
    p.num_seqs = 3;
    const int32_t *cu_dev = static_cast<const int32_t *>(dev(9));
    for (const std::vector<int32_t> &bad :
         {std::vector<int32_t>{1, 5, 9, 12}, std::vector<int32_t>{0, 9, 5, 12}, std::vector<int32_t>{0, 5, 9, 11},
          std::vector<int32_t>{0, 5, 9, 13}}) {
        auto h = host_cu(bad);
        EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, cu_dev, h.get(), out, sf, ws, ws_bytes, nullptr) ==
               KDA_ERR_INVALID_ARGUMENT);
        EXPECT(kda_chunk_fwd_noalloc(&p, q, k, v, g, beta, s0, cu_dev, h.get(), out, sf, nullptr) ==
               KDA_ERR_INVALID_ARGUMENT);
        EXPECT(kda_recurrent_fwd(&p, q, k, v, g, beta, s0, cu_dev, h.get(), out, sf, nullptr) ==
               KDA_ERR_INVALID_ARGUMENT);
    }
    EXPECT(kda_chunk_fwd(&p, q, k, v, g, beta, s0, static_cast<const int32_t *>(dev(9, 2)), nullptr, out, sf, ws,
                         ws_bytes, nullptr) == KDA_ERR_INVALID_ARGUMENT);  // misaligned cu_seqlens
    // empty problems launch nothing
    p = prefill();
    p.batch = 0;
    EXPECT(kda_chunk_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, 0, nullptr) == KDA_OK);
    EXPECT(kda_recurrent_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr) == KDA_OK);
    p.batch = 1;
    p.seq_len = 0;
    p.num_seqs = 0;
    auto cu0 = host_cu({0});
    EXPECT(kda_chunk_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, cu_dev, cu0.get(), nullptr, nullptr,
                         nullptr, 0, nullptr) == KDA_OK);
    // fused prologue: one defect per call
    {
        const float *tq = devf(10), *tk = devf(11), *tv = devf(12);
        kda_problem_t pp = prefill();
        EXPECT(kda_chunk_fwd_prologue(&pp, 5, 1e-6f, q, k, v, tq, tk, tv, g, beta, s0, nullptr, nullptr, out, sf, ws,
                                      ws_bytes, nullptr) == KDA_ERR_UNSUPPORTED);
        EXPECT(kda_chunk_fwd_prologue(&pp, 4, std::numeric_limits<float>::quiet_NaN(), q, k, v, tq, tk, tv, g, beta, s0,
                                      nullptr, nullptr, out, sf, ws, ws_bytes, nullptr) == KDA_ERR_INVALID_ARGUMENT);
        EXPECT(kda_chunk_fwd_prologue(&pp, 4, 1e-6f, q, k, v, nullptr, tk, tv, g, beta, s0, nullptr, nullptr, out, sf,
                                      ws, ws_bytes, nullptr) == KDA_ERR_INVALID_ARGUMENT);
        EXPECT(kda_chunk_fwd_prologue(&pp, 4, 1e-6f, q, k, v, tq, tk, tv, g, beta, s0, nullptr, nullptr, out, sf, ws,
                                      1024, nullptr) == KDA_ERR_WORKSPACE);
        pp.algo = KDA_ALGO_FUSED;
        EXPECT(kda_chunk_fwd_prologue(&pp, 4, 1e-6f, q, k, v, tq, tk, tv, g, beta, s0, nullptr, nullptr, out, sf, ws,
                                      ws_bytes, nullptr) == KDA_ERR_UNSUPPORTED);
        pp = prefill();
        pp.batch = 1;
        pp.seq_len = 12;
        pp.num_seqs = 3;
        auto badp = host_cu({0, 5, 13, 12});
        EXPECT(kda_chunk_fwd_prologue(&pp, 4, 1e-6f, q, k, v, tq, tk, tv, g, beta, s0, cu_dev, badp.get(), out, sf, ws,
                                      ws_bytes, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    }
    // tune: refused before any timing
    kda_query_result_t best;
    p = prefill();
    EXPECT(kda_tune(&p, q, k, v, g, beta, s0, nullptr, nullptr, out, sf, ws, ws_bytes, nullptr, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_tune(&p, q, k, v, g, beta, s0, nullptr, nullptr, out, s0, ws, ws_bytes, nullptr, &best) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_tune(&p, nullptr, k, v, g, beta, s0, nullptr, nullptr, out, sf, ws, ws_bytes, nullptr, &best) ==
           KDA_ERR_INVALID_ARGUMENT);
}

void backward_validation() {
    kda_problem_t p = prefill();
    void *q = dev(0), *k = dev(1), *v = dev(2), *d_out = dev(5), *ws = dev(20);
    float *g = devf(3), *beta = devf(4), *s0 = devf(6), *dsf = devf(7);
    void *dq = dev(10), *dk = dev(11), *dv = dev(12);
    float *dg = devf(13), *dbeta = devf(14), *ds0 = devf(15);
    size_t need = 0;
    EXPECT(kda_chunk_bwd_workspace(&p, &need) == KDA_OK && need > 0);
    EXPECT(kda_chunk_bwd_workspace(&p, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_bwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, d_out, dsf, nullptr, dk, dv, dg, dbeta, ds0, ws,
                         need, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_bwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, d_out, dsf, dq, dk, dv, dg, dbeta, ds0, ws,
                         need - 1, nullptr) == KDA_ERR_WORKSPACE);
    EXPECT(kda_chunk_bwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, d_out, dsf, dq, dq, dv, dg, dbeta, ds0, ws, need,
                         nullptr) == KDA_ERR_INVALID_ARGUMENT);  // dk aliases dq
    EXPECT(kda_chunk_bwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, d_out, dsf, dq, dk, dv, dg, dbeta,
                         devf(15, 4), ws, need, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    p.chunk_size = 48;
    EXPECT(kda_chunk_bwd(&p, q, k, v, g, beta, s0, nullptr, nullptr, d_out, dsf, dq, dk, dv, dg, dbeta, ds0, ws, need,
                         nullptr) == KDA_ERR_UNSUPPORTED);
    p = prefill();
    p.batch = 1;
    p.seq_len = 12;
    p.num_seqs = 3;
    auto bad = host_cu({0, 5, 4, 12});
    EXPECT(kda_chunk_bwd_workspace(&p, &need) == KDA_OK);
    EXPECT(kda_chunk_bwd(&p, q, k, v, g, beta, s0, static_cast<const int32_t *>(dev(9)), bad.get(), d_out, dsf, dq,
                         dk, dv, dg, dbeta, ds0, ws, need, nullptr) == KDA_ERR_INVALID_ARGUMENT);
}

void decode_and_epilogue_validation() {
    void *q = dev(0), *k = dev(1), *v = dev(2), *out = dev(5);
    float *g = devf(3), *beta = devf(4), *state = devf(6);
    EXPECT(kda_decode_step(-1, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, out, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step(256, 32, 96, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, out, nullptr) ==
           KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step(256, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, nullptr, out, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step(256, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, dev(5, 8), nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step(256, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, state, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step(std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::max(), 128, 128,
                           KDA_BF16, 1.f, q, k, v, g, beta, state, out, nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step(0, 32, 128, 128, KDA_BF16, 1.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr) == KDA_OK);
    void *gate = dev(7);
    float *w = devf(8);
    EXPECT(kda_decode_step_gated(256, 32, 128, 128, 7, 1.f, q, k, v, g, beta, state, gate, w, 1e-6f, out, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step_gated(256, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, gate, w,
                                 std::numeric_limits<float>::infinity(), out, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step_gated(256, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, nullptr, w, 1e-6f, out,
                                 nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step_gated(256, 32, 128, 128, KDA_BF16, 1.f, q, k, v, g, beta, state, gate, w, 1e-6f, gate,
                                 nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step_gated(std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::max(), 128, 128,
                                 KDA_BF16, 1.f, q, k, v, g, beta, state, gate, w, 1e-6f, out, nullptr) ==
           KDA_ERR_UNSUPPORTED);
    EXPECT(kda_decode_step_gated(0, 32, 128, 128, KDA_BF16, 1.f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, 0.f, nullptr, nullptr) == KDA_OK);
    EXPECT(kda_norm_gate(-1, 128, KDA_BF16, 1e-6f, q, k, g, out, nullptr) == KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_norm_gate(10, 96, KDA_BF16, 1e-6f, q, k, g, out, nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_norm_gate(10, 128, KDA_BF16, std::numeric_limits<float>::quiet_NaN(), q, k, g, out, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_norm_gate(10, 128, KDA_BF16, 1e-6f, q, k, g, k, nullptr) == KDA_ERR_INVALID_ARGUMENT);  // out = gate
    EXPECT(kda_norm_gate(std::numeric_limits<int64_t>::max(), 128, KDA_BF16, 1e-6f, q, k, g, out, nullptr) ==
           KDA_ERR_UNSUPPORTED);
    EXPECT(kda_norm_gate(0, 128, KDA_BF16, 1e-6f, nullptr, nullptr, nullptr, nullptr, nullptr) == KDA_OK);

    kda_prologue_t pr;
    std::memset(&pr, 0, sizeof pr);
    pr.batch = 2;
    pr.seq_len = 100;
    pr.num_heads = 4;
    pr.head_dim_k = 128;
    pr.head_dim_v = 128;
    pr.conv_width = 4;
    pr.io_dtype = KDA_BF16;
    pr.norm_eps = 1e-6f;
    const void *raw[3] = {dev(0), dev(1), dev(2)};
    const float *taps[3] = {devf(3), devf(4), devf(5)};
    EXPECT(kda_prologue(nullptr, raw[0], raw[1], raw[2], taps[0], taps[1], taps[2], devf(6), devf(7), nullptr, nullptr,
                        nullptr, dev(8), dev(9), dev(10), devf(11), devf(12), nullptr) == KDA_ERR_INVALID_ARGUMENT);
    pr.conv_width = 5;
    EXPECT(kda_prologue(&pr, raw[0], raw[1], raw[2], taps[0], taps[1], taps[2], devf(6), devf(7), nullptr, nullptr,
                        nullptr, dev(8), dev(9), dev(10), devf(11), devf(12), nullptr) == KDA_ERR_UNSUPPORTED);
    pr.conv_width = 4;
    pr.norm_eps = -1.f;
    EXPECT(kda_prologue(&pr, raw[0], raw[1], raw[2], taps[0], taps[1], taps[2], devf(6), devf(7), nullptr, nullptr,
                        nullptr, dev(8), dev(9), dev(10), devf(11), devf(12), nullptr) == KDA_ERR_INVALID_ARGUMENT);
    pr.norm_eps = 1e-6f;
    EXPECT(kda_prologue(&pr, raw[0], raw[1], raw[2], taps[0], taps[1], taps[2], devf(6), devf(7), nullptr, nullptr,
                        nullptr, dev(0), dev(9), dev(10), devf(11), devf(12), nullptr) == KDA_ERR_INVALID_ARGUMENT);
    pr.num_seqs = 2;  // packed without cu_seqlens
    EXPECT(kda_prologue(&pr, raw[0], raw[1], raw[2], taps[0], taps[1], taps[2], devf(6), devf(7), nullptr, nullptr,
                        nullptr, dev(8), dev(9), dev(10), devf(11), devf(12), nullptr) == KDA_ERR_INVALID_ARGUMENT);

    kda_problem_t p = prefill();
    p.chunk_size = 48;
    EXPECT(kda_dplr_chunk_fwd(&p, q, k, v, dev(20), dev(21), g, nullptr, nullptr, nullptr, out, nullptr, nullptr) ==
           KDA_ERR_UNSUPPORTED);
    p = prefill();
    EXPECT(kda_dplr_chunk_fwd(&p, q, k, v, nullptr, dev(21), g, nullptr, nullptr, nullptr, out, nullptr, nullptr) ==
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_dplr_chunk_fwd(&p, q, k, v, dev(20), dev(21), g, nullptr, nullptr, nullptr, dev(20), nullptr,
                              nullptr) == KDA_ERR_INVALID_ARGUMENT);
}

}  // namespace

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
    status_strings();
    query_cases();
    fuzz_query(iters);
    forward_validation();
    backward_validation();
    decode_and_epilogue_validation();
    std::printf("%d checks, %d failed\n", g_checks, g_failures);
    return g_failures ? 1 : 0;
}
