/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).
 *
 * The operator (Kimi Linear summary page, sections "Kimi Delta Attention:
 * fine-grained memory control" and "From linear attention to Gated DeltaNet"):
 * per sequence and head, an fp32 state S (d_k x d_v) is decayed per channel and
 * corrected by a rank-1 delta-rule update for every token t,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with a per-channel natural-log gate g_t (d_k values, exp(g_t) in (0, 1]) and a
 * per-head scalar beta_t.  The chunked entry point evaluates the same function
 * chunk by chunk ("Chunkwise parallel algorithm" section): inside a chunk the
 * rank-1 updates are packed with a WY/UT representation whose lower-triangular
 * inverse comes from forward substitution, the state is passed from chunk to
 * chunk, and the output merges the inter-chunk and intra-chunk parts.
 *
 * Conventions shared by every entry point
 *  - All pointers are device pointers unless the name ends in _host.  The caller
 *    owns every buffer; the library never frees or keeps a pointer after a call.
 *  - Tensors are dense, row-major, 16-byte aligned:
 *        q, k  [tokens, H, d_k]   io dtype (fp32 or bf16)
 *        v     [tokens, H, d_v]   io dtype
 *        g     [tokens, H, d_k]   fp32 natural-log gate (alpha = exp(g))
 *        beta  [tokens, H]        fp32
 *        out   [tokens, H, d_v]   io dtype
 *        state [num_seqs, H, d_k, d_v] fp32
 *    where "tokens" is B*T for a batch (sequence b owns tokens [b*T, (b+1)*T)) or the
 *    packed token count when cu_seqlens is given.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    queued asynchronously on it; no entry point synchronises.
 *  - On invalid arguments an entry point returns a status, launches nothing and
 *    records a message readable with kda_last_error() (thread-local).  Launch
 *    failures return KDA_ERR_HIP.  Nothing aborts and no C++ exception crosses
 *    the ABI.
 *  - q and k are expected to be L2-normalised over d_k (the model does so for
 *    eigenvalue stability, "Kimi Linear model composition" section); this is not
 *    checked.  NaN or Inf inputs give undefined results.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION 100 /* 1.0.0 */

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, negative or inconsistent size */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head dim, chunk size, dtype) */
    KDA_ERR_WORKSPACE = 3,        /* workspace smaller than kda_query reports */
    KDA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} kda_status_t;

/* Element types.  Structs and parameters carry them as int32_t (any value can cross the ABI;
 * values other than these are refused with KDA_ERR_INVALID_ARGUMENT). */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype_t;

/* How kda_chunk_fwd evaluates the chunks.
 *  KDA_ALGO_FUSED:    one kernel; each workgroup walks its sequence chunk by chunk and
 *                     does all per-chunk work itself (no workspace).
 *  KDA_ALGO_TWO_PASS: a parallel pass over all chunks computes the state-independent
 *                     chunk operands (gated keys/queries, the UT transform, P) into the
 *                     workspace, then a scan pass carries the state through the chunks.
 *  KDA_ALGO_AUTO:     two-pass when the workspace is large enough (kda_query reports the
 *                     size) and the problem is supported by it, else fused. */
typedef enum { KDA_ALGO_AUTO = 0, KDA_ALGO_FUSED = 1, KDA_ALGO_TWO_PASS = 2 } kda_algo_t;

/* Problem description shared by kda_chunk_fwd, kda_recurrent_fwd and kda_query. */
typedef struct {
    int32_t batch;       /* B: number of sequences of seq_len tokens; must be 1 with cu_seqlens */
    int32_t seq_len;     /* T per sequence, or the total packed token count with cu_seqlens (>= 0) */
    int32_t num_heads;   /* H >= 1 */
    int32_t head_dim_k;  /* d_k in {64, 128} */
    int32_t head_dim_v;  /* d_v in {64, 128} */
    int32_t num_seqs;    /* with cu_seqlens: number of sequences (cu_seqlens has num_seqs+1 entries); else ignored */
    int32_t io_dtype;    /* kda_dtype_t: dtype of q, k, v and out; g, beta and the state are always fp32 */
    int32_t chunk_size;  /* 16, 32 or 64; 0 = library default (32 for the forward, the largest
                            compiled chunk, 64, for kda_chunk_bwd) */
    float scale;         /* multiplies the output (1.0 for o_t = S_t^T q_t) */
    int32_t dv_tile;     /* state columns per workgroup: 0 = library choice; fused: 32, 64 or 128;
                            two-pass: 16, 32 or 64 */
    int32_t algo;        /* kda_algo_t */
} kda_problem_t;

/*
 * kda_chunk_fwd -- chunkwise KDA forward (prefill).
 * Kimi Linear summary page, "Chunkwise parallel algorithm" and "Less compute than
 * general DPLR" sections.
 *
 *  initial_state   [num_seqs, H, d_k, d_v] fp32, or NULL for a zero initial state.
 *  cu_seqlens      int32 [num_seqs+1] device offsets of a packed batch (cu[0] = 0,
 *                  non-decreasing, cu[num_seqs] = seq_len), or NULL for a plain batch.
 *                  Chunks restart at every sequence start and never cross a boundary;
 *                  a zero-length sequence passes its initial state through.  The
 *                  two-pass algorithm ranks the sequences on the device by chunk count
 *                  and starts the state scans of the longest ones first (the fused
 *                  algorithm, which has no workspace for the ranking, runs them in
 *                  batch order).
 *  cu_seqlens_host optional host copy of cu_seqlens: when given, its contents are
 *                  validated (otherwise they are a precondition).
 *  out             [tokens, H, d_v] io dtype (written).
 *  final_state     [num_seqs, H, d_k, d_v] fp32, or NULL to skip writing it.  It may be
 *                  the same pointer as initial_state (in-place state cache); no other
 *                  aliasing between arguments is allowed.
 *  workspace       device scratch for the two-pass algorithm, at least
 *                  kda_query().workspace_bytes bytes (256-byte aligned); its contents on
 *                  entry are ignored and on return unspecified.  With KDA_ALGO_AUTO a
 *                  smaller (or NULL) workspace selects the fused algorithm; with
 *                  KDA_ALGO_TWO_PASS it is an error (KDA_ERR_WORKSPACE).
 */
kda_status_t kda_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *initial_state,
                           const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                           float *final_state, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_recurrent_fwd -- the same function evaluated token by token on the GPU
 * (reference mode: no chunking, fp32 arithmetic throughout).  Kimi Linear summary page,
 * "Kimi Delta Attention: fine-grained memory control" section (the per-token recurrence with
 * a per-channel decay and the delta-rule correction) and "From linear attention to Gated
 * DeltaNet" (the rank-1 update read as one step of online gradient descent).  This is the
 * definition the chunked form re-associates exactly, evaluated without chunking: a GPU
 * second opinion for kda_chunk_fwd and the path for very short sequences.
 * Arguments, layouts, ownership and errors as for kda_chunk_fwd; problem->chunk_size,
 * dv_tile and algo are ignored and no workspace is used.
 */
kda_status_t kda_recurrent_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *initial_state,
                               const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                               float *final_state, void *stream);

/*
 * kda_chunk_fwd_prologue -- kda_chunk_fwd (two-pass algorithm) on the raw projections, with the
 * prologue of kda_prologue applied inside the kernels as they read their inputs (summary page,
 * "Kimi Linear model composition"; readings as for kda_prologue): q, k and v pass the causal
 * depthwise convolution of conv_width taps and Swish, q and k the L2 normalisation with
 * norm_eps, g = -softplus(g_raw), beta = sigmoid(beta_raw).  The convolution sees zeros before
 * every sequence's first token (use kda_prologue, then kda_chunk_fwd, to carry a convolution
 * state across calls).  The normalised q, k, v, g and beta are not written anywhere.
 *
 *  problem, initial_state, cu_seqlens, cu_seqlens_host, out, final_state, workspace, stream:
 *                  as for kda_chunk_fwd; problem->algo must not be KDA_ALGO_FUSED, and the
 *                  workspace is required (kda_query with KDA_ALGO_TWO_PASS reports its size).
 *  q_raw, k_raw    [tokens, H, d_k] io dtype;  v_raw [tokens, H, d_v] io dtype
 *  conv_q, conv_k  [H, d_k, conv_width] fp32;  conv_v [H, d_v, conv_width] fp32 (tap
 *                  conv_width - 1 on the current token), 4-byte aligned
 *  g_raw           [tokens, H, d_k] fp32;  beta_raw [tokens, H] fp32
 *  conv_width      1..4 (KDA_ERR_UNSUPPORTED otherwise);  norm_eps >= 0 and finite.
 * Errors as for kda_chunk_fwd; KDA_ERR_UNSUPPORTED also where the two-pass algorithm has no
 * variant for the problem.
 */
kda_status_t kda_chunk_fwd_prologue(const kda_problem_t *problem, int32_t conv_width, float norm_eps,
                                    const void *q_raw, const void *k_raw, const void *v_raw, const float *conv_q,
                                    const float *conv_k, const float *conv_v, const float *g_raw,
                                    const float *beta_raw, const float *initial_state, const int32_t *cu_seqlens,
                                    const int32_t *cu_seqlens_host, void *out, float *final_state, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * kda_chunk_bwd -- gradients of the chunkwise forward (training).
 * Kimi Linear summary page, "Chunkwise parallel algorithm" section: the WY/UT chunk form
 * is what makes the operator trainable at matrix-core speed; the gradients are the
 * reverse-mode derivative of the same chunk equations (one triangular inverse per chunk,
 * reused for its transpose), exact up to rounding.
 *
 * For the loss L = sum(d_out * out) + sum(d_final_state * final_state) of the forward with
 * the same arguments, writes dq, dk, dv, dg, dbeta and (optionally) d_initial_state.
 *  problem, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host
 *                  as for kda_chunk_fwd (the forward is recomputed; out is not needed;
 *                  the forward and reverse state scans of a packed batch run the
 *                  longest sequences first).
 *                  problem->chunk_size: 16, 32 or 64 (0 = default); problem->algo and
 *                  dv_tile are ignored.
 *  d_out           [tokens, H, d_v] io dtype: gradient of out.
 *  d_final_state   [num_seqs, H, d_k, d_v] fp32, or NULL for zero.
 *  dq, dk          [tokens, H, d_k] io dtype (written).
 *  dv              [tokens, H, d_v] io dtype (written).
 *  dg              [tokens, H, d_k] fp32 (written): gradient of the log-gate g.
 *  dbeta           [tokens, H] fp32 (written).
 *  d_initial_state [num_seqs, H, d_k, d_v] fp32, or NULL to skip it.
 *  workspace       device scratch of at least kda_chunk_bwd_workspace() bytes, 256-byte
 *                  aligned (chunk states, their gradients, two per-chunk d_v tiles and
 *                  one record of per-chunk operands for the reverse scan);
 *                  contents on entry ignored, on return unspecified.  Required.
 * No output may alias an input or another output.  Status and error behaviour as for
 * kda_chunk_fwd; KDA_ERR_UNSUPPORTED for a head dimension or chunk size without a compiled
 * variant.
 */
kda_status_t kda_chunk_bwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *initial_state,
                           const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, const void *d_out,
                           const float *d_final_state, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                           float *d_initial_state, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_dplr_chunk_fwd -- the general DPLR recurrence that KDA specialises, evaluated with the
 * same chunked single-pass kernel design as KDA's fused forward; a comparator for the
 * operator-speed claim of the Kimi Linear summary page ("Less compute than general DPLR"
 * section: KDA ties both low-rank vectors of the transition to the key, which leaves two
 * C x C chunk matrices instead of four and three fewer matrix products).
 *
 *     S_t = (Diag(exp(g_t)) + a_t b_t^T) S_{t-1} + k_t v_t^T,     o_t = scale * S_t^T q_t
 *
 *  a, b            [tokens, H, d_k] io dtype (the two low-rank vectors); k is the write key.
 *  Everything else as kda_chunk_fwd (no beta: KDA's beta is folded into a and k).
 *  problem->chunk_size: 16, 32 or 64 (0 = 64); problem->dv_tile: 32 or 64 (0 = 32);
 *  problem->algo is ignored.  Needs no workspace.
 * KDA is the case a = -beta k, b = exp(g) * k with write key beta k.
 */
kda_status_t kda_dplr_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                                const void *a, const void *b, const float *g, const float *initial_state,
                                const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                                float *final_state, void *stream);

/*
 * kda_chunk_bwd_workspace -- workspace bytes kda_chunk_bwd needs for `problem` (packed
 * batch when problem->num_seqs > 0, as in kda_query).  Writes *bytes; returns
 * KDA_ERR_UNSUPPORTED (and *bytes = 0) for problems kda_chunk_bwd does not support.
 */
kda_status_t kda_chunk_bwd_workspace(const kda_problem_t *problem, size_t *bytes);

/*
 * kda_decode_step -- one token for each of num_seqs independent sequences, updating
 * the per-sequence state in place (the fixed-size state slot that replaces a growing
 * KV cache; "Kimi Delta Attention" and evaluation sections of the summary page).
 *
 *  q, k, g [num_seqs, H, d_k]; v [num_seqs, H, d_v]; beta [num_seqs, H];
 *  state [num_seqs, H, d_k, d_v] fp32, read and overwritten; out [num_seqs, H, d_v].
 */
kda_status_t kda_decode_step(int32_t num_seqs, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                             int32_t io_dtype, float scale, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, float *state, void *out, void *stream);

/*
 * kda_decode_step_gated -- kda_decode_step with the output epilogue applied in the same pass:
 * the per-token update of the summary page's "Kimi Delta Attention" section, then the per-head
 * RMSNorm and output gate of its "Kimi Linear model composition" section (no formula on the
 * page; the reading, as for kda_norm_gate):
 *
 *     o   = scale S_t^T q_t                                   (one head, d_v values)
 *     out = o / sqrt(mean_j o_j^2 + eps) * weight * sigmoid(gate)
 *
 *  q, k, g, v, beta, state as for kda_decode_step (state updated in place);
 *  gate    [num_seqs, H, d_v] io dtype: the gate pre-activation of this token;
 *  weight  [d_v] fp32, shared by the heads;  eps >= 0 and finite;
 *  out     [num_seqs, H, d_v] io dtype: the gated, normalised output (o itself is not written).
 *  Pointers are device memory, 16-byte aligned (beta 4-byte); state and out alias nothing.
 *  One workgroup per (sequence, head) holds the whole state row block, so the norm needs no
 *  second pass over o.  Errors as for kda_decode_step; num_seqs == 0 launches nothing.
 */
kda_status_t kda_decode_step_gated(int32_t num_seqs, int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                                   int32_t io_dtype, float scale, const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, float *state, const void *gate,
                                   const float *weight, float eps, void *out, void *stream);

/* Shape of a kda_prologue call (same batch / packed conventions as kda_problem_t). */
typedef struct {
    int32_t batch;       /* B; must be 1 when num_seqs > 0 */
    int32_t seq_len;     /* tokens per sequence, or the packed token count when num_seqs > 0 */
    int32_t num_seqs;    /* 0: B sequences of seq_len tokens; > 0: packed by cu_seqlens */
    int32_t num_heads;   /* H */
    int32_t head_dim_k;  /* 64 or 128 */
    int32_t head_dim_v;  /* 64 or 128 */
    int32_t conv_width;  /* W, taps of the short convolution: 1..4 */
    int32_t io_dtype;    /* kda_dtype_t: raw q/k/v, outputs q/k/v and the convolution state */
    float norm_eps;      /* >= 0: q and k are divided by sqrt(sum x^2 + norm_eps) */
} kda_prologue_t;

/*
 * kda_prologue -- the steps before the operator ("Kimi Linear model composition" section of
 * the summary page: query, key and value pass a short convolution and Swish, query and key an
 * L2 normalisation, and the decay gate a GDN / Mamba-like decay function; the page gives no
 * formulas, these are the readings used):
 *
 *   c_t = sum_{i<W} w[i] x_{t-W+1+i}     causal depthwise convolution over time per channel
 *   y   = c sigmoid(c)                   Swish
 *   q, k = y / sqrt(sum_d y^2 + eps);  v = y
 *   g = -softplus(g_raw);  beta = sigmoid(beta_raw)
 *
 *  q_raw, k_raw [tokens, H, d_k], v_raw [tokens, H, d_v]   io_dtype
 *  conv_q, conv_k [H, d_k, W], conv_v [H, d_v, W]          fp32 filter taps (tap W-1 = current token)
 *  g_raw [tokens, H, d_k], beta_raw [tokens, H]            fp32
 *  cu_seqlens  int32 [num_seqs + 1] device (when num_seqs > 0), as for kda_chunk_fwd
 *  conv_state  [S, W-1, H, 2 d_k + d_v] io_dtype or NULL: the raw q | k | v inputs of the W-1
 *              tokens before each of the S sequences (NULL = zeros); conv_state_out, same
 *              shape or NULL, receives the last W-1 raw inputs of each sequence (so a sequence
 *              can be continued, one token at a time in decoding)
 *  q, k, v     outputs, shapes of the raw inputs, io_dtype; g, beta fp32
 *  Tensors 16-byte aligned (beta_raw and beta 4-byte); no output may alias an input,
 *  and conv_state_out must not be conv_state.  Errors as for kda_chunk_fwd.
 */
kda_status_t kda_prologue(const kda_prologue_t *problem, const void *q_raw, const void *k_raw, const void *v_raw,
                          const float *conv_q, const float *conv_k, const float *conv_v, const float *g_raw,
                          const float *beta_raw, const int32_t *cu_seqlens, const void *conv_state,
                          void *conv_state_out, void *q, void *k, void *v, float *g, float *beta, void *stream);

/*
 * kda_norm_gate -- output epilogue: per-head RMSNorm followed by the data-dependent output
 * gate, applied before the output projection ("Kimi Linear model composition" section of
 * the summary page; the page gives no formula, this is the reading used): for each of
 * `rows` rows of d values (one token and head),
 *
 *     out[r, :] = o[r, :] / sqrt(mean_j o[r, j]^2 + eps) * weight[:] * sigmoid(gate[r, :])
 *
 *  o, gate, out  [rows, d], io_dtype (bf16 results rounded to nearest even), row-major;
 *  weight        [d] fp32, shared by all heads; gate is the pre-activation (the low-rank
 *                projection that produces it is outside this operator).
 *  d is 64 or 128; eps >= 0 and finite.  out may be o itself (in place); no other aliasing.
 *  All pointers device memory, 16-byte aligned; nothing is allocated or retained.
 *  Errors: KDA_ERR_INVALID_ARGUMENT (sizes, eps, NULL or misaligned pointers, aliasing),
 *  KDA_ERR_UNSUPPORTED (d), KDA_ERR_HIP (launch).  rows == 0 launches nothing.
 */
kda_status_t kda_norm_gate(int64_t rows, int32_t d, int32_t io_dtype, float eps, const void *o,
                           const void *gate, const float *weight, void *out, void *stream);

/* Result of kda_query. */
typedef struct {
    int32_t version;           /* KDA_VERSION of the library */
    int32_t supported;         /* 1 if kda_chunk_fwd accepts the problem */
    int32_t algo;              /* algorithm used when the reported workspace is supplied */
    size_t workspace_bytes;    /* scratch the two-pass algorithm needs (0 if it is not used) */
    int32_t chunk_size;        /* chunk the forward will use */
    int32_t dv_tile;           /* state columns owned by one workgroup */
    int32_t threads_per_block; /* workgroup size */
    int32_t lds_bytes;         /* LDS per workgroup */
    int64_t grid_blocks;       /* workgroups launched */
    double flops;              /* algorithmic flops of the call (triangular parts only) */
    double hbm_bytes;          /* algorithmic HBM bytes: inputs + outputs + state in/out once */
    int32_t device_ok;         /* 1 if a device was queried (the fields below are valid) */
    int32_t compute_units;     /* of the current device */
    char arch[64];             /* gcnArchName of the current device */
    double peak_bf16_tflops;   /* published dense bf16 matrix peak used for roofline fractions */
    double peak_hbm_gbps;      /* published HBM peak */
    double tuned_ms;           /* kda_tune: measured time of one call with this configuration (0 otherwise) */
} kda_query_result_t;

#define KDA_QUERY_DEVICE 1u /* also fill the device fields (one HIP property query, no launch) */

/*
 * kda_query -- tuning/query entry point: reports how kda_chunk_fwd will run the
 * problem (chunk, tile, grid, LDS, workspace), its algorithmic flops and bytes, and
 * optionally the current device.  Kimi Linear summary page, "Chunkwise parallel algorithm"
 * section: the chunk length is a free parameter of the chunked evaluation (the result does
 * not depend on it, only the speed), and the intra-chunk work is matrix products sized by it;
 * this call reports the choice and the work it implies.  Launches nothing and allocates
 * nothing.  A problem with num_seqs > 0 describes a packed batch (batch must be 1, seq_len is
 * the token count); set num_seqs = 0 to describe a plain batch of `batch` sequences.
 * Returns KDA_OK (result filled, supported = 1), KDA_ERR_UNSUPPORTED (result->supported = 0;
 * the version, peaks and, with KDA_QUERY_DEVICE, the device fields are still filled) or
 * KDA_ERR_INVALID_ARGUMENT (NULL result or an invalid problem).
 */
kda_status_t kda_query(const kda_problem_t *problem, uint32_t flags, kda_query_result_t *result);

/*
 * kda_tune -- autotuning: runs kda_chunk_fwd on the caller's own tensors with every supported
 * candidate configuration (chunk size 16 / 32 / 64, d_v tile, fused or two-pass algorithm;
 * problem fields that are set are kept fixed), times each with HIP events on `stream`
 * (one warm-up call, then three timed calls), synchronises, and reports the fastest one in
 * *best as kda_query would for it, with tuned_ms set.  The outputs are overwritten by the
 * candidate runs (the last run leaves the result of the last candidate); initial_state must
 * not alias final_state.  Two-pass candidates need a workspace as large as kda_query reports
 * for them; smaller ones are skipped.  Nothing is allocated.  Same arguments and errors as
 * kda_chunk_fwd, plus KDA_ERR_UNSUPPORTED when no candidate runs.
 */
kda_status_t kda_tune(const kda_problem_t *problem, const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                      const int32_t *cu_seqlens_host, void *out, float *final_state, void *workspace,
                      size_t workspace_bytes, void *stream, kda_query_result_t *best);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd (two-pass algorithm) for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The chunk-offset table and per-chunk records live in a fixed array of the library on
 * each device (kda_noalloc_scratch_bytes(), 64 MiB, held until the process ends); nothing is
 * allocated or freed.  Arguments, layouts and errors as for kda_chunk_fwd, without the workspace;
 * problem->algo is ignored (always two-pass).  A problem whose workspace (kda_query with
 * KDA_ALGO_TWO_PASS) exceeds the array returns KDA_ERR_WORKSPACE before touching the device
 * (64 MiB holds, for instance, 4,096 tokens x 16 heads at d = 128, chunk 64).  All calls on one
 * device share its array: calls that overlap on a device (concurrent streams, threads) race and
 * must be ordered by the caller.
 */
kda_status_t kda_chunk_fwd_noalloc(const kda_problem_t *problem, const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, const float *initial_state,
                                   const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, void *out,
                                   float *final_state, void *stream);

/* Bytes of the fixed scratch array kda_chunk_fwd_noalloc uses on each device. */
size_t kda_noalloc_scratch_bytes(void);

/* Static description of a status code. */
const char *kda_status_string(kda_status_t status);

/* Message of the last failing call on this thread ("" if none). */
const char *kda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
