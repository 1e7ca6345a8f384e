/*
 * KDA oracle: plain, slow, fp64 CPU implementation of Kimi Delta Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library and includes nothing from it.
 *
 * What it computes (one independent run per sequence n and head h):
 *
 *   S_0   = initial state (d_k x d_v) or zeros
 *   for every token t of the sequence, in order:
 *     alpha_t = exp(g_t)                               per-channel forget gate
 *     S'      = Diag(alpha_t) S_{t-1}                  decay, one rate per d_k row
 *     p       = S'^T k_t                               what the memory returns for k_t
 *     S_t     = S' + beta_t k_t (v_t - p)^T            delta-rule rank-1 correction
 *     o_t     = scale * S_t^T q_t                      read-out with the updated state
 *
 * which equals S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
 *
 * Sources (Kimi Linear summary page):
 *   - "Kimi Delta Attention: fine-grained memory control" section: the head-wise
 *     forget gate of Gated DeltaNet becomes a per-channel (diagonal) gate, and
 *     the transition stays a delta-rule (specialised DPLR) matrix.
 *   - "From linear attention to Gated DeltaNet" section: the delta rule is online
 *     gradient descent on a reconstruction loss (so the memory maps a key back to
 *     its value) and the scalar gate acts like weight decay on the fast weight.
 *   The exact update order (decay, then the delta correction against the decayed
 *   state; output read after the update) is the reading written above; the pages
 *   print no formula.
 *
 * Inputs stream from their stored dtype (fp32, or bf16 given as raw uint16
 * bits); every arithmetic step runs in double with libm exp.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef KDA_ORACLE_MUTANT
#define KDA_ORACLE_MUTANT 0 /* tests rebuild with planted mistakes (1..N) to check the pins */
#endif

static double from_bf16(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    int64_t num_seqs;
    const int64_t *starts; /* first token of each sequence in the flattened token axis */
    const int64_t *lens;   /* number of tokens of each sequence */
    int H, dk, dv, io_bf16;
    double scale;
    const void *q, *k, *v;
    const float *g, *beta, *s0; /* s0: [num_seqs, H, dk, dv] or NULL (zeros) */
    int nsel;
    const int32_t *heads; /* heads to compute (nsel entries), or NULL for all */
    double *o;            /* [total_tokens, nsel, dv] */
    double *s_final;      /* [num_seqs, nsel, dk, dv] or NULL */
    int64_t next_unit;
    pthread_mutex_t lock;
} job_t;

static double load_io(const void *base, int io_bf16, int64_t idx) {
    if (io_bf16) return from_bf16(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

static void run_unit(job_t *J, int64_t unit, double *S, double *qv, double *kv, double *vv,
                     double *a, double *p) {
    const int64_t n = unit / J->nsel;
    const int hs = (int)(unit % J->nsel);
    const int h = J->heads ? J->heads[hs] : hs;
    const int H = J->H, dk = J->dk, dv = J->dv;

    if (J->s0) {
        const float *src = J->s0 + ((n * H + h) * (int64_t)dk) * dv;
        for (int64_t e = 0; e < (int64_t)dk * dv; ++e) S[e] = (double)src[e];
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    }

    const int64_t t0 = J->starts[n], len = J->lens[n];
    for (int64_t t = t0; t < t0 + len; ++t) {
        const int64_t row_k = (t * H + h) * (int64_t)dk;
        const int64_t row_v = (t * H + h) * (int64_t)dv;
        for (int i = 0; i < dk; ++i) {
            qv[i] = load_io(J->q, J->io_bf16, row_k + i);
            kv[i] = load_io(J->k, J->io_bf16, row_k + i);
            a[i] = exp((double)J->g[row_k + i]);
        }
        for (int j = 0; j < dv; ++j) vv[j] = load_io(J->v, J->io_bf16, row_v + j);
        const double b = (double)J->beta[t * H + h];

#if KDA_ORACLE_MUTANT == 1 /* planted: delta correction against the undecayed state */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += S[(int64_t)i * dv + j] * kv[i];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= a[i];
#else
        /* S' = Diag(alpha) S */
        for (int i = 0; i < dk; ++i) {
#if KDA_ORACLE_MUTANT == 2 /* planted: gate applied along d_v (columns) instead of d_k rows */
            for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= a[j % dk];
#else
            for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= a[i];
#endif
        }
        /* p = S'^T k */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += S[(int64_t)i * dv + j] * kv[i];
#endif

#if KDA_ORACLE_MUTANT == 4 /* planted: output read before the update */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * qv[i];
            J->o[(t * J->nsel + hs) * (int64_t)dv + j] = J->scale * acc;
        }
#endif
        /* S = S' + beta k (v - p)^T */
        for (int i = 0; i < dk; ++i) {
#if KDA_ORACLE_MUTANT == 3 /* planted: sign error in the correction */
            const double bk = -b * kv[i];
#else
            const double bk = b * kv[i];
#endif
            for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += bk * (vv[j] - p[j]);
        }
#if KDA_ORACLE_MUTANT != 4
        /* o = scale * S^T q */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
#if KDA_ORACLE_MUTANT == 5 /* planted: transposed read-out (S q instead of S^T q) */
            for (int i = 0; i < dk; ++i) acc += S[(int64_t)j * dv + i] * qv[i];
#else
            for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * qv[i];
#endif
            J->o[(t * J->nsel + hs) * (int64_t)dv + j] = J->scale * acc;
        }
#endif
    }
    if (J->s_final) {
        double *dst = J->s_final + ((n * J->nsel + hs) * (int64_t)dk) * dv;
        memcpy(dst, S, sizeof(double) * (size_t)dk * dv);
    }
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    const int dk = J->dk, dv = J->dv;
    const int dmax = dk > dv ? dk : dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *buf = (double *)malloc(sizeof(double) * (size_t)dmax * 5);
    if (!S || !buf) {
        free(S);
        free(buf);
        return (void *)1;
    }
    const int64_t units = J->num_seqs * J->nsel;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        run_unit(J, u, S, buf, buf + dmax, buf + 2 * dmax, buf + 3 * dmax, buf + 4 * dmax);
    }
    free(S);
    free(buf);
    return NULL;
}

/*
 * Token-by-token KDA over num_seqs independent sequences (batch rows or
 * cu_seqlens segments; a batch [B, T, H, d] is B sequences starting at b*T).
 * Tensors use the flattened token axis: q, k [tokens, H, dk]; v [tokens, H, dv];
 * g [tokens, H, dk]; beta [tokens, H].  Returns 0 on success, -1 on bad
 * arguments, -2 when memory or threads could not be obtained.
 */
int kda_oracle_fwd(int64_t num_seqs, const int64_t *starts, const int64_t *lens, int H, int dk, int dv,
                   int io_bf16, double scale, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *s0, int nsel, const int32_t *heads, double *o,
                   double *s_final, int nthreads) {
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || nsel <= 0 || !o || !starts || !lens) return -1;
    if (num_seqs > 0 && (!q || !k || !v || !g || !beta)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.num_seqs = num_seqs;
    J.starts = starts;
    J.lens = lens;
    J.H = H;
    J.dk = dk;
    J.dv = dv;
    J.io_bf16 = io_bf16;
    J.scale = scale;
    J.q = q;
    J.k = k;
    J.v = v;
    J.g = g;
    J.beta = beta;
    J.s0 = s0;
    J.nsel = nsel;
    J.heads = heads;
    J.o = o;
    J.s_final = s_final;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    const int64_t units = num_seqs * nsel;
    if (nthreads > units) nthreads = units > 0 ? (int)units : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -2;
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) rc = -2;
    for (int i = 0; i < started; ++i) {
        void *res = NULL;
        pthread_join(tid[i], &res);
        if (res) rc = -2;
    }
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return rc;
}

int kda_oracle_mutant(void) { return KDA_ORACLE_MUTANT; }
