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

/* ------------------------------------------------------------------ backward --
 *
 * Gradients of the recurrence above for a loss that is linear in the outputs:
 *   L = sum_t <dO_t, o_t> + <dS_final, S_T>
 * i.e. given dO (the gradient of the outputs) and dS_final (the gradient of the final
 * state, or zero), returns dq, dk, dv, dg, dbeta and d(initial state).  This is the
 * training side of the operator; the pages motivate the chunkwise WY/UT form by training
 * throughput ("Chunkwise parallel algorithm" section), the gradients themselves follow
 * from the recurrence by the chain rule, one token at a time in reverse order:
 *
 *   with S' = Diag(alpha) S_{t-1}, p = S'^T k, u = v - p, S_t = S' + beta k u^T:
 *     dS     += scale q dO_t^T             (o_t = scale S_t^T q)
 *     dq_t    = scale S_t dO_t
 *     du      = beta dS^T k                 -> dv_t = du,  dp = -du
 *     dbeta_t = k^T dS u
 *     dk_t    = beta dS u + S' dp           (outer product, then the prediction p)
 *     dS'     = dS + k dp^T
 *     dg_t    = rowsum(dS' .* S')           (d alpha_i * alpha_i: g is the log gate)
 *     dS_{t-1} = Diag(alpha) dS'
 *
 * The forward states are needed in reverse order: they are recomputed per segment of
 * ~sqrt(len) tokens from checkpoints saved on a first forward sweep (all in fp64).
 */
typedef struct {
    int64_t num_seqs;
    const int64_t *starts, *lens;
    int H, dk, dv, io_bf16;
    double scale;
    const void *q, *k, *v, *d_o;
    const float *g, *beta, *s0, *d_sf;
    int nsel;
    const int32_t *heads;
    double *dq, *dk_out, *dv_out, *dg, *dbeta, *ds0; /* ds0 may be NULL */
    int64_t next_unit;
    int failed;
    pthread_mutex_t lock;
} bjob_t;

/* one forward token step in place: S <- S' + beta k (v - p)^T; keeps S' and u if asked */
static void fwd_token(const bjob_t *J, int64_t t, int h, double *S, double *qv, double *kv, double *a,
                      double *vv, double *p) {
    const int H = J->H, dk = J->dk, dv = J->dv;
    const int64_t row_k = (t * H + h) * (int64_t)dk, row_v = (t * H + h) * (int64_t)dv;
    for (int i = 0; i < dk; ++i) {
        qv[i] = load_io(J->q, J->io_bf16, row_k + i);
        kv[i] = load_io(J->k, J->io_bf16, row_k + i);
        a[i] = exp((double)J->g[row_k + i]);
    }
    for (int j = 0; j < dv; ++j) vv[j] = load_io(J->v, J->io_bf16, row_v + j);
    const double b = (double)J->beta[t * H + h];
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= a[i];
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) p[j] += S[(int64_t)i * dv + j] * kv[i];
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += b * kv[i] * (vv[j] - p[j]);
}

static int run_unit_bwd(bjob_t *J, int64_t unit) {
    const int64_t n = unit / J->nsel;
    const int hs = (int)(unit % J->nsel);
    const int h = J->heads ? J->heads[hs] : hs;
    const int H = J->H, dk = J->dk, dv = J->dv, nsel = J->nsel;
    const int64_t DD = (int64_t)dk * dv;
    const int64_t t0 = J->starts[n], len = J->lens[n];

    int64_t seg = 1;
    while (seg * seg < len) ++seg;
    const int64_t nseg = len > 0 ? (len + seg - 1) / seg : 0;
    const int dmax = dk > dv ? dk : dv;
    double *ck = (double *)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * DD)); /* state before segment */
    double *st = (double *)malloc(sizeof(double) * (size_t)((seg + 1) * DD));              /* states inside segment */
    double *dS = (double *)malloc(sizeof(double) * (size_t)DD);
    double *dSp = (double *)malloc(sizeof(double) * (size_t)DD);
    double *Sp = (double *)malloc(sizeof(double) * (size_t)DD);
    double *buf = (double *)malloc(sizeof(double) * (size_t)dmax * 10);
    if (!ck || !st || !dS || !dSp || !Sp || !buf) {
        free(ck); free(st); free(dS); free(dSp); free(Sp); free(buf);
        return -2;
    }
    double *qv = buf, *kv = buf + dmax, *a = buf + 2 * dmax, *vv = buf + 3 * dmax, *p = buf + 4 * dmax;
    double *dov = buf + 5 * dmax, *u = buf + 6 * dmax, *du = buf + 7 * dmax, *tmp = buf + 8 * dmax;

    /* forward sweep: checkpoint the state entering each segment */
    double *S = st;
    if (J->s0) {
        const float *src = J->s0 + (n * H + h) * DD;
        for (int64_t e = 0; e < DD; ++e) S[e] = (double)src[e];
    } else {
        memset(S, 0, sizeof(double) * (size_t)DD);
    }
    for (int64_t sgi = 0; sgi < nseg; ++sgi) {
        memcpy(ck + sgi * DD, S, sizeof(double) * (size_t)DD);
        const int64_t e = (sgi + 1) * seg < len ? (sgi + 1) * seg : len;
        for (int64_t t = sgi * seg; t < e; ++t) fwd_token(J, t0 + t, h, S, qv, kv, a, vv, p);
    }

    /* reverse sweep */
    if (J->d_sf) {
        const float *src = J->d_sf + (n * H + h) * DD;
        for (int64_t e = 0; e < DD; ++e) dS[e] = (double)src[e];
    } else {
        memset(dS, 0, sizeof(double) * (size_t)DD);
    }
    for (int64_t sgi = nseg - 1; sgi >= 0; --sgi) {
        const int64_t b0 = sgi * seg, e = (sgi + 1) * seg < len ? (sgi + 1) * seg : len;
        /* st[i] = state before token b0 + i, st[e - b0] = state after the segment */
        memcpy(st, ck + sgi * DD, sizeof(double) * (size_t)DD);
        for (int64_t t = b0; t < e; ++t) {
            memcpy(st + (t - b0 + 1) * DD, st + (t - b0) * DD, sizeof(double) * (size_t)DD);
            fwd_token(J, t0 + t, h, st + (t - b0 + 1) * DD, qv, kv, a, vv, p);
        }
        for (int64_t t = e - 1; t >= b0; --t) {
            const int64_t tt = t0 + t;
            const double *Sprev = st + (t - b0) * DD, *Snew = st + (t - b0 + 1) * DD;
            const int64_t row_k = (tt * H + h) * (int64_t)dk, row_v = (tt * H + h) * (int64_t)dv;
            for (int i = 0; i < dk; ++i) {
                qv[i] = load_io(J->q, J->io_bf16, row_k + i);
                kv[i] = load_io(J->k, J->io_bf16, row_k + i);
                a[i] = exp((double)J->g[row_k + i]);
            }
            for (int j = 0; j < dv; ++j) {
                vv[j] = load_io(J->v, J->io_bf16, row_v + j);
                dov[j] = load_io(J->d_o, J->io_bf16, row_v + j);
            }
            const double b = (double)J->beta[tt * H + h];
            /* S' and u = v - S'^T k */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) Sp[(int64_t)i * dv + j] = a[i] * Sprev[(int64_t)i * dv + j];
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += Sp[(int64_t)i * dv + j] * kv[i];
                u[j] = vv[j] - acc;
            }
            /* o_t = scale S_t^T q */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
#if KDA_ORACLE_MUTANT == 15 /* planted: dq read from the decayed state before the update */
                for (int j = 0; j < dv; ++j) acc += Sp[(int64_t)i * dv + j] * dov[j];
#else
                for (int j = 0; j < dv; ++j) acc += Snew[(int64_t)i * dv + j] * dov[j];
#endif
                J->dq[(tt * nsel + hs) * (int64_t)dk + i] = J->scale * acc;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) dS[(int64_t)i * dv + j] += J->scale * qv[i] * dov[j];
            /* du = beta dS^T k; dbeta = k^T dS u */
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += dS[(int64_t)i * dv + j] * kv[i];
                du[j] = b * acc;
#if KDA_ORACLE_MUTANT == 13 /* planted: beta gradient with the wrong sign */
                db -= acc * u[j];
#else
                db += acc * u[j];
#endif
            }
            J->dbeta[tt * nsel + hs] = db;
            for (int j = 0; j < dv; ++j) J->dv_out[(tt * nsel + hs) * (int64_t)dv + j] = du[j];
            /* dk = beta dS u + S' dp, dp = -du */
            for (int i = 0; i < dk; ++i) {
                double acc1 = 0.0, acc2 = 0.0;
                for (int j = 0; j < dv; ++j) {
                    acc1 += dS[(int64_t)i * dv + j] * u[j];
                    acc2 += Sp[(int64_t)i * dv + j] * du[j];
                }
#if KDA_ORACLE_MUTANT == 11 /* planted: prediction path of the key gradient dropped */
                tmp[i] = b * acc1;
#else
                tmp[i] = b * acc1 - acc2;
#endif
            }
            for (int i = 0; i < dk; ++i) J->dk_out[(tt * nsel + hs) * (int64_t)dk + i] = tmp[i];
            /* dS' = dS - k du^T; dg = rowsum(dS' .* S'); dS_{t-1} = Diag(alpha) dS' */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    const double d = dS[(int64_t)i * dv + j] - kv[i] * du[j];
#if KDA_ORACLE_MUTANT == 12 /* planted: gate gradient against the undecayed state */
                    acc += d * Sprev[(int64_t)i * dv + j];
#else
                    acc += d * Sp[(int64_t)i * dv + j];
#endif
#if KDA_ORACLE_MUTANT == 14 /* planted: state gradient carried back without the decay */
                    dSp[(int64_t)i * dv + j] = d;
#else
                    dSp[(int64_t)i * dv + j] = a[i] * d;
#endif
                }
                J->dg[(tt * nsel + hs) * (int64_t)dk + i] = acc;
            }
            memcpy(dS, dSp, sizeof(double) * (size_t)DD);
        }
    }
    if (J->ds0) memcpy(J->ds0 + (n * nsel + hs) * DD, dS, sizeof(double) * (size_t)DD);
    free(ck); free(st); free(dS); free(dSp); free(Sp); free(buf);
    return 0;
}

static void *worker_bwd(void *arg) {
    bjob_t *J = (bjob_t *)arg;
    const int64_t units = J->num_seqs * J->nsel;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        if (run_unit_bwd(J, u) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

/*
 * Gradients of the token-by-token KDA (layouts as kda_oracle_fwd; d_o in the io dtype
 * with v's shape; d_sf [num_seqs, H, dk, dv] fp32 or NULL).  Outputs are fp64 with the
 * selected heads: dq, dk, dg [tokens, nsel, dk]; dv [tokens, nsel, dv]; dbeta
 * [tokens, nsel]; ds0 [num_seqs, nsel, dk, dv] or NULL.  Returns 0, -1 (arguments) or
 * -2 (memory / threads).
 */
int kda_oracle_bwd(int64_t num_seqs, const int64_t *starts, const int64_t *lens, int H, int dk, int dv,
                   int io_bf16, double scale, const void *q, const void *k, const void *v, const float *g,
                   const float *beta, const float *s0, const void *d_o, const float *d_sf, int nsel,
                   const int32_t *heads, double *dq, double *dk_out, double *dv_out, double *dg, double *dbeta,
                   double *ds0, int nthreads) {
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || nsel <= 0 || !starts || !lens) return -1;
    if (!dq || !dk_out || !dv_out || !dg || !dbeta) return -1;
    if (num_seqs > 0 && (!q || !k || !v || !g || !beta || !d_o)) return -1;
    bjob_t J;
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
    J.d_o = d_o;
    J.g = g;
    J.beta = beta;
    J.s0 = s0;
    J.d_sf = d_sf;
    J.nsel = nsel;
    J.heads = heads;
    J.dq = dq;
    J.dk_out = dk_out;
    J.dv_out = dv_out;
    J.dg = dg;
    J.dbeta = dbeta;
    J.ds0 = ds0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    const int64_t units = num_seqs * nsel;
    if (nthreads > units) nthreads = units > 0 ? (int)units : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -2;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker_bwd, &J) != 0) break;
        ++started;
    }
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&J.lock);
    if (started == 0 || J.failed) return -2;
    return 0;
}

/* ------------------------------------------------------- general DPLR comparator --
 *
 * The general diagonal-plus-low-rank recurrence that KDA specialises (Kimi Linear summary
 * page, "Less compute than general DPLR" section: both support fine-grained decay; KDA
 * ties both low-rank vectors to the key):
 *
 *   S_t = (Diag(exp(g_t)) + a_t b_t^T) S_{t-1} + k_t v_t^T,     o_t = scale * S_t^T q_t
 *
 * with independent per-token vectors a_t, b_t (d_k).  KDA is the case a = -beta k,
 * b = exp(g) * k and a write key beta k.  Same layouts as kda_oracle_fwd; a and b share
 * the io dtype of q and k.
 */
typedef struct {
    int64_t num_seqs;
    const int64_t *starts, *lens;
    int H, dk, dv, io_bf16;
    double scale;
    const void *q, *k, *v, *a, *b;
    const float *g, *s0;
    double *o, *s_final;
    int64_t next_unit;
    pthread_mutex_t lock;
} djob_t;

static void run_unit_dplr(djob_t *J, int64_t unit, double *S, double *buf) {
    const int64_t n = unit / J->H;
    const int h = (int)(unit % J->H);
    const int H = J->H, dk = J->dk, dv = J->dv;
    const int dmax = dk > dv ? dk : dv;
    double *qv = buf, *kv = buf + dmax, *av = buf + 2 * dmax, *bv = buf + 3 * dmax, *al = buf + 4 * dmax,
           *vv = buf + 5 * dmax, *u = buf + 6 * dmax;
    if (J->s0) {
        const float *src = J->s0 + ((n * H + h) * (int64_t)dk) * dv;
        for (int64_t e = 0; e < (int64_t)dk * dv; ++e) S[e] = (double)src[e];
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    }
    const int64_t t0 = J->starts[n], len = J->lens[n];
    for (int64_t t = t0; t < t0 + len; ++t) {
        const int64_t row_k = (t * H + h) * (int64_t)dk, row_v = (t * H + h) * (int64_t)dv;
        for (int i = 0; i < dk; ++i) {
            qv[i] = load_io(J->q, J->io_bf16, row_k + i);
            kv[i] = load_io(J->k, J->io_bf16, row_k + i);
            av[i] = load_io(J->a, J->io_bf16, row_k + i);
            bv[i] = load_io(J->b, J->io_bf16, row_k + i);
            al[i] = exp((double)J->g[row_k + i]);
        }
        for (int j = 0; j < dv; ++j) vv[j] = load_io(J->v, J->io_bf16, row_v + j);
        /* u = b^T S_{t-1} (uses the state before the decay) */
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) u[j] += bv[i] * S[(int64_t)i * dv + j];
#if KDA_ORACLE_MUTANT == 21 /* planted: low-rank term against the decayed state */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= al[i];
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) u[j] += bv[i] * S[(int64_t)i * dv + j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += av[i] * u[j] + kv[i] * vv[j];
#else
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(int64_t)i * dv + j] = al[i] * S[(int64_t)i * dv + j] + av[i] * u[j] + kv[i] * vv[j];
#endif
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * qv[i];
            J->o[(t * H + h) * (int64_t)dv + j] = J->scale * acc;
        }
    }
    if (J->s_final) memcpy(J->s_final + ((n * H + h) * (int64_t)dk) * dv, S, sizeof(double) * (size_t)dk * dv);
}

static void *worker_dplr(void *arg) {
    djob_t *J = (djob_t *)arg;
    const int dmax = J->dk > J->dv ? J->dk : J->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double *buf = (double *)malloc(sizeof(double) * (size_t)dmax * 7);
    if (!S || !buf) {
        free(S);
        free(buf);
        return (void *)1;
    }
    const int64_t units = J->num_seqs * J->H;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        run_unit_dplr(J, u, S, buf);
    }
    free(S);
    free(buf);
    return NULL;
}

/* General DPLR forward, token by token (fp64).  o [tokens, H, dv]; s_final
 * [num_seqs, H, dk, dv] or NULL.  Returns 0, -1 (arguments) or -2 (memory / threads). */
int kda_oracle_dplr_fwd(int64_t num_seqs, const int64_t *starts, const int64_t *lens, int H, int dk, int dv,
                        int io_bf16, double scale, const void *q, const void *k, const void *v, const void *a,
                        const void *b, const float *g, const float *s0, double *o, double *s_final, int nthreads) {
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !o || !starts || !lens) return -1;
    if (num_seqs > 0 && (!q || !k || !v || !a || !b || !g)) return -1;
    djob_t J;
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
    J.a = a;
    J.b = b;
    J.g = g;
    J.s0 = s0;
    J.o = o;
    J.s_final = s_final;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    const int64_t units = num_seqs * H;
    if (nthreads > units) nthreads = units > 0 ? (int)units : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -2;
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker_dplr, &J) != 0) break;
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
