/*
 * kda_oracle.c -- fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, includes or calls it, and it shares no source with it.
 *
 * What it computes (Kimi Linear paper notes, section 2 "KDA recurrence"):
 * per head, a fixed dk x dv state S is updated token by token as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                       (read-out uses the updated state)
 *
 * with alpha_t a per-channel decay vector (one forget rate per key channel,
 * the point of difference from Gated DeltaNet's single scalar per head).
 * Here alpha_t = exp(log_alpha_t) and beta_t is taken as given (it is already
 * a sigmoid output in the model).  The state starts at zero or from a supplied
 * checkpoint (Kimi Linear per-token dataflow notes, "KDA layer inputs, state
 * update and output"), and the chunk prefill and the fused recurrent decode
 * compute this same function (paper notes, section 3).
 *
 * The product (I - beta k k^T) X is evaluated as X - beta k (k^T X), i.e. the
 * same matrix product associated right to left; nothing else is reordered.
 * All arithmetic is IEEE double.  Inputs arrive in the exact dtype the GPU
 * receives (fp32, or bf16 as raw 16-bit patterns) and are widened exactly.
 *
 * Plain C, OpenMP over independent (sequence, head) pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static double widen(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    /* bf16 is the upper half of an IEEE binary32: exact widening */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One step of the recurrence on one head.
 *   S  : dk x dv, row c = key channel, column j = value channel (fp64, in/out)
 *   q,k: dk;  v: dv;  la: dk (log alpha);  o: dv (out);  y: dv scratch
 */
static void kda_step(double *S, int dk, int dv,
                     const double *q, const double *k, const double *v,
                     const double *la, double beta, double *o, double *y)
{
    /* X = Diag(alpha) S : every key channel c forgets at its own rate */
    for (int c = 0; c < dk; ++c) {
        double a = exp(la[c]);
        for (int j = 0; j < dv; ++j)
            S[(int64_t)c * dv + j] *= a;
    }
    /* y = k^T X */
    for (int j = 0; j < dv; ++j)
        y[j] = 0.0;
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            y[j] += k[c] * S[(int64_t)c * dv + j];
    /* S = X - beta k y^T + beta k v^T */
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            S[(int64_t)c * dv + j] += beta * k[c] * (v[j] - y[j]);
    /* o = S^T q with the updated state */
    for (int j = 0; j < dv; ++j)
        o[j] = 0.0;
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < dv; ++j)
            o[j] += q[c] * S[(int64_t)c * dv + j];
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Number of OpenMP threads a parallel region will use (for reporting). */
int oracle_max_threads(int nthreads) { return set_threads(nthreads); }

/* Optional preprocessing of the inputs (the options a caller may ask the
 * library to apply in-kernel; Kimi Linear paper notes, section 3 on the FLA
 * implementation: q/k L2 normalisation and the beta sigmoid):
 *   ORACLE_L2NORM_QK   q_t <- q_t / sqrt(q_t . q_t + 1e-6), the same for k_t
 *                      (per token and head, over the dk key channels)
 *   ORACLE_BETA_LOGIT  beta is given as a logit x: beta = 1 / (1 + exp(-x)) */
enum { ORACLE_L2NORM_QK = 1, ORACLE_BETA_LOGIT = 2 };

static void l2_normalise(double *x, int d)
{
    double ss = 0.0;
    for (int c = 0; c < d; ++c)
        ss += x[c] * x[c];
    double inv = 1.0 / sqrt(ss + 1e-6);
    for (int c = 0; c < d; ++c)
        x[c] *= inv;
}

/*
 * Prefill over a packed batch, with options.
 *   q,k: [T,H,dk]   v: [T,H,dv]    (dtype: 0 = fp32, 1 = bf16 bit patterns)
 *   log_alpha: [T,H,dk] fp32       beta: [T,H] fp32 (a logit with ORACLE_BETA_LOGIT)
 *   initial state: s0_f32 or s0_f64 [N,H,dk,dv] (at most one), or both NULL = zeros
 *   cu_seqlens: host [N+1] int32 offsets, or NULL = N equal rows of T/N
 *   flags: ORACLE_* bits above
 *   every, states: if every > 0 and states != NULL, the state entering token
 *      t0 + every*c of each sequence (c = 0 .. ceil(len/every) - 1, i.e. after
 *      every*c of its tokens) is written to states[(base_s + c)*H + h] with
 *      base_s = sum over earlier sequences of ceil(len/every): [NS,H,dk,dv] fp64
 *   o: [T,H,dv] fp64 out            final_state: [N,H,dk,dv] fp64 out or NULL
 * Returns 0, or -1 on bad arguments.
 */
int oracle_prefill_ex(const void *q, const void *k, const void *v,
                      const float *log_alpha, const float *beta,
                      const float *s0_f32, const double *s0_f64, const int32_t *cu_seqlens,
                      int64_t total_tokens, int32_t num_seqs, int32_t H,
                      int32_t dk, int32_t dv, int32_t dtype, int32_t flags,
                      int32_t every, double *states,
                      double *o, double *final_state, int32_t nthreads)
{
    if (num_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0 || total_tokens < 0 || every < 0)
        return -1;
    if (!cu_seqlens && total_tokens % num_seqs != 0)
        return -1;
    if (s0_f32 && s0_f64)
        return -1;
    set_threads(nthreads);
    const int64_t units = (int64_t)num_seqs * H;
    /* first snapshot row of every sequence */
    int64_t *snap_base = (int64_t *)calloc((size_t)num_seqs + 1, sizeof(int64_t));
    if (!snap_base)
        return -1;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t len = cu_seqlens ? (int64_t)cu_seqlens[s + 1] - cu_seqlens[s]
                                 : total_tokens / num_seqs;
        snap_base[s + 1] = snap_base[s] + (every > 0 && len > 0 ? (len + every - 1) / every : 0);
    }
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t u = 0; u < units; ++u) {
        const int32_t s = (int32_t)(u / H), h = (int32_t)(u % H);
        int64_t t0, t1;
        if (cu_seqlens) {
            t0 = cu_seqlens[s];
            t1 = cu_seqlens[s + 1];
        } else {
            int64_t len = total_tokens / num_seqs;
            t0 = (int64_t)s * len;
            t1 = t0 + len;
        }
        if (t0 < 0 || t1 < t0 || t1 > total_tokens) {
            bad |= 1;
            continue;
        }
        double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
        double *qv = (double *)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
        if (!S || !qv) {
            free(S);
            free(qv);
            bad |= 1;
            continue;
        }
        double *kv = qv + dk, *lv = kv + dk, *vv = lv + dk, *ov = vv + dv, *y = ov + dv;
        if (s0_f32) {
            const float *S0 = s0_f32 + ((int64_t)s * H + h) * dk * dv;
            for (int64_t i = 0; i < (int64_t)dk * dv; ++i)
                S[i] = (double)S0[i];
        } else if (s0_f64) {
            memcpy(S, s0_f64 + ((int64_t)s * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
        }
        for (int64_t t = t0; t < t1; ++t) {
            if (every > 0 && states && (t - t0) % every == 0)
                memcpy(states + ((snap_base[s] + (t - t0) / every) * H + h) * dk * dv, S,
                       sizeof(double) * (size_t)dk * dv);
            const int64_t rk = (t * H + h) * dk, rv = (t * H + h) * dv;
            for (int c = 0; c < dk; ++c) {
                qv[c] = widen(q, rk + c, dtype);
                kv[c] = widen(k, rk + c, dtype);
                lv[c] = (double)log_alpha[rk + c];
            }
            for (int j = 0; j < dv; ++j)
                vv[j] = widen(v, rv + j, dtype);
            if (flags & ORACLE_L2NORM_QK) {
                l2_normalise(qv, dk);
                l2_normalise(kv, dk);
            }
            double b = (double)beta[t * H + h];
            if (flags & ORACLE_BETA_LOGIT)
                b = 1.0 / (1.0 + exp(-b));
            kda_step(S, dk, dv, qv, kv, vv, lv, b, ov, y);
            memcpy(o + rv, ov, sizeof(double) * (size_t)dv);
        }
        if (final_state)
            memcpy(final_state + ((int64_t)s * H + h) * dk * dv, S,
                   sizeof(double) * (size_t)dk * dv);
        free(S);
        free(qv);
    }
    free(snap_base);
    return bad ? -1 : 0;
}

/* Prefill without options (fp32 initial state, no snapshots). */
int oracle_prefill(const void *q, const void *k, const void *v,
                   const float *log_alpha, const float *beta,
                   const float *initial_state, const int32_t *cu_seqlens,
                   int64_t total_tokens, int32_t num_seqs, int32_t H,
                   int32_t dk, int32_t dv, int32_t dtype,
                   double *o, double *final_state, int32_t nthreads)
{
    return oracle_prefill_ex(q, k, v, log_alpha, beta, initial_state, NULL, cu_seqlens,
                             total_tokens, num_seqs, H, dk, dv, dtype, 0, 0, NULL,
                             o, final_state, nthreads);
}

/*
 * One decode token for every (sequence, head): the same step applied once.
 *   state: [N,H,dk,dv] fp64, read and updated in place
 *   q,k: [N,H,dk]  v: [N,H,dv] (dtype as above)  log_alpha: [N,H,dk]  beta: [N,H]
 *   o: [N,H,dv] fp64 out
 */
int oracle_decode_step(double *state, const void *q, const void *k, const void *v,
                       const float *log_alpha, const float *beta,
                       int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                       int32_t dtype, double *o, int32_t nthreads)
{
    if (num_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    set_threads(nthreads);
    const int64_t units = (int64_t)num_seqs * H;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t u = 0; u < units; ++u) {
        double *qv = (double *)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
        if (!qv) {
            bad |= 1;
            continue;
        }
        double *kv = qv + dk, *lv = kv + dk, *vv = lv + dk, *ov = vv + dv, *y = ov + dv;
        const int64_t rk = u * dk, rv = u * dv;
        for (int c = 0; c < dk; ++c) {
            qv[c] = widen(q, rk + c, dtype);
            kv[c] = widen(k, rk + c, dtype);
            lv[c] = (double)log_alpha[rk + c];
        }
        for (int j = 0; j < dv; ++j)
            vv[j] = widen(v, rv + j, dtype);
        kda_step(state + u * dk * dv, dk, dv, qv, kv, vv, lv, (double)beta[u], ov, y);
        memcpy(o + rv, ov, sizeof(double) * (size_t)dv);
        free(qv);
    }
    return bad ? -1 : 0;
}

/*
 * Gradients of the recurrence (reverse mode, written out step by step).
 *
 * For a loss L whose gradients with respect to the outputs are d_o [T,H,dv]
 * and d_final [N,H,dk,dv] (NULL = 0), this returns dL/dq, dL/dk, dL/dv,
 * dL/dlog_alpha, dL/dbeta and dL/dinitial_state (the pages give no backward
 * pass; this is the chain rule applied to the three lines of kda_step in
 * reverse order, and a finite-difference test pins it to the forward above).
 *
 * One forward step is  X = Diag(a) S;  y = X^T k;  S' = X + beta k (v - y)^T;
 * o = S'^T q.  With G the gradient of S' (plus q do^T from the read-out):
 *   dq   = S' do
 *   dX   = G;   dk += beta G (v - y);   dbeta = k^T G (v - y);
 *   dv   = beta G^T k;   dy = -beta G^T k
 *   dX  += k dy^T;   dk += X dy
 *   dS   = Diag(a) dX;   dlog_alpha_c = sum_j dX[c,j] X[c,j]
 * States are recomputed forward from checkpoints every 64 tokens (the same
 * operations in the same order, so the recomputed states are the forward's).
 *
 * Outputs (fp64): dq, dk [T,H,dk]; dv [T,H,dv]; dla [T,H,dk]; dbeta [T,H];
 * ds0 [N,H,dk,dv] or NULL.  Returns 0, or -1 on bad arguments.
 */
enum { ORACLE_CKPT = 64 };

int oracle_backward(const void *q, const void *k, const void *v,
                    const float *log_alpha, const float *beta,
                    const float *initial_state, const int32_t *cu_seqlens,
                    int64_t total_tokens, int32_t num_seqs, int32_t H,
                    int32_t dk, int32_t dv, int32_t dtype,
                    const double *d_o, const double *d_final,
                    double *dq, double *dk_out, double *dv_out, double *dla, double *dbeta,
                    double *ds0, int32_t nthreads)
{
    if (num_seqs <= 0 || H <= 0 || dk <= 0 || dv <= 0 || total_tokens < 0 || !d_o)
        return -1;
    if (!cu_seqlens && total_tokens % num_seqs != 0)
        return -1;
    set_threads(nthreads);
    const int64_t units = (int64_t)num_seqs * H;
    const int64_t SZ = (int64_t)dk * dv;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t u = 0; u < units; ++u) {
        const int32_t s = (int32_t)(u / H), h = (int32_t)(u % H);
        int64_t t0, t1;
        if (cu_seqlens) {
            t0 = cu_seqlens[s];
            t1 = cu_seqlens[s + 1];
        } else {
            int64_t len = total_tokens / num_seqs;
            t0 = (int64_t)s * len;
            t1 = t0 + len;
        }
        if (t0 < 0 || t1 < t0 || t1 > total_tokens) {
            bad |= 1;
            continue;
        }
        const int64_t len = t1 - t0;
        const int64_t nck = (len + ORACLE_CKPT - 1) / ORACLE_CKPT;
        /* ckpt[c]: state before token t0 + 64c;  seg[i]: state before token i of a segment */
        double *ckpt = (double *)malloc(sizeof(double) * (size_t)((nck + 1) * SZ));
        double *seg = (double *)malloc(sizeof(double) * (size_t)((ORACLE_CKPT + 1) * SZ));
        double *G = (double *)calloc((size_t)SZ, sizeof(double));
        double *X = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(4 * dk + 6 * dv));
        if (!ckpt || !seg || !G || !X || !vec) {
            free(ckpt); free(seg); free(G); free(X); free(vec);
            bad |= 1;
            continue;
        }
        double *qv = vec, *kv = qv + dk, *lv = kv + dk, *av = lv + dk;
        double *vv = av + dk, *ov = vv + dv, *y = ov + dv, *dov = y + dv, *gk = dov + dv, *dy = gk + dv;

        /* the token's inputs, widened exactly */
        #define KDA_LOAD_TOKEN(t)                                              \
            do {                                                               \
                const int64_t rk_ = ((t) * H + h) * dk, rv_ = ((t) * H + h) * dv; \
                for (int c = 0; c < dk; ++c) {                                 \
                    qv[c] = widen(q, rk_ + c, dtype);                          \
                    kv[c] = widen(k, rk_ + c, dtype);                          \
                    lv[c] = (double)log_alpha[rk_ + c];                        \
                    av[c] = exp(lv[c]);                                        \
                }                                                              \
                for (int j = 0; j < dv; ++j)                                   \
                    vv[j] = widen(v, rv_ + j, dtype);                          \
            } while (0)

        /* forward: checkpoints */
        double *S = ckpt;
        memset(S, 0, sizeof(double) * (size_t)SZ);
        if (initial_state) {
            const float *S0 = initial_state + ((int64_t)s * H + h) * SZ;
            for (int64_t i = 0; i < SZ; ++i)
                S[i] = (double)S0[i];
        }
        for (int64_t c = 0; c < nck; ++c) {
            double *Sc = ckpt + c * SZ, *Sn = ckpt + (c + 1) * SZ;
            memcpy(Sn, Sc, sizeof(double) * (size_t)SZ);
            const int64_t a = t0 + c * ORACLE_CKPT, b = a + ORACLE_CKPT < t1 ? a + ORACLE_CKPT : t1;
            for (int64_t t = a; t < b; ++t) {
                KDA_LOAD_TOKEN(t);
                kda_step(Sn, dk, dv, qv, kv, vv, lv, (double)beta[t * H + h], ov, y);
            }
        }
        /* reverse */
        if (d_final)
            memcpy(G, d_final + ((int64_t)s * H + h) * SZ, sizeof(double) * (size_t)SZ);
        for (int64_t c = nck - 1; c >= 0; --c) {
            const int64_t a = t0 + c * ORACLE_CKPT, b = a + ORACLE_CKPT < t1 ? a + ORACLE_CKPT : t1;
            memcpy(seg, ckpt + c * SZ, sizeof(double) * (size_t)SZ);
            for (int64_t t = a; t < b; ++t) {
                double *Sn = seg + (t - a + 1) * SZ;
                memcpy(Sn, seg + (t - a) * SZ, sizeof(double) * (size_t)SZ);
                KDA_LOAD_TOKEN(t);
                kda_step(Sn, dk, dv, qv, kv, vv, lv, (double)beta[t * H + h], ov, y);
            }
            for (int64_t t = b - 1; t >= a; --t) {
                const double *Sprev = seg + (t - a) * SZ, *Snew = seg + (t - a + 1) * SZ;
                const int64_t rk = (t * H + h) * dk, rv = (t * H + h) * dv;
                const double bt = (double)beta[t * H + h];
                KDA_LOAD_TOKEN(t);
                for (int j = 0; j < dv; ++j)
                    dov[j] = d_o[rv + j];
                /* X = Diag(a) S_prev;  y = X^T k */
                for (int c2 = 0; c2 < dk; ++c2)
                    for (int j = 0; j < dv; ++j)
                        X[(int64_t)c2 * dv + j] = av[c2] * Sprev[(int64_t)c2 * dv + j];
                for (int j = 0; j < dv; ++j) {
                    y[j] = 0.0;
                    for (int c2 = 0; c2 < dk; ++c2)
                        y[j] += kv[c2] * X[(int64_t)c2 * dv + j];
                }
                /* read-out: dq = S' do;  G += q do^T */
                for (int c2 = 0; c2 < dk; ++c2) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc += Snew[(int64_t)c2 * dv + j] * dov[j];
                        G[(int64_t)c2 * dv + j] += qv[c2] * dov[j];
                    }
                    dq[rk + c2] = acc;
                }
                /* write: gk = G^T k;  dv = beta gk;  dy = -beta gk;  dbeta = gk . (v - y) */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    gk[j] = 0.0;
                    for (int c2 = 0; c2 < dk; ++c2)
                        gk[j] += G[(int64_t)c2 * dv + j] * kv[c2];
                    dv_out[rv + j] = bt * gk[j];
                    dy[j] = -bt * gk[j];
                    db += gk[j] * (vv[j] - y[j]);
                }
                dbeta[t * H + h] = db;
                /* dk = beta G (v - y) + X dy;  dX = G + k dy^T */
                for (int c2 = 0; c2 < dk; ++c2) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc += bt * G[(int64_t)c2 * dv + j] * (vv[j] - y[j]);
                        acc += X[(int64_t)c2 * dv + j] * dy[j];
                        G[(int64_t)c2 * dv + j] += kv[c2] * dy[j];
                    }
                    dk_out[rk + c2] = acc;
                }
                /* decay: dlog_alpha = sum_j dX X;  dS = Diag(a) dX */
                for (int c2 = 0; c2 < dk; ++c2) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc += G[(int64_t)c2 * dv + j] * X[(int64_t)c2 * dv + j];
                        G[(int64_t)c2 * dv + j] *= av[c2];
                    }
                    dla[rk + c2] = acc;
                }
            }
        }
        #undef KDA_LOAD_TOKEN
        if (ds0)
            memcpy(ds0 + ((int64_t)s * H + h) * SZ, G, sizeof(double) * (size_t)SZ);
        free(ckpt); free(seg); free(G); free(X); free(vec);
    }
    return bad ? -1 : 0;
}
