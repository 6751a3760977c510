/*
 * Oracle for the gradients of the gated delta-rule forward pass: reverse-mode
 * differentiation of the fp64 token recurrence, written out by hand.
 *
 * TEST INFRASTRUCTURE ONLY (like gdr_ref.c, which it does not call): the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * Forward step (gdr_ref.c; "Diagonal Plus Low Rank" notes, section 2, with the
 * write scaled by beta):
 *     X   = S_{t-1} Diag(alpha_t)
 *     S_t = X (I - b_t a_t^T) + beta_t v_t k_t^T,      o_t = S_t q_t
 * with (a, b) = (k, beta k) when a and b are not given (KDA, GDN, DeltaNet).
 *
 * Given dO = dL/dO and dS_final = dL/dS_final (NULL: zero), the reverse pass
 * keeps G = dL/dS_t and walks the tokens backwards:
 *     G      += do_t q_t^T                      dq_t = S_t^T do_t
 *     dbeta_t = v_t^T G k_t   (write term)      dv_t = beta_t G k_t
 *     dk_t    = beta_t G^T v_t (write term)
 *     da_t    = -G^T (X b_t)                    db_t = -X^T (G a_t)
 *     dX      = G - (G a_t) b_t^T
 *     dlog alpha_t[j] = sum_i dX_ij X_ij        (head gate: summed over j)
 *     G      <- dX Diag(alpha_t)                (= dL/dS_{t-1})
 * and at the start of the sequence dS0 = G.  Without a and b the a- and
 * b-gradients fold into k and beta: dk_t += da_t + beta_t db_t and
 * dbeta_t += k_t^T db_t.
 *
 * The states S_t are recomputed: the forward pass keeps a checkpoint every
 * kSeg tokens, and each segment is replayed forwards (all its states kept)
 * before its tokens are walked backwards.
 *
 * Layouts as in gdr_ref.c; gradients have the shapes of their inputs.  Every
 * gradient pointer may be NULL except dq, dk, dv, dbeta; da/db must be given
 * exactly when a/b are; dlog_alpha is required with a gate.  Gradients of
 * (sequence, head) chains that are not computed are left untouched.  The
 * spectral clip of the gate is not differentiated here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { kSeg = 64 };

typedef struct {
    const double *q, *k, *v, *a, *b, *log_alpha, *beta, *S0, *dO, *dSf;
    double *dq, *dk, *dv, *da, *db, *dla, *dbeta, *dS0;
    int gate, H, dk_, dv_;
} BwdArgs;

/* alpha_t of token-head th, one value per key channel */
static void gate_of(const BwdArgs *p, size_t th, double *alpha) {
    for (int j = 0; j < p->dk_; ++j) {
        if (p->gate == 2) alpha[j] = exp(p->log_alpha[th * p->dk_ + j]);
        else if (p->gate == 1) alpha[j] = exp(p->log_alpha[th]);
        else alpha[j] = 1.0;
    }
}

/* One forward step S <- S Diag(alpha)(I - b a^T) + beta v k^T, in place. */
static void step(const BwdArgs *p, size_t th, double *S, double *alpha, double *xb) {
    const int dk = p->dk_, dv = p->dv_;
    const double *kt = p->k + th * dk, *vt = p->v + th * dv;
    const double bt = p->beta[th];
    gate_of(p, th, alpha);
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) S[(size_t)i * dk + j] *= alpha[j];
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) {
            const double bj = p->b ? p->b[th * dk + j] : bt * kt[j];
            acc += S[(size_t)i * dk + j] * bj;
        }
        xb[i] = acc;
    }
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) {
            const double aj = p->a ? p->a[th * dk + j] : kt[j];
            S[(size_t)i * dk + j] += -xb[i] * aj + bt * vt[i] * kt[j];
        }
}

typedef struct {
    double *ckpt;   /* one state per segment start */
    double *seg;    /* states S_{t0-1} .. S_{t0+kSeg-1} of the segment being replayed */
    double *G, *X, *alpha, *xb, *ga, *tmp, *bvec;
} Scratch;

static void run_chain_bwd(const BwdArgs *p, int n, int h, long t0, long t1, Scratch *w) {
    const int dk = p->dk_, dv = p->dv_, H = p->H;
    const size_t SS = (size_t)dv * dk;
    const long len = t1 - t0;
    const long nseg = (len + kSeg - 1) / kSeg;
    /* forward: checkpoints at segment starts (the state before the segment's first token) */
    double *S = w->seg;
    if (p->S0) memcpy(S, p->S0 + ((size_t)n * H + h) * SS, sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    for (long s = 0; s < nseg; ++s) {
        memcpy(w->ckpt + (size_t)s * SS, S, sizeof(double) * SS);
        const long e = t0 + (s + 1) * kSeg < t1 ? t0 + (s + 1) * kSeg : t1;
        for (long t = t0 + s * kSeg; t < e; ++t) step(p, (size_t)t * H + h, S, w->alpha, w->xb);
    }
    /* G = dL/dS at the end of the sequence */
    if (p->dSf) memcpy(w->G, p->dSf + ((size_t)n * H + h) * SS, sizeof(double) * SS);
    else memset(w->G, 0, sizeof(double) * SS);
    for (long s = nseg - 1; s >= 0; --s) {
        const long sb = t0 + s * kSeg;
        const long e = sb + kSeg < t1 ? sb + kSeg : t1;
        /* replay: seg[0] = state before token sb, seg[i+1] = state after token sb + i */
        memcpy(w->seg, w->ckpt + (size_t)s * SS, sizeof(double) * SS);
        for (long t = sb; t < e; ++t) {
            double *nxt = w->seg + (size_t)(t - sb + 1) * SS;
            memcpy(nxt, nxt - SS, sizeof(double) * SS);
            step(p, (size_t)t * H + h, nxt, w->alpha, w->xb);
        }
        for (long t = e - 1; t >= sb; --t) {
            const size_t th = (size_t)t * H + h;
            const double *Sprev = w->seg + (size_t)(t - sb) * SS;
            const double *St = Sprev + SS;
            const double *qt = p->q + th * dk, *kt = p->k + th * dk, *vt = p->v + th * dv;
            const double *dot = p->dO + th * dv;
            const double bt = p->beta[th];
            double *G = w->G;
            /* o_t = S_t q_t */
            for (int j = 0; j < dk; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dv; ++i) acc += St[(size_t)i * dk + j] * dot[i];
                p->dq[th * dk + j] = acc;
            }
            for (int i = 0; i < dv; ++i)
                for (int j = 0; j < dk; ++j) G[(size_t)i * dk + j] += dot[i] * qt[j];
            /* write term beta v k^T */
            double dbeta = 0.0;
            for (int i = 0; i < dv; ++i) {
                double gk = 0.0;
                for (int j = 0; j < dk; ++j) gk += G[(size_t)i * dk + j] * kt[j];
                dbeta += vt[i] * gk;
                p->dv[th * dv + i] = bt * gk;
            }
            for (int j = 0; j < dk; ++j) {
                double gv = 0.0;
                for (int i = 0; i < dv; ++i) gv += G[(size_t)i * dk + j] * vt[i];
                w->tmp[j] = bt * gv; /* dk from the write term */
            }
            /* X = S_{t-1} Diag(alpha), and the rank-one factor */
            gate_of(p, th, w->alpha);
            const double *at = p->a ? p->a + th * dk : kt;
            for (int j = 0; j < dk; ++j) w->bvec[j] = p->b ? p->b[th * dk + j] : bt * kt[j];
            for (int i = 0; i < dv; ++i)
                for (int j = 0; j < dk; ++j)
                    w->X[(size_t)i * dk + j] = Sprev[(size_t)i * dk + j] * w->alpha[j];
            for (int i = 0; i < dv; ++i) {
                double xb = 0.0, ga = 0.0;
                for (int j = 0; j < dk; ++j) {
                    xb += w->X[(size_t)i * dk + j] * w->bvec[j];
                    ga += G[(size_t)i * dk + j] * at[j];
                }
                w->xb[i] = xb;
                w->ga[i] = ga;
            }
            double dbeta_b = 0.0;
            for (int j = 0; j < dk; ++j) {
                double da = 0.0, db = 0.0;
                for (int i = 0; i < dv; ++i) {
                    da -= G[(size_t)i * dk + j] * w->xb[i];
                    db -= w->X[(size_t)i * dk + j] * w->ga[i];
                }
                if (p->a) {
                    p->da[th * dk + j] = da;
                    p->db[th * dk + j] = db;
                    p->dk[th * dk + j] = w->tmp[j];
                } else {
                    p->dk[th * dk + j] = w->tmp[j] + da + bt * db;
                    dbeta_b += kt[j] * db;
                }
            }
            p->dbeta[th] = dbeta + dbeta_b;
            /* dX = G - (G a) b^T; dlog alpha; G <- dX Diag(alpha) */
            double dlh = 0.0;
            for (int j = 0; j < dk; ++j) {
                double dl = 0.0;
                for (int i = 0; i < dv; ++i) {
                    const double dx = G[(size_t)i * dk + j] - w->ga[i] * w->bvec[j];
                    dl += dx * w->X[(size_t)i * dk + j];
                    G[(size_t)i * dk + j] = dx * w->alpha[j];
                }
                if (p->gate == 2) p->dla[th * dk + j] = dl;
                dlh += dl;
            }
            if (p->gate == 1) p->dla[th] = dlh;
        }
    }
    if (p->dS0) memcpy(p->dS0 + ((size_t)n * H + h) * SS, w->G, sizeof(double) * SS);
}

int gdr_ref_bwd(const double *q, const double *k, const double *v, const double *a,
                const double *b, const double *log_alpha, int gate, const double *beta,
                const double *S0, const double *dO, const double *dS_final, double *dq,
                double *dk, double *dv, double *da, double *db, double *dlog_alpha,
                double *dbeta, double *dS0, const int32_t *cu_seqlens, int n_seq, int B, int H,
                int T, int dk_, int dv_, const int32_t *chains, int n_chains, int n_threads) {
    if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta) return -1;
    if ((a == NULL) != (b == NULL) || (a == NULL) != (da == NULL) || (b == NULL) != (db == NULL))
        return -2;
    if (gate < 0 || gate > 2 || (gate != 0 && (!log_alpha || !dlog_alpha))) return -3;
    if (B < 1 || H < 1 || T < 0 || dk_ < 1 || dv_ < 1) return -4;
    if (cu_seqlens && B != 1) return -5;
    const int N = cu_seqlens ? n_seq : B;
    if (N < 1) return -6;
    long max_len = T;
    if (cu_seqlens) {
        if (cu_seqlens[0] < 0 || cu_seqlens[N] > T) return -9;
        max_len = 0;
        for (int i = 0; i < N; ++i) {
            if (cu_seqlens[i + 1] < cu_seqlens[i]) return -9;
            if (cu_seqlens[i + 1] - cu_seqlens[i] > max_len) max_len = cu_seqlens[i + 1] - cu_seqlens[i];
        }
    }
    BwdArgs p = {q, k, v, a, b, log_alpha, beta, S0, dO, dS_final,
                 dq, dk, dv, da, db, dlog_alpha, dbeta, dS0, gate, H, dk_, dv_};
    const long total = chains ? n_chains : (long)N * H;
    const size_t SS = (size_t)dv_ * dk_;
    const long nseg_max = (max_len + kSeg - 1) / kSeg + 1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    int err = 0;
#pragma omp parallel
    {
        Scratch w;
        w.ckpt = (double *)malloc(sizeof(double) * SS * nseg_max);
        w.seg = (double *)malloc(sizeof(double) * SS * (kSeg + 1));
        w.G = (double *)malloc(sizeof(double) * SS);
        w.X = (double *)malloc(sizeof(double) * SS);
        w.alpha = (double *)malloc(sizeof(double) * dk_);
        w.xb = (double *)malloc(sizeof(double) * dv_);
        w.ga = (double *)malloc(sizeof(double) * dv_);
        w.tmp = (double *)malloc(sizeof(double) * dk_);
        w.bvec = (double *)malloc(sizeof(double) * dk_);
        if (!w.ckpt || !w.seg || !w.G || !w.X || !w.alpha || !w.xb || !w.ga || !w.tmp || !w.bvec) {
#pragma omp atomic write
            err = -7;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long c = 0; c < total; ++c) {
                int n, h;
                if (chains) {
                    n = chains[2 * c];
                    h = chains[2 * c + 1];
                } else {
                    n = (int)(c / H);
                    h = (int)(c % H);
                }
                if (n < 0 || n >= N || h < 0 || h >= H) {
#pragma omp atomic write
                    err = -8;
                    continue;
                }
                long t0, t1;
                if (cu_seqlens) {
                    t0 = cu_seqlens[n];
                    t1 = cu_seqlens[n + 1];
                } else {
                    t0 = (long)n * T;
                    t1 = t0 + T;
                }
                run_chain_bwd(&p, n, h, t0, t1, &w);
            }
        }
        free(w.ckpt);
        free(w.seg);
        free(w.G);
        free(w.X);
        free(w.alpha);
        free(w.xb);
        free(w.ga);
        free(w.tmp);
        free(w.bvec);
    }
    return err;
}
