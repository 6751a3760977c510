/*
 * Oracle for the gated delta-rule forward pass: a plain fp64 token-by-token
 * recurrence on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or constant with the GPU library.
 *
 * What it computes (per sequence n and head h), following the gated DPLR
 * recurrence of "Diagonal Plus Low Rank" (section 2, the original formula):
 *
 *     S   = S0[n,h]  (dv x dk; zero when S0 is NULL)
 *     for each token t of the sequence, in order:
 *         alpha = exp(log_alpha[t,h,:])  (channel gate)
 *               | exp(log_alpha[t,h]) * 1 (head gate)  | 1 (no gate)
 *         (a,b) = (a_t, b_t) if given, else (k_t, beta_t k_t)
 *         X     = S Diag(alpha)                  -- gate first ...
 *         S     = X - (X b) a^T + beta_t v_t k_t^T   -- ... then I - b a^T
 *         O[t]  = S q_t                          -- output uses the updated S
 *     S_final[n,h] = S
 *
 * The default (a, b) = (k, beta k) with the write scaled by beta is the KDA
 * special case given in the same notes ("relation to KDA": a = k, b = beta k,
 * v = beta v'); with a head gate it is Gated DeltaNet and with no gate it is
 * DeltaNet ("DeltaNet" notes, section 4.1, S_t = S_{t-1}(I - beta k k^T) +
 * beta v k^T).  When a and b are given, beta still scales the write term, as
 * in the GDN2 form (eq. 1 of "How to make GDN2 more stable"); passing
 * beta = 1 recovers the unscaled DPLR formula.
 *
 * clip != 0 adds the spectral clipping of the forget gate from "How to make
 * GDN2 more stable" (eq. 7): per token, rho = ||I - b_t a_t^T||_2 and the gate
 * becomes alpha = min(alpha, 1/rho) channel by channel before it is applied, so
 * that ||Diag(alpha)(I - b a^T)||_2 <= 1.  rho has the closed form of eq. 4;
 * vectors of any length are reduced to that unit-vector form by moving their
 * norms into eta (the page's remark under eq. 4).  With no gate alpha = 1 is
 * clipped like any other gate, giving alpha = 1/rho.
 *
 * Layouts (row-major, contiguous): tokens are the flattened [B*T] axis.
 *   q, k, a, b : [tokens, H, dk]      v : [tokens, H, dv]
 *   log_alpha  : [tokens, H] (gate 1) or [tokens, H, dk] (gate 2); unused for 0
 *   beta       : [tokens, H]
 *   S0, S_final: [N, H, dv, dk]       O : [tokens, H, dv]
 * Sequences: without cu_seqlens, sequence n is tokens [n*T, (n+1)*T), N = B;
 * with cu_seqlens (B must be 1), sequence n is [cu[n], cu[n+1]), N = n_seq.
 * chains/n_chains: optional list of (n, h) pairs (2*n_chains int32) to compute;
 * NULL computes every pair.  Returns 0, or a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ||I - b a^T||_2 for vectors a, b of length d ("How to make GDN2 more stable",
 * eq. 4): with eta = |b| |a| and c the cosine between b and a, that is the
 * norm of I - eta u w^T for unit u, w, namely (eta + sqrt(eta^2 - 4 eta c + 4)) / 2.
 * eta c = b.a, and eta^2 - 4 eta c + 4 >= (eta - 2)^2 >= 0 (the max() only
 * absorbs rounding). */
static double rank1_spectral_norm(const double *a, const double *b, int d) {
    double aa = 0.0, bb = 0.0, ab = 0.0;
    for (int j = 0; j < d; ++j) {
        aa += a[j] * a[j];
        bb += b[j] * b[j];
        ab += a[j] * b[j];
    }
    const double eta = sqrt(aa) * sqrt(bb);
    const double disc = eta * eta - 4.0 * ab + 4.0;
    return 0.5 * (eta + sqrt(disc > 0.0 ? disc : 0.0));
}

static void run_chain(int n, int h, const double *q, const double *k, const double *v,
                      const double *a, const double *b, const double *log_alpha, int gate,
                      int clip, const double *beta, const double *S0, double *O, double *S_final,
                      long t0, long t1, int H, int dk, int dv, double *S, double *alpha,
                      double *xb, double *bk) {
    if (S0)
        memcpy(S, S0 + ((size_t)n * H + h) * dv * dk, sizeof(double) * dv * dk);
    else
        memset(S, 0, sizeof(double) * dv * dk);
    for (long t = t0; t < t1; ++t) {
        const size_t th = (size_t)t * H + h;
        const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv;
        const double bt = beta[th];
        /* the gate alpha_t, one value per key channel */
        for (int j = 0; j < dk; ++j) {
            if (gate == 2) alpha[j] = exp(log_alpha[th * dk + j]);
            else if (gate == 1) alpha[j] = exp(log_alpha[th]);
            else alpha[j] = 1.0;
        }
        /* spectral clipping: alpha = min(alpha, 1 / ||I - b a^T||_2) */
        if (clip) {
            const double *a_t = a ? a + th * dk : kt;
            const double *b_t = bk;
            if (b) b_t = b + th * dk;
            else for (int j = 0; j < dk; ++j) bk[j] = bt * kt[j];
            const double inv_rho = 1.0 / rank1_spectral_norm(a_t, b_t, dk);
            for (int j = 0; j < dk; ++j)
                if (alpha[j] > inv_rho) alpha[j] = inv_rho;
        }
        /* X = S Diag(alpha): scale column j of S by alpha_j */
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j) S[(size_t)i * dk + j] *= alpha[j];
        /* S = X - (X b) a^T + beta v k^T */
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) {
                const double bj = b ? b[th * dk + j] : bt * kt[j];
                acc += S[(size_t)i * dk + j] * bj;
            }
            xb[i] = acc;
        }
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j) {
                const double aj = a ? a[th * dk + j] : kt[j];
                S[(size_t)i * dk + j] += -xb[i] * aj + bt * vt[i] * kt[j];
            }
        /* o_t = S_t q_t */
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * qt[j];
            O[th * dv + i] = acc;
        }
    }
    if (S_final)
        memcpy(S_final + ((size_t)n * H + h) * dv * dk, S, sizeof(double) * dv * dk);
}

int gdr_ref_fwd(const double *q, const double *k, const double *v, const double *a,
                const double *b, const double *log_alpha, int gate, int clip, const double *beta,
                const double *S0, double *O, double *S_final, const int32_t *cu_seqlens,
                int n_seq, int B, int H, int T, int dk, int dv, const int32_t *chains,
                int n_chains, int n_threads) {
    if (!q || !k || !v || !beta || !O) return -1;
    if ((a == NULL) != (b == NULL)) return -2;
    if (gate < 0 || gate > 2 || (gate != 0 && !log_alpha)) return -3;
    if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return -4;
    if (cu_seqlens && B != 1) return -5;
    const int N = cu_seqlens ? n_seq : B;
    if (N < 1) return -6;
    if (cu_seqlens) {
        if (cu_seqlens[0] < 0 || cu_seqlens[N] > T) return -9;
        for (int i = 0; i < N; ++i)
            if (cu_seqlens[i + 1] < cu_seqlens[i]) return -9;
    }
    const long total = chains ? n_chains : (long)N * H;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    int err = 0;
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *xb = (double *)malloc(sizeof(double) * (size_t)dv);
        double *bk = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!S || !alpha || !xb || !bk) {
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
                run_chain(n, h, q, k, v, a, b, log_alpha, gate, clip, beta, S0, O, S_final, t0,
                          t1, H, dk, dv, S, alpha, xb, bk);
            }
        }
        free(S);
        free(alpha);
        free(xb);
        free(bk);
    }
    return err;
}

int gdr_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
