/*
 * Oracle (test infrastructure only) -- token-by-token fp64 recurrence of the
 * gated delta rule, for scalar (GDN) and per-channel (KDA) log-gates.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code with the HIP library.
 *
 * What it computes, per sequence n, value head h (query/key head
 * h / (H_v / H_qk)) and value column c (columns of the state are independent):
 *
 *   S <- h0[n, h]            (or 0)                       state is [D_k, D_v]
 *   for each token t of the sequence:
 *     scalar gate:  S <- exp(g_t) * S
 *     channel gate: S[i, :] <- exp(gk_{t,i}) * S[i, :]
 *     r <- S^T k_t                      (what k_t currently reads out)
 *     S <- S + beta_t * k_t (v_t - r)^T (erase the old association, write the new)
 *     o_t <- scale * S^T q_t            (output after the same token's update)
 *   final[n, h] <- S
 *
 * i.e. S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T and
 * o_t = scale * S_t^T q_t.  Sources: FlashQLA announcement (Qwen), section
 * "further optimisation through gate decay", the GDN recurrence (transposed
 * here to the [D_k, D_v] state layout); 06 . Flash Linear Attention, section 8
 * (fused_recurrent): the token loop updates the state first and then reads
 * o = S^T q.  For per-channel gates the decay is applied before the read and
 * the erase (reading of the KDA source walk-through, section 3.3: w uses
 * k * exp(gk) with gk inclusive of the current token).
 *
 * Layouts (row-major, all fp64):
 *   q, k   [T_total, H_qk, D_k]      v, o [T_total, H_v, D_v]
 *   g      [T_total, H_v]            (gate_kind 0)
 *   gk     [T_total, H_v, D_k]       (gate_kind 1)
 *   beta   [T_total, H_v]
 *   h0, final [N, H_v, D_k, D_v]     (h0 may be NULL: zero state)
 *   cu     [N + 1] token offsets, cu[0] = 0, non-decreasing
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define COLS 16 /* value columns per work unit */

typedef struct {
    int N, H_qk, H_v, Dk, Dv, gate_kind;
    const int64_t *cu;
    const double *q, *k, *v, *g, *beta, *h0;
    double scale;
    double *o, *final_state;
    int64_t n_units;
    int64_t next_unit; /* shared counter, protected by mu */
    pthread_mutex_t mu;
} job_t;

static void run_unit(job_t *J, int64_t u, double *S) {
    const int nvb = (J->Dv + COLS - 1) / COLS;
    const int vb = (int)(u % nvb);
    const int h = (int)((u / nvb) % J->H_v);
    const int n = (int)(u / ((int64_t)nvb * J->H_v));
    const int c0 = vb * COLS;
    const int nc = (J->Dv - c0) < COLS ? (J->Dv - c0) : COLS;
    const int hq = h / (J->H_v / J->H_qk);
    const int Dk = J->Dk, Dv = J->Dv;

    for (int i = 0; i < Dk; i++)
        for (int c = 0; c < nc; c++)
            S[i * COLS + c] = J->h0 ? J->h0[(((int64_t)n * J->H_v + h) * Dk + i) * Dv + c0 + c] : 0.0;

    double r[COLS];
    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; t++) {
        const double *qt = J->q + (t * J->H_qk + hq) * Dk;
        const double *kt = J->k + (t * J->H_qk + hq) * Dk;
        const double *vt = J->v + (t * J->H_v + h) * Dv + c0;
        const double bt = J->beta[t * J->H_v + h];
        /* decay */
        if (J->gate_kind == 0) {
            const double a = exp(J->g[t * J->H_v + h]);
            for (int i = 0; i < Dk; i++)
                for (int c = 0; c < nc; c++) S[i * COLS + c] *= a;
        } else {
            const double *gkt = J->g + (t * J->H_v + h) * Dk;
            for (int i = 0; i < Dk; i++) {
                const double a = exp(gkt[i]);
                for (int c = 0; c < nc; c++) S[i * COLS + c] *= a;
            }
        }
        /* read: r = S^T k */
        for (int c = 0; c < nc; c++) r[c] = 0.0;
        for (int i = 0; i < Dk; i++)
            for (int c = 0; c < nc; c++) r[c] += S[i * COLS + c] * kt[i];
        /* erase + write: S += beta k (v - r)^T */
        for (int c = 0; c < nc; c++) r[c] = bt * (vt[c] - r[c]);
        for (int i = 0; i < Dk; i++)
            for (int c = 0; c < nc; c++) S[i * COLS + c] += kt[i] * r[c];
        /* output: o = scale S^T q */
        double *ot = J->o + (t * J->H_v + h) * Dv + c0;
        for (int c = 0; c < nc; c++) ot[c] = 0.0;
        for (int i = 0; i < Dk; i++)
            for (int c = 0; c < nc; c++) ot[c] += S[i * COLS + c] * qt[i];
        for (int c = 0; c < nc; c++) ot[c] *= J->scale;
    }
    if (J->final_state)
        for (int i = 0; i < Dk; i++)
            for (int c = 0; c < nc; c++)
                J->final_state[(((int64_t)n * J->H_v + h) * Dk + i) * Dv + c0 + c] = S[i * COLS + c];
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)J->Dk * COLS);
    if (!S) return NULL;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t u = J->next_unit++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->n_units) break;
        run_unit(J, u, S);
    }
    free(S);
    return NULL;
}

/* Returns 0 on success, -1 on a bad argument, -2 if threads could not start. */
int oracle_gdn_recurrent(int N, const int64_t *cu, int H_qk, int H_v, int Dk, int Dv, int gate_kind,
                         const double *q, const double *k, const double *v, const double *g,
                         const double *beta, double scale, const double *h0, double *o,
                         double *final_state, int n_threads) {
    if (N < 0 || !cu || H_qk <= 0 || H_v <= 0 || H_v % H_qk || Dk <= 0 || Dv <= 0) return -1;
    if (gate_kind != 0 && gate_kind != 1) return -1;
    for (int n = 0; n < N; n++)
        if (cu[n + 1] < cu[n]) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.N = N; J.H_qk = H_qk; J.H_v = H_v; J.Dk = Dk; J.Dv = Dv; J.gate_kind = gate_kind;
    J.cu = cu; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.scale = scale; J.o = o; J.final_state = final_state;
    J.n_units = (int64_t)N * H_v * ((Dv + COLS - 1) / COLS);
    pthread_mutex_init(&J.mu, NULL);
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 0; i < n_threads; i++) {
        if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
        started++;
    }
    if (started == 0) worker(&J); /* run inline */
    for (int i = 0; i < started; i++) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    return (J.next_unit >= J.n_units) ? 0 : -2;
}
