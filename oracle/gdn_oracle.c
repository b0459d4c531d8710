/*
 * gdn_oracle.c -- fp64 CPU oracle for the gated delta rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP library is checked against.  It shares no code, header, table or helper
 * with the GPU path, and the GPU path never links or calls it.  Only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark load it.
 *
 * What it computes (the plain definition, one token at a time, in fp64):
 *
 *   The gated delta rule keeps a state S_t (V x K) per (batch, head) and
 *   updates it as  S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T)
 *                        + beta_t v_t k_t^T,     o_t = S_t q_t,
 *   with a_t = exp(g_t).  For Gated DeltaNet g_t is one scalar per (token,
 *   head) and Diag(a_t) = a_t I; for Kimi-Delta-Attention g_t is a K-vector
 *   and the decay acts on the key index of S.
 *   (Recurrence as stated for the Gated DeltaNet / KDA forward; the per-key
 *   decay placement follows the KDA re-scan page, kernel_fun bwd_scan.py, whose
 *   per-chunk state update multiplies the rows of h = S^T by a K-vector of
 *   gate factors: docstring "h = exp2(gd) * h + DH" and the SIMT recurrence.)
 *
 *   Expanding the product gives the "predict and correct" step used below:
 *     S'  = S_{t-1} Diag(a_t)            (decay first)
 *     e   = v_t - S' k_t                 (prediction error)
 *     S_t = S' + beta_t e k_t^T          (delta correction)
 *     o_t = S_t q_t                      (read-out with the updated state)
 *
 *   The state is held as h = S^T (K x V), the layout [B,H,K,V] that the KDA
 *   re-scan page uses for h0 ("h0: (K, V, HV, B) fp32").
 *
 * Inputs are fp32 arrays holding exactly the values the GPU receives (bf16
 * values widen to fp32 exactly); everything is upcast to fp64 here, so the
 * oracle adds only fp64 rounding.
 *
 * Layouts (dense, row-major): q,k [B,T,H,K]; v [B,T,H,V]; beta [B,T,H];
 * g [B,T,H] (scalar gate) or [B,T,H,K] (per-key gate); h0 [B,H,K,V] or NULL.
 * Outputs are head-major for the selected heads: o [n][T][V], hT [n][K][V],
 * where head n is sel[n] = b*H + h (or every head in order when sel == NULL).
 *
 * Saved states (gdn_oracle_states_f64), what a backward pass re-reads (the
 * KDA re-scan page's h checkpoints and v_new):
 *   hck  [n][NT][K][V]  h at the start of each chunk of C tokens, before the
 *                       chunk's first token is applied (NT = ceil(T / C))
 *   vnew [n][T][V]      the delta written into the state at token t,
 *                       beta_t * e_t with e the prediction error above: the
 *                       state update is h <- Diag(a_t) h + k_t vnew_t^T
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, T, H, K, V;
    int gate_per_key;          /* 0: g[B,T,H]; 1: g[B,T,H,K] */
    const float *q, *k, *v, *beta, *g, *h0;
    int64_t n_sel;
    const int64_t *sel;        /* NULL: all B*H heads */
    double *o;                 /* [n_sel][T][V], may be NULL */
    double *hT;                /* [n_sel][K][V], may be NULL */
    int64_t chunk;             /* C of the checkpoints (>= 1 when hck is set) */
    double *hck;               /* [n_sel][NT][K][V], may be NULL */
    double *vnew;              /* [n_sel][T][V], may be NULL */
} oracle_job;

/* One (batch, head) pair, token by token. */
static void run_head(const oracle_job *J, int64_t n, double *h, double *kk,
                     double *qq, double *e, double *a) {
    const int64_t T = J->T, H = J->H, K = J->K, V = J->V;
    const int64_t bh = J->sel ? J->sel[n] : n;
    const int64_t b = bh / H, hd = bh % H;

    if (J->h0) {
        const float *src = J->h0 + bh * K * V;
        for (int64_t i = 0; i < K * V; ++i) h[i] = (double)src[i];
    } else {
        memset(h, 0, sizeof(double) * (size_t)(K * V));
    }

    const int64_t NT = J->hck ? (T + J->chunk - 1) / J->chunk : 0;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t row = (b * T + t) * H + hd;      /* token-head index */
        if (J->hck && t % J->chunk == 0)
            memcpy(J->hck + (n * NT + t / J->chunk) * K * V, h, sizeof(double) * (size_t)(K * V));
        const float *qt = J->q + row * K;
        const float *kt = J->k + row * K;
        const float *vt = J->v + row * V;
        const double bt = (double)J->beta[row];
        for (int64_t d = 0; d < K; ++d) {
            kk[d] = (double)kt[d];
            qq[d] = (double)qt[d];
        }
        if (J->gate_per_key) {
            const float *gt = J->g + row * K;
            for (int64_t d = 0; d < K; ++d) a[d] = exp((double)gt[d]);
        } else {
            const double at = exp((double)J->g[row]);
            for (int64_t d = 0; d < K; ++d) a[d] = at;
        }

        /* S' = S Diag(a): row d of h scales by a_d;  e = v - S' k. */
        for (int64_t j = 0; j < V; ++j) e[j] = (double)vt[j];
        for (int64_t d = 0; d < K; ++d) {
            double *hr = h + d * V;
            const double ad = a[d], kd = kk[d];
            for (int64_t j = 0; j < V; ++j) {
                hr[j] *= ad;
                e[j] -= hr[j] * kd;
            }
        }
        if (J->vnew) {
            double *vn = J->vnew + (n * T + t) * V;
            for (int64_t j = 0; j < V; ++j) vn[j] = bt * e[j];
        }
        /* S = S' + beta e k^T;  o = S q. */
        double *ot = J->o ? J->o + (n * T + t) * V : NULL;
        if (ot) memset(ot, 0, sizeof(double) * (size_t)V);
        for (int64_t d = 0; d < K; ++d) {
            double *hr = h + d * V;
            const double bk = bt * kk[d], qd = qq[d];
            for (int64_t j = 0; j < V; ++j) {
                hr[j] += bk * e[j];
                if (ot) ot[j] += hr[j] * qd;
            }
        }
    }
    if (J->hT) memcpy(J->hT + n * K * V, h, sizeof(double) * (size_t)(K * V));
}

typedef struct {
    const oracle_job *J;
    int64_t first, stride;
    int err;
    int joined;                /* 1 when a thread was started for it */
} worker_arg;

static void *worker(void *p) {
    worker_arg *w = (worker_arg *)p;
    const oracle_job *J = w->J;
    const int64_t K = J->K, V = J->V;
    double *h = (double *)malloc(sizeof(double) * (size_t)(K * V));
    double *kk = (double *)malloc(sizeof(double) * (size_t)K);
    double *qq = (double *)malloc(sizeof(double) * (size_t)K);
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    double *a = (double *)malloc(sizeof(double) * (size_t)K);
    if (!h || !kk || !qq || !e || !a) {
        w->err = 1;
    } else {
        for (int64_t n = w->first; n < J->n_sel; n += w->stride)
            run_head(J, n, h, kk, qq, e, a);
    }
    free(h); free(kk); free(qq); free(e); free(a);
    return NULL;
}

/*
 * Entry points.  Return 0 on success, nonzero on a bad argument or an
 * allocation failure.  nthreads <= 0 means one thread.
 */
int gdn_oracle_states_f64(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                          int gate_per_key, const float *q, const float *k,
                          const float *v, const float *beta, const float *g,
                          const float *h0, int64_t n_sel, const int64_t *sel,
                          double *o, double *hT, int64_t chunk, double *hck,
                          double *vnew, int nthreads) {
    if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1) return 1;
    if (!q || !k || !v || !beta || !g) return 1;
    if (hck && chunk < 1) return 1;
    if (!sel) n_sel = B * H;
    for (int64_t n = 0; sel && n < n_sel; ++n)
        if (sel[n] < 0 || sel[n] >= B * H) return 1;
    oracle_job J = {B, T, H, K, V, gate_per_key, q, k, v, beta, g, h0,
                    n_sel, sel, o, hT, chunk, hck, vnew};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_sel) nthreads = (int)(n_sel > 0 ? n_sel : 1);
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    worker_arg *args = (worker_arg *)calloc((size_t)nthreads, sizeof(worker_arg));
    if (!tid || !args) { free(tid); free(args); return 2; }
    int err = 0;
    for (int i = 0; i < nthreads; ++i) {
        args[i].J = &J; args[i].first = i; args[i].stride = nthreads;
        args[i].err = 0;
        args[i].joined = pthread_create(&tid[i], NULL, worker, &args[i]) == 0;
        if (!args[i].joined) worker(&args[i]);   /* run it on this thread */
    }
    for (int i = 0; i < nthreads; ++i) {
        if (args[i].joined) pthread_join(tid[i], NULL);
        if (args[i].err) err = 2;
    }
    free(tid); free(args);
    return err;
}

int gdn_oracle_f64(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                   int gate_per_key, const float *q, const float *k,
                   const float *v, const float *beta, const float *g,
                   const float *h0, int64_t n_sel, const int64_t *sel,
                   double *o, double *hT, int nthreads) {
    return gdn_oracle_states_f64(B, T, H, K, V, gate_per_key, q, k, v, beta, g, h0,
                                 n_sel, sel, o, hT, 0, NULL, NULL, nthreads);
}
