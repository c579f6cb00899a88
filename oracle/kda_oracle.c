/*
 * KDA (Kimi Delta Attention) oracle: a plain fp64 token-by-token recurrence with a
 * hand-derived backward. TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * CPU-baseline leg of the benchmark may call it; the product path never does.
 *
 * Definition (KDA recurrence, as stated for the gated delta rule with per-channel decay;
 * the FlashKDA backward page differentiates its chunk form, in which a chunk's output is
 * O = qd S_in + Mqk U and its outgoing state is diag(e^gam) S_in + kr^T U; FLA
 * chunk_kda_bwd page, driver chunk_kda_bwd):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,   S is K x V
 *   o_t = scale * S_t^T q_t                     (S_t after token t's own write)
 *
 * written in the equivalent residual form used below:
 *   St_t = Diag(exp g_t) S_{t-1};  r_t = v_t - St_t^T k_t;  S_t = St_t + beta_t k_t r_t^T.
 *
 * The backward is the vector-Jacobian product of
 *   L = sum_t <dO_t, o_t> + <dS_final, S_T>
 * with respect to q, k, v, g, beta and h0, derived by hand from the residual form:
 *   Sh  <- grad wrt S_t (starts at dS_final)
 *   Sh += scale q_t dO_t^T;          dq_t += scale S_t dO_t
 *   dbeta_t = k_t^T Sh r_t;          dr = beta_t Sh^T k_t;     dv_t = dr
 *   dk_t += beta_t Sh r_t - St_t dr
 *   Sh  <- Sh - k_t dr^T             (grad wrt St_t)
 *   dg_t = rowsum(Sh o St_t)         (d/dg through St_t = Diag(exp g_t) S_{t-1})
 *   Sh  <- Diag(exp g_t) Sh          (grad wrt S_{t-1})
 * and dh0 = Sh after the first token. Grouped value heads: v-head h reads q/k head
 * h / (HV/H); dq and dk are summed over the v-heads of a group.
 *
 * Varlen: sequences are given by cu_seqlens[0..N]; the state resets to h0[n] at each
 * sequence start. Work is split over (sequence, v-head) tasks run on pthreads; dq and dk
 * are first written per v-head and summed over each group in a fixed order afterwards, so
 * the result does not depend on the thread count.
 *
 * The backward recomputes the forward from checkpoints of S taken every CKPT tokens.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define CKPT 64

typedef struct {
    int N, H, HV, K, V;
    const int64_t* cu;  /* [N+1] */
    double scale;
    const double *q, *k, *v, *g, *beta, *h0, *dO, *dSf;
    double *o, *ST;                      /* forward outputs, nullable */
    double *dq_h, *dk_h;                 /* per-v-head [T][HV][K] scratch, nullable if no bwd */
    double *dv, *dg, *dbeta, *dh0;       /* backward outputs (nullable all => forward only) */
    int do_bwd;
    int next_task;
    pthread_mutex_t mu;
} job_t;

/* one (sequence n, v-head h) task */
static void run_task(job_t* J, int n, int h) {
    const int H = J->H, HV = J->HV, K = J->K, V = J->V;
    const int G = HV / H, hq = h / G;
    const int64_t bos = J->cu[n], eos = J->cu[n + 1];
    const int64_t L = eos - bos;
    const size_t KV = (size_t)K * V;
    double* S = (double*)calloc(KV, sizeof(double));
    double* St = (double*)malloc(KV * sizeof(double));
    double* r = (double*)malloc((size_t)V * sizeof(double));
    const int64_t nseg = (L + CKPT - 1) / CKPT;
    double* ckpt = J->do_bwd ? (double*)malloc((size_t)(nseg > 0 ? nseg : 1) * KV * sizeof(double)) : NULL;
    if (J->h0) memcpy(S, J->h0 + ((size_t)n * HV + h) * KV, KV * sizeof(double));

    /* ---------------- forward ---------------- */
    for (int64_t t = 0; t < L; ++t) {
        const int64_t tt = bos + t;
        if (J->do_bwd && t % CKPT == 0) memcpy(ckpt + (size_t)(t / CKPT) * KV, S, KV * sizeof(double));
        const double* kt = J->k + ((size_t)tt * H + hq) * K;
        const double* qt = J->q + ((size_t)tt * H + hq) * K;
        const double* vt = J->v + ((size_t)tt * HV + h) * V;
        const double* gt = J->g + ((size_t)tt * HV + h) * K;
        const double bt = J->beta[(size_t)tt * HV + h];
        for (int i = 0; i < K; ++i) {
            const double a = exp(gt[i]);
            for (int j = 0; j < V; ++j) St[(size_t)i * V + j] = a * S[(size_t)i * V + j];
        }
        for (int j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int i = 0; i < K; ++i) acc += St[(size_t)i * V + j] * kt[i];
            r[j] = vt[j] - acc;
        }
        for (int i = 0; i < K; ++i)
            for (int j = 0; j < V; ++j) S[(size_t)i * V + j] = St[(size_t)i * V + j] + bt * kt[i] * r[j];
        if (J->o) {
            double* ot = J->o + ((size_t)tt * HV + h) * V;
            for (int j = 0; j < V; ++j) {
                double acc = 0.0;
                for (int i = 0; i < K; ++i) acc += S[(size_t)i * V + j] * qt[i];
                ot[j] = J->scale * acc;
            }
        }
    }
    if (J->ST) memcpy(J->ST + ((size_t)n * HV + h) * KV, S, KV * sizeof(double));

    /* ---------------- backward ---------------- */
    if (J->do_bwd) {
        double* Sh = (double*)calloc(KV, sizeof(double));
        double* Sprev = (double*)malloc((size_t)CKPT * KV * sizeof(double)); /* S_{t-1} per token of a segment */
        double* Scur = (double*)malloc(KV * sizeof(double));
        double* dr = (double*)malloc((size_t)V * sizeof(double));
        double* tmpK = (double*)malloc((size_t)K * sizeof(double));
        if (J->dSf) memcpy(Sh, J->dSf + ((size_t)n * HV + h) * KV, KV * sizeof(double));
        for (int64_t sg = nseg - 1; sg >= 0; --sg) {
            const int64_t t0 = sg * CKPT;
            const int64_t t1 = (t0 + CKPT < L) ? t0 + CKPT : L;
            /* recompute S_{t-1} for every token of the segment */
            memcpy(Scur, ckpt + (size_t)sg * KV, KV * sizeof(double));
            for (int64_t t = t0; t < t1; ++t) {
                memcpy(Sprev + (size_t)(t - t0) * KV, Scur, KV * sizeof(double));
                const int64_t tt = bos + t;
                const double* kt = J->k + ((size_t)tt * H + hq) * K;
                const double* vt = J->v + ((size_t)tt * HV + h) * V;
                const double* gt = J->g + ((size_t)tt * HV + h) * K;
                const double bt = J->beta[(size_t)tt * HV + h];
                for (int i = 0; i < K; ++i) {
                    const double a = exp(gt[i]);
                    for (int j = 0; j < V; ++j) St[(size_t)i * V + j] = a * Scur[(size_t)i * V + j];
                }
                for (int j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < K; ++i) acc += St[(size_t)i * V + j] * kt[i];
                    r[j] = vt[j] - acc;
                }
                for (int i = 0; i < K; ++i)
                    for (int j = 0; j < V; ++j) Scur[(size_t)i * V + j] = St[(size_t)i * V + j] + bt * kt[i] * r[j];
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t tt = bos + t;
                const double* Sp = Sprev + (size_t)(t - t0) * KV;
                const double* kt = J->k + ((size_t)tt * H + hq) * K;
                const double* qt = J->q + ((size_t)tt * H + hq) * K;
                const double* vt = J->v + ((size_t)tt * HV + h) * V;
                const double* gt = J->g + ((size_t)tt * HV + h) * K;
                const double* dot = J->dO + ((size_t)tt * HV + h) * V;
                const double bt = J->beta[(size_t)tt * HV + h];
                /* St_t, r_t, S_t */
                for (int i = 0; i < K; ++i) {
                    const double a = exp(gt[i]);
                    for (int j = 0; j < V; ++j) St[(size_t)i * V + j] = a * Sp[(size_t)i * V + j];
                }
                for (int j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < K; ++i) acc += St[(size_t)i * V + j] * kt[i];
                    r[j] = vt[j] - acc;
                }
                for (int i = 0; i < K; ++i)
                    for (int j = 0; j < V; ++j) Scur[(size_t)i * V + j] = St[(size_t)i * V + j] + bt * kt[i] * r[j];
                /* output o_t = scale S_t^T q_t */
                double* dqt = J->dq_h + ((size_t)tt * HV + h) * K;
                for (int i = 0; i < K; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < V; ++j) {
                        Sh[(size_t)i * V + j] += J->scale * qt[i] * dot[j];
                        acc += Scur[(size_t)i * V + j] * dot[j];
                    }
                    dqt[i] = J->scale * acc;
                }
                /* write beta_t k_t r_t^T */
                double db = 0.0;
                for (int i = 0; i < K; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < V; ++j) acc += Sh[(size_t)i * V + j] * r[j];
                    tmpK[i] = acc; /* (Sh r)_i */
                    db += kt[i] * acc;
                }
                J->dbeta[(size_t)tt * HV + h] = db;
                for (int j = 0; j < V; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < K; ++i) acc += Sh[(size_t)i * V + j] * kt[i];
                    dr[j] = bt * acc;
                }
                double* dvt = J->dv + ((size_t)tt * HV + h) * V;
                for (int j = 0; j < V; ++j) dvt[j] = dr[j];
                double* dkt = J->dk_h + ((size_t)tt * HV + h) * K;
                for (int i = 0; i < K; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < V; ++j) acc += St[(size_t)i * V + j] * dr[j];
                    dkt[i] = bt * tmpK[i] - acc;
                }
                /* residual r = v - St^T k: grad into St, then through the decay */
                double* dgt = J->dg + ((size_t)tt * HV + h) * K;
                for (int i = 0; i < K; ++i) {
                    const double a = exp(gt[i]);
                    double acc = 0.0;
                    for (int j = 0; j < V; ++j) {
                        const double s = Sh[(size_t)i * V + j] - kt[i] * dr[j];
                        acc += s * St[(size_t)i * V + j];
                        Sh[(size_t)i * V + j] = a * s;
                    }
                    dgt[i] = acc;
                }
            }
        }
        if (J->dh0) memcpy(J->dh0 + ((size_t)n * HV + h) * KV, Sh, KV * sizeof(double));
        free(Sh); free(Sprev); free(Scur); free(dr); free(tmpK);
    }
    free(S); free(St); free(r); free(ckpt);
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int ntask = J->N * J->HV;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int t = J->next_task++;
        pthread_mutex_unlock(&J->mu);
        if (t >= ntask) break;
        run_task(J, t / J->HV, t % J->HV);
    }
    return NULL;
}

/*
 * Forward and (optionally) backward over packed sequences.
 * Layouts (row-major, fp64): q,k [T][H][K]; v,dO [T][HV][V]; g [T][HV][K]; beta [T][HV];
 * h0,dS_final,S_T,dh0 [N][HV][K][V]; o,dv [T][HV][V]; dq,dk [T][H][K]; dg [T][HV][K];
 * dbeta [T][HV]. h0 and dS_final may be NULL (zero). With dq == NULL only the forward
 * runs. nthreads <= 0 uses every online core. Returns the number of threads used, or a
 * negative value on bad arguments.
 */
int kda_oracle_run(int N, const int64_t* cu_seqlens, int H, int HV, int K, int V, double scale,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* h0, const double* dO, const double* dS_final,
                   double* o, double* S_T,
                   double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dh0,
                   int nthreads) {
    if (N <= 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0 || !cu_seqlens) return -1;
    if (!q || !k || !v || !g || !beta) return -1;
    const int64_t T = cu_seqlens[N];
    for (int n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.N = N; J.H = H; J.HV = HV; J.K = K; J.V = V; J.cu = cu_seqlens; J.scale = scale;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.dO = dO; J.dSf = dS_final;
    J.o = o; J.ST = S_T;
    J.do_bwd = dq != NULL;
    if (J.do_bwd) {
        if (!dO || !dk || !dv || !dg || !dbeta) return -1;
        J.dq_h = (double*)calloc((size_t)T * HV * K + 1, sizeof(double));
        J.dk_h = (double*)calloc((size_t)T * HV * K + 1, sizeof(double));
        J.dv = dv; J.dg = dg; J.dbeta = dbeta; J.dh0 = dh0;
    }
    pthread_mutex_init(&J.mu, NULL);
    int nt = nthreads > 0 ? nthreads : (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nt < 1) nt = 1;
    if (nt > N * HV) nt = N * HV;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    for (int i = 0; i < nt; ++i) pthread_create(&th[i], NULL, worker, &J);
    for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    if (J.do_bwd) {
        const int G = HV / H;
        for (int64_t t = 0; t < T; ++t)
            for (int hq = 0; hq < H; ++hq)
                for (int i = 0; i < K; ++i) {
                    double aq = 0.0, ak = 0.0;
                    for (int e = 0; e < G; ++e) {
                        const size_t idx = ((size_t)t * HV + (size_t)hq * G + e) * K + i;
                        aq += J.dq_h[idx];
                        ak += J.dk_h[idx];
                    }
                    dq[((size_t)t * H + hq) * K + i] = aq;
                    dk[((size_t)t * H + hq) * K + i] = ak;
                }
        free(J.dq_h); free(J.dk_h);
    }
    return nt;
}
