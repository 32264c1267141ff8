/*
 * kda_oracle.c -- plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The product path (the HIP
 * library under gated_delta_rule_chunkwise_amd/) never links, loads or calls
 * it, and this file shares no code, header or table with that path.
 *
 * What it computes (one independent chain per (sequence, head)):
 *
 *   KimiLinear article (intl.cloud.baidu.com), section 2.3 "KDA's
 *   Fine-Grained Gating Design": the state is decayed by a per-dimension gate
 *   vector a_t that acts on the rows of the state (one forgetting rate per key
 *   feature), then corrected by the delta rule of section 2.1 with strength
 *   beta_t.  Section 2.1 gives the delta-rule erase and write with the same
 *   scalar beta_t.  The pages print the write term as v k^T, which only type-
 *   checks with the identity operator on the left when d_k = d_v; with the gate
 *   on rows the state is d_k x d_v and the write term is k v^T (reading of the
 *   garbled orientation).  The read-out is not on the pages; the reading taken
 *   is o_t = S_t^T q_t, inclusive of token t, with no scale.
 *
 *   Per token, in this order:
 *       S <- Diag(exp(log_alpha_t)) S                     (decay first)
 *       S <- S - b_t k_t (k_t^T S) + w_t k_t v_t^T         (erase, write)
 *       o_t <- S^T q_t
 *   KDA is b_t = w_t = beta_t.  The generalised form with separate erase and
 *   write strengths (b_t, w_t) is the decoupled-gate variant that the Kimi
 *   Linear CoChat record quotes from citing papers ("Claims other papers make
 *   about this one").  It is the reference of the separate-strength entry
 *   points (forward and backward), and with b = 0, w = 1, a = 1 it gives the
 *   pure linear-attention form of section 2.1 exactly, which a pin checks.
 *
 * Everything is fp64, with plain loops and no BLAS, no blocking and no
 * reordering beyond the three steps above.  Chains run in parallel threads;
 * each chain is computed by exactly one thread, so the result does not depend
 * on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Layouts (all row-major, contiguous):
 *   q, k, log_alpha : [T_total, H, dk]
 *   v               : [T_total, H, dv]
 *   b_erase, w_write: [T_total, H]
 *   h0, hT          : [N, H, dk, dv]   (h0 may be NULL: zero initial state)
 *   o               : [T_total, H, dv]
 *   cu_seqlens      : [N + 1], cu_seqlens[0] = 0, non-decreasing
 */
typedef struct {
    const double *q, *k, *v, *log_alpha, *b_erase, *w_write, *h0;
    const int64_t *cu_seqlens;
    int64_t num_seqs, H, dk, dv;
    double *o, *hT;
    int64_t next_chain;           /* shared work counter, guarded by mu */
    pthread_mutex_t mu;
    int failed;
} oracle_job;

/* Runs one (sequence, head) chain token by token. Returns 0 or -1 (no memory). */
static int run_chain(const oracle_job *J, int64_t n, int64_t h)
{
    const int64_t H = J->H, dk = J->dk, dv = J->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !kS) { free(S); free(kS); return -1; }

    if (J->h0) memcpy(S, J->h0 + (n * H + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
    else memset(S, 0, sizeof(double) * (size_t)(dk * dv));

    for (int64_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
        const double *qt = J->q + (t * H + h) * dk;
        const double *kt = J->k + (t * H + h) * dk;
        const double *vt = J->v + (t * H + h) * dv;
        const double *lat = J->log_alpha + (t * H + h) * dk;
        const double bt = J->b_erase[t * H + h];
        const double wt = J->w_write[t * H + h];

        /* decay: row c of S is scaled by a_t[c] = exp(log_alpha_t[c]) */
        for (int64_t c = 0; c < dk; ++c) {
            const double a = exp(lat[c]);
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
        }
        /* erase and write: S += k (w v - b k^T S)^T */
        for (int64_t j = 0; j < dv; ++j) kS[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) kS[j] += kt[c] * S[c * dv + j];
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kt[c] * (wt * vt[j] - bt * kS[j]);
        /* read-out: o_t = S^T q_t */
        double *ot = J->o + (t * H + h) * dv;
        for (int64_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < dk; ++c) acc += qt[c] * S[c * dv + j];
            ot[j] = acc;
        }
    }
    if (J->hT) memcpy(J->hT + (n * H + h) * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
    free(S);
    free(kS);
    return 0;
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    const int64_t total = J->num_seqs * J->H;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t id = J->next_chain++;
        pthread_mutex_unlock(&J->mu);
        if (id >= total) break;
        if (run_chain(J, id / J->H, id % J->H) != 0) {
            pthread_mutex_lock(&J->mu);
            J->failed = 1;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

static int run_all(oracle_job *J, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    pthread_mutex_init(&J->mu, NULL);
    J->next_chain = 0;
    J->failed = 0;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) return -1;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, J) != 0) break;
        ++started;
    }
    if (started == 0) worker(J); /* no thread could start: run inline */
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&J->mu);
    return J->failed ? -1 : 0;
}

static int check_seqlens(const int64_t *cu, int64_t N)
{
    if (!cu || N < 0) return -2;
    if (cu[0] != 0) return -2;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -2;
    return 0;
}

/* Generalised recurrence (separate erase strength b and write strength w).
 * Returns 0 on success, -1 on allocation failure, -2 on bad arguments. */
int kda_oracle_gen_fwd(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *b_erase,
                       const double *w_write, const double *h0,
                       const int64_t *cu_seqlens, int64_t num_seqs, int64_t H,
                       int64_t dk, int64_t dv, double *o, double *hT,
                       int nthreads)
{
    if (H <= 0 || dk <= 0 || dv <= 0) return -2;
    if (check_seqlens(cu_seqlens, num_seqs) != 0) return -2;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !log_alpha || !b_erase || !w_write || !o))
        return -2;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha;
    J.b_erase = b_erase; J.w_write = w_write; J.h0 = h0;
    J.cu_seqlens = cu_seqlens; J.num_seqs = num_seqs; J.H = H; J.dk = dk; J.dv = dv;
    J.o = o; J.hT = hT;
    return run_all(&J, nthreads);
}

/* KDA forward over a packed batch: the generalised recurrence with
 * b_t = w_t = beta_t. */
int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta, const double *h0,
                   const int64_t *cu_seqlens, int64_t num_seqs, int64_t H,
                   int64_t dk, int64_t dv, double *o, double *hT, int nthreads)
{
    return kda_oracle_gen_fwd(q, k, v, log_alpha, beta, beta, h0, cu_seqlens,
                              num_seqs, H, dk, dv, o, hT, nthreads);
}

/* One recurrent decode step for B independent sequences: every sequence is a
 * chain of length one whose initial state is S[b]; S is overwritten with the
 * new state.  q, k, log_alpha: [B, H, dk]; v: [B, H, dv]; beta: [B, H];
 * S: [B, H, dk, dv] (in/out); o: [B, H, dv]. */
int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *log_alpha, const double *beta, double *S,
                      int64_t B, int64_t H, int64_t dk, int64_t dv, double *o,
                      int nthreads)
{
    if (B < 0 || !S) return -2;
    int64_t *cu = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B + 1));
    double *S_out = (double *)malloc(sizeof(double) * (size_t)(B * H * dk * dv + 1));
    if (!cu || !S_out) { free(cu); free(S_out); return -1; }
    for (int64_t b = 0; b <= B; ++b) cu[b] = b;
    int rc = kda_oracle_fwd(q, k, v, log_alpha, beta, S, cu, B, H, dk, dv, o, S_out, nthreads);
    if (rc == 0) memcpy(S, S_out, sizeof(double) * (size_t)(B * H * dk * dv));
    free(cu);
    free(S_out);
    return rc;
}

/* Input prologue, for the entry points that take raw projections.
 *
 * KimiLinear article (intl.cloud.baidu.com), section 3.2 "Balancing Numerical
 * Stability and Computational Efficiency": the chunkwise KDA keeps the state's
 * scale under control by normalising its inputs and by constraining and
 * reparameterising the gate values; the section gives no formulas.  The reading
 * taken is the set of maps the workloads draw their inputs through, with the
 * gate constraint as a caller-given floor:
 *     q_hat = q / max(||q||_2, eps),   k_hat = k / max(||k||_2, eps)
 *                                          (per token and head, over d_k)
 *     log_alpha = max(-softplus(a), lo),   softplus(a) = log(1 + e^a)
 *                                          (per token, head and key channel)
 *     beta = sigmoid(b) = 1 / (1 + e^-b)   (per token and head)
 * Layouts: q, k, a, q_hat, k_hat, log_alpha: [rows, dk]; b, beta: [rows], with
 * rows = tokens x heads.  softplus and sigmoid are evaluated in the forms that
 * cannot overflow: softplus(a) = max(a, 0) + log1p(e^-|a|), and sigmoid from
 * e^-|b|. */
int kda_oracle_prologue(const double *q, const double *k, const double *a, const double *b,
                        int64_t rows, int64_t dk, double lo, double eps,
                        double *q_hat, double *k_hat, double *log_alpha, double *beta)
{
    if (rows < 0 || dk <= 0 || !(eps > 0.0)) return -2;
    for (int64_t r = 0; r < rows; ++r) {
        const double *qr = q + r * dk, *kr = k + r * dk, *ar = a + r * dk;
        double nq = 0.0, nk = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            nq += qr[c] * qr[c];
            nk += kr[c] * kr[c];
        }
        nq = sqrt(nq);
        nk = sqrt(nk);
        const double dq = nq > eps ? nq : eps, dkn = nk > eps ? nk : eps;
        for (int64_t c = 0; c < dk; ++c) {
            q_hat[r * dk + c] = qr[c] / dq;
            k_hat[r * dk + c] = kr[c] / dkn;
            const double x = ar[c];
            const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
            const double la = -sp;
            log_alpha[r * dk + c] = la > lo ? la : lo;
        }
        const double e = exp(-fabs(b[r]));
        beta[r] = b[r] >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
    }
    return 0;
}

/* Backward of the input prologue: the chain rule through the maps above, per
 * row.  Given the gradients of the mapped values (dq_hat, dk_hat, dla, dbeta),
 * returns those of the raw ones:
 *     dq = (dq_hat - q_hat (q_hat . dq_hat)) / ||q||   where ||q|| > eps,
 *     dq = dq_hat / eps                                 otherwise (q_hat = q / eps);
 * dk likewise;
 *     da = -sigmoid(a) dla   where -softplus(a) > lo (the floor does not bind),
 *     da = 0                 otherwise;
 *     db = beta (1 - beta) dbeta.
 * Layouts as for kda_oracle_prologue.  Returns 0 or -2. */
int kda_oracle_prologue_bwd(const double *q, const double *k, const double *a, const double *b,
                            int64_t rows, int64_t dk, double lo, double eps,
                            const double *dq_hat, const double *dk_hat, const double *dla,
                            const double *dbeta, double *dq, double *dk_out, double *da, double *db)
{
    if (rows < 0 || dk <= 0 || !(eps > 0.0)) return -2;
    for (int64_t r = 0; r < rows; ++r) {
        const double *qr = q + r * dk, *kr = k + r * dk, *ar = a + r * dk;
        const double *gq = dq_hat + r * dk, *gk = dk_hat + r * dk, *gl = dla + r * dk;
        double nq = 0.0, nk = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            nq += qr[c] * qr[c];
            nk += kr[c] * kr[c];
        }
        nq = sqrt(nq);
        nk = sqrt(nk);
        /* projections q_hat . dq_hat and k_hat . dk_hat (used only when ||.|| > eps) */
        double pq = 0.0, pk = 0.0;
        if (nq > eps)
            for (int64_t c = 0; c < dk; ++c) pq += (qr[c] / nq) * gq[c];
        if (nk > eps)
            for (int64_t c = 0; c < dk; ++c) pk += (kr[c] / nk) * gk[c];
        for (int64_t c = 0; c < dk; ++c) {
            dq[r * dk + c] = nq > eps ? (gq[c] - (qr[c] / nq) * pq) / nq : gq[c] / eps;
            dk_out[r * dk + c] = nk > eps ? (gk[c] - (kr[c] / nk) * pk) / nk : gk[c] / eps;
            const double x = ar[c];
            const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
            const double e = exp(-fabs(x));
            const double sg = x >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);   /* sigmoid(a) = d softplus / da */
            da[r * dk + c] = -sp > lo ? -sg * gl[c] : 0.0;
        }
        const double e = exp(-fabs(b[r]));
        const double be = b[r] >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
        db[r] = be * (1.0 - be) * dbeta[r];
    }
    return 0;
}

/* Gradient of the KDA forward, for training.
 *
 * KimiLinear article (intl.cloud.baidu.com), sections 3 and 4.1: the chunkwise
 * form exists to make training on long sequences efficient, and section 3.2
 * notes that only a chunk-sized score block needs to be kept for the backward
 * pass.  The pages give no backward formulas; the gradient is the plain one,
 * reverse-mode differentiation of the per-token recurrence above (b = w =
 * beta), for a scalar loss whose gradients with respect to o and h_T are given
 * (d_o, d_hT; d_hT may be NULL for zero).
 *
 * Forward step t, with a = exp(log_alpha_t):
 *     Sd = Diag(a) S_{t-1};  r = Sd^T k_t;  u = beta_t (v_t - r);
 *     S_t = Sd + k_t u^T;    o_t = S_t^T q_t.
 * Reverse step t, with dS = dL/dS_t accumulated from later tokens:
 *     dS += q_t do_t^T;            dq_t = S_t do_t;
 *     du = dS^T k_t;               dk_t = dS u;
 *     dbeta_t = du . (v_t - r);    dv_t = beta_t du;
 *     dr = -beta_t du;             dk_t += Sd dr;
 *     dSd = dS + k_t dr^T;         dlog_alpha_t[c] = sum_j dSd[c,j] Sd[c,j];
 *     dS = Diag(a) dSd             (= dL/dS_{t-1});
 * and dh0 = dS once the sequence's first token is done.
 *
 * With separate erase and write strengths (the generalised recurrence, u =
 * w_t v_t - b_t r), the same reverse step has dw_t = du . v_t,
 * db_t = -du . r, dv_t = w_t du and dr = -b_t du; with w = b, dw + db is the
 * dbeta above.
 *
 * The reverse pass needs S_{t-1} and S_t for every t.  They are recomputed
 * from checkpoints (the state before every K-th token, K ~ sqrt(length)),
 * one block of K tokens at a time, by the same forward step in the same
 * order, so every value is the one a full forward pass gives; this only bounds
 * the memory.
 */
typedef struct {
    const double *q, *k, *v, *log_alpha, *beta, *h0, *d_o, *d_hT;
    const double *wr;             /* write strengths; NULL: tied to beta */
    const int64_t *cu_seqlens;
    int64_t num_seqs, H, dk, dv;
    double *dq, *dkk, *dvv, *dla, *dbeta, *dh0;
    double *dwr;                  /* gradient of wr (used when wr is given) */
    int64_t next_chain;
    pthread_mutex_t mu;
    int failed;
} oracle_bwd_job;

/* S <- state after token t, from S = state before token t (forward step). */
static void bwd_fwd_step(const oracle_bwd_job *J, int64_t t, int64_t h, double *S, double *r)
{
    const int64_t H = J->H, dk = J->dk, dv = J->dv;
    const double *kt = J->k + (t * H + h) * dk;
    const double *vt = J->v + (t * H + h) * dv;
    const double *lat = J->log_alpha + (t * H + h) * dk;
    const double bt = J->beta[t * H + h];
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp(lat[c]);
        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
    }
    for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < dv; ++j) r[j] += kt[c] * S[c * dv + j];
    if (J->wr) {
        const double wt = J->wr[t * H + h];
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kt[c] * (wt * vt[j] - bt * r[j]);
    } else {
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kt[c] * (bt * (vt[j] - r[j]));
    }
}

static int run_bwd_chain(const oracle_bwd_job *J, int64_t n, int64_t h)
{
    const int64_t H = J->H, dk = J->dk, dv = J->dv, M = dk * dv;
    const int64_t t0 = J->cu_seqlens[n], L = J->cu_seqlens[n + 1] - t0;
    int64_t K = 1;
    while (K * K < L) ++K;
    const int64_t nblk = L > 0 ? (L + K - 1) / K : 0;
    double *ck = (double *)malloc(sizeof(double) * (size_t)((nblk + 1) * M));  /* checkpoints */
    double *blk = (double *)malloc(sizeof(double) * (size_t)((K + 1) * M));    /* states of one block */
    double *dS = (double *)malloc(sizeof(double) * (size_t)M);
    double *Sd = (double *)malloc(sizeof(double) * (size_t)M);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    double *du = (double *)malloc(sizeof(double) * (size_t)dv);
    int rc = 0;
    if (!ck || !blk || !dS || !Sd || !r || !u || !du) { rc = -1; goto done; }

    /* forward: checkpoint the state before tokens 0, K, 2K, ... */
    if (J->h0) memcpy(ck, J->h0 + (n * H + h) * M, sizeof(double) * (size_t)M);
    else memset(ck, 0, sizeof(double) * (size_t)M);
    for (int64_t b = 0; b < nblk; ++b) {
        memcpy(ck + (b + 1) * M, ck + b * M, sizeof(double) * (size_t)M);
        for (int64_t i = b * K; i < L && i < (b + 1) * K; ++i) bwd_fwd_step(J, t0 + i, h, ck + (b + 1) * M, r);
    }

    if (J->d_hT) memcpy(dS, J->d_hT + (n * H + h) * M, sizeof(double) * (size_t)M);
    else memset(dS, 0, sizeof(double) * (size_t)M);

    for (int64_t b = nblk - 1; b >= 0; --b) {
        const int64_t i0 = b * K, i1 = (b + 1) * K < L ? (b + 1) * K : L;
        /* blk[i - i0] = state before token i, for i0 <= i <= i1 */
        memcpy(blk, ck + b * M, sizeof(double) * (size_t)M);
        for (int64_t i = i0; i < i1; ++i) {
            memcpy(blk + (i - i0 + 1) * M, blk + (i - i0) * M, sizeof(double) * (size_t)M);
            bwd_fwd_step(J, t0 + i, h, blk + (i - i0 + 1) * M, r);
        }
        for (int64_t i = i1 - 1; i >= i0; --i) {
            const int64_t t = t0 + i;
            const double *Sp = blk + (i - i0) * M, *St = blk + (i - i0 + 1) * M;
            const double *qt = J->q + (t * H + h) * dk;
            const double *kt = J->k + (t * H + h) * dk;
            const double *vt = J->v + (t * H + h) * dv;
            const double *lat = J->log_alpha + (t * H + h) * dk;
            const double *dot = J->d_o + (t * H + h) * dv;
            const double bt = J->beta[t * H + h];
            const double wt = J->wr ? J->wr[t * H + h] : bt;
            double *dqt = J->dq + (t * H + h) * dk;
            double *dkt = J->dkk + (t * H + h) * dk;
            double *dvt = J->dvv + (t * H + h) * dv;
            double *dlat = J->dla + (t * H + h) * dk;

            /* recompute Sd, r, u of this step */
            for (int64_t c = 0; c < dk; ++c) {
                const double a = exp(lat[c]);
                for (int64_t j = 0; j < dv; ++j) Sd[c * dv + j] = a * Sp[c * dv + j];
            }
            for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) r[j] += kt[c] * Sd[c * dv + j];
            if (J->wr)
                for (int64_t j = 0; j < dv; ++j) u[j] = wt * vt[j] - bt * r[j];
            else
                for (int64_t j = 0; j < dv; ++j) u[j] = bt * (vt[j] - r[j]);

            /* read-out o_t = S_t^T q_t */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] += qt[c] * dot[j];
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += St[c * dv + j] * dot[j];
                dqt[c] = acc;
            }
            /* write S_t = Sd + k u^T */
            for (int64_t j = 0; j < dv; ++j) du[j] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) du[j] += dS[c * dv + j] * kt[c];
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * u[j];
                dkt[c] = acc;
            }
            /* u = beta (v - r), or w v - b r */
            if (J->wr) {
                double dw = 0.0, db = 0.0;
                for (int64_t j = 0; j < dv; ++j) dw += du[j] * vt[j];
                for (int64_t j = 0; j < dv; ++j) db -= du[j] * r[j];
                J->dwr[t * H + h] = dw;
                J->dbeta[t * H + h] = db;
                for (int64_t j = 0; j < dv; ++j) dvt[j] = wt * du[j];
            } else {
                double db = 0.0;
                for (int64_t j = 0; j < dv; ++j) db += du[j] * (vt[j] - r[j]);
                J->dbeta[t * H + h] = db;
                for (int64_t j = 0; j < dv; ++j) dvt[j] = bt * du[j];
            }
            /* r = Sd^T k: dr = -beta du */
            for (int64_t j = 0; j < dv; ++j) du[j] = -bt * du[j];
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) acc += Sd[c * dv + j] * du[j];
                dkt[c] += acc;
            }
            /* dSd = dS + k dr^T; Sd = Diag(a) S_{t-1} */
            for (int64_t c = 0; c < dk; ++c) {
                const double a = exp(lat[c]);
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j) {
                    const double g = dS[c * dv + j] + kt[c] * du[j];
                    acc += g * Sd[c * dv + j];
                    dS[c * dv + j] = a * g;
                }
                dlat[c] = acc;
            }
        }
    }
    if (J->dh0) memcpy(J->dh0 + (n * H + h) * M, dS, sizeof(double) * (size_t)M);
done:
    free(ck); free(blk); free(dS); free(Sd); free(r); free(u); free(du);
    return rc;
}

static void *bwd_worker(void *arg)
{
    oracle_bwd_job *J = (oracle_bwd_job *)arg;
    const int64_t total = J->num_seqs * J->H;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t id = J->next_chain++;
        pthread_mutex_unlock(&J->mu);
        if (id >= total) break;
        if (run_bwd_chain(J, id / J->H, id % J->H) != 0) {
            pthread_mutex_lock(&J->mu);
            J->failed = 1;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

static int run_bwd_job(oracle_bwd_job *J, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    pthread_mutex_init(&J->mu, NULL);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) { pthread_mutex_destroy(&J->mu); return -1; }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, bwd_worker, J) != 0) break;
        ++started;
    }
    if (started == 0) bwd_worker(J);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&J->mu);
    return J->failed ? -1 : 0;
}

/* Layouts as for kda_oracle_fwd; d_o like o, d_hT and dh0 like h0.  Outputs
 * dq, dk_out, dlog_alpha: [T_total, H, dk]; dv_out: [T_total, H, dv];
 * dbeta: [T_total, H]; dh0 may be NULL.  Returns 0, -1 (no memory) or -2. */
int kda_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta, const double *h0,
                   const int64_t *cu_seqlens, int64_t num_seqs, int64_t H,
                   int64_t dk, int64_t dv, const double *d_o, const double *d_hT,
                   double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                   double *dbeta, double *dh0, int nthreads)
{
    if (H <= 0 || dk <= 0 || dv <= 0) return -2;
    if (check_seqlens(cu_seqlens, num_seqs) != 0) return -2;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !dq ||
                                     !dk_out || !dv_out || !dlog_alpha || !dbeta))
        return -2;
    oracle_bwd_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta; J.h0 = h0;
    J.d_o = d_o; J.d_hT = d_hT; J.cu_seqlens = cu_seqlens; J.num_seqs = num_seqs;
    J.H = H; J.dk = dk; J.dv = dv;
    J.dq = dq; J.dkk = dk_out; J.dvv = dv_out; J.dla = dlog_alpha; J.dbeta = dbeta; J.dh0 = dh0;
    return run_bwd_job(&J, nthreads);
}

/* Gradient of the generalised recurrence (kda_oracle_gen_fwd): as
 * kda_oracle_bwd with the erase strengths b_erase in place of beta, plus the
 * write strengths w_write [T_total, H]; d_b and d_w are their gradients. */
int kda_oracle_gen_bwd(const double *q, const double *k, const double *v,
                       const double *log_alpha, const double *b_erase, const double *w_write,
                       const double *h0, const int64_t *cu_seqlens, int64_t num_seqs, int64_t H,
                       int64_t dk, int64_t dv, const double *d_o, const double *d_hT,
                       double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                       double *d_b, double *d_w, double *dh0, int nthreads)
{
    if (H <= 0 || dk <= 0 || dv <= 0) return -2;
    if (check_seqlens(cu_seqlens, num_seqs) != 0) return -2;
    if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !log_alpha || !b_erase || !w_write || !d_o ||
                                     !dq || !dk_out || !dv_out || !dlog_alpha || !d_b || !d_w))
        return -2;
    oracle_bwd_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = b_erase; J.wr = w_write; J.h0 = h0;
    J.d_o = d_o; J.d_hT = d_hT; J.cu_seqlens = cu_seqlens; J.num_seqs = num_seqs;
    J.H = H; J.dk = dk; J.dv = dv;
    J.dq = dq; J.dkk = dk_out; J.dvv = dv_out; J.dla = dlog_alpha; J.dbeta = d_b; J.dwr = d_w;
    J.dh0 = dh0;
    return run_bwd_job(&J, nthreads);
}

int kda_oracle_version(void) { return 4; }
