/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test-suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * library; the two only ever see the same seeded input arrays.
 *
 * What it computes (one token at a time, no chunking, no reordering):
 *
 *   For every (sequence, head), starting from S = S_init (zeros if absent),
 *   and for t = 1..T in order
 *       Sbar = Diag(alpha_t) S                 decay each key-channel row
 *       old  = Sbar^T k_t                      what the decayed memory answers
 *       u    = beta_t (v_t - old)              the delta-rule correction
 *       S    = Sbar + k_t u^T                  erase + write
 *       o_t  = S^T q_t                         read-out AFTER the update
 *   which is S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = S_t^T q_t.
 *
 *   Sources: "Kimi Delta Attention 完全拆解" (pinghaoyang.com.cn), section
 *   "KDA 的核心：让遗忘从一个标量细化为逐通道向量" (the KDA update and its
 *   decayed-state form) and section "一次 KDA 前向究竟发生了什么" (the numbered
 *   decode sequence: decay, old value, corrected write, read-out); "Kimi K3模型
 *   架构详解" (gentlecold.top) section 3.2 "KDA的递推式" (decay first, then the
 *   delta write, read-out from the updated state); "Kimi K3 的 KDA"
 *   (marsggbo.github.io) section 3 (the five-step order).
 *
 *   S is [Dk x Dv]: rows are key channels, columns are value channels
 *   ("从线性注意力到 KDA", section "衰减为什么要按行做": the gate scales rows and
 *   carries only the key axis).
 *
 * Two further modes exist only to pin the oracle against what the pages fix:
 *   ORC_ERASE_OFF         S = Diag(alpha) S + beta k v^T  (gated linear attention,
 *                         "Kimi K3 的 KDA" section 5, erase-free expansion;
 *                         with alpha = 1, beta = 1 it is plain linear attention,
 *                         same page section 2).
 *   ORC_ERASE_THEN_DECAY  S = Diag(alpha)(I - beta k k^T) S + beta k v^T, the
 *                         order the pages warn is NOT the implemented one
 *                         ("从线性注意力到 KDA", section "术语坑", last item).
 *                         Used only by a test that requires it to DIFFER.
 *
 * Parallelism: work items are (sequence, head, block of value columns).  The
 * transition acts on the key axis only, so each column of S evolves on its own
 * (old_v, u_v and o_v involve column v alone); splitting columns changes no
 * arithmetic inside a column.
 *
 * Numerics: every input is an fp64 array holding exactly the values handed to
 * the GPU (bf16 / fp32 upcast exactly); all arithmetic is fp64, sequential in
 * the natural order above.
 *
 * Parity status: pinned by the closed forms, invariants, special cases and
 * independent formulations in the CPU test-suite; the general random case has
 * no printed values on the pages.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_KDA = 0, ORC_ERASE_OFF = 1, ORC_ERASE_THEN_DECAY = 2 };

typedef struct {
    const double *q, *k, *v, *alpha, *beta; /* [NTOK,H,Dk] x3 ([.,.,Dv] for v), [NTOK,H] */
    const int64_t *cu;                      /* [N+1] token offsets per sequence        */
    int64_t n_seq, H, Dk, Dv, col_block;
    const double *s_init;                   /* [N,H,Dk,Dv] or NULL                       */
    double *o;                              /* [NTOK,H,Dv]                               */
    double *s_final;                        /* [N,H,Dk,Dv] or NULL                       */
    int mode;
    int64_t n_items;
    int64_t next;                           /* shared work counter (guarded by lock)     */
    pthread_mutex_t lock;
} orc_job;

/* Runs the token loop for one (sequence, head, column block). */
static void orc_item(const orc_job *J, int64_t item, double *S, double *old)
{
    const int64_t ncb = (J->Dv + J->col_block - 1) / J->col_block;
    const int64_t cb = item % ncb;
    const int64_t h = (item / ncb) % J->H;
    const int64_t n = item / (ncb * J->H);
    const int64_t c0 = cb * J->col_block;
    const int64_t nc = (J->Dv - c0 < J->col_block) ? (J->Dv - c0) : J->col_block;
    const int64_t Dk = J->Dk, Dv = J->Dv, H = J->H;

    /* S is held as [Dk][nc] for this column block. */
    for (int64_t r = 0; r < Dk; ++r)
        for (int64_t c = 0; c < nc; ++c)
            S[r * nc + c] = J->s_init ? J->s_init[((n * H + h) * Dk + r) * Dv + c0 + c] : 0.0;

    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const double *q = J->q + (t * H + h) * Dk;
        const double *k = J->k + (t * H + h) * Dk;
        const double *v = J->v + (t * H + h) * Dv + c0;
        const double *a = J->alpha + (t * H + h) * Dk;
        const double b = J->beta[t * H + h];
        double *o = J->o + (t * H + h) * Dv + c0;

        if (J->mode == ORC_KDA) {
            /* Sbar = Diag(alpha) S */
            for (int64_t r = 0; r < Dk; ++r)
                for (int64_t c = 0; c < nc; ++c) S[r * nc + c] *= a[r];
            /* old = Sbar^T k */
            for (int64_t c = 0; c < nc; ++c) old[c] = 0.0;
            for (int64_t r = 0; r < Dk; ++r)
                for (int64_t c = 0; c < nc; ++c) old[c] += S[r * nc + c] * k[r];
            /* u = beta (v - old);  S = Sbar + k u^T */
            for (int64_t c = 0; c < nc; ++c) old[c] = b * (v[c] - old[c]);
            for (int64_t r = 0; r < Dk; ++r)
                for (int64_t c = 0; c < nc; ++c) S[r * nc + c] += k[r] * old[c];
        } else if (J->mode == ORC_ERASE_OFF) {
            for (int64_t r = 0; r < Dk; ++r)
                for (int64_t c = 0; c < nc; ++c)
                    S[r * nc + c] = a[r] * S[r * nc + c] + b * k[r] * v[c];
        } else { /* ORC_ERASE_THEN_DECAY */
            for (int64_t c = 0; c < nc; ++c) old[c] = 0.0;
            for (int64_t r = 0; r < Dk; ++r)
                for (int64_t c = 0; c < nc; ++c) old[c] += S[r * nc + c] * k[r];
            for (int64_t r = 0; r < Dk; ++r)
                for (int64_t c = 0; c < nc; ++c)
                    S[r * nc + c] = a[r] * (S[r * nc + c] - b * k[r] * old[c]) + b * k[r] * v[c];
        }
        /* o = S^T q  (the updated state) */
        for (int64_t c = 0; c < nc; ++c) o[c] = 0.0;
        for (int64_t r = 0; r < Dk; ++r)
            for (int64_t c = 0; c < nc; ++c) o[c] += S[r * nc + c] * q[r];
    }

    if (J->s_final)
        for (int64_t r = 0; r < Dk; ++r)
            for (int64_t c = 0; c < nc; ++c)
                J->s_final[((n * H + h) * Dk + r) * Dv + c0 + c] = S[r * nc + c];
}

static void *orc_worker(void *arg)
{
    orc_job *J = (orc_job *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)(J->Dk * J->col_block));
    double *old = (double *)malloc(sizeof(double) * (size_t)J->col_block);
    if (!S || !old) {
        free(S);
        free(old);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t item = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (item >= J->n_items) break;
        orc_item(J, item, S, old);
    }
    free(S);
    free(old);
    return NULL;
}

/*
 * kda_oracle_forward: runs the recurrence above for every sequence of a packed
 * batch.  Dense [B,T,...] inputs are the case cu = {0, T, 2T, ..., B*T}.
 *   q, k, alpha : [NTOK, H, Dk] fp64      v : [NTOK, H, Dv] fp64
 *   beta        : [NTOK, H] fp64          cu: [n_seq + 1] int64, cu[0] = 0
 *   s_init      : [n_seq, H, Dk, Dv] or NULL (zeros)
 *   o           : [NTOK, H, Dv] (written)  s_final: [n_seq, H, Dk, Dv] or NULL
 *   mode        : ORC_KDA, ORC_ERASE_OFF or ORC_ERASE_THEN_DECAY
 *   nthreads    : worker threads (>= 1)
 * Returns 0 on success, nonzero on a bad argument or allocation failure.
 */
int kda_oracle_forward(const double *q, const double *k, const double *v, const double *alpha,
                       const double *beta, const int64_t *cu, int64_t n_seq, int64_t H, int64_t Dk,
                       int64_t Dv, const double *s_init, double *o, double *s_final, int mode,
                       int nthreads)
{
    if (!q || !k || !v || !alpha || !beta || !cu || !o) return 1;
    if (n_seq < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return 1;
    if (mode < ORC_KDA || mode > ORC_ERASE_THEN_DECAY) return 1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu[n + 1] < cu[n]) return 1;
    if (nthreads < 1) nthreads = 1;

    orc_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.beta = beta; J.cu = cu;
    J.n_seq = n_seq; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.col_block = Dv < 16 ? Dv : 16;
    J.s_init = s_init; J.o = o; J.s_final = s_final; J.mode = mode;
    J.n_items = n_seq * H * ((Dv + J.col_block - 1) / J.col_block);
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (nthreads > J.n_items) nthreads = (int)(J.n_items > 0 ? J.n_items : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return 2;
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, orc_worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) rc = 2;
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret) rc = 2;
    }
    free(th);
    pthread_mutex_destroy(&J.lock);
    return rc;
}
