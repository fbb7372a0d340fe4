/*
 * fp64 CPU oracle for the gated delta rule (Gated DeltaNet / KDA-style per-key decay),
 * the DeltaLog decode bookkeeping and the causal short convolution.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Sources (web pages; cited by title and section):
 *   [LA-Infra]  "深度解析线性注意力机制演进与 AI Infra 实现" (todayforai.com, binnnliu)
 *   [Handbook]  "线性注意力与混合架构的推理", AI-infra handbooks (anrans.github.io)
 *   [DeltaLog]  "DeltaLog：延迟物化递归状态以加速线性注意力解码" reading notes
 *               (arXiv 2608.15533v1)
 *
 * State orientation: S is d_k x d_v (row = key channel, column = value channel) and the
 * read-out is o = S^T q, as in [Handbook] "同一个计算的两种写法" and [DeltaLog] §1.1.
 * ([LA-Infra] writes the transpose, S in R^{d_v x d_k} with o = S q; the two are the
 * same map.)
 *
 * Everything is plain fp64, one sequential loop per independent (sequence, head) unit;
 * units are spread over POSIX threads. No blocking, no chunking, no reordering.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* Gated delta rule, sequential recurrence                                               */
/* ------------------------------------------------------------------------------------ */
/*
 * One token of the recurrence, in the order the pages fix:
 *   [LA-Infra] "GDN：增加遗忘门": the whole state first decays by alpha_t, then the delta
 *     rule writes; "从重建误差到正则化": decay first, then the reconstruction error is
 *     taken against the *decayed* memory, then the correction is written.
 *   [LA-Infra] "KDA: By Channel的遗忘门" / "KDA实现逻辑概述": with a per-key-channel gate the
 *     decay is Diag(alpha_t) acting on the key axis (rows of the d_k x d_v state).
 *   [LA-Infra] "KDA实现逻辑概述" step list and [Handbook] "同一个计算的两种写法": the token
 *     reads the state after its own write, o_t = scale * S_t^T q_t.
 *
 *   Sbar = Diag(exp(g_t)) S            (scalar gate: exp(g_t) * S)
 *   vhat = Sbar^T k_t
 *   r    = beta_t (v_t - vhat)
 *   S    = Sbar + k_t r^T
 *   o_t  = scale * S^T q_t
 *
 * Optional L2 normalisation of q and k along the head dim ([LA-Infra] "去掉分母引入卷积"
 * and App. 2 "为什么要L2 Norm"; the pages add an epsilon guard without a value; the
 * reading used here is x / sqrt(x.x + eps)).
 */
typedef struct {
    int dk, dv, perkey, l2norm;
    double scale, eps;
} gdn_cfg;

static void l2n(const double* x, double* y, int n, int on, double eps) {
    if (!on) {
        memcpy(y, x, sizeof(double) * (size_t)n);
        return;
    }
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; i++) y[i] = x[i] * inv;
}

/* One token on one unit. S: dk x dv row-major, updated in place. o: dv outputs.
 * work: at least 2*dk + dv doubles. */
static void gdn_token(const gdn_cfg* c, double* S, const double* q_in, const double* k_in,
                      const double* v, const double* g, double beta, double* o, double* work) {
    const int dk = c->dk, dv = c->dv;
    double* q = work;
    double* k = work + dk;
    double* vhat = work + 2 * dk;
    l2n(q_in, q, dk, c->l2norm, c->eps);
    l2n(k_in, k, dk, c->l2norm, c->eps);
    /* decay */
    for (int i = 0; i < dk; i++) {
        double a = exp(c->perkey ? g[i] : g[0]);
        double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) row[j] *= a;
    }
    /* read against the decayed state */
    for (int j = 0; j < dv; j++) vhat[j] = 0.0;
    for (int i = 0; i < dk; i++) {
        const double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) vhat[j] += row[j] * k[i];
    }
    /* residual write: S += k r^T with r = beta (v - vhat) */
    for (int j = 0; j < dv; j++) vhat[j] = beta * (v[j] - vhat[j]); /* vhat now holds r */
    for (int i = 0; i < dk; i++) {
        double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) row[j] += k[i] * vhat[j];
    }
    /* read after write */
    for (int j = 0; j < dv; j++) o[j] = 0.0;
    for (int i = 0; i < dk; i++) {
        const double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; j++) o[j] += row[j] * q[i];
    }
    for (int j = 0; j < dv; j++) o[j] *= c->scale;
}

typedef struct {
    gdn_cfg cfg;
    int n_seqs, H;
    const int32_t* cu;
    const double *q, *k, *v, *g, *beta;
    double* states; /* [n_seqs, H, dk, dv] */
    double* o;      /* [T, H, dv] */
    int next;       /* shared work counter */
    pthread_mutex_t mu;
} prefill_job;

static int take_unit(pthread_mutex_t* mu, int* next, int total) {
    pthread_mutex_lock(mu);
    int u = *next;
    if (u < total) (*next)++;
    pthread_mutex_unlock(mu);
    return u < total ? u : -1;
}

static void* prefill_worker(void* arg) {
    prefill_job* J = (prefill_job*)arg;
    const gdn_cfg* c = &J->cfg;
    const int dk = c->dk, dv = c->dv, H = J->H;
    const int dg = c->perkey ? dk : 1;
    double* work = (double*)malloc(sizeof(double) * (size_t)(2 * dk + dv));
    int u;
    while ((u = take_unit(&J->mu, &J->next, J->n_seqs * H)) >= 0) {
        int n = u / H, h = u % H;
        double* S = J->states + (size_t)u * dk * dv;
        for (int t = J->cu[n]; t < J->cu[n + 1]; t++) {
            size_t th = (size_t)t * H + h;
            gdn_token(c, S, J->q + th * dk, J->k + th * dk, J->v + th * dv, J->g + th * dg,
                      J->beta[th], J->o + th * dv, work);
        }
    }
    free(work);
    return NULL;
}

static int run_pool(void* (*fn)(void*), void* job, int n_threads) {
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 0; i < n_threads; i++) {
        if (pthread_create(&th[i], NULL, fn, job) != 0) break;
        started++;
    }
    if (started == 0) fn(job);
    for (int i = 0; i < started; i++) pthread_join(th[i], NULL);
    return started == 0 ? 1 : started;
}

/*
 * Packed varlen recurrence over n_seqs sequences (cu_seqlens, [Handbook] "在真实模型上核对"
 * split-prefill semantics: a sequence's state is handed over in `states`).
 *   q, k : [T, H, dk]; v, o : [T, H, dv]; g : [T, H] (scalar) or [T, H, dk] (per key);
 *   beta : [T, H]; states : [n_seqs, H, dk, dv], initial on entry, final on return.
 * Returns the number of threads used.
 */
int gdn_oracle_recurrence(int n_seqs, const int32_t* cu_seqlens, int H, int dk, int dv,
                          int perkey, const double* q, const double* k, const double* v,
                          const double* g, const double* beta, double scale, int l2norm,
                          double eps, double* states, double* o, int n_threads) {
    prefill_job J;
    J.cfg.dk = dk;
    J.cfg.dv = dv;
    J.cfg.perkey = perkey;
    J.cfg.l2norm = l2norm;
    J.cfg.scale = scale;
    J.cfg.eps = eps;
    J.n_seqs = n_seqs;
    J.H = H;
    J.cu = cu_seqlens;
    J.q = q;
    J.k = k;
    J.v = v;
    J.g = g;
    J.beta = beta;
    J.states = states;
    J.o = o;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    int used = run_pool(prefill_worker, &J, n_threads);
    pthread_mutex_destroy(&J.mu);
    return used;
}

/* ------------------------------------------------------------------------------------ */
/* DeltaLog: dense base + append log, merged every M steps                               */
/* ------------------------------------------------------------------------------------ */
/*
 * [DeltaLog] §1.1: generic update S_t = D(lambda_t) S_{t-1} + a_t b_t^T, D(l) = diag(exp l).
 * [DeltaLog] §2.1: base Sbar, accumulated log-decay lbar since the last merge, logs
 *   K_log (a_i), U_log (b_i), Lambda_log (lbar snapshot at insertion), capacity C = M-1,
 *   current length L.
 * [DeltaLog] §2.2 Eq. (7): S_t = D(lbar) Sbar + sum_{i<L} D(lbar - Lambda_i) K_i U_i^T.
 * [DeltaLog] §2.3 Algorithm 1 / Eqs. (4)-(6): per step, lbar += lambda_t; form a_t, b_t;
 *   if L < C on entry append (a_t, b_t, lbar) and L += 1 (base untouched); if L == C on
 *   entry merge: Sbar = D(lbar) Sbar + sum_i D(lbar - Lambda_i) K_i U_i^T + a_t b_t^T,
 *   then lbar = 0, L = 0.
 * [DeltaLog] §2.4: reads come straight from base + log,
 *   x^T S = (x * e^{lbar})^T Sbar + sum_i [x^T D(lbar - Lambda_i) K_i] U_i^T.
 *
 * Two update kinds:
 *   mode 0 (gated delta rule, [DeltaLog] §2.7 "GDN"/"KDA"): a_t = k_t,
 *     b_t = beta_t (v_t - vhat) with vhat read from the *decayed* logical state, i.e. after
 *     lbar has been incremented (the decay-then-correct order of [LA-Infra] "GDN：增加遗忘门";
 *     [DeltaLog] §2.4 asks the operator to keep its own decay / correct / read order).
 *   mode 1 (plain additive write, the generic abstraction of [DeltaLog] §1.1): a_t = k_t,
 *     b_t = v_t. Used for the scalar teaching example of [DeltaLog] §2.3.
 * The token's output reads the updated logical state: o = scale * S_t^T q_t ([DeltaLog] §1.1).
 * K_log precision: bf16 for GDN/KDA ([DeltaLog] §2.7 table); klog_bf16 = 1 rounds logged keys
 * to bf16 (round to nearest even), everything else is fp64.
 */
static double round_bf16(double x) {
    float f = (float)x; /* logged keys are fp32 values first (exact for bf16/fp32 inputs) */
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (double)f; /* inf/nan unchanged */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    u &= 0xffff0000u;
    memcpy(&f, &u, 4);
    return (double)f;
}

typedef struct {
    gdn_cfg cfg;
    int n_units, M, mode, klog_bf16;
    const double *q, *k, *v, *g, *beta;
    double *base, *lbar, *klog, *ulog, *lamlog, *o;
    int32_t* len;
    int next;
    pthread_mutex_t mu;
} dl_job;

/* x^T S_logical for the unit, using the incremented log-decay lp (width dl). */
static void dl_read(const dl_job* J, int u, const double* lp, const double* x, double* out) {
    const int dk = J->cfg.dk, dv = J->cfg.dv, dl = J->cfg.perkey ? dk : 1, C = J->M - 1;
    const double* Sb = J->base + (size_t)u * dk * dv;
    const int L = J->len[u];
    for (int j = 0; j < dv; j++) out[j] = 0.0;
    for (int i = 0; i < dk; i++) {
        double xi = x[i] * exp(lp[J->cfg.perkey ? i : 0]);
        const double* row = Sb + (size_t)i * dv;
        for (int j = 0; j < dv; j++) out[j] += xi * row[j];
    }
    for (int e = 0; e < L; e++) {
        const double* Ke = J->klog + ((size_t)u * C + e) * dk;
        const double* Ue = J->ulog + ((size_t)u * C + e) * dv;
        const double* Le = J->lamlog + ((size_t)u * C + e) * dl;
        double coef = 0.0;
        for (int i = 0; i < dk; i++) {
            int di = J->cfg.perkey ? i : 0;
            coef += x[i] * exp(lp[di] - Le[di]) * Ke[i];
        }
        for (int j = 0; j < dv; j++) out[j] += coef * Ue[j];
    }
}

static void* dl_worker(void* arg) {
    dl_job* J = (dl_job*)arg;
    const int dk = J->cfg.dk, dv = J->cfg.dv, C = J->M - 1;
    const int dl = J->cfg.perkey ? dk : 1;
    double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 3 * dv + dl));
    double* q = buf;
    double* k = q + dk;
    double* vhat = k + dk;
    double* b = vhat + dv;
    double* qs = b + dv;
    double* lp = qs + dv;
    int u;
    while ((u = take_unit(&J->mu, &J->next, J->n_units)) >= 0) {
        l2n(J->q + (size_t)u * dk, q, dk, J->cfg.l2norm, J->cfg.eps);
        l2n(J->k + (size_t)u * dk, k, dk, J->cfg.l2norm, J->cfg.eps);
        const double* v = J->v + (size_t)u * dv;
        const double* g = J->g + (size_t)u * dl;
        double* lb = J->lbar + (size_t)u * dl;
        /* Algorithm 1: accumulate the current decay first */
        for (int d = 0; d < dl; d++) lp[d] = lb[d] + g[d];
        /* b_t */
        if (J->mode == 0) {
            dl_read(J, u, lp, k, vhat);
            for (int j = 0; j < dv; j++) b[j] = J->beta[u] * (v[j] - vhat[j]);
        } else {
            for (int j = 0; j < dv; j++) b[j] = v[j];
        }
        /* output from base + log + the current update (weight D(0) = I) */
        dl_read(J, u, lp, q, qs);
        double kq = 0.0;
        for (int i = 0; i < dk; i++) kq += k[i] * q[i];
        double* o = J->o + (size_t)u * dv;
        for (int j = 0; j < dv; j++) o[j] = J->cfg.scale * (qs[j] + kq * b[j]);
        /* commit: append or merge (decided by L on entry) */
        int L = J->len[u];
        if (L < C) {
            double* Ke = J->klog + ((size_t)u * C + L) * dk;
            double* Ue = J->ulog + ((size_t)u * C + L) * dv;
            double* Le = J->lamlog + ((size_t)u * C + L) * dl;
            for (int i = 0; i < dk; i++) Ke[i] = J->klog_bf16 ? round_bf16(k[i]) : k[i];
            for (int j = 0; j < dv; j++) Ue[j] = b[j];
            for (int d = 0; d < dl; d++) Le[d] = lp[d];
            for (int d = 0; d < dl; d++) lb[d] = lp[d];
            J->len[u] = L + 1;
        } else {
            double* Sb = J->base + (size_t)u * dk * dv;
            for (int i = 0; i < dk; i++) {
                double a = exp(lp[J->cfg.perkey ? i : 0]);
                double* row = Sb + (size_t)i * dv;
                for (int j = 0; j < dv; j++) row[j] *= a;
            }
            for (int e = 0; e < L; e++) {
                const double* Ke = J->klog + ((size_t)u * C + e) * dk;
                const double* Ue = J->ulog + ((size_t)u * C + e) * dv;
                const double* Le = J->lamlog + ((size_t)u * C + e) * dl;
                for (int i = 0; i < dk; i++) {
                    int di = J->cfg.perkey ? i : 0;
                    double w = exp(lp[di] - Le[di]) * Ke[i];
                    double* row = Sb + (size_t)i * dv;
                    for (int j = 0; j < dv; j++) row[j] += w * Ue[j];
                }
            }
            for (int i = 0; i < dk; i++) {
                double* row = Sb + (size_t)i * dv;
                for (int j = 0; j < dv; j++) row[j] += k[i] * b[j];
            }
            for (int d = 0; d < dl; d++) lb[d] = 0.0;
            J->len[u] = 0;
        }
    }
    free(buf);
    return NULL;
}

/*
 * One DeltaLog decode step for n_units independent (request, head) units.
 *   q, k : [n, dk]; v : [n, dv]; g : [n, dl]; beta : [n]
 *   base : [n, dk, dv]; lbar : [n, dl]; klog : [n, M-1, dk]; ulog : [n, M-1, dv];
 *   lamlog : [n, M-1, dl]; len : [n]; o : [n, dv].   dl = dk if perkey else 1.
 */
int gdn_oracle_deltalog_step(int n_units, int dk, int dv, int perkey, int M, int mode,
                             const double* q, const double* k, const double* v,
                             const double* g, const double* beta, double scale, int l2norm,
                             double eps, double* base, double* lbar, double* klog,
                             double* ulog, double* lamlog, int32_t* len, double* o,
                             int klog_bf16, int n_threads) {
    if (M < 2) return -1;
    dl_job J;
    J.cfg.dk = dk;
    J.cfg.dv = dv;
    J.cfg.perkey = perkey;
    J.cfg.l2norm = l2norm;
    J.cfg.scale = scale;
    J.cfg.eps = eps;
    J.n_units = n_units;
    J.M = M;
    J.mode = mode;
    J.klog_bf16 = klog_bf16;
    J.q = q;
    J.k = k;
    J.v = v;
    J.g = g;
    J.beta = beta;
    J.base = base;
    J.lbar = lbar;
    J.klog = klog;
    J.ulog = ulog;
    J.lamlog = lamlog;
    J.len = len;
    J.o = o;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    int used = run_pool(dl_worker, &J, n_threads);
    pthread_mutex_destroy(&J.mu);
    return used;
}

/*
 * The logical state of each unit from base + log, [DeltaLog] §2.2 Eq. (7):
 *   S = D(lbar) Sbar + sum_{i<L} D(lbar - Lambda_i) K_i U_i^T.   out : [n, dk, dv]
 */
void gdn_oracle_deltalog_materialize(int n_units, int dk, int dv, int perkey, int M,
                                     const double* base, const double* lbar,
                                     const double* klog, const double* ulog,
                                     const double* lamlog, const int32_t* len, double* out) {
    const int C = M - 1, dl = perkey ? dk : 1;
    for (int u = 0; u < n_units; u++) {
        const double* Sb = base + (size_t)u * dk * dv;
        const double* lb = lbar + (size_t)u * dl;
        double* S = out + (size_t)u * dk * dv;
        for (int i = 0; i < dk; i++) {
            double a = exp(lb[perkey ? i : 0]);
            for (int j = 0; j < dv; j++) S[(size_t)i * dv + j] = a * Sb[(size_t)i * dv + j];
        }
        for (int e = 0; e < len[u]; e++) {
            const double* Ke = klog + ((size_t)u * C + e) * dk;
            const double* Ue = ulog + ((size_t)u * C + e) * dv;
            const double* Le = lamlog + ((size_t)u * C + e) * dl;
            for (int i = 0; i < dk; i++) {
                int di = perkey ? i : 0;
                double w = exp(lb[di] - Le[di]) * Ke[i];
                for (int j = 0; j < dv; j++) S[(size_t)i * dv + j] += w * Ue[j];
            }
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Causal short convolution + SiLU                                                        */
/* ------------------------------------------------------------------------------------ */
/*
 * [LA-Infra] "去掉分母引入卷积": per channel, fixed-weight sliding window over the current and
 * the previous (width-1) tokens, weight column width-1 multiplies the current token, then
 * SiLU; no mixing across channels. Tokens before the start of a sequence count as zero.
 *   x, y : [T, channels]; w : [channels, width].
 */
void gdn_oracle_conv1d_silu(int n_seqs, const int32_t* cu_seqlens, int channels, int width,
                            const double* x, const double* w, double* y) {
    for (int n = 0; n < n_seqs; n++) {
        for (int t = cu_seqlens[n]; t < cu_seqlens[n + 1]; t++) {
            for (int c = 0; c < channels; c++) {
                double acc = 0.0;
                for (int j = 0; j < width; j++) {
                    int src = t - (width - 1) + j;
                    if (src < cu_seqlens[n]) continue;
                    acc += w[(size_t)c * width + j] * x[(size_t)src * channels + c];
                }
                y[(size_t)t * channels + c] = acc / (1.0 + exp(-acc));
            }
        }
    }
}
