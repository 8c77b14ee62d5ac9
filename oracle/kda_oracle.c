/*
 * CPU oracle for the Kimi Delta Attention (KDA) token mixer -- TEST
 * INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this file's library; the GPU library never does.
 *
 * Plain, slow, token-by-token, fp64 throughout.  Every input arrives as fp64
 * (bf16 and fp32 values widen to fp64 exactly).  Work is split over
 * (sequence, head) pairs with POSIX threads; each pair is computed by one
 * thread in token order, so results do not depend on the thread count.
 *
 * What it follows (page "Ling-3.0-flash: a 124B open MoE that runs like a 5B
 * and reaches for 1M tokens", section "KDA: constant-size memory over a very
 * long context"):
 *   - a fixed d x d state per head that every token updates in place: first a
 *     per-channel gated decay (the erase), then a delta-rule write of the new
 *     key/value association with strength beta; the output reads the state
 *     with the query;
 *   - q and k pass through a short causal conv and an L2 norm, v through a
 *     conv; the decay comes from a softplus gate, beta from a sigmoid, and a
 *     final sigmoid gate multiplies the output.
 * The page's own equation for the update was lost from the text; the update
 * used is the gated delta rule
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 * written below in its expanded, equivalent form
 *     S' = Diag(alpha_t) S_{t-1};  u = S'^T k_t;
 *     S_t = S' + beta_t k_t (v_t - u)^T;  o_t = S_t^T q_t.
 * Width of the conv (4 taps) and the head sizes (32 heads of 128) come from
 * the "Every architecture field" table of the page "Ling 3.0 Flash"
 * (llm-architectures-explained).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   conv: depthwise, one 4-tap filter per channel, no bias, no activation;
 *         tap j multiplies the raw input 3-j tokens back, so tap 3 is the
 *         current token; history before a sequence start is zero, or the
 *         caller's conv state (three raw tokens, oldest first);
 *   L2 norm: x / sqrt(sum x^2 + 1e-6) over the head's dk channels;
 *   decay: log alpha = -softplus(g) per key channel; beta = sigmoid(b) per
 *          head; no query scale; output gate y = o * sigmoid(z), no norm.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define L2_EPS 1e-6

/* softplus(x) = log(1 + e^x), in a form that neither overflows nor loses
 * the small tail */
static double softplus(double x) {
    return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
}

/* logistic sigmoid 1 / (1 + e^-x) */
static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* ------------------------------------------------------------------------ */
/* thread pool over (sequence, head) items                                  */
/* ------------------------------------------------------------------------ */

typedef void (*item_fn)(void* ctx, int64_t item);

typedef struct {
    item_fn fn;
    void* ctx;
    int64_t n_items;
    int64_t next;
    pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int64_t i = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (i >= p->n_items) break;
        p->fn(p->ctx, i);
    }
    return NULL;
}

static void run_items(item_fn fn, void* ctx, int64_t n_items, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.n_items = n_items;
    p.next = 0;
    pthread_mutex_init(&p.mu, NULL);
    if (nthreads == 1) {
        pool_worker(&p);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &p);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------------------ */
/* preprocess: short conv, L2 norm, gates                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t T;
    int H, dk, dv, N;
    const int64_t* cu;
    const double *q_in, *k_in, *v_in, *wq, *wk, *wv, *g, *b;
    const double* cs_in;
    double* cs_out;
    double *q_out, *k_out, *v_out, *la_out, *beta_out;
} prep_ctx;

/* Raw input of channel c (row stride `width`) at position tau of sequence n,
 * tau < 0 reaching into the history. */
static double raw_at(const prep_ctx* P, const double* x, int64_t width, int64_t c,
                     int64_t cs_off, int n, int64_t tau) {
    if (tau >= 0) return x[(P->cu[n] + tau) * width + c];
    if (P->cs_in == NULL) return 0.0;
    int64_t cs_width = (int64_t)P->H * (2 * P->dk + P->dv);
    return P->cs_in[((int64_t)n * 3 + (3 + tau)) * cs_width + cs_off + c];
}

/* conv of one channel over one sequence: out[tau] = sum_j w[j] x(tau-3+j) */
static void conv_channel(const prep_ctx* P, const double* x, const double* w,
                         int64_t width, int64_t c, int64_t cs_off, int n,
                         double* out, int64_t out_stride) {
    int64_t L = P->cu[n + 1] - P->cu[n];
    const double* wc = w + c * 4;
    for (int64_t tau = 0; tau < L; ++tau) {
        double acc = 0.0;
        for (int j = 0; j < 4; ++j) acc += wc[j] * raw_at(P, x, width, c, cs_off, n, tau - 3 + j);
        out[(P->cu[n] + tau) * out_stride] = acc;
    }
    if (P->cs_out) {
        int64_t cs_width = (int64_t)P->H * (2 * P->dk + P->dv);
        for (int m = 0; m < 3; ++m)
            P->cs_out[((int64_t)n * 3 + m) * cs_width + cs_off + c] =
                raw_at(P, x, width, c, cs_off, n, L - 3 + m);
    }
}

static void l2norm_rows(double* x, int64_t t0, int64_t t1, int64_t stride, int64_t off, int d) {
    for (int64_t t = t0; t < t1; ++t) {
        double* r = x + t * stride + off;
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += r[i] * r[i];
        double inv = 1.0 / sqrt(ss + L2_EPS);
        for (int i = 0; i < d; ++i) r[i] *= inv;
    }
}

static void prep_item(void* vctx, int64_t item) {
    const prep_ctx* P = (const prep_ctx*)vctx;
    int n = (int)(item / P->H);
    int h = (int)(item % P->H);
    int dk = P->dk, dv = P->dv, H = P->H;
    int64_t wk_ = (int64_t)H * dk, wv_ = (int64_t)H * dv;
    int64_t t0 = P->cu[n], t1 = P->cu[n + 1];
    /* outputs are [T, H, d]: channel c of head h sits at t*H*d + h*d + i */
    for (int i = 0; i < dk; ++i) {
        int64_t c = (int64_t)h * dk + i;
        conv_channel(P, P->q_in, P->wq, wk_, c, 0, n, P->q_out + c, wk_);
        conv_channel(P, P->k_in, P->wk, wk_, c, wk_, n, P->k_out + c, wk_);
    }
    for (int i = 0; i < dv; ++i) {
        int64_t c = (int64_t)h * dv + i;
        conv_channel(P, P->v_in, P->wv, wv_, c, 2 * wk_, n, P->v_out + c, wv_);
    }
    l2norm_rows(P->q_out, t0, t1, wk_, (int64_t)h * dk, dk);
    l2norm_rows(P->k_out, t0, t1, wk_, (int64_t)h * dk, dk);
    for (int64_t t = t0; t < t1; ++t) {
        for (int i = 0; i < dk; ++i) {
            int64_t idx = t * wk_ + (int64_t)h * dk + i;
            P->la_out[idx] = -softplus(P->g[idx]);
        }
        P->beta_out[t * H + h] = sigmoid(P->b[t * H + h]);
    }
}

/*
 * Preprocess of a packed batch.
 *   cu [N+1] token offsets (cu[0] = 0, cu[N] = T);
 *   q_in, k_in [T, H*dk], v_in [T, H*dv] raw projections;
 *   wq, wk [H*dk, 4], wv [H*dv, 4] conv taps (tap 3 = current token);
 *   g [T, H*dk] decay logits, b [T, H] write logits;
 *   cs_in  NULL or [N, 3, H*(2dk+dv)] history (q | k | v channels, oldest first);
 *   cs_out NULL or the same shape: the last three raw tokens of each sequence
 *          (reaching into cs_in for sequences shorter than three); must not
 *          alias cs_in;
 *   outputs q_out, k_out [T, H, dk], v_out [T, H, dv], la_out [T, H, dk], beta_out [T, H].
 * Returns 0, or -1 on a bad argument.
 */
int kdao_preprocess(int64_t T, int H, int dk, int dv, const int64_t* cu, int N,
                    const double* q_in, const double* k_in, const double* v_in,
                    const double* wq, const double* wk, const double* wv,
                    const double* g, const double* b, const double* cs_in, double* cs_out,
                    double* q_out, double* k_out, double* v_out, double* la_out,
                    double* beta_out, int nthreads) {
    if (T < 0 || H <= 0 || dk <= 0 || dv <= 0 || N < 0 || !cu) return -1;
    if (cu[0] != 0 || cu[N] != T) return -1;
    if (cs_out && cs_out == cs_in) return -1;
    prep_ctx P = {T, H, dk, dv, N, cu, q_in, k_in, v_in, wq, wk, wv, g, b, cs_in, cs_out,
                  q_out, k_out, v_out, la_out, beta_out};
    run_items(prep_item, &P, (int64_t)N * H, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* recurrence                                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t T;
    int H, dk, dv, N;
    const int64_t* cu;
    const double *q, *k, *v, *la, *beta, *z, *S0;
    double *y, *S_out;
} rec_ctx;

static void rec_item(void* vctx, int64_t item) {
    const rec_ctx* R = (const rec_ctx*)vctx;
    int n = (int)(item / R->H);
    int h = (int)(item % R->H);
    int H = R->H, dk = R->dk, dv = R->dv;
    size_t sdim = (size_t)dk * dv;
    double* S = (double*)malloc(sizeof(double) * sdim);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    const double* s0 = R->S0 ? R->S0 + ((int64_t)n * H + h) * (int64_t)sdim : NULL;
    for (size_t i = 0; i < sdim; ++i) S[i] = s0 ? s0[i] : 0.0;

    for (int64_t t = R->cu[n]; t < R->cu[n + 1]; ++t) {
        const double* qt = R->q + (t * H + h) * dk;
        const double* kt = R->k + (t * H + h) * dk;
        const double* vt = R->v + (t * H + h) * dv;
        const double* lat = R->la + (t * H + h) * dk;
        double bt = R->beta[t * H + h];
        /* erase: per-channel decay of the rows of S */
        for (int i = 0; i < dk; ++i) {
            double a = exp(lat[i]);
            double* row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) row[j] *= a;
        }
        /* u = S'^T k */
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double* row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) u[j] += row[j] * kt[i];
        }
        /* write: S += beta k (v - u)^T */
        for (int i = 0; i < dk; ++i) {
            double* row = S + (size_t)i * dv;
            double bk = bt * kt[i];
            for (int j = 0; j < dv; ++j) row[j] += bk * (vt[j] - u[j]);
        }
        /* read: o = S^T q, then the output gate */
        double* yt = R->y + (t * H + h) * dv;
        for (int j = 0; j < dv; ++j) yt[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double* row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) yt[j] += row[j] * qt[i];
        }
        if (R->z) {
            const double* zt = R->z + (t * H + h) * dv;
            for (int j = 0; j < dv; ++j) yt[j] *= sigmoid(zt[j]);
        }
    }
    if (R->S_out) memcpy(R->S_out + ((int64_t)n * H + h) * (int64_t)sdim, S, sizeof(double) * sdim);
    free(u);
    free(S);
}

/*
 * Recurrence over a packed batch of already-preprocessed tokens.
 *   q, k, la [T, H, dk]; v [T, H, dv]; beta [T, H]; z NULL or [T, H, dv] logits;
 *   S0 NULL (zeros) or [N, H, dk, dv]; outputs y [T, H, dv] and
 *   S_out NULL or [N, H, dk, dv].
 * Returns 0, or -1 on a bad argument.
 */
int kdao_recurrence(int64_t T, int H, int dk, int dv, const int64_t* cu, int N,
                    const double* q, const double* k, const double* v, const double* la,
                    const double* beta, const double* z, const double* S0,
                    double* y, double* S_out, int nthreads) {
    if (T < 0 || H <= 0 || dk <= 0 || dv <= 0 || N < 0 || !cu) return -1;
    if (cu[0] != 0 || cu[N] != T) return -1;
    rec_ctx R = {T, H, dk, dv, N, cu, q, k, v, la, beta, z, S0, y, S_out};
    run_items(rec_item, &R, (int64_t)N * H, nthreads);
    return 0;
}

/*
 * Gradients of the recurrence above (reverse mode, fp64), for a scalar loss
 * whose gradients with respect to the outputs y and the final state are dy
 * and dS_final.  Each token's forward step is
 *     S' = Diag(alpha) S_prev;  u = S'^T k;  d = beta (v - u);
 *     S = S' + k d^T;  o = S^T q;  y = o * sigmoid(z)
 * and the pass walks the tokens backwards applying the adjoint of each line
 * in reverse order.  The states before every token are kept from a forward
 * pass (memory grows with the sequence: small cases only).
 */
typedef struct {
    int64_t T;
    int H, dk, dv, N;
    const int64_t* cu;
    const double *q, *k, *v, *la, *beta, *z, *S0, *dy, *dSf;
    double *dq, *dk_, *dv_, *dla, *dbeta, *dz, *dS0;
} bwd_ctx;

static void bwd_item(void* vctx, int64_t item) {
    const bwd_ctx* R = (const bwd_ctx*)vctx;
    int n = (int)(item / R->H), h = (int)(item % R->H);
    int H = R->H, dk = R->dk, dv = R->dv;
    int64_t t0 = R->cu[n], t1 = R->cu[n + 1], len = t1 - t0;
    size_t sdim = (size_t)dk * dv;
    double* hist = (double*)malloc(sizeof(double) * sdim * (size_t)(len + 1)); /* S before token t0 + i */
    double* Sp = (double*)malloc(sizeof(double) * sdim);  /* S' */
    double* St = (double*)malloc(sizeof(double) * sdim);  /* S after the token */
    double* dS = (double*)malloc(sizeof(double) * sdim);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dd = (double*)malloc(sizeof(double) * (size_t)dv);
    double* o = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dO = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dvec = (double*)malloc(sizeof(double) * (size_t)dv);
    const int64_t soff = ((int64_t)n * H + h) * (int64_t)sdim;
    for (size_t i = 0; i < sdim; ++i) hist[i] = R->S0 ? R->S0[soff + i] : 0.0;

    /* forward, keeping the state before each token */
    for (int64_t t = t0; t < t1; ++t) {
        const double* prev = hist + (size_t)(t - t0) * sdim;
        double* next = hist + (size_t)(t - t0 + 1) * sdim;
        const double* kt = R->k + (t * H + h) * dk;
        const double* vt = R->v + (t * H + h) * dv;
        const double* lat = R->la + (t * H + h) * dk;
        double bt = R->beta[t * H + h];
        for (int i = 0; i < dk; ++i) {
            const double al = exp(lat[i]);
            for (int j = 0; j < dv; ++j) next[(size_t)i * dv + j] = al * prev[(size_t)i * dv + j];
        }
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) u[j] += next[(size_t)i * dv + j] * kt[i];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) next[(size_t)i * dv + j] += bt * kt[i] * (vt[j] - u[j]);
    }

    /* backward */
    for (size_t i = 0; i < sdim; ++i) dS[i] = R->dSf ? R->dSf[soff + i] : 0.0;
    for (int64_t t = t1 - 1; t >= t0; --t) {
        const double* prev = hist + (size_t)(t - t0) * sdim;
        const double* qt = R->q + (t * H + h) * dk;
        const double* kt = R->k + (t * H + h) * dk;
        const double* vt = R->v + (t * H + h) * dv;
        const double* lat = R->la + (t * H + h) * dk;
        const double* dyt = R->dy + (t * H + h) * dv;
        double bt = R->beta[t * H + h];
        /* recompute this token's forward values */
        for (int i = 0; i < dk; ++i) {
            const double al = exp(lat[i]);
            for (int j = 0; j < dv; ++j) Sp[(size_t)i * dv + j] = al * prev[(size_t)i * dv + j];
        }
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) u[j] += Sp[(size_t)i * dv + j] * kt[i];
        for (int j = 0; j < dv; ++j) dvec[j] = bt * (vt[j] - u[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) St[(size_t)i * dv + j] = Sp[(size_t)i * dv + j] + kt[i] * dvec[j];
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) o[j] += St[(size_t)i * dv + j] * qt[i];
        /* y = o * sigmoid(z) */
        if (R->z) {
            const double* zt = R->z + (t * H + h) * dv;
            double* dzt = R->dz + (t * H + h) * dv;
            for (int j = 0; j < dv; ++j) {
                double s = sigmoid(zt[j]);
                dO[j] = dyt[j] * s;
                dzt[j] = dyt[j] * o[j] * s * (1.0 - s);
            }
        } else {
            for (int j = 0; j < dv; ++j) dO[j] = dyt[j];
        }
        /* o = S^T q */
        double* dqt = R->dq + (t * H + h) * dk;
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += St[(size_t)i * dv + j] * dO[j];
                dS[(size_t)i * dv + j] += qt[i] * dO[j];
            }
            dqt[i] = acc;
        }
        /* S = S' + k d^T */
        double* dkt = R->dk_ + (t * H + h) * dk;
        for (int j = 0; j < dv; ++j) dd[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += dS[(size_t)i * dv + j] * dvec[j];
                dd[j] += dS[(size_t)i * dv + j] * kt[i];
            }
            dkt[i] = acc;
        }
        /* d = beta (v - u) */
        double db = 0.0;
        double* dvt = R->dv_ + (t * H + h) * dv;
        for (int j = 0; j < dv; ++j) {
            db += dd[j] * (vt[j] - u[j]);
            dvt[j] = bt * dd[j];
            dd[j] = -bt * dd[j]; /* now du */
        }
        R->dbeta[t * H + h] = db;
        /* u = S'^T k: dS' = dS + k du^T; dk += S' du */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += Sp[(size_t)i * dv + j] * dd[j];
                dS[(size_t)i * dv + j] += kt[i] * dd[j];
            }
            dkt[i] += acc;
        }
        /* S' = Diag(alpha) S_prev */
        double* dlat = R->dla + (t * H + h) * dk;
        for (int i = 0; i < dk; ++i) {
            const double al = exp(lat[i]);
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
                acc += dS[(size_t)i * dv + j] * prev[(size_t)i * dv + j];
                dS[(size_t)i * dv + j] *= al;
            }
            dlat[i] = al * acc;
        }
    }
    if (R->dS0) memcpy(R->dS0 + soff, dS, sizeof(double) * sdim);
    free(dvec); free(dO); free(o); free(dd); free(u); free(dS); free(St); free(Sp); free(hist);
}

/*
 * dq, dk, dla [T, H, dk]; dv [T, H, dv]; dbeta [T, H]; dz [T, H, dv] (only
 * with z); dS0 NULL or [N, H, dk, dv].  dy [T, H, dv]; dS_final NULL (zero)
 * or [N, H, dk, dv].  Returns 0, or -1 on a bad argument.
 */
int kdao_recurrence_backward(int64_t T, int H, int dk, int dv, const int64_t* cu, int N,
                             const double* q, const double* k, const double* v, const double* la,
                             const double* beta, const double* z, const double* S0,
                             const double* dy, const double* dS_final,
                             double* dq, double* dk_, double* dv_, double* dla, double* dbeta,
                             double* dz, double* dS0, int nthreads) {
    if (T < 0 || H <= 0 || dk <= 0 || dv <= 0 || N < 0 || !cu || !dy) return -1;
    if (cu[0] != 0 || cu[N] != T) return -1;
    if (z && !dz) return -1;
    bwd_ctx R = {T, H, dk, dv, N, cu, q, k, v, la, beta, z, S0, dy, dS_final,
                 dq, dk_, dv_, dla, dbeta, dz, dS0};
    run_items(bwd_item, &R, (int64_t)N * H, nthreads);
    return 0;
}
