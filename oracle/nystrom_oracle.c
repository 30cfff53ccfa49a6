/*
 * Streaming Nystrom attention -- CPU ORACLE.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load,
 * call or link this file.  The HIP library never includes, links or calls it,
 * and it includes nothing of the HIP library: the two share no code.
 *
 * What it computes: the streaming per-GQA-group operator defined on the docs.rs
 * source page of cortiq_engine/nystrom.rs (cortiq-engine 0.5.71), written as a
 * plain, slow, obviously checkable program:
 *
 *   out(q_p) = (sum_{j near} e_j v_j + F M T_far) / (sum_{j near} e_j + F M Z_far)
 *   near = { j : p - j < w } u { j < sink },   e_j = exp(q.k_j * scale)
 *   F_a  = exp(q . k~_a * scale)            M = pinv_reg(exp(Q~ K~^T * scale))
 *   T_far[b] = sum_{j far} exp(q~_b . k_j * scale) v_j,  Z_far[b] likewise
 *
 * (module doc at the top of that page).  Every function below cites the item of
 * that page it follows: NystromState::{new_group, prefill_group, step_group,
 * advance}, NystromGroup::prefill_shared, NystromHead::{seal, step,
 * far_insert}, seg_means, ridge_pinv, cholesky, and the constants RIDGE_REL,
 * DEN_EPS, EXACT_SLACK.
 *
 * Precision: inputs are f32 (as on the pages).  The frozen landmarks K~, Q~ and
 * the mixing matrix M are rounded to f32 once, because the pages store them as
 * f32 (prefill_shared, seal).  The score scale is the pages' f32 value
 * 1/sqrt(d) widened to f64 (prefill_shared sets it in f32 and seal widens it).
 * Everything else -- dots, exps, running maxima, T^/Z^ accumulators, the joint
 * division -- is carried in f64, so the oracle measures the method rather than
 * one particular f32 rounding order.
 *
 * Two readings where the pages leave a step open (both are listed with their
 * justification in the design notes of the repository):
 *   R5  a far denominator of exactly 0 keeps the far field (the page's test is
 *       "far_den >= 0").
 *   R7  when the aggregate rectifier drops the far field, the near weights are
 *       shifted by the near maximum c instead of the joint shift c_all.  The
 *       softmax formula is shift-invariant, so this is the same value; it only
 *       differs from the page's f32 code where that code's near weights would
 *       all underflow (c_all - c beyond the exp range).
 *
 * No blocking, fusion or reordering beyond what the page states: every loop runs
 * over the same index in the same order as the page describes the step.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Constants of the nystrom.rs source page: RIDGE_REL, DEN_EPS, EXACT_SLACK;
 * the 12-try ridge growth of ridge_pinv. */
#define ORC_RIDGE_REL 1e-6
#define ORC_DEN_EPS 1e-30
#define ORC_EXACT_SLACK 8
#define ORC_RIDGE_TRIES 12

/* O1Rect (nystrom.rs source page): Aggregate is the default rectifier. */
#define ORC_RECT_AGGREGATE 0
#define ORC_RECT_FM 1

/* Per-head diagnostics of one output row (not part of the method; the tests use
 * them to recognise rows where the aggregate rectifier's decision is within
 * rounding of its threshold). */
typedef struct {
    double far_den; /* sum_b gain_b * Z^_b before the rectifier                 */
    double far_abs; /* sum_b |gain_b * Z^_b|                                   */
    double den;     /* joint denominator actually divided by (before the floor) */
    double shift;   /* the exp shift the near weights used                      */
    int have_far;   /* far_len > 0                                              */
    int keep;       /* far field kept by the rectifier                          */
} orc_diag;

typedef struct orc_group {
    /* NystromState::new_group settings */
    int m, w, sink, hpk, rect;
    double ridge_rel; /* RIDGE_REL unless a test overrides it */
    /* geometry fixed by prefill_shared */
    int d, dv, t, m_eff, exact_only, sealed;
    double scale;
    /* shared per group: window ring, sinks, key landmarks */
    int cap, win_len, win_head, sink_len;
    float *win_k, *win_v, *sink_k, *sink_v;
    float *k_tilde;    /* [m_eff][d], f32 as stored by the page  */
    double *k_tilde64; /* [m_eff][d], f64 segment means          */
    /* private per Q head */
    float *q_tilde;    /* [hpk][m_eff][d] */
    double *q_tilde64; /* [hpk][m_eff][d] */
    double *au;        /* [hpk][m_eff][m_eff], f64 exp-Gram     */
    float *mu;         /* [hpk][m_eff][m_eff], row a = key landmark, column b = query landmark */
    double *lambda;    /* [hpk] ridge actually used */
    int *tries;        /* [hpk] Cholesky attempts (ORC_RIDGE_TRIES + 1 = fallback) */
    double *t_hat;     /* [hpk][m_eff][dv] at scale e^{-m_max[i]} */
    double *z_hat;     /* [hpk][m_eff] */
    double *m_max;     /* [hpk][m_eff] running max of far logits */
    long *far_len;     /* [hpk] */
    /* scratch, sized at prefill so step allocates nothing in skeleton mode */
    double *scr_s, *scr_fh, *scr_u, *scr_l, *scr_acc;
    int scr_s_cap;
    /* length the page's per-head score scratch has (what memory_bytes counts):
     * sink + w after seal, 0 after seal_exact, sink_len + win_len after a step */
    int scr_s_len;
} orc_group;

static double f32_scale_of(int d)
{
    /* prefill_shared: scale = 1 / sqrt(d) computed in f32; seal widens it. */
    float s = 1.0f / sqrtf((float)d);
    return (double)s;
}

static double dot_ff(const float *a, const float *b, int n)
{
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += (double)a[c] * (double)b[c];
    return s;
}

/* ------------------------------------------------------------------------- */
/* seg_means (nystrom.rs source page): contiguous segment means of the rows of
 * xs [t][d].  Segment i covers rows floor(i*t/m) .. floor((i+1)*t/m) - 1; rows
 * are summed in f64 in order, then scaled by 1/(row count).                  */
void orc_seg_means(const float *xs, int t, int d, int m, double *out)
{
    for (int i = 0; i < m; ++i) {
        long lo = (long)i * t / m, hi = (long)(i + 1) * t / m;
        double *o = out + (size_t)i * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        for (long j = lo; j < hi; ++j)
            for (int c = 0; c < d; ++c) o[c] += (double)xs[(size_t)j * d + c];
        double inv = 1.0 / (double)(hi - lo);
        for (int c = 0; c < d; ++c) o[c] *= inv;
    }
}

/* cholesky (nystrom.rs source page): the lower-triangular L with L L^T = G
 * for a symmetric positive definite G [n][n], written over G's lower triangle
 * (the strict upper triangle is left as it was).  Column k at a time: the
 * pivot is what remains of G[k][k] after the earlier columns' contributions;
 * it must be positive and finite, else the factorisation fails (returns 0).
 * Then L[k][k] = sqrt(pivot), L[i][k] = (remaining G[i][k]) / L[k][k] for
 * i > k, and column k's contribution L[i][k] L[j][k] is taken off every
 * remaining entry (i >= j > k).  Returns 1 on success.                      */
int orc_cholesky(double *g, int n)
{
    for (int k = 0; k < n; ++k) {
        const double pivot = g[k * n + k];
        if (!(pivot > 0.0) || !isfinite(pivot)) return 0;
        const double lkk = sqrt(pivot);
        g[k * n + k] = lkk;
        for (int i = k + 1; i < n; ++i) g[i * n + k] /= lkk;
        for (int j = k + 1; j < n; ++j)
            for (int i = j; i < n; ++i) g[i * n + j] -= g[i * n + k] * g[j * n + k];
    }
    return 1;
}

/* ridge_pinv (nystrom.rs source page): the ridge-regularised pseudo-inverse
 *   M = (A^T A + lambda I)^-1 A^T
 * of a square A [n][n], with lambda = ridge_rel * max(tr(A^T A) / n, DBL_MIN).
 * G = A^T A + lambda I = L L^T (cholesky above), so M follows from two
 * triangular solves with A^T as the right-hand side: L Y = A^T, then
 * L^T M = Y.  When the factorisation fails, lambda is multiplied by 10 and G
 * rebuilt, up to 12 attempts; after that M is the scaled identity
 * I / max(tr(A^T A) / n, DBL_MIN).
 * Returns the attempt that factored (1..12), or 13 for the scaled identity.
 * *lambda_out receives the lambda that factored; after the fallback it is
 * the initial lambda times 10^12 (the value the growth reached).           */
int orc_ridge_pinv(const double *a, int n, double ridge_rel, double *out, double *lambda_out)
{
    const size_t nn = (size_t)n * n;
    double *gram = (double *)calloc(nn, sizeof(double)); /* A^T A            */
    double *fac = (double *)malloc(sizeof(double) * nn);  /* G, then L        */
    /* A^T A as the sum over rows r of A of the outer product a_r a_r^T. */
    for (int r = 0; r < n; ++r)
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) gram[i * n + j] += a[r * n + i] * a[r * n + j];
    double trace = 0.0;
    for (int i = 0; i < n; ++i) trace += gram[i * n + i];
    const double scale_ref = trace / (double)n > DBL_MIN ? trace / (double)n : DBL_MIN;
    double lambda = ridge_rel * scale_ref;

    int attempt = 1;
    for (; attempt <= ORC_RIDGE_TRIES; ++attempt, lambda *= 10.0) {
        memcpy(fac, gram, sizeof(double) * nn);
        for (int i = 0; i < n; ++i) fac[i * n + i] += lambda;
        if (orc_cholesky(fac, n)) break;
    }
    if (attempt <= ORC_RIDGE_TRIES) {
        /* out starts as A^T, becomes Y (forward, rows top-down), then M
         * (backward, rows bottom-up); each row update runs over every
         * column of the right-hand side at once. */
        for (int i = 0; i < n; ++i)
            for (int c = 0; c < n; ++c) out[i * n + c] = a[c * n + i];
        for (int i = 0; i < n; ++i) {
            for (int k = 0; k < i; ++k)
                for (int c = 0; c < n; ++c) out[i * n + c] -= fac[i * n + k] * out[k * n + c];
            for (int c = 0; c < n; ++c) out[i * n + c] /= fac[i * n + i];
        }
        for (int i = n - 1; i >= 0; --i) {
            for (int k = i + 1; k < n; ++k)
                for (int c = 0; c < n; ++c) out[i * n + c] -= fac[k * n + i] * out[k * n + c];
            for (int c = 0; c < n; ++c) out[i * n + c] /= fac[i * n + i];
        }
    } else {
        for (size_t t = 0; t < nn; ++t) out[t] = 0.0;
        for (int i = 0; i < n; ++i) out[i * n + i] = 1.0 / scale_ref;
    }
    if (lambda_out) *lambda_out = lambda;
    free(gram);
    free(fac);
    return attempt;
}

/* Exact softmax attention over n keys, brute force (the operator the near field
 * reproduces when the far set is empty).                                      */
void orc_exact_attention(const float *q, const float *ks, const float *vs, int n, int d, int dv,
                         double scale, double *out)
{
    double c = -INFINITY;
    double *lg = (double *)malloc(sizeof(double) * (n > 0 ? n : 1));
    for (int j = 0; j < n; ++j) {
        lg[j] = dot_ff(q, ks + (size_t)j * d, d) * scale;
        if (lg[j] > c) c = lg[j];
    }
    double den = 0.0;
    for (int e = 0; e < dv; ++e) out[e] = 0.0;
    for (int j = 0; j < n; ++j) {
        double p = exp(lg[j] - c);
        den += p;
        for (int e = 0; e < dv; ++e) out[e] += p * (double)vs[(size_t)j * dv + e];
    }
    for (int e = 0; e < dv; ++e) out[e] /= den;
    free(lg);
}

/* ------------------------------------------------------------------------- */
static void release_arrays(orc_group *g)
{
    free(g->win_k); free(g->win_v); free(g->sink_k); free(g->sink_v);
    free(g->k_tilde); free(g->k_tilde64);
    free(g->q_tilde); free(g->q_tilde64); free(g->au); free(g->mu);
    free(g->lambda); free(g->tries);
    free(g->t_hat); free(g->z_hat); free(g->m_max); free(g->far_len);
    free(g->scr_s); free(g->scr_fh); free(g->scr_u); free(g->scr_l); free(g->scr_acc);
}

/* NystromState::new_group (nystrom.rs source page): settings only; requires
 * m >= 4, w >= 1, q_heads >= 1.  Returns NULL when those fail.               */
orc_group *orc_new_group(int m, int w, int sink, int q_heads, int rect)
{
    if (m < 4 || w < 1 || q_heads < 1 || sink < 0) return NULL;
    if (rect != ORC_RECT_AGGREGATE && rect != ORC_RECT_FM) return NULL;
    orc_group *g = (orc_group *)calloc(1, sizeof(orc_group));
    g->m = m; g->w = w; g->sink = sink; g->hpk = q_heads; g->rect = rect;
    g->ridge_rel = ORC_RIDGE_REL;
    g->exact_only = 1;
    return g;
}

void orc_free(orc_group *g)
{
    if (!g) return;
    release_arrays(g);
    free(g);
}

/* Test hook: the ridge factor (RIDGE_REL on the page). */
void orc_set_ridge_rel(orc_group *g, double ridge_rel) { g->ridge_rel = ridge_rel; }

/* NystromHead::far_insert (nystrom.rs source page): head h absorbs window slot
 * `slot`.  Per landmark i: l = q~_i . k_slot * scale; if l raises the running
 * max, the old mass is rescaled by e^{max_old - l} (0 when max_old = -inf);
 * then Z^_i += e^{l - max}, T^_i += e^{l - max} v_slot.  far_len += 1.        */
static void far_insert(orc_group *g, int h, int slot)
{
    const int d = g->d, dv = g->dv, m = g->m_eff;
    const float *kslot = g->win_k + (size_t)slot * d;
    const float *vslot = g->win_v + (size_t)slot * dv;
    const float *qt = g->q_tilde + (size_t)h * m * d;
    double *th = g->t_hat + (size_t)h * m * dv;
    double *zh = g->z_hat + (size_t)h * m;
    double *mx = g->m_max + (size_t)h * m;
    double *l = g->scr_l;
    for (int i = 0; i < m; ++i) l[i] = dot_ff(qt + (size_t)i * d, kslot, d) * g->scale;
    for (int i = 0; i < m; ++i) {
        if (l[i] > mx[i]) {
            double r = exp(mx[i] - l[i]);
            zh[i] *= r;
            for (int e = 0; e < dv; ++e) th[(size_t)i * dv + e] *= r;
            mx[i] = l[i];
        }
        double ei = exp(l[i] - mx[i]);
        zh[i] += ei;
        for (int e = 0; e < dv; ++e) th[(size_t)i * dv + e] += ei * (double)vslot[e];
    }
    g->far_len[h] += 1;
}

static void ensure_window_cap(orc_group *g, int rows)
{
    if (rows <= g->cap) return;
    int cap = g->cap ? g->cap : 16;
    while (cap < rows) cap *= 2;
    g->win_k = (float *)realloc(g->win_k, sizeof(float) * (size_t)cap * g->d);
    g->win_v = (float *)realloc(g->win_v, sizeof(float) * (size_t)cap * g->dv);
    g->cap = cap;
}

static void ensure_score_cap(orc_group *g, int n)
{
    if (n <= g->scr_s_cap) return;
    int cap = n + 64;
    g->scr_s = (double *)realloc(g->scr_s, sizeof(double) * cap);
    g->scr_s_cap = cap;
}

/* NystromState::advance (nystrom.rs source page): push (k, v) into the shared
 * window.  Skeleton mode with a full ring: every head absorbs the oldest slot
 * (one eviction, q_heads insertions), the slot is overwritten and win_head moves
 * on mod w.  Exact-only mode appends.  Otherwise the ring fills at win_len.   */
static void advance(orc_group *g, const float *k, const float *v)
{
    const int d = g->d, dv = g->dv;
    if (!g->exact_only && g->win_len == g->w) {
        int slot = g->win_head;
        for (int h = 0; h < g->hpk; ++h) far_insert(g, h, slot);
        memcpy(g->win_k + (size_t)slot * d, k, sizeof(float) * d);
        memcpy(g->win_v + (size_t)slot * dv, v, sizeof(float) * dv);
        g->win_head = (g->win_head + 1) % g->w;
    } else if (g->exact_only) {
        ensure_window_cap(g, g->win_len + 1);
        memcpy(g->win_k + (size_t)g->win_len * d, k, sizeof(float) * d);
        memcpy(g->win_v + (size_t)g->win_len * dv, v, sizeof(float) * dv);
        g->win_len += 1;
    } else {
        memcpy(g->win_k + (size_t)g->win_len * d, k, sizeof(float) * d);
        memcpy(g->win_v + (size_t)g->win_len * dv, v, sizeof(float) * dv);
        g->win_len += 1;
    }
}

/* NystromHead::step (nystrom.rs source page): the output row of head h for
 * query q.  Near part: exact logits over the sink rows and every window slot;
 * advance has run before this, so the slots already hold this position's own
 * key.  Far part: head h's T^, Z^ and running maxima through F M.           */
static void head_step(orc_group *g, int h, const float *q, double *out, double *out_alt,
                      orc_diag *diag)
{
    const int d = g->d, dv = g->dv, m = g->m_eff;
    const int ns = g->sink_len, n = ns + g->win_len;
    ensure_score_cap(g, n);
    double *lg = g->scr_s;

    /* Near field: exact logits over sinks then window slots; shared max c. */
    double c = -INFINITY;
    for (int s = 0; s < ns; ++s) {
        lg[s] = dot_ff(q, g->sink_k + (size_t)s * d, d) * g->scale;
        if (lg[s] > c) c = lg[s];
    }
    for (int s = 0; s < g->win_len; ++s) {
        lg[ns + s] = dot_ff(q, g->win_k + (size_t)s * d, d) * g->scale;
        if (lg[ns + s] > c) c = lg[ns + s];
    }

    /* Far field: row shift f, fh = e^{s - f}, u = fh . M, joint shift c_all,
     * gain_b = u_b e^{f + m_max_b - c_all}, far_den = sum gain_b Z^_b.       */
    double far_den = 0.0, far_abs = 0.0, c_all = c;
    int have_far = g->far_len[h] > 0, keep = 0;
    double *fh = g->scr_fh, *gain = g->scr_u;
    if (have_far) {
        const double *mx = g->m_max + (size_t)h * m;
        const double *zh = g->z_hat + (size_t)h * m;
        const float *mu = g->mu + (size_t)h * m * m;
        double f = -INFINITY;
        for (int a = 0; a < m; ++a) {
            fh[a] = dot_ff(q, g->k_tilde + (size_t)a * d, d) * g->scale;
            if (fh[a] > f) f = fh[a];
        }
        for (int a = 0; a < m; ++a) fh[a] = exp(fh[a] - f);
        for (int b = 0; b < m; ++b) {
            double s = 0.0;
            for (int a = 0; a < m; ++a) s += fh[a] * (double)mu[(size_t)a * m + b];
            /* O1Rect::Fm clamps this m-vector at zero; Aggregate leaves it. */
            gain[b] = (g->rect == ORC_RECT_FM && s < 0.0) ? 0.0 : s;
        }
        for (int b = 0; b < m; ++b)
            if (f + mx[b] > c_all) c_all = f + mx[b];
        for (int b = 0; b < m; ++b) {
            gain[b] *= exp(f + mx[b] - c_all);
            far_den += gain[b] * zh[b];
            far_abs += fabs(gain[b] * zh[b]);
        }
        keep = far_den >= 0.0; /* aggregate rectifier; R5: 0 keeps */
    }

    /* Joint numerator / denominator and the single division.  Branch `kept`
     * writes `out`; the other branch (when the far field exists) goes to
     * out_alt so a caller can recognise near-threshold rows. */
    for (int pass = 0; pass < 2; ++pass) {
        int use_far = (pass == 0) ? keep : (have_far && !keep);
        double *dst = (pass == 0) ? out : out_alt;
        if (pass == 1 && (!have_far || !dst)) break;
        double shift = use_far ? c_all : c; /* R7 */
        double den = use_far ? far_den : 0.0;
        double *acc = g->scr_acc;
        for (int e = 0; e < dv; ++e) acc[e] = 0.0;
        if (use_far) {
            const double *th = g->t_hat + (size_t)h * m * dv;
            for (int b = 0; b < m; ++b)
                for (int e = 0; e < dv; ++e) acc[e] += gain[b] * th[(size_t)b * dv + e];
        }
        for (int s = 0; s < n; ++s) {
            double p = exp(lg[s] - shift);
            const float *vv = s < ns ? g->sink_v + (size_t)s * dv : g->win_v + (size_t)(s - ns) * dv;
            den += p;
            for (int e = 0; e < dv; ++e) acc[e] += p * (double)vv[e];
        }
        double den_f = den > ORC_DEN_EPS ? den : ORC_DEN_EPS;
        for (int e = 0; e < dv; ++e) dst[e] = acc[e] / den_f;
        if (pass == 0 && diag) {
            diag->far_den = far_den;
            diag->far_abs = far_abs;
            diag->den = den;
            diag->shift = shift;
            diag->have_far = have_far;
            diag->keep = keep;
        }
    }
}

/* NystromGroup::prefill_shared + NystromHead::seal + the replay of
 * NystromState::prefill_group (nystrom.rs source page).
 *
 *   qs [q_heads][t][d], ks [t][d], vs [t][dv] are the prompt.
 *   frozen_kt [m_eff][d], frozen_qt [q_heads][m_eff][d], frozen_mu
 *   [q_heads][m_eff][m_eff] (each may be NULL) replace the landmarks / mixing
 *   matrix the page would compute -- a test hook; NULL follows the page.
 *   replay_out [t][q_heads][dv] (may be NULL) receives, for every replayed
 *   position j >= sink, the output step_group would give for that head's query
 *   at j right after j was inserted (rows j < sink are left untouched).
 * Returns 0 on success, -1 on bad arguments.                                 */
int orc_prefill_group(orc_group *g, const float *qs, const float *ks, const float *vs, int t,
                      int d, int dv, const float *frozen_kt, const float *frozen_qt,
                      const float *frozen_mu, double *replay_out)
{
    if (!g || t < 1 || d < 1 || dv < 1) return -1;
    release_arrays(g);
    g->win_k = g->win_v = g->sink_k = g->sink_v = g->k_tilde = g->q_tilde = g->mu = NULL;
    g->k_tilde64 = g->q_tilde64 = g->au = g->lambda = g->t_hat = g->z_hat = g->m_max = NULL;
    g->tries = NULL; g->far_len = NULL;
    g->scr_s = g->scr_fh = g->scr_u = g->scr_l = g->scr_acc = NULL;
    g->cap = 0; g->scr_s_cap = 0;

    /* prefill_shared: geometry, exact-only test, sinks, m_eff, K~. */
    g->d = d; g->dv = dv; g->t = t;
    g->scale = f32_scale_of(d);
    g->win_len = 0; g->win_head = 0; g->sink_len = 0;
    g->exact_only = t <= g->w + g->sink + ORC_EXACT_SLACK;
    g->far_len = (long *)calloc(g->hpk, sizeof(long));
    g->scr_acc = (double *)calloc(dv, sizeof(double));
    g->sealed = 1;

    if (g->exact_only) {
        /* Every prompt key is a permanent exact key; no skeleton. */
        ensure_window_cap(g, t + 64);
        memcpy(g->win_k, ks, sizeof(float) * (size_t)t * d);
        memcpy(g->win_v, vs, sizeof(float) * (size_t)t * dv);
        g->win_len = t;
        g->m_eff = 0;
        ensure_score_cap(g, t + 64);
        g->scr_s_len = 0; /* seal_exact reserves the scratch but leaves it empty */
        return 0;
    }

    g->sink_len = g->sink;
    g->sink_k = (float *)malloc(sizeof(float) * (size_t)(g->sink ? g->sink : 1) * d);
    g->sink_v = (float *)malloc(sizeof(float) * (size_t)(g->sink ? g->sink : 1) * dv);
    memcpy(g->sink_k, ks, sizeof(float) * (size_t)g->sink * d);
    memcpy(g->sink_v, vs, sizeof(float) * (size_t)g->sink * dv);

    int m_eff = t / 8;
    if (m_eff < 4) m_eff = 4;
    if (m_eff > g->m) m_eff = g->m;
    g->m_eff = m_eff;
    const int m = m_eff, H = g->hpk;

    g->k_tilde64 = (double *)malloc(sizeof(double) * (size_t)m * d);
    g->k_tilde = (float *)malloc(sizeof(float) * (size_t)m * d);
    orc_seg_means(ks, t, d, m, g->k_tilde64);
    for (size_t i = 0; i < (size_t)m * d; ++i) g->k_tilde[i] = (float)g->k_tilde64[i];
    if (frozen_kt) {
        memcpy(g->k_tilde, frozen_kt, sizeof(float) * (size_t)m * d);
        for (size_t i = 0; i < (size_t)m * d; ++i) g->k_tilde64[i] = (double)frozen_kt[i];
    }

    /* The ring holds exactly w slots in skeleton mode. */
    g->win_k = (float *)calloc((size_t)g->w * d, sizeof(float));
    g->win_v = (float *)calloc((size_t)g->w * dv, sizeof(float));
    g->cap = g->w;
    ensure_score_cap(g, g->sink + g->w);
    g->scr_s_len = g->sink + g->w;
    g->scr_fh = (double *)malloc(sizeof(double) * m);
    g->scr_u = (double *)malloc(sizeof(double) * m);
    g->scr_l = (double *)malloc(sizeof(double) * m);

    /* seal, per head: Q~, Au in f64, M = ridge_pinv(Au) rounded to f32, empty
     * far field with running max -inf. */
    g->q_tilde64 = (double *)malloc(sizeof(double) * (size_t)H * m * d);
    g->q_tilde = (float *)malloc(sizeof(float) * (size_t)H * m * d);
    g->au = (double *)malloc(sizeof(double) * (size_t)H * m * m);
    g->mu = (float *)malloc(sizeof(float) * (size_t)H * m * m);
    g->lambda = (double *)calloc(H, sizeof(double));
    g->tries = (int *)calloc(H, sizeof(int));
    g->t_hat = (double *)calloc((size_t)H * m * dv, sizeof(double));
    g->z_hat = (double *)calloc((size_t)H * m, sizeof(double));
    g->m_max = (double *)malloc(sizeof(double) * (size_t)H * m);
    double *mu64 = (double *)malloc(sizeof(double) * (size_t)m * m);
    for (int h = 0; h < H; ++h) {
        double *qt64 = g->q_tilde64 + (size_t)h * m * d;
        float *qt = g->q_tilde + (size_t)h * m * d;
        orc_seg_means(qs + (size_t)h * t * d, t, d, m, qt64);
        for (size_t i = 0; i < (size_t)m * d; ++i) qt[i] = (float)qt64[i];
        if (frozen_qt) {
            memcpy(qt, frozen_qt + (size_t)h * m * d, sizeof(float) * (size_t)m * d);
            for (size_t i = 0; i < (size_t)m * d; ++i) qt64[i] = (double)qt[i];
        }
        double *au = g->au + (size_t)h * m * m;
        for (int i = 0; i < m; ++i)
            for (int j = 0; j < m; ++j) {
                double s = 0.0;
                for (int c = 0; c < d; ++c) s += qt64[(size_t)i * d + c] * g->k_tilde64[(size_t)j * d + c];
                au[i * m + j] = exp(s * g->scale);
            }
        float *mu = g->mu + (size_t)h * m * m;
        if (frozen_mu) {
            memcpy(mu, frozen_mu + (size_t)h * m * m, sizeof(float) * (size_t)m * m);
            g->tries[h] = 0;
            g->lambda[h] = 0.0;
        } else {
            g->tries[h] = orc_ridge_pinv(au, m, g->ridge_rel, mu64, &g->lambda[h]);
            for (int i = 0; i < m * m; ++i) mu[i] = (float)mu64[i];
        }
        for (int i = 0; i < m; ++i) g->m_max[(size_t)h * m + i] = -INFINITY;
    }
    free(mu64);

    /* Replay positions sink..t-1 through advance (window fill, then delayed
     * far insertion), optionally recording each head's output at j. */
    for (int j = g->sink; j < t; ++j) {
        advance(g, ks + (size_t)j * d, vs + (size_t)j * dv);
        if (replay_out)
            for (int h = 0; h < H; ++h)
                head_step(g, h, qs + ((size_t)h * t + j) * d,
                          replay_out + ((size_t)j * H + h) * dv, NULL, NULL);
    }
    return 0;
}

/* NystromState::step_group (nystrom.rs source page): insert (k, v) once --
 * before any output, since the current token is in its own window -- then each
 * head's output.  q_all [q_heads][d], out_all [q_heads][dv]; out_alt (may be
 * NULL) gets each head's output under the other rectifier branch, diag (may
 * be NULL) one record per head.  Returns 0, or -1 before prefill.           */
int orc_step_group(orc_group *g, const float *q_all, const float *k, const float *v,
                   double *out_all, double *out_alt, orc_diag *diag)
{
    if (!g || !g->sealed) return -1;
    advance(g, k, v);
    g->scr_s_len = g->sink_len + g->win_len; /* every head's step resizes its scratch */
    for (int h = 0; h < g->hpk; ++h)
        head_step(g, h, q_all + (size_t)h * g->d, out_all + (size_t)h * g->dv,
                  out_alt ? out_alt + (size_t)h * g->dv : NULL, diag ? diag + h : NULL);
    return 0;
}

/* ---- getters (NystromState::{far_len, num_q_heads, memory_bytes}) -------- */
int orc_m_eff(const orc_group *g) { return g->m_eff; }
int orc_exact_only(const orc_group *g) { return g->exact_only; }
int orc_win_len(const orc_group *g) { return g->win_len; }
int orc_win_head(const orc_group *g) { return g->win_head; }
int orc_sink_len(const orc_group *g) { return g->sink_len; }
int orc_num_q_heads(const orc_group *g) { return g->hpk; }
long orc_far_len(const orc_group *g, int h) { return g->far_len ? g->far_len[h] : 0; }
double orc_scale(const orc_group *g) { return g->scale; }
double orc_lambda(const orc_group *g, int h) { return g->lambda ? g->lambda[h] : 0.0; }
int orc_ridge_tries(const orc_group *g, int h) { return g->tries ? g->tries[h] : 0; }

/* NystromState::memory_bytes (nystrom.rs source page): f32 words of the
 * vectors the group holds (window, sinks, K~) and each head holds (T^, Z^,
 * running max, Q~, M and its four scratch vectors), counted by length, as the
 * page counts them, times 4 bytes.
 *   skeleton:   window w (d + dv), sinks sink (d + dv), K~ m d; per head
 *               m dv + m + m + m d + m m + (sink + w) + 3 m.
 *   exact-only: window (t + steps)(d + dv); per head only the score scratch,
 *               empty until the first step and sized to every key after it.
 * A group never prefilled holds nothing.  (State an earlier prompt left in a
 * reused group is not counted: this oracle releases it at every prefill.)   */
size_t orc_memory_bytes(const orc_group *g)
{
    if (!g->sealed) return 0;
    const size_t d = (size_t)g->d, dv = (size_t)g->dv, m = (size_t)g->m_eff;
    size_t shared, per_head;
    if (g->exact_only) {
        shared = (size_t)g->win_len * (d + dv);
        per_head = (size_t)g->scr_s_len;
    } else {
        shared = (size_t)g->w * (d + dv) + (size_t)g->sink_len * (d + dv) + m * d;
        per_head = m * dv + m + m + m * d + m * m + (size_t)g->scr_s_len + 3 * m;
    }
    return (shared + (size_t)g->hpk * per_head) * sizeof(float);
}

/* Copies of the state.  Any pointer may be NULL.  Shapes: sink [sink_len][d|dv],
 * window [win_len][d|dv] in slot order, k_tilde [m][d], q_tilde [hpk][m][d],
 * mu [hpk][m][m], au [hpk][m][m] (f64 exp-Gram), t_hat [hpk][m][dv] (at scale
 * e^{-m_max}), z_hat / m_max [hpk][m].                                       */
void orc_export(const orc_group *g, float *sink_k, float *sink_v, float *win_k, float *win_v,
                float *k_tilde, float *q_tilde, float *mu, double *au, double *t_hat,
                double *z_hat, double *m_max)
{
    size_t m = (size_t)g->m_eff, H = (size_t)g->hpk;
    if (sink_k && g->sink_len) memcpy(sink_k, g->sink_k, sizeof(float) * g->sink_len * g->d);
    if (sink_v && g->sink_len) memcpy(sink_v, g->sink_v, sizeof(float) * g->sink_len * g->dv);
    if (win_k) memcpy(win_k, g->win_k, sizeof(float) * (size_t)g->win_len * g->d);
    if (win_v) memcpy(win_v, g->win_v, sizeof(float) * (size_t)g->win_len * g->dv);
    if (g->exact_only) return;
    if (k_tilde) memcpy(k_tilde, g->k_tilde, sizeof(float) * m * g->d);
    if (q_tilde) memcpy(q_tilde, g->q_tilde, sizeof(float) * H * m * g->d);
    if (mu) memcpy(mu, g->mu, sizeof(float) * H * m * m);
    if (au) memcpy(au, g->au, sizeof(double) * H * m * m);
    if (t_hat) memcpy(t_hat, g->t_hat, sizeof(double) * H * m * g->dv);
    if (z_hat) memcpy(z_hat, g->z_hat, sizeof(double) * H * m);
    if (m_max) memcpy(m_max, g->m_max, sizeof(double) * H * m);
}

/* f64 landmarks (segment means before the f32 rounding). */
void orc_export_landmarks64(const orc_group *g, double *k_tilde64, double *q_tilde64)
{
    size_t m = (size_t)g->m_eff;
    if (g->exact_only) return;
    if (k_tilde64) memcpy(k_tilde64, g->k_tilde64, sizeof(double) * m * g->d);
    if (q_tilde64) memcpy(q_tilde64, g->q_tilde64, sizeof(double) * g->hpk * m * g->d);
}

/* `steps` consecutive step_group calls (a plain loop, no other change):
 * q_all [steps][q_heads][d], k [steps][d], v [steps][dv] -> out_all
 * [steps][q_heads][dv]; out_alt and diag as in orc_step_group, per step (may
 * be NULL).  Returns 0, or -1 before prefill.                                */
int orc_step_many(orc_group *g, int steps, const float *q_all, const float *k, const float *v,
                  double *out_all, double *out_alt, orc_diag *diag)
{
    if (!g || !g->sealed) return -1;
    const size_t H = (size_t)g->hpk;
    for (int t = 0; t < steps; ++t)
        orc_step_group(g, q_all + (size_t)t * H * g->d, k + (size_t)t * g->d, v + (size_t)t * g->dv,
                       out_all + (size_t)t * H * g->dv, out_alt ? out_alt + (size_t)t * H * g->dv : NULL,
                       diag ? diag + (size_t)t * H : NULL);
    return 0;
}
