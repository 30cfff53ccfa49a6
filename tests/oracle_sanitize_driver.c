/*
 * Drives every entry point of the CPU oracle (oracle/nystrom_oracle.c) on
 * small seeded inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).  It checks no
 * numbers -- the pins in tests/test_oracle_pins.py do that -- only that every
 * path runs without an out-of-bounds access, a leak or undefined behaviour.
 *
 * Paths covered: skeleton prefill and decode with and without sinks, both
 * rectifiers, frozen landmarks, the replay outputs, an exact-only prompt whose
 * window grows past its first allocation, a re-prefill of the same group,
 * ridge_pinv's retry and fallback paths, a Cholesky of a non-positive-definite
 * matrix, exact attention, and every export.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct orc_group orc_group;
orc_group *orc_new_group(int m, int w, int sink, int q_heads, int rect);
void orc_free(orc_group *g);
int orc_prefill_group(orc_group *g, const float *qs, const float *ks, const float *vs, int t, int d, int dv,
                      const float *frozen_kt, const float *frozen_qt, const float *frozen_mu,
                      double *replay_out);
int orc_step_many(orc_group *g, int steps, const float *q_all, const float *k, const float *v,
                  double *out_all, double *out_alt, void *diag);
int orc_m_eff(const orc_group *g);
int orc_win_len(const orc_group *g);
int orc_sink_len(const orc_group *g);
size_t orc_memory_bytes(const orc_group *g);
void orc_export(const orc_group *g, float *sink_k, float *sink_v, float *win_k, float *win_v, float *k_tilde,
                float *q_tilde, float *mu, double *au, double *t_hat, double *z_hat, double *m_max);
void orc_export_landmarks64(const orc_group *g, double *k_tilde64, double *q_tilde64);
int orc_ridge_pinv(const double *a, int n, double ridge_rel, double *out, double *lambda_out);
int orc_cholesky(double *g, int n);
void orc_exact_attention(const float *q, const float *ks, const float *vs, int n, int d, int dv,
                         double scale, double *out);

/* test inputs only: a 64-bit LCG mapped to [-1, 1) */
static unsigned long long rng = 0x9e3779b97f4a7c15ULL;
static float draw(void)
{
    rng = rng * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float *fill(size_t n, float amp)
{
    float *p = (float *)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = amp * draw();
    return p;
}

static int run_group(int m, int w, int sink, int hpk, int rect, int t, int d, int steps, int frozen)
{
    orc_group *g = orc_new_group(m, w, sink, hpk, rect);
    if (!g) return 1;
    float *qs = fill((size_t)hpk * t * d, 2.0f), *ks = fill((size_t)t * d, 2.0f), *vs = fill((size_t)t * d, 1.0f);
    double *replay = (double *)calloc((size_t)t * hpk * d, sizeof(double));
    float *fk = NULL, *fq = NULL, *fm = NULL;
    const int me = t / 8 < 4 ? 4 : (t / 8 > m ? m : t / 8);
    if (frozen) {
        fk = fill((size_t)me * d, 1.0f);
        fq = fill((size_t)hpk * me * d, 1.0f);
        fm = fill((size_t)hpk * me * me, 0.1f);
    }
    int rc = orc_prefill_group(g, qs, ks, vs, t, d, d, fk, fq, fm, replay);
    float *q = fill((size_t)steps * hpk * d, 2.0f), *k = fill((size_t)steps * d, 2.0f), *v = fill((size_t)steps * d, 1.0f);
    double *out = (double *)calloc((size_t)steps * hpk * d, sizeof(double));
    double *alt = (double *)calloc((size_t)steps * hpk * d, sizeof(double));
    rc |= orc_step_many(g, steps, q, k, v, out, alt, NULL);
    /* exports sized from the group itself */
    const int M = orc_m_eff(g), S = orc_sink_len(g), W = orc_win_len(g);
    float *sk = fill((size_t)(S ? S : 1) * d, 0), *sv = fill((size_t)(S ? S : 1) * d, 0);
    float *wk = fill((size_t)W * d, 0), *wv = fill((size_t)W * d, 0);
    float *kt = fill((size_t)(M ? M : 1) * d, 0), *qt = fill((size_t)hpk * (M ? M : 1) * d, 0);
    float *mu = fill((size_t)hpk * (M ? M * M : 1), 0);
    double *au = (double *)calloc((size_t)hpk * (M ? M * M : 1), sizeof(double));
    double *th = (double *)calloc((size_t)hpk * (M ? M : 1) * d, sizeof(double));
    double *zh = (double *)calloc((size_t)hpk * (M ? M : 1), sizeof(double));
    double *mm = (double *)calloc((size_t)hpk * (M ? M : 1), sizeof(double));
    double *k64 = (double *)calloc((size_t)(M ? M : 1) * d, sizeof(double));
    double *q64 = (double *)calloc((size_t)hpk * (M ? M : 1) * d, sizeof(double));
    orc_export(g, sk, sv, wk, wv, kt, qt, mu, au, th, zh, mm);
    if (M) orc_export_landmarks64(g, k64, q64);
    rc |= orc_memory_bytes(g) == 0;
    /* a second prefill of the same group releases and rebuilds its arrays */
    rc |= orc_prefill_group(g, qs, ks, vs, t, d, d, NULL, NULL, NULL, NULL);
    rc |= orc_step_many(g, 3, q, k, v, out, NULL, NULL);
    orc_free(g);
    free(qs); free(ks); free(vs); free(replay); free(fk); free(fq); free(fm);
    free(q); free(k); free(v); free(out); free(alt);
    free(sk); free(sv); free(wk); free(wv); free(kt); free(qt); free(mu); free(au); free(th); free(mm);
    free(zh); free(k64); free(q64);
    return rc;
}

int main(void)
{
    int rc = 0;
    rc |= run_group(8, 16, 2, 1, 0, 64, 64, 70, 0);    /* skeleton, sinks, Aggregate */
    rc |= run_group(16, 24, 0, 3, 1, 100, 64, 40, 0);  /* no sinks, Fm, ragged segments */
    rc |= run_group(8, 16, 2, 2, 0, 64, 64, 20, 1);    /* frozen landmarks and M */
    rc |= run_group(32, 16, 2, 2, 0, 20, 64, 90, 0);   /* exact-only prompt; the window grows */
    rc |= run_group(4, 1, 0, 1, 0, 40, 64, 30, 0);     /* w = 1, m = 4 */

    /* ridge_pinv: a rank-one A (the ridge grows), an all-zero A and a NaN (fallbacks) */
    enum { N = 6 };
    double a[N * N], out[N * N], lam = 0.0;
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) a[i * N + j] = (double)(i + 1) * (double)(j + 2);
    rc |= orc_ridge_pinv(a, N, 1e-30, out, &lam) < 1;
    for (int i = 0; i < N * N; ++i) a[i] = 0.0;
    (void)orc_ridge_pinv(a, N, 1e-6, out, &lam);
    a[7] = NAN;
    (void)orc_ridge_pinv(a, N, 1e-6, out, &lam);
    /* Cholesky of a matrix that is not positive definite */
    double g2[4] = {1.0, 2.0, 2.0, 1.0};
    rc |= orc_cholesky(g2, 2) != 0;  /* must report the failed pivot */

    /* exact attention over a few keys */
    float *q = fill(64, 1.0f), *ks = fill(5 * 64, 1.0f), *vs = fill(5 * 32, 1.0f);
    double o[32];
    orc_exact_attention(q, ks, vs, 5, 64, 32, 0.125, o);
    free(q); free(ks); free(vs);

    printf(rc ? "oracle driver: an entry point reported failure\n" : "oracle driver: all paths ran\n");
    return rc;
}
