/* Drives every entry point of the fp64 oracle (oracle/vwl_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer on small seeded inputs:
 * both stored dtypes, the degenerate shapes (one token, no drafts, a
 * one-element window), -inf logits, out-of-range drafts and vocabulary
 * alignment entries, and the invalid-argument returns.  It checks return
 * codes and a few invariants (D within [0, ln 2], probabilities within
 * [0, 1]); the values themselves are pinned by the Python tests.  Exit
 * status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int vwl_oracle_asym(const void *a, const void *b, const void *t, int dtype, const int32_t *draft, int B, int K, int V,
                    double beta, double gamma, int delta_src, int gate, double *lse, double *D, double *geff,
                    int32_t *fused, double *gap, double *top, uint8_t *accept, double *margin, int32_t *accept_len,
                    int32_t *token, int nthreads);
int vwl_oracle_rapid(const void *z, const void *y, int dtype, const int32_t *draft, const float *u_accept,
                     const float *u_sample, int B, int G, int V, double eta, double T, double *rowstat, double *phat_d,
                     double *q_d, uint8_t *accept, double *acc_rel, double *tail_d_dist, int32_t *accept_len,
                     int32_t *token, double *resid_S, double *draw_slack, int32_t *tail_close, double tail_eps,
                     double *emit_dist, double *emit_scale, int nthreads);
int vwl_oracle_asym_xfam(const void *a, const void *b, int Vd, const void *t, int Vt, const int32_t *vmap, int dtype,
                         const int32_t *draft, int B, int K, double beta, double gamma, double *lse, double *D,
                         double *geff, int32_t *fused, double *gap, double *top, uint8_t *accept, double *margin,
                         int32_t *accept_len, int32_t *token, int nthreads);
int vwl_oracle_e2sci(const void *y, const void *z, int dtype, int B, int W, int V, const float *T_in,
                     const float *omega, const float *r_in, double alpha, double tau, double T_base, double T_min,
                     double T_max, double ewma, double *D, uint8_t *accept, int32_t *accept_len, double *r_out,
                     double *T_out, int nthreads);
int vwl_oracle_rapid_zhat(const double *z, const double *y, int V, double eta, double T, double *zhat);
int vwl_oracle_rapid_phat(const double *z, const double *y, int V, double eta, double T, double *phat);

static int failures = 0;
#define EXPECT(c)                                                                                                      \
    do {                                                                                                               \
        if (!(c)) {                                                                                                    \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c);                                                     \
            ++failures;                                                                                                \
        }                                                                                                              \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* splitmix64 */
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}
static double normal(void) { return sqrt(-2.0 * log(1.0 - unif())) * cos(6.283185307179586 * unif()); }

/* logits as stored: dtype 0 fp32, 1 bf16 (upper half of an fp32, rounded to nearest even) */
static void *logits(int dtype, size_t n, double scale, int with_neg_inf) {
    void *p = malloc(n * (dtype == 0 ? 4 : 2));
    for (size_t i = 0; i < n; ++i) {
        float f = (float)(scale * normal());
        if (with_neg_inf && i % 7 == 3)
            f = -INFINITY;
        if (dtype == 0) {
            ((float *)p)[i] = f;
        } else {
            uint32_t u;
            memcpy(&u, &f, 4);
            u += 0x7FFFu + ((u >> 16) & 1u);
            ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
        }
    }
    return p;
}

static void run_asym(int dtype, int B, int K, int V, int bad_draft, int ninf) {
    const int P = K + 1;
    void *a = logits(dtype, (size_t)B * P * V, 2.0, ninf), *b = logits(dtype, (size_t)B * P * V, 2.0, ninf),
         *t = logits(dtype, (size_t)B * P * V, 2.0, ninf);
    int32_t *draft = malloc(sizeof(int32_t) * (size_t)(B * K + 1));
    for (int i = 0; i < B * K; ++i)
        draft[i] = bad_draft && i == 0 ? V + 3 : (int32_t)(unif() * V);
    double *lse = malloc(sizeof(double) * B * P * 3), *D = malloc(sizeof(double) * B * P),
           *ge = malloc(sizeof(double) * B * P), *gap = malloc(sizeof(double) * B * P),
           *top = malloc(sizeof(double) * B * P), *margin = malloc(sizeof(double) * (B * K + 1));
    int32_t *fused = malloc(sizeof(int32_t) * B * P), *alen = malloc(sizeof(int32_t) * B),
            *tok = malloc(sizeof(int32_t) * B);
    uint8_t *acc = malloc((size_t)(B * K + 1));
    for (int ds = 0; ds < 3; ++ds)
        for (int gate = 0; gate < 2; ++gate) {
            EXPECT(vwl_oracle_asym(a, b, t, dtype, draft, B, K, V, 1.0, 0.5, ds, gate, lse, D, ge, fused, gap, top,
                                   acc, margin, alen, tok, 1) == 0);
            for (int r = 0; r < B * P; ++r)
                EXPECT(!(D[r] < -1e-12) && !(D[r] > log(2.0) + 1e-12));
            for (int bi = 0; bi < B; ++bi)
                EXPECT(alen[bi] >= 0 && alen[bi] <= K);
        }
    EXPECT(vwl_oracle_asym(a, b, t, 9, draft, B, K, V, 1.0, 0.5, 0, 0, lse, D, ge, fused, gap, top, acc, margin, alen,
                           tok, 1) == 1);
    free(a), free(b), free(t), free(draft), free(lse), free(D), free(ge), free(gap), free(top), free(margin);
    free(fused), free(alen), free(tok), free(acc);
}

static void run_rapid(int dtype, int B, int G, int V, int bad_draft) {
    const int P = G + 1;
    void *z = logits(dtype, (size_t)B * P * V, 2.0, 0), *y = logits(dtype, (size_t)B * P * V, 2.0, 0);
    int32_t *draft = malloc(sizeof(int32_t) * (size_t)(B * G + 1));
    float *ua = malloc(sizeof(float) * (size_t)(B * G + 1)), *us = malloc(sizeof(float) * (size_t)(B * P));
    for (int i = 0; i < B * G; ++i) {
        draft[i] = bad_draft && i == 0 ? -2 : (int32_t)(unif() * V);
        ua[i] = (float)unif();
    }
    for (int i = 0; i < B * P; ++i)
        us[i] = (float)unif();
    double *rowstat = malloc(sizeof(double) * B * P * 4), *phd = malloc(sizeof(double) * (B * G + 1)),
           *qd = malloc(sizeof(double) * (B * G + 1)), *accrel = malloc(sizeof(double) * (B * G + 1)),
           *tdd = malloc(sizeof(double) * (B * G + 1)), *rS = malloc(sizeof(double) * B),
           *slack = malloc(sizeof(double) * B), *emit = malloc(sizeof(double) * (size_t)B * V),
           *escale = malloc(sizeof(double) * (size_t)B * V);
    int32_t *alen = malloc(sizeof(int32_t) * B), *tok = malloc(sizeof(int32_t) * B),
            *tclose = malloc(sizeof(int32_t) * B);
    uint8_t *acc = malloc((size_t)(B * G + 1));
    for (int k = 0; k < 3; ++k) {
        const double eta = k * 10.0, T = k == 2 ? 0.7 : 1.0;
        EXPECT(vwl_oracle_rapid(z, y, dtype, draft, ua, us, B, G, V, eta, T, rowstat, phd, qd, acc, accrel, tdd, alen,
                                tok, rS, slack, tclose, 1e-6, emit, escale, 1) == 0);
        for (int bi = 0; bi < B; ++bi)
            EXPECT(alen[bi] >= 0 && alen[bi] <= G && tok[bi] >= 0 && tok[bi] < V);
        for (int i = 0; i < B * G; ++i)
            EXPECT(!(phd[i] < 0.0) && !(phd[i] > 1.0 + 1e-12) && !(qd[i] < 0.0) && !(qd[i] > 1.0 + 1e-12));
    }
    EXPECT(vwl_oracle_rapid(z, y, dtype, draft, ua, us, B, G, V, 1.0, 0.0, rowstat, phd, qd, acc, accrel, tdd, alen,
                            tok, rS, slack, tclose, 1e-6, emit, escale, 1) == 1);
    free(z), free(y), free(draft), free(ua), free(us), free(rowstat), free(phd), free(qd), free(accrel), free(tdd);
    free(rS), free(slack), free(emit), free(escale), free(alen), free(tok), free(tclose), free(acc);
}

static void run_xfam(int dtype, int B, int K, int Vd, int Vt) {
    const int P = K + 1;
    void *a = logits(dtype, (size_t)B * P * Vd, 2.0, 0), *b = logits(dtype, (size_t)B * P * Vd, 2.0, 0),
         *t = logits(dtype, (size_t)B * P * Vt, 2.0, 0);
    int32_t *vmap = malloc(sizeof(int32_t) * (size_t)Vt), *draft = malloc(sizeof(int32_t) * (size_t)(B * K + 1));
    for (int v = 0; v < Vt; ++v)
        vmap[v] = v % 3 == 0 ? -1 : (v % 11 == 5 ? Vd + 7 : (int32_t)(unif() * Vd));
    for (int i = 0; i < B * K; ++i)
        draft[i] = i == 1 ? Vt : (int32_t)(unif() * Vt);
    double *lse = malloc(sizeof(double) * B * P * 3), *D = malloc(sizeof(double) * B * P),
           *ge = malloc(sizeof(double) * B * P), *gap = malloc(sizeof(double) * B * P),
           *top = malloc(sizeof(double) * B * P), *margin = malloc(sizeof(double) * (B * K + 1));
    int32_t *fused = malloc(sizeof(int32_t) * B * P), *alen = malloc(sizeof(int32_t) * B),
            *tok = malloc(sizeof(int32_t) * B);
    uint8_t *acc = malloc((size_t)(B * K + 1));
    EXPECT(vwl_oracle_asym_xfam(a, b, Vd, t, Vt, vmap, dtype, draft, B, K, 1.0, 0.5, lse, D, ge, fused, gap, top, acc,
                                margin, alen, tok, 1) == 0);
    for (int r = 0; r < B * P; ++r)
        EXPECT(fused[r] == -1 || (fused[r] >= 0 && fused[r] < Vt && vmap[fused[r]] >= 0 && vmap[fused[r]] < Vd));
    for (int v = 0; v < Vt; ++v)
        vmap[v] = -1; /* no pair at all */
    EXPECT(vwl_oracle_asym_xfam(a, b, Vd, t, Vt, vmap, dtype, draft, B, K, 1.0, 0.5, lse, D, ge, fused, gap, top, acc,
                                margin, alen, tok, 1) == 0);
    for (int r = 0; r < B * P; ++r)
        EXPECT(fused[r] == -1);
    free(a), free(b), free(t), free(vmap), free(draft), free(lse), free(D), free(ge), free(gap), free(top);
    free(margin), free(fused), free(alen), free(tok), free(acc);
}

static void run_e2sci(int dtype, int B, int W, int V) {
    void *y = logits(dtype, (size_t)B * W * V, 2.0, 0), *z = logits(dtype, (size_t)B * W * V, 2.0, 0);
    float *T = malloc(sizeof(float) * B), *om = malloc(sizeof(float) * B), *r = malloc(sizeof(float) * B);
    for (int i = 0; i < B; ++i) {
        T[i] = (float)(0.3 * unif());
        om[i] = (float)(0.5 + unif());
        r[i] = (float)unif();
    }
    double *D = malloc(sizeof(double) * B * W), *ro = malloc(sizeof(double) * B), *To = malloc(sizeof(double) * B);
    uint8_t *acc = malloc((size_t)B * W);
    int32_t *alen = malloc(sizeof(int32_t) * B);
    EXPECT(vwl_oracle_e2sci(y, z, dtype, B, W, V, T, om, r, 1.0, 0.5, 0.1, 0.01, 0.3, 0.3, D, acc, alen, ro, To, 1) == 0);
    for (int i = 0; i < B; ++i)
        EXPECT(alen[i] >= 0 && alen[i] <= W && To[i] >= 0.01 - 1e-12 && To[i] <= 0.3 + 1e-12);
    EXPECT(vwl_oracle_e2sci(y, z, dtype, B, 0, V, T, om, r, 1.0, 0.5, 0.1, 0.01, 0.3, 0.3, D, acc, alen, ro, To, 1) == 1);
    free(y), free(z), free(T), free(om), free(r), free(D), free(ro), free(To), free(acc), free(alen);
}

static void run_rows(int V) {
    double *z = malloc(sizeof(double) * V), *y = malloc(sizeof(double) * V), *o = malloc(sizeof(double) * V);
    for (int v = 0; v < V; ++v) {
        z[v] = 2.0 * normal();
        y[v] = z[v] + normal();
    }
    EXPECT(vwl_oracle_rapid_zhat(z, y, V, 10.0, 1.0, o) == 0);
    EXPECT(vwl_oracle_rapid_phat(z, y, V, 10.0, 1.0, o) == 0);
    double s = 0.0;
    for (int v = 0; v < V; ++v)
        s += o[v];
    EXPECT(fabs(s - 1.0) < 1e-9 || s < 1.0); /* protected tail entries keep p, so the sum need not be one */
    EXPECT(vwl_oracle_rapid_phat(z, y, V, 10.0, 0.0, o) == 1);
    free(z), free(y), free(o);
}

int main(void) {
    for (int dt = 0; dt < 2; ++dt) {
        run_asym(dt, 3, 2, 37, 0, 0);
        run_asym(dt, 2, 0, 1, 0, 0);
        run_asym(dt, 2, 3, 129, 1, 1);
        run_rapid(dt, 3, 4, 53, 0);
        run_rapid(dt, 2, 0, 1, 0);
        run_rapid(dt, 2, 2, 17, 1);
        run_xfam(dt, 3, 2, 61, 47);
        run_e2sci(dt, 3, 4, 29);
        run_e2sci(dt, 2, 1, 1);
    }
    run_rows(1);
    run_rows(300);
    if (failures)
        fprintf(stderr, "%d check(s) failed\n", failures);
    else
        printf("oracle harness: all checks passed\n");
    return failures ? 1 : 0;
}
