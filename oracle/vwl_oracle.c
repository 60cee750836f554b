/*
 * Plain fp64 CPU oracle for the speculative verify / logit-fusion pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, calls or includes it, and it shares no code with the GPU library.
 *
 * Every stored logit is widened exactly to double (bf16 and fp32 both widen
 * exactly) and every quantity is then computed in double precision, row by
 * row, straight from its definition on the pages:
 *
 *   AsymSpec ("AsymSpec: Context-Asymmetric Speculative Decoding for Agentic
 *   LLMs" reading notes, section 4.1 "contrastive delta-fusion" and section
 *   4.2 "CDA gate"):
 *     delta_i   = a_i - b_i                               (4.1)
 *     fused_i   = argmax_v (t_i + beta * delta_i)          (4.1)
 *     D_i       = JSD(softmax(a_i) || softmax(b_i))        (4.2)
 *     geff_i    = gamma * exp(-D_i)                        (4.2)
 *     accept_i  = softmax(t_i)[d_i] > geff_i * softmax(b_i)[d_i]   (4.2)
 *     the first rejection emits the delta-fusion token     (4.2)
 *   and the variants of the same notes' mechanism ablation and
 *   counterfactual discussion: delta_i = a_i (the raw full-context logits)
 *   or delta_i = t_i - b_i (the two-model difference of contrastive /
 *   speculative contrastive decoding), and the fixed threshold gamma in
 *   place of the CDA threshold (section 4.2 contrasts the two).
 *
 *   RAPID ("RAPID: Long-Context Inference with Retrieval-Augmented
 *   Speculative Decoding" notes, key designs 2-4):
 *     p = softmax(z/T), q = softmax(y/T)
 *     zhat = z + eta*T*(q - p),  phat = softmax(zhat/T)    (design 2)
 *     phat_k := p_k where phat_k < 0.1 * max_j phat_j      (design 3)
 *     rejection sampling against phat; on rejection draw from
 *     norm(max(p - phat, p - q, 0))                        (design 4)
 *
 * Readings of points the pages leave open (natural-log JSD with 0*log 0 = 0,
 * row i tests draft i, the bonus row emits its own fusion token, lowest index
 * wins every argmax tie, strict comparisons, no renormalisation after tail
 * protection, inverse-CDF draws in vocabulary order, the bonus draw of RAPID
 * from p, a zero residual falling back to p) are applied here exactly as the
 * library documents them.
 *
 * Sums are plain sequential double sums; nothing is blocked, fused or
 * reordered.  Rows are independent and run in an OpenMP loop; each row's
 * arithmetic is sequential, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2 /* rows given as doubles (logits formed by the caller in fp64) */

/* Exact widening of one stored logit to double. */
static double widen(const void *base, int dtype, size_t i)
{
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F64)
        return ((const double *)base)[i];
    return (double)((const float *)base)[i];
}

/* Threads for the row loops of one call: nthreads > 0 asks for that many,
 * 0 for the OpenMP default of the process (taken once, at the first call),
 * so a one-thread call does not leave later calls single-threaded. */
static void set_threads(int nthreads)
{
#ifdef _OPENMP
    static int default_threads = 0;
    if (default_threads == 0)
        default_threads = omp_get_max_threads();
    omp_set_num_threads(nthreads > 0 ? nthreads : default_threads);
#else
    (void)nthreads;
#endif
}

int vwl_oracle_max_threads(void)
{
#ifdef _OPENMP
    set_threads(0);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* log sum_v exp(x_v) for a row of n doubles: max shift, plain sum.
 * A row that is entirely -inf has log-sum-exp -inf. */
static double logsumexp(const double *x, int n)
{
    double m = -INFINITY;
    for (int v = 0; v < n; ++v)
        if (x[v] > m)
            m = x[v];
    if (m == -INFINITY)
        return -INFINITY;
    double s = 0.0;
    for (int v = 0; v < n; ++v)
        s += exp(x[v] - m);
    return m + log(s);
}

/* Jensen-Shannon divergence of P = softmax(x) and Q = softmax(y) given their
 * log-sum-exps: 1/2 KL(P||M) + 1/2 KL(Q||M), M = (P+Q)/2, natural log; a term
 * whose probability is 0 contributes 0. */
static double jsd(const double *x, double Lx, const double *y, double Ly, int V)
{
    double kl = 0.0;
    for (int v = 0; v < V; ++v) {
        const double p = exp(x[v] - Lx);
        const double q = exp(y[v] - Ly);
        const double m = 0.5 * (p + q);
        if (p > 0.0)
            kl += p * log(p / m);
        if (q > 0.0)
            kl += q * log(q / m);
    }
    return 0.5 * kl;
}

/* ======================================================================
 * AsymSpec
 * ====================================================================== */

/*
 * Inputs: a, b, t stored rows [B][K+1][V] (dtype 0 = fp32, 1 = bf16 bits),
 * draft [B][K], beta, gamma (the float arguments, widened),
 * delta_src: 0 delta = a - b, 1 delta = a, 2 delta = t - b;
 * gate: 0 the CDA threshold gamma*exp(-D), 1 the fixed threshold gamma.
 * Outputs (all required):
 *   lse[R][3]      log-sum-exp of a, b, t per row (R = B*(K+1))
 *   D[R]           Jensen-Shannon divergence of softmax(a) and softmax(b)
 *                  (reported under either gate)
 *   geff[R]        the threshold in use: gamma * exp(-D), or gamma
 *   fused[R]       lowest index maximising t + beta*delta
 *   gap[R]         top1 - top2 of that score (0 for an exact tie)
 *   top[R]         top1, the maximum of that score
 *   accept[B][K]   acceptance flag of draft i at row i (0 for an id outside [0,V))
 *   margin[B][K]   log p_t(d) - log p_b(d) - log geff  (NaN for a bad id)
 *   accept_len[B], token[B]
 */
int vwl_oracle_asym(const void *a, const void *b, const void *t, int dtype,
                    const int32_t *draft, int B, int K, int V,
                    double beta, double gamma, int delta_src, int gate,
                    double *lse, double *D, double *geff, int32_t *fused, double *gap,
                    double *top, uint8_t *accept, double *margin,
                    int32_t *accept_len, int32_t *token, int nthreads)
{
    if (B < 1 || K < 0 || V < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64))
        return 1;
    if (delta_src < 0 || delta_src > 2 || gate < 0 || gate > 1)
        return 1;
    const int P = K + 1;
    const long R = (long)B * P;
    set_threads(nthreads);
    int bad_alloc = 0;

#pragma omp parallel
    {
        double *xa = malloc(sizeof(double) * (size_t)V);
        double *xb = malloc(sizeof(double) * (size_t)V);
        double *xt = malloc(sizeof(double) * (size_t)V);
        if (!xa || !xb || !xt) {
#pragma omp atomic write
            bad_alloc = 1;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < R; ++r) {
                const size_t off = (size_t)r * (size_t)V;
                for (int v = 0; v < V; ++v) {
                    xa[v] = widen(a, dtype, off + v);
                    xb[v] = widen(b, dtype, off + v);
                    xt[v] = widen(t, dtype, off + v);
                }
                /* softmax normalisers of the three rows */
                const double La = logsumexp(xa, V);
                const double Lb = logsumexp(xb, V);
                const double Lt = logsumexp(xt, V);
                lse[3 * r + 0] = La;
                lse[3 * r + 1] = Lb;
                lse[3 * r + 2] = Lt;

                const double Dr = jsd(xa, La, xb, Lb, V);
                D[r] = Dr;
                /* the acceptance threshold: CDA relaxes gamma by exp(-D) */
                geff[r] = (gate == 0) ? gamma * exp(-Dr) : gamma;

                /* fused token: lowest index of the maximum of t + beta*delta;
                 * gap = best - second best (counting multiplicity). */
                double best = -INFINITY, second = -INFINITY;
                int arg = 0;
                for (int v = 0; v < V; ++v) {
                    double delta;
                    if (delta_src == 0)
                        delta = xa[v] - xb[v];
                    else if (delta_src == 1)
                        delta = xa[v];
                    else
                        delta = xt[v] - xb[v];
                    const double s = xt[v] + beta * delta;
                    if (s > best) {
                        second = best;
                        best = s;
                        arg = v;
                    } else if (s > second) {
                        second = s;
                    }
                }
                fused[r] = arg;
                gap[r] = (V > 1) ? best - second : INFINITY;
                top[r] = best;

                /* acceptance of the draft tested at this row */
                const long bi = r / P;
                const int i = (int)(r % P);
                if (i < K) {
                    const int d = draft[bi * K + i];
                    if (d < 0 || d >= V) {
                        accept[bi * K + i] = 0;
                        margin[bi * K + i] = NAN;
                    } else {
                        const double pt = exp(xt[d] - Lt);
                        const double pb = exp(xb[d] - Lb);
                        accept[bi * K + i] = (pt > geff[r] * pb) ? 1 : 0;
                        margin[bi * K + i] = (xt[d] - Lt) - (xb[d] - Lb) - log(gamma) + (gate == 0 ? Dr : 0.0);
                    }
                }
            }
        }
        free(xa);
        free(xb);
        free(xt);
    }
    if (bad_alloc)
        return 2;

    /* first rejection among the K drafts; emit that row's fusion token */
    for (int bi = 0; bi < B; ++bi) {
        int n = K;
        for (int i = 0; i < K; ++i) {
            if (!accept[(long)bi * K + i]) {
                n = i;
                break;
            }
        }
        accept_len[bi] = n;
        token[bi] = fused[(long)bi * P + n];
    }
    return 0;
}

/* ======================================================================
 * RAPID
 * ====================================================================== */

/* Inverse-CDF draw in vocabulary order: the smallest k whose running sum
 * exceeds u*S.  `slack` receives the distance from u*S to the nearer end of
 * the chosen interval, relative to S. */
static int draw_inverse_cdf(const double *w, int V, double S, double u, double *slack)
{
    const double target = u * S;
    double c = 0.0;
    int last_pos = -1;
    for (int k = 0; k < V; ++k) {
        const double prev = c;
        c += w[k];
        if (w[k] > 0.0)
            last_pos = k;
        if (c > target) {
            const double lo = target - prev, hi = c - target;
            *slack = (lo < hi ? lo : hi) / S;
            return k;
        }
    }
    *slack = 0.0; /* only reachable through rounding: flagged as ambiguous */
    return last_pos < 0 ? V - 1 : last_pos;
}

/*
 * Inputs: z, y stored rows [B][G+1][V]; draft [B][G]; u_accept [B][G];
 * u_sample [B][G+1]; eta, T.
 * Outputs:
 *   rowstat[R][4]  L_z = LSE(z/T), L_y = LSE(y/T), Mhat = max zhat/T, L_zhat = LSE(zhat/T)
 *   phat_d[B][G], q_d[B][G]   phat and q at each draft (0 for a bad id)
 *   accept[B][G]
 *   acc_rel[B][G]  |u*q - phat| / max(u*q, phat): closeness of the accept test
 *   tail_d_dist[B][G]  |zhat_d/T - Mhat - ln 0.1| at the draft (inf for a bad id)
 *   accept_len[B], token[B]
 *   resid_S[B]     sum of the residual on the emitting row (-1 when the draw was from p)
 *   draw_slack[B]  relative distance of u*S to the chosen interval's ends
 *   tail_close[B]  number of tokens of the emitting row with |zhat/T - Mhat - ln 0.1| <= tail_eps
 *   emit_dist[B][V] (nullable) the distribution the token was drawn from
 *   emit_scale[B][V] (nullable) p + max(phat, q) per token of the emitting row
 *                   (p alone for a draw from p): the magnitude the residual's
 *                   subtractions start from, used for rounding allowances
 */
int vwl_oracle_rapid(const void *z, const void *y, int dtype,
                     const int32_t *draft, const float *u_accept, const float *u_sample,
                     int B, int G, int V, double eta, double T,
                     double *rowstat, double *phat_d, double *q_d, uint8_t *accept,
                     double *acc_rel, double *tail_d_dist,
                     int32_t *accept_len, int32_t *token,
                     double *resid_S, double *draw_slack, int32_t *tail_close, double tail_eps,
                     double *emit_dist, double *emit_scale, int nthreads)
{
    if (B < 1 || G < 0 || V < 1 || !(T > 0.0) || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return 1;
    const int P = G + 1;
    const long R = (long)B * P;
    const double tail_log = log(0.1);
    set_threads(nthreads);
    int bad_alloc = 0;

    /* Per row: the two softmaxes, the augmented target and the draft test. */
#pragma omp parallel
    {
        double *zs = malloc(sizeof(double) * (size_t)V);
        double *ys = malloc(sizeof(double) * (size_t)V);
        double *hs = malloc(sizeof(double) * (size_t)V);
        if (!zs || !ys || !hs) {
#pragma omp atomic write
            bad_alloc = 1;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < R; ++r) {
                const size_t off = (size_t)r * (size_t)V;
                for (int v = 0; v < V; ++v) {
                    zs[v] = widen(z, dtype, off + v) / T;
                    ys[v] = widen(y, dtype, off + v) / T;
                }
                const double Lz = logsumexp(zs, V);
                const double Ly = logsumexp(ys, V);
                /* zhat/T = z/T + eta*(q - p) */
                for (int v = 0; v < V; ++v) {
                    const double p = exp(zs[v] - Lz);
                    const double q = exp(ys[v] - Ly);
                    const double zhat = widen(z, dtype, off + v) + eta * T * (q - p);
                    hs[v] = zhat / T;
                }
                double Mh = -INFINITY;
                for (int v = 0; v < V; ++v)
                    if (hs[v] > Mh)
                        Mh = hs[v];
                const double Lh = logsumexp(hs, V);
                rowstat[4 * r + 0] = Lz;
                rowstat[4 * r + 1] = Ly;
                rowstat[4 * r + 2] = Mh;
                rowstat[4 * r + 3] = Lh;

                const long bi = r / P;
                const int i = (int)(r % P);
                if (i < G) {
                    const long k = bi * G + i;
                    const int x = draft[k];
                    if (x < 0 || x >= V) {
                        accept[k] = 0;
                        phat_d[k] = 0.0;
                        q_d[k] = 0.0;
                        acc_rel[k] = INFINITY;
                        tail_d_dist[k] = INFINITY;
                    } else {
                        const double p = exp(zs[x] - Lz);
                        const double q = exp(ys[x] - Ly);
                        const double praw = exp(hs[x] - Lh);
                        const double pmax = exp(Mh - Lh);
                        const double ph = (praw < 0.1 * pmax) ? p : praw;
                        double u = (double)u_accept[k];
                        if (!(u >= 0.0))
                            u = 0.0;
                        if (u >= 1.0)
                            u = 1.0 - 0x1p-24;
                        phat_d[k] = ph;
                        q_d[k] = q;
                        accept[k] = (u * q < ph) ? 1 : 0;
                        const double big = (u * q > ph) ? u * q : ph;
                        acc_rel[k] = big > 0.0 ? fabs(u * q - ph) / big : 0.0;
                        tail_d_dist[k] = fabs(hs[x] - Mh - tail_log);
                    }
                }
            }
        }
        free(zs);
        free(ys);
        free(hs);
    }
    if (bad_alloc)
        return 2;

    /* Per request: first rejection, then one draw on the emitting row. */
    int bad_alloc2 = 0;
#pragma omp parallel
    {
        double *w = malloc(sizeof(double) * (size_t)V);
        if (!w) {
#pragma omp atomic write
            bad_alloc2 = 1;
        } else {
#pragma omp for schedule(static)
            for (int bi = 0; bi < B; ++bi) {
                int n = G;
                for (int i = 0; i < G; ++i) {
                    if (!accept[(long)bi * G + i]) {
                        n = i;
                        break;
                    }
                }
                accept_len[bi] = n;
                const long r = (long)bi * P + n;
                const size_t off = (size_t)r * (size_t)V;
                const double Lz = rowstat[4 * r + 0], Ly = rowstat[4 * r + 1];
                const double Mh = rowstat[4 * r + 2], Lh = rowstat[4 * r + 3];
                const double pmax = exp(Mh - Lh);
                double S = 0.0;
                int close = 0;
                if (n < G) {
                    /* residual max(p - phat, p - q, 0) with tail protection */
                    for (int v = 0; v < V; ++v) {
                        const double zv = widen(z, dtype, off + v) / T;
                        const double yv = widen(y, dtype, off + v) / T;
                        const double p = exp(zv - Lz);
                        const double q = exp(yv - Ly);
                        const double h = (widen(z, dtype, off + v) + eta * T * (q - p)) / T;
                        const double praw = exp(h - Lh);
                        const double ph = (praw < 0.1 * pmax) ? p : praw;
                        double rv = p - ph;
                        if (p - q > rv)
                            rv = p - q;
                        if (rv < 0.0)
                            rv = 0.0;
                        w[v] = rv;
                        S += rv;
                        if (emit_scale)
                            emit_scale[(size_t)bi * V + v] = p + (ph > q ? ph : q);
                        if (fabs(h - Mh - tail_log) <= tail_eps)
                            ++close;
                    }
                }
                const int from_p = (n == G) || !(S > 0.0);
                if (from_p) {
                    S = 0.0;
                    for (int v = 0; v < V; ++v) {
                        w[v] = exp(widen(z, dtype, off + v) / T - Lz);
                        S += w[v];
                        if (emit_scale)
                            emit_scale[(size_t)bi * V + v] = w[v];
                    }
                }
                double u = (double)u_sample[(long)bi * P + n];
                if (!(u >= 0.0))
                    u = 0.0;
                if (u >= 1.0)
                    u = 1.0 - 0x1p-24;
                double slack;
                token[bi] = draw_inverse_cdf(w, V, S, u, &slack);
                resid_S[bi] = from_p ? -1.0 : S;
                draw_slack[bi] = slack;
                tail_close[bi] = close;
                if (emit_dist)
                    for (int v = 0; v < V; ++v)
                        emit_dist[(size_t)bi * V + v] = w[v] / S;
            }
        }
        free(w);
    }
    return bad_alloc2 ? 2 : 0;
}

/* ======================================================================
 * AsymSpec across model families (AsymSpec reading notes, the analysis of
 * why cross-family pairs work at a discount): the drafter's context gain
 * lives on the drafter's vocabulary and reaches the verifier through a
 * vocabulary alignment of string-identical tokens (plus paired special
 * tokens), with generation restricted to that shared subset.
 *
 * Inputs: a, b [B][K+1][Vd] drafter rows; t [B][K+1][Vt] verifier rows;
 * vmap[Vt]: the drafter id paired with each verifier token, or -1; draft
 * [B][K] in verifier ids.  Per row:
 *   La, Lb over the drafter vocabulary, Lt over the verifier's;
 *   D = JSD(softmax(a) || softmax(b)) on the drafter vocabulary;
 *   fused = lowest verifier id v with vmap[v] >= 0 maximising
 *           t[v] + beta * (a[vmap[v]] - b[vmap[v]])   (-1 if none is paired);
 *   accept: d = draft, paired e = vmap[d]:
 *           softmax(t)[d] > gamma * exp(-D) * softmax(b)[e]; a draft outside
 *           [0, Vt) or without a pair is rejected.
 * Outputs as vwl_oracle_asym (lse[R][3] = La, Lb, Lt).
 * ====================================================================== */
int vwl_oracle_asym_xfam(const void *a, const void *b, int Vd, const void *t, int Vt,
                         const int32_t *vmap, int dtype, const int32_t *draft, int B, int K,
                         double beta, double gamma,
                         double *lse, double *D, double *geff, int32_t *fused, double *gap,
                         double *top, uint8_t *accept, double *margin,
                         int32_t *accept_len, int32_t *token, int nthreads)
{
    if (B < 1 || K < 0 || Vd < 1 || Vt < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return 1;
    const int P = K + 1;
    const long R = (long)B * P;
    set_threads(nthreads);
    int bad_alloc = 0;
#pragma omp parallel
    {
        double *xa = malloc(sizeof(double) * (size_t)Vd);
        double *xb = malloc(sizeof(double) * (size_t)Vd);
        double *xt = malloc(sizeof(double) * (size_t)Vt);
        if (!xa || !xb || !xt) {
#pragma omp atomic write
            bad_alloc = 1;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < R; ++r) {
                for (int v = 0; v < Vd; ++v) {
                    xa[v] = widen(a, dtype, (size_t)r * (size_t)Vd + v);
                    xb[v] = widen(b, dtype, (size_t)r * (size_t)Vd + v);
                }
                for (int v = 0; v < Vt; ++v)
                    xt[v] = widen(t, dtype, (size_t)r * (size_t)Vt + v);
                const double La = logsumexp(xa, Vd), Lb = logsumexp(xb, Vd), Lt = logsumexp(xt, Vt);
                lse[3 * r + 0] = La;
                lse[3 * r + 1] = Lb;
                lse[3 * r + 2] = Lt;
                const double Dr = jsd(xa, La, xb, Lb, Vd);
                D[r] = Dr;
                geff[r] = gamma * exp(-Dr);
                /* fused token over the paired verifier tokens only */
                double best = -INFINITY, second = -INFINITY;
                int arg = -1;
                for (int v = 0; v < Vt; ++v) {
                    const int e = vmap[v];
                    if (e < 0 || e >= Vd)
                        continue;
                    const double sc = xt[v] + beta * (xa[e] - xb[e]);
                    if (arg < 0 || sc > best) {
                        second = best;
                        best = sc;
                        arg = v;
                    } else if (sc > second) {
                        second = sc;
                    }
                }
                fused[r] = arg;
                gap[r] = (arg >= 0 && second > -INFINITY) ? best - second : INFINITY;
                top[r] = best;
                const long bi = r / P;
                const int i = (int)(r % P);
                if (i < K) {
                    const int d = draft[bi * K + i];
                    const int e = (d >= 0 && d < Vt) ? vmap[d] : -1;
                    if (e < 0 || e >= Vd) {
                        accept[bi * K + i] = 0;
                        margin[bi * K + i] = NAN;
                    } else {
                        const double pt = exp(xt[d] - Lt);
                        const double pb = exp(xb[e] - Lb);
                        accept[bi * K + i] = (pt > geff[r] * pb) ? 1 : 0;
                        margin[bi * K + i] = (xt[d] - Lt) - (xb[e] - Lb) - log(gamma) + Dr;
                    }
                }
            }
        }
        free(xa);
        free(xb);
        free(xt);
    }
    if (bad_alloc)
        return 2;
    for (int bi = 0; bi < B; ++bi) {
        int n = K;
        for (int i = 0; i < K; ++i) {
            if (!accept[(long)bi * K + i]) {
                n = i;
                break;
            }
        }
        accept_len[bi] = n;
        token[bi] = fused[(long)bi * P + n];
    }
    return 0;
}

/* ======================================================================
 * E2-SCI adaptive JSD acceptance ("E2-SCI: Elastic Edge-Cloud Speculative
 * Decoding via Credit Inertia" notes, key design 3 "online adaptive
 * verification", with the credit state of key design 1)
 *
 * Inputs: y (drafter) and z (target) stored rows [B][W][V] (W draft
 * positions of one window per request); T_in[B] the threshold this window is
 * verified with; omega[B] the adaptive weight from the caller's predictor;
 * r_in[B] the smoothed acceptance rate before this window; alpha, tau
 * (tau_credit), T_base, T_min, T_max, ewma (the EWMA decay beta).
 * Outputs:
 *   D[B][W]        JSD(softmax(y_i) || softmax(z_i)), natural log
 *   accept[B][W]   D <= T_in (a divergence above the threshold rejects)
 *   accept_len[B]  first rejected position, or W
 *   r_out[B]       (1 - ewma) * r_in + ewma * accept_len / W
 *   T_out[B]       max(T_min, min(T_base + alpha * omega * (r_out - tau), T_max))
 * ====================================================================== */
int vwl_oracle_e2sci(const void *y, const void *z, int dtype, int B, int W, int V,
                     const float *T_in, const float *omega, const float *r_in,
                     double alpha, double tau, double T_base, double T_min, double T_max, double ewma,
                     double *D, uint8_t *accept, int32_t *accept_len, double *r_out, double *T_out,
                     int nthreads)
{
    if (B < 1 || W < 1 || V < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return 1;
    const long R = (long)B * W;
    set_threads(nthreads);
    int bad_alloc = 0;
#pragma omp parallel
    {
        double *xy = malloc(sizeof(double) * (size_t)V);
        double *xz = malloc(sizeof(double) * (size_t)V);
        if (!xy || !xz) {
#pragma omp atomic write
            bad_alloc = 1;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < R; ++r) {
                const size_t off = (size_t)r * (size_t)V;
                for (int v = 0; v < V; ++v) {
                    xy[v] = widen(y, dtype, off + v);
                    xz[v] = widen(z, dtype, off + v);
                }
                const double Dr = jsd(xy, logsumexp(xy, V), xz, logsumexp(xz, V), V);
                D[r] = Dr;
                accept[r] = (Dr <= (double)T_in[r / W]) ? 1 : 0;
            }
        }
        free(xy);
        free(xz);
    }
    if (bad_alloc)
        return 2;
    for (int bi = 0; bi < B; ++bi) {
        int n = W;
        for (int i = 0; i < W; ++i) {
            if (!accept[(long)bi * W + i]) {
                n = i;
                break;
            }
        }
        accept_len[bi] = n;
        /* credit state: EWMA of the window's accepted fraction */
        const double p_acc = (double)n / (double)W;
        const double r = (1.0 - ewma) * (double)r_in[bi] + ewma * p_acc;
        r_out[bi] = r;
        /* threshold of the next window: base plus the credit term, clamped */
        double T = T_base + alpha * (double)omega[bi] * (r - tau);
        if (T > T_max)
            T = T_max;
        if (T < T_min)
            T = T_min;
        T_out[bi] = T;
    }
    return 0;
}

/* ======================================================================
 * Row-level helpers exposed for the pins (same definitions, one row).
 * ====================================================================== */

/* Augmented target logits zhat = z + eta*T*(q - p) of one row (double in/out). */
int vwl_oracle_rapid_zhat(const double *z, const double *y, int V, double eta, double T,
                          double *zhat)
{
    if (V < 1 || !(T > 0.0))
        return 1;
    double *zs = malloc(sizeof(double) * (size_t)V);
    double *ys = malloc(sizeof(double) * (size_t)V);
    if (!zs || !ys) {
        free(zs);
        free(ys);
        return 2;
    }
    for (int v = 0; v < V; ++v) {
        zs[v] = z[v] / T;
        ys[v] = y[v] / T;
    }
    const double Lz = logsumexp(zs, V), Ly = logsumexp(ys, V);
    for (int v = 0; v < V; ++v)
        zhat[v] = z[v] + eta * T * (exp(ys[v] - Ly) - exp(zs[v] - Lz));
    free(zs);
    free(ys);
    return 0;
}

/* Tail-protected target of one row: phat_k = p_k where softmax(zhat/T)_k is
 * below 0.1 of its peak, softmax(zhat/T)_k elsewhere. */
int vwl_oracle_rapid_phat(const double *z, const double *y, int V, double eta, double T,
                          double *phat)
{
    if (V < 1 || !(T > 0.0))
        return 1;
    double *zh = malloc(sizeof(double) * (size_t)V);
    double *hs = malloc(sizeof(double) * (size_t)V);
    double *zs = malloc(sizeof(double) * (size_t)V);
    if (!zh || !hs || !zs) {
        free(zh);
        free(hs);
        free(zs);
        return 2;
    }
    vwl_oracle_rapid_zhat(z, y, V, eta, T, zh);
    for (int v = 0; v < V; ++v) {
        hs[v] = zh[v] / T;
        zs[v] = z[v] / T;
    }
    const double Lh = logsumexp(hs, V), Lz = logsumexp(zs, V);
    double Mh = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (hs[v] > Mh)
            Mh = hs[v];
    const double pmax = exp(Mh - Lh);
    for (int v = 0; v < V; ++v) {
        const double praw = exp(hs[v] - Lh);
        phat[v] = (praw < 0.1 * pmax) ? exp(zs[v] - Lz) : praw;
    }
    free(zh);
    free(hs);
    free(zs);
    return 0;
}
