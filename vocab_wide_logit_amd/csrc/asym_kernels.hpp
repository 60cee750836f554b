// AsymSpec verification pass (AsymSpec reading notes, section 4.1
// "contrastive delta-fusion" and section 4.2 "CDA gate"), with the variants
// of the notes' mechanism ablation as template choices:
//   DS    fusion source delta: a - b (the context gain), a (raw full-context
//         logits) or t - b (two-model difference, as in speculative
//         contrastive decoding)
//   GATE  the CDA threshold gamma*exp(-D), or the fixed threshold gamma
//         (no divergence: the JSD pass and the team wait are skipped, and a
//         is not read at all when delta = t - b)
// Each translation unit asym_<delta>.hip instantiates one fusion source.
// DS = kDeltaNone reads only a and b (no verifier row, no fused token): the
// two-tensor divergence pass behind E2-SCI and cross-family AsymSpec
// (pair_pass.hip).
//
// Launch 1, asym_rows_kernel: each logit row (one draft position of one
// request: a_i, b_i, t_i) is split over a team of W workgroups; each
// workgroup loads its chunk of the three rows once into registers and
//   pass AB softmax statistics of a, b, t: sums of 2^(x*log2e - c) against
//           one integer reference c per thread and tensor, taken from the
//           thread's first element (fp32 within a 16-byte group, fp64 across
//           groups and lanes; a sum that overflows is recomputed with a
//           reference per group), and the maximum of the fused score
//           t + beta*(a - b) per vector slot; its lowest index is searched
//           afterwards only by the threads that hold the workgroup maximum,
//           in the one slot that holds it -> the chunk record is published
//   pass C  once all W records of the row are in, the row log-sum-exps
//           L_a, L_b (combined in one fixed order by every member) and the
//           JSD terms of the chunk, from a and b still held in registers in
//           their stored form, one exponential per element (sqrt(p q) times
//           a polynomial in x = ln p - ln q); the row is read once.
// Each workgroup keeps two rows in flight: after publishing row r's record
// it runs passes A+B of row r+1 (already streamed from HBM straight into
// LDS) before it waits for row r's team and runs row r's pass C from a and
// b still held in registers.  The chunk of row r+2 streams into LDS
// meanwhile, and several teams share each compute unit.
//
// Launch 2, asym_finalize_kernel: one wave per row combines the W records
// (D, gamma*exp(-D), fused token, acceptance test of the draft); the wave
// that completes a request runs the first-rejection scan.
#pragma once

#include "vwl_device.hpp"
#include "vwl_internal.hpp"
#include "vwl_stage.hpp"

namespace vwl {

// Record words of one (row, member):
//   0..2  sums of 2^(x*log2e - c) for a, b, t (double bits)
//   3     references of the sums of a and b (two floats, log2 units)
//   4     reference of the sum of t (log2 units), maximum of the fused score
//   5     lowest index of the fused maximum (low 32 bits)
//   6     the chunk's share of D, sum_v (p ln(2p/(p+q)) + q ln(2q/(p+q))) / 2 (double bits)

// The delta-fusion score t + beta*delta, evaluated the same way everywhere.
template <int DS>
__device__ __forceinline__ float fused_score(float a, float b, float t, float beta) {
    if constexpr (DS == kDeltaAMinusB)
        return __fmaf_rn(beta, __fsub_rn(a, b), t);
    else if constexpr (DS == kDeltaA)
        return __fmaf_rn(beta, a, t);
    else
        return __fmaf_rn(beta, __fsub_rn(t, b), t);
}

// Whether a variant reads a at all, and whether it needs a's log-sum-exp.
template <int DS, int GATE>
struct AsymUse {
    static constexpr bool kLseA = GATE == kGateCda;
    static constexpr bool kReadA = kLseA || DS != kDeltaTMinusB;
    static constexpr bool kReadT = DS != kDeltaNone; // the verifier row and the fused token
    static constexpr int kTensors = kReadT ? 3 : 2;
};

// JSD term of one element.  With x = ln p - ln q (nats), d = |x| log2e,
// rho = 2^-d (ratio of the smaller to the larger probability) and
// Mx = max(p, q), the element contributes
//   p ln(2p/(p+q)) + q ln(2q/(p+q)) = -ln2 * Mx * g,
//   g = (1+rho)(log2(1+rho) - 1) + rho*d                    (|x| >= 1.2)
//     = (1+rho) * s * Q(s),  s = x^2                        (|x| <  1.2)
// The closed form cancels to O(x^2) from O(x) pieces, so below 1.2 the
// degree-4 polynomial Q (fitted to the exact even function x tanh(x/2) -
// 2 ln cosh(x/2) by jsd_poly_fit.py; 3.1e-7 relative in fp32) takes over;
// from 1.2 up the closed form is within 4.4e-7 relative.  Mx * g (<= 0) is returned.  x is
// formed from a - b and the row log-sum-exp difference, so it carries no
// rounding of the separate log-probabilities.  Finite for any finite or -inf
// logits (d is capped at 128, where rho*d underflows to 0; x is NaN only when
// both logits are -inf, and then Mx = 0).
constexpr float kJsdQ0 = -0x1.715472p-3f;
constexpr float kJsdQ1 = 0x1.7150ccp-6f;
constexpr float kJsdQ2 = -0x1.47a770p-9f;
constexpr float kJsdQ3 = 0x1.0cd8e2p-12f;
constexpr float kJsdQ4 = -0x1.465f7cp-16f;
constexpr float kJsdX0 = 1.2f; // polynomial below, closed form at and above

__device__ __forceinline__ float jsd_term(float la2, float lb2, float x) {
    const float M = __builtin_amdgcn_exp2f(fmaxf(la2, lb2));
    const float ax = fabsf(x);
    const float d = fminf(ax * kLog2e, 128.0f);
    const float rho = __builtin_amdgcn_exp2f(-d);
    const float opr = 1.0f + rho;
    // both forms, then a select: straight-line code across elements
    const float l2 = __builtin_amdgcn_logf(opr);
    const float g_closed = __fmaf_rn(opr, l2, __fmaf_rn(rho, d, -opr)); // opr*(l2 - 1) + rho*d
    const float s = x * x;
    float q = __fmaf_rn(kJsdQ4, s, kJsdQ3);
    q = __fmaf_rn(q, s, kJsdQ2);
    q = __fmaf_rn(q, s, kJsdQ1);
    q = __fmaf_rn(q, s, kJsdQ0);
    const float g_poly = opr * (s * q);
    return M * (ax < kJsdX0 ? g_poly : g_closed);
}

// One element's share of D, (p ln(2p/(p+q)) + q ln(2q/(p+q))) / 2, from the
// both-forms term above (any finite or -inf logits; exact fallback of the
// polynomial path below).
__device__ __forceinline__ float jsd_half_exact(float xa, float xb, float la_c, float lb_c, float dl) {
    return (-0.5f * 0.69314718055994531f) *
           jsd_term(__fmaf_rn(xa, kLog2e, -la_c), __fmaf_rn(xb, kLog2e, -lb_c), (xa - xb) - dl);
}

// The same share with one exponential: with x = ln p - ln q,
//   (p ln(2p/(p+q)) + q ln(2q/(p+q))) / 2 = sqrt(p q) * Psi(x) / 2,
//   Psi(x) = cosh(x/2) (x tanh(x/2) - 2 ln cosh(x/2)),
// since (p+q)/2 = sqrt(p q) cosh(x/2).  Psi is even and analytic (nearest
// singularities at x = +-i pi), so for |x| < kPsiX1 it is a polynomial in
// u = (x / kPsiX1)^2: Psi(x)/2 = u * P(u), P of degree 6 fitted by
// jsd_psi_fit.py (2.1e-7 relative in fp32 on |x| < 3).  sqrt(p q) = 2^h with h the mean
// of the two log2-probabilities.  Elements with u > 1 or NaN (|x| >= kPsiX1,
// -inf logits) are flagged and recomputed by jsd_half_exact.
constexpr float kPsiX1 = 3.0f;
constexpr float kPsiP0 = 0x1.1ffffep+0f;
constexpr float kPsiP1 = 0x1.22577cp-17f;
constexpr float kPsiP2 = 0x1.4360c6p-4f;
constexpr float kPsiP3 = -0x1.1b3e12p-5f;
constexpr float kPsiP4 = 0x1.2216eap-6f;
constexpr float kPsiP5 = -0x1.c2aa72p-8f;
constexpr float kPsiP6 = 0x1.64f9b8p-10f;
constexpr float kHalfLog2e = 0.72134752044448170f;

// Row constants of pass C, from the row log-sum-exps in log2 units.
struct JsdRow {
    float hmid;  // (L_a + L_b) / 2, log2 units
    float dlx;   // (L_a - L_b) ln 2 / kPsiX1
    float la_c, lb_c, dl; // L_a, L_b (log2 units) and L_a - L_b (nats), for the exact fallback
};

__device__ __forceinline__ JsdRow jsd_row(double La2, double Lb2) {
    JsdRow r;
    r.hmid = (float)(0.5 * (La2 + Lb2));
    r.dlx = (float)((La2 - Lb2) * (kLn2d / (double)kPsiX1));
    r.la_c = (float)La2;
    r.lb_c = (float)Lb2;
    r.dl = (float)((La2 - Lb2) * kLn2d);
    return r;
}

// D's share of one 16-byte vector of a and b (EPV elements), by the
// polynomial path; elements it does not cover make the whole vector take
// the exact path (rare: only elements with |x| >= kPsiX1 or -inf logits).
template <int DT>
__device__ __forceinline__ float jsd_vector(const uint4 &va, const uint4 &vb, const JsdRow &R) {
    constexpr int EPV = Elem<DT>::kPerVec;
    float J = 0.0f;
    uint32_t um = 0u; // largest u, compared as bits (u >= 0; NaN and inf compare above 1.0)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        const float xa = widen<DT>(va, e), xb = widen<DT>(vb, e);
        const float S = __builtin_amdgcn_exp2f(__fmaf_rn(xa + xb, kHalfLog2e, -R.hmid));
        const float xs = __fmaf_rn(xa - xb, 1.0f / kPsiX1, -R.dlx);
        const float u = xs * xs;
        float P = __fmaf_rn(kPsiP6, u, kPsiP5);
        P = __fmaf_rn(P, u, kPsiP4);
        P = __fmaf_rn(P, u, kPsiP3);
        P = __fmaf_rn(P, u, kPsiP2);
        P = __fmaf_rn(P, u, kPsiP1);
        P = __fmaf_rn(P, u, kPsiP0);
        J = __fmaf_rn(S * u, P, J);
        um = max(um, __float_as_uint(u));
    }
    if (um > 0x3f800000u) { // this lane: recompute the vector exactly
        J = 0.0f;
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            J += jsd_half_exact(widen<DT>(va, e), widen<DT>(vb, e), R.la_c, R.lb_c, R.dl);
    }
    return J;
}

// Row log-sum-exps, in log2 units, of N tensors from the W records of a
// row: log2 sum_w s_w 2^(c_w - C), C = max c_w, in fp64 and in one fixed
// order (lane w handles members w, w+64, ...; butterfly sums), so every
// caller gets the same bits.  F32ACC takes the final logarithm to fp32
// accuracy only (what the divergence pass rounds its constants to).  The references are integers, so each term is
// an exact power-of-two rescale.  Called by one whole wave.  Tensor k has its
// sums in word sw[k] and its reference in the low (hi[k] = false) or high
// half of word cw[k].  Records are `stride` words apart.
// log2 of a positive double to fp32 accuracy (about 1e-7 absolute): the
// exponent plus the fp32 logarithm of the mantissa.
__device__ __forceinline__ double log2_f32acc(double s) {
    int e = 0;
    const double m = frexp(s, &e);
    return (double)e + (double)__builtin_amdgcn_logf((float)m);
}

// 2^d for d <= 0 to fp32 accuracy (about 1e-7 relative): an exact power of
// two times the fp32 exponential of the fraction.
__device__ __forceinline__ double exp2_f32acc(double d) {
    const double k = floor(d);
    return ldexp((double)__builtin_amdgcn_exp2f((float)(d - k)), (int)fmax(k, -1100.0));
}

// One member's published log-sum-exp of a tensor over its chunk: the word
// of l = c + log2(S) (log2 units; -inf for S = 0; fp32-accurate logarithm)
// with -0.0 made +0.0 and the sign bit flipped, so every value gives a
// nonzero word and zero means "not yet published".  Self-contained: a
// reader that sees the word has the value, with no ordering against other
// stores.
__device__ __forceinline__ uint64_t lse_word(double S, float c) {
    const double l = (S == 0.0 ? -__builtin_inf() : (double)c + log2_f32acc(S)) + 0.0;
    return f64_bits(l) ^ 0x8000000000000000ull;
}
__device__ __forceinline__ double lse_of_word(uint64_t w) { return as_f64(w ^ 0x8000000000000000ull); }

// Record of one (row, member) for the finalize kernel (read after the row
// kernel ends) and, under the CDA gate, the two words pass C of the other
// members waits for.
__device__ __forceinline__ void publish_member(const AsymParams &P, long long row, int member, int nsums,
                                               const double *S, uint64_t w3, uint64_t w4, int fi, bool lse_words) {
    uint64_t *rec = P.rec + ((size_t)row * P.Wmax + member) * kRecWords;
    for (int k = 0; k < nsums; ++k)
        st_relaxed(rec + k, f64_bits(S[k]));
    st_relaxed(rec + 3, w3);
    if (nsums == 3) {
        st_relaxed(rec + 4, w4);
        st_relaxed(rec + 5, (uint64_t)(uint32_t)fi);
    }
    if (lse_words) {
        uint64_t *lw = P.lsum + ((size_t)row * P.Wmax + member) * 2;
        st_relaxed(lw + 0, lse_word(S[0], unpack_lo(w3)));
        st_relaxed(lw + 1, lse_word(S[1], unpack_hi(w3)));
    }
}

// The row's records and published words back to zero for the next call,
// by the finalize wave of the row after it has read them (lane w clears
// member w, the lane that read it).  Every call thus leaves its workspace
// zero-filled, whatever shape it had, so a later call of any shape finds
// zero where it waits for a published word.
__device__ __forceinline__ void clear_row_exchange(const AsymParams &P, long long row) {
    for (int w = threadIdx.x & 63; w < P.W; w += 64) {
        uint64_t *r = P.rec + ((size_t)row * P.Wmax + w) * kRecWords;
#pragma unroll
        for (int k = 0; k < kRecWords; ++k)
            st_relaxed(r + k, 0ull);
        uint64_t *lw = P.lsum + ((size_t)row * P.Wmax + w) * 2;
        st_relaxed(lw + 0, 0ull);
        st_relaxed(lw + 1, 0ull);
    }
}

// Row log-sum-exps (log2 units) of a and b from the W members' published
// words, by one whole wave (wave 0: it issues none of the staging loads, so
// waiting for its own loads here never waits for those): lane w takes
// members w, w + 64, ... in order, waiting (bounded) until each block of 64
// members' words is in, and folds them online; then M + log2 sum 2^(m - M)
// over the lanes (fp64, fp32-accurate exponentials and logarithm, one fixed
// order, so every caller gets the same bits).  Returns 2 when every word was
// in at the first look, 1 after waiting, 0 when the wait bound expired.
__device__ __forceinline__ void lse_fold(double l, double &m, double &s) {
    const double NEG_INF = -__builtin_inf();
    if (l > m) {
        s = (m == NEG_INF ? 0.0 : s * exp2_f32acc(m - l)) + 1.0;
        m = l;
    } else if (l > NEG_INF) {
        s += exp2_f32acc(l - m);
    } else if (!(l == NEG_INF)) {
        s = l; // NaN propagates
    }
}
__device__ __forceinline__ double lse_total(double m, double s) {
    const float Mf = wave_max((float)m);
    const double M = (double)Mf;
    const double t = (m == -__builtin_inf()) ? 0.0 : s * exp2_f32acc(m - M); // m - M < 1 (M is m rounded to fp32)
    const double tot = wave_sum(t);
    return (Mf == -__builtin_inff()) ? -__builtin_inf() : M + log2_f32acc(tot);
}
__device__ __forceinline__ uint32_t lse_poll(const uint64_t *lw, int W, double &La, double &Lb) {
    const int lane = threadIdx.x & 63;
    const double NEG_INF = -__builtin_inf();
    double ma = NEG_INF, sa = 0.0, mb = NEG_INF, sb = 0.0;
    uint32_t status = 2u;
    uint64_t t0 = 0;
    for (int w0 = 0; w0 < W; w0 += 64) {
        const int w = w0 + lane;
        uint64_t va = 0, vb = 0;
        for (;;) {
            if (w < W && va == 0)
                va = ld_relaxed(lw + (size_t)w * 2);
            if (w < W && vb == 0)
                vb = ld_relaxed(lw + (size_t)w * 2 + 1);
            if (__builtin_amdgcn_ballot_w64(w < W && (va == 0 || vb == 0)) == 0)
                break;
            if (status == 2u) {
                status = 1u;
                t0 = wall_clock64();
            }
            __builtin_amdgcn_s_sleep(1);
            if (wall_clock64() - t0 > kWaitLimitTicks)
                return 0u;
        }
        if (w < W) {
            lse_fold(lse_of_word(va), ma, sa);
            lse_fold(lse_of_word(vb), mb, sb);
        }
    }
    La = lse_total(ma, sa);
    Lb = lse_total(mb, sb);
    return status;
}

template <int N, bool F32ACC = false, bool PLAIN = false>
__device__ __forceinline__ void team_lse(const uint64_t *rec_row, int W, const int (&sw)[N], const int (&cw)[N],
                                         const bool (&hi)[N], double (&L)[N], int stride = kRecWords) {
    const int lane = threadIdx.x & 63;
    const float NEG = -3.0e38f;
    // PLAIN: records written by an earlier kernel, read with ordinary loads
    auto ld = [&](const uint64_t *p) { return PLAIN ? *p : ld_relaxed(p); };
    auto ref = [&](const uint64_t *r, int k) {
        const uint64_t x = ld(r + cw[k]);
        return hi[k] ? unpack_hi(x) : unpack_lo(x);
    };
    double a[N][2];
    float r[N][2], C[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        a[k][0] = a[k][1] = 0.0;
        r[k][0] = r[k][1] = NEG;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int w = lane + 64 * h;
        if (w < W) {
            const uint64_t *rw = rec_row + (size_t)w * stride;
#pragma unroll
            for (int k = 0; k < N; ++k) {
                r[k][h] = ref(rw, k);
                a[k][h] = as_f64(ld(rw + sw[k]));
            }
        }
    }
#pragma unroll
    for (int k = 0; k < N; ++k)
        C[k] = fmax_raw(r[k][0], r[k][1]);
    for (int w0 = 128; w0 < W; w0 += 64) { // teams wider than 128 members
        const int w = w0 + lane;
        if (w < W) {
            const uint64_t *rw = rec_row + (size_t)w0 * stride + lane * stride;
#pragma unroll
            for (int k = 0; k < N; ++k)
                C[k] = fmax_raw(C[k], ref(rw, k));
        }
    }
    double t[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        C[k] = wave_max(C[k]);
        t[k] = scale_pow2(a[k][0], r[k][0] - C[k]) + scale_pow2(a[k][1], r[k][1] - C[k]);
    }
    for (int w0 = 128; w0 < W; w0 += 64) { // teams wider than 128 members
        const int w = w0 + lane;
        if (w < W) {
            const uint64_t *rw = rec_row + (size_t)w0 * stride + lane * stride;
#pragma unroll
            for (int k = 0; k < N; ++k)
                t[k] += scale_pow2(as_f64(ld(rw + sw[k])), ref(rw, k) - C[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < N; ++k)
        L[k] = (double)C[k] + (F32ACC ? log2_f32acc(wave_sum(t[k])) : log2(wave_sum(t[k])));
}

// Online sum-of-exp state of one tensor over a thread's elements, fed one
// 16-byte group at a time.  The reference c (log2 units) is an integer at or
// above the running maximum of x*log2e, so the state means
// s = sum_v 2^(x_v*log2e - c) exactly as evaluated (the reference itself is
// never rounded), every exponent argument lies in [-inf, 0], and a change of
// reference rescales the running sum by an exact power of two.
struct OnlineLse {
    float c;   // reference, log2 units, integer-valued
    double s;
};

__device__ __forceinline__ void online_init(OnlineLse &st) {
    st.c = -3.0e38f;
    st.s = 0.0;
}

template <int EPV>
__device__ __forceinline__ void online_group(OnlineLse &st, const float (&x)[EPV]) {
    float g = x[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e)
        g = fmaxf(g, x[e]);
    // finite even for -inf rows
    const float c_new = fmaxf(st.c, __builtin_ceilf(fmaxf(g, -1e30f) * kLog2e));
    float acc = __builtin_amdgcn_exp2f(__fmaf_rn(x[0], kLog2e, -c_new));
#pragma unroll
    for (int e = 1; e < EPV; ++e)
        acc += __builtin_amdgcn_exp2f(__fmaf_rn(x[e], kLog2e, -c_new));
    st.s = scale_pow2(st.s, st.c - c_new) + (double)acc;
    st.c = c_new;
}

// Lazy variant of the same state: the reference is set once, from the
// thread's first element, and never moved while the sums stay finite, so no
// per-element maximum is needed.  Terms above 1 are exact in fp32 up to
// 2^128; a sum that overflows to +inf (an element more than 88 nats above the
// first one), or is NaN, sends the thread back to online_group, which gives
// the same state by its own rule.  Every exponent argument is still an
// element minus an integer, rounded once.
__device__ __forceinline__ float lazy_ref(float x0) {
    return __builtin_ceilf(fmaxf(x0, -1e30f) * kLog2e);
}

template <int EPV>
__device__ __forceinline__ float lazy_group_sum(const float (&x)[EPV], float c) {
    float e[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k)
        e[k] = __builtin_amdgcn_exp2f(__fmaf_rn(x[k], kLog2e, -c));
    if constexpr (EPV == 8)
        return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    else
        return (e[0] + e[1]) + (e[2] + e[3]);
}

__device__ __forceinline__ bool lse_sum_finite(double s) { return s <= 1.7976931348623157e308; }

// The thread's state over its vectors by online_group (the exact-reference
// path of a thread whose lazy sum overflowed).
template <int DT, int NV>
__device__ __forceinline__ OnlineLse lse_by_groups(const uint4 (&r)[NV], int nv) {
    constexpr int EPV = Elem<DT>::kPerVec;
    OnlineLse st;
    online_init(st);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if ((int)threadIdx.x + j * kThreads < nv) {
            float x[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                x[e] = widen<DT>(r[j], e);
            online_group<EPV>(st, x);
        }
    }
    return st;
}

// Rescale a thread's state to the workgroup reference C (fp64, exact).
__device__ __forceinline__ double rescale_to(const OnlineLse &st, float C) {
    return scale_pow2(st.s, st.c - C);
}


// Exact-reference pass AB of the two-tensor (divergence only) kind, the
// fallback of pair_pass_ab: softmax statistics of a and b against one
// reference per thread (moved by online_group where a sum overflows),
// reduced over the workgroup; thread 0 publishes record words 0, 1 (sums)
// and 3 (references).
template <int DT, int NV>
__device__ __forceinline__ void pair_pass_ab_exact(const AsymParams &P, long long row, int member, const RowSplit<DT> &sp,
                                             const uint4 (&ra)[NV], const uint4 (&rb)[NV], float sa, float sb,
                                             float *lds_f, double *lds_d) {
    constexpr int EPV = Elem<DT>::kPerVec;
    const int tid = threadIdx.x;
    OnlineLse la, lb;
    online_init(la);
    online_init(lb);
    if (tid < sp.nv) {
        la.c = lazy_ref(widen<DT>(ra[0], 0));
        lb.c = lazy_ref(widen<DT>(rb[0], 0));
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (tid + j * kThreads < sp.nv) {
            float xa[EPV], xb[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                xa[e] = widen<DT>(ra[j], e);
                xb[e] = widen<DT>(rb[j], e);
            }
            la.s += (double)lazy_group_sum<EPV>(xa, la.c);
            lb.s += (double)lazy_group_sum<EPV>(xb, lb.c);
        }
    }
    if (!lse_sum_finite(la.s))
        la = lse_by_groups<DT, NV>(ra, sp.nv);
    if (!lse_sum_finite(lb.s))
        lb = lse_by_groups<DT, NV>(rb, sp.nv);
    if (tid < sp.nsc) {
        const float x1a[1] = {sa}, x1b[1] = {sb};
        online_group<1>(la, x1a);
        online_group<1>(lb, x1b);
    }
    float mx[2] = {la.c, lb.c};
    __builtin_amdgcn_s_setprio(2); // the workgroup's serial section: reductions and publish
    block_max<2, false>(mx, lds_f);
    double S[2] = {rescale_to(la, mx[0]), rescale_to(lb, mx[1])};
    block_sum<2, false>(S, lds_d);
    if (tid == 0)
        publish_member(P, row, member, 2, S, pack2(mx[0], mx[1]), 0, 0, true);
    __builtin_amdgcn_s_setprio(0);
}

// Exact-reference passes A+B over one row's chunk held in registers (raw
// a, b, t plus the head/tail scalar), the fallback of asym_pass_ab: softmax
// statistics against one reference per thread, the fused maximum and its
// lowest index, reduced over the workgroup; thread 0 publishes the record.
template <int DT, int NV, int DS, int GATE>
__device__ __forceinline__ void asym_pass_ab_exact(const AsymParams &P, long long row, int member, const RowSplit<DT> &sp,
                                             const uint4 (&ra)[NV], const uint4 (&rb)[NV], const uint4 (&rt)[NV],
                                             float sa, float sb, float st, float *lds_f, double *lds_d, int *lds_i) {
    constexpr int EPV = Elem<DT>::kPerVec;
    constexpr bool LSE_A = AsymUse<DS, GATE>::kLseA;
    constexpr bool READ_A = AsymUse<DS, GATE>::kReadA;
    const int tid = threadIdx.x;
    const float NEG_INF = -__builtin_inff();
    const bool has_sc = tid < sp.nsc;
    OnlineLse la, lb, lt;
    online_init(la);
    online_init(lb);
    online_init(lt);
    if (tid < sp.nv) {
        if (LSE_A)
            la.c = lazy_ref(widen<DT>(ra[0], 0));
        lb.c = lazy_ref(widen<DT>(rb[0], 0));
        lt.c = lazy_ref(widen<DT>(rt[0], 0));
    }
    float vm[NV]; // fused maximum per vector slot
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        vm[j] = NEG_INF;
        if (tid + j * kThreads < sp.nv) {
            float xa[EPV], xb[EPV], xt[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                xa[e] = READ_A ? widen<DT>(ra[j], e) : 0.0f;
                xb[e] = widen<DT>(rb[j], e);
                xt[e] = widen<DT>(rt[j], e);
                vm[j] = fmaxf(vm[j], fused_score<DS>(xa[e], xb[e], xt[e], P.beta));
            }
            if (LSE_A)
                la.s += (double)lazy_group_sum<EPV>(xa, la.c);
            lb.s += (double)lazy_group_sum<EPV>(xb, lb.c);
            lt.s += (double)lazy_group_sum<EPV>(xt, lt.c);
        }
    }
    if (LSE_A && !lse_sum_finite(la.s))
        la = lse_by_groups<DT, NV>(ra, sp.nv);
    if (!lse_sum_finite(lb.s))
        lb = lse_by_groups<DT, NV>(rb, sp.nv);
    if (!lse_sum_finite(lt.s))
        lt = lse_by_groups<DT, NV>(rt, sp.nv);
    float fmax_t = vm[0];
#pragma unroll
    for (int j = 1; j < NV; ++j)
        fmax_t = fmaxf(fmax_t, vm[j]);
    float fs = NEG_INF;
    if (has_sc) {
        fs = fused_score<DS>(sa, sb, st, P.beta);
        fmax_t = fmaxf(fmax_t, fs);
        const float x1a[1] = {sa}, x1b[1] = {sb}, x1t[1] = {st};
        if (LSE_A)
            online_group<1>(la, x1a);
        online_group<1>(lb, x1b);
        online_group<1>(lt, x1t);
    }
    float mx[4] = {la.c, lb.c, lt.c, fmax_t};
    __builtin_amdgcn_s_setprio(2); // the workgroup's serial section: reductions and publish
    block_max<4, false>(mx, lds_f);
    const float Ca = mx[0], Cb = mx[1], Ct = mx[2], Fm = mx[3];

    // lowest index of the workgroup's fused maximum: only its holders
    // search, in the first vector slot whose maximum it is
    int fi = 0x7fffffff;
    if (fmax_t == Fm) {
        if (has_sc && fs == Fm)
            fi = scalar_index<DT>(sp, tid);
        bool found = false;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (!found && tid + j * kThreads < sp.nv && vm[j] == Fm) {
                found = true;
                int e_hit = EPV - 1;
#pragma unroll
                for (int e = EPV - 1; e >= 0; --e) {
                    const float ea = READ_A ? widen<DT>(ra[j], e) : 0.0f;
                    if (fused_score<DS>(ea, widen<DT>(rb[j], e), widen<DT>(rt[j], e), P.beta) == Fm)
                        e_hit = e;
                }
                fi = min(fi, sp.first_elem + (tid + j * kThreads) * EPV + e_hit);
            }
        }
    }
    double S[3] = {rescale_to(la, Ca), rescale_to(lb, Cb), rescale_to(lt, Ct)};
    block_sum_min<3, false>(S, fi, lds_d, lds_i);
    if (tid == 0)
        publish_member(P, row, member, 3, S, pack2(Ca, Cb), pack2(Ct, Fm), fi, GATE == kGateCda);
    __builtin_amdgcn_s_setprio(0);
}

// The wave's index, computed where it is used: an LDS address held across
// the row loop would take a register the loop needs (and be spilled to
// scratch, whose reload waits for the staging loads in flight).
__device__ __forceinline__ int fresh_wave() {
    int w = (int)threadIdx.x;
    asm volatile("" : "+v"(w));
    return __builtin_amdgcn_readfirstlane(w >> 6);
}

// LDS of the fast row reductions.
struct RowLds {
    double q[3 * 64];   // quad partial sums (quad_sum_post)
    float wmax[kWaves]; // fused maximum per wave
    float cref[3];      // the workgroup's references of a, b, t (log2 units)
    uint32_t flag;      // set when a thread's sum against them overflowed
    int idx;            // lowest index of the fused maximum (LDS atomic min)
};

// The workgroup's references for the chunk just taken: by wave 0, the
// integer ceiling of the largest first element of its lanes' first vectors,
// per tensor (lane 63 writes them; the caller's next barrier publishes
// them).  Every thread then sums 2^(x*log2e - c) against the same c, so the
// workgroup needs no maximum of references and no rescaling; the element
// that gave c contributes at least 1/2, so nothing that matters underflows,
// and a sum that overflows (an element 88 nats above c) sends the whole
// workgroup to the exact-reference pass.
template <int DT, int NV, bool READ_A, bool READ_T>
__device__ __forceinline__ void wg_refs(RowLds &L, const RowSplit<DT> &sp, const uint4 (&ra)[NV],
                                        const uint4 (&rb)[NV], const uint4 (&rt)[NV]) {
    const float NEG_INF = -__builtin_inff();
    const bool v0 = (int)threadIdx.x < sp.nv;
    float m[3] = {READ_A && v0 ? widen<DT>(ra[0], 0) : NEG_INF, v0 ? widen<DT>(rb[0], 0) : NEG_INF,
                  READ_T && v0 ? widen<DT>(rt[0], 0) : NEG_INF};
    wave_max_last_n<3>(m);
    if (threadIdx.x == 63) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            L.cref[k] = lazy_ref(m[k]);
    }
}

// Fast pass AB of the two-tensor kind (E2-SCI, cross-family drafter rows):
// sums of a and b against the workgroup references; lane 63 of wave 0
// publishes record words 0, 1 and 3.
template <int DT, int NV>
__device__ __forceinline__ void pair_pass_ab(const AsymParams &P, long long row, int member, const RowSplit<DT> &sp,
                                             const uint4 (&ra)[NV], const uint4 (&rb)[NV], float sa, float sb,
                                             RowLds &L, float *lds_f, double *lds_d) {
    constexpr int EPV = Elem<DT>::kPerVec;
    const int tid = threadIdx.x;
    const float ca = L.cref[0], cb = L.cref[1];
    float ga[NV], gb[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        ga[j] = gb[j] = 0.0f;
        if (tid + j * kThreads < sp.nv) {
            float xa[EPV], xb[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                xa[e] = widen<DT>(ra[j], e);
                xb[e] = widen<DT>(rb[j], e);
            }
            ga[j] = lazy_group_sum<EPV>(xa, ca);
            gb[j] = lazy_group_sum<EPV>(xb, cb);
        }
    }
    double S[2] = {0.0, 0.0};
#pragma unroll
    for (int j = 0; j < NV; j += 2) {
        S[0] += (double)(j + 1 < NV ? ga[j] + ga[j + 1] : ga[j]);
        S[1] += (double)(j + 1 < NV ? gb[j] + gb[j + 1] : gb[j]);
    }
    if (tid < sp.nsc) {
        S[0] += (double)__builtin_amdgcn_exp2f(__fmaf_rn(sa, kLog2e, -ca));
        S[1] += (double)__builtin_amdgcn_exp2f(__fmaf_rn(sb, kLog2e, -cb));
    }
    if (!(lse_sum_finite(S[0]) && lse_sum_finite(S[1])))
        L.flag = 1u;
    __builtin_amdgcn_s_setprio(2); // the workgroup's serial section: reductions and publish
    quad_sum_post<2>(S, L.q);
    lds_barrier();
    if (L.flag != 0u) { // rare: the exact-reference pass (uniform branch)
        pair_pass_ab_exact<DT, NV>(P, row, member, sp, ra, rb, sa, sb, lds_f, lds_d);
        if (tid == 63)
            L.flag = 0u;
        return;
    }
    if (tid < 64) {
        quad_sum_finish<2>(S, L.q);
        if (tid == 63)
            publish_member(P, row, member, 2, S, pack2(ca, cb), 0, 0, true);
    }
    __builtin_amdgcn_s_setprio(0);
}

// Fast passes A+B over one row's chunk held in registers (raw a, b, t plus
// the head/tail scalar): sums against the workgroup references, the fused
// maximum per vector slot; one workgroup maximum, then the lowest index of
// it (only its holders search, in the first slot that holds it, and merge
// by an LDS atomic minimum); lane 63 of wave 0 publishes the record.
template <int DT, int NV, int DS, int GATE>
__device__ __forceinline__ void asym_pass_ab(const AsymParams &P, long long row, int member, const RowSplit<DT> &sp,
                                             const uint4 (&ra)[NV], const uint4 (&rb)[NV], const uint4 (&rt)[NV],
                                             float sa, float sb, float st, RowLds &L, float *lds_f, double *lds_d,
                                             int *lds_i) {
    constexpr int EPV = Elem<DT>::kPerVec;
    constexpr bool LSE_A = AsymUse<DS, GATE>::kLseA;
    constexpr bool READ_A = AsymUse<DS, GATE>::kReadA;
    const int tid = threadIdx.x;
    const float NEG_INF = -__builtin_inff();
    const bool has_sc = tid < sp.nsc;
    const float ca = L.cref[0], cb = L.cref[1], ct = L.cref[2];
    float vm[NV], ga[NV], gb[NV], gt[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        vm[j] = NEG_INF;
        ga[j] = gb[j] = gt[j] = 0.0f;
        if (tid + j * kThreads < sp.nv) {
            float xa[EPV], xb[EPV], xt[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                xa[e] = READ_A ? widen<DT>(ra[j], e) : 0.0f;
                xb[e] = widen<DT>(rb[j], e);
                xt[e] = widen<DT>(rt[j], e);
                vm[j] = fmaxf(vm[j], fused_score<DS>(xa[e], xb[e], xt[e], P.beta));
            }
            if (LSE_A)
                ga[j] = lazy_group_sum<EPV>(xa, ca);
            gb[j] = lazy_group_sum<EPV>(xb, cb);
            gt[j] = lazy_group_sum<EPV>(xt, ct);
        }
    }
    double S[3] = {0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < NV; j += 2) {
        if (LSE_A)
            S[0] += (double)(j + 1 < NV ? ga[j] + ga[j + 1] : ga[j]);
        S[1] += (double)(j + 1 < NV ? gb[j] + gb[j + 1] : gb[j]);
        S[2] += (double)(j + 1 < NV ? gt[j] + gt[j + 1] : gt[j]);
    }
    float fmax_t = vm[0];
#pragma unroll
    for (int j = 1; j < NV; ++j)
        fmax_t = fmaxf(fmax_t, vm[j]);
    float fs = NEG_INF;
    if (has_sc) {
        fs = fused_score<DS>(sa, sb, st, P.beta);
        fmax_t = fmaxf(fmax_t, fs);
        if (LSE_A)
            S[0] += (double)__builtin_amdgcn_exp2f(__fmaf_rn(sa, kLog2e, -ca));
        S[1] += (double)__builtin_amdgcn_exp2f(__fmaf_rn(sb, kLog2e, -cb));
        S[2] += (double)__builtin_amdgcn_exp2f(__fmaf_rn(st, kLog2e, -ct));
    }
    if (!(lse_sum_finite(S[0]) && lse_sum_finite(S[1]) && lse_sum_finite(S[2])))
        L.flag = 1u;
    __builtin_amdgcn_s_setprio(2); // the workgroup's serial section: reductions and publish
    float fm[1] = {fmax_t};
    wave_max_last_n<1>(fm);
    if ((tid & 63) == 63)
        L.wmax[fresh_wave()] = fm[0];
    quad_sum_post<3>(S, L.q);
    lds_barrier();
    if (L.flag != 0u) { // rare: the exact-reference pass (uniform branch)
        asym_pass_ab_exact<DT, NV, DS, GATE>(P, row, member, sp, ra, rb, rt, sa, sb, st, lds_f, lds_d, lds_i);
        if (tid == 63)
            L.flag = 0u;
        return;
    }
    float Fm = L.wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        Fm = fmax_raw(Fm, L.wmax[w]);
    if (fmax_t == Fm) {
        int fi = 0x7fffffff;
        if (has_sc && fs == Fm)
            fi = scalar_index<DT>(sp, tid);
        bool found = false;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (!found && tid + j * kThreads < sp.nv && vm[j] == Fm) {
                found = true;
                int e_hit = EPV - 1;
#pragma unroll
                for (int e = EPV - 1; e >= 0; --e) {
                    const float ea = READ_A ? widen<DT>(ra[j], e) : 0.0f;
                    if (fused_score<DS>(ea, widen<DT>(rb[j], e), widen<DT>(rt[j], e), P.beta) == Fm)
                        e_hit = e;
                }
                fi = min(fi, sp.first_elem + (tid + j * kThreads) * EPV + e_hit);
            }
        }
        __hip_atomic_fetch_min(&L.idx, fi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (tid < 64)
        quad_sum_finish<3>(S, L.q);
    lds_barrier();
    if (tid == 63) {
        const int fi = L.idx;
        L.idx = 0x7fffffff;
        publish_member(P, row, member, 3, S, pack2(ca, cb), pack2(ct, Fm), fi, GATE == kGateCda);
    }
    __builtin_amdgcn_s_setprio(0);
}

// Resident waves per SIMD the row kernel is built for: the CDA variants keep
// a pending row's a and b in registers across the team wait.
template <int NV, int DS, int GATE>
constexpr int asym_rows_waves() {
    if constexpr (DS == kDeltaNone)
        return NV <= 2 ? 4 : NV <= 4 ? 3 : 2;
    else if constexpr (GATE == kGateCda)
        return NV <= 1 ? 4 : NV <= 4 ? 3 : 2;
    else
        return NV <= 4 ? 4 : 3;
}

// The workgroup reductions run without their closing barriers: every reuse
// of lds_f, lds_d and lds_i is separated from the previous reads by another
// barrier (the next reduction's, the team wait's, the combine's, or the
// staging barriers of the next row).  The serial sections of a row (the
// reductions, the record's publish, the team wait and the combine) run at
// wave priority 2: other workgroups' waves on the SIMD are then held back in
// favour of the short chains that every member of a team waits on.  The
// element passes run at priority 0, except on a member that found its team
// already complete when it came to wait (the team was waiting for it): its
// pass C and the next row's passes A+B run at priority 1, so the team's
// slowest member takes issue slots from co-resident members of other teams
// that are ahead of their own teams.  The members of a team share their CUs
// with different workgroups for the whole launch, so without this their
// speeds differ persistently and the team runs at its slowest member's pace.
// AsymSpec across families, staged verifier pass: the inverse alignment per
// part of the verifier row, built by the workgroups of the drafter's row
// kernel before they leave (the pass that reads it is the next launch).
// Workgroup b takes verifier tokens b*256 + tid, b*256 + tid + grid*256, ...
// For a pair (v, d) with v the i-th token of part p, the 16-bit key
// xkey[p][d] = i + 1 is set with an atomic OR on its 32-bit word; a key that
// was already set means two verifier tokens of one part share drafter token
// d, which sets the flag (the pass then meets the pairs in verifier order and
// ignores the keys).  An entry of vmap outside [-1, Vd) counts as unpaired
// and sets the map bit of dev_err.
template <int DT>
__device__ __forceinline__ void xfam_invert_slice(const AsymParams &P) {
    for (long long v = (long long)blockIdx.x * kThreads + threadIdx.x; v < P.Vt;
         v += (long long)gridDim.x * kThreads) {
        const int d = P.vmap[v];
        if (d < -1 || d >= P.V) {
            set_dev_err(P.dev_err, 8);
            continue;
        }
        if (d < 0)
            continue;
        const int pi = (int)(v / P.xpartlen);
        const uint32_t key = (uint32_t)(v - (long long)pi * P.xpartlen) + 1u;
        const size_t k = (size_t)pi * P.V + d;
        const int shift = (int)(k & 1) * 16;
        uint32_t *word = reinterpret_cast<uint32_t *>(P.xkey) + k / 2;
        const uint32_t old = __hip_atomic_fetch_or(word, key << shift, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((old >> shift) & 0xffffu)
            __hip_atomic_fetch_or(P.xdup, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int DT, int NV, int DS, int GATE>
__global__ __launch_bounds__(kThreads, (asym_rows_waves<NV, DS, GATE>())) void asym_rows_kernel(AsymParams P) {
    constexpr bool READ_A = AsymUse<DS, GATE>::kReadA;
    constexpr bool READ_T = AsymUse<DS, GATE>::kReadT;
    constexpr int NT = AsymUse<DS, GATE>::kTensors;
    __shared__ AsymStage<NV, NT> stage;
    __shared__ float lds_f[kWaves * 4];
    __shared__ double lds_d[kWaves * 3];
    __shared__ int lds_i[kWaves];
    __shared__ double sh_row[2];
    __shared__ uint32_t sh_u[2];
    __shared__ RowLds rl;

    const int tid = threadIdx.x;
    if (tid == 0)
        sh_u[0] = __hip_atomic_fetch_add(&P.ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 63) {
        rl.flag = 0u;
        rl.idx = 0x7fffffff;
    }
    __syncthreads();
    const uint32_t ticket = __builtin_amdgcn_readfirstlane(sh_u[0]);
    const int team = (int)(ticket / (uint32_t)P.W);
    const int member = (int)(ticket % (uint32_t)P.W);
    if (team >= P.R) {
        if constexpr (DS == kDeltaNone)
            if (P.xparts > 0)
                xfam_invert_slice<DT>(P);
        return;
    }
    const uint4 *A4 = static_cast<const uint4 *>(P.a);
    const uint4 *B4 = static_cast<const uint4 *>(P.b);
    const uint4 *T4 = static_cast<const uint4 *>(P.t);
    const int V = P.V, W = P.W;
    const bool wave0 = tid < 64;
    uint32_t na = 0u, nb = 0u, nt = 0u; // head/tail scalars of the staged row (raw bits)

    // Rows of this team: team, team + n_teams, ...  Two are in flight: the
    // pending row waits for its team while the next row's passes A+B run.
    auto issue = [&](long long r) {
        if (!wave0)
            prefetch_bulk<DT, NV, NT, READ_A>(stage, r, V, W, member, P.chunk, A4, B4, T4);
        else
            prefetch_scalars<DT, READ_A, READ_T>(r, V, W, member, P.chunk, P.a, P.b, P.t, na, nb, nt);
    };
    // Two register banks: the row whose passes A+B run next is taken into
    // one while the pending row's a and b (waiting for their pass C) stay in
    // the other, alternating, so no bank is ever copied.
    uint4 ra0[NV], rb0[NV], rt0[NV], ra1[NV], rb1[NV], rt1[NV];
    float sa0, sb0, st0, sa1, sb1, st1;
    RowSplit<DT> sp0, sp1;
    // The staged row: LDS -> registers; wave 0 also sets the workgroup's
    // references for the row (published by the closing barrier).
    auto take = [&](uint4(&ra)[NV], uint4(&rb)[NV], uint4(&rt)[NV], float &sa, float &sb, float &st,
                    const RowSplit<DT> &sp) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads(); // every wave's pieces have landed
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            if (READ_A)
                ra[j] = stage.v[0][j][tid];
            rb[j] = stage.v[1][j][tid];
            if (READ_T)
                rt[j] = stage.v[NT - 1][j][tid];
        }
        sa = widen_raw<DT>(na);
        sb = widen_raw<DT>(nb);
        st = widen_raw<DT>(nt);
        if (wave0)
            wg_refs<DT, NV, READ_A, READ_T>(rl, sp, ra, rb, rt);
        lds_barrier(); // every wave has read its vectors before the refill
    };
    auto pass_ab = [&](long long r, const RowSplit<DT> &sp, const uint4(&ra)[NV], const uint4(&rb)[NV],
                       const uint4(&rt)[NV], float sa, float sb, float st) {
        if constexpr (READ_T)
            asym_pass_ab<DT, NV, DS, GATE>(P, r, member, sp, ra, rb, rt, sa, sb, st, rl, lds_f, lds_d, lds_i);
        else
            pair_pass_ab<DT, NV>(P, r, member, sp, ra, rb, sa, sb, rl, lds_f, lds_d);
    };

    long long row = team;
    issue(row);
    sp0 = row_split<DT>(row, V, W, member, P.chunk);
    take(ra0, rb0, rt0, sa0, sb0, st0, sp0);
    if (row + P.n_teams < P.R)
        issue(row + P.n_teams);
    pass_ab(row, sp0, ra0, rb0, rt0, sa0, sb0, st0);
    if constexpr (GATE == kGateFixed) {
        // no divergence: each row is one pass, with the next row streaming in
        for (long long next = row + P.n_teams; next < P.R; next += P.n_teams) {
            sp0 = row_split<DT>(next, V, W, member, P.chunk);
            take(ra0, rb0, rt0, sa0, sb0, st0, sp0);
            if (next + P.n_teams < P.R)
                issue(next + P.n_teams);
            pass_ab(next, sp0, ra0, rb0, rt0, sa0, sb0, st0);
        }
        return;
    }
    // One step: passes A+B of the next row (into bank N), then the pending
    // row's (bank Q) team wait, combine and pass C.  Returns false when the
    // pending row was the team's last, or on a timeout.
    auto step = [&](uint4(&raN)[NV], uint4(&rbN)[NV], uint4(&rtN)[NV], float &saN, float &sbN, float &stN,
                    RowSplit<DT> &spN, const uint4(&paQ)[NV], const uint4(&pbQ)[NV], float psa, float psb,
                    const RowSplit<DT> &psp, bool &timed_out) -> bool {
        const long long next = row + P.n_teams;
        const bool has_next = next < P.R;
        if (has_next) {
            spN = row_split<DT>(next, V, W, member, P.chunk);
            take(raN, rbN, rtN, saN, sbN, stN, spN);
            if (next + P.n_teams < P.R)
                issue(next + P.n_teams);
            pass_ab(next, spN, raN, rbN, rtN, saN, sbN, stN);
        }

        // ---- the pending row: its team's log-sum-exps of a and b, waited
        // for and combined by wave 0, then pass C ----
        __builtin_amdgcn_s_setprio(2);
        if (wave0) {
            double La = 0.0, Lb = 0.0;
            const uint32_t st = lse_poll(P.lsum + (size_t)row * P.Wmax * 2, W, La, Lb);
            if (tid == 0) {
                sh_row[0] = La;
                sh_row[1] = Lb;
                sh_u[1] = st;
            }
        }
        lds_barrier();
        const uint32_t seen = __builtin_amdgcn_readfirstlane(sh_u[1]);
        if (seen == 0u) {
            if (tid == 0)
                set_dev_err(P.dev_err, 4);
            timed_out = true;
            return false;
        }
        const bool straggler = seen == 2u; // the team was waiting for this member
        if (straggler)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        const JsdRow jr = jsd_row(sh_row[0], sh_row[1]); // row log-sum-exps, log2 units
        float J = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (tid + j * kThreads < psp.nv)
                J += jsd_vector<DT>(paQ[j], pbQ[j], jr);
        if (tid < psp.nsc)
            J += jsd_half_exact(psa, psb, jr.la_c, jr.lb_c, jr.dl);
        double Jd[1] = {(double)J};
        __builtin_amdgcn_s_setprio(2);
        quad_sum_post<1>(Jd, rl.q);
        lds_barrier();
        if (tid < 64) {
            quad_sum_finish<1>(Jd, rl.q);
            if (tid == 63)
                P.rec[((size_t)row * P.Wmax + member) * kRecWords + 6] = f64_bits(Jd[0]);
        }
        if (straggler)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        if (!has_next)
            return false;
        row = next;
        return true;
    };
    bool timed_out = false;
    for (;;) {
        if (!step(ra1, rb1, rt1, sa1, sb1, st1, sp1, ra0, rb0, sa0, sb0, sp0, timed_out))
            break;
        if (!step(ra0, rb0, rt0, sa0, sb0, st0, sp0, ra1, rb1, sa1, sb1, sp1, timed_out))
            break;
    }
    if (timed_out)
        return;
    if constexpr (DS == kDeltaNone)
        if (P.xparts > 0)
            xfam_invert_slice<DT>(P);
}

// Row i of request bi, by one whole wave.
template <int DT, int GATE>
__device__ __forceinline__ void asym_finalize_row(const AsymParams &P, long long bi, int i, int lane,
                                                  uint32_t *sh_acc, int *sh_fi) {
    const int Pn = P.K + 1;
    const long long row = bi * Pn + i;
    const size_t row_off = (size_t)row * (size_t)P.V;
    // In flight together with the team sums: the draft's logits (lane 0) and
    // the fused-maximum and JSD words of the lane's first two members.
    int d = -1;
    double td = 0.0, bd = 0.0;
    if (lane == 0 && i < P.K) {
        d = P.draft[bi * P.K + i];
        if (d >= 0 && d < P.V) {
            td = (double)load_scalar<DT>(P.t, row_off + d);
            bd = (double)load_scalar<DT>(P.b, row_off + d);
        }
    }
    const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
    uint64_t w4[2] = {0, 0}, w5[2] = {0, 0}, w6[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int w = lane + 64 * h;
        if (w < P.W) {
            const uint64_t *r = rec_row + (size_t)w * kRecWords;
            w4[h] = ld_relaxed(r + 4);
            w5[h] = ld_relaxed(r + 5);
            if (GATE == kGateCda)
                w6[h] = ld_relaxed(r + 6);
        }
    }
    double L2[2];
    team_lse<2>(rec_row, P.W, {1, 2}, {3, 4}, {true, false}, L2);
    const double Lb = L2[0] * kLn2d, Lt = L2[1] * kLn2d;
    float fbest = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (lane + 64 * h < P.W)
            fbest = fmax_raw(fbest, unpack_hi(w4[h]));
    for (int w = lane + 128; w < P.W; w += 64) // teams wider than 128 members
        fbest = fmax_raw(fbest, unpack_hi(ld_relaxed(rec_row + (size_t)w * kRecWords + 4)));
    fbest = wave_max(fbest);
    double jsum = 0.0;
    int fidx = 0x7fffffff;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (lane + 64 * h < P.W) {
            if (GATE == kGateCda)
                jsum += as_f64(w6[h]);
            if (unpack_hi(w4[h]) == fbest)
                fidx = min(fidx, (int)(uint32_t)w5[h]);
        }
    }
    for (int w = lane + 128; w < P.W; w += 64) {
        const uint64_t *r = rec_row + (size_t)w * kRecWords;
        if (GATE == kGateCda)
            jsum += as_f64(ld_relaxed(r + 6));
        if (unpack_hi(ld_relaxed(r + 4)) == fbest)
            fidx = min(fidx, (int)(uint32_t)ld_relaxed(r + 5));
    }
    jsum = wave_sum(jsum);
    fidx = wave_min_int(fidx);
    clear_row_exchange(P, row);
    if (lane != 0)
        return;
    const double Dr = GATE == kGateCda ? jsum : 0.0; // enters the test only under CDA
    if (GATE == kGateCda) {
        P.D[row] = (float)Dr;
        P.geff[row] = (float)((double)P.gamma * exp(-Dr));
    } else {
        P.D[row] = __builtin_nanf("");
        P.geff[row] = P.gamma;
    }
    P.fused[row] = fidx;
    uint32_t acc = 0;
    if (i < P.K) {
        if (d < 0 || d >= P.V) {
            set_dev_err(P.dev_err, 1);
        } else {
            const double margin = (td - Lt) - (bd - Lb) - P.log_gamma + Dr;
            acc = margin > 0.0 ? 1u : 0u;
        }
        P.accept[bi * P.K + i] = (uint8_t)acc;
    }
    sh_acc[i] = acc;
    sh_fi[i] = fidx;
}

// One workgroup per request, one wave per row (up to 16 waves; wave w takes
// rows w, w + 16, ...): combine the row's W records and write its outputs; the rows' accept
// flags and fused tokens meet in LDS, and one thread runs the request's
// first-rejection scan.  Under the fixed gate D is not computed (NaN is
// written) and the threshold is gamma.
template <int DT, int GATE>
__global__ __launch_bounds__(kFinMaxThreads) void asym_finalize_kernel(AsymParams P) {
    __shared__ uint32_t sh_acc[kMaxDrafts + 1];
    __shared__ int sh_fi[kMaxDrafts + 1];
    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        P.ctl[0] = 0u; // ticket counter of the row kernel, for the next call
    const int Pn = P.K + 1;
    const long long bi = blockIdx.x;
    for (int i = (int)(threadIdx.x >> 6); i < Pn; i += (int)(blockDim.x >> 6)) {
        asym_finalize_row<DT, GATE>(P, bi, i, lane, sh_acc, sh_fi);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = P.K;
        for (int k = 0; k < P.K; ++k) {
            if (sh_acc[k] == 0u) {
                n = k;
                break;
            }
        }
        P.acc_len[bi] = n;
        P.token[bi] = sh_fi[n];
    }
}

template <int DT, int NV, int DS, int GATE>
static int blocks_per_cu_t() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, asym_rows_kernel<DT, NV, DS, GATE>, kThreads, 0) !=
        hipSuccess)
        return 0;
    return n;
}

template <int DT, int DS, int GATE>
static int blocks_per_cu_nv(int nv) {
    switch (nv) {
    case 1: return blocks_per_cu_t<DT, 1, DS, GATE>();
    case 2: return blocks_per_cu_t<DT, 2, DS, GATE>();
    case 4: return blocks_per_cu_t<DT, 4, DS, GATE>();
    case 8: return blocks_per_cu_t<DT, 8, DS, GATE>();
    }
    return 0;
}

template <int DS>
int asym_blocks_per_cu_ds(int dt, int nv, int gate) {
    if constexpr (DS == kDeltaNone) { // the divergence pass exists under the CDA kind only
        if (gate != kGateCda)
            return 0;
        return dt == DT_BF16 ? blocks_per_cu_nv<DT_BF16, DS, kGateCda>(nv) : blocks_per_cu_nv<DT_F32, DS, kGateCda>(nv);
    } else {
        if (dt == DT_BF16)
            return gate == kGateCda ? blocks_per_cu_nv<DT_BF16, DS, kGateCda>(nv)
                                    : blocks_per_cu_nv<DT_BF16, DS, kGateFixed>(nv);
        return gate == kGateCda ? blocks_per_cu_nv<DT_F32, DS, kGateCda>(nv)
                                : blocks_per_cu_nv<DT_F32, DS, kGateFixed>(nv);
    }
}

template <int DT, int NV, int DS, int GATE>
static hipError_t launch_t(const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    hipLaunchKernelGGL((asym_rows_kernel<DT, NV, DS, GATE>), dim3(plan.grid), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (after_rows) {
        e = hipEventRecord(after_rows, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((asym_finalize_kernel<DT, GATE>), dim3((unsigned)p.B), dim3(fin_threads(p.K + 1)), 0, s, p);
    return hipGetLastError();
}

template <int DT, int DS, int GATE>
static hipError_t launch_nv(const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    switch (plan.nv) {
    case 1: return launch_t<DT, 1, DS, GATE>(plan, p, s, after_rows);
    case 2: return launch_t<DT, 2, DS, GATE>(plan, p, s, after_rows);
    case 4: return launch_t<DT, 4, DS, GATE>(plan, p, s, after_rows);
    case 8: return launch_t<DT, 8, DS, GATE>(plan, p, s, after_rows);
    }
    return hipErrorInvalidValue;
}

template <int DS>
hipError_t launch_asym_ds(int dt, int gate, const Plan &plan, const AsymParams &p, hipStream_t s,
                          hipEvent_t after_rows) {
    if (dt == DT_BF16)
        return gate == kGateCda ? launch_nv<DT_BF16, DS, kGateCda>(plan, p, s, after_rows)
                                : launch_nv<DT_BF16, DS, kGateFixed>(plan, p, s, after_rows);
    return gate == kGateCda ? launch_nv<DT_F32, DS, kGateCda>(plan, p, s, after_rows)
                            : launch_nv<DT_F32, DS, kGateFixed>(plan, p, s, after_rows);
}

} // namespace vwl
