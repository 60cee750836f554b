// RAPID verification pass (RAPID notes, key design 2 "retrieval-augmented
// target distribution", key design 3 "tail protection", key design 4
// "adjusted residual sampling", and the rejection-sampling loop of the
// overall framework).
//
// Launch 1 (rows): each row (target z_i, RAG drafter y_i) is split over a
// team of W workgroups that keep their chunk in registers:
//   first pass   online softmax statistics of z/T and y/T -> record published
//   team         after all W records are in: L_z, L_y (fp64, fixed order)
//   second pass  p, q, h = zhat/T = z/T + eta*(q - p) from z, y still held in
//                registers; online statistics of h, its maximum and the
//                maximum's lowest index -> record
// Several teams share each compute unit, so one team's wait overlaps the
// others' loads and arithmetic.
// Launch 2 (finalise): one wave per row: Mhat (recomputed in fp64 at the
// argmax), L_zhat, the draft's tail-protected phat and q, the acceptance
// test; the wave that completes a request runs the first-rejection scan.
// Launches 3-6 work on the emitting row of each request only, in fp64: the
// row's normalisers refined in fp64, the augmented target's log-sum-exp, then
// per-chunk sums of the residual max(p - phat, p - q, 0) (or of p), then the
// inverse-CDF crossing of u * S in vocabulary order.
#include "vwl_device.hpp"
#include "vwl_internal.hpp"

namespace vwl {

// Record words of one (row, member):
//   0, 1  sums of 2^(x*log2e/T - c) for x = z and y (double bits)
//   2     their references cz, cy (two floats, log2 units)
//   3     sum of 2^(h*log2e - ch) for h = zhat/T (double bits)
//   4     maximum of h*log2e (float), its lowest index (int)
//   5     ch (float, log2 units)
__device__ __forceinline__ uint64_t pack_fi(float f, int i) {
    return (uint64_t)__float_as_uint(f) | ((uint64_t)(uint32_t)i << 32);
}

__device__ __forceinline__ double clamp_uniform(float u, int32_t *dev_err) {
    double x = (double)u;
    if (!(x >= 0.0) || !(x < 1.0)) {
        set_dev_err(dev_err, 2);
        x = (x >= 1.0) ? 1.0 - 0x1p-24 : 0.0;
    }
    return x;
}

__device__ __forceinline__ double as_f64(uint64_t w) { return __longlong_as_double((long long)w); }
__device__ __forceinline__ uint64_t f64_bits(double x) { return (uint64_t)__double_as_longlong(x); }

// Row log-sum-exp in log2 units from the W records (fixed order; same
// scheme as the AsymSpec kernel).  Called by one whole wave.
__device__ __forceinline__ double team_lse2_r(const uint64_t *rec_row, int W, int word, int cword, bool hi) {
    const int lane = threadIdx.x & 63;
    float C = -__builtin_inff();
    for (int w = lane; w < W; w += 64) {
        const uint64_t x = ld_relaxed(rec_row + (size_t)w * kRecWords + cword);
        C = fmaxf(C, __uint_as_float(hi ? (uint32_t)(x >> 32) : (uint32_t)x));
    }
    C = wave_max(C);
    double s = 0.0;
    for (int w = lane; w < W; w += 64) {
        const uint64_t *r = rec_row + (size_t)w * kRecWords;
        const uint64_t x = ld_relaxed(r + cword);
        const double sw = as_f64(ld_relaxed(r + word));
        if (sw > 0.0)
            s += sw * exp2((double)__uint_as_float(hi ? (uint32_t)(x >> 32) : (uint32_t)x) - (double)C);
    }
    s = wave_sum(s);
    return (double)C + log2(s);
}

// Online sum-of-exp state of one tensor over a thread's elements, fed one
// 16-byte group of raw logits x at a time, for the exponent x*c (log2 units,
// c = log2e/T).  The product is evaluated as an fma with the reference
// subtracted before rounding, plus the low part of c, so no rounding of x/T
// or of x*c at the logits' magnitude enters the exponent.  The reference is
// kept as the exact fp32 value used, so the state means
// s = sum_v 2^(x_v*c - ref); the running sum is rescaled once per group.
struct OnlineLseR {
    float c;   // reference, log2 units (>= max x*c up to rounding)
    double s;
};

struct ExpCoef {
    float hi, lo; // c = hi + lo, hi <= c, lo > 0 (so -inf logits stay -inf)
};

__device__ __forceinline__ float scaled_arg(float x, ExpCoef k, float ref) {
    return __fmaf_rn(x, k.lo, __fmaf_rn(x, k.hi, -ref));
}

template <int EPV>
__device__ __forceinline__ void online_group_r(OnlineLseR &st, const float (&x)[EPV], ExpCoef k) {
    float g = x[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e)
        g = fmaxf(g, x[e]);
    const float c_new = fmaxf(st.c, fmaxf(g, -1e30f) * k.hi); // finite even for -inf rows
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e)
        acc += __builtin_amdgcn_exp2f(scaled_arg(x[e], k, c_new));
    const float scale = __builtin_amdgcn_exp2f(st.c - c_new);
    st.s = __fma_rn(st.s, (double)scale, (double)acc);
    st.c = c_new;
}

// Rescale a thread's state to the workgroup reference C (fp64 result).
__device__ __forceinline__ double rescale_to_r(const OnlineLseR &st, float C) {
    if (!(st.s > 0.0))
        return 0.0;
    return st.s * (double)__builtin_amdgcn_exp2f(st.c - C);
}

// The augmentation of one element in the second pass.  p = 2^(z*c - Lz2)
// and q = 2^(y*c - Ly2) with the row log-sum-exps (log2 units) as float
// pairs, so p and q carry only the exp2 rounding.  h = zhat/T in log2 units is
// z*c + eta*log2e*(q - p); happ is its fp32 value (for the maximum and the
// reference), and h_arg(ref) its exponent relative to a reference with the
// same exact-product treatment as above.
struct AugCoef {
    ExpCoef c;
    float lz_hi, lz_lo, ly_hi, ly_lo, eta2;
};

__device__ __forceinline__ float aug_dqp(const AugCoef &k, float z, float y) {
    const float p = __builtin_amdgcn_exp2f(scaled_arg(z, k.c, k.lz_hi) - k.lz_lo);
    const float q = __builtin_amdgcn_exp2f(scaled_arg(y, k.c, k.ly_hi) - k.ly_lo);
    return q - p;
}
__device__ __forceinline__ float aug_happ(const AugCoef &k, float z, float dqp) {
    return __fmaf_rn(k.eta2, dqp, z * k.c.hi);
}
__device__ __forceinline__ float aug_harg(const AugCoef &k, float z, float dqp, float ref) {
    return __fmaf_rn(k.eta2, dqp, scaled_arg(z, k.c, ref));
}

template <int EPV>
__device__ __forceinline__ void online_group_h(OnlineLseR &st, const AugCoef &k, const float (&z)[EPV],
                                               const float (&dqp)[EPV], const float (&happ)[EPV]) {
    float g = happ[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e)
        g = fmaxf(g, happ[e]);
    const float c_new = fmaxf(st.c, fmaxf(g, -1e30f));
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e)
        acc += __builtin_amdgcn_exp2f(aug_harg(k, z[e], dqp[e], c_new));
    const float scale = __builtin_amdgcn_exp2f(st.c - c_new);
    st.s = __fma_rn(st.s, (double)scale, (double)acc);
    st.c = c_new;
}

__device__ __forceinline__ void split_f64(double x, float &hi, float &lo) {
    hi = (float)x;
    lo = (float)(x - (double)hi);
}

template <int DT, int NV>
__global__ __launch_bounds__(kThreads, (NV <= 2 ? 4 : 3)) void rapid_rows_kernel(RapidParams P) {
    constexpr int EPV = Elem<DT>::kPerVec;
    __shared__ float lds_f[kWaves * 2];
    __shared__ double lds_d[kWaves * 2];
    __shared__ int lds_i[kWaves];
    __shared__ double sh_row[2];
    __shared__ uint32_t sh_u[2];

    const int tid = threadIdx.x;
    if (tid == 0)
        sh_u[0] = __hip_atomic_fetch_add(&P.ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t ticket = sh_u[0];
    const int team = (int)(ticket / (uint32_t)P.W);
    const int member = (int)(ticket % (uint32_t)P.W);
    const uint4 *Z4 = static_cast<const uint4 *>(P.z);
    const uint4 *Y4 = static_cast<const uint4 *>(P.y);
    const float NEG_INF = -__builtin_inff();
    const ExpCoef kc{P.c_hi, P.c_lo};

    for (long long row = team; row < P.R; row += P.n_teams) {
        const RowSplit<DT> sp = row_split<DT>(row, P.V, P.W, member, P.chunk);
        const size_t row_off = (size_t)row * (size_t)P.V;
        const bool has_sc = tid < sp.nsc;
        const int sidx = has_sc ? scalar_index<DT>(sp, tid) : 0;

        uint4 rz[NV], ry[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int k = tid + j * kThreads;
            if (k < sp.nv) {
                rz[j] = Z4[sp.vec0 + k];
                ry[j] = Y4[sp.vec0 + k];
            }
        }
        float sz = NEG_INF, sy = NEG_INF;
        if (has_sc) {
            sz = load_scalar<DT>(P.z, row_off + sidx);
            sy = load_scalar<DT>(P.y, row_off + sidx);
        }

        // ---- first pass: online softmax statistics of z/T and y/T ----
        OnlineLseR lz{NEG_INF, 0.0}, ly{NEG_INF, 0.0};
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (tid + j * kThreads < sp.nv) {
                float xz[EPV], xy[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    xz[e] = widen<DT>(rz[j], e);
                    xy[e] = widen<DT>(ry[j], e);
                }
                online_group_r<EPV>(lz, xz, kc);
                online_group_r<EPV>(ly, xy, kc);
            }
        if (has_sc) {
            const float a1[1] = {sz}, b1[1] = {sy};
            online_group_r<1>(lz, a1, kc);
            online_group_r<1>(ly, b1, kc);
        }
        float mx[2] = {lz.c, ly.c};
        block_max<2>(mx, lds_f);
        double S[2] = {rescale_to_r(lz, mx[0]), rescale_to_r(ly, mx[1])};
        block_sum<2>(S, lds_d);

        const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
        uint32_t *ctr = P.row_ctr + (size_t)row * 16;
        if (tid == 0) {
            uint64_t *rec = P.rec + ((size_t)row * P.Wmax + member) * kRecWords;
            st_relaxed(rec + 0, f64_bits(S[0]));
            st_relaxed(rec + 1, f64_bits(S[1]));
            st_relaxed(rec + 2, (uint64_t)__float_as_uint(mx[0]) | ((uint64_t)__float_as_uint(mx[1]) << 32));
            publish_add(ctr, 1u);
            sh_u[1] = wait_at_least(ctr, (uint32_t)P.W) ? 1u : 0u;
        }
        __syncthreads();
        if (!sh_u[1]) {
            if (tid == 0)
                set_dev_err(P.dev_err, 4);
            return;
        }
        if (tid < 64) {
            const double Lz2 = team_lse2_r(rec_row, P.W, 0, 2, false);
            const double Ly2 = team_lse2_r(rec_row, P.W, 1, 2, true);
            if (tid == 0) {
                sh_row[0] = Lz2;
                sh_row[1] = Ly2;
            }
        }
        __syncthreads();

        // ---- second pass: h = zhat/T = z/T + eta*(q - p); online statistics ----
        AugCoef ak;
        ak.c = kc;
        split_f64(sh_row[0], ak.lz_hi, ak.lz_lo);
        split_f64(sh_row[1], ak.ly_hi, ak.ly_lo);
        ak.eta2 = P.eta2;
        OnlineLseR lh{NEG_INF, 0.0};
        float hmax_t = NEG_INF;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (tid + j * kThreads < sp.nv) {
                float xz[EPV], dq[EPV], ha[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    xz[e] = widen<DT>(rz[j], e);
                    dq[e] = aug_dqp(ak, xz[e], widen<DT>(ry[j], e));
                    ha[e] = aug_happ(ak, xz[e], dq[e]);
                    hmax_t = fmaxf(hmax_t, ha[e]);
                }
                online_group_h<EPV>(lh, ak, xz, dq, ha);
            }
        float hs = NEG_INF;
        if (has_sc) {
            const float dq1[1] = {aug_dqp(ak, sz, sy)};
            hs = aug_happ(ak, sz, dq1[0]);
            hmax_t = fmaxf(hmax_t, hs);
            const float z1[1] = {sz}, h1[1] = {hs};
            online_group_h<1>(lh, ak, z1, dq1, h1);
        }
        float hm[2] = {lh.c, hmax_t};
        block_max<2>(hm, lds_f);
        const float Ch = hm[0], Hm = hm[1];
        double Sh[1] = {rescale_to_r(lh, Ch)};
        block_sum<1>(Sh, lds_d);
        int hi = 0x7fffffff;
        if (hmax_t == Hm) {
            if (has_sc && hs == Hm)
                hi = sidx;
            bool found = false;
#pragma unroll
            for (int j = 0; j < NV; ++j)
                if (!found && tid + j * kThreads < sp.nv)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const float z1 = widen<DT>(rz[j], e);
                        if (!found && aug_happ(ak, z1, aug_dqp(ak, z1, widen<DT>(ry[j], e))) == Hm) {
                            hi = min(hi, sp.first_elem + (tid + j * kThreads) * EPV + e);
                            found = true;
                        }
                    }
        }
        hi = block_min_int(hi, lds_i);
        if (tid == 0) {
            uint64_t *rec = P.rec + ((size_t)row * P.Wmax + member) * kRecWords;
            rec[3] = f64_bits(Sh[0]);
            rec[4] = pack_fi(Hm, hi);
            rec[5] = (uint64_t)__float_as_uint(Ch);
        }
    }
}

// One wave per row: row statistics from the W records (Mhat recomputed in
// fp64 at the argmax), the tail-protected acceptance test of the draft, and
// the first-rejection scan by the wave that completes a request.
template <int DT>
__global__ __launch_bounds__(kThreads) void rapid_finalize_kernel(RapidParams P) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        P.ctl[0] = 0u; // ticket counter of the row kernel, for the next call
    if (row >= P.R)
        return;
    const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
    const double Lz = team_lse2_r(rec_row, P.W, 0, 2, false) * kLn2d;
    const double Ly = team_lse2_r(rec_row, P.W, 1, 2, true) * kLn2d;
    const double Lh = team_lse2_r(rec_row, P.W, 3, 5, false) * kLn2d;
    float mh = -__builtin_inff();
    for (int w = lane; w < P.W; w += 64)
        mh = fmaxf(mh, __uint_as_float((uint32_t)ld_relaxed(rec_row + (size_t)w * kRecWords + 4)));
    mh = wave_max(mh);
    int hidx = 0x7fffffff;
    for (int w = lane; w < P.W; w += 64) {
        const uint64_t w4 = ld_relaxed(rec_row + (size_t)w * kRecWords + 4);
        if (__uint_as_float((uint32_t)w4) == mh)
            hidx = min(hidx, (int)(uint32_t)(w4 >> 32));
    }
    hidx = wave_min_int(hidx);
    if (lane != 0)
        return;
    const double T = P.T, eta_d = P.eta_d;
    const size_t row_off = (size_t)row * (size_t)P.V;
    // Mhat: the augmented logit at the argmax, recomputed in fp64
    double Mh = (double)mh * kLn2d;
    if (hidx >= 0 && hidx < P.V) {
        const double zx = (double)load_scalar<DT>(P.z, row_off + hidx) / T;
        const double yx = (double)load_scalar<DT>(P.y, row_off + hidx) / T;
        Mh = zx + eta_d * (exp(yx - Ly) - exp(zx - Lz));
    } else {
        hidx = -1;
    }
    double *rs = P.rowstat + (size_t)row * kRowStatWords;
    rs[0] = Lz;
    rs[1] = Ly;
    rs[2] = Mh;
    rs[3] = Lh;
    rs[4] = (double)hidx;
    const int Pn = P.G + 1;
    const long long bi = row / Pn;
    const int i = (int)(row - bi * Pn);
    uint32_t acc = 0;
    if (i < P.G) {
        const long long k = bi * P.G + i;
        const int x = P.draft[k];
        float phd = 0.f, qd = 0.f;
        if (x < 0 || x >= P.V) {
            set_dev_err(P.dev_err, 1);
        } else {
            const double zx = (double)load_scalar<DT>(P.z, row_off + x) / T;
            const double yx = (double)load_scalar<DT>(P.y, row_off + x) / T;
            const double p = exp(zx - Lz);
            const double q = exp(yx - Ly);
            const double h = zx + eta_d * (q - p);
            const double ph = (h - Mh < -2.302585092994046) ? p : exp(h - Lh);
            const double u = clamp_uniform(P.u_accept[k], P.dev_err);
            acc = (u * q < ph) ? 1u : 0u;
            phd = (float)ph;
            qd = (float)q;
        }
        P.accept[k] = (uint8_t)acc;
        if (P.p_hat_draft)
            P.p_hat_draft[k] = phd;
        if (P.q_draft)
            P.q_draft[k] = qd;
    }
    st_relaxed(P.row_info + (size_t)row * 2 + 1, acc);
    P.row_ctr[(size_t)row * 16] = 0u; // arrivals of the row kernel, for the next call
    uint32_t *rq = P.req_ctr + (size_t)bi * 16;
    const uint32_t done = publish_add(rq, 1u);
    if (done == (uint32_t)P.G) {
        const size_t r0 = (size_t)bi * Pn;
        int n = P.G;
        for (int k = 0; k < P.G; ++k)
            if (ld_relaxed(P.row_info + (r0 + k) * 2 + 1) == 0u) {
                n = k;
                break;
            }
        P.acc_len[bi] = n;
        st_relaxed(rq, 0u);
    }
}

// ---------------------------------------------------------------------------
// Emitting row, all in fp64.  With n the accept length: n < G uses the
// residual max(p - phat, p - q, 0) of row n; otherwise p.  The row's
// normalisers are refined in fp64 before use, so the residual's three
// probabilities share fp64-accurate normalisers:
//   launch 3  per chunk: sum exp(z/T - L_z), sum exp(y/T - L_y) around the
//             row pass's values          -> L_z, L_y (fp64), Mhat at the argmax
//   launch 4  per chunk: sum exp(h - Mhat) -> L_zhat (fp64)
//   launch 5  per chunk: residual and target sums
//   launch 6  the inverse-CDF crossing of u * S in vocabulary order
// Every workgroup combines the per-chunk partials in chunk order, so all of
// them derive the same bits.  Per-request partials [B][We][8]:
//   0 residual sum, 1 target sum, 2 sum of exp(h - Mhat), 3 sum of
//   exp(z/T - L_z), 4 sum of exp(y/T - L_y).
// ---------------------------------------------------------------------------
struct EmitRow {
    long long row;
    size_t row_off;
    int n;
    bool resid; // n < G: the residual of row n
};

__device__ __forceinline__ EmitRow emit_row(const RapidParams &P, int bi) {
    int n = P.acc_len[bi];
    if (n < 0 || n > P.G) // only after an abandoned row pass; keeps the row index in range
        n = P.G;
    EmitRow e;
    e.n = n;
    e.resid = n < P.G;
    e.row = (long long)bi * (P.G + 1) + n;
    e.row_off = (size_t)e.row * (size_t)P.V;
    return e;
}

// Refined statistics of the emitting row (st[0] L_z, st[1] L_y, st[2] Mhat,
// st[3] L_zhat when with_lh), computed by thread 0 and shared through LDS.
template <int DT>
__device__ __forceinline__ void emit_stats(const RapidParams &P, int bi, const EmitRow &er, bool with_lh,
                                           double *sh_st) {
    if (threadIdx.x == 0) {
        const double *rs = P.rowstat + (size_t)er.row * kRowStatWords;
        const double *parts = P.emit + (size_t)bi * P.We * kEmitWords;
        double sz = 0.0, sy = 0.0, shh = 0.0;
        for (int k = 0; k < P.We; ++k) {
            sz += parts[kEmitWords * k + 3];
            sy += parts[kEmitWords * k + 4];
        }
        const double Lz = rs[0] + log(sz), Ly = rs[1] + log(sy);
        double Mh = rs[2];
        const int hidx = (int)rs[4];
        if (hidx >= 0 && hidx < P.V) {
            const double zx = (double)load_scalar<DT>(P.z, er.row_off + hidx) / P.T;
            const double yx = (double)load_scalar<DT>(P.y, er.row_off + hidx) / P.T;
            Mh = zx + P.eta_d * (exp(yx - Ly) - exp(zx - Lz));
        }
        sh_st[0] = Lz;
        sh_st[1] = Ly;
        sh_st[2] = Mh;
        if (with_lh) {
            for (int k = 0; k < P.We; ++k)
                shh += parts[kEmitWords * k + 2];
            sh_st[3] = Mh + log(shh);
        }
    }
    __syncthreads();
}

template <int DT>
__device__ __forceinline__ double emit_h(const RapidParams &P, size_t row_off, int v, const double *st,
                                         double &p, double &q) {
    const double zs = (double)load_scalar<DT>(P.z, row_off + v) / P.T;
    const double ys = (double)load_scalar<DT>(P.y, row_off + v) / P.T;
    p = exp(zs - st[0]);
    q = exp(ys - st[1]);
    return zs + P.eta_d * (q - p);
}

template <int DT>
__device__ __forceinline__ void emit_weights(const RapidParams &P, size_t row_off, int v, const double *st,
                                             bool resid, double &r, double &p) {
    if (!resid) {
        p = exp((double)load_scalar<DT>(P.z, row_off + v) / P.T - st[0]);
        r = 0.0;
        return;
    }
    double q;
    const double h = emit_h<DT>(P, row_off, v, st, p, q);
    const double ph = (h - st[2] < -2.302585092994046) ? p : exp(h - st[3]);
    double x = p - ph;
    if (p - q > x)
        x = p - q;
    r = x > 0.0 ? x : 0.0;
}

constexpr int kEmitPerThread = kEmitChunk / kThreads; // contiguous elements per thread

template <int DT>
__global__ __launch_bounds__(kThreads) void rapid_emit_norm_kernel(RapidParams P) {
    __shared__ double lds_d[kWaves * 2];
    const int w = (int)(blockIdx.x % (unsigned)P.We), bi = (int)(blockIdx.x / (unsigned)P.We);
    const EmitRow er = emit_row(P, bi);
    const double *rs = P.rowstat + (size_t)er.row * kRowStatWords;
    const double Lz = rs[0], Ly = rs[1];
    const int v0 = w * kEmitChunk + threadIdx.x * kEmitPerThread;
    double s[2] = {0.0, 0.0};
    for (int e = 0; e < kEmitPerThread; ++e) {
        const int v = v0 + e;
        if (v < P.V) {
            s[0] += exp((double)load_scalar<DT>(P.z, er.row_off + v) / P.T - Lz);
            if (er.resid)
                s[1] += exp((double)load_scalar<DT>(P.y, er.row_off + v) / P.T - Ly);
        }
    }
    block_sum<2>(s, lds_d);
    if (threadIdx.x == 0) {
        double *o = P.emit + ((size_t)bi * P.We + w) * kEmitWords;
        o[3] = s[0];
        o[4] = er.resid ? s[1] : 1.0;
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rapid_emit_lse_kernel(RapidParams P) {
    __shared__ double lds_d[kWaves];
    __shared__ double sh_st[4];
    const int w = (int)(blockIdx.x % (unsigned)P.We), bi = (int)(blockIdx.x / (unsigned)P.We);
    const EmitRow er = emit_row(P, bi);
    if (!er.resid)
        return; // no residual on this request
    emit_stats<DT>(P, bi, er, false, sh_st);
    const double st[3] = {sh_st[0], sh_st[1], sh_st[2]};
    const int v0 = w * kEmitChunk + threadIdx.x * kEmitPerThread;
    double s[1] = {0.0};
    for (int e = 0; e < kEmitPerThread; ++e) {
        const int v = v0 + e;
        if (v < P.V) {
            double p, q;
            s[0] += exp(emit_h<DT>(P, er.row_off, v, st, p, q) - st[2]);
        }
    }
    block_sum<1>(s, lds_d);
    if (threadIdx.x == 0)
        P.emit[((size_t)bi * P.We + w) * kEmitWords + 2] = s[0];
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rapid_emit_sum_kernel(RapidParams P) {
    __shared__ double lds_d[kWaves * 2];
    __shared__ double sh_st[4];
    const int w = (int)(blockIdx.x % (unsigned)P.We), bi = (int)(blockIdx.x / (unsigned)P.We);
    const EmitRow er = emit_row(P, bi);
    emit_stats<DT>(P, bi, er, er.resid, sh_st);
    const double st[4] = {sh_st[0], sh_st[1], sh_st[2], sh_st[3]};
    const int v0 = w * kEmitChunk + threadIdx.x * kEmitPerThread;
    double s[2] = {0.0, 0.0};
    for (int e = 0; e < kEmitPerThread; ++e) {
        const int v = v0 + e;
        if (v < P.V) {
            double r, p;
            emit_weights<DT>(P, er.row_off, v, st, er.resid, r, p);
            s[0] += r;
            s[1] += p;
        }
    }
    block_sum<2>(s, lds_d);
    if (threadIdx.x == 0) {
        double *o = P.emit + ((size_t)bi * P.We + w) * kEmitWords;
        o[0] = s[0];
        o[1] = s[1];
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rapid_emit_pick_kernel(RapidParams P) {
    __shared__ double sh_scan[kThreads + 1];
    __shared__ int lds_i[kWaves];
    __shared__ double sh_st[4];
    const int w = (int)(blockIdx.x % (unsigned)P.We), bi = (int)(blockIdx.x / (unsigned)P.We);
    const int tid = threadIdx.x;
    const EmitRow er = emit_row(P, bi);
    const double *parts = P.emit + (size_t)bi * P.We * kEmitWords;

    // totals and this chunk's prefix, summed in chunk order by every thread
    double Sr = 0.0, Sp = 0.0;
    for (int k = 0; k < P.We; ++k) {
        Sr += parts[kEmitWords * k];
        Sp += parts[kEmitWords * k + 1];
    }
    const bool use_r = er.resid && (Sr > 0.0);
    const int sel = use_r ? 0 : 1;
    const double S = use_r ? Sr : Sp;
    double pre = 0.0;
    for (int k = 0; k < w; ++k)
        pre += parts[kEmitWords * k + sel];
    const double mine = parts[kEmitWords * w + sel];
    const double u = clamp_uniform(P.u_sample[er.row], (w == 0 && tid == 0) ? P.dev_err : nullptr);
    const double target = u * S;
    const bool crossing_here = (pre <= target) && (target < pre + mine);
    const bool write_dist = P.emit_dist != nullptr;
    if (!crossing_here && !write_dist)
        return;

    emit_stats<DT>(P, bi, er, use_r, sh_st);
    const double st[4] = {sh_st[0], sh_st[1], sh_st[2], sh_st[3]};
    const int v0 = w * kEmitChunk + tid * kEmitPerThread;
    double wt[kEmitPerThread];
    double tsum = 0.0;
    for (int e = 0; e < kEmitPerThread; ++e) {
        const int v = v0 + e;
        double r = 0.0, p = 0.0;
        if (v < P.V)
            emit_weights<DT>(P, er.row_off, v, st, use_r, r, p);
        wt[e] = use_r ? r : p;
        tsum += wt[e];
    }
    if (write_dist) {
        const double invS = 1.0 / S;
        for (int e = 0; e < kEmitPerThread; ++e) {
            const int v = v0 + e;
            if (v < P.V)
                P.emit_dist[(size_t)bi * P.V + v] = (float)(wt[e] * invS);
        }
    }
    if (!crossing_here)
        return;
    // exclusive scan of the per-thread sums, in thread order
    sh_scan[tid] = tsum;
    __syncthreads();
    if (tid == 0) {
        double c = pre;
        for (int k = 0; k < kThreads; ++k) {
            const double x = sh_scan[k];
            sh_scan[k] = c;
            c += x;
        }
        sh_scan[kThreads] = c;
    }
    __syncthreads();
    int found = 0x7fffffff, last_pos = -1;
    double c = sh_scan[tid];
    for (int e = 0; e < kEmitPerThread; ++e) {
        const int v = v0 + e;
        if (v >= P.V)
            break;
        c += wt[e];
        if (wt[e] > 0.0)
            last_pos = v;
        if (c > target && found == 0x7fffffff)
            found = v;
    }
    found = block_min_int(found, lds_i);
    if (found == 0x7fffffff) {
        // only reachable through rounding at the chunk's end: the last
        // element of the chunk with positive weight
        const int neg = block_min_int(-last_pos, lds_i);
        found = -neg;
    }
    if (tid == 0 && found >= 0)
        P.token[bi] = found;
}

template <int DT, int NV>
static int blocks_per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rapid_rows_kernel<DT, NV>, kThreads, 0) != hipSuccess)
        return 0;
    return n;
}

int rapid_blocks_per_cu(int dt, int nv) {
    if (dt == DT_BF16) {
        switch (nv) {
        case 1: return blocks_per_cu<DT_BF16, 1>();
        case 2: return blocks_per_cu<DT_BF16, 2>();
        case 4: return blocks_per_cu<DT_BF16, 4>();
        case 8: return blocks_per_cu<DT_BF16, 8>();
        }
    } else {
        switch (nv) {
        case 1: return blocks_per_cu<DT_F32, 1>();
        case 2: return blocks_per_cu<DT_F32, 2>();
        case 4: return blocks_per_cu<DT_F32, 4>();
        case 8: return blocks_per_cu<DT_F32, 8>();
        }
    }
    return 0;
}

template <int DT, int NV>
static hipError_t launch_t(const Plan &plan, const RapidParams &p, hipStream_t s, hipEvent_t after_rows) {
    hipLaunchKernelGGL((rapid_rows_kernel<DT, NV>), dim3(plan.grid), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (after_rows) {
        e = hipEventRecord(after_rows, s);
        if (e != hipSuccess)
            return e;
    }
    const unsigned fin = (unsigned)((p.R + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((rapid_finalize_kernel<DT>), dim3(fin), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const dim3 eg((unsigned)p.We * (unsigned)p.B);
    hipLaunchKernelGGL((rapid_emit_norm_kernel<DT>), eg, dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((rapid_emit_lse_kernel<DT>), eg, dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((rapid_emit_sum_kernel<DT>), eg, dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((rapid_emit_pick_kernel<DT>), eg, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_rapid(int dt, const Plan &plan, const RapidParams &p, hipStream_t s, hipEvent_t after_rows) {
    if (dt == DT_BF16) {
        switch (plan.nv) {
        case 1: return launch_t<DT_BF16, 1>(plan, p, s, after_rows);
        case 2: return launch_t<DT_BF16, 2>(plan, p, s, after_rows);
        case 4: return launch_t<DT_BF16, 4>(plan, p, s, after_rows);
        case 8: return launch_t<DT_BF16, 8>(plan, p, s, after_rows);
        }
    } else {
        switch (plan.nv) {
        case 1: return launch_t<DT_F32, 1>(plan, p, s, after_rows);
        case 2: return launch_t<DT_F32, 2>(plan, p, s, after_rows);
        case 4: return launch_t<DT_F32, 4>(plan, p, s, after_rows);
        case 8: return launch_t<DT_F32, 8>(plan, p, s, after_rows);
        }
    }
    return hipErrorInvalidValue;
}

// Zero fill used to prepare a workspace (a kernel, not a memset node).
__global__ void fill_zero_kernel(uint32_t *p, size_t n_words, uint8_t *tail, int n_tail) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words; i += stride)
        p[i] = 0u;
    if (blockIdx.x == 0 && (int)threadIdx.x < n_tail)
        tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t s) {
    if (bytes == 0)
        return hipSuccess;
    const size_t words = bytes / 4;
    const int n_tail = (int)(bytes - words * 4);
    uint8_t *tail = static_cast<uint8_t *>(ptr) + words * 4;
    size_t blocks = (words + kThreads - 1) / kThreads;
    if (blocks > 4096)
        blocks = 4096;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       static_cast<uint32_t *>(ptr), words, tail, n_tail);
    return hipGetLastError();
}

} // namespace vwl
